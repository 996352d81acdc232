// Output-feature mixed W8 (symmetric) / W4 (asymmetric) x A8 (symmetric).
//
// MixLLM page, section 3.3: two-step dequantization.  Per 128-column group the
// kernel first forms the exact integer product acc = xq . (q - z) on the int8
// matrix cores (q - z fits int8 for both row sets, so nothing overflows), then
// multiplies by the scales (s_w per row and group; s_a per token or per token
// and group) and adds into an fp32 accumulator -- the group accumulator and
// the global accumulator of the page's pipeline.  Both row sets run in one
// launch (the page runs them concurrently) and the epilogue writes each output
// straight to its original column (the page's fused scatter epilogue).
//
// gfx950 design: v_mfma_i32_16x16x64_i8 with the activations as the A operand
// (16 tokens) and the weights as the B operand (16 packed rows).  A workgroup
// stages a BM x 128 activation tile in LDS per group; each wave streams the
// pre-packed weight fragments of its own two 16-row tiles straight into
// registers (one 16-byte load per lane for 8-bit rows, 8 bytes for 4-bit
// rows).  4-bit codes are expanded to int8 (q - z) with byte-parallel integer
// arithmetic: (q + 128 - z) never carries out of its byte, and flipping bit 7
// turns it into the two's-complement q - z.  The int32 -> fp32 conversion is
// a single full-rate instruction on CDNA, so the page's bias trick for it is
// not needed here.
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

namespace {

// ---------------------------------------------------------------------------
// activation quantization: s = fp16(max|x| / 127) in fp32, xq = clamp(rint(x / s))
// ---------------------------------------------------------------------------
__device__ __forceinline__ _Float16 act_scale(float amax) {
  if (amax == 0.0f) return (_Float16)1.0f;
  _Float16 s = (_Float16)(amax / 127.0f);
  if (s == (_Float16)0.0f) s = __builtin_bit_cast(_Float16, (unsigned short)1);
  return s;
}

__device__ __forceinline__ uint32_t quant4(const _Float16* v, float s) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q = __builtin_rintf((float)v[i] / s);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    out |= (uint32_t(int(q)) & 0xffu) << (8 * i);
  }
  return out;
}

// one workgroup per token row; 256 threads x 8 elements per pass
__global__ __launch_bounds__(256) void quant_act_kernel(const _Float16* __restrict__ x, int K, int ga,
                                                        int8_t* __restrict__ xq, _Float16* __restrict__ xs) {
  const int m = blockIdx.x, tid = threadIdx.x;
  const _Float16* xr = x + size_t(m) * K;
  __shared__ float red[4];
  if (ga == 128) {
    // 16 threads per group of 128
    for (int base = 0; base < K; base += 2048) {
      const int k = base + 8 * tid;
      u32x4 raw = {0, 0, 0, 0};
      if (k < K) raw = ld16(xr + k);
      const half8 v = __builtin_bit_cast(half8, raw);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)v[i]));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      if (k < K) {
        const _Float16 s16 = act_scale(amax);
        const float s = (float)s16;
        _Float16 e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = v[i];
        const uint2 q = make_uint2(quant4(e, s), quant4(e + 4, s));
        *reinterpret_cast<uint2*>(xq + size_t(m) * K + k) = q;
        if ((tid & 15) == 0) xs[size_t(m) * (K / 128) + k / 128] = s16;
      }
    }
    return;
  }
  float amax = 0.0f;
  for (int k = 8 * tid; k < K; k += 2048) {
    const half8 v = __builtin_bit_cast(half8, ld16(xr + k));
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)v[i]));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const _Float16 s16 = act_scale(amax);
  const float s = (float)s16;
  if (tid == 0) xs[m] = s16;
  for (int k = 8 * tid; k < K; k += 2048) {
    const half8 v = __builtin_bit_cast(half8, ld16(xr + k));
    _Float16 e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = v[i];
    *reinterpret_cast<uint2*>(xq + size_t(m) * K + k) = make_uint2(quant4(e, s), quant4(e + 4, s));
  }
}

// ---------------------------------------------------------------------------
// two-step int8 GEMM
// ---------------------------------------------------------------------------
struct W48Args {
  const int32_t* rows;
  const _Float16* s;
  const uint8_t* z;
  const int8_t* c8;
  const uint8_t* c4;
  const int8_t* xq;
  const _Float16* xs;
  _Float16* y;
  int32_t* acc_out;  // debug: int32 [M][N][G] group products, else null
  int N, K, M, T8, T4, ga;
};

constexpr int kNT = 2;  // 16-row weight tiles per wave

__device__ __forceinline__ int lds_chunk(int row, int c) { return row * 8 + (c ^ (row & 7)); }

// int8 (q - z) for 16 nibbles of one lane (two dwords) and zero z.
__device__ __forceinline__ i32x4 expand4(uint2 w, uint32_t zc) {
  const uint32_t m = 0x0f0f0f0fu, f = 0x80808080u;
  i32x4 r;
  r[0] = int(((w.x & m) + zc) ^ f);
  r[1] = int((((w.x >> 4) & m) + zc) ^ f);
  r[2] = int(((w.y & m) + zc) ^ f);
  r[3] = int((((w.y >> 4) & m) + zc) ^ f);
  return r;
}

template <int BM>
__global__ __launch_bounds__(256) void w48_kernel(W48Args a) {
  constexpr int TM = BM / 16;
  __shared__ u32x4 as_[BM * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int m0 = blockIdx.x * BM;
  const int T = a.T8 + a.T4;
  const int t0 = (blockIdx.y * 4 + wave) * kNT;  // first packed tile of this wave
  const int G = a.K / 128, KT = a.K / 64;

  f32x4 tot[TM][kNT];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j) tot[i][j] = f32x4{0, 0, 0, 0};

  for (int grp = 0; grp < G; ++grp) {
    // stage the BM x 128 activation tile
    __syncthreads();
    for (int idx = tid; idx < BM * 8; idx += 256) {
      const int row = idx >> 3, c = idx & 7, m = m0 + row;
      u32x4 v = {0, 0, 0, 0};
      if (m < a.M) v = ld16(a.xq + size_t(m) * a.K + size_t(grp) * 128 + 16 * c);
      as_[lds_chunk(row, c)] = v;
    }
    __syncthreads();

    i32x4 c[TM][kNT];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j) c[i][j] = i32x4{0, 0, 0, 0};
    float sw[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int t = t0 + j;
      sw[j] = 0.0f;
      if (t >= T) continue;
      sw[j] = (float)a.s[(size_t(t) * G + grp) * 16 + r16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = 2 * grp + h;
        i32x4 B;
        if (t < a.T8) {
          B = __builtin_bit_cast(i32x4, ld16(a.c8 + (size_t(t) * KT + kt) * 1024 + 16 * lane));
        } else {
          const int t4 = t - a.T8;
          const uint2 w = *reinterpret_cast<const uint2*>(a.c4 + (size_t(t4) * KT + kt) * 512 + 8 * lane);
          const uint32_t z = a.z[(size_t(t4) * G + grp) * 16 + r16];
          B = expand4(w, (128u - z) * 0x01010101u);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const i32x4 A = __builtin_bit_cast(i32x4, as_[lds_chunk(16 * i + r16, 4 * h + g)]);
          c[i][j] = mfma16_i8(A, B, c[i][j]);
        }
      }
    }
    if (a.acc_out) {
      // debug: exact group products, scattered to original rows
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int t = t0 + j;
        if (t >= T) continue;
        const int n = a.rows[16 * t + r16];
        if (n < 0) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = m0 + 16 * i + 4 * g + v;
            if (m < a.M) a.acc_out[(size_t(m) * a.N + n) * G + grp] = c[i][j][v];
          }
      }
      continue;
    }
    if (a.ga == 128) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = min(m0 + 16 * i + 4 * g + v, a.M - 1);
          const float sa = (float)a.xs[size_t(m) * G + grp];
#pragma unroll
          for (int j = 0; j < kNT; ++j) tot[i][j][v] = __builtin_fmaf(float(c[i][j][v]), sw[j] * sa, tot[i][j][v]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) tot[i][j][v] = __builtin_fmaf(float(c[i][j][v]), sw[j], tot[i][j][v]);
    }
  }
  if (a.acc_out) return;

  // epilogue: per-token scale, fused scatter to the original rows
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int t = t0 + j;
    if (t >= T) continue;
    const int n = a.rows[16 * t + r16];
    if (n < 0) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * i + 4 * g + v;
        if (m >= a.M) continue;
        const float sa = a.ga == 128 ? 1.0f : (float)a.xs[m];
        a.y[size_t(m) * a.N + n] = (_Float16)(tot[i][j][v] * sa);
      }
  }
}

// ---------------------------------------------------------------------------
// Large batches: 128 tokens x 128 packed rows per workgroup.  Workgroups are
// homogeneous: the first ceil(T8 / 8) row blocks hold 8-bit tiles, the rest
// 4-bit tiles.  Per 128-column group everything the matrix cores read is
// brought into LDS by global->LDS loads in MFMA fragment order -- activation
// fragments gathered 16 tokens at a time, weight fragments as packed, the
// group's weight scales and zero points -- so operand reads are conflict-free
// lane-linear reads and no staging registers are needed.  4-bit fragments
// land raw (512 B) and each wave expands the ones it multiplies into int8
// (q - z) in registers right before its MFMAs.  LDS is double-buffered: the
// next group's loads fly while the current group runs; one wait and one
// barrier per group.  Wave (wm, wn) owns tokens 64 wm + [0, 64) and rows
// 64 wn + [0, 64): 4 x 4 MFMA tiles, two k halves per group.
// ---------------------------------------------------------------------------
constexpr int kTB = 128;   // tokens and packed rows per workgroup

// LDS map (bytes): A[2] 16 KiB each, B[2] 16 KiB each (8-bit fragments, or
// the raw 4-bit fragments in the first 8 KiB), weight scales[2] 256 B each,
// zero points[2] 256 B each
constexpr int kLdsA = 0, kLdsB = 32768, kLdsS = 65536, kLdsZ = 66048, kLdsW48 = 66560;

// global->LDS loads with per-lane addresses: lane l's 16 (4) bytes land at
// LDS address lds + 16 l (4 l).  No output registers: completion is waited
// for with an explicit s_waitcnt vmcnt(0) before the barrier that publishes
// the data.
__device__ __forceinline__ void gdma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void gdma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// Non-temporal forms for data a launch reads once (the weight streams of the
// small-M kernel): the caches give those lines up first.
__device__ __forceinline__ void gdma16_once(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void gdma4_once(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt" ::"v"(g), "s"(lds) : "memory", "m0");
}

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// GA: activation scales per (token, group), else per token.  ACC: store the
// exact int32 group sums to a.acc_out instead of scaling them (the integer
// step of this kernel, checked bit for bit).
template <bool GA, bool ACC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void w48_tile_kernel(W48Args a) {
  __shared__ u32x4 lds[kLdsW48 / 16];
  uint8_t* const base = reinterpret_cast<uint8_t*>(lds);
  const uint32_t lbase = lds_u32(lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * kTB;
  const int nb8 = (a.T8 + 7) / 8;
  const bool q4 = int(blockIdx.y) >= nb8;
  // first packed tile of this workgroup and the end of its row set
  const int t0 = q4 ? a.T8 + (int(blockIdx.y) - nb8) * 8 : int(blockIdx.y) * 8;
  const int tend = q4 ? a.T8 + a.T4 : a.T8;
  const int G = a.K / 128, KT = a.K / 64;

  // Loads of one group into buffer `buf`.  Wave w brings activation
  // fragments f = w + 4 q (token tile f / 2, k half f % 2) and weight
  // fragments f (row tile f / 2, k tile 2 grp + f % 2); wave 0 the scales,
  // wave 1 the zero points.  Tokens and tiles past the end are clamped to the
  // last valid one (read, then discarded).
  auto issue = [&](int grp, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = wave + 4 * q, i = f >> 1, h = f & 1;
      const int m = min(m0 + 16 * i + r16, a.M - 1);
      gdma16(a.xq + size_t(m) * a.K + size_t(grp) * 128 + 64 * h + 16 * g,
             lbase + kLdsA + buf * 16384 + f * 1024);
      const int t = min(t0 + i, tend - 1), kt = 2 * grp + h;
      if (!q4) {
        gdma16(a.c8 + (size_t(t) * KT + kt) * 1024 + 16 * lane, lbase + kLdsB + buf * 16384 + f * 1024);
      } else {
        const uint8_t* src = a.c4 + (size_t(t - a.T8) * KT + kt) * 512;
        gdma4(src + 4 * lane, lbase + kLdsB + buf * 16384 + f * 512);
        gdma4(src + 256 + 4 * lane, lbase + kLdsB + buf * 16384 + f * 512 + 256);
      }
    }
    if (wave == 0) {
      const int t = min(t0 + (lane >> 3), tend - 1);
      gdma4(a.s + (size_t(t) * G + grp) * 16 + 2 * (lane & 7), lbase + kLdsS + buf * 256);
    } else if (wave == 1 && q4) {
      const int t = min(t0 + ((lane & 31) >> 2), tend - 1);
      gdma4(a.z + (size_t(t - a.T8) * G + grp) * 16 + 4 * (lane & 3), lbase + kLdsZ + buf * 256);
    }
  };

  f32x4 tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[i][j] = f32x4{0, 0, 0, 0};

  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
  __syncthreads();
  for (int grp = 0; grp < G; ++grp) {
    const int buf = grp & 1;
    if (grp + 1 < G) issue(grp + 1, buf ^ 1);
    const uint8_t* A = base + kLdsA + buf * 16384;
    const uint8_t* B = base + kLdsB + buf * 16384;
    const _Float16* S = reinterpret_cast<const _Float16*>(base + kLdsS + buf * 256);
    i32x4 c[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[i][j] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[i] = *reinterpret_cast<const i32x4*>(A + (2 * (4 * wm + i) + h) * 1024 + 16 * lane);
      if (q4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int f = 2 * (4 * wn + j) + h;
          const uint2 w = *reinterpret_cast<const uint2*>(B + f * 512 + 8 * lane);
          const uint32_t z = base[kLdsZ + buf * 256 + 16 * (4 * wn + j) + r16];
          bv[j] = expand4(w, (128u - z) * 0x01010101u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[j] = *reinterpret_cast<const i32x4*>(B + (2 * (4 * wn + j) + h) * 1024 + 16 * lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[i][j] = mfma16_i8(av[i], bv[j], c[i][j]);
    }
    if constexpr (ACC) {
      // the group sums as they are, at their original rows
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 4 * wn + j;
        const int n = t < tend ? a.rows[16 * t + r16] : -1;
        if (n < 0) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
            if (m < a.M) a.acc_out[(size_t(m) * a.N + n) * G + grp] = c[i][j][v];
          }
      }
    } else {
    // step two: scale the exact group sums into the fp32 accumulators
    float sw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sw[j] = (float)S[(4 * wn + j) * 16 + r16];
    if constexpr (GA) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = min(m0 + 64 * wm + 16 * i + 4 * g + v, a.M - 1);
          const float sa = (float)a.xs[size_t(m) * G + grp];
#pragma unroll
          for (int j = 0; j < 4; ++j) tot[i][j][v] = __builtin_fmaf(float(c[i][j][v]), sw[j] * sa, tot[i][j][v]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) tot[i][j][v] = __builtin_fmaf(float(c[i][j][v]), sw[j], tot[i][j][v]);
    }
    }
    if (grp + 1 < G) {
      // the next group's loads have landed (this wave's), then everyone's;
      // the barrier also retires this group's reads of `buf`
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
      __syncthreads();
    }
  }

  if constexpr (ACC) return;
  // per-token scale, fused scatter to the original rows
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 4 * wn + j;
    if (t >= tend) continue;
    const int n = a.rows[16 * t + r16];
    if (n < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
        if (m >= a.M) continue;
        const float sa = GA ? 1.0f : (float)a.xs[m];
        a.y[size_t(m) * a.N + n] = (_Float16)(tot[i][j][v] * sa);
      }
  }
}

// ---------------------------------------------------------------------------
// Small batches (M <= 64, per-token activation scales): the weights dominate,
// so the kernel streams them.  A workgroup owns four packed tiles (64 rows,
// homogeneous 8-bit or 4-bit) and walks K one 128-column group at a time
// through a 5-stage (M > 32: 4-stage) LDS pipeline: per group each wave issues the same number
// of global->LDS loads (its share of the activation fragments, its tile's
// weight fragments, scales and zero points), so every wait is a fixed vmcnt.
// One barrier per group publishes the shared activation fragments.
// ---------------------------------------------------------------------------
template <int TM>   // token tiles: M <= 16 TM
struct StreamCfg {
  // Stages - 1 groups per workgroup are in flight, two workgroups per CU:
  // five stages still fit two workgroups in the LDS for M <= 32, four for
  // M <= 64.  (Deeper pipelines for the 4-bit rows, whose stages are
  // smaller, measured the same: the loads themselves bound the kernel.)
  static constexpr int kStages = TM <= 2 ? 5 : 4;
  static constexpr int NA = (2 * TM + 3) / 4;           // activation loads per wave per group
  static constexpr int kA = 4 * NA * 1024;              // activation fragments per stage
  static constexpr int kB = 4 * 2048;                   // weight fragments, 2 KiB per wave
  static constexpr int kS = 4 * 256;                    // scales, 256 B per wave
  static constexpr int kZ = 4 * 256;                    // zero points, 256 B per wave
  static constexpr int kStage = kA + kB + kS + kZ;
  static constexpr int kLoads8 = NA + 3;                // loads per wave per group, 8-bit rows
  static constexpr int kLoads4 = NA + 3;                // 4-bit rows
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One workgroup's four tiles, all 8-bit (Q4 false) or all 4-bit rows.  ACC:
// store each group's exact int32 sums to a.acc_out instead of scaling them.
template <int TM, bool Q4, bool ACC>
__device__ __forceinline__ void stream_tiles(const W48Args& a, uint8_t* base, int t0, int tend) {
  using C = StreamCfg<TM>;
  constexpr int kStages = C::kStages;
  constexpr int kLoads = Q4 ? C::kLoads4 : C::kLoads8;
  const uint32_t lbase = lds_u32(base);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int t = min(t0 + wave, tend - 1);   // this wave's tile (clamped; results discarded)
  const int G = a.K / 128, KT = a.K / 64;

  auto stage = [&](int grp) { return (grp % kStages) * C::kStage; };
  auto issue = [&](int grp) {
    const uint32_t st = lbase + stage(grp);
#pragma unroll
    for (int q = 0; q < C::NA; ++q) {
      const int f = wave + 4 * q, i = min(f >> 1, TM - 1), h = f & 1;
      const int m = min(16 * i + r16, a.M - 1);
      gdma16(a.xq + size_t(m) * a.K + size_t(grp) * 128 + 64 * h + 16 * g, st + f * 1024);
    }
    const uint32_t sb = st + C::kA + wave * 2048;
    if constexpr (!Q4) {
      gdma16_once(a.c8 + (size_t(t) * KT + 2 * grp) * 1024 + 16 * lane, sb);
      gdma16_once(a.c8 + (size_t(t) * KT + 2 * grp + 1) * 1024 + 16 * lane, sb + 1024);
    } else {
      // the group's two 512-byte fragments are contiguous: one 1 KiB load
      gdma16_once(a.c4 + (size_t(t - a.T8) * KT + 2 * grp) * 512 + 16 * lane, sb);
    }
    gdma4_once(a.s + (size_t(t) * G + grp) * 16 + 2 * (lane & 7), st + C::kA + C::kB + wave * 256);
    if constexpr (Q4)
      gdma4_once(a.z + (size_t(t - a.T8) * G + grp) * 16 + 4 * (lane & 3), st + C::kA + C::kB + C::kS + wave * 256);
  };

  f32x4 tot[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) tot[i] = f32x4{0, 0, 0, 0};
  // the previous group's int32 sums and weight scale: they are scaled into
  // tot while the current group's MFMAs run, so no step waits for its own
  // matrix-core results
  i32x4 cp[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) cp[i] = i32x4{0, 0, 0, 0};
  float swp = 0.0f;

  // ACC: this lane's original row (-1: none), loaded and awaited before the
  // first global->LDS load, so no later wait of the compiler's covers them
  int n_acc = -1;
  if constexpr (ACC) {
    if (t0 + wave < tend) n_acc = a.rows[16 * (t0 + wave) + r16];
    wait_vm<0>();
  }
  for (int p = 0; p < kStages - 1 && p < G; ++p) issue(p);
  for (int grp = 0; grp < G; ++grp) {
    // this wave's loads of group grp have landed once at most the loads of the
    // (up to kStages - 2) later groups are in flight
    static_assert(kStages - 2 <= 3, "wait cases");
    const int later = min(G - 1 - grp, kStages - 2);
    if (later >= 3)
      wait_vm<3 * kLoads>();
    else if (later == 2)
      wait_vm<2 * kLoads>();
    else if (later == 1)
      wait_vm<kLoads>();
    else
      wait_vm<0>();
    __syncthreads();   // every wave's loads of grp landed; every wave is done with grp - 1
    if (grp + kStages - 1 < G) issue(grp + kStages - 1);   // into grp - 1's stage
    // every LDS read of the step first, then one wait
    const uint8_t* st = base + stage(grp);
    const uint8_t* B = st + C::kA + wave * 2048;
    i32x4 av[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) av[i][h] = *reinterpret_cast<const i32x4*>(st + (2 * i + h) * 1024 + 16 * lane);
    const float sw = (float)reinterpret_cast<const _Float16*>(st + C::kA + C::kB + wave * 256)[r16];
    i32x4 bv[2];
    if constexpr (!Q4) {
      bv[0] = *reinterpret_cast<const i32x4*>(B + 16 * lane);
      bv[1] = *reinterpret_cast<const i32x4*>(B + 1024 + 16 * lane);
    } else {
      const uint2 w0 = *reinterpret_cast<const uint2*>(B + 8 * lane);
      const uint2 w1 = *reinterpret_cast<const uint2*>(B + 512 + 8 * lane);
      const uint32_t z = st[C::kA + C::kB + C::kS + wave * 256 + r16];
      const uint32_t zb = (128u - z) * 0x01010101u;
      bv[0] = expand4(w0, zb);
      bv[1] = expand4(w1, zb);
    }
    i32x4 c[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      c[i] = mfma16_i8(av[i][0], bv[0], i32x4{0, 0, 0, 0});
      c[i] = mfma16_i8(av[i][1], bv[1], c[i]);
    }
    if constexpr (ACC) {
      // the group sums as they are, at their original rows (stores add to the
      // vector-memory count, which only makes the fixed waits above stricter)
      if (n_acc >= 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = 16 * i + 4 * g + v;
            if (m < a.M) a.acc_out[(size_t(m) * a.N + n_acc) * G + grp] = c[i][v];
          }
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[i][v] = __builtin_fmaf(float(cp[i][v]), swp, tot[i][v]);
#pragma unroll
    for (int i = 0; i < TM; ++i) cp[i] = c[i];
    swp = sw;
  }
  if constexpr (ACC) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) tot[i][v] = __builtin_fmaf(float(cp[i][v]), swp, tot[i][v]);

  if (t0 + wave >= tend) return;
  const int n = a.rows[16 * (t0 + wave) + r16];
  if (n < 0) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * i + 4 * g + v;
      if (m < a.M) a.y[size_t(m) * a.N + n] = (_Float16)(tot[i][v] * (float)a.xs[m]);
    }
}

template <int TM, bool ACC>
__global__ __launch_bounds__(256) void w48_stream_kernel(W48Args a) {
  using C = StreamCfg<TM>;
  static_assert(2 * C::kStages * C::kStage <= 160 * 1024, "two workgroups per CU");
  __shared__ u32x4 lds[C::kStages * C::kStage / 16];
  uint8_t* const base = reinterpret_cast<uint8_t*>(lds);
  const int nb8 = (a.T8 + 3) / 4;
  if (int(blockIdx.x) < nb8)
    stream_tiles<TM, false, ACC>(a, base, int(blockIdx.x) * 4, a.T8);
  else
    stream_tiles<TM, true, ACC>(a, base, a.T8 + (int(blockIdx.x) - nb8) * 4, a.T8 + a.T4);
}

W48Args make_args(const W48ImageView& im, const int8_t* xq, const uint16_t* xs, int ga, uint16_t* y,
                  int32_t* acc, int M) {
  W48Args a;
  a.rows = im.rows;
  a.s = reinterpret_cast<const _Float16*>(im.s);
  a.z = im.z;
  a.c8 = im.c8;
  a.c4 = im.c4;
  a.xq = xq;
  a.xs = reinterpret_cast<const _Float16*>(xs);
  a.y = reinterpret_cast<_Float16*>(y);
  a.acc_out = acc;
  a.N = im.N;
  a.K = im.K;
  a.M = M;
  a.T8 = im.T8;
  a.T4 = im.T4;
  a.ga = ga;
  return a;
}

template <bool ACC>
void launch_stream(const W48Args& a, hipStream_t s) {
  const dim3 grid(unsigned((a.T8 + 3) / 4 + (a.T4 + 3) / 4));
  if (a.M <= 16)
    hipLaunchKernelGGL((w48_stream_kernel<1, ACC>), grid, dim3(256), 0, s, a);
  else if (a.M <= 32)
    hipLaunchKernelGGL((w48_stream_kernel<2, ACC>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((w48_stream_kernel<4, ACC>), grid, dim3(256), 0, s, a);
}

template <bool ACC>
void launch_tile(const W48Args& a, hipStream_t s) {
  const unsigned by = unsigned((a.T8 + 7) / 8 + (a.T4 + 7) / 8);
  const dim3 grid(unsigned((a.M + kTB - 1) / kTB), by);
  if (a.ga == 128)
    hipLaunchKernelGGL((w48_tile_kernel<true, ACC>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((w48_tile_kernel<false, ACC>), grid, dim3(256), 0, s, a);
}

// Picks the kernel for (M, ga).  A call with a.acc_out set takes the same
// route with the kernel's group-sum store in place of its scaling step, so
// the exported int32 sums are those of the kernel that runs the product.
int launch(const W48Args& a, void* stream) {
  const int T = a.T8 + a.T4;
  const unsigned gy = unsigned((T + 4 * kNT - 1) / (4 * kNT));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool acc = a.acc_out != nullptr;
  const int tile_rows = (a.T8 + 7) / 8 + (a.T4 + 7) / 8;   // 128-row workgroups of the tile kernel
  if (a.M > 64 && a.M <= 128 && a.ga != 128 && tile_rows <= device_compute_units()) {
    // Neither kernel splits K.  Here the tile kernel's single row of
    // workgroups leaves CUs idle while each walks all of K, so two 64-token
    // passes of the stream kernel, which reads the weights at HBM speed, are
    // faster.  Per-token scales make a token range a self-contained call.
    W48Args c = a;
    for (int m0 = 0; m0 < a.M; m0 += 64) {
      c.M = a.M - m0 < 64 ? a.M - m0 : 64;
      c.xq = a.xq + size_t(m0) * size_t(a.K);
      c.xs = a.xs ? a.xs + m0 : nullptr;
      c.y = a.y ? a.y + size_t(m0) * size_t(a.N) : nullptr;
      c.acc_out = acc ? a.acc_out + size_t(m0) * size_t(a.N) * size_t(a.K / 128) : nullptr;
      const int rc = launch(c, stream);
      if (rc != 0) return rc;
    }
    return 0;
  }
  if (a.M <= 64 && a.ga != 128) {
    if (acc)
      launch_stream<true>(a, s);
    else
      launch_stream<false>(a, s);
  } else if (a.M > 64) {
    if (acc)
      launch_tile<true>(a, s);
    else
      launch_tile<false>(a, s);
  } else if (a.M <= 32) {   // group activation scales, M <= 64
    hipLaunchKernelGGL(w48_kernel<32>, dim3(unsigned((a.M + 31) / 32), gy), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(w48_kernel<64>, dim3(unsigned((a.M + 63) / 64), gy), dim3(256), 0, s, a);
  }
  return int(hipGetLastError());
}

}  // namespace

int launch_quant_act(const uint16_t* x, int M, int K, int ga, int8_t* xq, uint16_t* xs, void* stream) {
  hipLaunchKernelGGL(quant_act_kernel, dim3(unsigned(M)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<const _Float16*>(x), K, ga, xq, reinterpret_cast<_Float16*>(xs));
  return int(hipGetLastError());
}

int launch_w48(const W48ImageView& im, const int8_t* xq, const uint16_t* xs, int ga, uint16_t* y, int M,
               void* stream) {
  return launch(make_args(im, xq, xs, ga, y, nullptr, M), stream);
}

int launch_w48_acc(const W48ImageView& im, const int8_t* xq, int ga, int32_t* acc, int M, void* stream) {
  return launch(make_args(im, xq, nullptr, ga, nullptr, acc, M), stream);
}

}  // namespace gbb
