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
  // The stream kernel's K split: kseg8 (kseg4) segments of seg8 (seg4)
  // 128-column groups, the last one shorter, for the 8-bit (4-bit) row
  // blocks.  With a split, every row's partial sums go to part, fp32
  // [segment][M][packed row] (zero between calls).
  float* part;
  int N, K, M, T8, T4, ga;
  int kseg8, seg8, kseg4, seg4;
  int tiles;   // the stream kernel's packed tiles per wave (1 or 2)
  int tt;      // the tile kernel's 16-token tiles per workgroup (8 or 4)
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
// Large batches: tiles of 128 (or 64) tokens x 128 packed 4-bit rows or x 64
// packed 8-bit rows per workgroup, one row set per workgroup.  Wave w owns NJ
// packed row tiles (two 4-bit tiles or one 8-bit tile) for all TT 16-token
// tiles (TT = 8 or 4), so each weight fragment is read and, for 4-bit rows,
// expanded to int8 (q - z) by one wave only, and its expansion serves TT
// MFMAs.  Per 128-column group everything the matrix cores read reaches LDS
// by global->LDS loads in MFMA fragment order: the activation fragments (16
// tokens x 64 columns each, shared by the four waves), each wave's own weight
// fragments, scales and zero points, so no staging registers are needed and
// every operand read is a lane-linear LDS read.  Groups flow through two LDS
// stages: the next group's loads fly while the current group runs; one fixed
// vmcnt wait and one barrier per group.  A 128-token tile takes 52 KiB, so
// three workgroups share a CU; a 64-token tile 36 KiB, so four do.  Each token tile's int32 sums are scaled into fp32
// while the next tile's MFMAs run.  Workgroups are dealt to the XCDs in
// contiguous stretches of a grouped tile order, so the tiles in flight on an
// XCD share their activation and weight tiles in its L2.
// ---------------------------------------------------------------------------
constexpr int kTB = 128;   // tokens per workgroup of the larger tile
// 1.5 2^23 and its fp32 bits: the float with bits kOffI + n is kOffF + n for
// |n| < 2^22 (every int32 group sum: |127 * 127 * 128| < 2^21)
constexpr int32_t kOffI = 0x4B400000;
constexpr float kOffF = 12582912.0f;

// TT 16-token tiles per workgroup (8 or 4)
template <bool Q4, int TT>
struct TileCfg {
  static constexpr int NJ = Q4 ? 2 : 1;             // packed row tiles per wave
  static constexpr int kRows = 64 * NJ;             // packed rows per workgroup
  static constexpr int kStages = 2;
  static constexpr int kA = TT * 2 * 1024;          // activation fragments (TT token tiles x 2 k halves)
  static constexpr int kBw = 2048;                  // weight fragments of one wave (NJ tiles x 2 halves)
  static constexpr int kB = 4 * kBw;
  static constexpr int kS = 4 * 256;                // weight scales, 256 B per wave
  static constexpr int kZ = Q4 ? 4 * 256 : 0;       // zero points, 256 B per wave
  static constexpr int kStage = kA + kB + kS + kZ;
};
// LDS bytes of the stages (one size serves both row sets), and of the
// per-group activation scales staged after them: two buffers of 16 TT tokens
// x the scales of a group pair (4 bytes).
template <int TT>
constexpr int tile_lds() {
  return TileCfg<true, TT>::kStages * TileCfg<true, TT>::kStage;
}
template <int TT>
constexpr int tile_xs() {
  return 2 * 16 * TT * 4;
}
static_assert(TileCfg<false, 8>::kStages * TileCfg<false, 8>::kStage <= tile_lds<8>(), "one LDS size serves both");
static_assert(3 * tile_lds<8>() <= 160 * 1024, "three 128-token workgroups per CU");
static_assert(2 * (tile_lds<8>() + tile_xs<8>()) <= 160 * 1024, "two with staged scales");
static_assert(4 * tile_lds<4>() <= 160 * 1024, "four 64-token workgroups per CU");
static_assert(3 * (tile_lds<4>() + tile_xs<4>()) <= 160 * 1024, "three with staged scales");
// resident workgroups per CU of the tile kernel as the token-tile rule
// counts them (at 128 tokens with per-group activation scales two: that
// kernel took 204 VGPRs; at 164 since its token tiles run in halves three
// fit, which measured the same)
__host__ __device__ constexpr int tile_wgs_per_cu(int TT, bool ga) { return TT == 8 ? (ga ? 2 : 3) : 4; }

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

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// One workgroup's tile: tokens m0 ... m0 + 16 TT - 1, packed tiles t0 ... t0 +
// 4 NJ - 1 of one row set.  Q4: the row set (4-bit or 8-bit rows).  GA:
// activation scales per (token, group), else per token.  ACC: store the exact
// int32 group sums to a.acc_out instead of scaling them (the integer step of
// this kernel, checked bit for bit).
// XS (with GA): the activation scales reach LDS with the group's loads (an
// even group count and a 4-byte aligned scale array), else each output
// reads its scale from memory.
template <int TT, bool Q4, bool GA, bool ACC, bool XS>
__device__ __forceinline__ void tile_body(const W48Args& a, uint8_t* base, int m0, int t0, int seg) {
  using C = TileCfg<Q4, TT>;
  constexpr int kLds = tile_lds<TT>();
  constexpr int S = C::kStages, NJ = C::NJ;
  const uint32_t lbase = lds_u32(base);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int tend = Q4 ? a.T8 + a.T4 : a.T8;   // end of this row set's packed tiles
  const int tw = t0 + NJ * wave;              // this wave's first packed tile
  const int G = a.K / 128, KT = a.K / 64;
  // this workgroup's K segment: groups g0 ... gend - 1
  const int sg = Q4 ? a.seg4 : a.seg8;
  const int g0 = seg * sg, gend = min(G, g0 + sg);

  // Loads of group grp into its stage.  Tokens and tiles past the end are
  // clamped to the last valid one (read, then discarded).
  auto issue = [&](int grp) {
    const uint32_t sb = lbase + uint32_t((grp % S) * C::kStage);
#pragma unroll
    for (int q = 0; q < TT / 2; ++q) {   // activation fragment f: token tile f / 2, k half f % 2
      const int f = wave + 4 * q, i = f >> 1, h = f & 1;
      const int m = min(m0 + 16 * i + r16, a.M - 1);
      gdma16(a.xq + size_t(m) * a.K + size_t(grp) * 128 + 64 * h + 16 * g, sb + f * 1024);
    }
    const uint32_t bb = sb + C::kA + wave * C::kBw;
    if constexpr (!Q4) {   // one 8-bit tile: two 1 KiB fragments
      const int tt = min(tw, tend - 1);
      gdma16(a.c8 + (size_t(tt) * KT + 2 * grp) * 1024 + 16 * lane, bb);
      gdma16(a.c8 + (size_t(tt) * KT + 2 * grp + 1) * 1024 + 16 * lane, bb + 1024);
    } else {   // two 4-bit tiles: each group's two 512-byte fragments are one contiguous KiB
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tt = min(tw + j, tend - 1);
        gdma16(a.c4 + (size_t(tt - a.T8) * KT + 2 * grp) * 512 + 16 * lane, bb + j * 1024);
      }
    }
    {   // scales: lanes 8 j + 0..7 bring tile j's 16 (the other lanes repeat them)
      const int tt = min(tw + ((lane >> 3) & (NJ - 1)), tend - 1);
      gdma4(a.s + (size_t(tt) * G + grp) * 16 + 2 * (lane & 7), sb + C::kA + C::kB + wave * 256);
    }
    if constexpr (GA && XS && !ACC) {   // waves 0 ... TT / 4 - 1: tokens 64 w + lane, the group pair's scales
      if (wave < TT / 4)
        gdma4(a.xs + size_t(min(m0 + 64 * wave + lane, a.M - 1)) * G + (grp & ~1),
              lbase + uint32_t(kLds + (grp & 1) * (16 * TT * 4) + wave * 256));
    }
    if constexpr (Q4) {   // zero points: lanes 4 j + 0..3 bring tile j's 16
      const int tt = min(tw + ((lane >> 2) & 1), tend - 1);
      gdma4(a.z + (size_t(tt - a.T8) * G + grp) * 16 + 4 * (lane & 3), sb + C::kA + C::kB + C::kS + wave * 256);
    }
  };

  f32x4 tot[TT][NJ];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) tot[i][j] = f32x4{0, 0, 0, 0};

  // Offset sums (per-token scales): each group's MFMAs start from the bits
  // of kOffF = 1.5 2^23 instead of 0, so the int32 result read as fp32 is
  // kOffF + sum exactly (|sum| < 2^22) and scaling it takes one fma instead
  // of a conversion and an fma.  The offsets' total kOffF (s_a + s_b) comes
  // off after every pair of groups (and after a segment's last group), so
  // the running sum never holds more than two offsets: its extra rounding
  // stays within a few s_w against sums of ~10^4 s_w.
  constexpr bool kOff = !GA && !ACC;
  const i32x4 cinit = kOff ? i32x4{kOffI, kOffI, kOffI, kOffI} : i32x4{0, 0, 0, 0};
  float pend[NJ];   // scales whose offsets are still in tot
#pragma unroll
  for (int j = 0; j < NJ; ++j) pend[j] = 0.0f;

  issue(g0);
  for (int grp = g0; grp < gend; ++grp) {
    wait_vm<0>();      // this wave's loads of group grp have landed
    __syncthreads();   // everyone's have; every wave is done with grp - 1's stage
    if (grp + 1 < gend) issue(grp + 1);   // into grp - 1's stage
    const uint8_t* st = base + (grp % S) * C::kStage;
    const uint8_t* B = st + C::kA + wave * C::kBw;
    const _Float16* Sv = reinterpret_cast<const _Float16*>(st + C::kA + C::kB + wave * 256);
    float sw[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) sw[j] = (float)Sv[16 * j + r16];
    uint32_t zb[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      zb[j] = Q4 ? (128u - st[C::kA + C::kB + C::kS + wave * 256 + 16 * j + r16]) * 0x01010101u : 0u;
    auto bfrag = [&](int h, int j) -> i32x4 {
      if constexpr (Q4)
        return expand4(*reinterpret_cast<const uint2*>(B + j * 1024 + h * 512 + 8 * lane), zb[j]);
      else
        return *reinterpret_cast<const i32x4*>(B + h * 1024 + 16 * lane);
    };
    auto afrag = [&](int i, int h) -> i32x4 {
      return *reinterpret_cast<const i32x4*>(st + (2 * i + h) * 1024 + 16 * lane);
    };
    // step two for token tile i: the exact sums into fp32, scaled (or stored)
    auto finish = [&](int i, const i32x4 (&ci)[NJ]) {
      if constexpr (ACC) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int tt = tw + j;
          const int n = tt < tend ? a.rows[16 * tt + r16] : -1;
          if (n < 0) continue;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = m0 + 16 * i + 4 * g + v;
            if (m < a.M) a.acc_out[(size_t(m) * a.N + n) * G + grp] = ci[j][v];
          }
        }
      } else if constexpr (GA) {
        // XS: the scales of tokens 16 i + 4 g ... + 3 in one 16-byte LDS read
        u32x4 xp = u32x4{0, 0, 0, 0};
        if constexpr (XS)
          xp = *reinterpret_cast<const u32x4*>(base + kLds + (grp & 1) * (16 * TT * 4) + 4 * (16 * i + 4 * g));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float sa = XS ? ((grp & 1) ? hi_half(xp[v]) : lo_half(xp[v]))
                              : (float)a.xs[size_t(min(m0 + 16 * i + 4 * g + v, a.M - 1)) * G + grp];
#pragma unroll
          for (int j = 0; j < NJ; ++j) tot[i][j][v] = __builtin_fmaf(float(ci[j][v]), sw[j] * sa, tot[i][j][v]);
        }
      } else if constexpr (kOff) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int32_t e = ci[j][v];   // (a bit cast of the vector element itself reads element 0)
            tot[i][j][v] = __builtin_fmaf(__builtin_bit_cast(float, e), sw[j], tot[i][j][v]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) tot[i][j][v] = __builtin_fmaf(float(ci[j][v]), sw[j], tot[i][j][v]);
      }
    };

    // token tiles in runs of four: each run's first k half for all its
    // tiles, then the second half tile by tile, each tile's sums scaled
    // while the next tile's MFMAs run; only four tiles' sums are live at a
    // time (with all eight the offset sums spilled at three waves per SIMD)
    i32x4 b0[NJ], b1[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) b0[j] = bfrag(0, j);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b1[j] = bfrag(1, j);
#pragma unroll
    for (int i0 = 0; i0 < TT; i0 += 4) {
      i32x4 c[4][NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 a0 = afrag(i0 + i, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) c[i][j] = mfma16_i8(a0, b0[j], cinit);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 a1 = afrag(i0 + i, 1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) c[i][j] = mfma16_i8(a1, b1[j], c[i][j]);
        if (i > 0) finish(i0 + i - 1, c[i - 1]);
      }
      finish(i0 + 3, c[3]);
    }
    if constexpr (kOff) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) pend[j] += sw[j];
      if (((grp - g0) & 1) || grp + 1 == gend) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float off = kOffF * pend[j];
          pend[j] = 0.0f;
#pragma unroll
          for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) tot[i][j][v] -= off;
        }
      }
    }
  }
  if constexpr (ACC) return;

  if (a.part) {
    // K split: this segment's sums at the packed rows; w48_reduce_kernel
    // adds the segments, applies the per-token scale and scatters
    const int P = 16 * (a.T8 + a.T4);
    float* pp = a.part + size_t(seg) * size_t(a.M) * size_t(P);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int tt = tw + j;
      if (tt >= tend || a.rows[16 * tt + r16] < 0) continue;   // padding rows: no partials
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + 16 * i + 4 * g + v;
          if (m < a.M) pp[size_t(m) * P + 16 * tt + r16] = tot[i][j][v];
        }
    }
    return;
  }
  // per-token scale, fused scatter to the original rows
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int tt = tw + j;
    if (tt >= tend) continue;
    const int n = a.rows[16 * tt + r16];
    if (n < 0) continue;
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * i + 4 * g + v;
        if (m >= a.M) continue;
        const float sa = GA ? 1.0f : (float)a.xs[m];
        a.y[size_t(m) * a.N + n] = (_Float16)(tot[i][j][v] * sa);
      }
  }
}

// Tile order: ntm token tiles x (nrb8 8-bit + nrb4 4-bit) row blocks (8-bit
// row blocks first), walked in groups of kGroupRows row blocks: within a
// group the row blocks vary fastest, so the workgroups in flight on an XCD
// share both their activation and their weight tiles in its L2.
constexpr int kGroupRows = 8;

// per_xcd tiles of that order per XCD; token tiles of 16 TT tokens.
template <int TT, bool GA, bool ACC, bool XS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TT == 8 ? (GA || ACC ? 2 : 3)
                                                                                : (GA && !XS ? 3 : 4)))) void
w48_tile_kernel(W48Args a, int ntm, int nrb8, int nrb4, int per_xcd) {
  __shared__ u32x4 lds[(tile_lds<TT>() + (GA && XS ? tile_xs<TT>() : 0)) / 16];
  // workgroup i runs on XCD i % 8, which owns tiles [x per_xcd, (x + 1) per_xcd)
  // with a K split, each row block stands for kseg8 (kseg4) consecutive
  // (row block, K segment) units of the order
  const int bid = int(blockIdx.x);
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  const int nu8 = nrb8 * a.kseg8, nrb = nu8 + nrb4 * a.kseg4;
  if (t >= ntm * nrb) return;
  const int q = t / (kGroupRows * ntm), r = t - q * (kGroupRows * ntm);
  const int gr = min(kGroupRows, nrb - q * kGroupRows);   // row units in this group
  const int tm = r / gr, ru = q * kGroupRows + (r - tm * gr);
  uint8_t* const base = reinterpret_cast<uint8_t*>(lds);
  if (ru < nu8) {
    tile_body<TT, false, GA, ACC, XS>(a, base, tm * 16 * TT, (ru / a.kseg8) * 4, ru % a.kseg8);
  } else {
    const int r4 = ru - nu8;
    tile_body<TT, true, GA, ACC, XS>(a, base, tm * 16 * TT, a.T8 + (r4 / a.kseg4) * 8, r4 % a.kseg4);
  }
}

// ---------------------------------------------------------------------------
// Small batches (M <= 64, per-token activation scales): the weights dominate,
// so the kernel streams them.  A workgroup owns four packed tiles (64 rows,
// homogeneous 8-bit or 4-bit), or eight (two per wave) where K is split, and
// walks K one 128-column group at a time through an LDS pipeline: per group
// each wave issues the same number of global->LDS loads (its share of the
// activation fragments, its tiles' weight fragments, scales and zero
// points), so every wait is a fixed vmcnt.  One barrier per group publishes
// the shared activation fragments.
// ---------------------------------------------------------------------------
// TM token tiles (M <= 16 TM); GA: per-group activation scales; TW packed
// tiles per wave, so that a workgroup's one copy of a group's activation
// fragments serves 64 TW weight rows.
template <int TM, bool GA, int TW>
struct StreamCfg {
  // Stages - 1 groups per workgroup are in flight, two workgroups per CU:
  // with one tile per wave, five stages for M <= 32 and four for M <= 64
  // (deeper pipelines for the 4-bit rows, whose stages are smaller, measured
  // the same); with two, whose stages are twice as large, three and two.
  static constexpr int kStages = TW == 1 ? (TM > 2 ? 4 : 5) : (TM > 2 ? 2 : 3);
  static constexpr int NA = (2 * TM + 3) / 4;           // activation loads per wave per group
  static constexpr int kA = 4 * NA * 1024;              // activation fragments per stage
  static constexpr int kB = 4 * TW * 2048;              // weight fragments, 2 KiB per tile
  static constexpr int kS = 4 * TW * 256;               // scales, 256 B per tile
  static constexpr int kZ = 4 * TW * 256;               // zero points, 256 B per tile
  static constexpr int kX = GA ? 4 * 256 : 0;           // GA: the group pair's activation scales, per wave
  static constexpr int kStage = kA + kB + kS + kZ + kX;
  static constexpr int kLoads8 = NA + 3 * TW + (GA ? 1 : 0);   // loads per wave per group, 8-bit rows
  static constexpr int kLoads4 = NA + 3 * TW + (GA ? 1 : 0);   // 4-bit rows
  static_assert(2 * kStages * kStage <= 160 * 1024, "two workgroups per CU");
  static_assert(3 * kLoads8 < 64, "vmcnt range");
};

// One workgroup's four tiles, all 8-bit (Q4 false) or all 4-bit rows.  ACC:
// store each group's exact int32 sums to a.acc_out instead of scaling them.
// GA: activation scales per (token, group), [M][G] with G even: each group
// brings the scales of its pair of groups for every token (4 bytes a token,
// so the loads stay dword-aligned), and they multiply the weight scale.
template <int TM, bool GA, bool Q4, bool ACC, int TW>
__device__ __forceinline__ void stream_tiles(const W48Args& a, uint8_t* base, int t0, int tend, int seg,
                                             int seg_groups) {
  constexpr bool SA = GA && !ACC;   // the activation scales are loaded (ACC stores unscaled sums)
  using C = StreamCfg<TM, SA, TW>;
  constexpr int kStages = C::kStages;
  constexpr int kLoads = Q4 ? C::kLoads4 : C::kLoads8;
  const uint32_t lbase = lds_u32(base);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  int t[TW];   // this wave's tiles, t0 + wave + 4 k (clamped; results discarded)
#pragma unroll
  for (int k = 0; k < TW; ++k) t[k] = min(t0 + wave + 4 * k, tend - 1);
  const int G = a.K / 128, KT = a.K / 64;
  // this workgroup's K segment: groups g0 ... g0 + ng - 1
  const int g0 = seg * seg_groups, ng = min(G - g0, seg_groups);

  auto stage = [&](int j) { return (j % kStages) * C::kStage; };
  auto issue = [&](int j) {
    const int grp = g0 + j;
    const uint32_t st = lbase + stage(j);
#pragma unroll
    for (int q = 0; q < C::NA; ++q) {
      const int f = wave + 4 * q, i = min(f >> 1, TM - 1), h = f & 1;
      const int m = min(16 * i + r16, a.M - 1);
      gdma16(a.xq + size_t(m) * a.K + size_t(grp) * 128 + 64 * h + 16 * g, st + f * 1024);
    }
#pragma unroll
    for (int k = 0; k < TW; ++k) {
      const int slot = TW * wave + k;   // this tile's weight, scale and zero slots in the stage
      const uint32_t sb = st + C::kA + slot * 2048;
      if constexpr (!Q4) {
        gdma16_once(a.c8 + (size_t(t[k]) * KT + 2 * grp) * 1024 + 16 * lane, sb);
        gdma16_once(a.c8 + (size_t(t[k]) * KT + 2 * grp + 1) * 1024 + 16 * lane, sb + 1024);
      } else {
        // the group's two 512-byte fragments are contiguous: one 1 KiB load
        gdma16_once(a.c4 + (size_t(t[k] - a.T8) * KT + 2 * grp) * 512 + 16 * lane, sb);
      }
      gdma4_once(a.s + (size_t(t[k]) * G + grp) * 16 + 2 * (lane & 7), st + C::kA + C::kB + slot * 256);
      if constexpr (Q4)
        gdma4_once(a.z + (size_t(t[k] - a.T8) * G + grp) * 16 + 4 * (lane & 3),
                   st + C::kA + C::kB + C::kS + slot * 256);
    }
    if constexpr (SA)   // lane m: the scales of groups (grp & ~1) and (grp | 1) of token m
      gdma4(a.xs + size_t(min(lane, a.M - 1)) * G + (grp & ~1), st + C::kA + C::kB + C::kS + C::kZ + wave * 256);
  };

  f32x4 tot[TW][TM];
  // the previous group's int32 sums and weight scales: they are scaled into
  // tot while the current group's MFMAs run, so no step waits for its own
  // matrix-core results
  i32x4 cp[TW][TM];
  float swp[TW];
#pragma unroll
  for (int k = 0; k < TW; ++k) {
    swp[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      tot[k][i] = f32x4{0, 0, 0, 0};
      cp[k][i] = i32x4{0, 0, 0, 0};
    }
  }
  f32x4 sap[TM];   // GA: the previous group's activation scales of this lane's outputs
#pragma unroll
  for (int i = 0; i < TM; ++i) sap[i] = f32x4{0, 0, 0, 0};
  // Offset sums with per-token scales and four token tiles, as in the tile
  // kernel: a group's MFMAs start from the bits of 1.5 2^23, one fma scales
  // each sum, and the offsets come off after every second scaled group and
  // after the last.  (With one or two token tiles the saved conversions do
  // not pay for the subtractions: 28672 x 8192 at M = 1 took 31 us against
  // 28, M = 64 53 against 57.)
  constexpr bool kOff = !GA && !ACC && TM == 4;
  const i32x4 cinit = kOff ? i32x4{kOffI, kOffI, kOffI, kOffI} : i32x4{0, 0, 0, 0};
  float pend[TW];   // scales whose offsets are still in tot
#pragma unroll
  for (int k = 0; k < TW; ++k) pend[k] = 0.0f;
  // tot += the previous group's sums times their scales
  auto scale_prev = [&]() {
#pragma unroll
    for (int k = 0; k < TW; ++k)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if constexpr (kOff) {
            const int32_t e = cp[k][i][v];   // (a bit cast of the vector element itself reads element 0)
            tot[k][i][v] = __builtin_fmaf(__builtin_bit_cast(float, e), swp[k], tot[k][i][v]);
          } else {
            tot[k][i][v] = __builtin_fmaf(float(cp[k][i][v]), GA ? swp[k] * sap[i][v] : swp[k], tot[k][i][v]);
          }
        }
    if constexpr (kOff) {
#pragma unroll
      for (int k = 0; k < TW; ++k) pend[k] += swp[k];
    }
  };
  auto drop_offsets = [&]() {
#pragma unroll
    for (int k = 0; k < TW; ++k) {
      const float off = kOffF * pend[k];
      pend[k] = 0.0f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) tot[k][i][v] -= off;
    }
  };

  // ACC: this lane's original row (-1: none), loaded and awaited before the
  // first global->LDS load, so no later wait of the compiler's covers them
  int n_acc[TW];
#pragma unroll
  for (int k = 0; k < TW; ++k) n_acc[k] = -1;
  if constexpr (ACC) {
#pragma unroll
    for (int k = 0; k < TW; ++k)
      if (t0 + wave + 4 * k < tend) n_acc[k] = a.rows[16 * (t0 + wave + 4 * k) + r16];
    wait_vm<0>();
  }
  for (int p = 0; p < kStages - 1 && p < ng; ++p) issue(p);
  for (int j = 0; j < ng; ++j) {
    const int grp = g0 + j;
    // this wave's loads of step j have landed once at most the loads of the
    // (up to kStages - 2) later steps are in flight
    static_assert(kStages - 2 <= 3, "wait cases");
    const int later = min(ng - 1 - j, kStages - 2);
    if (later >= 3)
      wait_vm<3 * kLoads>();
    else if (later == 2)
      wait_vm<2 * kLoads>();
    else if (later == 1)
      wait_vm<kLoads>();
    else
      wait_vm<0>();
    __syncthreads();   // every wave's loads of step j landed; every wave is done with j - 1
    if (j + kStages - 1 < ng) issue(j + kStages - 1);   // into step j - 1's stage
    // every LDS read of the step first, then one wait
    const uint8_t* st = base + stage(j);
    i32x4 av[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) av[i][h] = *reinterpret_cast<const i32x4*>(st + (2 * i + h) * 1024 + 16 * lane);
    float sw[TW];
#pragma unroll
    for (int k = 0; k < TW; ++k)
      sw[k] = (float)reinterpret_cast<const _Float16*>(st + C::kA + C::kB + (TW * wave + k) * 256)[r16];
    f32x4 sac[TM];   // GA: this group's activation scales of the lane's outputs (token 16 i + 4 g + v)
    if constexpr (SA) {
      const _Float16* X = reinterpret_cast<const _Float16*>(st + C::kA + C::kB + C::kS + C::kZ + wave * 256);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) sac[i][v] = (float)X[2 * (16 * i + 4 * g + v) + (grp & 1)];
    }
    i32x4 bv[TW][2];
#pragma unroll
    for (int k = 0; k < TW; ++k) {
      const uint8_t* B = st + C::kA + (TW * wave + k) * 2048;
      if constexpr (!Q4) {
        bv[k][0] = *reinterpret_cast<const i32x4*>(B + 16 * lane);
        bv[k][1] = *reinterpret_cast<const i32x4*>(B + 1024 + 16 * lane);
      } else {
        const uint2 w0 = *reinterpret_cast<const uint2*>(B + 8 * lane);
        const uint2 w1 = *reinterpret_cast<const uint2*>(B + 512 + 8 * lane);
        const uint32_t z = st[C::kA + C::kB + C::kS + (TW * wave + k) * 256 + r16];
        const uint32_t zb = (128u - z) * 0x01010101u;
        bv[k][0] = expand4(w0, zb);
        bv[k][1] = expand4(w1, zb);
      }
    }
    i32x4 c[TW][TM];
#pragma unroll
    for (int k = 0; k < TW; ++k)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        c[k][i] = mfma16_i8(av[i][0], bv[k][0], cinit);
        c[k][i] = mfma16_i8(av[i][1], bv[k][1], c[k][i]);
      }
    if constexpr (ACC) {
      // the group sums as they are, at their original rows (stores add to the
      // vector-memory count, which only makes the fixed waits above stricter)
#pragma unroll
      for (int k = 0; k < TW; ++k) {
        if (n_acc[k] < 0) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = 16 * i + 4 * g + v;
            if (m < a.M) a.acc_out[(size_t(m) * a.N + n_acc[k]) * G + grp] = c[k][i][v];
          }
      }
      continue;
    }
    scale_prev();   // group j - 1 (at j = 0 zero sums with zero scales)
    if constexpr (kOff)
      if (j >= 2 && (j & 1) == 0) drop_offsets();   // groups j - 2 and j - 1
#pragma unroll
    for (int k = 0; k < TW; ++k) {
#pragma unroll
      for (int i = 0; i < TM; ++i) cp[k][i] = c[k][i];
      swp[k] = sw[k];
    }
    if constexpr (SA) {
#pragma unroll
      for (int i = 0; i < TM; ++i) sap[i] = sac[i];
    }
  }
  if constexpr (ACC) return;
  scale_prev();   // the last group
  if constexpr (kOff) drop_offsets();

#pragma unroll
  for (int k = 0; k < TW; ++k) {
    const int tk = t0 + wave + 4 * k;
    if (tk >= tend) continue;
    const int n = a.rows[16 * tk + r16];
    if (n < 0) continue;
    if (a.part) {
      // this segment's partial sums, at the packed row; w48_reduce_kernel
      // adds the segments, applies the activation scale and scatters
      const int P = 16 * (a.T8 + a.T4), pr = 16 * tk + r16;
      float* pp = a.part + size_t(seg) * size_t(a.M) * size_t(P);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 16 * i + 4 * g + v;
          if (m < a.M) pp[size_t(m) * P + pr] = tot[k][i][v];
        }
      continue;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * i + 4 * g + v;
        if (m < a.M) a.y[size_t(m) * a.N + n] = (_Float16)(GA ? tot[k][i][v] : tot[k][i][v] * (float)a.xs[m]);
      }
  }
}

template <int TM, bool GA, bool ACC, int TW>
__global__ __launch_bounds__(256) void w48_stream_kernel(W48Args a) {
  using C = StreamCfg<TM, GA && !ACC, TW>;
  __shared__ u32x4 lds[C::kStages * C::kStage / 16];
  uint8_t* const base = reinterpret_cast<uint8_t*>(lds);
  // workgroup = (K segment, row block of 4 TW packed tiles): the 8-bit row
  // blocks' kseg8 segments first, then the 4-bit row blocks' kseg4
  constexpr int RB = 4 * TW;
  const int nb8 = (a.T8 + RB - 1) / RB, nb4 = (a.T4 + RB - 1) / RB, w8 = nb8 * a.kseg8, b = int(blockIdx.x);
  if (b < w8) {
    stream_tiles<TM, GA, false, ACC, TW>(a, base, (b % nb8) * RB, a.T8, b / nb8, a.seg8);
  } else {
    const int c = b - w8;
    stream_tiles<TM, GA, true, ACC, TW>(a, base, a.T8 + (c % nb4) * RB, a.T8 + a.T4, c / nb4, a.seg4);
  }
}

// For every token m and packed row p of original row n = rows[p] >= 0:
// y[m][n] = fp16(s_a[m] * (the partial sums of [m][p] over the row's
// segments -- kseg8 for the 8-bit rows (p < P8), kseg4 for the others --
// added in segment order, so the result does not depend on the order the
// segments ran in)).  The partials read are cleared, which leaves the
// workspace zero.  One element per thread; the row index, the scale and all
// of the partials are loaded before anything waits (a padding row's
// partials are in bounds and zero), so the loads overlap.
__global__ __launch_bounds__(256) void w48_reduce_kernel(float* part, const int32_t* rows, const _Float16* xs,
                                                         _Float16* y, int M, int N, int P, int P8, int kseg8,
                                                         int kseg4, int per_token) {
  const size_t plane = size_t(M) * size_t(P);
  const size_t e = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= plane) return;
  const int m = int(e / size_t(P)), p = int(e % size_t(P));
  const int k = p < P8 ? kseg8 : kseg4;
  const int n = rows[p];
  const float sa = per_token ? (float)xs[m] : 1.0f;   // per-group scales are inside the partials
  float v[16];
#pragma unroll
  for (int sg = 0; sg < 16; ++sg) v[sg] = sg < k ? part[size_t(sg) * plane + e] : 0.0f;
  if (n < 0) return;
  float t = v[0];
#pragma unroll
  for (int sg = 1; sg < 16; ++sg)
    if (sg < k) t += v[sg];
#pragma unroll
  for (int sg = 0; sg < 16; ++sg)
    if (sg < k) part[size_t(sg) * plane + e] = 0.0f;
  y[size_t(m) * size_t(N) + n] = (_Float16)(t * sa);
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
  a.part = nullptr;
  a.kseg8 = a.kseg4 = 1;
  a.seg8 = a.seg4 = im.K / 128;
  a.tiles = 1;
  a.tt = 8;
  return a;
}

template <bool GA, bool ACC>
void launch_stream_ga(const W48Args& a, hipStream_t s) {
  const int RB = 4 * a.tiles;   // packed tiles per workgroup
  const dim3 grid(unsigned((a.T8 + RB - 1) / RB * a.kseg8 + (a.T4 + RB - 1) / RB * a.kseg4));
  if (a.tiles == 2) {
    if (a.M <= 16)
      hipLaunchKernelGGL((w48_stream_kernel<1, GA, ACC, 2>), grid, dim3(256), 0, s, a);
    else if (a.M <= 32)
      hipLaunchKernelGGL((w48_stream_kernel<2, GA, ACC, 2>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((w48_stream_kernel<4, GA, ACC, 2>), grid, dim3(256), 0, s, a);
  } else {
    if (a.M <= 16)
      hipLaunchKernelGGL((w48_stream_kernel<1, GA, ACC, 1>), grid, dim3(256), 0, s, a);
    else if (a.M <= 32)
      hipLaunchKernelGGL((w48_stream_kernel<2, GA, ACC, 1>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((w48_stream_kernel<4, GA, ACC, 1>), grid, dim3(256), 0, s, a);
  }
  if (!ACC && a.part) {
    const int P = 16 * (a.T8 + a.T4);
    const size_t total = size_t(a.M) * size_t(P);
    hipLaunchKernelGGL(w48_reduce_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, a.part, a.rows,
                       a.xs, a.y, a.M, a.N, P, 16 * a.T8, a.kseg8, a.kseg4, GA ? 0 : 1);
  }
}

template <bool ACC>
void launch_stream(const W48Args& a, hipStream_t s) {
  if (a.ga == 128)
    launch_stream_ga<true, ACC>(a, s);
  else
    launch_stream_ga<false, ACC>(a, s);
}

template <int TT, bool ACC>
void launch_tile_tt(const W48Args& a, hipStream_t s) {
  const int ntm = (a.M + 16 * TT - 1) / (16 * TT), nrb8 = (a.T8 + 3) / 4, nrb4 = (a.T4 + 7) / 8;
  const int per_xcd = (ntm * (nrb8 * a.kseg8 + nrb4 * a.kseg4) + 7) / 8;
  const dim3 grid(unsigned(8 * per_xcd));
  // per-group scales staged in LDS when they can be loaded two groups at a time
  const bool xs_lds = (a.K / 128) % 2 == 0 && reinterpret_cast<uintptr_t>(a.xs) % 4 == 0;
  if (a.ga == 128 && xs_lds)
    hipLaunchKernelGGL((w48_tile_kernel<TT, true, ACC, true>), grid, dim3(256), 0, s, a, ntm, nrb8, nrb4, per_xcd);
  else if (a.ga == 128)
    hipLaunchKernelGGL((w48_tile_kernel<TT, true, ACC, false>), grid, dim3(256), 0, s, a, ntm, nrb8, nrb4, per_xcd);
  else
    hipLaunchKernelGGL((w48_tile_kernel<TT, false, ACC, false>), grid, dim3(256), 0, s, a, ntm, nrb8, nrb4, per_xcd);
}

template <bool ACC>
void launch_tile(const W48Args& a, hipStream_t s) {
  if (a.tt == 4)
    launch_tile_tt<4, ACC>(a, s);
  else
    launch_tile_tt<8, ACC>(a, s);
  if (!ACC && a.part) {
    const int P = 16 * (a.T8 + a.T4);
    const size_t total = size_t(a.M) * size_t(P);
    hipLaunchKernelGGL(w48_reduce_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, a.part, a.rows,
                       a.xs, a.y, a.M, a.N, P, 16 * a.T8, a.kseg8, a.kseg4, a.ga == 128 ? 0 : 1);
  }
}

}  // namespace

namespace {

// Segment sizes for k8 (k4) segments of the 8-bit (4-bit) row blocks, with
// fewer segments when ws_bytes cannot hold the fp32 partials (segments x M
// x packed rows).
W48Split split_for(int k8, int k4, int K, int T8, int T4, int M, size_t ws_bytes) {
  const int G = K / 128;
  const size_t P = size_t(16) * size_t(T8 + T4);
  auto need = [&](int kk) { return kk > 1 ? size_t(kk) * size_t(M) * P * 4 : size_t(0); };
  int kmax = max(k8, k4);
  while (kmax > 1 && need(kmax) > ws_bytes) {
    k8 = min(k8, kmax - 1);
    k4 = min(k4, kmax - 1);
    kmax = max(k8, k4);
  }
  W48Split p;
  p.seg8 = (G + k8 - 1) / k8;
  p.kseg8 = (G + p.seg8 - 1) / p.seg8;
  p.seg4 = (G + k4 - 1) / k4;
  p.kseg4 = (G + p.seg4 - 1) / p.seg4;
  p.ws_bytes = need(max(p.kseg8, p.kseg4));
  p.tiles = 1;
  p.tt = 8;
  return p;
}

}  // namespace

// The stream kernel's K split for a pass of M <= 64 tokens.  An 8-bit row
// block streams twice the bytes of a 4-bit one.  Counting it twice, when the
// row blocks of one tile per wave (64 rows) number at most 3/4 of the CUs,
// the kernel takes two tiles per wave (128-row blocks, so each workgroup's
// activation fragments serve twice the weights), and each row block's
// groups are cut into segments of at least 8 groups (1024 columns), at most
// 16, so that the workgroups, two per CU, stream about equal bytes: an
// 8-bit row block takes twice the segments of a 4-bit one.  (With more row
// blocks the second launch costs more than the extra workgroups gain:
// 14336 x 4096 at M = 64, 248 units, ran 25 us split against 22 us; and
// 128-row blocks without a split leave CUs idle: 28672 x 8192 at M = 1, 30
// against 35 us.)  With fewer than ws_bytes for the fp32 partials
// (segments x M x packed rows), fewer segments.
W48Split w48_split(int K, int T8, int T4, int M, size_t ws_bytes) {
  const int G = K / 128, cus = device_compute_units();
  const int kcap = max(1, min(16, G / 8));
  int k8 = 1, k4 = 1, tiles = 1;
  if (4 * (2 * ((T8 + 3) / 4) + (T4 + 3) / 4) <= 3 * cus) {
    tiles = 2;
    const int nb8 = (T8 + 7) / 8, nb4 = (T4 + 7) / 8;
    if (nb4) {
      k4 = max(1, min(kcap, 2 * cus / (2 * nb8 + nb4)));
      k8 = nb8 ? min(kcap, 2 * k4) : 1;
    } else {
      k8 = max(1, min(kcap, 2 * cus / nb8));
    }
  }
  W48Split p = split_for(k8, k4, K, T8, T4, M, ws_bytes);
  // without a split (too little workspace), 64-row blocks fill more CUs
  p.tiles = p.kseg8 > 1 || p.kseg4 > 1 ? tiles : 1;
  return p;
}

// The tile kernel's token tile for an unsplit launch.  Its workgroups run
// in rounds of the resident slots (three 128-token or four 64-token
// workgroups per CU with per-token activation scales), and a 4-bit row
// block's workgroup takes about twice as long as an 8-bit one's.  A round
// only partly filled still costs a whole workgroup's time (28672 x 8192 at
// M = 512: 808 4-bit workgroups for 768 slots).  At full occupancy a 64-token
// workgroup takes about 6/8 of the time of a 128-token one (each 4-bit
// expansion and weight load serves half as many MFMAs), so 64-token tiles are
// taken when their rounds end sooner by that measure.  With per-group
// activation scales the 128-token tile was measured at two workgroups per
// CU against four 64-token ones of about the same duration each: there
// 64-token tiles are taken unless the launch runs eight rounds or more of
// 128-token tiles, where the two are within a few per cent.
// Measured on 28672 x 8192 and 8192 x 28672, M = 129 ... 4096 (both tiles
// give bit-identical outputs).
static int tile_token_tiles(int T8, int T4, int M, int ga) {
  const int cus = device_compute_units();
  const long u = long((T8 + 3) / 4) + 2L * long((T4 + 7) / 8);   // row blocks in 8-bit units
  auto rounds = [&](int tt) {
    const long units = long((M + 16 * tt - 1) / (16 * tt)) * u;
    const long slots2 = 2L * tile_wgs_per_cu(tt, ga == 128) * cus;
    return (units + slots2 - 1) / slots2;
  };
  if (ga == 128) return rounds(8) < 8 ? 4 : 8;
  return 6L * rounds(4) < 8L * rounds(8) ? 4 : 8;
}

// The tile kernel's K split (M > 64).  A 4-bit row block (128 rows) does
// twice the matrix-core work of an 8-bit one (64 rows).  Counting it twice,
// when the token tiles x row blocks fill at most half of the resident
// workgroup slots (three per CU, two with per-group activation scales),
// each row block's groups are cut into segments of at least 8 groups, at
// most 16, about enough to fill those slots, a 4-bit row block into twice
// as many as an 8-bit one.  (Above half, the partials' round trip through
// memory costs more than the extra workgroups gain: 14336 x 4096 at M = 256
// ran 64 us split against 56 us.)  With fewer than ws_bytes for the
// partials, fewer segments.
W48Split w48_tile_split(int K, int T8, int T4, int M, int ga, size_t ws_bytes) {
  const int ntm = (M + kTB - 1) / kTB, nrb8 = (T8 + 3) / 4, nrb4 = (T4 + 7) / 8, G = K / 128;
  const int slots = (ga == 128 ? 2 : 3) * device_compute_units();
  const int kcap = max(1, min(16, G / 8));
  const int u = ntm * (nrb8 + 2 * nrb4);
  int k8 = 1, k4 = 1;
  if (2 * u <= slots) {
    if (nrb8) {
      k8 = max(1, min(kcap, slots / u));
      k4 = min(kcap, 2 * k8);
    } else {
      k4 = max(1, min(kcap, slots / (ntm * nrb4)));
    }
  }
  W48Split p = split_for(k8, k4, K, T8, T4, M, ws_bytes);
  if (p.kseg8 == 1 && p.kseg4 == 1) p.tt = tile_token_tiles(T8, T4, M, ga);
  return p;
}

// Whether (M, ga) runs the stream kernel, in one pass (M <= 64) or in 64-token
// passes (M <= 128 where the tile kernel's single row of workgroups would
// leave CUs idle).  Per-group activation scales need an even group count
// (their loads take two groups' scales at a time) and take one pass only:
// their scaling makes the stream kernel slower than the tile kernel at two
// passes (28672 x 8192 at M = 96: 127 against 118 us).
bool w48_streams(int K, int T8, int T4, int M, int ga) {
  if (ga == 128) return M <= 64 && (K / 128) % 2 == 0;
  if (M > 128) return false;
  return M <= 64 || (T8 + 3) / 4 + (T4 + 7) / 8 <= device_compute_units();
}

namespace {

// Picks the kernel for (M, ga).  A call with a.acc_out set takes the same
// route with the kernel's group-sum store in place of its scaling step, so
// the exported int32 sums are those of the kernel that runs the product; it
// takes the K split of a call with workspace enough for it (the group sums do
// not depend on the split, but the segment bounds are then exercised).
int launch(const W48Args& a0, void* workspace, size_t ws_bytes, void* stream) {
  W48Args a = a0;
  const int T = a.T8 + a.T4;
  const unsigned gy = unsigned((T + 4 * kNT - 1) / (4 * kNT));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool acc = a.acc_out != nullptr;
  // per-group activation scales are loaded two groups (4 bytes) at a time
  const bool xs_ok = a.ga != 128 || reinterpret_cast<uintptr_t>(a.xs) % 4 == 0;
  if (a.M > 64 && xs_ok && w48_streams(a.K, a.T8, a.T4, a.M, a.ga)) {
    // Here the tile kernel's single row of workgroups leaves CUs idle, and
    // two 64-token passes of the stream kernel, which reads the weights at
    // HBM speed (and splits K where its own grid is small), are faster even
    // than the tile kernel split (8192 x 28672 at M = 128: 134 against
    // 175 us).  A token range is a self-contained call (its rows of the
    // activation scales, per token or per group, come with it); the passes
    // run one after the other on the stream, so they share the workspace.
    W48Args c = a;
    for (int m0 = 0; m0 < a.M; m0 += 64) {
      c.M = a.M - m0 < 64 ? a.M - m0 : 64;
      c.xq = a.xq + size_t(m0) * size_t(a.K);
      c.xs = a.xs ? a.xs + size_t(m0) * size_t(a.ga == 128 ? a.K / 128 : 1) : nullptr;
      c.y = a.y ? a.y + size_t(m0) * size_t(a.N) : nullptr;
      c.acc_out = acc ? a.acc_out + size_t(m0) * size_t(a.N) * size_t(a.K / 128) : nullptr;
      const int rc = launch(c, workspace, ws_bytes, stream);
      if (rc != 0) return rc;
    }
    return 0;
  }
  if (a.M <= 64 && xs_ok && w48_streams(a.K, a.T8, a.T4, a.M, a.ga)) {
    const W48Split sp = w48_split(a.K, a.T8, a.T4, a.M, acc ? SIZE_MAX : workspace ? ws_bytes : 0);
    a.kseg8 = sp.kseg8;
    a.seg8 = sp.seg8;
    a.kseg4 = sp.kseg4;
    a.seg4 = sp.seg4;
    a.tiles = sp.tiles;
    if (!acc && (sp.kseg8 > 1 || sp.kseg4 > 1)) a.part = static_cast<float*>(workspace);
    if (acc)
      launch_stream<true>(a, s);
    else
      launch_stream<false>(a, s);
  } else if (a.M > 64) {
    const W48Split sp = w48_tile_split(a.K, a.T8, a.T4, a.M, a.ga, acc ? SIZE_MAX : workspace ? ws_bytes : 0);
    a.kseg8 = sp.kseg8;
    a.seg8 = sp.seg8;
    a.kseg4 = sp.kseg4;
    a.seg4 = sp.seg4;
    a.tt = sp.tt;
    if (!acc && (sp.kseg8 > 1 || sp.kseg4 > 1)) a.part = static_cast<float*>(workspace);
    if (acc)
      launch_tile<true>(a, s);
    else
      launch_tile<false>(a, s);
  } else if (a.M <= 32) {   // group activation scales over an odd number of groups, M <= 64
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
               void* workspace, size_t ws_bytes, void* stream) {
  return launch(make_args(im, xq, xs, ga, y, nullptr, M), workspace, ws_bytes, stream);
}

int launch_w48_acc(const W48ImageView& im, const int8_t* xq, int ga, int32_t* acc, int M, void* stream) {
  return launch(make_args(im, xq, nullptr, ga, nullptr, acc, M), nullptr, 0, stream);
}

}  // namespace gbb
