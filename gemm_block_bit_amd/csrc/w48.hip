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

int launch(const W48Args& a, void* stream) {
  const int T = a.T8 + a.T4;
  const unsigned gy = unsigned((T + 4 * kNT - 1) / (4 * kNT));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.M <= 32) {
    hipLaunchKernelGGL(w48_kernel<32>, dim3(unsigned((a.M + 31) / 32), gy), dim3(256), 0, s, a);
  } else if (a.M <= 64) {
    hipLaunchKernelGGL(w48_kernel<64>, dim3(unsigned((a.M + 63) / 64), gy), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(w48_kernel<128>, dim3(unsigned((a.M + 127) / 128), gy), dim3(256), 0, s, a);
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

int launch_w48_acc(const W48ImageView& im, const int8_t* xq, int32_t* acc, int M, void* stream) {
  return launch(make_args(im, xq, nullptr, im.K, nullptr, acc, M), stream);
}

}  // namespace gbb
