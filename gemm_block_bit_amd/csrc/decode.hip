// Decode kernel: y = x . dequant(W)^T for M <= 32 over the block image.
//
// What it computes follows the ScaleBITS explainer page (section 1.2.2: each
// 64x128 block has one bitwidth so no per-element branching is needed; section
// 3.2: dequantization fused into the product, blocks handled independently)
// and the affine dequantization (q - z) * s of the MixLLM page, section 2.1.
//
// gfx950 design:
//  * one wave owns one 64-row block row and walks a segment of its 128-column
//    blocks; the bitwidth is read once per block as a scalar, so the switch on
//    it is wave-uniform;
//  * the codes of a block are b KiB; every KiB is one 16-byte load per lane,
//    fully coalesced, and holds exactly the lane's share of the A operands of
//    the 16 v_mfma_f32_16x16x32_f16 tiles of the block (16 rows x 32 columns);
//  * unpacking is one AND (plus a shift) and one OR per code pair: the code
//    lands in the mantissa of fp16 1024.0, giving the value 1024 + q;
//  * the matrix cores form C = sum_k x_k (1024 + q_k) per 16-row tile and
//    group (x is the B operand, one column per token), and a fifth MFMA
//    against all-ones forms X = sum_k x_k; the group epilogue then adds
//    s * (C - (1024 * bias_planes + z) * X) = s * sum_k x_k (q_k - z) to the
//    fp32 accumulator with two fused multiply-adds per output;
//  * K is split into segments when that is needed to fill the GPU; partial
//    sums go to fp32 workspace through device-scope stores and the last
//    workgroup of each row group (an atomic counter that resets itself) adds
//    them in segment order, so results are deterministic.
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

struct DecodeArgs {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  const _Float16* x;
  _Float16* y;
  float* part;
  uint32_t* ctr;
  int N, K, M, nbr, nbc, seg_len, nseg;
};

// One block with planes of width W0 (shift 0) and W1 (shift W0; 0 = none).
template <int W0, int W1, int MT>
__device__ __forceinline__ void decode_block(const uint8_t* __restrict__ cb, const half8 (&xf)[4][MT],
                                             const float (&xsum)[MT], const u32x4 (&szv)[4],
                                             f32x4 (&acc)[4][MT]) {
  constexpr int NP0 = 16 / W0;
  constexpr int NP1 = W1 ? 16 / W1 : 1;
  uint32_t w0[4 * W0];
  uint32_t w1[4 * (W1 ? W1 : 1)];
#pragma unroll
  for (int t = 0; t < W0; ++t) {
    const u32x4 v = ld16(cb + 1024 * t);
    w0[4 * t] = v[0], w0[4 * t + 1] = v[1], w0[4 * t + 2] = v[2], w0[4 * t + 3] = v[3];
  }
  if constexpr (W1 != 0) {
#pragma unroll
    for (int t = 0; t < W1; ++t) {
      const u32x4 v = ld16(cb + 1024 * (W0 + t));
      w1[4 * t] = v[0], w1[4 * t + 1] = v[1], w1[4 * t + 2] = v[2], w1[4 * t + 3] = v[3];
    }
  }
  // sum over planes of 2^shift * 1024: the bias every code carries
  constexpr float kBias = 1024.0f * (1.0f + (W1 ? float(1 << W0) : 0.0f));
  constexpr float kHi = float(1 << W0);
  float biasx[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) biasx[mt] = kBias * xsum[mt];

#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f32x4 c0[MT], c1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) c0[mt] = f32x4{0, 0, 0, 0}, c1[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int u = 4 * rt + kt;
      uint32_t a[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int P = 4 * u + p;
        a[p] = pair_bits<W0>(w0[P / NP0], P % NP0) | kMagicPair;
      }
      const half8 A = as_half8(a[0], a[1], a[2], a[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) c0[mt] = mfma16(A, xf[kt][mt], c0[mt]);
      if constexpr (W1 != 0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int P = 4 * u + p;
          a[p] = pair_bits<W1>(w1[P / NP1], P % NP1) | kMagicPair;
        }
        const half8 B = as_half8(a[0], a[1], a[2], a[3]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) c1[mt] = mfma16(B, xf[kt][mt], c1[mt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t e = szv[rt][v];
        const float corr = __builtin_fmaf(hi_half(e), xsum[mt], biasx[mt]);
        const float c = W1 ? __builtin_fmaf(kHi, c1[mt][v], c0[mt][v]) : c0[mt][v];
        acc[rt][mt][v] = __builtin_fmaf(lo_half(e), c - corr, acc[rt][mt][v]);
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int rg = blockIdx.x / a.nseg, seg = blockIdx.x - rg * a.nseg;
  const int br = rg * 4 + wave;
  const int c_begin = seg * a.seg_len;
  const int c_end = min(a.nbc, c_begin + a.seg_len);

  f32x4 acc[4][MT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0, 0, 0, 0};

  const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
  if (br < a.nbr) {
    for (int bc = c_begin; bc < c_end; ++bc) {
      const int blk = br * a.nbc + bc;
      const int b = uniform(a.bits[blk]);
      const uint32_t off = uint32_t(uniform(int(a.offs[blk])));
      half8 xf[4][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r16;
        const _Float16* xp = a.x + size_t(m) * a.K + size_t(bc) * 128 + 8 * g;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          u32x4 v = {0, 0, 0, 0};
          if (m < a.M) v = ld16(xp + 32 * kt);
          xf[kt][mt] = __builtin_bit_cast(half8, v);
        }
      }
      u32x4 szv[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) szv[rt] = ld16(a.sz + size_t(blk) * 64 + 16 * rt + 4 * g);
      float xsum[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 s = {0, 0, 0, 0};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s = mfma16(ones, xf[kt][mt], s);
        xsum[mt] = s[0];
      }
      const uint8_t* cb = a.codes + size_t(off) * 1024 + 16 * lane;
      switch (b) {
        case 1: decode_block<1, 0, MT>(cb, xf, xsum, szv, acc); break;
        case 2: decode_block<2, 0, MT>(cb, xf, xsum, szv, acc); break;
        case 3: decode_block<2, 1, MT>(cb, xf, xsum, szv, acc); break;
        case 4: decode_block<4, 0, MT>(cb, xf, xsum, szv, acc); break;
        case 6: decode_block<4, 2, MT>(cb, xf, xsum, szv, acc); break;
        default: decode_block<4, 4, MT>(cb, xf, xsum, szv, acc); break;
      }
    }
  }

  // lane holds D[row 16 rt + 4 g + v][token 16 mt + r16]
  const int nrow = br * 64 + 4 * g;
  if (a.nseg == 1) {
    if (br < a.nbr) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r16;
        if (m >= a.M) continue;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          _Float16* yp = a.y + size_t(m) * a.N + nrow + 16 * rt;
          half2v lo = {(_Float16)acc[rt][mt][0], (_Float16)acc[rt][mt][1]};
          half2v hi = {(_Float16)acc[rt][mt][2], (_Float16)acc[rt][mt][3]};
          *reinterpret_cast<uint2*>(yp) = make_uint2(as_u32(lo), as_u32(hi));
        }
      }
    }
    return;
  }

  // Split K: hand the partial sums over through device-scope (sc1) atomic
  // stores and loads, which are coherent across the XCDs' L2 caches without
  // writing back or invalidating whole caches.  The barrier waits for every
  // store of the workgroup to complete before one lane bumps the row group's
  // counter; the workgroup that brings it to nseg sums the partials in
  // segment order and resets the counter for the next call.
  if (br < a.nbr) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + r16;
      if (m >= a.M) continue;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        float* pp = a.part + (size_t(seg) * a.M + m) * a.N + nrow + 16 * rt;
#pragma unroll
        for (int v = 0; v < 4; ++v) __hip_atomic_store(pp + v, acc[rt][mt][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __shared__ int s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.ctr + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == uint32_t(a.nseg - 1);
    if (last) __hip_atomic_store(a.ctr + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int n = rg * 256 + threadIdx.x;
  if (n >= a.N) return;
  for (int m = 0; m < a.M; ++m) {
    float s = 0.0f;
    for (int sg = 0; sg < a.nseg; ++sg)
      s += __hip_atomic_load(a.part + (size_t(sg) * a.M + m) * a.N + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.y[size_t(m) * a.N + n] = (_Float16)s;
  }
}

DecodePlan decode_plan(int N, int K, int M) {
  DecodePlan p;
  const int nbr = N / 64, nbc = K / 128;
  p.nrg = (nbr + 3) / 4;
  // aim for about 1024 workgroups (4 per CU); cap the split by the partial-sum
  // traffic it adds (nseg * M * N * 8 bytes against about N * K / 2 of codes)
  const int want = 1024;
  int nseg = (want + p.nrg - 1) / p.nrg;
  const int cap = max(1, K / (64 * M));
  nseg = max(1, min(min(nseg, cap), nbc));
  p.seg_len = (nbc + nseg - 1) / nseg;
  p.nseg = (nbc + p.seg_len - 1) / p.seg_len;
  if (p.nseg > 1) {
    // the counters sit in a fixed region at the start of every workspace, so
    // one zero-filled buffer serves calls of any shape: partial sums of one
    // call never land where another call's counters live
    p.ctr_bytes = kCounterBytes;
    p.part_bytes = size_t(p.nseg) * size_t(M) * size_t(N) * 4;
  } else {
    p.ctr_bytes = p.part_bytes = 0;
  }
  return p;
}

int launch_decode(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* workspace,
                  const DecodePlan& plan, void* stream) {
  DecodeArgs a;
  a.bits = im.bits;
  a.offs = im.offs;
  a.sz = im.sz;
  a.codes = im.codes;
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.ctr = static_cast<uint32_t*>(workspace);
  a.part = plan.nseg > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ctr_bytes) : nullptr;
  a.N = im.N;
  a.K = im.K;
  a.M = M;
  a.nbr = im.nbr;
  a.nbc = im.nbc;
  a.seg_len = plan.seg_len;
  a.nseg = plan.nseg;
  const dim3 grid(unsigned(plan.nrg * plan.nseg)), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= 16)
    hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, s, a);
  return int(hipGetLastError());
}

const char* device_error_text(int err) {
  return err == 0 ? nullptr : hipGetErrorString(hipError_t(err));
}

}  // namespace gbb
