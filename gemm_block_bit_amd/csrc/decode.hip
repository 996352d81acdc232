// Decode kernel: y = x . dequant(W)^T for M <= 32 over the block image.
//
// What it computes follows the ScaleBITS explainer page (section 1.2.2: each
// 64x128 block has one bitwidth so no per-element branching is needed; section
// 3.2: dequantization fused into the product, blocks handled independently)
// and the affine dequantization (q - z) * s of the MixLLM page, section 2.1.
//
// gfx950 design
//  * A workgroup owns one 64-row block row (and, only when the matrix has too
//    few block rows to fill the GPU, one of a few K segments of it).  Its
//    waves split the block columns; their sums meet in LDS and are added in a
//    fixed order.
//  * A block of bitwidth b is b KiB of codes: b coalesced 16-byte loads per
//    lane, each holding exactly the lane's codes for the B operands of
//    v_mfma_f32_16x16x32_f16 (32 columns x 16 rows per tile, 16 tiles per
//    block; b = 3, 6, 8 are split into planes of widths 2+1, 4+2, 4+4).  The
//    bitwidth is read once per block as a scalar, so the switch on it is
//    wave-uniform.
//  * Each wave runs a two-stage pipeline over its work units (one bit plane
//    of one block, at most 4 KiB): the activations, scales/zeros and codes of
//    the next unit are loaded while the current unit is computed.
//  * Unpacking is one AND (plus a shift) and one OR per code pair: the code
//    lands in the mantissa of fp16 1024.0, giving 1024 + q exactly.  The
//    matrix cores form C = sum_k x_k (1024 + q_k) per 16-row tile and group
//    (x is the A operand, one row per token) and X = sum_k x_k against an
//    all-ones B operand; the epilogue adds s (C - (1024 bias + z) X) to fp32
//    accumulators, which equals s sum_k x_k (q_k - z).
//  * With K segments, partial sums cross workgroups (and XCDs) through
//    device-scope (sc1) stores and loads, which need no cache writeback; the
//    last workgroup of a block row (an atomic counter that resets itself)
//    adds them in segment order, so results are deterministic.
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

namespace {

struct DecodeArgs {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  const _Float16* x;
  _Float16* y;
  float* part;
  uint32_t* ctr;
  int N, K, M, nbr, nbc, seg_cols, nseg;
};

__device__ __forceinline__ int plane0_w(int b) { return b == 3 ? 2 : (b >= 4 ? 4 : b); }
__device__ __forceinline__ int plane1_w(int b) { return b == 3 ? 1 : (b == 6 ? 2 : (b == 8 ? 4 : 0)); }

// registers of one work unit (one bit plane of one block) in flight
template <int MT>
struct UnitBuf {
  u32x4 code[4];     // the plane's w KiB of codes (lane's 16 bytes of each)
  uint32_t sz[4];    // fp16 s | fp16 z << 16 of row 16 rt + r16
  half8 xa[4][MT];   // A operands: x[16 mt + r16][32 kt + 8 g .. + 7]
};

// Loads of one unit: activations and scales first, then exactly w code
// slots.  Every stage waits for all loads before its unit is used, so the
// load count may differ from unit to unit.
template <int MT>
__device__ __forceinline__ void issue(UnitBuf<MT>& u, const DecodeArgs& a, int br, int col, int w, uint32_t kib) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const size_t blk = size_t(br) * a.nbc + col;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + r16;
    const _Float16* xp = a.x + size_t(m) * a.K + size_t(col) * 128 + 8 * g;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      u32x4 v = {0, 0, 0, 0};
      if (m < a.M) v = ld16(xp + 32 * kt);
      u.xa[kt][mt] = __builtin_bit_cast(half8, v);
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) u.sz[rt] = a.sz[blk * 64 + 16 * rt + r16];
  const uint8_t* cp = a.codes + size_t(kib) * 1024 + 16 * lane;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (t < w) u.code[t] = ld16(cp + 1024 * t);
}

// One plane of width W.  LOW: the plane holding the low bits, which carries
// the zero point; otherwise the plane's codes weigh 2^shift.
// D[token][row] of each 16x16 tile: lane holds tokens 16 mt + 4 g + v, row r16.
template <int W, bool LOW, int MT>
__device__ __forceinline__ void plane_mma(const UnitBuf<MT>& u, int shift, const f32x4 (&xsum)[MT],
                                          f32x4 (&acc)[4][MT]) {
  constexpr int NP = 16 / W;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f32x4 c[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) c[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int t = 4 * rt + kt;
      uint32_t p4[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int P = 4 * t + p, d = P / NP;
        p4[p] = pair_bits<W>(u.code[d >> 2][d & 3], P % NP) | kMagicPair;
      }
      const half8 B = as_half8(p4[0], p4[1], p4[2], p4[3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) c[mt] = mfma16(u.xa[kt][mt], B, c[mt]);
    }
    const uint32_t e = u.sz[rt];
    const float s = LOW ? lo_half(e) : __builtin_ldexpf(lo_half(e), shift);
    const float z = LOW ? hi_half(e) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float corr = __builtin_fmaf(z, xsum[mt][v], 1024.0f * xsum[mt][v]);
        acc[rt][mt][v] = __builtin_fmaf(s, c[mt][v] - corr, acc[rt][mt][v]);
      }
    }
  }
}

template <int MT>
__device__ __forceinline__ void compute(const UnitBuf<MT>& u, int w, bool low, int shift, f32x4 (&acc)[4][MT]) {
  const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
  f32x4 xsum[MT];  // X[token] = sum of the group's activations, per lane token
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xsum[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) xsum[mt] = mfma16(u.xa[kt][mt], ones, xsum[mt]);
  }
  if (low) {
    if (w == 4)
      plane_mma<4, true, MT>(u, 0, xsum, acc);
    else if (w == 2)
      plane_mma<2, true, MT>(u, 0, xsum, acc);
    else
      plane_mma<1, true, MT>(u, 0, xsum, acc);
  } else {
    if (w == 4)
      plane_mma<4, false, MT>(u, shift, xsum, acc);
    else if (w == 2)
      plane_mma<2, false, MT>(u, shift, xsum, acc);
    else
      plane_mma<1, false, MT>(u, shift, xsum, acc);
  }
}

// The unit after (j, plane p) in a chunk of S blocks with bitwidths in bvec.
struct UnitCursor {
  int j, p;       // block in the chunk, plane (0 low, 1 high)
  int w, shift;   // plane width and weight 2^shift of its codes
  uint32_t kib;   // first code KiB of the plane
};

__device__ __forceinline__ UnitCursor unit_at(int bvec, int ovec, int j, int p) {
  UnitCursor u;
  u.j = j;
  u.p = p;
  const int b = __builtin_amdgcn_readlane(bvec, j);
  const int w0 = plane0_w(b);
  u.w = p == 0 ? w0 : plane1_w(b);
  u.shift = p == 0 ? 0 : w0;
  u.kib = uint32_t(__builtin_amdgcn_readlane(ovec, j)) + uint32_t(p == 0 ? 0 : w0);
  return u;
}

__device__ __forceinline__ UnitCursor unit_next(const UnitCursor& c, int bvec, int ovec) {
  const int b = __builtin_amdgcn_readlane(bvec, c.j);
  if (c.p == 0 && plane1_w(b) != 0) return unit_at(bvec, ovec, c.j, 1);
  return unit_at(bvec, ovec, c.j + 1, 0);
}

// Wait for every load of this wave; the scheduling barriers keep the loads
// issued after it from being hoisted above it.
__device__ __forceinline__ void wait_all_loads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int NW, int MT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 3 : 1))) void decode_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int br = blockIdx.x / a.nseg, seg = blockIdx.x - br * a.nseg;
  // this workgroup's columns, split evenly between its waves
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;

  f32x4 acc[4][MT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0, 0, 0, 0};

  // Units (bit planes of blocks) in column order; the loads of the next unit
  // are in flight while the current one is computed.
  for (int col0 = w_begin; col0 < w_end; col0 += 64) {
    const int S = min(64, w_end - col0);
    const bool in = lane < S;
    const size_t blk = size_t(br) * a.nbc + col0 + (in ? lane : 0);
    const int bvec = in ? int(a.bits[blk]) : 0;
    const int ovec = in ? int(a.offs[blk]) : 0;
    UnitBuf<MT> A, B;
    UnitCursor ca = unit_at(bvec, ovec, 0, 0), cb;
    issue<MT>(A, a, br, col0 + ca.j, ca.w, ca.kib);
    while (true) {
      wait_all_loads();
      cb = unit_next(ca, bvec, ovec);
      const bool hb = cb.j < S;
      if (hb) issue<MT>(B, a, br, col0 + cb.j, cb.w, cb.kib);
      compute<MT>(A, ca.w, ca.p == 0, ca.shift, acc);
      if (!hb) break;
      wait_all_loads();
      ca = unit_next(cb, bvec, ovec);
      const bool ha = ca.j < S;
      if (ha) issue<MT>(A, a, br, col0 + ca.j, ca.w, ca.kib);
      compute<MT>(B, cb.w, cb.p == 0, cb.shift, acc);
      if (!ha) break;
    }
  }

  // waves meet in LDS; wave w < 4 adds row tile w over the waves in order
  __shared__ f32x4 red[NW][4][MT][64];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][rt][mt][lane] = acc[rt][mt];
  __syncthreads();
  if (wave < 4) {
    const int rt = wave;
    const int n = br * 64 + 16 * rt + r16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 s = red[0][rt][mt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w][rt][mt][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * mt + 4 * g + v;
        if (m >= a.M) continue;
        if (a.nseg == 1)
          a.y[size_t(m) * a.N + n] = (_Float16)s[v];
        else
          __hip_atomic_store(a.part + (size_t(seg) * a.M + m) * a.N + n, s[v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (a.nseg == 1) return;

  // K segments: the barrier waits for every partial store of the workgroup;
  // the workgroup that completes the block row's count sums the segments.
  __shared__ int s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.ctr + br, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == uint32_t(a.nseg - 1);
    if (last) __hip_atomic_store(a.ctr + br, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const size_t stride = size_t(a.M) * a.N;
  for (int o = threadIdx.x; o < 64 * a.M; o += NW * 64) {
    const int m = o >> 6, n = br * 64 + (o & 63);
    const float* pp = a.part + size_t(m) * a.N + n;
    float s = 0.0f;
    for (int s0 = 0; s0 < a.nseg; s0 += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = s0 + i < a.nseg
                   ? __hip_atomic_load(pp + size_t(s0 + i) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    a.y[size_t(m) * a.N + n] = (_Float16)s;
  }
}

}  // namespace

DecodePlan decode_plan(int N, int K, int M) {
  DecodePlan p;
  const int nbr = N / 64, nbc = K / 128;
  p.nw = 4;
  // one workgroup per block row when that gives about 8 waves per CU;
  // otherwise split K into segments of at least 2 columns per wave, capped
  // by the partial-sum traffic (nseg * M * N * 8 bytes against ~N * K / 2)
  const int target_waves = 2048;
  int nseg = 1;
  if (nbr * p.nw < target_waves) {
    nseg = (target_waves + nbr * p.nw - 1) / (nbr * p.nw);
    nseg = min(nseg, max(1, nbc / (2 * p.nw)));
    nseg = min(nseg, max(1, K / (64 * M)));
  }
  p.seg_cols = (nbc + nseg - 1) / nseg;
  p.nseg = (nbc + p.seg_cols - 1) / p.seg_cols;
  if (p.nseg > 1) {
    // counters live in a fixed region at the start of every workspace, so one
    // zero-filled buffer serves calls of any shape
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
  a.seg_cols = plan.seg_cols;
  a.nseg = plan.nseg;
  const dim3 grid(unsigned(im.nbr * plan.nseg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= 16)
    hipLaunchKernelGGL((decode_kernel<4, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<4, 2>), grid, dim3(256), 0, s, a);
  return int(hipGetLastError());
}

const char* device_error_text(int err) {
  return err == 0 ? nullptr : hipGetErrorString(hipError_t(err));
}

}  // namespace gbb
