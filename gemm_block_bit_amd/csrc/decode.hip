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
//    bitwidth is read once per block as a scalar, so every branch on it is
//    wave-uniform.
//  * Each wave streams its blocks through a 13-slot (24 for M > 16) LDS ring
//    filled by
//    global->LDS loads (global_load_lds_dword[x4]), one load per "record":
//    per block one scale/zero record, the activation record(s) and the b code
//    slots.  Whole blocks are issued ahead as long as they fit in the ring, so
//    up to 12 (23) loads are in flight while a block is computed; the wait for a
//    block is an exact vmcnt, and the in-flight data costs no registers.
//  * The high plane of a 2-plane block is unpacked with the fp16 exponent of
//    2^(10 + shift): its codes come out as 2^(10 + shift) + q 2^shift and
//    accumulate into the same MFMA accumulator as the low plane.
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

// Records in flight per wave: a per-wave ring of RING 1 KiB LDS slots filled
// by global->LDS loads, one load per record.  A block has at most
// 1 + 4 MT + 8 records, which must fit: 13 slots for MT = 1 (three 4-wave
// workgroups per CU), 24 for MT = 2.
template <int MT>
struct Ring {
  static constexpr int kSlots = MT == 1 ? 13 : 24;
  static_assert(1 + 4 * MT + 8 <= kSlots, "a block's records fit in the ring");
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left alone (gfx9 encoding), and
// a compiler barrier so no LDS read is moved above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most n (uniform, 0 <= n < 24) of this wave's loads are
// outstanding.
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break;
    case 22: wait_vmcnt<22>(); break;
    default: wait_vmcnt<23>(); break;
  }
}

// One global->LDS load of 16 or 4 bytes per lane: lane l's bytes land at LDS
// address lds + l * size.  Written as inline assembly with no output
// registers (the data goes to LDS), so the compiler does not track it: every
// read of the ring is preceded by an explicit vmcnt wait instead, and each
// load first waits for this wave's earlier LDS reads (lgkmcnt), so a slot is
// never refilled while a read of it is outstanding.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

// A copy of v in a vector register.  Code-pair extraction is
// ((word >> shift) & mask) | exponent; with mask and exponent in vector
// registers it is one v_and_or_b32 (VOP3 can take neither a literal nor two
// scalar operands on gfx9), i.e. two instructions per pair.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}

// Records of one block, in ring order: its scale/zero (256 B: entry
// 4 r16 + t is row 16 t + r16), nx activation records (M = 1: the 128
// activations of the block column, 256 B; else 4 tokens x 128 activations
// each, 1 KiB), then its b code slots (1 KiB each).
template <int R>
__device__ __forceinline__ void issue_block(const DecodeArgs& a, int nx, int br, int col, uint32_t kib, int b,
                                            const u32x4* ring, int first) {
  const int lane = threadIdx.x & 63;
  int n = first;
  dma4(a.sz + (size_t(br) * a.nbc + col) * 64 + lane, lds_addr(ring + (n % R) * 64));
  ++n;
  if (a.M == 1) {
    dma4(a.x + size_t(col) * 128 + 2 * lane, lds_addr(ring + (n % R) * 64));
    ++n;
  } else {
    for (int xi = 0; xi < nx; ++xi, ++n) {
      const int m = min(4 * xi + (lane >> 4), a.M - 1);
      dma16(a.x + size_t(m) * a.K + size_t(col) * 128 + 8 * (lane & 15), lds_addr(ring + (n % R) * 64));
    }
  }
  const uint8_t* cp = a.codes + size_t(kib) * 1024 + 16 * lane;
  for (int q = 0; q < b; ++q, ++n) dma16(cp + 1024 * q, lds_addr(ring + (n % R) * 64));
}

// B operand of tile (rt, kt) of a plane of width PW whose lane dwords are
// w[slot][0..3]: its four code pairs with the fp16 exponent pattern `magic`.
// Codes of weight 2^shift become 2^(10 + shift) + q 2^shift, so every plane
// adds into the same accumulator.
template <int PW>
__device__ __forceinline__ half8 tile_b(const u32x4 (&w)[PW], int rt, int kt, uint32_t magic, uint32_t mask) {
  constexpr int NP = 16 / PW;
  uint32_t p4[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int P = 4 * (4 * rt + kt) + p, d = P / NP, i = P % NP;
    p4[p] = ((w[d >> 2][d & 3] >> (PW * i)) & mask) | magic;
  }
  return as_half8(p4[0], p4[1], p4[2], p4[3]);
}

// All 16 tiles of one plane of width PW whose slots start at ring record
// `rec`, issued k-tile by k-tile so the four row-tile accumulation chains
// interleave on the matrix cores.
template <int PW, int MT, int R>
__device__ __forceinline__ void plane_mma(const u32x4* ring, int rec, uint32_t magic, const half8 (&xa)[4][MT],
                                          f32x4 (&c)[4][MT]) {
  const int lane = threadIdx.x & 63;
  const uint32_t mask = in_vgpr(((1u << PW) - 1u) * 0x00010001u);
  u32x4 w[PW];
#pragma unroll
  for (int t = 0; t < PW; ++t) w[t] = ring[((rec + t) % R) * 64 + lane];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const half8 B = tile_b<PW>(w, rt, kt, magic, mask);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) c[rt][mt] = mfma16(xa[kt][mt], B, c[rt][mt]);
    }
}

// One block whose records start at ring record `first`: planes of width W0
// (shift 0) and W1 (shift W0; 0 = none).  acc += s (C - (bias + z) X) with
// C = sum_k x_k (bias_k + q_k 2^shift) and bias = sum over planes of 1024 2^shift.
template <int W0, int W1, int MT, int R = Ring<MT>::kSlots>
__device__ __forceinline__ void block_mma(const DecodeArgs& a, const u32x4* ring, int first, int nx,
                                          f32x4 (&acc)[4][MT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const u32x4 sz = ring[(first % R) * 64 + r16];
  half8 xa[4][MT];
  if (a.M == 1) {
    const u32x4* xr = ring + ((first + 1) % R) * 64;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) xa[kt][0] = __builtin_bit_cast(half8, xr[4 * kt + g]);
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(16 * mt + r16, a.M - 1);
      const u32x4* xr = ring + ((first + 1 + (m >> 2)) % R) * 64;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) xa[kt][mt] = __builtin_bit_cast(half8, xr[16 * (m & 3) + 4 * kt + g]);
    }
  }
  const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
  f32x4 xsum[MT], c[4][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xsum[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) xsum[mt] = mfma16(xa[kt][mt], ones, xsum[mt]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) c[rt][mt] = f32x4{0, 0, 0, 0};
  }
  const int codes = first + 1 + nx;
  plane_mma<W0, MT, R>(ring, codes, in_vgpr(kMagicPair), xa, c);
  if constexpr (W1 != 0) plane_mma<W1, MT, R>(ring, codes + W0, in_vgpr(kMagicPair + W0 * 0x04000400u), xa, c);
  constexpr float bias = 1024.0f * (1.0f + (W1 ? float(1 << W0) : 0.0f));
  // lane holds tokens 16 mt + 4 g + v; with one token only v = 0 is live
  const int nv = a.M == 1 ? 1 : 4;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const float s = lo_half(sz[rt]), z = hi_half(sz[rt]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (v >= nv) break;
        const float corr = __builtin_fmaf(z, xsum[mt][v], bias * xsum[mt][v]);
        acc[rt][mt][v] = __builtin_fmaf(s, c[rt][mt][v] - corr, acc[rt][mt][v]);
      }
  }
}

template <int NW, int MT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void decode_kernel(DecodeArgs a) {
  constexpr int R = Ring<MT>::kSlots;
  // wave-uniform values go through readfirstlane so the compiler keeps them
  // in scalar registers and branches on them with scalar branches
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int br = blockIdx.x / a.nseg, seg = blockIdx.x - br * a.nseg;
  // this workgroup's columns, split evenly between its waves
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;
  const int nx = a.M == 1 ? 1 : (a.M + 3) / 4;

  __shared__ u32x4 lds[NW * R * 64];   // per-wave rings; reused for the reduction
  const u32x4* ring = lds + wave * R * 64;

  f32x4 acc[4][MT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0, 0, 0, 0};

  for (int col0 = w_begin; col0 < w_end; col0 += 64) {
    const int S = min(64, w_end - col0);
    const bool in = lane < S;
    const size_t blk = size_t(br) * a.nbc + col0 + (in ? lane : 0);
    const int bvec = in ? int(a.bits[blk]) : 0;
    const int ovec = in ? int(a.offs[blk]) : 0;
    // The compiler tracks only these two loads; wait for them here, before any
    // ring load is issued, so that it never waits for them (and with them for
    // every in-flight ring load) inside the block loop.
    wait_vmcnt<0>();
    // Blocks in column order.  Block j's records are ring records
    // [first_j, first_j + 1 + nx + b_j); blocks are issued ahead as long as
    // all their records fit in the R slots after the block being computed.
    int issued = 0;   // records issued so far
    int jn = 0;       // next block to issue
    int first = 0;    // first record of block j
    for (int j = 0; j < S; ++j) {
      const int bj = uniform(__builtin_amdgcn_readlane(bvec, j));
      while (jn < S) {
        const int bn = uniform(__builtin_amdgcn_readlane(bvec, jn));
        if (issued + 1 + nx + bn > first + R) break;
        issue_block<R>(a, nx, br, col0 + jn, uint32_t(uniform(__builtin_amdgcn_readlane(ovec, jn))), bn, ring, issued);
        issued = uniform(issued + 1 + nx + bn);
        ++jn;
      }
      // block j's last record is first + nx + bj; later records may still fly
      wait_vmcnt_at_most(issued - (first + 1 + nx + bj));
      switch (bj) {
        case 1: block_mma<1, 0, MT>(a, ring, first, nx, acc); break;
        case 2: block_mma<2, 0, MT>(a, ring, first, nx, acc); break;
        case 3: block_mma<2, 1, MT>(a, ring, first, nx, acc); break;
        case 4: block_mma<4, 0, MT>(a, ring, first, nx, acc); break;
        case 6: block_mma<4, 2, MT>(a, ring, first, nx, acc); break;
        default: block_mma<4, 4, MT>(a, ring, first, nx, acc); break;
      }
      first = uniform(first + 1 + nx + bj);
    }
  }
  __syncthreads();

  // waves meet in LDS; wave w < 4 adds row tile w over the waves in order
  static_assert(NW * 4 * MT <= NW * R, "reduction fits in the rings");
  f32x4 (*red)[4][MT][64] = reinterpret_cast<f32x4 (*)[4][MT][64]>(lds);
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
