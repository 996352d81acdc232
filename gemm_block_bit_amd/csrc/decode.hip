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
//    lane.  The four words of one 1 KiB slot at one bit field are exactly a
//    v_mfma_f32_16x16x32_f16 B operand (16 rows x 32 columns), so unpacking
//    is one AND per word (plus one shift shared by a few fields): the masked
//    field q << o read as fp16 is the subnormal q 2^(o - 24), which the matrix
//    cores multiply exactly.  o depends only on the row tile, so each row
//    tile's accumulator carries one power of two, removed in the epilogue.
//    b = 3, 6, 8 are two planes (2+1, 4+2, 4+4) with accumulators of their own.
//  * The matrix cores form C = sum_k x_k q_k 2^(o - 24) per 16-row tile and
//    X = sum_k x_k against an all-ones B operand; the epilogue adds
//    s (2^(24 - o) C - z X) = s sum_k x_k (q_k - z) to fp32 accumulators.
//  * Each wave streams its blocks through LDS rings filled by global->LDS
//    loads (global_load_lds_dword[x4]), so data in flight costs no
//    registers.  For M > 1 one ring of 1 KiB slots (12 for M <= 8, 13 for
//    M <= 16, 32 above) holds per block a scale/zero slot, ceil(M / 4)
//    activation slots and the b code slots; the two-row kernel for
//    17 <= M <= 32 keeps the activations in a buffer of their own beside a
//    12-slot ring of scale/zero and code records.  The multi-token epilogue
//    folds 2^(24 - o) into s and z once per row tile (exact).  A single
//    token has its own kernel with an 8-slot code ring
//    and a 4-entry ring of 512-byte scale/zero + activation records: 10 KiB
//    per wave, 16 waves per CU.  Blocks are issued ahead while they fit; the
//    wait for a block is a vmcnt bound, and a block's slots are refilled as
//    soon as its LDS reads have completed.
//  * With K segments, each workgroup hands its partial sums over with one
//    device-scope 64-bit atomic add per output element: the partial, rounded
//    to a multiple of 2^-28, in the high bits and a count in the low bits.
//    The add that completes the count returns the whole sum, so the last
//    contributor writes y and clears the word, one memory round trip after
//    its partial is known.  Integer addition is exact and order-free, so
//    results do not depend on which workgroup finishes first.  Partials too
//    large for the fixed-point field (or not finite) go through an fp32
//    atomic accumulator instead, published before their count.
#include "decode_common.h"

namespace gbb {

namespace {

// MFMAs of one plane of width W whose slots are w[0..W): tile 4 kt + rt is
// bit field i = (4 kt + rt) % (16 / W) of slot (4 kt + rt) / (16 / W).  The
// field is shifted down by sh and masked at offset o = W (i % Q), so the B
// operand holds q 2^(o - 24); o is a function of rt alone.  Tiles go k-tile
// by k-tile so the four row-tile accumulation chains interleave.
template <int W, int MT>
__device__ __forceinline__ void plane_mma(const u32x4 (&w)[W], const half8 (&xa)[4][MT], f32x4 (&c)[4][MT]) {
  using G = PlaneGeom<W>;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int u = 4 * kt + rt, j = u / G::NP, i = u % G::NP;
      const int o = G::off(rt), sh = W * i - o;
      const uint32_t mask = (((1u << W) - 1u) * 0x00010001u) << o;
      const half8 B = as_half8((w[j][0] >> sh) & mask, (w[j][1] >> sh) & mask, (w[j][2] >> sh) & mask,
                               (w[j][3] >> sh) & mask);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) c[rt][mt] = mfma16(xa[kt][mt], B, c[rt][mt]);
    }
}

// A block column's activation fragments from the ring: lane holds tokens
// 16 mt + r16 (rows past M repeat row M - 1), columns 32 kt + 8 g ... + 7.
template <int MT, int RS = Ring<MT>::kSlots>
__device__ __forceinline__ void read_x(const u32x4* ring, uint32_t xb, int M, half8 (&xa)[4][MT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(16 * mt + r16, M - 1);
    const u32x4* xr = ring + (wrap<RS>(xb + 1024 * (m >> 2)) >> 4);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) xa[kt][mt] = __builtin_bit_cast(half8, xr[16 * (m & 3) + 4 * kt + g]);
  }
}

// One block of planes W0 (shift 0) and W1 (shift W0; 0 = none) on the
// activation fragments xa: read its scale/zero slot (ring byte offset szb)
// and code slots (cb), let `refill` reuse the slots, then
// acc += s (sum over planes of 2^(24 + shift - o) C - z X), where X (xsum)
// is the sum of the block column's activations per token -- formed here by
// MFMAs on a ones operand when SumX, else passed in from the block of the
// same column in another row.  The plane weight 2^(24 - o) of the first
// plane is folded into s and z once per row tile (exact: powers of two), so
// each output takes one fewer vector instruction with the same roundings.
template <int W0, int W1, int MT, bool SumX, int RS = Ring<MT>::kSlots, class Refill>
__device__ __forceinline__ void block_core(const u32x4* ring, uint32_t szb, uint32_t cb, const half8 (&xa)[4][MT],
                                           f32x4 (&xsum)[MT], f32x4 (&acc)[4][MT], Refill&& refill) {
  const int lane = threadIdx.x & 63, r16 = lane & 15;
  const u32x4 sz = ring[(wrap<RS>(szb) >> 4) + r16];
  u32x4 w0[W0], w1[W1 ? W1 : 1];
#pragma unroll
  for (int q = 0; q < W0; ++q) w0[q] = ring[(wrap<RS>(cb + 1024 * q) >> 4) + lane];
#pragma unroll
  for (int q = 0; q < W1; ++q) w1[q] = ring[(wrap<RS>(cb + 1024 * (W0 + q)) >> 4) + lane];
  wait_lds();
  refill();

  f32x4 c0[4][MT], c1[4][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) c0[rt][mt] = c1[rt][mt] = f32x4{0, 0, 0, 0};
  if constexpr (SumX) {
    const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xsum[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xsum[mt] = mfma16(xa[kt][mt], ones, xsum[mt]);
  }
  plane_mma<W0, MT>(w0, xa, c0);
  if constexpr (W1 != 0) plane_mma<W1, MT>(w1, xa, c1);
  // lane holds tokens 16 mt + 4 g + v
  constexpr int W1g = W1 ? W1 : 1;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    constexpr int o0[4] = {PlaneGeom<W0>::off(0), PlaneGeom<W0>::off(1), PlaneGeom<W0>::off(2),
                           PlaneGeom<W0>::off(3)};
    constexpr int o1[4] = {PlaneGeom<W1g>::off(0), PlaneGeom<W1g>::off(1), PlaneGeom<W1g>::off(2),
                           PlaneGeom<W1g>::off(3)};
    const float s = lo_half(sz[rt]) * pow2(24 - o0[rt]);
    const float z = hi_half(sz[rt]) * pow2(o0[rt] - 24);
    constexpr float k10[4] = {pow2(W0 - o1[0] + o0[0]), pow2(W0 - o1[1] + o0[1]), pow2(W0 - o1[2] + o0[2]),
                              pow2(W0 - o1[3] + o0[3])};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float t = c0[rt][mt][v];
        if constexpr (W1 != 0) t = __builtin_fmaf(c1[rt][mt][v], k10[rt], t);
        acc[rt][mt][v] = __builtin_fmaf(s, __builtin_fmaf(-z, xsum[mt][v], t), acc[rt][mt][v]);
      }
  }
}

// One block whose records start at ring byte offsets sz (scale/zero slot),
// xb (first activation slot) and cb (first code slot).
template <int W0, int W1, int MT, int RS, class Refill>
__device__ __forceinline__ void block_mma(const u32x4* ring, uint32_t szb, uint32_t xb, uint32_t cb, int M,
                                          f32x4 (&acc)[4][MT], Refill&& refill) {
  half8 xa[4][MT];
  read_x<MT, RS>(ring, xb, M, xa);
  f32x4 xsum[MT];
  block_core<W0, W1, MT, true, RS>(ring, szb, cb, xa, xsum, acc, refill);
}

// Ring slots per wave for 2 <= M <= 16: a block's records (scale/zero,
// ceil(M / 4) activation slots, at most eight code slots) fit in twelve for
// M <= 8 and in thirteen for M <= 16, so the rings of a four-wave workgroup
// take 48 or 52 KiB and three workgroups share a CU (three waves per SIMD).
// Llama-3-70B projections: 6-11 % faster on gate|up and down than 16 slots
// with two workgroups per CU; the 8B shapes are within a few per cent.
constexpr int kRing8 = 12;
constexpr int kRing16 = 13;

// Workgroup wg of a launch of one problem: block row wg / nseg, K segment
// wg % nseg.
template <int NW, int MT, int RS>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, int wg) {
  constexpr int R = RS;
  // wave-uniform values go through readfirstlane so the compiler keeps them
  // in scalar registers and branches on them with scalar branches
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int br = int(unsigned(wg) / unsigned(a.nseg)), seg = wg - br * a.nseg;
  // this workgroup's columns, split evenly between its waves
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;
  const int M = a.M;
  const int nx = (M + 3) / 4;   // activation slots (and loads) per block
  // byte offset of lane's activation chunk in activation record xi
  uint32_t xoff[8];
#pragma unroll
  for (int xi = 0; xi < 8; ++xi) xoff[xi] = uint32_t(min(4 * xi + g, M - 1)) * uint32_t(2 * a.K) + 16 * r16;

  __shared__ u32x4 lds[NW * R * 64];   // per-wave rings; reused for the reduction
  const u32x4* ring = lds + wave * R * 64;
  const uint32_t ring_lds = lds_addr(ring);

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
    const int o0 = int(a.offs[size_t(br) * a.nbc + col0]);
    // The compiler tracks only these loads; wait for them here, before any
    // ring load is issued, so that it never waits for them (and with them for
    // every in-flight ring load) inside the block loop.
    wait_vmcnt<0>();
    // The chunk's blocks are consecutive in the image, so their scale/zero
    // records, activation columns and codes are three contiguous streams.
    const uint32_t* szp = a.sz + (size_t(br) * a.nbc + col0) * 64;
    const _Float16* xp = a.x + size_t(col0) * 128;
    const uint8_t* cp = a.codes + size_t(uniform(o0)) * 1024;
    int jn = 0;          // next block to issue
    int used = 0;        // ring slots holding blocks not yet read
    uint32_t sbn = 0;    // ring byte offset of the next block to issue
    int issued = 0;      // loads issued
    auto fill = [&]() {
      while (jn < S) {
        const int bn = uniform(__builtin_amdgcn_readlane(bvec, jn));
        const int ns = 1 + nx + bn;
        if (used + ns > R) break;
        dma4_once(szp, 4 * lane, ring_lds, sbn);
        szp += 64;
        for (int xi = 0; xi < nx; ++xi) dma16(xp, xoff[xi], ring_lds, wrap<R>(sbn + 1024 * (1 + xi)));
        xp += 128;
        uint32_t sc = sbn + 1024 * (1 + nx);
        for (int q = 0; q < bn; ++q) {
          dma16_once(cp, 16 * lane, ring_lds, wrap<R>(sc));
          cp += 1024;
          sc += 1024;
        }
        sbn = wrap<R>(sc);
        used += ns;
        issued += 1 + nx + bn;
        ++jn;
      }
    };
    fill();
    uint32_t sb = 0;   // ring byte offset of block j
    int done = 0;      // loads of blocks 0..j
    for (int j = 0; j < S; ++j) {
      const int bj = uniform(__builtin_amdgcn_readlane(bvec, j));
      done += 1 + nx + bj;
      wait_vmcnt_at_most(issued - done);
      auto refill = [&]() {
        used -= 1 + nx + bj;
        fill();
      };
      const uint32_t xb = sb + 1024, cb = sb + 1024 * (1 + nx);
      switch (bj) {
        case 1: block_mma<1, 0, MT, R>(ring, sb, xb, cb, M, acc, refill); break;
        case 2: block_mma<2, 0, MT, R>(ring, sb, xb, cb, M, acc, refill); break;
        case 3: block_mma<2, 1, MT, R>(ring, sb, xb, cb, M, acc, refill); break;
        case 4: block_mma<4, 0, MT, R>(ring, sb, xb, cb, M, acc, refill); break;
        case 6: block_mma<4, 2, MT, R>(ring, sb, xb, cb, M, acc, refill); break;
        default: block_mma<4, 4, MT, R>(ring, sb, xb, cb, M, acc, refill); break;
      }
      sb = wrap<R>(sb + 1024 * (1 + nx + bj));
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
    size_t idx[4 * MT];
    float val[4 * MT];
    bool act[4 * MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 s = red[0][rt][mt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w][rt][mt][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * mt + 4 * g + v;
        idx[4 * mt + v] = size_t(min(m, M - 1)) * a.N + n;
        val[4 * mt + v] = s[v];
        act[4 * mt + v] = m < M;
      }
    }
    if (a.nseg == 1) {
#pragma unroll
      for (int k = 0; k < 4 * MT; ++k)
        if (act[k]) a.y[idx[k]] = (_Float16)val[k];
    } else {
      splitk_publish_all<4 * MT>(a, idx, val, act);
    }
  }
}

template <int NW, int MT, int RS = Ring<MT>::kSlots>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 3))) void decode_kernel(DecodeArgs a) {
  decode_body<NW, MT, RS>(a, int(blockIdx.x));
}

// Two block rows per wave (17 <= M <= 32).  At that batch a block column's
// activations are eight 1 KiB slots against ~2-3 KiB of codes per block.
// A workgroup owns two consecutive block rows; for each column a wave reads
// the activations into registers once and runs both rows' blocks on them.
// The activations have a one-column buffer of their own, refilled with the
// next column as soon as the current one is in registers, so the code ring
// holds only scale/zero records and codes: [sz A | codes A], [sz B | codes B]
// records in column order, each released as soon as its block has read it.
// Twelve slots take any record (at most 1 + 8), so each wave needs 20 KiB
// of LDS and two four-wave workgroups share a CU: two waves per SIMD, which
// hide each other's LDS and matrix-core latencies.
constexpr int kRing2 = 12;   // code ring slots per wave
constexpr int kXs2 = 8;      // activation slots per wave (4 tokens each)

// Sequence numbers of the last load of the next six records in the ring, a
// shift register indexed only by constants (no private-memory array).
struct RecordEnds {
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0, q4 = 0, q5 = 0;
  __device__ void set(int pos, int v) {
    switch (pos) {
      case 0: q0 = v; break;
      case 1: q1 = v; break;
      case 2: q2 = v; break;
      case 3: q3 = v; break;
      case 4: q4 = v; break;
      default: q5 = v; break;
    }
  }
  __device__ void pop() {
    q0 = q1;
    q1 = q2;
    q2 = q3;
    q3 = q4;
    q4 = q5;
  }
};

template <int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode2_kernel(DecodeArgs a) {
  constexpr int NW = 4;
  constexpr int R = kRing2;
  static_assert(1 + 8 <= R, "any block's records fit in the ring");
  static_assert(R / 2 <= 6, "records take two slots or more, so at most six sit in the ring");
  static_assert(4 * MT <= kXs2, "a column's activations fit in the activation slots");
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int rp = blockIdx.x / a.nseg, seg = blockIdx.x - rp * a.nseg;
  const int brA = 2 * rp;
  const bool hasB = brA + 1 < a.nbr;   // else row B repeats row A, unstored
  const int brB = hasB ? brA + 1 : brA;
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;
  const int M = a.M;
  const int nx = (M + 3) / 4;
  uint32_t xoff[8];
#pragma unroll
  for (int xi = 0; xi < 8; ++xi) xoff[xi] = uint32_t(min(4 * xi + g, M - 1)) * uint32_t(2 * a.K) + 16 * r16;

  // per wave: the code ring, then the activation slots; reused for the reduction
  __shared__ u32x4 lds[NW * (R + kXs2) * 64];
  const u32x4* ring = lds + wave * (R + kXs2) * 64;
  const u32x4* xbuf = ring + R * 64;
  const uint32_t ring_lds = lds_addr(ring);
  constexpr uint32_t kXbuf = R * 1024;   // activation slots, relative to the ring

  f32x4 acc[2][4][MT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[r][rt][mt] = f32x4{0, 0, 0, 0};

  for (int col0 = w_begin; col0 < w_end; col0 += 64) {
    const int S = min(64, w_end - col0);
    const bool in = lane < S;
    const size_t blkA = size_t(brA) * a.nbc + col0, blkB = size_t(brB) * a.nbc + col0;
    const int bvecA = in ? int(a.bits[blkA + lane]) : 0;
    const int bvecB = in ? int(a.bits[blkB + lane]) : 0;
    const int oA = int(a.offs[blkA]), oB = int(a.offs[blkB]);
    wait_vmcnt<0>();   // the compiler tracks only these loads
    const uint32_t* szpA = a.sz + blkA * 64;
    const uint32_t* szpB = a.sz + blkB * 64;
    const _Float16* xp = a.x + size_t(col0) * 128;
    const uint8_t* cpA = a.codes + size_t(uniform(oA)) * 1024;
    const uint8_t* cpB = a.codes + size_t(uniform(oB)) * 1024;
    int issued = 0;      // loads issued
    int ri = 0, rc = 0;  // records issued / consumed: A0, B0, A1, B1, ...
    int used = 0;        // ring slots of issued records not yet released
    uint32_t sbn = 0;    // ring byte offset of the next record to issue
    RecordEnds ends;
    for (int xi = 0; xi < nx; ++xi) dma16(xp, xoff[xi], ring_lds, kXbuf + 1024 * xi);
    issued += nx;
    int xend = issued;   // loads up to the current column's activations
    auto fill = [&]() {
      while (ri < 2 * S) {
        const int col = ri >> 1;
        const bool rowB = (ri & 1) != 0;
        const int b = uniform(__builtin_amdgcn_readlane(rowB ? bvecB : bvecA, col));
        if (used + 1 + b > R) break;
        if (!rowB) {
          dma4_once(szpA, 4 * lane, ring_lds, sbn);
          szpA += 64;
          for (int q = 0; q < b; ++q) {
            dma16_once(cpA, 16 * lane, ring_lds, wrap<R>(sbn + 1024 * (1 + q)));
            cpA += 1024;
          }
        } else {
          dma4_once(szpB, 4 * lane, ring_lds, sbn);
          szpB += 64;
          for (int q = 0; q < b; ++q) {
            dma16_once(cpB, 16 * lane, ring_lds, wrap<R>(sbn + 1024 * (1 + q)));
            cpB += 1024;
          }
        }
        sbn = wrap<R>(sbn + 1024 * (1 + b));
        used += 1 + b;
        issued += 1 + b;
        ends.set(ri - rc, issued);
        ++ri;
      }
    };
    fill();
    uint32_t sb = 0;   // ring byte offset of the next record to consume
    for (int j = 0; j < S; ++j) {
      const int bA = uniform(__builtin_amdgcn_readlane(bvecA, j));
      const int bB = uniform(__builtin_amdgcn_readlane(bvecB, j));
      // row A's record and the column's activations
      wait_vmcnt_at_most(issued - max(ends.q0, xend));
      half8 xa[4][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = min(16 * mt + r16, M - 1);
        const u32x4* xr = xbuf + 64 * (m >> 2);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) xa[kt][mt] = __builtin_bit_cast(half8, xr[16 * (m & 3) + 4 * kt + g]);
      }
      f32x4 xsum[MT];
      // after row A's reads: release its record, bring the next column's
      // activations into the (now read) activation slots, refill the ring
      auto afterA = [&]() {
        used -= 1 + bA;
        ends.pop();
        ++rc;
        if (j + 1 < S) {
          xp += 128;
          for (int xi = 0; xi < nx; ++xi) dma16(xp, xoff[xi], ring_lds, kXbuf + 1024 * xi);
          issued += nx;
          xend = issued;
        }
        fill();
      };
      const uint32_t cbA = wrap<R>(sb + 1024);
      switch (bA) {
        case 1: block_core<1, 0, MT, true, R>(ring, sb, cbA, xa, xsum, acc[0], afterA); break;
        case 2: block_core<2, 0, MT, true, R>(ring, sb, cbA, xa, xsum, acc[0], afterA); break;
        case 3: block_core<2, 1, MT, true, R>(ring, sb, cbA, xa, xsum, acc[0], afterA); break;
        case 4: block_core<4, 0, MT, true, R>(ring, sb, cbA, xa, xsum, acc[0], afterA); break;
        case 6: block_core<4, 2, MT, true, R>(ring, sb, cbA, xa, xsum, acc[0], afterA); break;
        default: block_core<4, 4, MT, true, R>(ring, sb, cbA, xa, xsum, acc[0], afterA); break;
      }
      sb = wrap<R>(sb + 1024 * (1 + bA));
      // row B's record (issued at the latest by afterA's refill)
      wait_vmcnt_at_most(issued - ends.q0);
      auto afterB = [&]() {
        used -= 1 + bB;
        ends.pop();
        ++rc;
        fill();
      };
      const uint32_t cbB = wrap<R>(sb + 1024);
      switch (bB) {
        case 1: block_core<1, 0, MT, false, R>(ring, sb, cbB, xa, xsum, acc[1], afterB); break;
        case 2: block_core<2, 0, MT, false, R>(ring, sb, cbB, xa, xsum, acc[1], afterB); break;
        case 3: block_core<2, 1, MT, false, R>(ring, sb, cbB, xa, xsum, acc[1], afterB); break;
        case 4: block_core<4, 0, MT, false, R>(ring, sb, cbB, xa, xsum, acc[1], afterB); break;
        case 6: block_core<4, 2, MT, false, R>(ring, sb, cbB, xa, xsum, acc[1], afterB); break;
        default: block_core<4, 4, MT, false, R>(ring, sb, cbB, xa, xsum, acc[1], afterB); break;
      }
      sb = wrap<R>(sb + 1024 * (1 + bB));
    }
  }
  __syncthreads();

  // waves meet in LDS; wave w adds row tile w of both rows over the waves
  static_assert(NW * 2 * 4 * MT <= NW * (R + kXs2), "reduction fits in the rings");
  f32x4 (*red)[2][4][MT][64] = reinterpret_cast<f32x4 (*)[2][4][MT][64]>(lds);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wave][r][rt][mt][lane] = acc[r][rt][mt];
  __syncthreads();
  const int rt = wave;
  size_t idx[8 * MT];
  float val[8 * MT];
  bool act[8 * MT];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int n = (r ? brB : brA) * 64 + 16 * rt + r16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 s = red[0][r][rt][mt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w][r][rt][mt][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * mt + 4 * g + v, k = 4 * (MT * r + mt) + v;
        idx[k] = size_t(min(m, M - 1)) * a.N + n;
        val[k] = s[v];
        act[k] = m < M && (r == 0 || hasB);   // a repeated row A is not stored
      }
    }
  }
  // One K segment: y.  Else this segment's fp32 partials, which a second
  // launch adds in segment order: at 32 tokens the split-K words would take
  // a memory-side atomic per output and segment (about 2 M per launch), and
  // those cost more than the second launch.
  float* const dst = a.nseg == 1 ? nullptr : a.part + size_t(seg) * size_t(M) * size_t(a.N);
#pragma unroll
  for (int k = 0; k < 8 * MT; ++k) {
    if (!act[k]) continue;
    if (dst)
      dst[idx[k]] = val[k];
    else
      a.y[idx[k]] = (_Float16)val[k];
  }
}

// Single-token decode.  With one token the activations of a block column are
// 256 bytes, so each wave keeps two small rings: an 8-slot ring of 1 KiB code
// slots and a 4-entry ring of 512-byte records (scale/zero 256 B, then the
// block column's activations 256 B).  That is 10 KiB of LDS per wave, so four
// 4-wave workgroups (16 waves) are resident per CU, which hides the latency
// of each wave's LDS reads and matrix-core results behind the others.
constexpr int kCodeSlots1 = 8;
constexpr uint32_t kCodeMask1 = kCodeSlots1 * 1024 - 1;
constexpr int kMetaSlots1 = 4;
constexpr uint32_t kMetaMask1 = kMetaSlots1 * 512 - 1;
constexpr int kWaveLds1 = kCodeSlots1 * 1024 + kMetaSlots1 * 512;   // bytes per wave

template <int W0, int W1, class Refill>
__device__ __forceinline__ void block1(const u32x4* code, const u32x4* meta, uint32_t cj, uint32_t mj, float (&acc)[4],
                                       Refill&& refill) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const u32x4 sz = meta[(mj >> 4) + r16];
  half8 xa[4][1];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) xa[kt][0] = __builtin_bit_cast(half8, meta[(mj >> 4) + 16 + 4 * kt + g]);
  u32x4 w0[W0], w1[W1 ? W1 : 1];
#pragma unroll
  for (int q = 0; q < W0; ++q) w0[q] = code[(((cj + 1024 * q) & kCodeMask1) >> 4) + lane];
#pragma unroll
  for (int q = 0; q < W1; ++q) w1[q] = code[(((cj + 1024 * (W0 + q)) & kCodeMask1) >> 4) + lane];
  wait_lds();
  refill();

  const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
  f32x4 xsum = f32x4{0, 0, 0, 0}, c0[4][1], c1[4][1];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) c0[rt][0] = c1[rt][0] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) xsum = mfma16(xa[kt][0], ones, xsum);
  plane_mma<W0, 1>(w0, xa, c0);
  if constexpr (W1 != 0) plane_mma<W1, 1>(w1, xa, c1);
  constexpr int W1g = W1 ? W1 : 1;
  constexpr float k0[4] = {pow2(24 - PlaneGeom<W0>::off(0)), pow2(24 - PlaneGeom<W0>::off(1)),
                           pow2(24 - PlaneGeom<W0>::off(2)), pow2(24 - PlaneGeom<W0>::off(3))};
  constexpr float k1[4] = {pow2(24 + W0 - PlaneGeom<W1g>::off(0)), pow2(24 + W0 - PlaneGeom<W1g>::off(1)),
                           pow2(24 + W0 - PlaneGeom<W1g>::off(2)), pow2(24 + W0 - PlaneGeom<W1g>::off(3))};
  // every row of the tiles is the one token: use element 0
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const float s = lo_half(sz[rt]), z = hi_half(sz[rt]);
    float t = c0[rt][0][0] * k0[rt];
    if constexpr (W1 != 0) t = __builtin_fmaf(c1[rt][0][0], k1[rt], t);
    acc[rt] = __builtin_fmaf(s, __builtin_fmaf(-z, xsum[0], t), acc[rt]);
  }
}

template <int NW>
__device__ __forceinline__ void decode1_body(const DecodeArgs& a, int wg);
// The arguments are passed one by one, those needed first leading, so the
// dispatcher can place them in scalar registers before the first instruction
// (kernel argument preloading) instead of every wave loading them from
// memory: with one round of short workgroups that load is on the critical
// path (Llama-3-8B layer set: 8.25 -> 8.07 us per launch).
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void decode1_kernel(
    const uint8_t* bits, const uint32_t* offs, const uint32_t* sz, const uint8_t* codes, const _Float16* x, int nbc,
    int seg_cols, int nseg, _Float16* y, uint64_t* acc, float* facc, int N, int K, int M, int nbr) {
  DecodeArgs a;
  a.bits = bits;
  a.offs = offs;
  a.sz = sz;
  a.codes = codes;
  a.x = x;
  a.y = y;
  a.acc = acc;
  a.facc = facc;
  a.part = nullptr;
  a.N = N;
  a.K = K;
  a.M = M;
  a.nbr = nbr;
  a.nbc = nbc;
  a.seg_cols = seg_cols;
  a.nseg = nseg;
  decode1_body<NW>(a, int(blockIdx.x));
}
template <int NW>
__device__ __forceinline__ void decode1_body(const DecodeArgs& a, int wg) {
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int br = int(unsigned(wg) / unsigned(a.nseg)), seg = wg - br * a.nseg;
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;
  const uint32_t voff = 16 * lane;   // lane's 16 bytes of a 1 KiB record

  __shared__ u32x4 lds[NW * kWaveLds1 / 16];   // per-wave rings; reused for the reduction
  const u32x4* code = lds + wave * (kWaveLds1 / 16);
  const u32x4* meta = code + kCodeSlots1 * 64;
  const uint32_t code_lds = lds_addr(code), meta_lds = lds_addr(meta);

  float acc[4] = {0, 0, 0, 0};
  for (int col0 = w_begin; col0 < w_end; col0 += 64) {
    const int S = min(64, w_end - col0);
    const bool in = lane < S;
    const size_t blk0 = size_t(br) * a.nbc + col0;
    const int bvec = in ? int(a.bits[blk0 + lane]) : 0;
    const int o0 = int(a.offs[blk0]);
    // the compiler tracks only these loads: wait for them before any ring load
    wait_vmcnt<0>();
    // the chunk's blocks are consecutive in the image: scale/zero records,
    // activation columns and codes are three contiguous streams
    const uint32_t* szp = a.sz + blk0 * 64;
    const _Float16* xp = a.x + size_t(col0) * 128;
    const uint8_t* cp = a.codes + size_t(uniform(o0)) * 1024;
    int jn = 0, cfree = kCodeSlots1, mfree = kMetaSlots1, issued = 0;
    uint32_t cn = 0, mn = 0;   // ring offsets of the next block to issue
    auto fill = [&]() {
      while (jn < S) {
        const int bn = uniform(__builtin_amdgcn_readlane(bvec, jn));
        if (bn > cfree || mfree == 0) break;
        dma4_once(szp, 4 * lane, meta_lds, mn);
        dma4(xp, 4 * lane, meta_lds, mn + 256);
        for (int q = 0; q < bn; ++q) dma16_once(cp + 1024 * q, voff, code_lds, (cn + 1024 * q) & kCodeMask1);
        szp += 64;
        xp += 128;
        cp += 1024 * bn;
        cn = (cn + 1024 * bn) & kCodeMask1;
        mn = (mn + 512) & kMetaMask1;
        cfree -= bn;
        mfree -= 1;
        issued += 2 + bn;
        ++jn;
      }
    };
    fill();
    uint32_t cj = 0, mj = 0;
    int done = 0;
    for (int j = 0; j < S; ++j) {
      const int bj = uniform(__builtin_amdgcn_readlane(bvec, j));
      done += 2 + bj;
      wait_vmcnt_coarse(issued - done);
      auto refill = [&]() {
        cfree += bj;
        mfree += 1;
        fill();
      };
      switch (bj) {
        case 1: block1<1, 0>(code, meta, cj, mj, acc, refill); break;
        case 2: block1<2, 0>(code, meta, cj, mj, acc, refill); break;
        case 3: block1<2, 1>(code, meta, cj, mj, acc, refill); break;
        case 4: block1<4, 0>(code, meta, cj, mj, acc, refill); break;
        case 6: block1<4, 2>(code, meta, cj, mj, acc, refill); break;
        default: block1<4, 4>(code, meta, cj, mj, acc, refill); break;
      }
      cj = (cj + 1024 * bj) & kCodeMask1;
      mj = (mj + 512) & kMetaMask1;
    }
  }
  __syncthreads();

  // waves meet in LDS; lane l of wave 0 adds row 16 (l / 16) + l % 16 of
  // the block row over the waves in order
  static_assert(NW * 4 * 64 * 4 <= NW * kWaveLds1, "reduction fits in the rings");
  float (*red)[4][64] = reinterpret_cast<float (*)[4][64]>(lds);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) red[wave][rt][lane] = acc[rt];
  __syncthreads();
  if (wave != 0) return;
  float s = red[0][g][r16];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w][g][r16];
  const size_t n = size_t(br) * 64 + lane;
  if (a.nseg == 1)
    a.y[n] = (_Float16)s;
  else
    splitk_publish(a, n, s, true);
}

// Grouped launch: independent problems (each its own image, activations,
// outputs and split-K accumulators, all with the same M) share one grid.
// Problem i owns workgroups [wg0, wg0 + its own grid); each workgroup finds
// its problem with a scan over the (uniform) table in the kernel arguments
// and then runs exactly the single-problem code.
struct BatchProblem {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  const _Float16* x;
  _Float16* y;
  uint64_t* acc;
  float* facc;
  int N, K, nbr, nbc, seg_cols, nseg, wg0, pad;
};
struct DecodeBatch {
  BatchProblem p[kMaxBatch];
  int n, M;
};
static_assert(sizeof(DecodeBatch) <= 4096, "kernel arguments");

__device__ __forceinline__ int batch_problem(const DecodeBatch& b, int wg) {
  int i = 0;
  for (int j = 1; j < b.n; ++j) i = wg >= b.p[j].wg0 ? j : i;
  return uniform(i);
}

__device__ __forceinline__ DecodeArgs batch_args(const DecodeBatch& b, int i) {
  const BatchProblem& p = b.p[i];
  DecodeArgs a;
  a.bits = p.bits;
  a.offs = p.offs;
  a.sz = p.sz;
  a.codes = p.codes;
  a.x = p.x;
  a.y = p.y;
  a.acc = p.acc;
  a.facc = p.facc;
  a.part = nullptr;
  a.N = p.N;
  a.K = p.K;
  a.M = b.M;
  a.nbr = p.nbr;
  a.nbc = p.nbc;
  a.seg_cols = p.seg_cols;
  a.nseg = p.nseg;
  return a;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void decode1_batch_kernel(
    DecodeBatch b) {
  const int i = batch_problem(b, int(blockIdx.x));
  decode1_body<NW>(batch_args(b, i), int(blockIdx.x) - b.p[i].wg0);
}

template <int NW, int MT, int RS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 3))) void decode_batch_kernel(DecodeBatch b) {
  const int i = batch_problem(b, int(blockIdx.x));
  decode_body<NW, MT, RS>(batch_args(b, i), int(blockIdx.x) - b.p[i].wg0);
}

}  // namespace

DecodePlan decode_plan(int N, int K, int M) {
  DecodePlan p;
  const int nbr = N / 64, nbc = K / 128;
  p.nw = 4;
  p.rows = 1;
  int nseg = 1;
  if (M == 1) {
    // Single token: every wave takes k blocks of a block row (k = 4, 2 or
    // 1), with the largest k that still gives at least 1024 workgroups (four
    // per CU, the resident count) so the dispatcher can balance the CUs; k = 1
    // when none reaches it.  At 768 or more workgroups a smaller k is not
    // taken when it would split K into more than 16 segments: the hand-off
    // atomics per output then cost more than the balance gains (Llama-3-8B
    // down projection, 4096 x 14336: 9.0 against 10.0 us).  Measured on
    // Llama-3-8B/70B-shaped projections.
    auto segs = [&](int kk) { return (nbc + 4 * kk - 1) / (4 * kk); };
    int k = 4;
    while (k > 1 && nbr * segs(k) < 1024 && !(nbr * segs(k) >= 768 && segs(k / 2) > 16)) k /= 2;
    while ((nbc + 4 * k - 1) / (4 * k) > kMaxSegments) k *= 2;
    nseg = (nbc + 4 * k - 1) / (4 * k);
  } else {
    // 4-wave workgroups resident per CU: three for M <= 16 (48 or 52 KiB of
    // LDS rings each), two for the two-row kernel (80 KiB), one for one row
    // at M > 16 (128 KiB).  A workgroup owns one block row, or two for M > 16 on
    // matrices of at least 2^26 weights (smaller ones lose more to the halved
    // workgroup count than they gain: Llama-3 sweeps at M = 20 and 32).  One
    // workgroup per row unit when that fills
    // the resident slots; else split K into as many segments as still fit
    // in one resident wave of workgroups, with at least 2 columns per wave,
    // capped by the hand-off traffic (nseg * M * N * 8 bytes against
    // ~N * K / 2; twice that for M > 16, where the sweeps favour the split).
    if (M > 16 && size_t(N) * size_t(K) >= (size_t(1) << 26)) p.rows = 2;
    const int resident = (M <= 16 ? 3 : (p.rows == 2 ? 2 : 1)) * 256;
    const int units = (nbr + p.rows - 1) / p.rows;
    if (units < resident) {
      nseg = resident / units;
      nseg = min(nseg, max(1, nbc / (2 * p.nw)));
      nseg = min(nseg, max(1, K / ((M > 16 ? 32 : 64) * M)));
    }
  }
  nseg = min(nseg, kMaxSegments);
  p.seg_cols = (nbc + nseg - 1) / nseg;
  p.nseg = (nbc + p.seg_cols - 1) / p.seg_cols;
  // split-K words and overflow floats per output (8 + 4 bytes), or for the
  // two-row kernel fp32 partials per output and segment
  p.ws_bytes = p.nseg == 1 ? 0 : size_t(M) * size_t(N) * (p.rows == 2 ? 4 * size_t(p.nseg) : 12);
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
  // a K split hands off through the split-K words (one block row per
  // workgroup) or through fp32 partials and a second launch (two rows)
  const bool words = plan.nseg > 1 && plan.rows == 1, partials = plan.nseg > 1 && plan.rows == 2;
  a.acc = words ? static_cast<uint64_t*>(workspace) : nullptr;
  a.facc = words ? reinterpret_cast<float*>(static_cast<char*>(workspace) + size_t(M) * im.N * 8) : nullptr;
  a.part = partials ? static_cast<float*>(workspace) : nullptr;
  a.N = im.N;
  a.K = im.K;
  a.M = M;
  a.nbr = im.nbr;
  a.nbc = im.nbc;
  a.seg_cols = plan.seg_cols;
  a.nseg = plan.nseg;
  const int units = (im.nbr + plan.rows - 1) / plan.rows;
  const dim3 grid(unsigned(units * plan.nseg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 1)
    hipLaunchKernelGGL((decode1_kernel<4>), grid, dim3(256), 0, s, a.bits, a.offs, a.sz, a.codes, a.x, a.nbc,
                       a.seg_cols, a.nseg, a.y, a.acc, a.facc, a.N, a.K, a.M, a.nbr);
  else if (M <= 8)   // a block's records (1 + ceil(M / 4) + 8 slots) fit in 12 slots
    hipLaunchKernelGGL((decode_kernel<4, 1, kRing8>), grid, dim3(256), 0, s, a);
  else if (M <= 16)   // 1 + 4 + 8 slots fit in 13
    hipLaunchKernelGGL((decode_kernel<4, 1, kRing16>), grid, dim3(256), 0, s, a);
  else if (plan.rows == 1)
    hipLaunchKernelGGL((decode_kernel<4, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode2_kernel<2>), grid, dim3(256), 0, s, a);
  if (a.part) return launch_split_reduce(a.part, y, M, im.N, plan.nseg, stream);
  return int(hipGetLastError());
}

int launch_decode_batch(int n, const BlockImageView* ims, const uint16_t* const* x, uint16_t* const* y, int M,
                        const DecodePlan* plans, void* const* workspaces, void* stream) {
  DecodeBatch b;
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    BatchProblem& p = b.p[i];
    const BlockImageView& im = ims[i];
    p.bits = im.bits;
    p.offs = im.offs;
    p.sz = im.sz;
    p.codes = im.codes;
    p.x = reinterpret_cast<const _Float16*>(x[i]);
    p.y = reinterpret_cast<_Float16*>(y[i]);
    p.acc = plans[i].nseg > 1 ? static_cast<uint64_t*>(workspaces[i]) : nullptr;
    p.facc = plans[i].nseg > 1
                 ? reinterpret_cast<float*>(static_cast<char*>(workspaces[i]) + size_t(M) * im.N * 8)
                 : nullptr;
    p.N = im.N;
    p.K = im.K;
    p.nbr = im.nbr;
    p.nbc = im.nbc;
    p.seg_cols = plans[i].seg_cols;
    p.nseg = plans[i].nseg;
    p.wg0 = wg;
    p.pad = 0;
    wg += im.nbr * plans[i].nseg;   // one block row per workgroup at M <= 16
  }
  b.n = n;
  b.M = M;
  const dim3 grid{static_cast<unsigned>(wg), 1u, 1u};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 1)
    hipLaunchKernelGGL((decode1_batch_kernel<4>), grid, dim3(256), 0, s, b);
  else if (M <= 8)
    hipLaunchKernelGGL((decode_batch_kernel<4, 1, kRing8>), grid, dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL((decode_batch_kernel<4, 1, kRing16>), grid, dim3(256), 0, s, b);
  return int(hipGetLastError());
}

const char* device_error_text(int err) {
  return err == 0 ? nullptr : hipGetErrorString(hipError_t(err));
}

}  // namespace gbb
