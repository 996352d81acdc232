// Prefill kernel: y = x . dequant(W)^T for larger M over the block image.
//
// Large batched products are compute bound and the dequantization must be
// hidden under the matrix math (MixLLM page, section 2.2 on batched serving
// and section 3.3 on overlapping dequantization with the matrix product).
//
// gfx950 design: a workgroup of eight waves (two per SIMD, one workgroup per
// CU) computes a 128 (tokens) x 512 (output rows) tile of y; wave w owns
// block row 8 t + w, all 128 tokens.  The block image stores each 1 KiB of
// codes so that the 16 bytes a lane loads are, field by field, exactly its
// v_mfma_f32_16x16x32_f16 B operands (16 rows x 32 columns per tile).  So a
// wave turns the codes of one 64x128 block into B operands in registers, one
// 32-column tile at a time -- fp16((q - z) s) per element: OR the code into
// the mantissa of 1024.0, subtract 1024 + z (exact, a small integer) and
// multiply by s (rounded once) -- and uses each of them for the eight
// 16-token tiles (128 MFMAs per block and wave).  The dequantization of the
// next column tile is independent of the current tile's MFMAs, and the other
// wave on the SIMD fills the matrix cores while one does vector work.  The
// plane widths, slots and shifts are uniform per block, so one branch-free
// code path serves all bitwidths and the accumulators never move.  Codes and
// scale/zero records reach a per-wave LDS stage by global->LDS loads issued
// as soon as the previous block's last code slot has been read; the shared
// activation tile (128 tokens x 128 columns per K step) reaches LDS one step
// ahead, double buffered, in MFMA fragment order (one 1 KiB fragment per 16
// tokens x 32 columns, lane l's 16 bytes at 16 l), so every A read is one
// conflict-free 16-byte LDS read.  Workgroups are mapped XCD by XCD to
// contiguous, grouped stretches of tiles so that each XCD's L2 sees the reuse
// of activation rows and weight blocks.

#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

namespace {

constexpr int kBM = 128;                 // tokens per tile
constexpr int kWaves = 8;                // waves per workgroup, one block row each
constexpr int kBN = 64 * kWaves;         // output rows per tile
constexpr int kMT = kBM / 16;            // 16-token tiles per tile
constexpr int kGroupM = 8;

struct PrefillArgs {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  const _Float16* x;
  _Float16* y;
  float* part;       // K split: fp32 partial y per segment [kseg][M][N] (zero between calls)
  int N, K, M, nbr, nbc, tiles_m, tiles_n, per_xcd, cus_xcd;
  int kseg, seg_cols;   // K segments per tile (1: no split) and block columns per segment
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// One global->LDS load of 16 bytes per lane from sbase + voff: lane l's bytes
// land at LDS address lds + 16 l.  No output registers; completion is
// awaited with an explicit vmcnt wait before the LDS is read.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_all_loads() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One K step of one wave for a block of bitwidth b (planes W0 + W1): the
// B operands of column tile kt + 1 are formed while the 8 x 4 MFMAs of column
// tile kt run.  Tile 4 kt + rt is field (4 kt + rt) % (16 / W) of slot
// (4 kt + rt) / (16 / W) of a plane of width W -- one slot per column tile
// and plane -- and the second plane holds the high bits.  The plane widths,
// slots and shifts are uniform per block, so one branch-free code path
// serves every bitwidth (a missing second plane has an empty mask) and the
// accumulators stay in the matrix-core registers.
template <int MT, class Refill>
__device__ __forceinline__ void kstep(int b, const u32x4* __restrict__ st, const u32x4* __restrict__ xb, int lane,
                                      f32x4 (&acc)[MT][4], Refill&& refill) {
  const int W0 = b == 3 ? 2 : (b >= 4 ? 4 : b);
  const int W1 = b == 3 ? 1 : (b == 6 ? 2 : (b == 8 ? 4 : 0));
  const int L0 = W0 == 4 ? 2 : (W0 == 2 ? 3 : 4);   // log2(16 / W0)
  const int L1 = W1 == 4 ? 2 : (W1 == 2 ? 3 : 4);
  const uint32_t M0 = ((1u << W0) - 1u) * 0x00010001u;
  const uint32_t M1 = (((1u << W1) - 1u) * 0x00010001u) << W0;
  const u32x4 sz = st[512 + lane];
  half2v s2[4], z2[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const uint32_t e = sz[rt];
    s2[rt] = as_half2((e & 0xffffu) * 0x00010001u);
    const _Float16 nz = -((_Float16)1024.0f + __builtin_bit_cast(_Float16, (unsigned short)(e >> 16)));
    z2[rt] = half2v{nz, nz};   // exact: an integer below 2048
  }
  auto deq = [&](int kt, u32x4 (&B)[4]) {
    const u32x4 c0 = st[64 * ((4 * kt) >> L0) + lane];
    const u32x4 c1 = st[64 * (W0 + ((4 * kt) >> L1)) + lane];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int u = 4 * kt + rt;
      const uint32_t s0 = uint32_t(W0 * (u & ((1 << L0) - 1)));
      const uint32_t r1 = uint32_t(W1 * (u & ((1 << L1) - 1)) - W0) & 31u;   // rotate the field to bit W0
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = ((c0[k] >> s0) & M0) | kMagicPair;
        const uint32_t q = (__builtin_amdgcn_alignbit(c1[k], c1[k], r1) & M1) | lo;
        o[k] = as_u32((as_half2(q) + z2[rt]) * s2[rt]);
      }
      B[rt] = u32x4{o[0], o[1], o[2], o[3]};
    }
  };
  u32x4 B[2][4];
  deq(0, B[0]);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    if (kt < 3) deq(kt + 1, B[(kt + 1) & 1]);
    if (kt == 2) refill();   // every code slot of the block has been read
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const half8 A = __builtin_bit_cast(half8, xb[(4 * mt + kt) * 64 + lane]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = mfma16(A, __builtin_bit_cast(half8, B[kt & 1][rt]), acc[mt][rt]);
    }
    // Interleave: two MFMAs, then up to eight vector instructions (the next
    // tile's dequantization), so both pipes stay fed; left to itself the
    // scheduler clumps them (+2-3 % on the Llama-3-70B MLP shapes).
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
    }
  }
}

// Tiles of XCD x are [first, first + count).  When they fill whole rounds
// of the XCD's CUs (one workgroup per CU) and leave a last round at most half
// full, the last `split` tiles run as two 64-token halves each, so that last
// round keeps every CU busy for half as long instead of half the CUs for a
// whole tile.  The halves need no reduction: they own disjoint outputs.
struct XcdWork {
  int first, count, split;
};
__host__ __device__ inline XcdWork xcd_work(int ntiles, int per_xcd, int cus_xcd, int x) {
  XcdWork w;
  w.first = x * per_xcd;
  w.count = max(0, min(per_xcd, ntiles - w.first));
  const int r = w.count % cus_xcd;
  w.split = (w.count >= cus_xcd && r > 0 && 2 * r <= cus_xcd) ? r : 0;
  return w;
}

// The results of one wave (block row br, tokens m0 + 16 mt + 4 g + v) of a
// tile: rounded to fp16 and stored, or with a K split stored as this
// segment's fp32 partials (split_reduce_kernel adds them afterwards).
template <int MT>
__device__ __forceinline__ void tile_epilogue(const PrefillArgs& a, const f32x4 (&acc)[MT][4], int m0, int br,
                                              bool has_rows, int seg) {
  if (!has_rows) return;
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  float* pp = a.part + size_t(seg) * size_t(a.M) * size_t(a.N);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 16 * mt + 4 * g + v;
      if (m >= a.M) continue;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const size_t o = size_t(m) * a.N + br * 64 + 16 * rt + r16;
        if (a.kseg == 1)
          a.y[o] = (_Float16)acc[mt][rt][v];
        else
          pp[o] = acc[mt][rt][v];
      }
    }
}

// y = the sum of the kseg partials, in segment order (so the result does not
// depend on the order the segments ran in), rounded once; the partials are
// cleared, so the workspace is zero again after the call.  Four outputs per
// thread (N is a multiple of 64).
__global__ __launch_bounds__(256) void split_reduce_kernel(float* part, _Float16* y, size_t quads, int kseg) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= quads) return;
  f32x4* p4 = reinterpret_cast<f32x4*>(part);
  f32x4 t = p4[i];
  p4[i] = f32x4{0, 0, 0, 0};
  for (int sg = 1; sg < kseg; ++sg) {
    t += p4[size_t(sg) * quads + i];
    p4[size_t(sg) * quads + i] = f32x4{0, 0, 0, 0};
  }
  typedef _Float16 half4v __attribute__((ext_vector_type(4)));
  reinterpret_cast<half4v*>(y)[i] = half4v{(_Float16)t[0], (_Float16)t[1], (_Float16)t[2], (_Float16)t[3]};
}

// Work item j of XCD x: a whole tile (t, seg) of the K split, or one 64-token
// half of a tile of the last round (no K split then).  Returns false for
// items past the XCD's work.
struct WorkItem {
  int tm, tn, m0, seg, tile, half;
};
__device__ __forceinline__ bool work_item(const PrefillArgs& a, int bid, int bm, WorkItem& it) {
  const int ntiles = a.tiles_m * a.tiles_n * a.kseg;
  const XcdWork w = xcd_work(ntiles, a.per_xcd, a.cus_xcd, bid & 7);
  const int j = bid >> 3, whole = w.count - (a.kseg == 1 ? w.split : 0);
  int t;
  it.half = -1;
  if (j < whole) {
    t = w.first + j;
  } else {
    const int v = j - whole;
    if (a.kseg != 1 || v >= 2 * w.split) return false;
    t = w.first + whole + (v >> 1);
    it.half = v & 1;
  }
  it.seg = t % a.kseg;
  t /= a.kseg;
  it.tile = t;
  const int gsize = kGroupM * a.tiles_n;
  const int first_m = (t / gsize) * kGroupM;
  const int gm = min(kGroupM, a.tiles_m - first_m);
  it.tm = first_m + (t % gsize) % gm;
  it.tn = (t % gsize) / gm;
  it.m0 = it.tm * bm + (it.half > 0 ? bm / 2 : 0);
  return it.half < 0 || it.m0 < a.M;
}

// One tile of MT 16-token tiles (tokens m0 ...) x 512 rows (block rows
// 8 tn ...): wave w owns block row 8 tn + w.
template <int MT>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int m0, int tn, u32x4 (*xs)[kMT * 4 * 64],
                                             u32x4 (*stage)[9 * 64], int seg) {
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const bool has_rows = tn * kWaves + wave < a.nbr;
  // waves past the last block row repeat it (their outputs are not stored),
  // so the step loop has no branch around the matrix-core work
  const int br = min(tn * kWaves + wave, a.nbr - 1);   // this wave's block row

  // wave w loads the activation fragments (mt, kt) = (f' / 4, f' % 4) with
  // f' = kFrag w + f; token rows past M repeat row M - 1 (their outputs are
  // not stored)
  constexpr int kFrag = MT * 4 / kWaves;
  uint32_t xoff[kFrag];
#pragma unroll
  for (int f = 0; f < kFrag; ++f) {
    const int fr = kFrag * wave + f, mt = fr >> 2, kt = fr & 3;
    const int m = min(m0 + 16 * mt + r16, a.M - 1);
    xoff[f] = uint32_t((size_t(m) * a.K + 32 * kt + 8 * g) * 2);
  }
  const uint32_t xs_lds = lds_addr(&xs[0][0]);
  auto load_x = [&](int bc, int buf) {
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
      dma16(a.x, xoff[f] + uint32_t(bc) * 256,
            xs_lds + uint32_t(buf) * (kMT * 4 * 1024) + uint32_t(kFrag * wave + f) * 1024);
  };

  // this wave's block row: bitwidths and code offsets 64 columns at a time
  // this workgroup's K segment: block columns [bc0, bc1); bitwidths and
  // offsets come 64 block columns at a time from window base wb
  const int bc0 = seg * a.seg_cols, bc1 = min(a.nbc, bc0 + a.seg_cols);
  int wb = bc0;
  const size_t row_blk = size_t(br) * a.nbc;
  int bvec = 0, ovec = 0;
  auto load_meta = [&](int col0) {
    const int c = min(col0 + lane, a.nbc - 1);
    bvec = int(a.bits[row_blk + c]);
    ovec = int(a.offs[row_blk + c]);
  };
  const uint32_t st_lds = uint32_t(uniform(int(lds_addr(&stage[wave][0]))));
  auto load_block = [&](int bc) {   // codes and scale/zero of block (br, bc) into the stage
    const int bj = uniform(__builtin_amdgcn_readlane(bvec, bc - wb));
    const uint8_t* cb = a.codes + size_t(uniform(__builtin_amdgcn_readlane(ovec, bc - wb))) * 1024;
    for (int q = 0; q < bj; ++q) dma16(cb + 1024 * q, 16 * lane, st_lds + 1024 * q);
    dma16(a.sz + (row_blk + bc) * 64, 16 * r16, st_lds + 8192);
  };

  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  load_meta(wb);
  load_x(bc0, 0);
  load_block(bc0);
  for (int bc = bc0; bc < bc1; ++bc) {
    const int buf = (bc - bc0) & 1;
    wait_all_loads();   // this wave's fragments and block of step bc
    __syncthreads();    // every wave's fragments of step bc are in LDS; step bc - 1's reads are done
    const int b = uniform(__builtin_amdgcn_readlane(bvec, bc - wb));   // before the next window
    const bool more = bc + 1 < bc1;
    if (more) {
      load_x(bc + 1, buf ^ 1);
      if (bc + 1 - wb == 64) {
        wb += 64;
        load_meta(wb);
      }
    }
    // the next block's codes go into the stage as soon as this block's last
    // code slot has been read (inside the step, before its last MFMAs)
    auto refill = [&]() {
      if (more) {
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        load_block(bc + 1);
      }
    };
    kstep<MT>(b, &stage[wave][0], &xs[buf][0], lane, acc, refill);
  }
  tile_epilogue<MT>(a, acc, m0, br, has_rows, seg);
}


__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs a) {
  // activation tiles, double buffered: fragment (mt, kt) at 1 KiB (4 mt + kt)
  __shared__ u32x4 xs[2][kMT * 4 * 64];
  // per wave: a block's codes (up to 8 KiB) and its scale/zero entries (1 KiB)
  __shared__ u32x4 stage[kWaves][9 * 64];

  // XCD-aware tile order: the hardware deals workgroups round robin to the 8
  // XCDs, so workgroup i runs on XCD i % 8; give each XCD a contiguous range
  // of work items (tiles, or K segments of tiles), walked in groups of
  // kGroupM token tiles, whole tiles first and the split halves (if any)
  // last.
  WorkItem it;
  if (!work_item(a, int(blockIdx.x), kBM, it)) return;
  // the item is the same for the whole workgroup: keep it in scalar registers
  const int m0 = uniform(it.m0), tn = uniform(it.tn), seg = uniform(it.seg);
  if (it.half < 0 && a.M - m0 > kBM / 2) {
    prefill_tile<kMT>(a, m0, tn, xs, stage, seg);
  } else {   // a 64-token half, or a tile whose tokens fit in its first half
    prefill_tile<kMT / 2>(a, m0, tn, xs, stage, seg);
  }
}

// ---------------------------------------------------------------------------
// 64x64 blocks (version-2 image, the other GPU block size of the ScaleBITS
// explainer page, section 4.2).  The same workgroup and tile as above; K
// advances one 64-column block column per step.  A plane of width W is W
// half-slots of 512 bytes: lane l's 8 bytes of half-slot j are two words d
// whose field f holds the column pair c = 2 d + f / P of tile
// u = 4 kt + rt = j P + f % P (P = 8 / W, kt = 0, 1).  So the B operand of
// tile u takes words 0, 0, 1, 1 of half-slot u / P at fields u % P,
// u % P + P, u % P, u % P + P.  Per wave the stage holds a block's codes
// (up to eight half-slots, 4 KiB) and its scale/zero entries (1 KiB).
constexpr int kStage64 = 5 * 64;   // u32x4 per wave

template <int MT, class Refill>
__device__ __forceinline__ void kstep64(int b, const u32x4* __restrict__ st, const u32x4* __restrict__ xb, int lane,
                                        f32x4 (&acc)[MT][4], Refill&& refill) {
  const int W0 = b == 3 ? 2 : (b >= 4 ? 4 : b);
  const int W1 = b == 3 ? 1 : (b == 6 ? 2 : (b == 8 ? 4 : 0));
  const int L0 = W0 == 4 ? 1 : (W0 == 2 ? 2 : 3);   // log2(8 / W0)
  const int L1 = W1 == 4 ? 1 : (W1 == 2 ? 2 : 3);
  const uint32_t M0 = ((1u << W0) - 1u) * 0x00010001u;
  const uint32_t M1 = (((1u << W1) - 1u) * 0x00010001u) << W0;
  const uint2* st2 = reinterpret_cast<const uint2*>(st);   // half-slot j: st2[64 j + lane]
  const u32x4 sz = st[256 + lane];
  half2v s2[4], z2[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const uint32_t e = sz[rt];
    s2[rt] = as_half2((e & 0xffffu) * 0x00010001u);
    const _Float16 nz = -((_Float16)1024.0f + __builtin_bit_cast(_Float16, (unsigned short)(e >> 16)));
    z2[rt] = half2v{nz, nz};   // exact: an integer below 2048
  }
  auto deq = [&](int kt, u32x4 (&B)[4]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int u = 4 * kt + rt;
      const int P0 = 1 << L0, P1 = 1 << L1;
      const uint2 w = st2[64 * (u >> L0) + lane];
      const uint2 h = st2[64 * (W0 + (u >> L1)) + lane];
      const uint32_t s0 = uint32_t(W0 * (u & (P0 - 1)));          // fields of column pairs 0 and 2
      const uint32_t s0b = s0 + uint32_t(W0 * P0);                // 1 and 3 (8 bits higher)
      const uint32_t r1 = uint32_t(W1 * (u & (P1 - 1)) - W0) & 31u;
      const uint32_t r1b = uint32_t(W1 * (u & (P1 - 1)) + W1 * P1 - W0) & 31u;
      const uint32_t src0[4] = {w.x, w.x, w.y, w.y}, src1[4] = {h.x, h.x, h.y, h.y};
      const uint32_t sh0[4] = {s0, s0b, s0, s0b}, sh1[4] = {r1, r1b, r1, r1b};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = ((src0[k] >> sh0[k]) & M0) | kMagicPair;
        const uint32_t q = (__builtin_amdgcn_alignbit(src1[k], src1[k], sh1[k]) & M1) | lo;
        o[k] = as_u32((as_half2(q) + z2[rt]) * s2[rt]);
      }
      B[rt] = u32x4{o[0], o[1], o[2], o[3]};
    }
  };
  u32x4 B[2][4];
  deq(0, B[0]);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    if (kt == 0) {
      deq(1, B[1]);
      refill();   // every code slot of the block has been read
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const half8 A = __builtin_bit_cast(half8, xb[(2 * mt + kt) * 64 + lane]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[mt][rt] = mfma16(A, __builtin_bit_cast(half8, B[kt][rt]), acc[mt][rt]);
    }
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
    }
  }
}

// One tile of MT 16-token tiles (tokens m0 ...) x 512 rows of a 64x64 image.
template <int MT>
__device__ __forceinline__ void prefill64_tile(const PrefillArgs& a, int m0, int tn, u32x4 (*xs)[kMT * 2 * 64],
                                               u32x4 (*stage)[kStage64], int seg) {
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const bool has_rows = tn * kWaves + wave < a.nbr;
  const int br = min(tn * kWaves + wave, a.nbr - 1);

  // activation fragments of one 64-column step: (mt, kt) at 1 KiB (2 mt + kt)
  constexpr int kFrag = MT * 2 / kWaves;
  uint32_t xoff[kFrag];
#pragma unroll
  for (int f = 0; f < kFrag; ++f) {
    const int fr = kFrag * wave + f, mt = fr >> 1, kt = fr & 1;
    const int m = min(m0 + 16 * mt + r16, a.M - 1);
    xoff[f] = uint32_t((size_t(m) * a.K + 32 * kt + 8 * g) * 2);
  }
  const uint32_t xs_lds = lds_addr(&xs[0][0]);
  auto load_x = [&](int bc, int buf) {
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
      dma16(a.x, xoff[f] + uint32_t(bc) * 128,
            xs_lds + uint32_t(buf) * (kMT * 2 * 1024) + uint32_t(kFrag * wave + f) * 1024);
  };

  // this workgroup's K segment: block columns [bc0, bc1); bitwidths and
  // offsets come 64 block columns at a time from window base wb
  const int bc0 = seg * a.seg_cols, bc1 = min(a.nbc, bc0 + a.seg_cols);
  int wb = bc0;
  const size_t row_blk = size_t(br) * a.nbc;
  int bvec = 0, ovec = 0;
  auto load_meta = [&](int col0) {
    const int c = min(col0 + lane, a.nbc - 1);
    bvec = int(a.bits[row_blk + c]);
    ovec = int(a.offs[row_blk + c]);
  };
  const uint32_t st_lds = uint32_t(uniform(int(lds_addr(&stage[wave][0]))));
  auto load_block = [&](int bc) {   // codes (b half-slots) and scale/zero of block (br, bc)
    const int bj = uniform(__builtin_amdgcn_readlane(bvec, bc - wb));
    const uint8_t* cb = a.codes + size_t(uniform(__builtin_amdgcn_readlane(ovec, bc - wb))) * 512;
    for (int q = 0; q + 1 < bj; q += 2) dma16(cb + 512 * q, 16 * lane, st_lds + 512 * q);   // two half-slots
    if (bj & 1) {   // the last half-slot: 512 bytes from the first 32 lanes
      if (lane < 32) dma16(cb + 512 * (bj - 1), 16 * lane, st_lds + 512 * (bj - 1));
    }
    dma16(a.sz + (row_blk + bc) * 64, 16 * r16, st_lds + 4096);
  };

  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  load_meta(wb);
  load_x(bc0, 0);
  load_block(bc0);
  for (int bc = bc0; bc < bc1; ++bc) {
    const int buf = (bc - bc0) & 1;
    wait_all_loads();   // this wave's fragments and block of step bc
    __syncthreads();    // every wave's fragments of step bc are in LDS; step bc - 1's reads are done
    const int b = uniform(__builtin_amdgcn_readlane(bvec, bc - wb));   // before the next window
    const bool more = bc + 1 < bc1;
    if (more) {
      load_x(bc + 1, buf ^ 1);
      if (bc + 1 - wb == 64) {
        wb += 64;
        load_meta(wb);
      }
    }
    auto refill = [&]() {
      if (more) {
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        load_block(bc + 1);
      }
    };
    kstep64<MT>(b, &stage[wave][0], &xs[buf][0], lane, acc, refill);
  }
  tile_epilogue<MT>(a, acc, m0, br, has_rows, seg);
}

__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill64_kernel(
    PrefillArgs a) {
  __shared__ u32x4 xs[2][kMT * 2 * 64];        // activations, double buffered: 16 KiB per 64-column step
  __shared__ u32x4 stage[kWaves][kStage64];     // per wave: codes (4 KiB) + scale/zero (1 KiB)
  WorkItem it;
  if (!work_item(a, int(blockIdx.x), kBM, it)) return;
  const int m0 = uniform(it.m0), tn = uniform(it.tn), seg = uniform(it.seg);
  if (it.half < 0 && a.M - m0 > kBM / 2) {
    prefill64_tile<kMT>(a, m0, tn, xs, stage, seg);
  } else {
    prefill64_tile<kMT / 2>(a, m0, tn, xs, stage, seg);
  }
}

// Compute units of the current device (the runtime answers from its cached
// device properties, so this is cheap host work per launch).
int compute_units() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  return v;
}

}  // namespace

int prefill_tiles(int N, int M) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

int device_compute_units() { return compute_units(); }

// K split: when the tile grid would fill at most half of the CUs, each tile
// is cut into up to 16 K segments of at least 1024 columns, as many as fill
// the CUs once, and as many as the caller's workspace holds (kseg fp32
// partials of y).
PrefillPlan prefill_plan(int N, int K, int M, int bc, size_t ws_bytes) {
  PrefillPlan p;
  const int nbc = K / bc, nbr = N / 64;
  const int tiles = ((M + kBM - 1) / kBM) * ((nbr * 64 + kBN - 1) / kBN);
  const int cus = compute_units();
  int k = 1;
  if (2 * tiles <= cus) k = min(min(cus / tiles, 16), max(1, nbc / (1024 / bc)));
  auto need = [&](int kk) { return kk > 1 ? size_t(kk) * size_t(M) * size_t(N) * 4 : size_t(0); };
  while (k > 1 && need(k) > ws_bytes) --k;
  p.seg_cols = (nbc + k - 1) / k;
  p.kseg = (nbc + p.seg_cols - 1) / p.seg_cols;
  p.ws_bytes = need(p.kseg);
  p.tiles = tiles;
  return p;
}

int launch_prefill(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* workspace,
                   const PrefillPlan& plan, void* stream) {
  PrefillArgs a;
  a.bits = im.bits;
  a.offs = im.offs;
  a.sz = im.sz;
  a.codes = im.codes;
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.N = im.N;
  a.K = im.K;
  a.M = M;
  a.nbr = im.nbr;
  a.nbc = im.nbc;
  a.kseg = plan.kseg;
  a.seg_cols = plan.kseg > 1 ? plan.seg_cols : im.nbc;
  a.part = plan.kseg > 1 ? static_cast<float*>(workspace) : nullptr;
  a.tiles_m = (M + kBM - 1) / kBM;
  a.tiles_n = (im.nbr * 64 + kBN - 1) / kBN;
  const int ntiles = a.tiles_m * a.tiles_n * a.kseg;
  a.per_xcd = (ntiles + 7) / 8;
  a.cus_xcd = max(1, compute_units() / 8);
  int items = 0;
  for (int x = 0; x < 8; ++x) {
    const XcdWork w = xcd_work(ntiles, a.per_xcd, a.cus_xcd, x);
    items = max(items, w.count + (a.kseg == 1 ? w.split : 0));
  }
  const dim3 grid(unsigned(8 * items)), block(kWaves * 64);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (im.bc == 64)
    hipLaunchKernelGGL(prefill64_kernel, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(prefill_kernel, grid, block, 0, s, a);
  if (plan.kseg > 1) return launch_split_reduce(a.part, y, M, im.N, plan.kseg, stream);
  return int(hipGetLastError());
}

int launch_split_reduce(float* part, uint16_t* y, int M, int N, int kseg, void* stream) {
  const size_t quads = size_t(M) * size_t(N) / 4;
  hipLaunchKernelGGL(split_reduce_kernel, dim3(unsigned((quads + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), part, reinterpret_cast<_Float16*>(y), quads, kseg);
  return int(hipGetLastError());
}

}  // namespace gbb
