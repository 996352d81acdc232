// Prefill kernel: y = x . dequant(W)^T for larger M over the block image.
//
// Large batched products are compute bound and the dequantization must be
// hidden under the matrix math (MixLLM page, section 2.2 on batched serving
// and section 3.3 on overlapping dequantization with the matrix product).
//
// gfx950 design: a workgroup computes a 128 (tokens) x 128 (output rows) tile
// of y and walks K one 128-column block column at a time.  Per step its four
// waves (a) copy the 128x128 fp16 activation tile into LDS and (b) dequantize
// the two 64x128 weight blocks of the tile into LDS: a lane unpacks the codes
// it loaded (one coalesced 16-byte load per KiB of codes), forms 1024 + q with
// the fp16 magic, subtracts 1024 + z and multiplies by s with packed fp16
// arithmetic -- exactly fp16((q - z) * s), since q - z is an exact small
// integer and the product is rounded once.  Then each wave runs
// v_mfma_f32_16x16x32_f16 on its 64x64 sub-tile from LDS.  Both LDS tiles are
// XOR-swizzled on 16-byte chunks so that the 16 rows a lane group touches at
// one column fall in distinct banks.  Workgroups are mapped XCD by XCD to
// contiguous, grouped stretches of tiles so that each XCD's L2 sees the reuse
// of activation rows and weight blocks.
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

namespace {

constexpr int kBM = 128;  // tokens per tile
constexpr int kBN = 128;  // output rows per tile (two block rows)
constexpr int kGroupM = 8;

struct PrefillArgs {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  const _Float16* x;
  _Float16* y;
  int N, K, M, nbr, nbc, tiles_m, tiles_n, per_xcd;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

// Code pairs of the column half h (column tiles kt = 2h, 2h + 1) of one plane
// of width W: tile 4 kt + rt is field (4 kt + rt) % (16 / W) of slot
// (4 kt + rt) / (16 / W), so the half lives in the slots [8h / NP, ..] and,
// for W = 1, in the byte of each half word selected by h.
template <int W>
struct PlaneHalf {
  static constexpr int NP = 16 / W;
  static constexpr int NS = W == 1 ? 1 : 8 / NP;  // slots of one half
  uint32_t w[NS][4];
  __device__ __forceinline__ void load(const uint8_t* cb, int h) {
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const u32x4 v = ld16(reinterpret_cast<const uint32_t*>(cb + 1024 * ((8 * h) / NP + t)));
#pragma unroll
      for (int c = 0; c < 4; ++c) w[t][c] = W == 1 ? v[c] >> (8 * h) : v[c];
    }
  }
  // pair of word c of local tile ul = 4 (kt - 2h) + rt
  __device__ __forceinline__ uint32_t pair(int ul, int c) const {
    return (w[ul / NP][c] >> (W * (ul % NP))) & (((1u << W) - 1u) * 0x00010001u);
  }
};

// Dequantize the column half h of one block into LDS rows base_row + 0..63:
// exactly fp16((q - z) s), as (1024 + q) - (1024 + z) is an exact small
// integer in fp16 and the product is rounded once.
template <int W0, int W1>
__device__ __forceinline__ void dequant_half(const uint8_t* __restrict__ blk_codes, const uint32_t* __restrict__ blk_sz,
                                             int h, int lane, u32x4* __restrict__ lds, int base_row) {
  const int g = lane >> 4, r16 = lane & 15;
  const uint8_t* cb = blk_codes + 16 * lane;
  PlaneHalf<W0> p0;
  PlaneHalf<W1 ? W1 : 1> p1;
  p0.load(cb, h);
  if constexpr (W1 != 0) p1.load(cb + 1024 * W0, h);
  // entry 4 r16 + rt of the block's scale/zero record is row 16 rt + r16
  const u32x4 sz = ld16(blk_sz + 4 * r16);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const uint32_t e = sz[rt];
    const half2v s2 = as_half2((e & 0xffffu) * 0x00010001u);
    const _Float16 zf = __builtin_bit_cast(_Float16, (unsigned short)(e >> 16));
    const _Float16 nz = -((_Float16)1024.0f + zf);  // exact: an integer below 2048
    const half2v z2 = {nz, nz};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ul = 4 * k2 + rt;
      uint32_t o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t q = p0.pair(ul, c);
        if constexpr (W1 != 0) q |= p1.pair(ul, c) << W0;
        const half2v v = (as_half2(q | kMagicPair) + z2) * s2;
        o[c] = as_u32(v);
      }
      lds[swz(base_row + 16 * rt + r16, 4 * (2 * h + k2) + g)] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  __shared__ u32x4 xs[kBM * 16];
  __shared__ u32x4 ws[kBN * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  // XCD-aware tile order: the hardware deals workgroups round robin to the 8
  // XCDs, so workgroup i runs on XCD i % 8; give each XCD a contiguous range
  // of tiles, walked in groups of kGroupM row tiles.
  const int bid = blockIdx.x;
  const int t = (bid & 7) * a.per_xcd + (bid >> 3);
  const int ntiles = a.tiles_m * a.tiles_n;
  if (t >= ntiles) return;
  const int gsize = kGroupM * a.tiles_n;
  const int first_m = (t / gsize) * kGroupM;
  const int gm = min(kGroupM, a.tiles_m - first_m);
  const int tm = first_m + (t % gsize) % gm;
  const int tn = (t % gsize) / gm;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  // weight work of this wave: block row n0/64 + (wave >> 1), column half wave & 1
  const int br = (n0 >> 6) + (wave >> 1);
  const int hk = wave & 1;
  const int wrow = 64 * (wave >> 1);

  for (int bc = 0; bc < a.nbc; ++bc) {
    u32x4 xr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = j * 256 + tid, row = idx >> 4, c = idx & 15;
      const int m = m0 + row;
      xr[j] = u32x4{0, 0, 0, 0};
      if (m < a.M) xr[j] = ld16(a.x + size_t(m) * a.K + size_t(bc) * 128 + 8 * c);
    }
    __syncthreads();  // the previous step's MFMA reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = j * 256 + tid, row = idx >> 4, c = idx & 15;
      xs[swz(row, c)] = xr[j];
    }
    if (br < a.nbr) {
      const int blk = br * a.nbc + bc;
      const int b = uniform(a.bits[blk]);
      const uint8_t* cb = a.codes + size_t(uniform(int(a.offs[blk]))) * 1024;
      const uint32_t* sb = a.sz + size_t(blk) * 64;
      switch (b) {
        case 1: dequant_half<1, 0>(cb, sb, hk, lane, ws, wrow); break;
        case 2: dequant_half<2, 0>(cb, sb, hk, lane, ws, wrow); break;
        case 3: dequant_half<2, 1>(cb, sb, hk, lane, ws, wrow); break;
        case 4: dequant_half<4, 0>(cb, sb, hk, lane, ws, wrow); break;
        case 6: dequant_half<4, 2>(cb, sb, hk, lane, ws, wrow); break;
        default: dequant_half<4, 4>(cb, sb, hk, lane, ws, wrow); break;
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) ws[swz(wrow + 16 * rt + r16, 4 * (2 * hk + k2) + g)] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 A[4], B[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = __builtin_bit_cast(half8, xs[swz(wm * 64 + i * 16 + r16, 4 * ks + g)]);
        B[i] = __builtin_bit_cast(half8, ws[swz(wn * 64 + i * 16 + r16, 4 * ks + g)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(A[i], B[j], acc[i][j]);
    }
  }

  // lane holds D[token 4 g + v][row r16] of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * 64 + i * 16 + 4 * g + v;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + r16;
        if (n < a.N) a.y[size_t(m) * a.N + n] = (_Float16)acc[i][j][v];
      }
    }
  }
}

}  // namespace

int launch_prefill(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* stream) {
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
  a.tiles_m = (M + kBM - 1) / kBM;
  a.tiles_n = (im.nbr * 64 + kBN - 1) / kBN;
  const int ntiles = a.tiles_m * a.tiles_n;
  a.per_xcd = (ntiles + 7) / 8;
  const dim3 grid(unsigned(8 * a.per_xcd)), block(256);
  hipLaunchKernelGGL(prefill_kernel, grid, block, 0, static_cast<hipStream_t>(stream), a);
  return int(hipGetLastError());
}

}  // namespace gbb
