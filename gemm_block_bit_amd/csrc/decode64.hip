// Decode kernels over images of 64x64 blocks: y = x . dequant(W)^T for
// M <= 32 (larger batches run as 32-token chunks of them).
//
// The ScaleBITS explainer page names 64x64 as the other GPU block size
// (section 4.2); each block has one bitwidth, and each (row, 64-column
// group) one fp16 scale and zero (MixLLM page, section 2.1).
//
// The design is that of the 64x128 decode kernels with half-size records: a
// block is a 256-byte scale/zero record, 64 activation columns and b
// half-slots of 512 bytes of codes.  A half-slot holds two words per lane,
// and each word read at two field positions gives two words of an MFMA B
// operand, so unpacking stays one AND per operand word (shift included) and
// the subnormal q 2^(o - 24) trick carries over unchanged; a block covers
// two 32-column k tiles.  Rings count 512-byte slots; a half-slot or a
// 4-token activation slot (512 bytes) is one 16-byte global->LDS load by the
// wave's first 32 lanes.
#include "decode_common.h"

namespace gbb {

namespace {

constexpr uint32_t kHS = 512;   // bytes per half-slot (ring slot)

// MFMAs of one plane of width W of a 64x64 block, half-slots w[0..W) (two
// words per lane each).  Tile 4 kt + rt (kt = 0, 1) is operand u of the
// plane: half-slot u / (8 / W), field i = u % (8 / W); B operand word c is
// field (c & 1) (8 / W) + i of word c >> 1, moved to offset o = off(rt).
template <int W, int MT>
__device__ __forceinline__ void plane_mma64(const uint2 (&w)[W], const half8 (&xa)[2][MT], f32x4 (&c)[4][MT]) {
  using G = PlaneGeom<W>;
  constexpr int P = 8 / W;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int u = 4 * kt + rt, j = u / P, i = u % P;
      const int o = G::off(rt), sh0 = W * i - o, sh1 = W * (P + i) - o;
      const uint32_t mask = (((1u << W) - 1u) * 0x00010001u) << o;
      const half8 B = as_half8((w[j].x >> sh0) & mask, (w[j].x >> sh1) & mask, (w[j].y >> sh0) & mask,
                               (w[j].y >> sh1) & mask);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) c[rt][mt] = mfma16(xa[kt][mt], B, c[rt][mt]);
    }
}

// A block column's activation fragments from the ring: 4-token slots of 64
// columns (128 bytes per token); lane holds tokens 16 mt + r16 (rows past M
// repeat row M - 1), columns 32 kt + 8 g ... + 7.
template <int MT, int RS>
__device__ __forceinline__ void read_x64(const u32x4* ring, uint32_t xb, int M, half8 (&xa)[2][MT]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(16 * mt + r16, M - 1);
    const u32x4* xr = ring + (wrap<RS, kHS>(xb + kHS * (m >> 2)) >> 4);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) xa[kt][mt] = __builtin_bit_cast(half8, xr[8 * (m & 3) + 4 * kt + g]);
  }
}

// One block of planes W0 (shift 0) and W1 (shift W0; 0 = none): scale/zero
// record at ring byte offset szb, codes at cb; `refill` runs once the LDS
// reads are done.  acc += s (sum over planes of 2^(24 + shift - o) C - z X),
// with 2^(24 - o) of the first plane folded into s and z (exact).
template <int W0, int W1, int MT, int RS, class Refill>
__device__ __forceinline__ void block_core64(const u32x4* ring, uint32_t szb, uint32_t cb, const half8 (&xa)[2][MT],
                                             f32x4 (&acc)[4][MT], Refill&& refill) {
  const int lane = threadIdx.x & 63, r16 = lane & 15;
  const uint2* ring2 = reinterpret_cast<const uint2*>(ring);
  const u32x4 sz = ring[(wrap<RS, kHS>(szb) >> 4) + r16];
  uint2 w0[W0], w1[W1 ? W1 : 1];
#pragma unroll
  for (int q = 0; q < W0; ++q) w0[q] = ring2[(wrap<RS, kHS>(cb + kHS * q) >> 3) + lane];
#pragma unroll
  for (int q = 0; q < W1; ++q) w1[q] = ring2[(wrap<RS, kHS>(cb + kHS * (W0 + q)) >> 3) + lane];
  wait_lds();
  refill();

  f32x4 c0[4][MT], c1[4][MT], xsum[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xsum[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) c0[rt][mt] = c1[rt][mt] = f32x4{0, 0, 0, 0};
  }
  const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xsum[mt] = mfma16(xa[kt][mt], ones, xsum[mt]);
  plane_mma64<W0, MT>(w0, xa, c0);
  if constexpr (W1 != 0) plane_mma64<W1, MT>(w1, xa, c1);
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

// Ring slots (512 bytes) per wave: a block takes 1 + ceil(M / 4) + b slots
// (at most 11 for M <= 8, 13 for M <= 16, 17 for M <= 32).  The rings take
// the LDS of the 64x128 kernels' rings: 48, 52 and 128 KiB per four-wave
// workgroup.
constexpr int kRing64_8 = 24;
constexpr int kRing64_16 = 26;
constexpr int kRing64_32 = 64;

// Workgroup wg: block row wg / nseg, K segment wg % nseg; a.nbc and
// a.seg_cols count 64-column blocks.
template <int NW, int MT, int RS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 3))) void decode64_kernel(DecodeArgs a) {
  constexpr int R = RS;
  static_assert(1 + 4 * MT + 8 <= R, "a block's records fit in the ring");
  const int wg = int(blockIdx.x);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int br = int(unsigned(wg) / unsigned(a.nseg)), seg = wg - br * a.nseg;
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;
  const int M = a.M;
  const int nx = (M + 3) / 4;   // activation slots (and loads) per block
  // lanes 0 ... 31 load a 4-token activation slot: token 4 xi + lane / 8,
  // columns 8 (lane % 8) ... + 7
  uint32_t xoff[8];
#pragma unroll
  for (int xi = 0; xi < 8; ++xi) xoff[xi] = uint32_t(min(4 * xi + ((lane >> 3) & 3), M - 1)) * uint32_t(2 * a.K) + 16 * (lane & 7);

  __shared__ u32x4 lds[NW * R * 32];   // per-wave rings; reused for the reduction
  const u32x4* ring = lds + wave * R * 32;
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
    wait_vmcnt<0>();   // the compiler tracks only these loads
    const uint32_t* szp = a.sz + (size_t(br) * a.nbc + col0) * 64;
    const _Float16* xp = a.x + size_t(col0) * 64;
    const uint8_t* cp = a.codes + size_t(uniform(o0)) * kHS;
    int jn = 0, used = 0, issued = 0;
    uint32_t sbn = 0;
    auto fill = [&]() {
      while (jn < S) {
        const int bn = uniform(__builtin_amdgcn_readlane(bvec, jn));
        const int ns = 1 + nx + bn;
        if (used + ns > R) break;
        dma4_once(szp, 4 * lane, ring_lds, sbn);
        szp += 64;
        for (int xi = 0; xi < nx; ++xi)
          if (lane < 32) dma16(xp, xoff[xi], ring_lds, wrap<R, kHS>(sbn + kHS * (1 + xi)));
        xp += 64;
        uint32_t sc = sbn + kHS * (1 + nx);
        for (int q = 0; q < bn; ++q) {
          if (lane < 32) dma16_once(cp, 16 * lane, ring_lds, wrap<R, kHS>(sc));
          cp += kHS;
          sc += kHS;
        }
        sbn = wrap<R, kHS>(sc);
        used += ns;
        issued += ns;
        ++jn;
      }
    };
    fill();
    uint32_t sb = 0;
    int done = 0;
    for (int j = 0; j < S; ++j) {
      const int bj = uniform(__builtin_amdgcn_readlane(bvec, j));
      done += 1 + nx + bj;
      wait_vmcnt_at_most(issued - done);
      auto refill = [&]() {
        used -= 1 + nx + bj;
        fill();
      };
      const uint32_t xb = sb + kHS, cb = sb + kHS * (1 + nx);
      half8 xa[2][MT];
      read_x64<MT, R>(ring, xb, M, xa);
      switch (bj) {
        case 1: block_core64<1, 0, MT, R>(ring, sb, cb, xa, acc, refill); break;
        case 2: block_core64<2, 0, MT, R>(ring, sb, cb, xa, acc, refill); break;
        case 3: block_core64<2, 1, MT, R>(ring, sb, cb, xa, acc, refill); break;
        case 4: block_core64<4, 0, MT, R>(ring, sb, cb, xa, acc, refill); break;
        case 6: block_core64<4, 2, MT, R>(ring, sb, cb, xa, acc, refill); break;
        default: block_core64<4, 4, MT, R>(ring, sb, cb, xa, acc, refill); break;
      }
      sb = wrap<R, kHS>(sb + kHS * (1 + nx + bj));
    }
  }
  __syncthreads();

  // waves meet in LDS; wave w < 4 adds row tile w over the waves in order
  static_assert(NW * 4 * MT * 1024 <= NW * R * kHS, "reduction fits in the rings");
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

// Single token: per wave a 16-half-slot code ring (8 KiB) and a 4-entry ring
// of 512-byte records (scale/zero 256 B, then the block's 64 activations);
// 10 KiB per wave, four 4-wave workgroups per CU.
constexpr int kCodeSlots64 = 16;
constexpr uint32_t kCodeMask64 = kCodeSlots64 * kHS - 1;
constexpr int kMetaSlots64 = 4;
constexpr uint32_t kMetaMask64 = kMetaSlots64 * 512 - 1;
constexpr int kWaveLds64 = kCodeSlots64 * kHS + kMetaSlots64 * 512;

template <int W0, int W1, class Refill>
__device__ __forceinline__ void block1_64(const u32x4* code, const u32x4* meta, uint32_t cj, uint32_t mj,
                                          float (&acc)[4], Refill&& refill) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const uint2* code2 = reinterpret_cast<const uint2*>(code);
  const u32x4 sz = meta[(mj >> 4) + r16];
  half8 xa[2][1];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) xa[kt][0] = __builtin_bit_cast(half8, meta[(mj >> 4) + 16 + 4 * kt + g]);
  uint2 w0[W0], w1[W1 ? W1 : 1];
#pragma unroll
  for (int q = 0; q < W0; ++q) w0[q] = code2[(((cj + kHS * q) & kCodeMask64) >> 3) + lane];
#pragma unroll
  for (int q = 0; q < W1; ++q) w1[q] = code2[(((cj + kHS * (W0 + q)) & kCodeMask64) >> 3) + lane];
  wait_lds();
  refill();

  const half8 ones = as_half8(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);
  f32x4 xsum = f32x4{0, 0, 0, 0}, c0[4][1], c1[4][1];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) c0[rt][0] = c1[rt][0] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) xsum = mfma16(xa[kt][0], ones, xsum);
  plane_mma64<W0, 1>(w0, xa, c0);
  if constexpr (W1 != 0) plane_mma64<W1, 1>(w1, xa, c1);
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
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void decode1_64_kernel(DecodeArgs a) {
  const int wg = int(blockIdx.x);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int br = int(unsigned(wg) / unsigned(a.nseg)), seg = wg - br * a.nseg;
  const int wg_begin = seg * a.seg_cols;
  const int wg_cols = min(a.nbc, wg_begin + a.seg_cols) - wg_begin;
  const int w_begin = wg_begin + (wg_cols * wave) / NW;
  const int w_end = wg_begin + (wg_cols * (wave + 1)) / NW;

  __shared__ u32x4 lds[NW * kWaveLds64 / 16];   // per-wave rings; reused for the reduction
  const u32x4* code = lds + wave * (kWaveLds64 / 16);
  const u32x4* meta = code + kCodeSlots64 * kHS / 16;
  const uint32_t code_lds = lds_addr(code), meta_lds = lds_addr(meta);

  float acc[4] = {0, 0, 0, 0};
  for (int col0 = w_begin; col0 < w_end; col0 += 64) {
    const int S = min(64, w_end - col0);
    const bool in = lane < S;
    const size_t blk0 = size_t(br) * a.nbc + col0;
    const int bvec = in ? int(a.bits[blk0 + lane]) : 0;
    const int o0 = int(a.offs[blk0]);
    wait_vmcnt<0>();   // the compiler tracks only these loads
    const uint32_t* szp = a.sz + blk0 * 64;
    const _Float16* xp = a.x + size_t(col0) * 64;
    const uint8_t* cp = a.codes + size_t(uniform(o0)) * kHS;
    int jn = 0, cfree = kCodeSlots64, mfree = kMetaSlots64, issued = 0;
    uint32_t cn = 0, mn = 0;
    auto fill = [&]() {
      while (jn < S) {
        const int bn = uniform(__builtin_amdgcn_readlane(bvec, jn));
        if (bn > cfree || mfree == 0) break;
        dma4_once(szp, 4 * lane, meta_lds, mn);
        if (lane < 32) dma4(xp, 4 * lane, meta_lds, mn + 256);
        for (int q = 0; q < bn; ++q)
          if (lane < 32) dma16_once(cp + kHS * q, 16 * lane, code_lds, (cn + kHS * q) & kCodeMask64);
        szp += 64;
        xp += 64;
        cp += kHS * bn;
        cn = (cn + kHS * bn) & kCodeMask64;
        mn = (mn + 512) & kMetaMask64;
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
        case 1: block1_64<1, 0>(code, meta, cj, mj, acc, refill); break;
        case 2: block1_64<2, 0>(code, meta, cj, mj, acc, refill); break;
        case 3: block1_64<2, 1>(code, meta, cj, mj, acc, refill); break;
        case 4: block1_64<4, 0>(code, meta, cj, mj, acc, refill); break;
        case 6: block1_64<4, 2>(code, meta, cj, mj, acc, refill); break;
        default: block1_64<4, 4>(code, meta, cj, mj, acc, refill); break;
      }
      cj = (cj + kHS * bj) & kCodeMask64;
      mj = (mj + 512) & kMetaMask64;
    }
  }
  __syncthreads();

  // waves meet in LDS; lane l of wave 0 adds row 16 (l / 16) + l % 16 of the
  // block row over the waves in order
  static_assert(NW * 4 * 64 * 4 <= NW * kWaveLds64, "reduction fits in the rings");
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

}  // namespace

// The 64x128 plan computed for the same shape, with one block row per
// workgroup at every M and the K segments counted in 64-column blocks: a
// wave streams the same bytes as on the 64x128 image.
DecodePlan decode_plan64(int N, int K, int M) {
  // The 64x128 plan over K rounded up to whole 128-column groups (a single
  // 64-column block column would otherwise count as none), then re-cut in
  // 64-column units.
  DecodePlan p = decode_plan(N, (K + 127) / 128 * 128, M);
  const int nbr = N / 64, nbc64 = K / 64;
  if (p.rows == 2) {   // one row per workgroup: one 128 KiB workgroup per CU at M > 16
    p.rows = 1;
    int nseg = 1;
    if (nbr < 256) {
      nseg = 256 / nbr;
      nseg = min(nseg, max(1, (K / 128) / (2 * p.nw)));
      nseg = min(nseg, max(1, K / (32 * M)));
    }
    p.nseg = min(nseg, kMaxSegments);
  }
  p.seg_cols = (nbc64 + p.nseg - 1) / p.nseg;
  p.nseg = (nbc64 + p.seg_cols - 1) / p.seg_cols;
  p.ws_bytes = p.nseg > 1 ? size_t(M) * size_t(N) * 12 : 0;
  return p;
}

int launch_decode64(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* workspace,
                    const DecodePlan& plan, void* stream) {
  DecodeArgs a;
  a.bits = im.bits;
  a.offs = im.offs;
  a.sz = im.sz;
  a.codes = im.codes;
  a.x = reinterpret_cast<const _Float16*>(x);
  a.y = reinterpret_cast<_Float16*>(y);
  a.acc = plan.nseg > 1 ? static_cast<uint64_t*>(workspace) : nullptr;
  a.facc = plan.nseg > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + size_t(M) * im.N * 8) : nullptr;
  a.part = nullptr;
  a.N = im.N;
  a.K = im.K;
  a.M = M;
  a.nbr = im.nbr;
  a.nbc = im.nbc;
  a.seg_cols = plan.seg_cols;
  a.nseg = plan.nseg;
  const dim3 grid{static_cast<unsigned>(im.nbr * plan.nseg), 1u, 1u};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 1)
    hipLaunchKernelGGL((decode1_64_kernel<4>), grid, dim3(256), 0, s, a);
  else if (M <= 8)
    hipLaunchKernelGGL((decode64_kernel<4, 1, kRing64_8>), grid, dim3(256), 0, s, a);
  else if (M <= 16)
    hipLaunchKernelGGL((decode64_kernel<4, 1, kRing64_16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode64_kernel<4, 2, kRing64_32>), grid, dim3(256), 0, s, a);
  return int(hipGetLastError());
}

}  // namespace gbb
