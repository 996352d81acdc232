// Offline quantizer and packer for both weight images (host only).
//
// Quantization follows the affine map of the MixLLM page, section 2.1:
// q = clamp(rint(w / s) + z, range), w' = (q - z) * s, with min/max ranges per
// (row, 128-column group).  Every decision is taken in binary64 and rounds
// half to even; scales are stored as binary16.  Build without -ffast-math and
// with -ffp-contract=off so the arithmetic is plain IEEE.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"
#include "layout.h"

namespace gbb {

// ---------------------------------------------------------------------------
// error text
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

gbb_status fail(gbb_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gbb_status ok() { return GBB_OK; }

// ---------------------------------------------------------------------------
// binary16 conversions
// ---------------------------------------------------------------------------
double half_to_double(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = std::ldexp(double(m), -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = std::ldexp(double(m | 1024), e - 25);
  return sign ? -v : v;
}

uint16_t double_to_half(double d) {
  uint64_t u;
  std::memcpy(&u, &d, 8);
  const uint16_t sign = uint16_t((u >> 48) & 0x8000u);
  const uint64_t a = u & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull) return sign | (a > 0x7ff0000000000000ull ? 0x7e00 : 0x7c00);
  const int ebits = int(a >> 52);
  if (ebits == 0) return sign;                       // binary64 subnormal: far below 2^-25
  const int e = ebits - 1023;                        // value = 1.f * 2^e
  if (e < -25) return sign;                          // below half the smallest subnormal
  if (e > 15) return sign | 0x7c00;
  const uint64_t m = (a & ((1ull << 52) - 1)) | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);  // bits dropped from the 53-bit significand
  uint64_t keep = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (keep & 1))) ++keep;
  if (e >= -14) return uint16_t(sign | ((uint32_t(e + 15) << 10) + uint32_t(keep - 1024)));  // carry may reach inf
  return uint16_t(sign | uint32_t(keep));            // subnormal (keep == 1024 is the smallest normal)
}

// Runs f(i) for i in [0, n) on up to hardware_concurrency threads; each i
// writes a disjoint part of the output, so the result does not depend on the
// thread count.
template <class F>
static void parallel_for(long n, F&& f) {
  unsigned nt = std::max(1u, std::thread::hardware_concurrency());
  nt = unsigned(std::min<long>(nt, std::max<long>(1, n)));
  if (nt <= 1) {
    for (long i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(nt);
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (long i = t; i < n; i += nt) f(i);
    });
  for (auto& x : th) x.join();
}

// ---------------------------------------------------------------------------
// group quantizers (binary64 decisions)
// ---------------------------------------------------------------------------
namespace {

struct GroupQ {
  uint16_t s16, z16;
  double s, z;
};

// min/max asymmetric scale and zero over n values at `levels` = 2^b - 1.
GroupQ asym_scale_zero(const double* v, int n, double levels) {
  double lo = v[0], hi = v[0];
  for (int i = 1; i < n; ++i) {
    lo = std::min(lo, v[i]);
    hi = std::max(hi, v[i]);
  }
  GroupQ g;
  if (hi > lo) {
    g.s16 = double_to_half((hi - lo) / levels);
    if ((g.s16 & 0x7fff) == 0) g.s16 = 0x0001;  // 2^-24
  } else {
    g.s16 = lo != 0 ? double_to_half(std::fabs(lo)) : uint16_t(0x3c00);
  }
  g.s = half_to_double(g.s16);
  g.z = std::min(std::max(std::nearbyint(-lo / g.s), 0.0), levels) + 0.0;  // +0 for -0
  g.z16 = double_to_half(g.z);
  return g;
}

inline uint8_t asym_code(double v, const GroupQ& g, double levels) {
  const double q = std::nearbyint(v / g.s) + g.z;
  return uint8_t(std::min(std::max(q, 0.0), levels));
}

// 8-bit symmetric: s = fp16(max|v| / 127), q = clamp(rint(v / s), -127, 127).
uint16_t sym8_scale(const double* v, int n) {
  double a = 0;
  for (int i = 0; i < n; ++i) a = std::max(a, std::fabs(v[i]));
  if (a == 0) return 0x3c00;
  uint16_t s = double_to_half(a / 127.0);
  if ((s & 0x7fff) == 0) s = 0x0001;
  return s;
}

inline int8_t sym8_code(double v, double s) {
  const double q = std::nearbyint(v / s);
  return int8_t(std::min(std::max(q, -127.0), 127.0));
}

bool all_finite(const uint16_t* W, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if ((W[i] & 0x7c00) == 0x7c00) return false;
  return true;
}

}  // namespace

// ---------------------------------------------------------------------------
// block image
// ---------------------------------------------------------------------------
// bc: block columns (and group size), 128 or 64.
static gbb_status check_bits(const uint8_t* bits, int N, int K, int bc = kGroup) {
  if (!bits) return fail(GBB_E_ARG, "bits is NULL");
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  if (N % kBlockRows || K % bc)
    return fail(GBB_E_SHAPE, "N must be a multiple of 64 and K of %d (N=%d K=%d)", bc, N, K);
  const size_t nblk = size_t(N / kBlockRows) * size_t(K / bc);
  for (size_t i = 0; i < nblk; ++i)
    if (!valid_bits(bits[i]))
      return fail(GBB_E_BITS, "block %zu has bitwidth %d, not in {1,2,3,4,6,8}", i, int(bits[i]));
  return GBB_OK;
}

static size_t packed_bytes_unchecked(const uint8_t* bits, int N, int K, int bc = kGroup) {
  const BlockLayout l = block_layout(N, K, bc);
  size_t units = 0;
  for (size_t i = 0; i < l.nblk; ++i) units += bits[i];
  return l.codes_off + size_t(8 * bc) * units;
}

// Write one plane of a block: codes q[64][128] (row, column within the block),
// plane width w, bit shift sh, into dst (w KiB).
static void write_plane(const uint8_t (*q)[128], int w, int sh, uint8_t* dst) {
  const int npair = 16 / w;
  const uint32_t mask = (1u << w) - 1u;
  for (int j = 0; j < w; ++j)
    for (int lane = 0; lane < 64; ++lane)
      for (int c = 0; c < 4; ++c) {
        uint32_t word = 0;
        for (int i = 0; i < npair; ++i) {
          const int u = j * npair + i, kt = u >> 2, rt = u & 3;
          const int row = 16 * rt + (lane & 15);
          const int col = 32 * kt + 8 * (lane >> 4) + 2 * c;
          word |= ((uint32_t(q[row][col]) >> sh) & mask) << (w * i);
          word |= ((uint32_t(q[row][col + 1]) >> sh) & mask) << (16 + w * i);
        }
        std::memcpy(dst + 1024 * j + 16 * lane + 4 * c, &word, 4);
      }
}

// The same for a 64x64 block (codes q[64][64]) into w half-slots of 512 B.
static void write_plane64(const uint8_t (*q)[64], int w, int sh, uint8_t* dst) {
  const int per = 8 / w;
  const uint32_t mask = (1u << w) - 1u;
  for (int j = 0; j < w; ++j)
    for (int lane = 0; lane < 64; ++lane)
      for (int d = 0; d < 2; ++d) {
        uint32_t word = 0;
        for (int f = 0; f < 16 / w; ++f) {
          const int c = 2 * d + f / per, u = j * per + f % per, kt = u >> 2, rt = u & 3;
          const int row = 16 * rt + (lane & 15);
          const int col = 32 * kt + 8 * (lane >> 4) + 2 * c;
          word |= ((uint32_t(q[row][col]) >> sh) & mask) << (w * f);
          word |= ((uint32_t(q[row][col + 1]) >> sh) & mask) << (16 + w * f);
        }
        std::memcpy(dst + 512 * j + 8 * lane + 4 * d, &word, 4);
      }
}

// Quantize and pack with blocks of 64 rows x bc columns (bc = 128 or 64;
// groups of bc columns).
static gbb_status pack_blocks(const uint16_t* W, int N, int K, const uint8_t* bits, uint16_t* scale, uint16_t* zero,
                              unsigned flags, void* image, size_t image_cap, int bc) {
  gbb_status st = check_bits(bits, N, K, bc);
  if (st != GBB_OK) return st;
  if (!W || !image) return fail(GBB_E_ARG, "W and image must not be NULL");
  if (flags & ~GBB_PACK_GIVEN_SZ) return fail(GBB_E_ARG, "unknown flag bits 0x%x", flags);
  const bool given = flags & GBB_PACK_GIVEN_SZ;
  if (given && (!scale || !zero)) return fail(GBB_E_ARG, "GBB_PACK_GIVEN_SZ needs scale and zero");
  const size_t need = packed_bytes_unchecked(bits, N, K, bc);
  if (image_cap < need) return fail(GBB_E_SPACE, "image needs %zu bytes, capacity %zu", need, image_cap);
  if (!all_finite(W, size_t(N) * size_t(K))) return fail(GBB_E_ARG, "W holds inf or NaN");

  const int nbr = N / kBlockRows, nbc = K / bc, G = nbc;
  if (given) {
    for (size_t r = 0; r < size_t(N); ++r)
      for (int g = 0; g < G; ++g) {
        const int b = bits[(r / kBlockRows) * nbc + g];
        const double s = half_to_double(scale[r * G + g]), z = half_to_double(zero[r * G + g]);
        if (!(s > 0) || !std::isfinite(s))
          return fail(GBB_E_ARG, "given scale of row %zu group %d is not finite and > 0", r, g);
        if (!(z >= 0 && z <= double((1 << b) - 1) && z == std::floor(z)))
          return fail(GBB_E_BITS, "given zero of row %zu group %d is not an integer in [0, 2^b-1]", r, g);
      }
  }

  const BlockLayout l = block_layout(N, K, bc);
  const size_t unit = size_t(8 * bc);   // code bytes per bit of width per block
  uint8_t* img = static_cast<uint8_t*>(image);
  std::memset(img, 0, l.codes_off);
  std::vector<size_t> units(l.nblk + 1, 0);
  for (size_t i = 0; i < l.nblk; ++i) units[i + 1] = units[i] + bits[i];

  BlockHeader h{};
  h.magic = kMagicBlocks;
  h.version = bc == kGroup ? kVersion : kVersion64;
  h.N = uint32_t(N);
  h.K = uint32_t(K);
  h.nbr = uint32_t(nbr);
  h.nbc = uint32_t(nbc);
  h.bits_off = l.bits_off;
  h.offs_off = l.offs_off;
  h.sz_off = l.sz_off;
  h.codes_off = l.codes_off;
  h.codes_bytes = unit * units[l.nblk];
  std::memcpy(img, &h, sizeof h);
  std::memcpy(img + l.bits_off, bits, l.nblk);
  for (size_t i = 0; i <= l.nblk; ++i) {
    const uint32_t o = uint32_t(units[i]);
    std::memcpy(img + l.offs_off + 4 * i, &o, 4);
  }

  parallel_for(long(l.nblk), [&](long blk) {
    const int br = int(blk / nbc), bcol = int(blk % nbc);
    const int b = bits[blk];
    const double levels = double((1 << b) - 1);
    uint8_t q[64][128];
    uint8_t q64[64][64];
    double v[128];
    for (int r = 0; r < 64; ++r) {
      const size_t row = size_t(br) * 64 + r;
      const uint16_t* src = W + row * size_t(K) + size_t(bcol) * bc;
      for (int k = 0; k < bc; ++k) v[k] = half_to_double(src[k]);
      GroupQ gq;
      if (given) {
        gq.s16 = scale[row * G + bcol];
        gq.z16 = zero[row * G + bcol];
        gq.s = half_to_double(gq.s16);
        gq.z = half_to_double(gq.z16);
      } else {
        gq = asym_scale_zero(v, bc, levels);
        if (scale) scale[row * G + bcol] = gq.s16;
        if (zero) zero[row * G + bcol] = gq.z16;
      }
      for (int k = 0; k < bc; ++k) {
        const uint8_t c = asym_code(v[k], gq, levels);
        if (bc == kGroup)
          q[r][k] = c;
        else
          q64[r][k] = c;
      }
      const uint32_t e = uint32_t(gq.s16) | (uint32_t(gq.z16) << 16);
      std::memcpy(img + l.sz_off + 256 * size_t(blk) + 4 * (4 * (r % 16) + r / 16), &e, 4);
    }
    uint8_t* dst = img + l.codes_off + unit * units[blk];
    const int w0 = plane0_width(b), w1 = plane1_width(b);
    if (bc == kGroup) {
      write_plane(q, w0, 0, dst);
      if (w1) write_plane(q, w1, w0, dst + unit * w0);
    } else {
      write_plane64(q64, w0, 0, dst);
      if (w1) write_plane64(q64, w1, w0, dst + unit * w0);
    }
  });
  return GBB_OK;
}

}  // namespace gbb

using namespace gbb;

extern "C" const char* gbb_last_error(void) { return g_last_error.c_str(); }

extern "C" size_t gbb_packed_bytes(const uint8_t* bits, int N, int K) {
  if (check_bits(bits, N, K) != GBB_OK) return 0;
  return packed_bytes_unchecked(bits, N, K);
}

extern "C" gbb_status gbb_pack_blocks(const uint16_t* W, int N, int K, const uint8_t* bits,
                                      uint16_t* scale, uint16_t* zero, unsigned flags, void* image,
                                      size_t image_cap) {
  return pack_blocks(W, N, K, bits, scale, zero, flags, image, image_cap, kGroup);
}

extern "C" size_t gbb_packed_bytes_64x64(const uint8_t* bits, int N, int K) {
  if (check_bits(bits, N, K, 64) != GBB_OK) return 0;
  return packed_bytes_unchecked(bits, N, K, 64);
}

extern "C" gbb_status gbb_pack_blocks_64x64(const uint16_t* W, int N, int K, const uint8_t* bits,
                                            uint16_t* scale, uint16_t* zero, unsigned flags, void* image,
                                            size_t image_cap) {
  return pack_blocks(W, N, K, bits, scale, zero, flags, image, image_cap, 64);
}

extern "C" gbb_status gbb_check_image(const void* image, size_t image_bytes, int N, int K) {
  if (!image) return fail(GBB_E_ARG, "image is NULL");
  if (image_bytes < 64) return fail(GBB_E_FORMAT, "image shorter than its header");
  BlockHeader h;
  std::memcpy(&h, image, sizeof h);
  if (h.magic != kMagicBlocks || (h.version != kVersion && h.version != kVersion64))
    return fail(GBB_E_FORMAT, "not a block image (version 1 or 2)");
  if (int(h.N) != N || int(h.K) != K) return fail(GBB_E_FORMAT, "image is %ux%u, call says %dx%d", h.N, h.K, N, K);
  const BlockLayout l = block_layout(N, K, h.version == kVersion ? kGroup : 64);
  if (h.bits_off != l.bits_off || h.offs_off != l.offs_off || h.sz_off != l.sz_off || h.codes_off != l.codes_off)
    return fail(GBB_E_FORMAT, "section offsets do not match the layout for %dx%d", N, K);
  if (image_bytes < h.codes_off + h.codes_bytes) return fail(GBB_E_FORMAT, "image truncated");
  return GBB_OK;
}

// ---------------------------------------------------------------------------
// W4/W8 image
// ---------------------------------------------------------------------------
static gbb_status check_w48(int N, int K, const int32_t* rows8, int n8) {
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  if (K % kGroup) return fail(GBB_E_SHAPE, "K must be a multiple of 128 (K=%d)", K);
  if (n8 < 0 || n8 > N) return fail(GBB_E_SHAPE, "n8=%d outside [0, N=%d]", n8, N);
  if (n8 > 0 && !rows8) return fail(GBB_E_ARG, "rows8 is NULL");
  for (int i = 0; i < n8; ++i) {
    if (rows8[i] < 0 || rows8[i] >= N) return fail(GBB_E_SHAPE, "rows8[%d]=%d outside [0, N)", i, rows8[i]);
    if (i && rows8[i] <= rows8[i - 1]) return fail(GBB_E_SHAPE, "rows8 must be strictly ascending");
  }
  return GBB_OK;
}

extern "C" size_t gbb_w48_packed_bytes(int N, int K, int n8) {
  if (N <= 0 || K <= 0 || K % kGroup || n8 < 0 || n8 > N) {
    fail(GBB_E_ARG, "bad shape N=%d K=%d n8=%d", N, K, n8);
    return 0;
  }
  return w48_layout(N, K, n8).total;
}

extern "C" gbb_status gbb_pack_w48(const uint16_t* W, int N, int K, const int32_t* rows8, int n8,
                                   uint16_t* scale, uint8_t* zero, void* image, size_t image_cap) {
  gbb_status st = check_w48(N, K, rows8, n8);
  if (st != GBB_OK) return st;
  if (!W || !image) return fail(GBB_E_ARG, "W and image must not be NULL");
  const W48Layout l = w48_layout(N, K, n8);
  if (image_cap < l.total) return fail(GBB_E_SPACE, "image needs %zu bytes, capacity %zu", l.total, image_cap);
  if (!all_finite(W, size_t(N) * size_t(K))) return fail(GBB_E_ARG, "W holds inf or NaN");

  const int n4 = N - n8, G = K / kGroup, KT = K / 64;
  std::vector<int32_t> packed_rows(size_t(16) * (l.T8 + l.T4), -1);
  {
    std::vector<char> is8(size_t(N), 0);
    for (int i = 0; i < n8; ++i) is8[size_t(rows8[i])] = 1;
    int j8 = 0, j4 = 0;
    for (int r = 0; r < N; ++r) {
      if (is8[size_t(r)])
        packed_rows[size_t(j8++)] = r;
      else
        packed_rows[size_t(16) * l.T8 + size_t(j4++)] = r;
    }
  }
  uint8_t* img = static_cast<uint8_t*>(image);
  std::memset(img, 0, l.total);
  W48Header h{};
  h.magic = kMagicW48;
  h.version = kVersion;
  h.N = uint32_t(N);
  h.K = uint32_t(K);
  h.n8 = uint32_t(n8);
  h.n4 = uint32_t(n4);
  h.T8 = uint32_t(l.T8);
  h.T4 = uint32_t(l.T4);
  h.rows_off = l.rows_off;
  h.s_off = l.s_off;
  h.z_off = l.z_off;
  h.c8_off = l.c8_off;
  h.c4_off = l.c4_off;
  std::memcpy(img, &h, 72);
  std::memcpy(img + l.rows_off, packed_rows.data(), 4 * packed_rows.size());

  uint16_t* s_sec = reinterpret_cast<uint16_t*>(img + l.s_off);
  uint8_t* z_sec = img + l.z_off;
  int8_t* c8 = reinterpret_cast<int8_t*>(img + l.c8_off);
  uint8_t* c4 = img + l.c4_off;

  // one packed tile of 16 rows per task
  parallel_for(long(l.T8 + l.T4), [&](long t) {
    const bool eight = t < l.T8;
    std::vector<int8_t> q8(eight ? 16 * size_t(K) : 0, 0);
    std::vector<uint8_t> q4(eight ? 0 : 16 * size_t(K), 0);
    double v[kGroup];
    for (int r = 0; r < 16; ++r) {
      const int row = packed_rows[size_t(16) * t + r];
      if (row < 0) continue;  // padding: codes 0, scale 0
      const uint16_t* src = W + size_t(row) * size_t(K);
      for (int g = 0; g < G; ++g) {
        for (int k = 0; k < kGroup; ++k) v[k] = half_to_double(src[g * kGroup + k]);
        uint16_t s16;
        uint8_t zz = 0;
        if (eight) {
          s16 = sym8_scale(v, kGroup);
          const double s = half_to_double(s16);
          for (int k = 0; k < kGroup; ++k) q8[size_t(r) * K + g * kGroup + k] = sym8_code(v[k], s);
        } else {
          const GroupQ gq = asym_scale_zero(v, kGroup, 15.0);
          s16 = gq.s16;
          zz = uint8_t(gq.z);
          for (int k = 0; k < kGroup; ++k) q4[size_t(r) * K + g * kGroup + k] = asym_code(v[k], gq, 15.0);
          z_sec[(size_t(t - l.T8) * G + g) * 16 + r] = zz;
        }
        s_sec[(size_t(t) * G + g) * 16 + r] = s16;
        if (scale) scale[size_t(row) * G + g] = s16;
        if (zero) zero[size_t(row) * G + g] = zz;
      }
    }
    for (int kt = 0; kt < KT; ++kt) {
      for (int lane = 0; lane < 64; ++lane) {
        const int r = lane & 15, c0 = 64 * kt + 16 * (lane >> 4);
        if (eight) {
          int8_t* dst = c8 + (size_t(t) * KT + kt) * 1024 + 16 * lane;
          for (int e = 0; e < 16; ++e) dst[e] = q8[size_t(r) * K + c0 + e];
        } else {
          uint8_t* dst = c4 + (size_t(t - l.T8) * KT + kt) * 512 + 8 * lane;
          for (int j = 0; j < 2; ++j)
            for (int i = 0; i < 4; ++i) {
              const int e = 8 * j + i;
              dst[4 * j + i] = uint8_t(q4[size_t(r) * K + c0 + e] | (q4[size_t(r) * K + c0 + e + 4] << 4));
            }
        }
      }
    }
  });
  return GBB_OK;
}

// ---------------------------------------------------------------------------
// Offline bitwidth allocation and channel reordering (ScaleBITS explainer,
// sections 1.2.1, 2.2 and 4.2), with a weight-magnitude proxy in place of the
// gradient sensitivity, which needs a model and calibration data.
//
// Objective of block i at bitwidth b: S_i * e_i(b), with S_i = sum |w| over
// the block (exact in binary64: fp16 values are multiples of 2^-24 and a
// block sums to less than 2^29) and e_i(b) = sum (w - w'_b)^2 under this
// file's group quantizer, summed in binary64 in row-major order.  Every
// block starts at 3 bits and moves one step of {1,2,3,4,6,8} at a time.
// A round: over the budget, lower the k = max(1, floor(gamma nblk + 1/2))
// blocks of least per-bit cost; within it, raise the blocks of largest
// per-bit gain whose step still fits (at most k); when none fits, trade the
// max(1, k / 2) best raises for as many cheapest lowerings if that lowers the
// objective and keeps the budget, else stop; at most 64 + floor(4 / gamma)
// rounds.  Ties go to the lower block index.
// ---------------------------------------------------------------------------
namespace {

constexpr int kAllowed[6] = {1, 2, 3, 4, 6, 8};
int bit_index(int b) { return b <= 4 ? b - 1 : (b == 6 ? 4 : 5); }
int step_up(int b) { return b == 4 ? 6 : (b == 6 ? 8 : b + 1); }
int step_down(int b) { return b == 6 ? 4 : (b == 8 ? 6 : b - 1); }

struct Ranked {
  double key;
  int idx;
};

}  // namespace

extern "C" gbb_status gbb_allocate_bits(const uint16_t* W, int N, int K, double target_bits, double gamma,
                                        uint8_t* bits) {
  if (!W || !bits) return fail(GBB_E_ARG, "W and bits must not be NULL");
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive");
  if (N % kBlockRows || K % kGroup) return fail(GBB_E_SHAPE, "N must be a multiple of 64 and K of 128");
  if (!(target_bits >= 1.0 && target_bits <= 8.0)) return fail(GBB_E_ARG, "target_bits must lie in [1, 8]");
  if (!(gamma > 0.0 && gamma <= 1.0)) return fail(GBB_E_ARG, "gamma must lie in (0, 1]");
  if (!all_finite(W, size_t(N) * size_t(K))) return fail(GBB_E_ARG, "W holds inf or NaN");
  const int nbr = N / kBlockRows, nbc = K / kGroup, n = nbr * nbc;

  // block statistics: S[i] and E[i][bit_index(b)]
  std::vector<double> S(n), E(size_t(n) * 6);
  parallel_for(n, [&](long i) {
    const int br = int(i / nbc), bc = int(i % nbc);
    double v[kGroup], s = 0;
    for (int r = 0; r < kBlockRows; ++r)
      for (int c = 0; c < kGroup; ++c)
        s += std::fabs(half_to_double(W[size_t(br * kBlockRows + r) * K + size_t(bc) * kGroup + c]));
    S[i] = s;
    for (int t = 0; t < 6; ++t) {
      const double levels = double((1 << kAllowed[t]) - 1);
      double e = 0;
      for (int r = 0; r < kBlockRows; ++r) {
        const uint16_t* src = W + size_t(br * kBlockRows + r) * K + size_t(bc) * kGroup;
        for (int c = 0; c < kGroup; ++c) v[c] = half_to_double(src[c]);
        const GroupQ gq = asym_scale_zero(v, kGroup, levels);
        for (int c = 0; c < kGroup; ++c) {
          const float qz = float(asym_code(v[c], gq, levels)) - float(gq.z);
          const double d = v[c] - double(qz * float(gq.s));
          e += d * d;
        }
      }
      E[size_t(i) * 6 + t] = e;
    }
  });

  std::vector<int> b(n, 3);
  const int k = std::max(1, int(std::floor(gamma * n + 0.5)));
  const double budget = target_bits * n;
  auto err = [&](int i, int bw) { return E[size_t(i) * 6 + bit_index(bw)]; };
  auto up = [&](int i) {
    const int b2 = step_up(b[i]);
    return S[i] * (err(i, b[i]) - err(i, b2)) / double(b2 - b[i]);
  };
  auto down = [&](int i) {
    const int b2 = step_down(b[i]);
    return S[i] * (err(i, b2) - err(i, b[i])) / double(b[i] - b2);
  };
  // ascending key, ties to the lower index
  auto by_key = [](const Ranked& x, const Ranked& y) { return x.key < y.key || (x.key == y.key && x.idx < y.idx); };
  std::vector<Ranked> rk;
  rk.reserve(n);
  const int rounds = 64 + int(std::floor(4.0 / gamma));
  for (int round = 0; round < rounds; ++round) {
    long total = 0;
    for (int i = 0; i < n; ++i) total += b[i];
    if (double(total) > budget) {
      rk.clear();
      for (int i = 0; i < n; ++i)
        if (b[i] > 1) rk.push_back({down(i), i});
      std::sort(rk.begin(), rk.end(), by_key);
      for (int j = 0; j < k && j < int(rk.size()); ++j) b[rk[j].idx] = step_down(b[rk[j].idx]);
      continue;
    }
    double slack = budget - double(total);
    rk.clear();
    for (int i = 0; i < n; ++i)
      if (b[i] < 8) rk.push_back({-up(i), i});
    std::sort(rk.begin(), rk.end(), by_key);
    const std::vector<Ranked> ups = rk;
    int raised = 0;
    for (const Ranked& u : ups) {
      if (raised == k) break;
      const int step = step_up(b[u.idx]) - b[u.idx];
      if (double(step) <= slack) {
        b[u.idx] = step_up(b[u.idx]);
        slack -= double(step);
        ++raised;
      }
    }
    if (raised) continue;
    const int h = std::max(1, k / 2);
    std::vector<int> chosen;
    for (int j = 0; j < h && j < int(ups.size()); ++j) chosen.push_back(ups[j].idx);
    // pay for the raises with the cheapest lowerings of other blocks until
    // the bits freed cover the overshoot of the budget
    long need_bits = total;
    for (int i : chosen) need_bits += step_up(b[i]) - b[i];
    const double need = double(need_bits) - budget;
    rk.clear();
    for (int i = 0; i < n; ++i)
      if (b[i] > 1) rk.push_back({down(i), i});
    std::sort(rk.begin(), rk.end(), by_key);
    std::vector<int> downs;
    long freed = 0;
    for (const Ranked& d : rk) {
      if (double(freed) >= need) break;
      if (std::find(chosen.begin(), chosen.end(), d.idx) != chosen.end()) continue;
      downs.push_back(d.idx);
      freed += b[d.idx] - step_down(b[d.idx]);
    }
    double gain = 0, cost = 0;
    for (int i : chosen) gain += S[i] * (err(i, b[i]) - err(i, step_up(b[i])));
    for (int i : downs) cost += S[i] * (err(i, step_down(b[i])) - err(i, b[i]));
    if (chosen.empty() || double(freed) < need || !(gain > cost)) break;
    for (int i : chosen) b[i] = step_up(b[i]);
    for (int i : downs) b[i] = step_down(b[i]);
  }
  for (int i = 0; i < n; ++i) bits[i] = uint8_t(b[i]);
  return GBB_OK;
}

extern "C" gbb_status gbb_channel_order(const uint16_t* W, int N, int K, int32_t* row_order, int32_t* col_order) {
  if (!W || !row_order || !col_order) return fail(GBB_E_ARG, "W, row_order and col_order must not be NULL");
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive");
  if (!all_finite(W, size_t(N) * size_t(K))) return fail(GBB_E_ARG, "W holds inf or NaN");
  // exact L1 norms in units of 2^-24 (the fp16 quantum)
  std::vector<int64_t> rl(N, 0), cl(K, 0);
  for (int r = 0; r < N; ++r)
    for (int c = 0; c < K; ++c) {
      const int64_t a = int64_t(std::ldexp(std::fabs(half_to_double(W[size_t(r) * K + c])), 24));
      rl[r] += a;
      cl[c] += a;
    }
  auto order = [](const std::vector<int64_t>& l1, int32_t* out) {
    std::vector<int32_t> idx(l1.size());
    for (size_t i = 0; i < idx.size(); ++i) idx[i] = int32_t(i);
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return l1[a] > l1[b]; });
    std::copy(idx.begin(), idx.end(), out);
  };
  order(rl, row_order);
  order(cl, col_order);
  return GBB_OK;
}
