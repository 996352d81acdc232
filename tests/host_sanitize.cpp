// Host-side driver for the packer, the allocation and the channel order,
// built with -fsanitize=address,undefined (tests/test_host_sanitizers.py):
// every host entry point on valid inputs of several shapes and bitmaps, and
// its error paths.  Exits non-zero on a failed expectation; the sanitizers
// abort on any memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "gbb.h"

static int failures = 0;

#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

// Random finite fp16 bit patterns around 2^-6 ... 2^5, both signs, with a few zeros.
static std::vector<uint16_t> random_weights(int N, int K, uint32_t seed) {
  std::mt19937 g(seed);
  std::vector<uint16_t> w(size_t(N) * size_t(K));
  for (auto& v : w) {
    const uint32_t r = g();
    if ((r & 255u) == 0) {
      v = 0;
      continue;
    }
    const uint16_t sign = uint16_t((r >> 8) & 1u) << 15;
    const uint16_t exp = uint16_t(9 + (r >> 9) % 12) << 10;
    v = uint16_t(sign | exp | ((r >> 16) & 1023u));
  }
  return w;
}

static void check_blocks(int N, int K, const std::vector<uint8_t>& bits, uint32_t seed) {
  const auto W = random_weights(N, K, seed);
  const size_t bytes = gbb_packed_bytes(bits.data(), N, K);
  EXPECT(bytes > 0);
  std::vector<uint8_t> img(bytes), img2(bytes);
  std::vector<uint16_t> s(size_t(N) * (K / 128)), z(s.size());
  EXPECT(gbb_pack_blocks(W.data(), N, K, bits.data(), s.data(), z.data(), 0, img.data(), bytes) == GBB_OK);
  EXPECT(gbb_check_image(img.data(), bytes, N, K) == GBB_OK);
  EXPECT(gbb_check_image(img.data(), bytes, N + 64, K) != GBB_OK);
  // the returned scales and zero points reproduce the image byte for byte
  EXPECT(gbb_pack_blocks(W.data(), N, K, bits.data(), s.data(), z.data(), GBB_PACK_GIVEN_SZ, img2.data(), bytes) ==
         GBB_OK);
  EXPECT(std::memcmp(img.data(), img2.data(), bytes) == 0);
  EXPECT(gbb_pack_blocks(W.data(), N, K, bits.data(), nullptr, nullptr, 0, img2.data(), bytes) == GBB_OK);
  EXPECT(std::memcmp(img.data(), img2.data(), bytes) == 0);
  // too small an output, bad arguments
  EXPECT(gbb_pack_blocks(W.data(), N, K, bits.data(), nullptr, nullptr, 0, img2.data(), bytes - 1) == GBB_E_SPACE);
  EXPECT(gbb_pack_blocks(nullptr, N, K, bits.data(), nullptr, nullptr, 0, img2.data(), bytes) == GBB_E_ARG);
  EXPECT(gbb_pack_blocks(W.data(), N, K + 64, bits.data(), nullptr, nullptr, 0, img2.data(), bytes) != GBB_OK);

  std::vector<uint8_t> alloc(bits.size());
  for (double target : {1.0, 2.1, 3.0, 4.5, 8.0}) {
    EXPECT(gbb_allocate_bits(W.data(), N, K, target, 0.05, alloc.data()) == GBB_OK);
    long total = 0;
    for (uint8_t b : alloc) total += b;
    EXPECT(double(total) <= target * double(alloc.size()) + 1e-9);
  }
  EXPECT(gbb_allocate_bits(W.data(), N, K, 0.5, 0.05, alloc.data()) == GBB_E_ARG);
  EXPECT(gbb_allocate_bits(W.data(), N, K, 3.0, 0.0, alloc.data()) == GBB_E_ARG);
  EXPECT(gbb_allocate_bits(W.data(), N + 1, K, 3.0, 0.05, alloc.data()) != GBB_OK);

  std::vector<int32_t> ro(N), co(K);
  EXPECT(gbb_channel_order(W.data(), N, K, ro.data(), co.data()) == GBB_OK);
  std::vector<char> seen_r(N, 0), seen_c(K, 0);
  for (int32_t r : ro) {
    EXPECT(r >= 0 && r < N);
    if (r >= 0 && r < N) seen_r[r] = 1;
  }
  for (int32_t c : co) {
    EXPECT(c >= 0 && c < K);
    if (c >= 0 && c < K) seen_c[c] = 1;
  }
  for (char v : seen_r) EXPECT(v);
  for (char v : seen_c) EXPECT(v);
  EXPECT(gbb_channel_order(W.data(), N, K, nullptr, co.data()) == GBB_E_ARG);
}

static void check_w48(int N, int K, const std::vector<int32_t>& rows8, uint32_t seed) {
  const auto W = random_weights(N, K, seed);
  const int n8 = int(rows8.size());
  const size_t bytes = gbb_w48_packed_bytes(N, K, n8);
  EXPECT(bytes > 0);
  std::vector<uint8_t> img(bytes);
  std::vector<uint16_t> s(size_t(N) * (K / 128));
  std::vector<uint8_t> z(s.size());
  EXPECT(gbb_pack_w48(W.data(), N, K, rows8.data(), n8, s.data(), z.data(), img.data(), bytes) == GBB_OK);
  EXPECT(gbb_pack_w48(W.data(), N, K, rows8.data(), n8, nullptr, nullptr, img.data(), bytes) == GBB_OK);
  EXPECT(gbb_pack_w48(W.data(), N, K, rows8.data(), n8, nullptr, nullptr, img.data(), bytes - 1) == GBB_E_SPACE);
  if (n8 >= 2) {   // not strictly ascending
    std::vector<int32_t> bad(rows8);
    bad[1] = bad[0];
    EXPECT(gbb_pack_w48(W.data(), N, K, bad.data(), n8, nullptr, nullptr, img.data(), bytes) != GBB_OK);
  }
  if (n8 >= 1) {   // out of range
    std::vector<int32_t> bad(rows8);
    bad[n8 - 1] = N;
    EXPECT(gbb_pack_w48(W.data(), N, K, bad.data(), n8, nullptr, nullptr, img.data(), bytes) != GBB_OK);
  }
}

int main() {
  std::mt19937 g(7);
  const int allowed[6] = {1, 2, 3, 4, 6, 8};
  const int shapes[3][2] = {{64, 128}, {192, 384}, {128, 1280}};
  uint32_t seed = 1;
  for (const auto& sh : shapes) {
    const int N = sh[0], K = sh[1];
    const size_t nblk = size_t(N / 64) * size_t(K / 128);
    std::vector<uint8_t> bits(nblk);
    for (auto& b : bits) b = uint8_t(allowed[g() % 6]);
    check_blocks(N, K, bits, seed++);
    for (int u : {1, 8}) {
      std::vector<uint8_t> uni(nblk, uint8_t(u));
      check_blocks(N, K, uni, seed++);
    }
    std::vector<uint8_t> bad(nblk, 5);   // not an allowed bitwidth
    std::vector<uint8_t> img(1 << 20);
    const auto W = random_weights(N, K, seed++);
    EXPECT(gbb_pack_blocks(W.data(), N, K, bad.data(), nullptr, nullptr, 0, img.data(), img.size()) == GBB_E_BITS);
  }
  check_w48(48, 256, {3, 17, 40}, 100);
  check_w48(200, 384, {}, 101);
  std::vector<int32_t> all(40);
  for (int i = 0; i < 40; ++i) all[i] = i;
  check_w48(40, 256, all, 102);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer driver: ok\n");
  return 0;
}
