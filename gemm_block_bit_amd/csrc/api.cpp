// C-ABI entry points of the device path: argument checks, image section
// addresses and kernel dispatch.  No allocation, no synchronization.
#include <cstdint>
#include <cstring>

#include "internal.h"
#include "layout.h"

using namespace gbb;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gbb_status device_status(int err, const char* what) {
  const char* msg = device_error_text(err);
  if (!msg) return GBB_OK;
  return fail(GBB_E_DEVICE, "%s: HIP error %d (%s)", what, err, msg);
}

gbb_status check_block_args(const void* image, int N, int K, int M) {
  if (!image) return fail(GBB_E_ARG, "image is NULL");
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  if (N > kMaxRows) return fail(GBB_E_SHAPE, "N=%d exceeds %d", N, kMaxRows);
  if (M < 0) return fail(GBB_E_ARG, "M must not be negative (M=%d)", M);
  if (N % kBlockRows || K % kGroup)
    return fail(GBB_E_SHAPE, "N must be a multiple of 64 and K of 128 (N=%d K=%d)", N, K);
  if (!aligned16(image)) return fail(GBB_E_ALIGN, "image is not 16-byte aligned");
  return GBB_OK;
}

BlockImageView block_view(const void* image, int N, int K) {
  const BlockLayout l = block_layout(N, K);
  const uint8_t* b = static_cast<const uint8_t*>(image);
  BlockImageView v;
  v.bits = b + l.bits_off;
  v.offs = reinterpret_cast<const uint32_t*>(b + l.offs_off);
  v.sz = reinterpret_cast<const uint32_t*>(b + l.sz_off);
  v.codes = b + l.codes_off;
  v.N = N;
  v.K = K;
  v.nbr = N / kBlockRows;
  v.nbc = K / kGroup;
  return v;
}

gbb_status check_w48_args(const void* image, int N, int K, int n8) {
  if (!image) return fail(GBB_E_ARG, "image is NULL");
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  if (K % kGroup) return fail(GBB_E_SHAPE, "K must be a multiple of 128 (K=%d)", K);
  if (n8 < 0 || n8 > N) return fail(GBB_E_SHAPE, "n8=%d outside [0, N=%d]", n8, N);
  if (!aligned16(image)) return fail(GBB_E_ALIGN, "image is not 16-byte aligned");
  return GBB_OK;
}

W48ImageView w48_view(const void* image, int N, int K, int n8) {
  const W48Layout l = w48_layout(N, K, n8);
  const uint8_t* b = static_cast<const uint8_t*>(image);
  W48ImageView v;
  v.rows = reinterpret_cast<const int32_t*>(b + l.rows_off);
  v.s = reinterpret_cast<const uint16_t*>(b + l.s_off);
  v.z = b + l.z_off;
  v.c8 = reinterpret_cast<const int8_t*>(b + l.c8_off);
  v.c4 = b + l.c4_off;
  v.N = N;
  v.K = K;
  v.n8 = n8;
  v.n4 = N - n8;
  v.T8 = l.T8;
  v.T4 = l.T4;
  return v;
}

// For 32 < M the prefill kernel gives each CU one tile of 128 tokens x 512
// rows over the whole of K and does not split K, so few tiles leave most CUs
// idle (the Llama-3-70B down projection, 8192 x 28672, has 16 tiles at
// M <= 128: ~0.8 ms whatever M is).  When ceil(M / 32) chunks of the prefill
// grid still fit in one wave of CUs, the decode kernels run the batch in
// 32-token chunks instead; each chunk rereads the weights, but at 48 us per
// chunk on that shape that is far cheaper.
bool decode_in_chunks(int N, int M) {
  if (M <= 32) return false;
  return size_t((M + 31) / 32) * size_t(prefill_tiles(N, M)) <= size_t(device_compute_units());
}

// Workspace of the decode launches of a batch of M tokens run as 32-token
// chunks: the largest over the full chunks and the last, shorter one.
size_t chunked_workspace(int N, int K, int M) {
  size_t need = decode_plan(N, K, 32).ws_bytes;
  if (M % 32) need = need > decode_plan(N, K, M % 32).ws_bytes ? need : decode_plan(N, K, M % 32).ws_bytes;
  return need;
}

}  // namespace

extern "C" int gbb_version(void) { return 100; }

extern "C" size_t gbb_gemm_mixed_w_workspace(int N, int K, int M) {
  if (N <= 0 || K <= 0 || M <= 0 || N % kBlockRows || K % kGroup) return 0;
  if (M > 32) return decode_in_chunks(N, M) ? chunked_workspace(N, K, M) : 0;
  const DecodePlan p = decode_plan(N, K, M);
  return p.ws_bytes;
}

extern "C" gbb_status gbb_gemm_mixed_w_path(const void* image, int N, int K, const uint16_t* x, uint16_t* y,
                                            int M, void* workspace, size_t ws_bytes, int path, void* stream) {
  gbb_status st = check_block_args(image, N, K, M);
  if (st != GBB_OK) return st;
  if (M == 0) return GBB_OK;
  if (!x || !y) return fail(GBB_E_ARG, "x and y must not be NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(GBB_E_ALIGN, "x and y must be 16-byte aligned");
  if (path < 0 || path > 2) return fail(GBB_E_ARG, "path must be 0, 1 or 2 (got %d)", path);
  if (path == 1 && M > 32) return fail(GBB_E_ARG, "the decode kernel takes M <= 32 (M=%d)", M);
  const char* xb = reinterpret_cast<const char*>(x);
  const char* yb = reinterpret_cast<const char*>(y);
  if (xb < yb + size_t(M) * N * 2 && yb < xb + size_t(M) * K * 2) return fail(GBB_E_ARG, "x and y overlap");
  const BlockImageView v = block_view(image, N, K);
  if (path == 0 && decode_in_chunks(N, M)) {
    const size_t need = chunked_workspace(N, K, M);
    if (need) {
      if (!workspace) return fail(GBB_E_ARG, "workspace of %zu bytes is required", need);
      if (ws_bytes < need) return fail(GBB_E_SPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
      if (!aligned16(workspace)) return fail(GBB_E_ALIGN, "workspace is not 16-byte aligned");
    }
    for (int m0 = 0; m0 < M; m0 += 32) {
      const int mc = M - m0 < 32 ? M - m0 : 32;
      const gbb_status st = device_status(launch_decode(v, x + size_t(m0) * K, y + size_t(m0) * N, mc, workspace,
                                                        decode_plan(N, K, mc), stream),
                                          "decode launch");
      if (st != GBB_OK) return st;
    }
    return GBB_OK;
  }
  const bool decode = path == 1 || (path == 0 && M <= 32);
  if (decode) {
    const DecodePlan p = decode_plan(N, K, M);
    const size_t need = p.ws_bytes;
    if (need) {
      if (!workspace) return fail(GBB_E_ARG, "workspace of %zu bytes is required", need);
      if (ws_bytes < need) return fail(GBB_E_SPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
      if (!aligned16(workspace)) return fail(GBB_E_ALIGN, "workspace is not 16-byte aligned");
    }
    return device_status(launch_decode(v, x, y, M, workspace, p, stream), "decode launch");
  }
  if (size_t(M) * size_t(K) >= (size_t(1) << 31))
    return fail(GBB_E_SHAPE, "the prefill kernel takes M * K < 2^31 (M=%d K=%d)", M, K);
  return device_status(launch_prefill(v, x, y, M, stream), "prefill launch");
}

extern "C" gbb_status gbb_gemm_mixed_w(const void* image, int N, int K, const uint16_t* x, uint16_t* y, int M,
                                       void* workspace, size_t ws_bytes, void* stream) {
  return gbb_gemm_mixed_w_path(image, N, K, x, y, M, workspace, ws_bytes, 0, stream);
}

extern "C" gbb_status gbb_unpack_codes(const void* image, int N, int K, uint8_t* q, void* stream) {
  gbb_status st = check_block_args(image, N, K, 1);
  if (st != GBB_OK) return st;
  if (!q) return fail(GBB_E_ARG, "q is NULL");
  return device_status(launch_unpack(block_view(image, N, K), q, nullptr, nullptr, stream), "unpack launch");
}

extern "C" gbb_status gbb_dequant(const void* image, int N, int K, float* w32, uint16_t* w16, void* stream) {
  gbb_status st = check_block_args(image, N, K, 1);
  if (st != GBB_OK) return st;
  if (!w32 && !w16) return fail(GBB_E_ARG, "w32 and w16 are both NULL");
  return device_status(launch_unpack(block_view(image, N, K), nullptr, w32, w16, stream), "dequant launch");
}

extern "C" gbb_status gbb_quant_act_i8(const uint16_t* x, int M, int K, int ga, int8_t* xq, uint16_t* xs,
                                       void* stream) {
  if (!x || !xq || !xs) return fail(GBB_E_ARG, "x, xq and xs must not be NULL");
  if (M <= 0 || K <= 0) return fail(GBB_E_ARG, "M and K must be positive (M=%d K=%d)", M, K);
  if (K % kGroup) return fail(GBB_E_SHAPE, "K must be a multiple of 128 (K=%d)", K);
  if (ga != K && ga != 128) return fail(GBB_E_ARG, "ga must be K or 128 (ga=%d)", ga);
  if (!aligned16(x) || !aligned16(xq)) return fail(GBB_E_ALIGN, "x and xq must be 16-byte aligned");
  return device_status(launch_quant_act(x, M, K, ga, xq, xs, stream), "activation quantization launch");
}

extern "C" gbb_status gbb_gemm_w48a8(const void* image, int N, int K, int n8, const int8_t* xq,
                                     const uint16_t* xs, int ga, uint16_t* y, int M, void* stream) {
  gbb_status st = check_w48_args(image, N, K, n8);
  if (st != GBB_OK) return st;
  if (M < 0) return fail(GBB_E_ARG, "M must not be negative (M=%d)", M);
  if (M == 0) return GBB_OK;
  if (!xq || !xs || !y) return fail(GBB_E_ARG, "xq, xs and y must not be NULL");
  if (ga != K && ga != 128) return fail(GBB_E_ARG, "ga must be K or 128 (ga=%d)", ga);
  if (!aligned16(xq)) return fail(GBB_E_ALIGN, "xq must be 16-byte aligned");
  return device_status(launch_w48(w48_view(image, N, K, n8), xq, xs, ga, y, M, stream), "w48 launch");
}

extern "C" gbb_status gbb_w48_group_acc(const void* image, int N, int K, int n8, const int8_t* xq,
                                        int32_t* acc, int M, void* stream) {
  gbb_status st = check_w48_args(image, N, K, n8);
  if (st != GBB_OK) return st;
  if (M <= 0) return fail(GBB_E_ARG, "M must be positive (M=%d)", M);
  if (!xq || !acc) return fail(GBB_E_ARG, "xq and acc must not be NULL");
  if (!aligned16(xq)) return fail(GBB_E_ALIGN, "xq must be 16-byte aligned");
  return device_status(launch_w48_acc(w48_view(image, N, K, n8), xq, acc, M, stream), "w48 acc launch");
}
