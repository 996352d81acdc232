// C-ABI entry points of the device path: argument checks, image section
// addresses and kernel dispatch.  No allocation, no synchronization.
#include <algorithm>
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

// bc: block columns, 128 (64x128 blocks) or 64 (64x64 blocks).
gbb_status check_block_args(const void* image, int N, int K, int M, int bc = kGroup) {
  if (!image) return fail(GBB_E_ARG, "image is NULL");
  if (N <= 0 || K <= 0) return fail(GBB_E_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  if (N > kMaxRows) return fail(GBB_E_SHAPE, "N=%d exceeds %d", N, kMaxRows);
  if (K > kMaxCols) return fail(GBB_E_SHAPE, "K=%d exceeds %d", K, kMaxCols);
  if (M < 0) return fail(GBB_E_ARG, "M must not be negative (M=%d)", M);
  if (N % kBlockRows || K % bc)
    return fail(GBB_E_SHAPE, "N must be a multiple of 64 and K of %d (N=%d K=%d)", bc, N, K);
  if (!aligned16(image)) return fail(GBB_E_ALIGN, "image is not 16-byte aligned");
  return GBB_OK;
}

BlockImageView block_view(const void* image, int N, int K, int bc = kGroup) {
  const BlockLayout l = block_layout(N, K, bc);
  const uint8_t* b = static_cast<const uint8_t*>(image);
  BlockImageView v;
  v.bits = b + l.bits_off;
  v.offs = reinterpret_cast<const uint32_t*>(b + l.offs_off);
  v.sz = reinterpret_cast<const uint32_t*>(b + l.sz_off);
  v.codes = b + l.codes_off;
  v.N = N;
  v.K = K;
  v.nbr = N / kBlockRows;
  v.nbc = K / bc;
  v.bc = bc;
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

// For 32 < M: ceil(M / 32) decode launches of 32 tokens each stream the
// whole matrix, so their cost grows with the chunk count, while the prefill
// kernel (one tile of 128 tokens x 512 rows per CU, K cut into segments when
// the tiles fill at most half of the CUs: prefill_plan) costs about the same
// for any M up to its tile and grows slowly beyond.  The batch runs as
// chunks when
//     chunks x max(CUs / 4, g) <= 3/4 CUs,
// g the split prefill's workgroups and a ragged last chunk counted as half
// (a decode launch of few tokens costs about half one of 32): chunks win
// on small matrices up to about three chunks, on matrices whose prefill
// grid is larger only for a 32-token chunk plus a short one, and never
// when the prefill grid fills the CUs.  Measured on Llama-3 shapes in
// graphs: 70B q 8192 x 8192 at M = 64 / 128 in 49 / 97 us as chunks against
// 37 / 50 us as split prefill; 70B k 1024 x 8192 at M = 96 in 33 us as
// chunks against 41 us; 70B down projection at M = 64 in 60 us as split
// prefill against 117 us as chunks.
bool decode_in_chunks(int N, int K, int M, int bc) {
  if (M <= 32) return false;
  const PrefillPlan p = prefill_plan(N, K, M, bc, SIZE_MAX);
  const size_t cus = size_t(device_compute_units());
  const size_t g = size_t(p.tiles) * size_t(p.kseg);
  const size_t halves = size_t(2) * size_t(M / 32) + (M % 32 ? 1 : 0);   // chunks, in halves
  return size_t(2) * halves * std::max(cus / 4, g) <= 3 * cus;
}

// Workspace of the decode launches of a batch of M tokens run as 32-token
// chunks: the largest over the full chunks and the last, shorter one.
size_t chunked_workspace(int N, int K, int M) {
  size_t need = decode_plan(N, K, 32).ws_bytes;
  if (M % 32) need = need > decode_plan(N, K, M % 32).ws_bytes ? need : decode_plan(N, K, M % 32).ws_bytes;
  return need;
}

// The prefill kernel, with the K split that the caller's workspace holds (none
// without one: the call then runs unsplit, as it would on any workspace too
// small for the split).
gbb_status run_prefill(const BlockImageView& v, const uint16_t* x, uint16_t* y, int M, void* workspace,
                       size_t ws_bytes, void* stream) {
  const PrefillPlan plan = prefill_plan(v.N, v.K, M, v.bc, workspace && aligned16(workspace) ? ws_bytes : 0);
  return device_status(launch_prefill(v, x, y, M, workspace, plan, stream), "prefill launch");
}

}  // namespace

extern "C" int gbb_version(void) { return 100; }

extern "C" size_t gbb_gemm_mixed_w_workspace(int N, int K, int M) {
  if (N <= 0 || K <= 0 || M <= 0 || N % kBlockRows || K % kGroup) return 0;
  if (M > 32)
    return decode_in_chunks(N, K, M, kGroup) ? chunked_workspace(N, K, M) : prefill_plan(N, K, M, kGroup, SIZE_MAX).ws_bytes;
  const DecodePlan p = decode_plan(N, K, M);
  return p.ws_bytes;
}

// The least workspace gbb_gemm_mixed_w runs (N, K, M) with: the decode
// launches' accumulators, for the whole batch or its 32-token chunks.  The
// prefill kernel splits K only as far as the workspace it is given holds.
size_t gbb::required_workspace(int N, int K, int M) {
  if (M > 32 && !decode_in_chunks(N, K, M, kGroup)) return 0;
  return gbb_gemm_mixed_w_workspace(N, K, M);
}

extern "C" size_t gbb_gemm_mixed_w_path_workspace(int N, int K, int M, int path) {
  if (N <= 0 || K <= 0 || M <= 0 || N % kBlockRows || K % kGroup) return 0;
  if (path == 0) return gbb_gemm_mixed_w_workspace(N, K, M);
  if (path == 1) return M <= 32 ? decode_plan(N, K, M).ws_bytes : 0;
  if (path == 2) return prefill_plan(N, K, M, kGroup, SIZE_MAX).ws_bytes;
  return 0;
}

gbb_status gbb::check_gemm_args(const void* image, int N, int K, const uint16_t* x, const uint16_t* y, int M,
                                int path, int bc) {
  gbb_status st = check_block_args(image, N, K, M, bc);
  if (st != GBB_OK) return st;
  if (M == 0) return GBB_OK;
  if (!x || !y) return fail(GBB_E_ARG, "x and y must not be NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(GBB_E_ALIGN, "x and y must be 16-byte aligned");
  if (path < 0 || path > 2) return fail(GBB_E_ARG, "path must be 0, 1 or 2 (got %d)", path);
  if (path == 1 && M > 32) return fail(GBB_E_ARG, "the decode kernel takes M <= 32 (M=%d)", M);
  const char* xb = reinterpret_cast<const char*>(x);
  const char* yb = reinterpret_cast<const char*>(y);
  if (xb < yb + size_t(M) * N * 2 && yb < xb + size_t(M) * K * 2) return fail(GBB_E_ARG, "x and y overlap");
  return GBB_OK;
}

extern "C" gbb_status gbb_gemm_mixed_w_path(const void* image, int N, int K, const uint16_t* x, uint16_t* y,
                                            int M, void* workspace, size_t ws_bytes, int path, void* stream) {
  gbb_status st = check_gemm_args(image, N, K, x, y, M, path);
  if (st != GBB_OK || M == 0) return st;
  const BlockImageView v = block_view(image, N, K);
  if (path == 0 && decode_in_chunks(N, K, M, kGroup)) {
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
  return run_prefill(v, x, y, M, workspace, ws_bytes, stream);
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
  return device_status(launch_w48(w48_view(image, N, K, n8), xq, xs, ga, y, M, nullptr, 0, stream), "w48 launch");
}

extern "C" size_t gbb_gemm_w48a8_workspace(int N, int K, int n8, int M, int ga) {
  if (N <= 0 || K <= 0 || K % kGroup || n8 < 0 || n8 > N || M <= 0 || (ga != K && ga != 128)) return 0;
  const W48Layout l = w48_layout(N, K, n8);
  if (w48_streams(K, l.T8, l.T4, M, ga)) return w48_split(K, l.T8, l.T4, M < 64 ? M : 64, SIZE_MAX).ws_bytes;
  if (M > 64) return w48_tile_split(K, l.T8, l.T4, M, ga, SIZE_MAX).ws_bytes;
  return 0;   // group activation scales over an odd group count at M <= 64: the register-staged kernel
}

extern "C" gbb_status gbb_gemm_w48a8_split(const void* image, int N, int K, int n8, const int8_t* xq,
                                           const uint16_t* xs, int ga, uint16_t* y, int M, void* workspace,
                                           size_t ws_bytes, void* stream) {
  gbb_status st = check_w48_args(image, N, K, n8);
  if (st != GBB_OK) return st;
  if (M < 0) return fail(GBB_E_ARG, "M must not be negative (M=%d)", M);
  if (M == 0) return GBB_OK;
  if (!xq || !xs || !y) return fail(GBB_E_ARG, "xq, xs and y must not be NULL");
  if (ga != K && ga != 128) return fail(GBB_E_ARG, "ga must be K or 128 (ga=%d)", ga);
  if (!aligned16(xq)) return fail(GBB_E_ALIGN, "xq must be 16-byte aligned");
  if (workspace && !aligned16(workspace)) return fail(GBB_E_ALIGN, "workspace is not 16-byte aligned");
  return device_status(launch_w48(w48_view(image, N, K, n8), xq, xs, ga, y, M, workspace, workspace ? ws_bytes : 0,
                                  stream),
                       "w48 launch");
}

extern "C" gbb_status gbb_w48_group_acc(const void* image, int N, int K, int n8, const int8_t* xq, int ga,
                                        int32_t* acc, int M, void* stream) {
  gbb_status st = check_w48_args(image, N, K, n8);
  if (st != GBB_OK) return st;
  if (M <= 0) return fail(GBB_E_ARG, "M must be positive (M=%d)", M);
  if (!xq || !acc) return fail(GBB_E_ARG, "xq and acc must not be NULL");
  if (ga != K && ga != 128) return fail(GBB_E_ARG, "ga must be K or 128 (ga=%d)", ga);
  if (!aligned16(xq)) return fail(GBB_E_ALIGN, "xq must be 16-byte aligned");
  return device_status(launch_w48_acc(w48_view(image, N, K, n8), xq, ga, acc, M, stream), "w48 acc launch");
}

namespace {

// Workspace bytes of problem i of a grouped call (each region 256-aligned).
size_t batch_ws_one(int N, int K, int M) {
  const size_t w = M <= 16 ? decode_plan(N, K, M).ws_bytes : gbb_gemm_mixed_w_workspace(N, K, M);
  return (w + 255) & ~size_t(255);
}

}  // namespace

extern "C" size_t gbb_gemm_mixed_w_batched_workspace(int n, const int* N, const int* K, int M) {
  if (n < 1 || n > kMaxBatch || !N || !K || M <= 0) return 0;
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (N[i] <= 0 || K[i] <= 0 || N[i] % kBlockRows || K[i] % kGroup) return 0;
    total += batch_ws_one(N[i], K[i], M);
  }
  return total;
}

extern "C" gbb_status gbb_gemm_mixed_w_batched(int n, const void* const* images, const int* N, const int* K,
                                               const uint16_t* const* x, uint16_t* const* y, int M, void* workspace,
                                               size_t ws_bytes, void* stream) {
  if (n < 1 || n > kMaxBatch) return fail(GBB_E_ARG, "n must be in 1 ... %d (n=%d)", kMaxBatch, n);
  if (!images || !N || !K || !x || !y) return fail(GBB_E_ARG, "images, N, K, x and y must not be NULL");
  for (int i = 0; i < n; ++i) {
    const gbb_status st = check_gemm_args(images[i], N[i], K[i], x[i], y[i], M, 0);
    if (st != GBB_OK) return fail(st, "problem %d: %s", i, gbb_last_error());
  }
  if (M == 0) return GBB_OK;
  size_t off[kMaxBatch + 1];
  off[0] = 0;
  for (int i = 0; i < n; ++i) off[i + 1] = off[i] + batch_ws_one(N[i], K[i], M);
  if (off[n]) {
    if (!workspace) return fail(GBB_E_ARG, "workspace of %zu bytes is required", off[n]);
    if (ws_bytes < off[n]) return fail(GBB_E_SPACE, "workspace needs %zu bytes, got %zu", off[n], ws_bytes);
    if (!aligned16(workspace)) return fail(GBB_E_ALIGN, "workspace is not 16-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  if (M > 16) {   // one launch (or chunk sequence) per problem, as gbb_gemm_mixed_w
    for (int i = 0; i < n; ++i) {
      const gbb_status st = gbb_gemm_mixed_w(images[i], N[i], K[i], x[i], y[i], M, ws ? ws + off[i] : nullptr,
                                             off[i + 1] - off[i], stream);
      if (st != GBB_OK) return st;
    }
    return GBB_OK;
  }
  BlockImageView views[kMaxBatch];
  DecodePlan plans[kMaxBatch];
  void* wss[kMaxBatch];
  for (int i = 0; i < n; ++i) {
    views[i] = block_view(images[i], N[i], K[i]);
    plans[i] = decode_plan(N[i], K[i], M);
    wss[i] = ws ? ws + off[i] : nullptr;
  }
  return device_status(launch_decode_batch(n, views, x, y, M, plans, wss, stream), "grouped decode launch");
}

// ---------------------------------------------------------------------------
// 64x64 blocks
// ---------------------------------------------------------------------------
namespace {

size_t workspace64(int N, int K, int M) {
  if (M <= 32) return decode_plan64(N, K, M).ws_bytes;
  if (!decode_in_chunks(N, K, M, 64)) return prefill_plan(N, K, M, 64, SIZE_MAX).ws_bytes;   // the prefill kernel
  size_t need = decode_plan64(N, K, 32).ws_bytes;   // 32-token chunks
  if (M % 32) need = std::max(need, decode_plan64(N, K, M % 32).ws_bytes);
  return need;
}

}  // namespace

extern "C" size_t gbb_gemm_mixed_w_64x64_workspace(int N, int K, int M) {
  if (N <= 0 || K <= 0 || M <= 0 || N % kBlockRows || K % 64) return 0;
  return workspace64(N, K, M);
}

extern "C" size_t gbb_gemm_mixed_w_64x64_path_workspace(int N, int K, int M, int path) {
  if (N <= 0 || K <= 0 || M <= 0 || N % kBlockRows || K % 64) return 0;
  if (path == 0) return workspace64(N, K, M);
  if (path == 1) return M <= 32 ? decode_plan64(N, K, M).ws_bytes : 0;
  if (path == 2) return prefill_plan(N, K, M, 64, SIZE_MAX).ws_bytes;
  return 0;
}

extern "C" gbb_status gbb_gemm_mixed_w_64x64_path(const void* image, int N, int K, const uint16_t* x, uint16_t* y,
                                                  int M, void* workspace, size_t ws_bytes, int path, void* stream) {
  gbb_status st = check_gemm_args(image, N, K, x, y, M, path, 64);
  if (st != GBB_OK || M == 0) return st;
  const BlockImageView v = block_view(image, N, K, 64);
  const bool chunks = path == 0 && decode_in_chunks(N, K, M, 64);
  const bool decode = path == 1 || (path == 0 && M <= 32);
  if (chunks || decode) {
    const size_t need = decode ? decode_plan64(N, K, M).ws_bytes : workspace64(N, K, M);
    if (need) {
      if (!workspace) return fail(GBB_E_ARG, "workspace of %zu bytes is required", need);
      if (ws_bytes < need) return fail(GBB_E_SPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
      if (!aligned16(workspace)) return fail(GBB_E_ALIGN, "workspace is not 16-byte aligned");
    }
    for (int m0 = 0; m0 < M; m0 += 32) {   // one launch for M <= 32
      const int mc = M - m0 < 32 ? M - m0 : 32;
      st = device_status(launch_decode64(v, x + size_t(m0) * K, y + size_t(m0) * N, mc, workspace,
                                         decode_plan64(N, K, mc), stream),
                         "decode launch");
      if (st != GBB_OK) return st;
    }
    return GBB_OK;
  }
  if (size_t(M) * size_t(K) >= (size_t(1) << 31))
    return fail(GBB_E_SHAPE, "the prefill kernel takes M * K < 2^31 (M=%d K=%d)", M, K);
  return run_prefill(v, x, y, M, workspace, ws_bytes, stream);
}

extern "C" gbb_status gbb_gemm_mixed_w_64x64(const void* image, int N, int K, const uint16_t* x, uint16_t* y, int M,
                                             void* workspace, size_t ws_bytes, void* stream) {
  return gbb_gemm_mixed_w_64x64_path(image, N, K, x, y, M, workspace, ws_bytes, 0, stream);
}

extern "C" gbb_status gbb_unpack_codes_64x64(const void* image, int N, int K, uint8_t* q, void* stream) {
  gbb_status st = check_block_args(image, N, K, 1, 64);
  if (st != GBB_OK) return st;
  if (!q) return fail(GBB_E_ARG, "q is NULL");
  return device_status(launch_unpack(block_view(image, N, K, 64), q, nullptr, nullptr, stream), "unpack launch");
}

extern "C" gbb_status gbb_dequant_64x64(const void* image, int N, int K, float* w32, uint16_t* w16, void* stream) {
  gbb_status st = check_block_args(image, N, K, 1, 64);
  if (st != GBB_OK) return st;
  if (!w32 && !w16) return fail(GBB_E_ARG, "w32 and w16 are both NULL");
  return device_status(launch_unpack(block_view(image, N, K, 64), nullptr, w32, w16, stream), "dequant launch");
}
