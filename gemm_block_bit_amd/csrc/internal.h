// Internal declarations shared by the host sources and the kernel launchers.
#pragma once
#include <cstddef>
#include <cstdint>

#include "gbb.h"

namespace gbb {

// Records the text for gbb_last_error() (thread-local) and returns `st`.
gbb_status fail(gbb_status st, const char* fmt, ...);
gbb_status ok();

// Argument checks of gbb_gemm_mixed_w_path (path 0 = automatic), shared by
// the entry points that run it.
gbb_status check_gemm_args(const void* image, int N, int K, const uint16_t* x, const uint16_t* y, int M,
                           int path, int bc = 128);

// IEEE binary16 <-> binary64, round-to-nearest-even (host).
double half_to_double(uint16_t h);
uint16_t double_to_half(double d);

// ---- kernel launchers (defined in the .hip files) ----------------------------
struct BlockImageView {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  int N, K, nbr, nbc;
  int bc;   // block columns: 128, or 64 for 64x64 blocks
};

// Decode (M <= 32) launch plan: one workgroup of nw waves per block row and
// K segment.  Split-K calls keep, per output element, one 64-bit fixed-point
// accumulator (first M * N * 8 bytes of the workspace) and one fp32 overflow
// accumulator (next M * N * 4 bytes); both return to zero when a call ends.
constexpr int kMaxRows = 1 << 20;   // N limit of the block format's entry points
constexpr int kMaxCols = 1 << 20;   // K limit: the decode kernels address a token's row with a
                                    // 32-bit byte offset (up to 32 tokens x 2 K bytes)
constexpr int kMaxSegments = 32;    // K segments per block row (fits the count field)
struct DecodePlan {
  int nw, nseg, seg_cols;
  int rows;   // block rows per workgroup (1, or 2 for large matrices at M > 16)
  size_t ws_bytes;
};
DecodePlan decode_plan(int N, int K, int M);

int launch_decode(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M,
                  void* workspace, const DecodePlan& plan, void* stream);
// n <= kMaxBatch independent problems with the same M <= 16 in one launch;
// problem i uses plans[i] (from decode_plan) and workspaces[i].
constexpr int kMaxBatch = 32;
int launch_decode_batch(int n, const BlockImageView* ims, const uint16_t* const* x, uint16_t* const* y, int M,
                        const DecodePlan* plans, void* const* workspaces, void* stream);
struct PrefillPlan {
  int kseg, seg_cols, tiles;
  size_t ws_bytes;   // kseg fp32 partials of y when kseg > 1
};
// The prefill launch for (N, K, M) on blocks of bc columns with a workspace
// of ws_bytes (a K split only when its counts and partials fit).
PrefillPlan prefill_plan(int N, int K, int M, int bc, size_t ws_bytes);
// The least workspace a 64x128 block call of (N, K, M) runs with (the decode
// accumulators; 0 on the prefill route, whose K split fits what it is given).
size_t required_workspace(int N, int K, int M);
// y[M][N] (fp16) = the sum over kseg of fp32 partials part[kseg][M][N] in
// segment order, and the partials cleared to zero; N a multiple of 64.
int launch_split_reduce(float* part, uint16_t* y, int M, int N, int kseg, void* stream);
int launch_prefill(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* workspace,
                   const PrefillPlan& plan, void* stream);
// 64x64-block images, M <= 32: the plan (seg_cols and nbc in 64-column
// blocks, one block row per workgroup) and the launch.
DecodePlan decode_plan64(int N, int K, int M);
int launch_decode64(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* workspace,
                    const DecodePlan& plan, void* stream);
// Workgroup tiles of the prefill kernel for N rows and M tokens, and the
// current device's compute units (looked up once per device).
int prefill_tiles(int N, int M);
int device_compute_units();
int launch_unpack(const BlockImageView& im, uint8_t* q, float* w32, uint16_t* w16, void* stream);

struct W48ImageView {
  const int32_t* rows;
  const uint16_t* s;
  const uint8_t* z;
  const int8_t* c8;
  const uint8_t* c4;
  int N, K, n8, n4, T8, T4;
};
int launch_quant_act(const uint16_t* x, int M, int K, int ga, int8_t* xq, uint16_t* xs, void* stream);
// The stream kernel's K split: kseg8 (kseg4) segments of seg8 (seg4)
// 128-column groups for the 8-bit (4-bit) row blocks, whose fp32 partials
// take ws_bytes (0 without a split).
struct W48Split {
  int kseg8, seg8, kseg4, seg4;
  size_t ws_bytes;
  int tiles;   // the stream kernel's packed tiles per wave (1 or 2)
  int tt;      // the tile kernel's 16-token tiles per workgroup (8 or 4)
};
W48Split w48_split(int K, int T8, int T4, int M, size_t ws_bytes);
// The tile kernel's K split (M > 64), the same layout of partials.
W48Split w48_tile_split(int K, int T8, int T4, int M, int ga, size_t ws_bytes);
bool w48_streams(int K, int T8, int T4, int M, int ga);
// workspace (16-byte aligned, zero at rest) of ws_bytes bounds the stream
// kernel's K split; NULL runs it unsplit.
int launch_w48(const W48ImageView& im, const int8_t* xq, const uint16_t* xs, int ga, uint16_t* y,
               int M, void* workspace, size_t ws_bytes, void* stream);
int launch_w48_acc(const W48ImageView& im, const int8_t* xq, int ga, int32_t* acc, int M, void* stream);

// Returns a message for a HIP error code, or nullptr for success.
const char* device_error_text(int err);

}  // namespace gbb
