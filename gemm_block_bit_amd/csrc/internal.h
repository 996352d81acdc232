// Internal declarations shared by the host sources and the kernel launchers.
#pragma once
#include <cstddef>
#include <cstdint>

#include "gbb.h"

namespace gbb {

// Records the text for gbb_last_error() (thread-local) and returns `st`.
gbb_status fail(gbb_status st, const char* fmt, ...);
gbb_status ok();

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
};

// Decode (M <= 32) launch plan: one workgroup of nw waves per block row and
// K segment.  Split-K calls keep, per output element, one 64-bit fixed-point
// accumulator (first M * N * 8 bytes of the workspace) and one fp32 overflow
// accumulator (next M * N * 4 bytes); both return to zero when a call ends.
constexpr int kMaxRows = 1 << 20;   // N limit of the block format's entry points
constexpr int kMaxSegments = 32;    // K segments per block row (fits the count field)
struct DecodePlan {
  int nw, nseg, seg_cols;
  int rows;   // block rows per workgroup (1, or 2 for large matrices at M > 16)
  size_t ws_bytes;
};
DecodePlan decode_plan(int N, int K, int M);

int launch_decode(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M,
                  void* workspace, const DecodePlan& plan, void* stream);
int launch_prefill(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* stream);
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
int launch_w48(const W48ImageView& im, const int8_t* xq, const uint16_t* xs, int ga, uint16_t* y,
               int M, void* stream);
int launch_w48_acc(const W48ImageView& im, const int8_t* xq, int32_t* acc, int M, void* stream);

// Returns a message for a HIP error code, or nullptr for success.
const char* device_error_text(int err);

}  // namespace gbb
