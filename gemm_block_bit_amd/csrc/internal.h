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
// K segment.  Split-K calls keep one u32 counter per block row in the first
// kCounterBytes of the workspace (N up to 1 048 576 rows).
constexpr size_t kCounterBytes = 65536;
struct DecodePlan {
  int nw, nseg, seg_cols;
  size_t part_bytes, ctr_bytes;
};
DecodePlan decode_plan(int N, int K, int M);

int launch_decode(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M,
                  void* workspace, const DecodePlan& plan, void* stream);
int launch_prefill(const BlockImageView& im, const uint16_t* x, uint16_t* y, int M, void* stream);
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
