// Debug exports over a device block image: the codes and the exactly
// dequantized weights (q - z) * s in fp32 and rounded to fp16, for
// bit-exactness tests of the packed layout.  One wave per block (64x128 or
// 64x64).
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace gbb {

namespace {

struct UnpackArgs {
  const uint8_t* bits;
  const uint32_t* offs;
  const uint32_t* sz;
  const uint8_t* codes;
  uint8_t* q;
  float* w32;
  _Float16* w16;
  int N, K, nbr, nbc;
};

// Field i of word c of slot j of a plane of width W holds the code pair of
// tile 4 kt + rt = j (16 / W) + i: row 16 rt + lane % 16, columns
// 32 kt + 8 (lane / 16) + 2 c (low half) and + 1 (high half).
template <int W>
__device__ __forceinline__ uint32_t plane_pair(const uint8_t* cb, int u, int c) {
  constexpr int NP = 16 / W;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(cb + 1024 * (u / NP) + 4 * c);
  return (w >> (W * (u % NP))) & (((1u << W) - 1u) * 0x00010001u);
}

template <int W0, int W1>
__device__ void unpack_block(const UnpackArgs& a, int blk, int lane) {
  const int br = blk / a.nbc, bc = blk % a.nbc;
  const uint8_t* cb = a.codes + size_t(a.offs[blk]) * 1024 + 16 * lane;
  for (int u = 0; u < 16; ++u) {
    const int kt = u >> 2, rt = u & 3;
    const int row = br * 64 + 16 * rt + (lane & 15);
    const uint32_t e = a.sz[size_t(blk) * 64 + 4 * (lane & 15) + rt];
    const float s = lo_half(e), z = hi_half(e);
    for (int c = 0; c < 4; ++c) {
      uint32_t pr = plane_pair<W0>(cb, u, c);
      if constexpr (W1 != 0) pr |= plane_pair<W1>(cb + 1024 * W0, u, c) << W0;
      const int col = bc * 128 + 32 * kt + 8 * (lane >> 4) + 2 * c;
      const uint32_t qa = pr & 0xffffu, qb = pr >> 16;
      const size_t o = size_t(row) * a.K + col;
      if (a.q) a.q[o] = uint8_t(qa), a.q[o + 1] = uint8_t(qb);
      const float va = (float(qa) - z) * s, vb = (float(qb) - z) * s;
      if (a.w32) a.w32[o] = va, a.w32[o + 1] = vb;
      if (a.w16) a.w16[o] = (_Float16)va, a.w16[o + 1] = (_Float16)vb;
    }
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(UnpackArgs a) {
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blk >= a.nbr * a.nbc) return;
  switch (a.bits[blk]) {
    case 1: unpack_block<1, 0>(a, blk, lane); break;
    case 2: unpack_block<2, 0>(a, blk, lane); break;
    case 3: unpack_block<2, 1>(a, blk, lane); break;
    case 4: unpack_block<4, 0>(a, blk, lane); break;
    case 6: unpack_block<4, 2>(a, blk, lane); break;
    default: unpack_block<4, 4>(a, blk, lane); break;
  }
}

// 64x64 blocks: word c of tile u = 4 kt + rt (kt = 0, 1) is field
// (c & 1) (8 / W) + u % (8 / W) of word c >> 1 of half-slot u / (8 / W).
template <int W>
__device__ __forceinline__ uint32_t plane_pair64(const uint8_t* cb, int u, int c) {
  constexpr int P = 8 / W;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(cb + 512 * (u / P) + 4 * (c >> 1));
  return (w >> (W * ((c & 1) * P + u % P))) & (((1u << W) - 1u) * 0x00010001u);
}

template <int W0, int W1>
__device__ void unpack_block64(const UnpackArgs& a, int blk, int lane) {
  const int br = blk / a.nbc, bc = blk % a.nbc;
  const uint8_t* cb = a.codes + size_t(a.offs[blk]) * 512 + 8 * lane;
  for (int u = 0; u < 8; ++u) {
    const int kt = u >> 2, rt = u & 3;
    const int row = br * 64 + 16 * rt + (lane & 15);
    const uint32_t e = a.sz[size_t(blk) * 64 + 4 * (lane & 15) + rt];
    const float s = lo_half(e), z = hi_half(e);
    for (int c = 0; c < 4; ++c) {
      uint32_t pr = plane_pair64<W0>(cb, u, c);
      if constexpr (W1 != 0) pr |= plane_pair64<W1>(cb + 512 * W0, u, c) << W0;
      const int col = bc * 64 + 32 * kt + 8 * (lane >> 4) + 2 * c;
      const uint32_t qa = pr & 0xffffu, qb = pr >> 16;
      const size_t o = size_t(row) * a.K + col;
      if (a.q) a.q[o] = uint8_t(qa), a.q[o + 1] = uint8_t(qb);
      const float va = (float(qa) - z) * s, vb = (float(qb) - z) * s;
      if (a.w32) a.w32[o] = va, a.w32[o + 1] = vb;
      if (a.w16) a.w16[o] = (_Float16)va, a.w16[o + 1] = (_Float16)vb;
    }
  }
}

__global__ __launch_bounds__(256) void unpack64_kernel(UnpackArgs a) {
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blk >= a.nbr * a.nbc) return;
  switch (a.bits[blk]) {
    case 1: unpack_block64<1, 0>(a, blk, lane); break;
    case 2: unpack_block64<2, 0>(a, blk, lane); break;
    case 3: unpack_block64<2, 1>(a, blk, lane); break;
    case 4: unpack_block64<4, 0>(a, blk, lane); break;
    case 6: unpack_block64<4, 2>(a, blk, lane); break;
    default: unpack_block64<4, 4>(a, blk, lane); break;
  }
}

}  // namespace

int launch_unpack(const BlockImageView& im, uint8_t* q, float* w32, uint16_t* w16, void* stream) {
  UnpackArgs a;
  a.bits = im.bits;
  a.offs = im.offs;
  a.sz = im.sz;
  a.codes = im.codes;
  a.q = q;
  a.w32 = w32;
  a.w16 = reinterpret_cast<_Float16*>(w16);
  a.N = im.N;
  a.K = im.K;
  a.nbr = im.nbr;
  a.nbc = im.nbc;
  const int nblk = im.nbr * im.nbc;
  if (im.bc == 64)
    hipLaunchKernelGGL(unpack64_kernel, dim3(unsigned((nblk + 3) / 4)), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(unpack_kernel, dim3(unsigned((nblk + 3) / 4)), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return int(hipGetLastError());
}

}  // namespace gbb
