// Allocation-free block GEMM: gbb_gemm_mixed_w with its split-K workspace in
// a fixed array of device memory that the library owns, for callers that
// cannot allocate (code under graph capture, tight serving loops).
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, from the first call on that GPU
// until the process ends.  In host code the array's name is not a device
// address, so its address is looked up once per device with
// hipGetSymbolAddress and only that pointer is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = GBB_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 16-byte words");

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Zero-fill of the array (a kernel, not a memset, so that a call recorded
// into a graph replays it correctly).
__global__ __launch_bounds__(256) void clear_scratch_kernel(uint4* __restrict__ p, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;    // device address of `scratch` on that device
  bool cleared = false;   // a zero-fill has been issued outside stream capture
};
std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

gbb_status hip_fail(hipError_t err, const char* what) {
  return gbb::fail(GBB_E_DEVICE, "%s: HIP error %d (%s)", what, int(err), hipGetErrorString(err));
}

// The current device's scratch address.  Set-up happens once per device, on
// the first call with that device current: the symbol's address is looked up
// (and the return code checked), then the array is zero-filled on `stream`
// before the call's kernels, since the split-K hand-off expects zero
// accumulators.  Every call leaves them zero again.  A fill issued while
// `stream` is being captured only runs when the graph does, so set-up is
// repeated by the next call until one fill has been issued outside capture.
gbb_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return gbb::fail(GBB_E_DEVICE, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_fail(err, "hipGetSymbolAddress(scratch)");
    if (!p) return gbb::fail(GBB_E_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    d.ptr = p;
  }
  if (!d.cleared) {
    hipLaunchKernelGGL(clear_scratch_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(d.ptr),
                       kScratchBytes / 16);
    err = hipGetLastError();
    if (err != hipSuccess) return hip_fail(err, "scratch clear launch");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusActive;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) d.cleared = true;
  }
  *out = d.ptr;
  return GBB_OK;
}

}  // namespace

extern "C" gbb_status gbb_gemm_mixed_w_noalloc(const void* image, int N, int K, const uint16_t* x, uint16_t* y,
                                               int M, void* stream) {
  gbb_status st = gbb::check_gemm_args(image, N, K, x, y, M, 0);
  if (st != GBB_OK || M == 0) return st;
  // the prefill route's K split takes as many segments as the array holds
  const size_t need = gbb::required_workspace(N, K, M);
  if (need > kScratchBytes)
    return gbb::fail(GBB_E_SPACE, "N=%d K=%d M=%d needs %zu bytes of split-K workspace, above the %zu bytes of "
                     "the allocation-free entry point (use gbb_gemm_mixed_w with a workspace)",
                     N, K, M, need, kScratchBytes);
  void* ws = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = scratch_for(s, &ws);
  if (st != GBB_OK) return st;
  return gbb_gemm_mixed_w(image, N, K, x, y, M, ws, kScratchBytes, stream);
}
