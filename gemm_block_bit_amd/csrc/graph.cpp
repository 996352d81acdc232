// Whole-layer execution: a sequence of block-GEMM calls captured into one
// HIP graph and replayed with a single launch.  Host code only.
#include <hip/hip_runtime.h>

#include <new>

#include "internal.h"

struct gbb_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

gbb_status hip_fail(hipError_t err, const char* what) {
  return gbb::fail(GBB_E_DEVICE, "%s: HIP error %d (%s)", what, int(err), hipGetErrorString(err));
}

}  // namespace

extern "C" gbb_status gbb_graph_create(int n, const void* const* images, const int* N, const int* K,
                                       const uint16_t* const* x, uint16_t* const* y, int M, void* workspace,
                                       size_t ws_bytes, gbb_graph** out) {
  if (!out) return gbb::fail(GBB_E_ARG, "out is NULL");
  *out = nullptr;
  if (n < 1) return gbb::fail(GBB_E_ARG, "n must be at least 1 (n=%d)", n);
  if (M < 1) return gbb::fail(GBB_E_ARG, "M must be at least 1 (M=%d)", M);
  if (!images || !N || !K || !x || !y) return gbb::fail(GBB_E_ARG, "images, N, K, x and y must not be NULL");

  hipStream_t s = nullptr;
  hipError_t err = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (err != hipSuccess) return hip_fail(err, "stream creation");
  err = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
  if (err != hipSuccess) {
    (void)hipStreamDestroy(s);
    return hip_fail(err, "begin capture");
  }
  gbb_status st = GBB_OK;
  for (int i = 0; i < n && st == GBB_OK; ++i)
    st = gbb_gemm_mixed_w(images[i], N[i], K[i], x[i], y[i], M, workspace, ws_bytes, s);
  hipGraph_t graph = nullptr;
  err = hipStreamEndCapture(s, &graph);
  (void)hipStreamDestroy(s);
  if (st != GBB_OK) {   // keep the failing call's message
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (err != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return hip_fail(err, "end capture");
  }
  hipGraphExec_t exec = nullptr;
  err = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (err != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return hip_fail(err, "graph instantiation");
  }
  gbb_graph* g = new (std::nothrow) gbb_graph{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return gbb::fail(GBB_E_ARG, "out of host memory");
  }
  *out = g;
  return GBB_OK;
}

extern "C" gbb_status gbb_graph_launch(const gbb_graph* g, void* stream) {
  if (!g) return gbb::fail(GBB_E_ARG, "graph is NULL");
  const hipError_t err = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GBB_OK : hip_fail(err, "graph launch");
}

extern "C" gbb_status gbb_graph_destroy(gbb_graph* g) {
  if (!g) return GBB_OK;
  const hipError_t e1 = hipGraphExecDestroy(g->exec);
  const hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  if (e1 != hipSuccess) return hip_fail(e1, "graph destruction");
  if (e2 != hipSuccess) return hip_fail(e2, "graph destruction");
  return GBB_OK;
}
