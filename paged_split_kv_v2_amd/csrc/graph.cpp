// Step graphs: the kernel launches of one decode step (a planned cascade
// run, a chunked MLA run, a flat decode) recorded once by HIP stream capture
// and replayed with one graph launch, so that a decode loop pays one host
// call per step instead of one per kernel and the kernels follow each other
// without host round trips.
//
// The run entry points only launch kernels on the caller's stream (plans are
// uploaded, workspaces sized and outputs allocated beforehand), so a capture
// of them records kernel nodes alone; pdk_graph_nodes reports the node kinds
// so that a caller can check this.

#include <hip/hip_runtime.h>

#include <vector>

#include "internal.h"
#include "pdk.h"

struct pdk_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

using namespace pdk;

extern "C" {

int pdk_graph_begin(hipStream_t stream) {
  if (stream == nullptr) return fail(PDK_ERR_ARG, "capture needs a stream other than the null stream");
  hipError_t e = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(PDK_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
  return PDK_OK;
}

int pdk_graph_end(hipStream_t stream, pdk_graph** out) {
  if (stream == nullptr) return fail(PDK_ERR_ARG, "capture needs a stream other than the null stream");
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(stream, &g);  // ends the capture in every case
  if (e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return fail(PDK_ERR_HIP, "end capture: %s", hipGetErrorString(e));
  }
  if (!out) {
    (void)hipGraphDestroy(g);
    return fail(PDK_ERR_ARG, "NULL graph out");
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(PDK_ERR_HIP, "instantiate: %s", hipGetErrorString(e));
  }
  *out = new pdk_graph{g, x};
  return PDK_OK;
}

int pdk_graph_launch(const pdk_graph* g, hipStream_t stream) {
  if (!g || !g->exec) return fail(PDK_ERR_ARG, "NULL graph");
  hipError_t e = hipGraphLaunch(g->exec, stream);
  if (e != hipSuccess) return fail(PDK_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
  return PDK_OK;
}

int pdk_graph_nodes(const pdk_graph* g, int32_t* kernel_nodes, int32_t* other_nodes) {
  if (!g || !g->graph || !kernel_nodes || !other_nodes) return fail(PDK_ERR_ARG, "NULL argument");
  size_t n = 0;
  hipError_t e = hipGraphGetNodes(g->graph, nullptr, &n);
  if (e != hipSuccess) return fail(PDK_ERR_HIP, "graph nodes: %s", hipGetErrorString(e));
  std::vector<hipGraphNode_t> nodes(n);
  if (n > 0 && (e = hipGraphGetNodes(g->graph, nodes.data(), &n)) != hipSuccess)
    return fail(PDK_ERR_HIP, "graph nodes: %s", hipGetErrorString(e));
  int32_t k = 0, o = 0;
  for (size_t i = 0; i < n; ++i) {
    hipGraphNodeType t;
    if ((e = hipGraphNodeGetType(nodes[i], &t)) != hipSuccess)
      return fail(PDK_ERR_HIP, "node type: %s", hipGetErrorString(e));
    (t == hipGraphNodeTypeKernel ? k : o) += 1;
  }
  *kernel_nodes = k;
  *other_nodes = o;
  return PDK_OK;
}

void pdk_graph_free(pdk_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
