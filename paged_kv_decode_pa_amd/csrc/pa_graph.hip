// Capture of the layer step (pa_step) into a HIP graph for replay.
#include <new>

#include <hip/hip_runtime.h>

#include "../../include/pa.h"

struct pa_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" {

int pa_step_graph_create(const pa_step_args* a, void* stream, pa_step_graph** out) {
  return pa_step_graph_create_n(a, 1, stream, out);
}

int pa_step_graph_create_n(const pa_step_args* a, int num_steps, void* stream,
                           pa_step_graph** out) {
  if (!a || num_steps < 1 || !out || !stream) return PA_EINVAL;  // capture needs a created stream
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return PA_ELAUNCH;
  int st = PA_OK;
  for (int i = 0; i < num_steps && st == PA_OK; ++i) st = pa_step(a + i, stream);
  hipGraph_t graph = nullptr;
  const hipError_t end = hipStreamEndCapture(s, &graph);
  if (st != PA_OK || end != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return st != PA_OK ? st : PA_ELAUNCH;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return PA_ELAUNCH;
  }
  // move the executable graph's resources to the device now, so the first
  // replay does not pay for it
  if (hipGraphUpload(exec, s) != hipSuccess) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return PA_ELAUNCH;
  }
  pa_step_graph* g = new (std::nothrow) pa_step_graph{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return PA_ELAUNCH;
  }
  *out = g;
  return PA_OK;
}

int pa_step_graph_launch(pa_step_graph* g, void* stream) {
  if (!g) return PA_EINVAL;
  return hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK
                                                                                 : PA_ELAUNCH;
}

int pa_step_graph_destroy(pa_step_graph* g) {
  if (!g) return PA_OK;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
  return PA_OK;
}

}  // extern "C"
