// graph.cpp -- native HIP graphs of library calls (declared in include/pa.h):
// capture the calls issued on a stream, instantiate once, replay per step.
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "pa.h"

struct pa_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

namespace {

// A failed runtime call also sets the thread's last-error state, which the
// caller's next error check (hipGetLastError after its own launch) would report;
// the status code returned here is the error report, so that state is cleared.
int fail()
{
    (void)hipGetLastError();
    return PA_ERR_GRAPH;
}

}  // namespace

extern "C" {

int pa_graph_begin(hipStream_t stream)
{
    if (!stream)
        return PA_ERR_NULL;
    return hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) == hipSuccess ? PA_OK
                                                                                         : fail();
}

int pa_graph_end(hipStream_t stream, pa_graph **out)
{
    if (!stream)
        return PA_ERR_NULL;
    if (out)
        *out = nullptr;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess || st == hipStreamCaptureStatusNone)
        return fail();   // nothing to end
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(stream, &g);
    if (!out) {
        if (g)
            (void)hipGraphDestroy(g);
        return PA_ERR_NULL;
    }
    if (e != hipSuccess || !g) {
        if (g)
            (void)hipGraphDestroy(g);
        return fail();
    }
    hipGraphExec_t x = nullptr;
    if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess || !x) {
        (void)hipGraphDestroy(g);
        return fail();
    }
    pa_graph *p = new (std::nothrow) pa_graph{g, x};
    if (!p) {
        (void)hipGraphExecDestroy(x);
        (void)hipGraphDestroy(g);
        return fail();
    }
    *out = p;
    return PA_OK;
}

int pa_graph_launch(const pa_graph *graph, hipStream_t stream)
{
    if (!graph || !stream)
        return PA_ERR_NULL;
    return hipGraphLaunch(graph->exec, stream) == hipSuccess ? PA_OK : fail();
}

int pa_graph_node_counts(const pa_graph *graph, size_t *kernels, size_t *others)
{
    if (!graph || !kernels || !others)
        return PA_ERR_NULL;
    size_t n = 0;
    if (hipGraphGetNodes(graph->graph, nullptr, &n) != hipSuccess)
        return fail();
    std::vector<hipGraphNode_t> nodes(n);
    if (n && hipGraphGetNodes(graph->graph, nodes.data(), &n) != hipSuccess)
        return fail();
    size_t k = 0;
    for (size_t i = 0; i < n; ++i) {
        hipGraphNodeType t;
        if (hipGraphNodeGetType(nodes[i], &t) != hipSuccess)
            return fail();
        k += t == hipGraphNodeTypeKernel;
    }
    *kernels = k;
    *others = n - k;
    return PA_OK;
}

void pa_graph_destroy(pa_graph *graph)
{
    if (!graph)
        return;
    (void)hipGraphExecDestroy(graph->exec);
    (void)hipGraphDestroy(graph->graph);
    delete graph;
}

}  // extern "C"
