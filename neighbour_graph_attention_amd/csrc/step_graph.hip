// One step of the hot path -- nl_build, edge_csr (no readback), block_attn_forward -- captured
// once as a HIP graph and replayed with a single launch.
//
// deepmd-kit issue "perf: DPA4 .pt2 LAMMPS (C++ AOTI) inference 3-6x slower than Python (ASE)
// due to CPU-side edge construction and data marshalling", section "Proposed optimizations":
// capture the inference step in a graph to remove the per-kernel launch overhead.  The step's
// kernels take every buffer by pointer and none of the three calls synchronises, copies or sets
// memory when edge_csr's readback is off, so the whole step captures as kernel nodes only.
// Replays read the positions, features and weights the pointers name at replay time and write
// the same outputs; the caller changes inputs in place between replays.  The box and the other
// scalars are taken at capture.
#include "nga_internal.h"

#include <new>

namespace {

struct StepGraph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

}  // namespace

extern "C" int nga_step_graph_create(
    const double* pos, int64_t n_atoms, const double* h_box, double rcut, int32_t sel,
    int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* ws_nl, size_t ws_nl_bytes,
    int64_t* row_ptr, int32_t* col, int32_t* shift, int32_t* dst, double* edge_vec,
    int64_t e_cap, void* ws_csr, size_t ws_csr_bytes, int dtype, int32_t c, int32_t n_heads,
    int32_t n_layers, const void* weights, const void* x, void* y, void* ws_attn,
    size_t ws_attn_bytes, void** graph_out) {
    using namespace nga;
    if (!graph_out) return NGA_EINVAL;
    *graph_out = nullptr;
    hipStream_t cs;
    int rc = hip_status(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    if (rc) return rc;
    rc = hip_status(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
    if (rc) {
        hipStreamDestroy(cs);
        return rc;
    }
    rc = nl_build(pos, n_atoms, h_box, rcut, sel, nbr, nbr_shift, nnei, ws_nl, ws_nl_bytes, cs);
    if (rc == NGA_OK)
        rc = edge_csr(nbr, nbr_shift, nnei, n_atoms, sel, pos, h_box, row_ptr, col, shift, dst,
                      edge_vec, e_cap, nullptr, ws_csr, ws_csr_bytes, cs);
    if (rc == NGA_OK)
        rc = block_attn_forward(dtype, row_ptr, nullptr, n_atoms, e_cap, sel, c, n_heads,
                                n_layers, weights, x, y, ws_attn, ws_attn_bytes, cs);
    hipGraph_t graph = nullptr;
    const int rc_end = hip_status(hipStreamEndCapture(cs, &graph));
    hipStreamDestroy(cs);
    if (rc == NGA_OK) rc = rc_end;
    if (rc != NGA_OK) {
        if (graph) hipGraphDestroy(graph);
        return rc;
    }
    hipGraphExec_t exec = nullptr;
    rc = hip_status(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    if (rc) {
        hipGraphDestroy(graph);
        return rc;
    }
    StepGraph* g = new (std::nothrow) StepGraph{graph, exec};
    if (!g) {
        hipGraphExecDestroy(exec);
        hipGraphDestroy(graph);
        return NGA_EHIP;
    }
    *graph_out = g;
    return NGA_OK;
}

extern "C" int nga_step_graph_launch(void* graph, void* stream) {
    if (!graph) return NGA_EINVAL;
    StepGraph* g = static_cast<StepGraph*>(graph);
    return nga::hip_status(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
}

extern "C" int nga_step_graph_destroy(void* graph) {
    if (!graph) return NGA_OK;
    StepGraph* g = static_cast<StepGraph*>(graph);
    int rc = nga::hip_status(hipGraphExecDestroy(g->exec));
    const int rc2 = nga::hip_status(hipGraphDestroy(g->graph));
    delete g;
    return rc ? rc : rc2;
}
