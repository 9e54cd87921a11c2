// Fused per-centre attention kernels (block_attn_fused.hip).
#pragma once

#include "nga_internal.h"

namespace nga {

// True if a fused kernel covers these shapes.
bool fused_supported(int dtype, int32_t nnei_cap, int32_t c, int32_t heads);
const char* fused_name(int dtype, int32_t c, int32_t heads);
// Workspace floats the fused path needs (weights repacked in operand order).
size_t fused_workspace_floats(int32_t c, int32_t layers);
// log_dtilde: NULL, or ln D~ [layers][n_edges][heads] for smooth attention.
int run_fused(int dtype, const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
              int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
              const void* weights, const void* x, const void* log_dtilde, void* y, void* packed,
              uint32_t* status, hipStream_t s);

}  // namespace nga
