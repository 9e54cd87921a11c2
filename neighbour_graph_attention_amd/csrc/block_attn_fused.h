// Fused per-centre attention kernels for fp32 features with 16-wide heads:
// block_attn_f32.hip (fp32 matrix cores, what NGA_F32 runs) and block_attn_fused.hip (f16
// matrix cores on hi/lo split pairs, what NGA_F32_SPLIT16 runs).
#pragma once

#include "nga_internal.h"

namespace nga {

// fp32 on v_mfma_f32_16x16x4_f32 (block_attn_f32.hip): 1, 2 or 4 heads of 16, rows <= 192.
bool f32_fused_supported(int32_t nnei_cap, int32_t c, int32_t heads);
// Workspace floats: the weights repacked in operand order.
size_t f32_fused_workspace_floats(int32_t c, int32_t layers);
// log_dtilde: NULL, or ln D~ [layers][n_edges][heads] for smooth attention.
int run_f32_fused(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                  int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
                  const float* weights, const float* x, const float* log_dtilde, float* y,
                  float* packed, uint32_t* status, hipStream_t s);

// f16 hi/lo split pairs on v_mfma_f32_16x16x32_f16 (block_attn_fused.hip), the same shapes.
bool fused_supported(int dtype, int32_t nnei_cap, int32_t c, int32_t heads);
const char* fused_name(int dtype, int32_t c, int32_t heads);
// Workspace floats the split path needs (weights repacked as split pairs, their exponents).
size_t fused_workspace_floats(int32_t c, int32_t layers);
int run_fused(int dtype, const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
              int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
              const void* weights, const void* x, const void* log_dtilde, void* y, void* packed,
              uint32_t* status, hipStream_t s);

}  // namespace nga
