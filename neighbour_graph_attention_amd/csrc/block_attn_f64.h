// fp64 block attention on matrix cores (block_attn_f64.hip).
#pragma once

#include "nga_internal.h"

namespace nga {

// True if the fp64 matrix-core path covers these shapes (head width 8, 16 or 32, rows <= 128).
bool f64_mfma_supported(int32_t nnei_cap, int32_t c, int32_t heads);

// log_dtilde: NULL, or ln D~ [layers][n_edges][heads] for smooth attention.
// Stacked layers through slot-indexed workspace buffers qkv [E][3c], o [E][c] and, for more
// than one layer, xbuf [E][c].
int run_f64_mfma(const int64_t* row_ptr, const int32_t* order, int64_t n_centres, int64_t n_edges,
                 int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers, const double* weights,
                 const double* x, const double* log_dtilde, double* y, double* qkv, double* o,
                 double* xbuf, uint32_t* status, hipStream_t s);

// True if the fused fp64 kernel covers these shapes (c <= 32, head width 8 or 16, rows <= 64).
bool fused_f64_supported(int32_t nnei_cap, int32_t c, int32_t heads);

// Whole layer stack in one launch, one work-group per centre; needs only the status word.
int run_fused_f64(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                  int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
                  const double* weights, const double* x, const double* log_dtilde, double* y,
                  uint32_t* status, hipStream_t s);

}  // namespace nga
