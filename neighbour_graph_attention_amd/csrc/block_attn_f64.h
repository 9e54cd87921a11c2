// fp64 block attention on matrix cores (block_attn_f64.hip).
#pragma once

#include "nga_internal.h"

namespace nga {

constexpr double kLn2F64 = 0.69314718055994530942;
constexpr double kLog2eF64 = 1.44269504088896340736;

// k-th Taylor coefficient of 2^f = e^(f ln 2): (ln 2)^k / k!.
constexpr double exp2_taylor(int k) {
    double c = 1.0;
    for (int i = 1; i <= k; ++i) c = c * kLn2F64 / i;
    return c;
}

// 2^y for the softmax exponents y = (s - max s) log2(e) / sqrt(d) <= 0, finite or NaN (-inf
// gives NaN: callers pass masked keys as -4096, whose 2^y is 0).  y = n + f with n = rint(y), |f| <= 1/2; 2^f from its
// Taylor series to degree 12 (the remainder is below 3e-16 of 2^f for |f ln 2| <= 0.347), times
// 2^n by ldexp, which gives 0 once n is below the subnormal range (n is clamped to -2000 before
// the integer conversion).  NaN propagates through f.  Against a correctly rounded 2^y the
// relative error is a few units in the last place.  Unlike the general exp it needs no range
// checks: 17 instructions instead of about 25.
__device__ inline double exp2_nonpos(double y) {
    const double n = __builtin_rint(y);
    const double f = y - n;
    double p = exp2_taylor(12);
#pragma unroll
    for (int k = 11; k >= 0; --k) p = __builtin_fma(p, f, exp2_taylor(k));
    return __builtin_ldexp(p, (int)__builtin_fmax(n, -2000.0));
}

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
