// Row-gather / row-scatter GEMM on the vector ALUs, for any channel count and either
// precision: out[out_rows(m)][u] = sum_{t < k} a[a_rows(m)][t] * W_{u / c}[t][u % c], with nmat
// matrices W of [k][c] side by side in the output columns (k = c unless set).  Used by the
// generic attention path, the pair-axis route and LocalAtten.
#pragma once

#include "nga_internal.h"

namespace nga {
namespace {

constexpr int kGemmBM = 64, kGemmBN = 64, kGemmBK = 16;

template <typename T>
struct GemmArgs {
    const T* a;
    const int32_t* a_rows;  // nullable: row m of A is a[a_rows[m]]
    const T* w;             // nmat matrices [c][c] side by side in the output columns
    T* out;
    const int32_t* out_rows;  // nullable: row m of the result goes to out[out_rows[m]]
    const int64_t* e_dev;     // rows m < *e_dev are computed (NULL: all n_edges rows)
    int64_t n_edges;          // bound on the rows and on gathered / scattered row indices
    int c;                    // output columns per matrix
    int nmat;
    int k = 0;                // reduction length (0: c)
    int lda;
    int ldo;
    uint32_t* status;
};

// out[m][u] = sum_t A[m][t] * W_{u / c}[t][u % c], 64x64 tiles, 4x4 per thread.
template <typename T>
__global__ void __launch_bounds__(256) gemm_rows_kernel(GemmArgs<T> g) {
    __shared__ T sa[kGemmBK][kGemmBM + 1];
    __shared__ T sw[kGemmBK][kGemmBN + 1];
    const int64_t E = g.e_dev ? (*g.e_dev < g.n_edges ? *g.e_dev : g.n_edges) : g.n_edges;
    const int K = g.k > 0 ? g.k : g.c;
    const int64_t m0 = (int64_t)blockIdx.x * kGemmBM;
    const int u0 = blockIdx.y * kGemmBN;
    if (m0 >= E) return;
    const int nout = g.nmat * g.c;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    T acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = T(0);
    for (int k0 = 0; k0 < K; k0 += kGemmBK) {
        for (int idx = threadIdx.x; idx < kGemmBM * kGemmBK; idx += 256) {
            int r = idx / kGemmBK, kk = idx % kGemmBK;
            int64_t m = m0 + r;
            T v = T(0);
            if (m < E && k0 + kk < K) {
                int64_t row = g.a_rows ? (int64_t)g.a_rows[m] : m;
                if (row >= 0 && row < g.n_edges) v = g.a[row * g.lda + k0 + kk];
            }
            sa[kk][r] = v;
        }
        for (int idx = threadIdx.x; idx < kGemmBK * kGemmBN; idx += 256) {
            int kk = idx / kGemmBN, cc = idx % kGemmBN;
            int u = u0 + cc, t = k0 + kk;
            T v = T(0);
            if (u < nout && t < K) {
                int mat = u / g.c, col = u % g.c;
                v = g.w[((int64_t)mat * K + t) * g.c + col];
            }
            sw[kk][cc] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGemmBK; ++kk) {
            T av[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = sa[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = sw[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * wv[j];
        }
        __syncthreads();
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t m = m0 + ty * 4 + i;
        if (m >= E) continue;
        int64_t row = m;
        if (g.a_rows) {
            int64_t ar = g.a_rows[m];
            if (ar < 0 || ar >= g.n_edges) bad = true;
        }
        if (g.out_rows) {
            row = g.out_rows[m];
            if (row < 0 || row >= g.n_edges) { bad = true; continue; }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int u = u0 + tx * 4 + j;
            if (u < nout) g.out[row * g.ldo + u] = acc[i][j];
        }
    }
    if (bad) raise_bits(g.status, kBitIndex);
}

template <typename T>
int launch_gemm(const GemmArgs<T>& g, int64_t m_bound, hipStream_t s) {
    const int nout = g.nmat * g.c;
    dim3 grid((unsigned)((m_bound + kGemmBM - 1) / kGemmBM), (unsigned)((nout + kGemmBN - 1) / kGemmBN));
    hipLaunchKernelGGL((gemm_rows_kernel<T>), grid, dim3(256), 0, s, g);
    return last_launch_status();
}

}  // namespace
}  // namespace nga
