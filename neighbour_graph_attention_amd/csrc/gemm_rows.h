// Row-gather / row-scatter GEMM on the vector ALUs, for any channel count and either
// precision: out[out_rows(m)][u] = sum_{t < k} a[a_rows(m)][t] * W_{u / c}[t][u % c], with nmat
// matrices W of [k][c] side by side in the output columns (k = c unless set).  Used by the
// generic attention path, the pair-axis route and LocalAtten.  In fp32, without row gather or
// scatter, the product runs on the matrix cores instead (gemm_f32_mfma_kernel).
#pragma once

#include <type_traits>

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

// The fp32 product on the matrix cores, for the plain case (no row gather or scatter, no
// device-side row bound): a 64-row x 64-column output tile per work-group, 16 rows per
// wavefront as four 16x16 tiles of v_mfma_f32_16x16x4f32 (fp32 products, fp32 sums: the
// arithmetic of the vector kernel up to summation order).  The work-group's 64 columns of
// W' (W' = [W_0 | W_1 | ..], K x nmat c) sit in LDS transposed, k contiguous, so that a lane's
// four k values of one column are one 16-byte read; a lane's four k values of its A row are
// one 16-byte global load.  In MFMA step s, the k slot q of the 16x16x4 operation (lanes
// 16 q .. 16 q + 15) carries k = k0 + 4 q + s on both operands.
constexpr int kMfmaBM = 64, kMfmaBN = 64;

template <int KT>  // K = 16 KT
__global__ void __launch_bounds__(256) gemm_f32_mfma_kernel(GemmArgs<float> g, int64_t M) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int K = 16 * KT, LDW = K + 4;
    __shared__ __align__(16) float sWt[kMfmaBN * LDW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.y * kMfmaBN;
    const int64_t m0 = (int64_t)blockIdx.x * kMfmaBM;
    const int j = lane & 15, q = lane >> 4;
    // A: row m0 + 16 wave + j, k = 16 kk + 4 q .. + 3 for kk < KT; loads first, then staging
    const int64_t row = m0 + wave * 16 + j;
    const bool live = row < M;
    const f4* arow = reinterpret_cast<const f4*>(g.a + (live ? row : m0) * g.lda);
    f4 av[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) av[kk] = live ? arow[4 * kk + q] : f4{0.f, 0.f, 0.f, 0.f};
    // W': thread (column cc, k group k4) reads W'[4 k4 .. 4 k4 + 3][n0 + cc], coalesced over cc
    for (int idx = tid; idx < K / 4 * kMfmaBN; idx += 256) {
        const int cc = idx % kMfmaBN, k4 = idx / kMfmaBN;
        const int u = n0 + cc, mat = u / g.c, col = u - mat * g.c;
        const float* w = g.w + ((int64_t)mat * K + 4 * k4) * g.c + col;
        f4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = w[e * g.c];
        *reinterpret_cast<f4*>(&sWt[cc * LDW + 4 * k4]) = v;
    }
    __syncthreads();
    f4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
        f4 bv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bv[t] = *reinterpret_cast<const f4*>(&sWt[(16 * t + j) * LDW + 16 * kk + 4 * q]);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[kk][st], bv[t][st], acc[t], 0, 0, 0);
    }
    // D[i][jj] of tile t sits in lane jj + 16 (i / 4), register i % 4
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wave * 16 + 4 * q + r;
        if (m < M) {
            float* o = g.out + m * g.ldo + n0 + j;
#pragma unroll
            for (int t = 0; t < 4; ++t) o[16 * t] = acc[t][r];
        }
    }
}

// Work-groups of `threads` threads that the device holds at once for `kernel`.
inline int64_t resident_groups(const void* kernel, int threads) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return (int64_t)per_cu * cus;
}

// The same product when all of W' fits in LDS (K x N <= 16384 floats): a persistent
// work-group stages W' once, transposed as above, and takes 64-row blocks b, b + G, ...,
// each wavefront 16 rows x all N columns (NT 16x16 tiles); the next block's A fragments are
// loaded while the current block's products run.
template <int KT, int NT>  // K = 16 KT, N = 16 NT
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
gemm_f32_mfma_full_kernel(GemmArgs<float> g, int64_t M) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int K = 16 * KT, N = 16 * NT, LDW = K + 4;
    __shared__ __align__(16) float sWt[N * LDW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, q = lane >> 4;
    const int64_t nblk = (M + kMfmaBM - 1) / kMfmaBM;
    auto load_a = [&](f4 (&av)[KT], int64_t blk) {
        const int64_t row = blk * kMfmaBM + wave * 16 + j;
        const bool live = row < M;
        const f4* arow = reinterpret_cast<const f4*>(g.a + (live ? row : 0) * g.lda);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) av[kk] = live ? arow[4 * kk + q] : f4{0.f, 0.f, 0.f, 0.f};
    };
    int64_t b = blockIdx.x;
    f4 av[KT], an[KT];
    load_a(av, b);
    for (int idx = tid; idx < K / 4 * N; idx += 256) {
        const int cc = idx % N, k4 = idx / N;
        const int mat = cc / g.c, col = cc - mat * g.c;
        const float* w = g.w + ((int64_t)mat * K + 4 * k4) * g.c + col;
        f4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = w[e * g.c];
        *reinterpret_cast<f4*>(&sWt[cc * LDW + 4 * k4]) = v;
    }
    __syncthreads();
    for (; b < nblk; b += gridDim.x) {
        if (b + gridDim.x < nblk) load_a(an, b + gridDim.x);
        f4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            f4 bv[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                bv[t] = *reinterpret_cast<const f4*>(&sWt[(16 * t + j) * LDW + 16 * kk + 4 * q]);
            // NT independent accumulation chains per k slot
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[kk][st], bv[t][st], acc[t], 0, 0, 0);
            // keep each k step's W' reads next to its products (registers, not latency, bound
            // how many can be in flight)
            __builtin_amdgcn_sched_barrier(0);
        }
        // D[i][jj] of tile t sits in lane jj + 16 (i / 4), register i % 4
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = b * kMfmaBM + wave * 16 + 4 * q + r;
            if (m < M) {
                float* o = g.out + m * g.ldo + j;
#pragma unroll
                for (int t = 0; t < NT; ++t) o[16 * t] = acc[t][r];
            }
        }
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) av[kk] = an[kk];
    }
}

template <int KT, int NT>
void launch_mfma_full(const GemmArgs<float>& g, int64_t M, hipStream_t s) {
    const void* k = reinterpret_cast<const void*>(&gemm_f32_mfma_full_kernel<KT, NT>);
    const int64_t nblk = (M + kMfmaBM - 1) / kMfmaBM;
    const int64_t res = resident_groups(k, 256);
    const dim3 grid((unsigned)(nblk < res ? nblk : res));
    hipLaunchKernelGGL((gemm_f32_mfma_full_kernel<KT, NT>), grid, dim3(256), 0, s, g, M);
}

// gemm_f32_mfma_full_kernel for this product, if an instance covers it; false otherwise.
inline bool try_mfma_full(const GemmArgs<float>& g, int kt, int64_t M, hipStream_t s) {
    const int nt = g.nmat * g.c / 16;
    switch (kt * 100 + nt) {
        case 104: launch_mfma_full<1, 4>(g, M, s); return true;
        case 108: launch_mfma_full<1, 8>(g, M, s); return true;
        case 116: launch_mfma_full<1, 16>(g, M, s); return true;
        case 204: launch_mfma_full<2, 4>(g, M, s); return true;
        case 208: launch_mfma_full<2, 8>(g, M, s); return true;
        case 216: launch_mfma_full<2, 16>(g, M, s); return true;
        case 404: launch_mfma_full<4, 4>(g, M, s); return true;
        case 408: launch_mfma_full<4, 8>(g, M, s); return true;
        case 416: launch_mfma_full<4, 16>(g, M, s); return true;
        case 804: launch_mfma_full<8, 4>(g, M, s); return true;
        case 808: launch_mfma_full<8, 8>(g, M, s); return true;
        case 1604: launch_mfma_full<16, 4>(g, M, s); return true;
        default: return false;
    }
}

// Whether gemm_f32_mfma_kernel covers this product; its K (= 16 KT) as KT, else 0.
inline int mfma_gemm_kt(const GemmArgs<float>& g) {
    const int K = g.k > 0 ? g.k : g.c;
    const int nout = g.nmat * g.c;
    if (g.a_rows || g.out_rows || g.e_dev) return 0;
    if (g.c % 16 != 0 || nout % kMfmaBN != 0 || g.lda % 4 != 0 || g.lda < K || g.ldo < nout)
        return 0;
    if ((reinterpret_cast<uintptr_t>(g.a) & 15) != 0) return 0;
    if (K != 16 && K != 32 && K != 64 && K != 128 && K != 256) return 0;
    return K / 16;
}

template <int KT>
void launch_mfma_gemm(const GemmArgs<float>& g, int64_t m_bound, hipStream_t s) {
    const int64_t M = m_bound < g.n_edges ? m_bound : g.n_edges;
    const dim3 grid((unsigned)((M + kMfmaBM - 1) / kMfmaBM), (unsigned)(g.nmat * g.c / kMfmaBN));
    hipLaunchKernelGGL((gemm_f32_mfma_kernel<KT>), grid, dim3(256), 0, s, g, M);
}

template <typename T>
int launch_gemm(const GemmArgs<T>& g, int64_t m_bound, hipStream_t s) {
    if constexpr (std::is_same<T, float>::value) {
        if (m_bound > 0 && g.n_edges > 0 && (m_bound + kMfmaBM - 1) / kMfmaBM < 2147483647) {
            const int kt = mfma_gemm_kt(g);
            if (kt > 0 && try_mfma_full(g, kt, m_bound < g.n_edges ? m_bound : g.n_edges, s))
                return last_launch_status();
            switch (kt) {
                case 1: launch_mfma_gemm<1>(g, m_bound, s); return last_launch_status();
                case 2: launch_mfma_gemm<2>(g, m_bound, s); return last_launch_status();
                case 4: launch_mfma_gemm<4>(g, m_bound, s); return last_launch_status();
                case 8: launch_mfma_gemm<8>(g, m_bound, s); return last_launch_status();
                case 16: launch_mfma_gemm<16>(g, m_bound, s); return last_launch_status();
                default: break;
            }
        }
    }
    const int nout = g.nmat * g.c;
    dim3 grid((unsigned)((m_bound + kGemmBM - 1) / kGemmBM), (unsigned)((nout + kGemmBN - 1) / kGemmBN));
    hipLaunchKernelGGL((gemm_rows_kernel<T>), grid, dim3(256), 0, s, g);
    return last_launch_status();
}

}  // namespace
}  // namespace nga
