// fp64 block attention on CDNA matrix cores (v_mfma_f64_16x16x4_f64).
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense ...", section
// "Proposed fix: block-dense attention on the graph": the per-centre blocks go through
// dense matrix products with a mask for the ragged tail; section "Measurements": the
// diamond runs it reports are fp64.
//
// The fp64 workloads have few centres (tens to a thousand), so one work-group per centre
// would leave most compute units idle.  Each layer is therefore three launches that spread
// over all edges or over (centre, head) pairs:
//   qkv[s] = x[row(s)] [Wq | Wk | Wv]   row-gather GEMM, 32x64 tiles, one 16x32 block per wave
//   o[s]   = attention of head h of the centre of s, one work-group per (centre, head):
//            K_h and V_h rows staged in LDS, Q read per query tile, S^T = K Q^T, masked
//            softmax, O^T = V^T P^T
//   y[row(s)] = o[s] Wo                  row-scatter GEMM
// (row(s) = order[s] when an order is given, else s; intermediate layers stay slot-indexed.)
//
// Matrix-core layout of the f64 16x16x4 product, checked on the GPU with an in-bounds
// probe: A[i][k] from lane i + 16k, B[k][j] from lane j + 16k, and D[i][j] lands in lane
// j + 16*(i%4), register i/4 -- rows interleave across registers, unlike the f32 form.  The
// scores' result registers feed the value product directly as B operands by walking the
// keys of a tile in the order b = 16kt + g + 4r (lane group g, register r).
#include "block_attn_f64.h"

namespace nga {

namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

__device__ inline d4 mfma64(double a, double b, d4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

struct GemmF64Args {
    const double* a;
    const int32_t* a_rows;    // nullable: row m of A is a[a_rows[m]]
    const double* w;          // nmat matrices [c][c] side by side in the output columns
    double* out;
    const int32_t* out_rows;  // nullable: row m of the result goes to out[out_rows[m]]
    const int64_t* e_dev;     // rows m < min(*e_dev, n_edges) are computed
    int64_t n_edges;
    int c;
    int nmat;
    int lda;
    int ldo;
    uint32_t* status;
};

constexpr int kKc = 16;  // k chunk staged in LDS
constexpr int kPerB = kKc * 64 / 256;  // values of each B chunk per thread

// out[m][u] = sum_t A[m][t] W_{u / c}[t][u % c]; work-group tile TM x 64, wave w owns rows
// (TM/2)*(w/2) .. +TM/2 and columns 32*(w%2) .. +32 as (TM/32) x 2 matrix-core tiles.
template <int TM>
__global__ void __launch_bounds__(256) gemm_f64_kernel(GemmF64Args g) {
    constexpr int PA = TM * kKc / 256;  // values of each A chunk per thread
    constexpr int BI = TM / 32;         // 16-row matrix-core tiles per wave
    __shared__ double sA[TM][kKc + 1];
    __shared__ double sB[kKc][64 + 1];
    const int64_t E = *g.e_dev < g.n_edges ? *g.e_dev : g.n_edges;
    const int64_t m0 = (int64_t)blockIdx.x * TM;
    const int u0 = blockIdx.y * 64;
    if (m0 >= E) return;
    const int nout = g.nmat * g.c;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int wr = (TM / 2) * (w >> 1), wc = 32 * (w & 1);
    bool bad = false;
    d4 acc[BI][2];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = d4{0.0, 0.0, 0.0, 0.0};

    // Chunk k0 of A (TM x kKc) and B (kKc x 64) as PA + kPerB values per thread; the next
    // chunk is loaded into registers while the current one is multiplied out of LDS.  A thread
    // reads the same PA rows of A (k = k0 + a_kk) and the same column of W
    // (k = k0 + b_k + 4j) in every chunk, so the row gather and the column offset are
    // resolved once.
    const int a_kk = tid % kKc, b_k = tid / 64;
    int64_t a_off[PA];  // offset of row m0 + tid / kKc + (256 / kKc) j in A, or -1 for zeros
#pragma unroll
    for (int j = 0; j < PA; ++j) {
        const int64_t m = m0 + tid / kKc + (256 / kKc) * j;
        a_off[j] = -1;
        if (m < E) {
            const int64_t row = g.a_rows ? (int64_t)g.a_rows[m] : m;
            if (row >= 0 && row < g.n_edges) a_off[j] = row * g.lda;
            else bad = true;
        }
    }
    const int u = u0 + tid % 64;
    const bool u_in = u < nout;
    const double* wcol = g.w + (u_in ? (int64_t)(u / g.c) * g.c * g.c + (u % g.c) : 0);
    double pa[PA], pb[kPerB];
    auto fetch = [&](int k0) {
        const bool a_k_in = k0 + a_kk < g.c;
#pragma unroll
        for (int j = 0; j < PA; ++j)
            pa[j] = (a_off[j] >= 0 && a_k_in) ? g.a[a_off[j] + k0 + a_kk] : 0.0;
#pragma unroll
        for (int j = 0; j < kPerB; ++j) {
            const int t = k0 + b_k + 4 * j;
            pb[j] = (u_in && t < g.c) ? wcol[(int64_t)t * g.c] : 0.0;
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < g.c; k0 += kKc) {
#pragma unroll
        for (int j = 0; j < PA; ++j) {
            const int idx = tid + 256 * j;
            sA[idx / kKc][idx % kKc] = pa[j];
        }
#pragma unroll
        for (int j = 0; j < kPerB; ++j) {
            const int idx = tid + 256 * j;
            sB[idx / 64][idx % 64] = pb[j];
        }
        __syncthreads();
        if (k0 + kKc < g.c) fetch(k0 + kKc);
#pragma unroll
        for (int ks = 0; ks < kKc / 4; ++ks) {
            double a[BI], b[2];
#pragma unroll
            for (int i = 0; i < BI; ++i) a[i] = sA[wr + 16 * i + li][4 * ks + gq];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = sB[4 * ks + gq][wc + 16 * j + li];
#pragma unroll
            for (int i = 0; i < BI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma64(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wr + 16 * i + gq + 4 * r;
            if (m >= E) continue;
            int64_t row = m;
            if (g.out_rows) {
                row = g.out_rows[m];
                if (row < 0 || row >= g.n_edges) { bad = true; continue; }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = u0 + wc + 16 * j + li;
                if (u < nout) g.out[row * g.ldo + u] = acc[i][j][r];
            }
        }
    if (bad) raise_bits(g.status, kBitIndex);
}

struct CoreF64Args {
    const double* qkv;  // [E][3c] slot-indexed: q | k | v
    double* o;          // [E][c] slot-indexed
    const int64_t* row_ptr;
    int64_t n_centres;
    int64_t n_edges;
    int nnei_cap;
    int c;
    double scale;  // 1 / sqrt(d)
    const double* ldt;     // smooth attention: this layer's ln D~ [n_edges][heads], or NULL
    const int32_t* order;  // edge row of each slot (NULL: the slot itself), for ldt
    uint32_t* status;
};

constexpr int kF64TileMax = 8;  // rows per centre up to 128
constexpr int kCoreWaves = 8;   // wavefronts per attention-core work-group

// The query tiles of wavefront w (w, w + kCoreWaves, ...) for a centre of NT = ceil(n / 16)
// key tiles, K and V of head h in sK / sV (rows NT*16 and beyond unused, rows n .. 16 NT - 1
// zero).
template <int D, int NT>
__device__ __forceinline__ void core_query_tiles(const CoreF64Args& A,
                                                 const double (*__restrict__ sK)[D + 1],
                                                 const double (*__restrict__ sV)[D + 1],
                                                 const int64_t r0, const int n, const int h,
                                                 const double scale2) {
    constexpr int KSTEP = (D + 3) / 4;  // k-steps of the score product
    constexpr int DT = (D + 15) / 16;   // 16-row tiles of O^T
    const int c = A.c, c3 = 3 * A.c;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    for (int qt = w; qt < NT; qt += kCoreWaves) {
        const int a = 16 * qt + li;
        // Q operand: lane (gq, li) holds Q[a][4kk + gq] for k-step kk.
        double q[KSTEP];
#pragma unroll
        for (int kk = 0; kk < KSTEP; ++kk) {
            const int t = 4 * kk + gq;
            q[kk] = (a < n && t < D) ? A.qkv[(r0 + a) * c3 + h * D + t] : 0.0;
        }
        d4 s[NT];
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            d4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int kk = 0; kk < KSTEP; ++kk) {
                const int t = 4 * kk + gq;
                const double kval = t < D ? sK[16 * kt + li][t] : 0.0;
                acc = mfma64(kval, q[kk], acc);
            }
            s[kt] = acc;  // lane (gq, li), register r: key 16kt + gq + 4r, query a
            // Keeps the scheduler from hoisting every tile's LDS reads at once.
            __builtin_amdgcn_sched_barrier(0);
        }
        double m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (16 * kt + gq + 4 * r >= n) s[kt][r] = -INFINITY;
                m = fmax(m, s[kt][r]);
            }
        m = fmax(m, __shfl_xor(m, 16, 64));
        m = fmax(m, __shfl_xor(m, 32, 64));
        double z = 0.0;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool masked = 16 * kt + gq + 4 * r >= n;
                const double p = exp2_nonpos(masked ? -4096.0 : (s[kt][r] - m) * scale2);
                s[kt][r] = p;
                z += p;
            }
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        // Smooth attention: sum_j e_j / D~ times the softmax = exp(s_j - ln D~), i.e. the
        // weighted sum times exp(m - ln D~) in place of 1/Z.
        double f = 1.0 / z;
        if (A.ldt) {
            f = 0.0;
            if (a < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
                if (row >= 0 && row < A.n_edges)
                    f = exp(m * A.scale - A.ldt[row * gridDim.y + h]);
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            d4 acc = {0.0, 0.0, 0.0, 0.0};
            const int tcol = 16 * dt + li;
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const double vval = tcol < D ? sV[16 * kt + gq + 4 * r][tcol] : 0.0;
                    acc = mfma64(vval, s[kt][r], acc);
                    if (r == 3) __builtin_amdgcn_sched_barrier(0);
                }
            // lane (gq, li), register r: O[a = 16qt + li][t = 16dt + gq + 4r]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * dt + gq + 4 * r;
                if (a < n && t < D) A.o[(r0 + a) * c + h * D + t] = acc[r] * f;
            }
        }
    }
}

// One work-group per (centre = blockIdx.x, head = blockIdx.y) of kCoreWaves wavefronts; wave w
// takes query tiles w, w + kCoreWaves, ...  K_h and V_h of the centre sit in LDS (rows past n
// are zero).  Eight wavefronts of at most 128 VGPRs give four per SIMD, twice what four
// wavefronts per work-group reached.
template <int D>
__global__ void __launch_bounds__(64 * kCoreWaves, 2) attn_core_f64_kernel(CoreF64Args A) {
    constexpr int DP = D + 1;  // padded LDS row (doubles)
    __shared__ double sK[16 * kF64TileMax][DP];
    __shared__ double sV[16 * kF64TileMax][DP];

    const int centre = blockIdx.x, h = blockIdx.y;
    // The CSR as a whole: it starts at 0 and ends within the edge rows.
    if (centre == 0 && h == 0 && threadIdx.x == 0) {
        if (A.row_ptr[0] != 0 || A.row_ptr[A.n_centres] > A.n_edges) raise_bits(A.status, kBitCap);
    }
    const int64_t r0 = A.row_ptr[centre], r1 = A.row_ptr[centre + 1];
    const int n = (int)(r1 - r0);
    if (n <= 0) return;
    if (n > A.nnei_cap || n > 16 * kF64TileMax || r0 < 0 || r1 > A.n_edges) {
        if (threadIdx.x == 0 && h == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int nt = (n + 15) >> 4;
    const double scale2 = A.scale * kLog2eF64;  // softmax exponents in base 2
    const int c = A.c, c3 = 3 * A.c;
    for (int idx = threadIdx.x; idx < 16 * nt * D; idx += 64 * kCoreWaves) {
        const int b = idx / D, t = idx % D;
        double kv = 0.0, vv = 0.0;
        if (b < n) {
            const double* rowp = A.qkv + (r0 + b) * c3 + h * D + t;
            kv = rowp[c];
            vv = rowp[2 * c];
        }
        sK[b][t] = kv;
        sV[b][t] = vv;
    }
    __syncthreads();

    switch (nt) {
        case 1: core_query_tiles<D, 1>(A, sK, sV, r0, n, h, scale2); break;
        case 2: core_query_tiles<D, 2>(A, sK, sV, r0, n, h, scale2); break;
        case 3: core_query_tiles<D, 3>(A, sK, sV, r0, n, h, scale2); break;
        case 4: core_query_tiles<D, 4>(A, sK, sV, r0, n, h, scale2); break;
        case 5: core_query_tiles<D, 5>(A, sK, sV, r0, n, h, scale2); break;
        case 6: core_query_tiles<D, 6>(A, sK, sV, r0, n, h, scale2); break;
        case 7: core_query_tiles<D, 7>(A, sK, sV, r0, n, h, scale2); break;
        default: core_query_tiles<D, 8>(A, sK, sV, r0, n, h, scale2); break;
    }
}

// Rows per GEMM work-group.  More, smaller work-groups win on these small row counts:
// 32 / 64 / 128 rows measured 0.291 / 0.294 / 0.308 ms of attention at diamond-216.
constexpr int kGemmRows = 32;

int launch_gemm(const GemmF64Args& g, int64_t m_bound, hipStream_t s) {
    constexpr int TM = kGemmRows;
    const int nout = g.nmat * g.c;
    dim3 grid((unsigned)((m_bound + TM - 1) / TM), (unsigned)((nout + 63) / 64));
    hipLaunchKernelGGL(gemm_f64_kernel<TM>, grid, dim3(256), 0, s, g);
    return last_launch_status();
}

int launch_core(const CoreF64Args& a, int64_t n_centres, int heads, int d, hipStream_t s) {
    dim3 grid((unsigned)n_centres, (unsigned)heads), block(64 * kCoreWaves);
    if (d == 8) hipLaunchKernelGGL(attn_core_f64_kernel<8>, grid, block, 0, s, a);
    else if (d == 16) hipLaunchKernelGGL(attn_core_f64_kernel<16>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_core_f64_kernel<32>, grid, block, 0, s, a);
    return last_launch_status();
}

}  // namespace

bool f64_mfma_supported(int32_t nnei_cap, int32_t c, int32_t heads) {
    if (heads < 1 || c % heads != 0) return false;
    const int d = c / heads;
    if (d != 8 && d != 16 && d != 32) return false;
    return nnei_cap >= 1 && nnei_cap <= 16 * kF64TileMax;
}

int run_f64_mfma(const int64_t* row_ptr, const int32_t* order, int64_t n_centres, int64_t n_edges,
                 int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers, const double* weights,
                 const double* x, const double* log_dtilde, double* y, double* qkv, double* o,
                 double* xbuf, uint32_t* status, hipStream_t s) {
    const int64_t* e_dev = row_ptr + n_centres;
    const size_t cc = (size_t)c * c;
    const int d = c / heads;
    int rc;
    for (int l = 0; l < layers; ++l) {
        const double* W = weights + (size_t)l * 4 * cc;
        GemmF64Args g1;
        g1.a = (l == 0) ? x : xbuf;
        g1.a_rows = (l == 0) ? order : nullptr;
        g1.w = W;
        g1.out = qkv;
        g1.out_rows = nullptr;
        g1.e_dev = e_dev;
        g1.n_edges = n_edges;
        g1.c = c;
        g1.nmat = 3;
        g1.lda = c;
        g1.ldo = 3 * c;
        g1.status = status;
        if ((rc = launch_gemm(g1, n_edges, s))) return rc;
        CoreF64Args a;
        a.qkv = qkv;
        a.o = o;
        a.row_ptr = row_ptr;
        a.n_centres = n_centres;
        a.n_edges = n_edges;
        a.nnei_cap = nnei_cap;
        a.c = c;
        a.scale = 1.0 / std::sqrt((double)d);
        a.ldt = log_dtilde ? log_dtilde + (size_t)l * n_edges * heads : nullptr;
        a.order = order;
        a.status = status;
        if ((rc = launch_core(a, n_centres, heads, d, s))) return rc;
        GemmF64Args g2 = g1;
        g2.a = o;
        g2.a_rows = nullptr;
        g2.w = W + 3 * cc;
        g2.nmat = 1;
        g2.ldo = c;
        const bool last = (l == layers - 1);
        g2.out = last ? y : xbuf;
        g2.out_rows = last ? order : nullptr;
        if ((rc = launch_gemm(g2, n_edges, s))) return rc;
    }
    return NGA_OK;
}

}  // namespace nga
