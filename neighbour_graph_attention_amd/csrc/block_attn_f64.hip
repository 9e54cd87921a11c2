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
#include <atomic>

#include "block_attn_f64.h"

namespace nga {

namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

__device__ inline d4 mfma64(double a, double b, d4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// A matrix-core result scaled by f and held in place by an empty asm: every later reader,
// behind whatever branches, reads this vector multiply's result, never the product's
// registers themselves (an fp64 product writes them some 19 wait states after issue, and a
// branch that skips a masked region could otherwise reach a reader sooner).
__device__ __forceinline__ d4 settle_d4(d4 v, double f) {
    double a0 = v[0] * f, a1 = v[1] * f, a2 = v[2] * f, a3 = v[3] * f;
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    return d4{a0, a1, a2, a3};
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
    double one;  // 1.0, a run-time value the compiler cannot fold (settle_d4)
};

constexpr int kKc = 16;  // k chunk staged in LDS
constexpr int kPerB = kKc * 64 / 256;  // values of each B chunk per thread

// out[m][u] = sum_t A[m][t] W_{u / c}[t][u % c]; work-group tile TM x 64, wave w owns rows
// (TM/2)*(w/2) .. +TM/2 and columns 32*(w%2) .. +32 as (TM/32) x 2 matrix-core tiles.
// C > 0: c is known at compile time and a multiple of 64, so every column and k index is in
// range, the k loop unrolls and the loads need no guards (rows past E read row 0 and are
// replaced by zeros); C = 0: any c, checked at run time.
template <int TM, int C>
__global__ void __launch_bounds__(256) gemm_f64_kernel(GemmF64Args g) {
    static_assert(C % 64 == 0, "compile-time widths are multiples of 64");
    constexpr bool kFixed = C > 0;
    const int c = kFixed ? C : g.c;
    constexpr int PA = TM * kKc / 256;  // values of each A chunk per thread
    constexpr int BI = TM / 32;         // 16-row matrix-core tiles per wave
    __shared__ double sA[TM][kKc + 1];
    __shared__ double sB[kKc][64 + 1];
    const int64_t E = *g.e_dev < g.n_edges ? *g.e_dev : g.n_edges;
    const int64_t m0 = (int64_t)blockIdx.x * TM;
    const int u0 = blockIdx.y * 64;
    if (m0 >= E) return;
    const int nout = g.nmat * c;
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
    const bool u_in = kFixed || u < nout;
    const double* wcol = g.w + (u_in ? (int64_t)(u / c) * c * c + (u % c) : 0);
    double pa[PA], pb[kPerB];
    auto fetch = [&](int k0) {
        if constexpr (kFixed) {
#pragma unroll
            for (int j = 0; j < PA; ++j) {
                const double v = g.a[(a_off[j] >= 0 ? a_off[j] : 0) + k0 + a_kk];
                pa[j] = a_off[j] >= 0 ? v : 0.0;
            }
#pragma unroll
            for (int j = 0; j < kPerB; ++j) pb[j] = wcol[(int64_t)(k0 + b_k + 4 * j) * C];
        } else {
            const bool a_k_in = k0 + a_kk < c;
#pragma unroll
            for (int j = 0; j < PA; ++j)
                pa[j] = (a_off[j] >= 0 && a_k_in) ? g.a[a_off[j] + k0 + a_kk] : 0.0;
#pragma unroll
            for (int j = 0; j < kPerB; ++j) {
                const int t = k0 + b_k + 4 * j;
                pb[j] = (u_in && t < c) ? wcol[(int64_t)t * c] : 0.0;
            }
        }
    };
    // One k chunk: the staged chunk from registers into LDS, the next chunk's loads, the
    // chunk's products.
    auto chunk = [&](int k0) {
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
        if (k0 + kKc < c) fetch(k0 + kKc);
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
    };
    fetch(0);
    if constexpr (kFixed) {
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += kKc) chunk(k0);
    } else {
        for (int k0 = 0; k0 < c; k0 += kKc) chunk(k0);
    }
    // The stores below sit behind row and index branches: they read the products' results
    // through this multiply (see settle_d4).
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = settle_d4(acc[i][j], g.one);
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
                if (kFixed || u < nout) g.out[row * g.ldo + u] = acc[i][j][r];
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
        // NT = ceil(n / 16), so only keys of the last tile can lie past n.
        double m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (kt == NT - 1 && 16 * kt + gq + 4 * r >= n) s[kt][r] = -INFINITY;
                m = fmax(m, s[kt][r]);
            }
        m = fmax(m, __shfl_xor(m, 16, 64));
        m = fmax(m, __shfl_xor(m, 32, 64));
        double z = 0.0;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool masked = kt == NT - 1 && 16 * kt + gq + 4 * r >= n;
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
    if (r1 == r0) return;
    if (r1 < r0 || r1 - r0 > A.nnei_cap || r1 - r0 > 16 * kF64TileMax || r0 < 0 ||
        r1 > A.n_edges) {
        if (threadIdx.x == 0 && h == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int n = (int)(r1 - r0);
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

// ---------------------------------------------------------------------------------------------
// Attention core and output projection of one centre in one work-group, every head.
//
// With the core split over (centre, head) work-groups, the output projection y = o Wo needs
// all heads of a row, so it ran as a third launch per layer over an o buffer in HBM.  Here a
// work-group of kCoreWaves wavefronts takes a whole centre: wavefront w owns query tile w, and
// for each head h in turn it forms S^T = K_h Q_h^T, the masked softmax and O_h = P V_h exactly
// as the per-head core does, then adds O_h Wo[hD .. hD+D-1][:] into a 16 x c tile of y held in
// its registers.  O_h serves as that product's A operand as it stands: lane (g, l), register r
// of value tile dt holds O_h[query l][channel 16 dt + 4r + g], which is A[i = l][k = g] of the
// k-step over channels 16 dt + 4r .. +3; B[k][j] = Wo[hD + 16 dt + 4r + k][16u + j] is read
// per lane from the weights (L2-resident), and the result lands in lane (g, l), register r' as
// y[query 4r' + g][channel 16u + l].  A wavefront that has finished head h loads K and V of
// head h + 1 into the second of two LDS buffers while the others still read the first, so
// one barrier per head suffices.  Heads are summed into y in order 0, 1, ... and, within a
// head, channel groups in order, as the row GEMM sums its k chunks: the result is bit for bit
// the core-then-GEMM one.
//
// One work-group per centre holds 135 KB of LDS and up to 256 VGPRs per wavefront, so a
// compute unit runs one such work-group (two wavefronts per SIMD) against two of the per-head
// core.  It pays when the centres fill most compute units in every round (use_core_wo).
struct CoreWoF64Args {
    const double* qkv;          // [E][3c] slot-indexed: q | k | v
    const double* wo;           // this layer's Wo [c][c] (y = o Wo)
    double* out;                // [*][c]
    const int32_t* out_rows;    // nullable: y of slot s goes to out[out_rows[s]]
    const int64_t* row_ptr;
    int64_t n_centres;
    int64_t n_edges;
    int nnei_cap;
    double scale;               // 1 / sqrt(d)
    const double* ldt;          // smooth attention: this layer's ln D~ [n_edges][heads], or NULL
    const int32_t* order;       // edge row of each slot (NULL: the slot itself), for ldt
    uint32_t* status;
    double one;                 // 1.0, a run-time value the compiler cannot fold (settle_d4)
};

template <int D, int C, int NT, bool SM>
__device__ __forceinline__ void core_wo_centre(const CoreWoF64Args& A,
                                               double (*__restrict__ sK)[16 * kF64TileMax][D + 1],
                                               double (*__restrict__ sV)[16 * kF64TileMax][D + 1],
                                               const int64_t r0, const int n) {
    constexpr int H = C / D;
    constexpr int UO = C / 16;          // 16-wide output tiles of y
    constexpr int KSTEP = D / 4;        // k-steps over a head's channels
    constexpr int DT = (D + 15) / 16;   // 16-channel tiles of O_h
    constexpr int kThreads = 64 * kCoreWaves;
    constexpr int kIter = (16 * NT * D + kThreads - 1) / kThreads;  // K/V values per thread
    constexpr int c3 = 3 * C;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const bool active = w < NT;
    const int a = 16 * w + li;          // this lane's query (row of the centre)
    const double scale2 = A.scale * kLog2eF64;

    double kst[kIter], vst[kIter];
    // K_h and V_h for a buffer: all of the thread's global loads, then its LDS stores.
    auto fetch_kv = [&](int h) {
#pragma unroll
        for (int j = 0; j < kIter; ++j) {
            const int idx = threadIdx.x + kThreads * j, b = idx / D, t = idx % D;
            kst[j] = 0.0;
            vst[j] = 0.0;
            if (idx < 16 * NT * D && b < n) {
                const double* rowp = A.qkv + (r0 + b) * c3 + h * D + t;
                kst[j] = rowp[C];
                vst[j] = rowp[2 * C];
            }
        }
    };
    auto store_kv = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kIter; ++j) {
            const int idx = threadIdx.x + kThreads * j;
            if (idx < 16 * NT * D) {
                sK[buf][idx / D][idx % D] = kst[j];
                sV[buf][idx / D][idx % D] = vst[j];
            }
        }
    };
    // Q_h operand of this lane: Q[a][4kk + gq] for k-step kk.
    double q[KSTEP];
    auto fetch_q = [&](int h) {
#pragma unroll
        for (int kk = 0; kk < KSTEP; ++kk)
            q[kk] = (active && a < n) ? A.qkv[(r0 + a) * c3 + h * D + 4 * kk + gq] : 0.0;
    };

    d4 yacc[UO];
#pragma unroll
    for (int u = 0; u < UO; ++u) yacc[u] = d4{0.0, 0.0, 0.0, 0.0};

    fetch_kv(0);
    store_kv(0);
    fetch_q(0);
    __syncthreads();
#pragma unroll 1
    for (int h = 0; h < H; ++h) {
        const int buf = h & 1;
        if (active) {
            // Scores, with each key tile's operands read from LDS one tile ahead of its
            // products (two wavefronts per SIMD leave little else to cover the LDS latency).
            d4 s[NT];
            double kcur[KSTEP], knext[KSTEP];
#pragma unroll
            for (int kk = 0; kk < KSTEP; ++kk) kcur[kk] = sK[buf][li][4 * kk + gq];
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                if (kt + 1 < NT) {
#pragma unroll
                    for (int kk = 0; kk < KSTEP; ++kk)
                        knext[kk] = sK[buf][16 * (kt + 1) + li][4 * kk + gq];
                }
                d4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int kk = 0; kk < KSTEP; ++kk) acc = mfma64(kcur[kk], q[kk], acc);
                s[kt] = acc;  // lane (gq, li), register r: key 16kt + gq + 4r, query a
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < KSTEP; ++kk) kcur[kk] = knext[kk];
            }
            double m = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (kt == NT - 1 && 16 * kt + gq + 4 * r >= n) s[kt][r] = -INFINITY;
                    m = fmax(m, s[kt][r]);
                }
            m = fmax(m, __shfl_xor(m, 16, 64));
            m = fmax(m, __shfl_xor(m, 32, 64));
            double z = 0.0;
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool masked = kt == NT - 1 && 16 * kt + gq + 4 * r >= n;
                    const double p = exp2_nonpos(masked ? -4096.0 : (s[kt][r] - m) * scale2);
                    s[kt][r] = p;
                    z += p;
                }
            z += __shfl_xor(z, 16, 64);
            z += __shfl_xor(z, 32, 64);
            // Smooth attention: sum_j e_j / D~ times the softmax = exp(s_j - ln D~), i.e. the
            // weighted sum times exp(m - ln D~) in place of 1/Z.  Rows past n get 0.
            double f = 1.0 / z;
            if constexpr (SM) {
                f = 0.0;
                if (a < n) {
                    const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
                    if (row >= 0 && row < A.n_edges) f = exp(m * A.scale - A.ldt[row * H + h]);
                }
            }
            if (a >= n) f = 0.0;
            // Weighted values, the value operands again read one key tile ahead.
            d4 o[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                d4 acc = {0.0, 0.0, 0.0, 0.0};
                const int tcol = 16 * dt + li;
                double vcur[4], vnext[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vcur[r] = tcol < D ? sV[buf][gq + 4 * r][tcol] : 0.0;
#pragma unroll
                for (int kt = 0; kt < NT; ++kt) {
                    if (kt + 1 < NT) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            vnext[r] = tcol < D ? sV[buf][16 * (kt + 1) + gq + 4 * r][tcol] : 0.0;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc = mfma64(vcur[r], s[kt][r], acc);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) vcur[r] = vnext[r];
                }
                // lane (gq, li), register r: O_h[query 16w + li][channel 16dt + gq + 4r]
                o[dt] = settle_d4(acc, f);
            }
            // y[query][16u + j] += sum over the head's channels k of O_h[query][k] Wo[hD + k][16u + j];
            // the weights of tile u + 1 load while tile u multiplies.
            const double* wo_h = A.wo + (int64_t)(h * D + gq) * C + li;
            double wcur[KSTEP], wnext[KSTEP];
#pragma unroll
            for (int ks = 0; ks < KSTEP; ++ks) wcur[ks] = wo_h[(int64_t)(4 * ks) * C];
#pragma unroll
            for (int u = 0; u < UO; ++u) {
                if (u + 1 < UO) {
#pragma unroll
                    for (int ks = 0; ks < KSTEP; ++ks)
                        wnext[ks] = wo_h[(int64_t)(4 * ks) * C + 16 * (u + 1)];
                }
#pragma unroll
                for (int ks = 0; ks < KSTEP; ++ks) yacc[u] = mfma64(o[ks / 4][ks % 4], wcur[ks], yacc[u]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KSTEP; ++ks) wcur[ks] = wnext[ks];
            }
            // Read back at once (see settle_d4): the next head's products and the final stores
            // read this multiply's result, whatever branches lie between.
#pragma unroll
            for (int u = 0; u < UO; ++u) yacc[u] = settle_d4(yacc[u], A.one);
        }
        if (h + 1 < H) {
            fetch_kv(h + 1);
            store_kv(buf ^ 1);
            fetch_q(h + 1);
        }
        __syncthreads();
    }
    if (!active) return;
    // lane (gq, li), register r: y[query 16w + 4r + gq][channel 16u + li]
    bool bad = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int qa = 16 * w + 4 * r + gq;
        if (qa >= n) continue;
        int64_t row = r0 + qa;
        if (A.out_rows) {
            row = A.out_rows[r0 + qa];
            if (row < 0 || row >= A.n_edges) { bad = true; continue; }
        }
        double* orow = A.out + row * C + li;
#pragma unroll
        for (int u = 0; u < UO; ++u) orow[16 * u] = yacc[u][r];
    }
    if (bad) raise_bits(A.status, kBitIndex);
}

// SM: smooth attention (ldt given), in instances of its own so that the general exponential
// and its constants take no registers in the plain softmax.
template <int D, int C, bool SM>
__global__ void __launch_bounds__(64 * kCoreWaves, 1) core_wo_f64_kernel(CoreWoF64Args A) {
    __shared__ double sK[2][16 * kF64TileMax][D + 1];
    __shared__ double sV[2][16 * kF64TileMax][D + 1];
    const int centre = blockIdx.x;
    if (centre == 0 && threadIdx.x == 0) {
        if (A.row_ptr[0] != 0 || A.row_ptr[A.n_centres] > A.n_edges) raise_bits(A.status, kBitCap);
    }
    const int64_t r0 = A.row_ptr[centre], r1 = A.row_ptr[centre + 1];
    if (r1 == r0) return;
    if (r1 < r0 || r1 - r0 > A.nnei_cap || r1 - r0 > 16 * kF64TileMax || r0 < 0 ||
        r1 > A.n_edges) {
        if (threadIdx.x == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int n = (int)(r1 - r0);
    switch ((n + 15) >> 4) {
        case 1: core_wo_centre<D, C, 1, SM>(A, sK, sV, r0, n); break;
        case 2: core_wo_centre<D, C, 2, SM>(A, sK, sV, r0, n); break;
        case 3: core_wo_centre<D, C, 3, SM>(A, sK, sV, r0, n); break;
        case 4: core_wo_centre<D, C, 4, SM>(A, sK, sV, r0, n); break;
        case 5: core_wo_centre<D, C, 5, SM>(A, sK, sV, r0, n); break;
        case 6: core_wo_centre<D, C, 6, SM>(A, sK, sV, r0, n); break;
        case 7: core_wo_centre<D, C, 7, SM>(A, sK, sV, r0, n); break;
        default: core_wo_centre<D, C, 8, SM>(A, sK, sV, r0, n); break;
    }
}

// True if core_wo_f64_kernel has an instance for this shape.
bool core_wo_supported(int c, int d) { return c == 128 && (d == 16 || d == 32); }

template <int D>
void launch_core_wo_d(const CoreWoF64Args& a, int64_t n_centres, hipStream_t s) {
    if (a.ldt)
        hipLaunchKernelGGL((core_wo_f64_kernel<D, 128, true>), dim3((unsigned)n_centres),
                           dim3(64 * kCoreWaves), 0, s, a);
    else
        hipLaunchKernelGGL((core_wo_f64_kernel<D, 128, false>), dim3((unsigned)n_centres),
                           dim3(64 * kCoreWaves), 0, s, a);
}

// The per-head core and the row GEMM spread a layer over every compute unit; the merged kernel
// takes one compute unit per centre.  Measured at c = 128, 4 heads of 32, rows of 120 on a
// 256-CU MI355X: the two launches cost about 92 us per round of 256 centres (64 centres: 30
// us, 216: 84 us), the merged kernel about 66 us per round however full (64 or 216 centres).
// So it is used when ceil(n / CUs) rounds of it beat n / CUs rounds of the other, with those
// two costs: 66 ceil(r) <= 92 r, taken as 18 ceil(r) <= 25 r.
bool use_core_wo(int64_t n_centres) {
    static std::atomic<int> cus_of[64];  // compute units per device, 0 until asked
    int dev = 0;
    if (n_centres <= 0 || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    int cus = cus_of[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess || cus <= 0)
            return false;
        cus_of[dev].store(cus, std::memory_order_relaxed);
    }
    const int64_t rounds = (n_centres + cus - 1) / cus;
    return 18 * rounds * cus <= 25 * n_centres;
}

int launch_core_wo(const CoreWoF64Args& a, int64_t n_centres, int d, hipStream_t s) {
    if (d == 16) launch_core_wo_d<16>(a, n_centres, s);
    else launch_core_wo_d<32>(a, n_centres, s);
    return last_launch_status();
}

// Rows per GEMM work-group.  More, smaller work-groups win on these small row counts:
// 32 / 64 / 128 rows measured 0.291 / 0.294 / 0.308 ms of attention at diamond-216.
constexpr int kGemmRows = 32;

int launch_gemm(const GemmF64Args& g, int64_t m_bound, hipStream_t s) {
    constexpr int TM = kGemmRows;
    const int nout = g.nmat * g.c;
    dim3 grid((unsigned)((m_bound + TM - 1) / TM), (unsigned)((nout + 63) / 64));
    if (g.c == 128) hipLaunchKernelGGL((gemm_f64_kernel<TM, 128>), grid, dim3(256), 0, s, g);
    else if (g.c == 64) hipLaunchKernelGGL((gemm_f64_kernel<TM, 64>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((gemm_f64_kernel<TM, 0>), grid, dim3(256), 0, s, g);
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

bool f64_core_wo_selected(int64_t n_centres, int32_t c, int32_t heads) {
    return heads >= 1 && c % heads == 0 && core_wo_supported(c, c / heads) &&
           use_core_wo(n_centres);
}

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
        g1.one = 1.0;
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
        const bool last = (l == layers - 1);
        if (f64_core_wo_selected(n_centres, c, heads)) {
            CoreWoF64Args b;
            b.qkv = qkv;
            b.wo = W + 3 * cc;
            b.out = last ? y : xbuf;
            b.out_rows = last ? order : nullptr;
            b.row_ptr = row_ptr;
            b.n_centres = n_centres;
            b.n_edges = n_edges;
            b.nnei_cap = nnei_cap;
            b.scale = a.scale;
            b.ldt = a.ldt;
            b.order = order;
            b.status = status;
            b.one = 1.0;
            if ((rc = launch_core_wo(b, n_centres, d, s))) return rc;
            continue;
        }
        if ((rc = launch_core(a, n_centres, heads, d, s))) return rc;
        GemmF64Args g2 = g1;
        g2.a = o;
        g2.a_rows = nullptr;
        g2.w = W + 3 * cc;
        g2.nmat = 1;
        g2.ldo = c;
        g2.out = last ? y : xbuf;
        g2.out_rows = last ? order : nullptr;
        if ((rc = launch_gemm(g2, n_edges, s))) return rc;
    }
    return NGA_OK;
}

}  // namespace nga
