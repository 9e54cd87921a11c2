// local_attn_forward: LocalAtten, attention with the centres as queries and each centre's edges
// as keys and values, one query per segment.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense and OOM-prone --
// move to block-dense attention via the destination CSR", section "Graph-native
// alternatives": LocalAtten maps directly to variable-length attention with queries = centers
// and keys = edges, destination_row_ptr giving the segments, streamed in bounded tiles with a
// running max and denominator (the online-softmax recurrence) so that memory stays O(E c).
//
// With one query per segment the key and value projections need not be formed per edge.
// Per head h (columns h*d .. h*d+d-1):
//   s_j = (xc Wq . x_j Wk)_h / sqrt(d) = x_j . R_h,   R_h = xc M_h,  M_h = Wq[:, h] Wk[:, h]^T / sqrt(d)
//   o_h Wo[h, :] = (sum_j w_j x_j) Wv[:, h] Wo[h, :] = (U_h / Z_h) P_h,  P_h = Wv[:, h] Wo[h, :]
// so a layer is: R = Xc [M_0 | .. | M_{H-1}] (one GEMM over the centres), a streaming pass over
// the edges (scores x_j . R_h, online softmax, U_h = sum_j p_j x_j; 2 H c multiply-adds per edge
// row, each edge row read once: HBM-bound by construction), and Yc = [U_h / Z_h]_h [P_0; ..;
// P_{H-1}] (one GEMM with reduction length H c).  M and P are c x Hc per layer, built on the
// device.
//
// The streaming pass runs one work-group (4 wavefronts) per centre.  Edge rows go through LDS in
// chunks of up to 64 (fewer for wide rows, keeping the LDS within 64 KB): one score per
// (head, row), then wave h (heads h, h+4, ...) updates the running max, the rescale and the sum
// of its heads, and the per-(head, channel) weighted sums stay in registers across chunks.
#include "nga_internal.h"
#include "gemm_rows.h"

namespace nga {

namespace {

constexpr int kLocalThreads = 256;
constexpr int kLocalChunk = 64;  // score slots per head (one wavefront); rows per chunk <= this
constexpr size_t kLocalLds = 64 * 1024;
constexpr int kLocalMaxC = 256;
constexpr int kLocalMaxHeads = 16;

template <typename T>
__device__ inline T exp_t(T v);
template <>
__device__ inline double exp_t<double>(double v) { return exp(v); }
template <>
__device__ inline float exp_t<float>(float v) { return expf(v); }

// M_h[s][u] = sum over head h's columns t of Wq[s][t] Wk[u][t] / sqrt(d): H matrices [c][c].
template <typename T>
__global__ void build_m_kernel(const T* __restrict__ W, int c, int heads, T* __restrict__ M) {
    const int d = c / heads;
    const T scale = T(1) / sqrt(T(d));
    const T* Wq = W;
    const T* Wk = W + (size_t)c * c;
    const int64_t total = (int64_t)heads * c * c;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int h = (int)(idx / ((int64_t)c * c));
        const int s = (int)(idx / c % c), u = (int)(idx % c);
        T acc = T(0);
        for (int t = h * d; t < (h + 1) * d; ++t) acc += Wq[(size_t)s * c + t] * Wk[(size_t)u * c + t];
        M[idx] = acc * scale;
    }
}

// P[h c + u][col] = sum over head h's columns t of Wv[u][t] Wo[t][col]: one matrix [H c][c].
template <typename T>
__global__ void build_p_kernel(const T* __restrict__ W, int c, int heads, T* __restrict__ P) {
    const int d = c / heads;
    const T* Wv = W + 2 * (size_t)c * c;
    const T* Wo = W + 3 * (size_t)c * c;
    const int64_t total = (int64_t)heads * c * c;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int hu = (int)(idx / c), col = (int)(idx % c);
        const int h = hu / c, u = hu % c;
        T acc = T(0);
        for (int t = h * d; t < (h + 1) * d; ++t) acc += Wv[(size_t)u * c + t] * Wo[(size_t)t * c + col];
        P[idx] = acc;
    }
}

template <typename T>
struct LocalArgs {
    const int64_t* row_ptr;
    const int32_t* order;
    const T* r;   // [n_centres][H c]: R_h of each centre
    const T* x;   // [n_edges][c]
    T* un;        // [n_centres][H c]: U_h / Z_h of each centre
    int64_t n_centres;
    int64_t n_edges;
    int c;
    int heads;
    int chunk;  // edge rows per LDS chunk
    uint32_t* status;
};

// 16-byte vectors: 4 floats or 2 doubles.
template <typename T>
struct Vec;
template <>
struct Vec<float> {
    typedef float type __attribute__((ext_vector_type(4)));
    static constexpr int n = 4;
};
template <>
struct Vec<double> {
    typedef double type __attribute__((ext_vector_type(2)));
    static constexpr int n = 2;
};

constexpr int kLocalMaxSlots = 8;  // vector columns per thread in the weighted sums

template <typename V, typename T>
__device__ inline V vsplat(T v) {
    V r;
#pragma unroll
    for (int e = 0; e < (int)(sizeof(V) / sizeof(T)); ++e) r[e] = v;
    return r;
}

// SLOTS: vector columns per thread in the weighted sums (1 when the head x column vectors fit
// one per thread); PRE > 0: the chunk's rows (at most PRE vectors per thread) are loaded into
// registers one chunk ahead, so their HBM latency overlaps the current chunk's arithmetic.
template <typename T, int SLOTS, int PRE>
__global__ void __launch_bounds__(kLocalThreads) local_stream_kernel(LocalArgs<T> A) {
    typedef typename Vec<T>::type V;
    constexpr int EV = Vec<T>::n;
    const int c = A.c, H = A.heads, hc = H * c;
    const int cv = c / EV;          // vectors per row
    const int sxv = cv + 1;         // LDS row stride in vectors (16-byte aligned rows)
    const int nv = hc / EV;         // (head, vector column) slots
    // weighted sums: thread -> (slot, row partition); np partitions of the chunk's rows
    const int np = nv >= kLocalThreads ? 1 : kLocalThreads / nv;
    const int chunk = A.chunk;
    const int xsv = chunk * sxv > np * nv ? chunk * sxv : np * nv;  // chunk rows or partials
    extern __shared__ __align__(16) unsigned char local_smem[];
    V* sX = reinterpret_cast<V*>(local_smem);       // [chunk][cv + 1]
    V* sR = sX + xsv;                                // [H][cv]
    T* sS = reinterpret_cast<T*>(sR + nv);           // [H][kLocalChunk + 1] scores, then weights
    T* sM = sS + H * (kLocalChunk + 1);              // [H] running max
    T* sZ = sM + H;                                  // [H] running sum
    T* sAl = sZ + H;                                 // [H] rescale of this chunk
    V* sP = sX;                                      // [np][nv] partial sums at the end

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t i = blockIdx.x;
    const int64_t r0 = A.row_ptr[i], r1 = A.row_ptr[i + 1];
    if (r0 < 0 || r1 < r0 || r1 > A.n_edges) {
        if (tid == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int64_t n = r1 - r0;
    bool bad_index = false;
    const V* rg = reinterpret_cast<const V*>(A.r + i * hc);
    for (int t = tid; t < nv; t += kLocalThreads) sR[t] = rg[t];
    for (int h = tid; h < H; h += kLocalThreads) {
        sM[h] = T(-INFINITY);
        sZ[h] = T(0);
    }
    const int part = tid / (np > 1 ? nv : kLocalThreads);  // row partition of this thread
    V U[SLOTS];
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) U[k] = vsplat<V>(T(0));

    // vector idx of the chunk starting at edge j0 (rows rws), or zero past the row end
    auto fetch = [&](int64_t j0, int rws, int idx) -> V {
        V v = vsplat<V>(T(0));
        if (idx < rws * cv) {
            const int j = idx / cv, t = idx - j * cv;
            const int64_t slot = r0 + j0 + j;
            const int64_t row = A.order ? (int64_t)A.order[slot] : slot;
            if (row >= 0 && row < A.n_edges)
                v = reinterpret_cast<const V*>(A.x + row * c)[t];
            else
                bad_index = true;
        }
        return v;
    };
    V pre[PRE > 0 ? PRE : 1];
    if constexpr (PRE > 0) {
        const int rws = (int)(n < chunk ? n : chunk);
#pragma unroll
        for (int q = 0; q < PRE; ++q) pre[q] = fetch(0, rws, tid + q * kLocalThreads);
    }
    __syncthreads();

    for (int64_t j0 = 0; j0 < n; j0 += chunk) {
        const int rows = (int)(n - j0 < chunk ? n - j0 : chunk);
        if constexpr (PRE > 0) {
#pragma unroll
            for (int q = 0; q < PRE; ++q) {
                const int idx = tid + q * kLocalThreads;
                if (idx < rows * cv) sX[(idx / cv) * sxv + idx % cv] = pre[q];
            }
            if (j0 + chunk < n) {  // the next chunk, in flight during this one
                const int64_t jn = j0 + chunk;
                const int rn = (int)(n - jn < chunk ? n - jn : chunk);
#pragma unroll
                for (int q = 0; q < PRE; ++q) pre[q] = fetch(jn, rn, tid + q * kLocalThreads);
            }
        } else {
            for (int idx = tid; idx < rows * cv; idx += kLocalThreads)
                sX[(idx / cv) * sxv + idx % cv] = fetch(j0, rows, idx);
        }
        __syncthreads();
        // scores: pair p = h * 64 + j, one head per wavefront; R_h reads are broadcasts.  With
        // at most one head per wavefront, lane j of wavefront h keeps its own score for the
        // softmax step below, and the barrier between the two steps is not needed.
        const bool own = H <= kLocalThreads / 64;
        T s_own = T(-INFINITY);
        for (int p = tid; p < H * kLocalChunk; p += kLocalThreads) {
            const int h = p / kLocalChunk, j = p - h * kLocalChunk;
            T s = T(-INFINITY);
            if (j < rows) {
                V acc = vsplat<V>(T(0));
                for (int u = 0; u < cv; ++u) acc += sX[j * sxv + u] * sR[h * cv + u];
                s = acc[0];
#pragma unroll
                for (int e = 1; e < EV; ++e) s += acc[e];
            }
            if (own)
                s_own = s;
            else
                sS[h * (kLocalChunk + 1) + j] = s;
        }
        if (!own) __syncthreads();
        // online softmax: wavefront w owns heads w, w+4, ...
        for (int h = wave; h < H; h += kLocalThreads / 64) {
            const T s = own ? s_own : sS[h * (kLocalChunk + 1) + lane];
            T m = s;
            for (int off = 32; off > 0; off >>= 1) {
                const T o = __shfl_xor(m, off, 64);
                m = o > m ? o : m;
            }
            const T mold = sM[h];
            const T mnew = m > mold ? m : mold;
            const T p = lane < rows ? exp_t<T>(s - mnew) : T(0);
            T z = p;
            for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
            const T alpha = exp_t<T>(mold - mnew);  // 0 on the first chunk
            sS[h * (kLocalChunk + 1) + lane] = p;
            if (lane == 0) {
                sAl[h] = alpha;
                sZ[h] = sZ[h] * alpha + z;
                sM[h] = mnew;
            }
        }
        __syncthreads();
        // weighted sums of the raw rows: slot k of this thread is the vector column
        // (tid % nv) + k * 256 (np == 1) or tid % nv (np > 1), over rows part, part + np, ...
        if (part < np) {
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int slot = (np > 1 ? tid % nv : tid) + k * kLocalThreads;
                if ((np > 1 && k > 0) || slot >= nv) break;
                const int h = slot / cv, t = slot - h * cv;
                V acc = U[k] * sAl[h];
                const T* ps = sS + h * (kLocalChunk + 1);
                for (int j = part; j < rows; j += np) acc += ps[j] * sX[j * sxv + t];
                U[k] = acc;
            }
        }
        __syncthreads();
    }
    // partial sums of the row partitions -> sP, then U_h / Z_h (zero without edges)
    if (np > 1) {
        if (part < np) sP[part * nv + tid % nv] = U[0];
        __syncthreads();
        for (int slot = tid; slot < nv; slot += kLocalThreads) {
            V acc = sP[slot];
            for (int q = 1; q < np; ++q) acc += sP[q * nv + slot];
            const T z = sZ[slot / cv];
            reinterpret_cast<V*>(A.un + i * hc)[slot] = n > 0 ? acc / z : vsplat<V>(T(0));
        }
    } else {
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
            const int slot = tid + k * kLocalThreads;
            if (slot < nv) {
                const T z = sZ[slot / cv];
                reinterpret_cast<V*>(A.un + i * hc)[slot] = n > 0 ? U[k] / z : vsplat<V>(T(0));
            }
        }
    }
    if (bad_index) raise_bits(A.status, kBitIndex);
}

// LDS bytes of the streaming kernel for `chunk` rows per chunk.
size_t local_lds_bytes(int c, int heads, int chunk, size_t es) {
    const size_t row = (size_t)c * es + 16;  // one padded row
    size_t xs = (size_t)chunk * row;
    const size_t hc = (size_t)heads * c * es;
    const int ev = (int)(16 / es);
    const int nv = heads * c / ev;
    const int np = nv >= kLocalThreads ? 1 : kLocalThreads / nv;
    const size_t partials = (size_t)np * nv * 16;  // reuse of the chunk buffer at the end
    if (partials > xs) xs = partials;
    return xs + hc + es * ((size_t)heads * (kLocalChunk + 1) + 3 * (size_t)heads);
}

// Edge rows per chunk that keep the LDS within kLocalLds (0 if not even one fits).
int local_chunk_rows(int c, int heads, size_t es) {
    for (int rows = kLocalChunk; rows >= 1; --rows)
        if (local_lds_bytes(c, heads, rows, es) <= kLocalLds) return rows;
    return 0;
}

struct LocalWs {
    void* r;
    void* un;
    void* m;
    void* p;
    void* xbuf;
    size_t bytes;
};

LocalWs carve_local(void* ws, int64_t n_centres, int c, int heads, int layers, size_t es) {
    Carver cv(ws);
    LocalWs w;
    const size_t hc = (size_t)heads * c;
    w.r = cv.take<char>((size_t)n_centres * hc * es);
    w.un = cv.take<char>((size_t)n_centres * hc * es);
    w.m = cv.take<char>(hc * c * es);
    w.p = cv.take<char>(hc * c * es);
    w.xbuf = cv.take<char>(layers > 1 ? (size_t)n_centres * c * es : 0);
    w.bytes = cv.off;
    return w;
}

template <typename T>
int run_local(const int64_t* row_ptr, const int32_t* order, int64_t n_centres, int64_t n_edges,
              int c, int heads, int layers, int chunk, const T* weights, const T* xc, const T* x,
              T* yc, const LocalWs& w, uint32_t* status, hipStream_t s) {
    T* R = static_cast<T*>(w.r);
    T* Un = static_cast<T*>(w.un);
    T* M = static_cast<T*>(w.m);
    T* P = static_cast<T*>(w.p);
    T* xbuf = static_cast<T*>(w.xbuf);
    const int hc = heads * c;
    const size_t cc = (size_t)c * c;
    const size_t lds = local_lds_bytes(c, heads, chunk, sizeof(T));
    const dim3 prep_grid((unsigned)((hc * c + 255) / 256));
    int rc;
    for (int l = 0; l < layers; ++l) {
        const T* W = weights + (size_t)l * 4 * cc;
        hipLaunchKernelGGL((build_m_kernel<T>), prep_grid, dim3(256), 0, s, W, c, heads, M);
        hipLaunchKernelGGL((build_p_kernel<T>), prep_grid, dim3(256), 0, s, W, c, heads, P);
        if ((rc = last_launch_status())) return rc;
        GemmArgs<T> g1;  // R = Xc [M_0 | .. | M_{H-1}]
        g1.a = l == 0 ? xc : xbuf;
        g1.a_rows = nullptr;
        g1.w = M;
        g1.out = R;
        g1.out_rows = nullptr;
        g1.e_dev = nullptr;
        g1.n_edges = n_centres;
        g1.c = c;
        g1.nmat = heads;
        g1.lda = c;
        g1.ldo = hc;
        g1.status = status;
        if ((rc = launch_gemm(g1, n_centres, s))) return rc;
        LocalArgs<T> a{row_ptr, order, R, x, Un, n_centres, n_edges, c, heads, chunk, status};
        const int nv = hc / Vec<T>::n;
        const int loads = (chunk * (c / Vec<T>::n) + kLocalThreads - 1) / kLocalThreads;
        if (nv <= kLocalThreads && loads <= 4)
            hipLaunchKernelGGL((local_stream_kernel<T, 1, 4>), dim3((unsigned)n_centres),
                               dim3(kLocalThreads), lds, s, a);
        else
            hipLaunchKernelGGL((local_stream_kernel<T, kLocalMaxSlots, 0>), dim3((unsigned)n_centres),
                               dim3(kLocalThreads), lds, s, a);
        if ((rc = last_launch_status())) return rc;
        GemmArgs<T> g2 = g1;  // Yc = Un [P_0; ..; P_{H-1}]
        g2.a = Un;
        g2.w = P;
        g2.out = l == layers - 1 ? yc : xbuf;
        g2.nmat = 1;
        g2.k = hc;
        g2.lda = hc;
        g2.ldo = c;
        if ((rc = launch_gemm(g2, n_centres, s))) return rc;
    }
    return NGA_OK;
}

bool local_args_ok(int64_t n_centres, int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                   size_t es) {
    return n_centres >= 0 && n_centres < INT32_MAX && n_edges >= 0 && c >= 4 && c % 4 == 0 &&
           c <= kLocalMaxC && heads >= 1 && heads <= kLocalMaxHeads && c % heads == 0 &&
           layers >= 1 && local_chunk_rows(c, heads, es) >= 1;
}

}  // namespace

}  // namespace nga

extern "C" size_t local_attn_workspace_bytes(int dtype, int64_t n_centres, int32_t c,
                                             int32_t n_heads, int32_t n_layers) {
    if (dtype != NGA_F64 && dtype != NGA_F32) return 0;
    const size_t es = dtype == NGA_F64 ? sizeof(double) : sizeof(float);
    if (!nga::local_args_ok(n_centres, 0, c, n_heads, n_layers, es)) return 0;
    return nga::carve_local(nullptr, n_centres, c, n_heads, n_layers, es).bytes;
}

extern "C" int local_attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order,
                                  int64_t n_centres, int64_t n_edges, int32_t c, int32_t n_heads,
                                  int32_t n_layers, const void* weights, const void* xc,
                                  const void* x, void* yc, void* ws, size_t ws_bytes,
                                  void* stream) {
    using namespace nga;
    if (dtype != NGA_F64 && dtype != NGA_F32) return NGA_EDTYPE;
    const size_t es = dtype == NGA_F64 ? sizeof(double) : sizeof(float);
    if (!local_args_ok(n_centres, n_edges, c, n_heads, n_layers, es)) return NGA_EINVAL;
    if (!row_ptr) return NGA_EINVAL;
    if (n_centres > 0 && (!xc || !yc || !weights)) return NGA_EINVAL;
    if (n_edges > 0 && !x) return NGA_EINVAL;
    if (n_centres > 0) {
        const char* a = static_cast<const char*>(xc);
        const char* b = static_cast<const char*>(yc);
        const size_t span = (size_t)n_centres * c * es;
        if (a < b + span && b < a + span) return NGA_EINVAL;
    }
    const size_t need = local_attn_workspace_bytes(dtype, n_centres, c, n_heads, n_layers);
    if (!ws || ws_bytes < need) return NGA_EWORKSPACE;
    if (n_centres == 0) return NGA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* status = &static_cast<WsHeader*>(ws)->status;
    const LocalWs w = carve_local(ws, n_centres, c, n_heads, n_layers, es);
    const int chunk = local_chunk_rows(c, n_heads, es);
    if (dtype == NGA_F64)
        return run_local<double>(row_ptr, order, n_centres, n_edges, c, n_heads, n_layers, chunk,
                                 static_cast<const double*>(weights),
                                 static_cast<const double*>(xc), static_cast<const double*>(x),
                                 static_cast<double*>(yc), w, status, s);
    return run_local<float>(row_ptr, order, n_centres, n_edges, c, n_heads, n_layers, chunk,
                            static_cast<const float*>(weights), static_cast<const float*>(xc),
                            static_cast<const float*>(x), static_cast<float*>(yc), w, status, s);
}
