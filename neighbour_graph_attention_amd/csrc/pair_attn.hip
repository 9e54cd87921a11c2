// pair_attn_forward: the ragged pair-axis route, kept as a measured comparator.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense and OOM-prone --
// move to block-dense attention via the destination CSR", section "Root cause": the route the
// block-dense attention replaces enumerates the P = sum nnei^2 centre pairs, materialises
// (P, channels) intermediates and reduces them with a segment softmax and index_add, atomics
// included; section "Cross-checks" prints one such allocation (P pairs x 128 fp64 channels,
// 5.14 GiB at 216 diamond atoms).  The kernels below take those steps one at a time over
// slot-indexed buffers (slot = position in the CSR), each a separate pass through HBM as a
// tensor-op implementation makes them.  The only addition is the chunking by whole centres,
// which bounds the per-pair buffers: at the 65,536- and 96,241-atom Fe workloads P * c * 4
// bytes would be 474 and 628 GB, more than one GPU holds.
#include "nga_internal.h"
#include "gemm_rows.h"

#include <vector>

namespace nga {

namespace {

constexpr int kPairBlock = 256;
constexpr int64_t kMaxPairGrid = 1 << 18;

template <typename T>
struct Atomics;

// Scatter-max through the integer orderings of the bit patterns: non-negative values order
// as signed integers, negative ones (sign bit set, -0.0 included) in reverse as unsigned
// ones.  The target starts at -inf.
template <>
struct Atomics<float> {
    __device__ static void max(float* a, float v) {
        if (__float_as_int(v) >= 0)
            atomicMax(reinterpret_cast<int*>(a), __float_as_int(v));
        else
            atomicMin(reinterpret_cast<unsigned int*>(a), __float_as_uint(v));
    }
    __device__ static void add(float* a, float v) { unsafeAtomicAdd(a, v); }
    __device__ static float exp(float v) { return expf(v); }
};

template <>
struct Atomics<double> {
    __device__ static void max(double* a, double v) {
        const long long b = __double_as_longlong(v);
        if (b >= 0)
            atomicMax(reinterpret_cast<long long*>(a), b);
        else
            atomicMin(reinterpret_cast<unsigned long long*>(a), (unsigned long long)b);
    }
    __device__ static void add(double* a, double v) { unsafeAtomicAdd(a, v); }
    __device__ static double exp(double v) { return ::exp(v); }
};

inline dim3 pair_grid(int64_t total) {
    int64_t b = (total + kPairBlock - 1) / kPairBlock;
    return dim3((unsigned)(b < 1 ? 1 : (b > kMaxPairGrid ? kMaxPairGrid : b)));
}

#define NGA_GRID_STRIDE(idx, total)                                                            \
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < (total);          \
         idx += (int64_t)gridDim.x * blockDim.x)

template <typename T>
__global__ void fill_kernel(T* p, int64_t n, T v) {
    NGA_GRID_STRIDE(i, n) p[i] = v;
}

// n_i^2 per centre (the pair counts, scanned into pair offsets).
__global__ void pair_counts_kernel(const int64_t* row_ptr, int64_t n_centres, int32_t* counts) {
    NGA_GRID_STRIDE(i, n_centres) {
        const int64_t n = row_ptr[i + 1] - row_ptr[i];
        counts[i] = (int32_t)(n * n);
    }
}

// One work-group per centre of the chunk: its n^2 (query slot, key slot) pairs, query-major,
// at its pair offset relative to the chunk's first pair.
__global__ void enum_pairs_kernel(const int64_t* row_ptr, const int64_t* pair_ptr, int64_t i0,
                                  int32_t* pq, int32_t* pk) {
    const int64_t i = i0 + blockIdx.x;
    const int64_t r0 = row_ptr[i];
    const int n = (int)(row_ptr[i + 1] - r0);
    const int64_t base = pair_ptr[i] - pair_ptr[i0];
    for (int64_t idx = threadIdx.x; idx < (int64_t)n * n; idx += blockDim.x) {
        pq[base + idx] = (int32_t)(r0 + idx / n);
        pk[base + idx] = (int32_t)(r0 + idx % n);
    }
}

// prod[p][t] = q[pq[p]][t] * k[pk[p]][t]
template <typename T>
__global__ void pair_prod_kernel(const T* __restrict__ qkv, int c, const int32_t* __restrict__ pq,
                                 const int32_t* __restrict__ pk, int64_t np, T* __restrict__ prod) {
    NGA_GRID_STRIDE(idx, np * c) {
        const int64_t p = idx / c;
        const int t = (int)(idx - p * c);
        prod[idx] = qkv[(int64_t)pq[p] * 3 * c + t] * qkv[(int64_t)pk[p] * 3 * c + c + t];
    }
}

// s[p][h] = scale * sum of prod[p] over head h's channels; m[pq[p]][h] = max (scatter-max).
template <typename T>
__global__ void pair_scores_kernel(const T* __restrict__ prod, int c, int heads, T scale,
                                   const int32_t* __restrict__ pq, int64_t np, T* __restrict__ s,
                                   T* m) {
    const int d = c / heads;
    NGA_GRID_STRIDE(idx, np * heads) {
        const int64_t p = idx / heads;
        const int h = (int)(idx - p * heads);
        const T* r = prod + p * c + h * d;
        T acc = T(0);
        for (int t = 0; t < d; ++t) acc += r[t];
        acc *= scale;
        s[idx] = acc;
        Atomics<T>::max(&m[(int64_t)pq[p] * heads + h], acc);
    }
}

// e[p][h] = exp(s[p][h] - m[pq[p]][h]) in place of s; z[pq[p]][h] += e (scatter-add).
template <typename T>
__global__ void pair_exp_kernel(T* s, const T* m, T* z, const int32_t* __restrict__ pq, int heads,
                                int64_t np) {
    NGA_GRID_STRIDE(idx, np * heads) {
        const int64_t p = idx / heads;
        const int64_t a = (int64_t)pq[p] * heads + (idx - p * heads);
        const T e = Atomics<T>::exp(s[idx] - m[a]);
        s[idx] = e;
        Atomics<T>::add(&z[a], e);
    }
}

// w[p][h] = e[p][h] / z[pq[p]][h], in place.
template <typename T>
__global__ void pair_weights_kernel(T* s, const T* z, const int32_t* __restrict__ pq, int heads,
                                    int64_t np) {
    NGA_GRID_STRIDE(idx, np * heads) {
        const int64_t p = idx / heads;
        s[idx] = s[idx] / z[(int64_t)pq[p] * heads + (idx - p * heads)];
    }
}

// wv[p][t] = w[p][h(t)] * v[pk[p]][t], over the prod buffer.
template <typename T>
__global__ void pair_wv_kernel(const T* __restrict__ qkv, int c, int heads,
                               const T* __restrict__ w, const int32_t* __restrict__ pk,
                               int64_t np, T* __restrict__ wv) {
    const int d = c / heads;
    NGA_GRID_STRIDE(idx, np * c) {
        const int64_t p = idx / c;
        const int t = (int)(idx - p * c);
        wv[idx] = w[p * heads + t / d] * qkv[(int64_t)pk[p] * 3 * c + 2 * c + t];
    }
}

// o[pq[p]][t] += wv[p][t]  (index_add).
template <typename T>
__global__ void index_add_kernel(const T* __restrict__ wv, int c, const int32_t* __restrict__ pq,
                                 int64_t np, T* o) {
    NGA_GRID_STRIDE(idx, np * c) {
        const int64_t p = idx / c;
        Atomics<T>::add(&o[(int64_t)pq[p] * c + (idx - p * c)], wv[idx]);
    }
}

#undef NGA_GRID_STRIDE

struct PairWs {
    void* qkv;
    void* o;
    void* xbuf;
    void* m;
    void* z;
    int32_t* counts;
    int64_t* tile_sums;
    int64_t* pair_ptr;
    int32_t* pq;
    int32_t* pk;
    void* prod;
    void* s;
    size_t bytes;
};

PairWs carve_pair(void* ws, int64_t n_centres, int64_t e, int c, int heads, int layers,
                  int64_t chunk, size_t es) {
    Carver cv(ws);
    PairWs w;
    w.qkv = cv.take<char>((size_t)e * 3 * c * es);
    w.o = cv.take<char>((size_t)e * c * es);
    w.xbuf = cv.take<char>(layers > 1 ? (size_t)e * c * es : 0);
    w.m = cv.take<char>((size_t)e * heads * es);
    w.z = cv.take<char>((size_t)e * heads * es);
    w.counts = cv.take<int32_t>((size_t)n_centres);
    w.tile_sums = cv.take<int64_t>((size_t)scan_tiles(n_centres));
    w.pair_ptr = cv.take<int64_t>((size_t)n_centres + 1);
    w.pq = cv.take<int32_t>((size_t)chunk);
    w.pk = cv.take<int32_t>((size_t)chunk);
    w.prod = cv.take<char>((size_t)chunk * c * es);
    w.s = cv.take<char>((size_t)chunk * heads * es);
    w.bytes = cv.off;
    return w;
}

struct Chunk {
    int64_t i0, i1, np;
};

template <typename T>
int run_pair(const int64_t* row_ptr, const int32_t* order, const std::vector<Chunk>& chunks,
             int64_t n_centres, int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
             const T* weights, const T* x, T* y, const PairWs& w, uint32_t* status,
             hipStream_t s) {
    int rc;
    // Pair offsets on the device, from the same row_ptr the chunks were planned from.
    hipLaunchKernelGGL(pair_counts_kernel, pair_grid(n_centres), dim3(kPairBlock), 0, s, row_ptr,
                       n_centres, w.counts);
    if ((rc = last_launch_status())) return rc;
    if ((rc = scan_counts(w.counts, n_centres, INT32_MAX, w.tile_sums, w.pair_ptr, s))) return rc;

    T* qkv = static_cast<T*>(w.qkv);
    T* o = static_cast<T*>(w.o);
    T* xbuf = static_cast<T*>(w.xbuf);
    T* m = static_cast<T*>(w.m);
    T* z = static_cast<T*>(w.z);
    T* prod = static_cast<T*>(w.prod);
    T* sc = static_cast<T*>(w.s);
    const int64_t* e_dev = row_ptr + n_centres;
    const size_t cc = (size_t)c * c;
    const int d = c / heads;
    const T scale = T(1) / std::sqrt(T(d));
    for (int l = 0; l < layers; ++l) {
        const T* W = weights + (size_t)l * 4 * cc;
        GemmArgs<T> g1;
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
        hipLaunchKernelGGL((fill_kernel<T>), pair_grid(n_edges * heads), dim3(kPairBlock), 0, s, m,
                           n_edges * heads, T(-INFINITY));
        hipLaunchKernelGGL((fill_kernel<T>), pair_grid(n_edges * heads), dim3(kPairBlock), 0, s, z,
                           n_edges * heads, T(0));
        hipLaunchKernelGGL((fill_kernel<T>), pair_grid(n_edges * c), dim3(kPairBlock), 0, s, o,
                           n_edges * c, T(0));
        if ((rc = last_launch_status())) return rc;
        for (const Chunk& ch : chunks) {
            const int64_t np = ch.np;
            hipLaunchKernelGGL(enum_pairs_kernel, dim3((unsigned)(ch.i1 - ch.i0)), dim3(kPairBlock),
                               0, s, row_ptr, w.pair_ptr, ch.i0, w.pq, w.pk);
            hipLaunchKernelGGL((pair_prod_kernel<T>), pair_grid(np * c), dim3(kPairBlock), 0, s,
                               qkv, c, w.pq, w.pk, np, prod);
            hipLaunchKernelGGL((pair_scores_kernel<T>), pair_grid(np * heads), dim3(kPairBlock), 0,
                               s, prod, c, heads, scale, w.pq, np, sc, m);
            hipLaunchKernelGGL((pair_exp_kernel<T>), pair_grid(np * heads), dim3(kPairBlock), 0, s,
                               sc, m, z, w.pq, heads, np);
            hipLaunchKernelGGL((pair_weights_kernel<T>), pair_grid(np * heads), dim3(kPairBlock), 0,
                               s, sc, z, w.pq, heads, np);
            hipLaunchKernelGGL((pair_wv_kernel<T>), pair_grid(np * c), dim3(kPairBlock), 0, s, qkv,
                               c, heads, sc, w.pk, np, prod);
            hipLaunchKernelGGL((index_add_kernel<T>), pair_grid(np * c), dim3(kPairBlock), 0, s,
                               prod, c, w.pq, np, o);
            if ((rc = last_launch_status())) return rc;
        }
        GemmArgs<T> g2 = g1;
        g2.a = o;
        g2.a_rows = nullptr;
        g2.w = W + 3 * cc;
        g2.nmat = 1;
        g2.lda = c;
        g2.ldo = c;
        const bool last = (l == layers - 1);
        g2.out = last ? y : xbuf;
        g2.out_rows = last ? order : nullptr;
        if ((rc = launch_gemm(g2, n_edges, s))) return rc;
    }
    return NGA_OK;
}

bool pair_args_ok(int64_t n_centres, int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                  int64_t pair_chunk) {
    return n_centres >= 0 && n_centres < INT32_MAX && n_edges >= 0 && n_edges < INT32_MAX &&
           c >= 1 && heads >= 1 && c % heads == 0 && layers >= 1 && pair_chunk >= 1 &&
           pair_chunk <= INT32_MAX;
}

}  // namespace

}  // namespace nga

extern "C" size_t pair_attn_workspace_bytes(int dtype, int64_t n_centres, int64_t n_edges,
                                            int32_t c, int32_t n_heads, int32_t n_layers,
                                            int64_t pair_chunk) {
    if (dtype != NGA_F64 && dtype != NGA_F32) return 0;
    if (!nga::pair_args_ok(n_centres, n_edges, c, n_heads, n_layers, pair_chunk)) return 0;
    const size_t es = dtype == NGA_F64 ? sizeof(double) : sizeof(float);
    return nga::carve_pair(nullptr, n_centres, n_edges, c, n_heads, n_layers, pair_chunk, es).bytes;
}

extern "C" int pair_attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order,
                                 int64_t n_centres, int64_t n_edges, int32_t c, int32_t n_heads,
                                 int32_t n_layers, const void* weights, const void* x, void* y,
                                 int64_t pair_chunk, void* ws, size_t ws_bytes, void* stream) {
    using namespace nga;
    if (dtype != NGA_F64 && dtype != NGA_F32) return NGA_EDTYPE;
    if (!pair_args_ok(n_centres, n_edges, c, n_heads, n_layers, pair_chunk)) return NGA_EINVAL;
    if (!row_ptr) return NGA_EINVAL;
    if (n_edges > 0 && (!x || !y || !weights)) return NGA_EINVAL;
    const size_t es = dtype == NGA_F64 ? sizeof(double) : sizeof(float);
    if (n_edges > 0) {
        const char* xb = static_cast<const char*>(x);
        const char* yb = static_cast<const char*>(y);
        const size_t span = (size_t)n_edges * c * es;
        if (xb < yb + span && yb < xb + span) return NGA_EINVAL;
    }
    const size_t need =
        pair_attn_workspace_bytes(dtype, n_centres, n_edges, c, n_heads, n_layers, pair_chunk);
    if (!ws || ws_bytes < need) return NGA_EWORKSPACE;
    if (n_centres == 0 || n_edges == 0) return NGA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // Plan: read row_ptr back and cut the centres into chunks of at most pair_chunk pairs.
    std::vector<int64_t> hrp((size_t)n_centres + 1);
    int rc = hip_status(hipMemcpyAsync(hrp.data(), row_ptr, hrp.size() * sizeof(int64_t),
                                       hipMemcpyDeviceToHost, s));
    if (rc) return rc;
    if ((rc = hip_status(hipStreamSynchronize(s)))) return rc;
    if (hrp[0] != 0 || hrp[n_centres] > n_edges) return NGA_ECAP;
    std::vector<Chunk> chunks;
    Chunk cur{0, 0, 0};
    for (int64_t i = 0; i < n_centres; ++i) {
        const int64_t n = hrp[i + 1] - hrp[i];
        if (n < 0) return NGA_ECAP;
        const int64_t pairs = n * n;
        if (pairs > pair_chunk) return NGA_EINVAL;
        if (cur.np + pairs > pair_chunk) {
            chunks.push_back(cur);
            cur = Chunk{i, i, 0};
        }
        cur.i1 = i + 1;
        cur.np += pairs;
    }
    if (cur.i1 > cur.i0) chunks.push_back(cur);

    PairWs w = carve_pair(ws, n_centres, n_edges, c, n_heads, n_layers, pair_chunk, es);
    uint32_t* status = &static_cast<WsHeader*>(ws)->status;
    if (dtype == NGA_F64)
        return run_pair<double>(row_ptr, order, chunks, n_centres, n_edges, c, n_heads, n_layers,
                                static_cast<const double*>(weights),
                                static_cast<const double*>(x), static_cast<double*>(y), w, status,
                                s);
    return run_pair<float>(row_ptr, order, chunks, n_centres, n_edges, c, n_heads, n_layers,
                           static_cast<const float*>(weights), static_cast<const float*>(x),
                           static_cast<float*>(y), w, status, s);
}
