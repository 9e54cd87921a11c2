// block_attn_forward: block-dense multi-head neighbour attention through the destination CSR.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense and OOM-prone --
// move to block-dense attention via the destination CSR", section "Proposed fix: block-dense
// attention on the graph": gather each centre's (nnei, c) block through the destination CSR,
// run dense attention math with per-row masks for the ragged tail, scatter back to the edge
// axis, so the P = sum nnei^2 pair axis never exists.  Section "Graph-native alternatives":
// the attention is self-attention among one centre's edges, destination_row_ptr being the
// segment offsets.
//
// This file holds the host entry point and the path that works for any shape: three
// kernels per layer over slot-indexed workspace buffers (slot = position in the CSR):
//   qkv[s]  = x[order(s)] [Wq | Wk | Wv]           (row-gather GEMM)
//   o[s]    = per-centre attention of qkv rows      (one work-group per centre)
//   y[order(s)] = o[s] Wo                           (row-scatter GEMM)
// The fused fp32 kernel for 16-wide heads lives in block_attn_f32.hip (its f16 split-pair
// variant, dtype NGA_F32_SPLIT16, in block_attn_fused.hip), the fp64 kernels in
// block_attn_f64_fused.hip and block_attn_f64.hip; this path covers every other shape.
#include "nga_internal.h"
#include "block_attn_f64.h"
#include "block_attn_fused.h"
#include "gemm_rows.h"

namespace nga {

namespace {

template <typename T>
__device__ inline T exp_t(T v);
template <>
__device__ inline double exp_t<double>(double v) { return exp(v); }
template <>
__device__ inline float exp_t<float>(float v) { return expf(v); }

template <typename T>
struct CoreArgs {
    const T* qkv;  // [E][3c] slot-indexed: q | k | v
    T* o;          // [E][c] slot-indexed
    const int64_t* row_ptr;
    int n_centres;
    int64_t n_edges;
    int nnei_cap;
    int c;
    int heads;
    int d;
    T scale;
    const T* ldt;          // smooth attention: this layer's ln D~ [n_edges][heads], or NULL
    const int32_t* order;  // edge row of each slot (NULL: the slot itself), for ldt
    uint32_t* status;
};

// One work-group per centre; each thread owns (query row a, head h) pairs and streams the
// centre's keys once, in tiles of kCoreKeys, with the online-softmax recurrence ([P2]
// "Graph-native alternatives": a running max and denominator over bounded tiles, memory
// O(E c)): per tile the scores, the tile max, a rescale of the running sum and weighted
// values when the max grows, then exp / sum / weighted values.  Rows of any length.
constexpr int kCoreKeys = 16;

template <typename T, int DMAX>
__global__ void __launch_bounds__(256) attn_core_kernel(CoreArgs<T> A) {
    const int i = blockIdx.x;
    const int64_t r0 = A.row_ptr[i], r1 = A.row_ptr[i + 1];
    // A decreasing row_ptr, or a row outside [0, n_edges), is reported and the row skipped.
    if (r0 < 0 || r1 < r0 || r1 > A.n_edges || r1 - r0 > A.nnei_cap) {
        if (threadIdx.x == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int n = (int)(r1 - r0);
    if (n == 0) return;
    const int c = A.c, c3 = 3 * A.c, d = A.d;
    for (int idx = threadIdx.x; idx < n * A.heads; idx += blockDim.x) {
        const int a = idx / A.heads, h = idx % A.heads;
        const T* q = A.qkv + (r0 + a) * c3 + h * d;
        T qr[DMAX];
#pragma unroll
        for (int t = 0; t < DMAX; ++t) qr[t] = t < d ? q[t] * A.scale : T(0);
        T m = -INFINITY, z = T(0);
        T acc[DMAX];
#pragma unroll
        for (int t = 0; t < DMAX; ++t) acc[t] = T(0);
        for (int b0 = 0; b0 < n; b0 += kCoreKeys) {
            const int nb = n - b0 < kCoreKeys ? n - b0 : kCoreKeys;
            T s[kCoreKeys];
            T mt = -INFINITY;
#pragma unroll
            for (int k = 0; k < kCoreKeys; ++k) {
                s[k] = -INFINITY;
                if (k < nb) {
                    const T* kb = A.qkv + (r0 + b0 + k) * c3 + c + h * d;
                    T v = T(0);
#pragma unroll
                    for (int t = 0; t < DMAX; ++t)
                        if (t < d) v += qr[t] * kb[t];
                    s[k] = v;
                    mt = v > mt ? v : mt;
                }
            }
            if (mt > m) {  // the running max grows: rescale what was summed so far
                const T alpha = exp_t<T>(m - mt);  // 0 for the first tile
                z *= alpha;
#pragma unroll
                for (int t = 0; t < DMAX; ++t) acc[t] *= alpha;
                m = mt;
            }
#pragma unroll
            for (int k = 0; k < kCoreKeys; ++k) {
                if (k < nb) {
                    const T* vb = A.qkv + (r0 + b0 + k) * c3 + 2 * c + h * d;
                    const T p = exp_t<T>(s[k] - m);
                    z += p;
#pragma unroll
                    for (int t = 0; t < DMAX; ++t)
                        if (t < d) acc[t] += p * vb[t];
                }
            }
        }
        T* out = A.o + (r0 + a) * c + h * d;
        // Smooth attention: sum_j e_j / D~ times the softmax = exp(s_j - ln D~), i.e. the
        // weighted sum times exp(m - ln D~) in place of 1/Z.
        T f = T(0);
        if (A.ldt) {
            const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
            if (row >= 0 && row < A.n_edges) f = exp_t<T>(m - A.ldt[row * A.heads + h]);
        }
#pragma unroll
        for (int t = 0; t < DMAX; ++t)
            if (t < d) out[t] = A.ldt ? acc[t] * f : acc[t] / z;
    }
}

__global__ void check_rows_kernel(const int64_t* row_ptr, int n_centres, int64_t n_edges,
                                  uint32_t* status) {
    if (row_ptr[n_centres] > n_edges || row_ptr[0] != 0) raise_bits(status, kBitCap);
}

struct GenericWs {
    void* qkv;
    void* o;
    void* xbuf;
    size_t bytes;
};

GenericWs carve_generic(void* ws, int64_t e, int c, int layers, size_t es) {
    Carver cv(ws);
    GenericWs w;
    w.qkv = cv.take<char>((size_t)e * 3 * c * es);
    w.o = cv.take<char>((size_t)e * c * es);
    w.xbuf = cv.take<char>(layers > 1 ? (size_t)e * c * es : 0);
    w.bytes = cv.off;
    return w;
}

template <typename T>
int launch_core(const CoreArgs<T>& A, hipStream_t s) {
    dim3 grid((unsigned)A.n_centres), block(256);
    if (A.d <= 8) hipLaunchKernelGGL((attn_core_kernel<T, 8>), grid, block, 0, s, A);
    else if (A.d <= 16) hipLaunchKernelGGL((attn_core_kernel<T, 16>), grid, block, 0, s, A);
    else if (A.d <= 32) hipLaunchKernelGGL((attn_core_kernel<T, 32>), grid, block, 0, s, A);
    else if (A.d <= 64) hipLaunchKernelGGL((attn_core_kernel<T, 64>), grid, block, 0, s, A);
    else hipLaunchKernelGGL((attn_core_kernel<T, 128>), grid, block, 0, s, A);
    return last_launch_status();
}

template <typename T>
int run_generic(const int64_t* row_ptr, const int32_t* order, int64_t n_centres, int64_t n_edges,
                int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers, const T* weights,
                const T* x, const T* ldt, T* y, void* ws, hipStream_t s) {
    GenericWs w = carve_generic(ws, n_edges, c, layers, sizeof(T));
    uint32_t* status = &static_cast<WsHeader*>(ws)->status;
    const int64_t* e_dev = row_ptr + n_centres;
    T* qkv = static_cast<T*>(w.qkv);
    T* o = static_cast<T*>(w.o);
    T* xbuf = static_cast<T*>(w.xbuf);
    const int d = c / heads;
    const size_t cc = (size_t)c * c;
    int rc;
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
        CoreArgs<T> A;
        A.qkv = qkv;
        A.o = o;
        A.row_ptr = row_ptr;
        A.n_centres = (int)n_centres;
        A.n_edges = n_edges;
        A.nnei_cap = nnei_cap;
        A.c = c;
        A.heads = heads;
        A.d = d;
        A.scale = T(1) / std::sqrt(T(d));
        A.ldt = ldt ? ldt + (size_t)l * n_edges * heads : nullptr;
        A.order = order;
        A.status = status;
        if ((rc = launch_core(A, s))) return rc;
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

// The f16 split-pair arithmetic exists only as the fused kernel for its shapes.
bool use_split16(int dtype, int32_t nnei_cap, int32_t c, int32_t heads) {
    return fused_supported(dtype, nnei_cap, c, heads);
}

bool use_f32_fused(int dtype, int32_t nnei_cap, int32_t c, int32_t heads) {
    return dtype == NGA_F32 && f32_fused_supported(nnei_cap, c, heads);
}

bool known_dtype(int dtype) {
    return dtype == NGA_F64 || dtype == NGA_F32 || dtype == NGA_F32_SPLIT16;
}

}  // namespace

}  // namespace nga

extern "C" size_t block_attn_workspace_bytes(int dtype, int64_t n_edges, int32_t nnei_cap,
                                             int32_t c, int32_t n_heads, int32_t n_layers) {
    if (!nga::known_dtype(dtype)) return 0;
    if (n_edges < 0 || c < 1 || n_heads < 1 || n_layers < 1 || nnei_cap < 1) return 0;
    if (dtype == NGA_F32_SPLIT16) {
        if (!nga::use_split16(dtype, nnei_cap, c, n_heads)) return 0;
        nga::Carver cv(nullptr);
        cv.take<float>(nga::fused_workspace_floats(c, n_layers));
        return cv.off;
    }
    if (nga::use_f32_fused(dtype, nnei_cap, c, n_heads)) {
        nga::Carver cv(nullptr);
        cv.take<float>(nga::f32_fused_workspace_floats(c, n_layers));
        return cv.off;
    }
    if (dtype == NGA_F64 && nga::fused_f64_supported(nnei_cap, c, n_heads))
        return nga::Carver(nullptr).off;  // the status word only
    const size_t es = dtype == NGA_F64 ? sizeof(double) : sizeof(float);
    return nga::carve_generic(nullptr, n_edges, c, n_layers, es).bytes;
}

extern "C" const char* nga_attn_variant(int dtype, int32_t nnei_cap, int32_t c, int32_t n_heads) {
    if (!nga::known_dtype(dtype)) return "unsupported";
    if (dtype == NGA_F32_SPLIT16)
        return nga::use_split16(dtype, nnei_cap, c, n_heads) ? nga::fused_name(dtype, c, n_heads)
                                                             : "unsupported";
    if (nga::use_f32_fused(dtype, nnei_cap, c, n_heads)) return "fused_f32";
    if (dtype == NGA_F64 && nga::fused_f64_supported(nnei_cap, c, n_heads)) return "fused_f64";
    if (dtype == NGA_F64 && nga::f64_mfma_supported(nnei_cap, c, n_heads)) return "mfma_f64";
    return dtype == NGA_F64 ? "generic_f64" : "generic_f32";
}

namespace nga {
// block_attn_f64.hip: true if the fp64 matrix-core path runs the attention core and the output
// projection as one work-group per centre (c = 128, heads of 16 or 32, enough centres to fill
// the current device's compute units in every round) rather than per (centre, head) followed
// by a row GEMM.
bool f64_core_wo_selected(int64_t n_centres, int32_t c, int32_t heads);
}  // namespace nga

extern "C" const char* nga_attn_plan(int dtype, int64_t n_centres, int32_t nnei_cap, int32_t c,
                                     int32_t n_heads) {
    const char* v = nga_attn_variant(dtype, nnei_cap, c, n_heads);
    if (dtype == NGA_F64 && nga::f64_mfma_supported(nnei_cap, c, n_heads) &&
        !nga::fused_f64_supported(nnei_cap, c, n_heads))
        return nga::f64_core_wo_selected(n_centres, c, n_heads) ? "mfma_f64.merged"
                                                                : "mfma_f64.per_head";
    return v;
}

namespace nga {
namespace {

int attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                 int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t n_heads, int32_t n_layers,
                 const void* weights, const void* x, const void* ldt, void* y, void* ws,
                 size_t ws_bytes, void* stream) {
    if (!known_dtype(dtype)) return NGA_EDTYPE;
    if (n_centres < 0 || n_centres >= INT32_MAX || n_edges < 0 || nnei_cap < 1 || c < 1 ||
        n_heads < 1 || c % n_heads != 0 || n_layers < 1)
        return NGA_EINVAL;
    if (c / n_heads > 128) return NGA_EINVAL;
    // The split-pair arithmetic has no kernel outside its shapes.
    if (dtype == NGA_F32_SPLIT16 && !use_split16(dtype, nnei_cap, c, n_heads)) return NGA_EDTYPE;
    if (!row_ptr) return NGA_EINVAL;
    if (n_edges > 0 && (!x || !y || !weights)) return NGA_EINVAL;
    const size_t es = dtype == NGA_F64 ? sizeof(double) : sizeof(float);
    if (n_edges > 0) {
        const char* xb = static_cast<const char*>(x);
        const char* yb = static_cast<const char*>(y);
        const size_t span = (size_t)n_edges * c * es;
        if (xb < yb + span && yb < xb + span) return NGA_EINVAL;
    }
    const size_t need = block_attn_workspace_bytes(dtype, n_edges, nnei_cap, c, n_heads, n_layers);
    if (!ws || ws_bytes < need) return NGA_EWORKSPACE;
    if (n_centres == 0 || n_edges == 0) return NGA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* status = &static_cast<WsHeader*>(ws)->status;
    if (use_f32_fused(dtype, nnei_cap, c, n_heads)) {  // the fused kernel checks row_ptr itself
        Carver cv(ws);
        float* packed = cv.take<float>(f32_fused_workspace_floats(c, n_layers));
        return run_f32_fused(row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads, n_layers,
                             static_cast<const float*>(weights), static_cast<const float*>(x),
                             static_cast<const float*>(ldt), static_cast<float*>(y), packed,
                             status, s);
    }
    if (dtype == NGA_F32_SPLIT16) {  // the fused kernel checks row_ptr itself
        Carver cv(ws);
        float* packed = cv.take<float>(fused_workspace_floats(c, n_layers));
        return run_fused(dtype, row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads, n_layers,
                         weights, x, ldt, y, packed, status, s);
    }
    if (dtype == NGA_F64 && fused_f64_supported(nnei_cap, c, n_heads))  // checks row_ptr itself
        return run_fused_f64(row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads, n_layers,
                             static_cast<const double*>(weights), static_cast<const double*>(x),
                             static_cast<const double*>(ldt), static_cast<double*>(y), status, s);
    if (dtype == NGA_F64 && f64_mfma_supported(nnei_cap, c, n_heads)) {  // its core checks row_ptr
        GenericWs w = carve_generic(ws, n_edges, c, n_layers, sizeof(double));
        return run_f64_mfma(row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads, n_layers,
                            static_cast<const double*>(weights), static_cast<const double*>(x),
                            static_cast<const double*>(ldt), static_cast<double*>(y),
                            static_cast<double*>(w.qkv),
                            static_cast<double*>(w.o), static_cast<double*>(w.xbuf), status, s);
    }
    hipLaunchKernelGGL(check_rows_kernel, dim3(1), dim3(1), 0, s, row_ptr, (int)n_centres, n_edges,
                       status);
    if (int rc = last_launch_status()) return rc;
    if (dtype == NGA_F64)
        return run_generic<double>(row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads,
                                   n_layers, static_cast<const double*>(weights),
                                   static_cast<const double*>(x), static_cast<const double*>(ldt),
                                   static_cast<double*>(y), ws, s);
    return run_generic<float>(row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads, n_layers,
                              static_cast<const float*>(weights), static_cast<const float*>(x),
                              static_cast<const float*>(ldt), static_cast<float*>(y), ws, s);
}

}  // namespace
}  // namespace nga

extern "C" int block_attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order,
                                  int64_t n_centres, int64_t n_edges, int32_t nnei_cap,
                                  int32_t c, int32_t n_heads, int32_t n_layers,
                                  const void* weights, const void* x, void* y, void* ws,
                                  size_t ws_bytes, void* stream) {
    return nga::attn_forward(dtype, row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads,
                             n_layers, weights, x, nullptr, y, ws, ws_bytes, stream);
}

extern "C" int block_attn_forward_smooth(int dtype, const int64_t* row_ptr, const int32_t* order,
                                         int64_t n_centres, int64_t n_edges, int32_t nnei_cap,
                                         int32_t c, int32_t n_heads, int32_t n_layers,
                                         const void* weights, const void* x,
                                         const void* log_dtilde, void* y, void* ws,
                                         size_t ws_bytes, void* stream) {
    if (n_edges > 0 && !log_dtilde) return NGA_EINVAL;
    return nga::attn_forward(dtype, row_ptr, order, n_centres, n_edges, nnei_cap, c, n_heads,
                             n_layers, weights, x, log_dtilde, y, ws, ws_bytes, stream);
}
