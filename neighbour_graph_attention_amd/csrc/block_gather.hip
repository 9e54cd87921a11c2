// block_gather / block_scatter: the padded per-centre block of the destination CSR and its
// scatter back to the edge axis, as standalone copies.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense and OOM-prone --
// move to block-dense attention via the destination CSR", section "Proposed fix: block-dense
// attention on the graph": gather per-centre (nloc, nnei_max, c) blocks through the
// destination CSR, run dense math on them, scatter back to the edge axis.  The fused attention
// kernels never materialise that block; these two calls do, so that the raggedness boundary
// can be measured (HBM rate) and inspected on its own.
//
// Both are pure HBM streams.  One work-group per centre; each thread moves 16-byte (or 8- or
// 4-byte, when a row's bytes are not a multiple of 16) vectors, issuing U loads before any of
// their stores.  Without `order` a centre's rows are one contiguous run of the edge axis and
// its block is one contiguous run of the output, so both sides are fully coalesced.
#include "nga_internal.h"

namespace nga {

namespace {

struct GatherArgs {
    const int64_t* row_ptr;
    const int32_t* order;
    int64_t n_centres;
    int64_t n_edges;
    int cap;
    int vpr;       // vectors per feature row
    int vpr_log2;  // log2(vpr) when vpr is a power of two, else -1
    const void* src;
    void* dst;
    uint32_t* status;
};

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

// Row k and column v of vector index idx within a centre.
__device__ inline void split_index(int idx, const GatherArgs& A, int& k, int& v) {
    if (A.vpr_log2 >= 0) {
        k = idx >> A.vpr_log2;
        v = idx & (A.vpr - 1);
    } else {
        k = idx / A.vpr;
        v = idx - k * A.vpr;
    }
}

// Rows of one centre: r0 .. r1-1 of the edge axis.  False (and the error reported) if the
// CSR is malformed here: a decreasing row_ptr, a row outside [0, n_edges) or one over cap.
__device__ inline bool centre_rows(const GatherArgs& A, int64_t i, int64_t& r0, int& n) {
    if (i == 0 && threadIdx.x == 0 &&
        (A.row_ptr[0] != 0 || A.row_ptr[A.n_centres] > A.n_edges))
        raise_bits(A.status, kBitCap);
    r0 = A.row_ptr[i];
    const int64_t r1 = A.row_ptr[i + 1];
    if (r1 < r0 || r0 < 0 || r1 > A.n_edges || r1 - r0 > A.cap) {
        if (threadIdx.x == 0) raise_bits(A.status, kBitCap);
        return false;
    }
    n = (int)(r1 - r0);
    return true;
}

// block[i][k] = x[e_k] for k < n_i, 0 for n_i <= k < cap.
template <typename V>
__global__ void __launch_bounds__(kGatherThreads) block_gather_kernel(GatherArgs A) {
    const int64_t i = blockIdx.x;
    int64_t r0;
    int n;
    const int total = A.cap * A.vpr;
    V* out = static_cast<V*>(A.dst) + i * (int64_t)total;
    const V zero = {};
    if (!centre_rows(A, i, r0, n)) {
        // The block of a malformed row is zero-filled, so no output stays stale.
        for (int idx = threadIdx.x; idx < total; idx += kGatherThreads) out[idx] = zero;
        return;
    }
    const V* x = static_cast<const V*>(A.src);
    const int nv = n * A.vpr;
    bool bad = false;
    for (int base = threadIdx.x; base < total; base += kGatherThreads * kGatherUnroll) {
        V v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int idx = base + u * kGatherThreads;
            v[u] = zero;
            if (idx < nv) {
                int k, c;
                split_index(idx, A, k, c);
                const int64_t row = A.order ? (int64_t)A.order[r0 + k] : r0 + k;
                if (row >= 0 && row < A.n_edges)
                    v[u] = x[row * A.vpr + c];
                else
                    bad = true;
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int idx = base + u * kGatherThreads;
            if (idx < total) out[idx] = v[u];
        }
    }
    if (bad) raise_bits(A.status, kBitIndex);
}

// y[e_k] = block[i][k] for k < n_i; padding rows are not read.
template <typename V>
__global__ void __launch_bounds__(kGatherThreads) block_scatter_kernel(GatherArgs A) {
    const int64_t i = blockIdx.x;
    int64_t r0;
    int n;
    if (!centre_rows(A, i, r0, n)) return;
    const V* in = static_cast<const V*>(A.src) + i * (int64_t)(A.cap * A.vpr);
    V* y = static_cast<V*>(A.dst);
    const int nv = n * A.vpr;
    bool bad = false;
    for (int base = threadIdx.x; base < nv; base += kGatherThreads * kGatherUnroll) {
        V v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int idx = base + u * kGatherThreads;
            if (idx < nv) v[u] = in[idx];
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int idx = base + u * kGatherThreads;
            if (idx < nv) {
                int k, c;
                split_index(idx, A, k, c);
                const int64_t row = A.order ? (int64_t)A.order[r0 + k] : r0 + k;
                if (row >= 0 && row < A.n_edges)
                    y[row * A.vpr + c] = v[u];
                else
                    bad = true;
            }
        }
    }
    if (bad) raise_bits(A.status, kBitIndex);
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

int run_copy(bool gather, int dtype, const int64_t* row_ptr, const int32_t* order,
             int64_t n_centres, int64_t n_edges, int32_t cap, int32_t c, const void* src,
             void* dst, void* ws, size_t ws_bytes, void* stream) {
    if (dtype != NGA_F64 && dtype != NGA_F32) return NGA_EDTYPE;
    if (n_centres < 0 || n_centres >= INT32_MAX || n_edges < 0 || cap < 1 || c < 1)
        return NGA_EINVAL;
    const int64_t row_bytes = (int64_t)c * (dtype == NGA_F64 ? 8 : 4);
    if ((int64_t)cap * row_bytes / 4 >= INT32_MAX) return NGA_EINVAL;  // vector indices per centre
    if (!ws || ws_bytes < sizeof(WsHeader)) return NGA_EWORKSPACE;
    if (n_centres == 0) return NGA_OK;
    if (!row_ptr || !src || !dst) return NGA_EINVAL;
    {  // the edge-axis array and the block must not overlap
        const size_t edge_span = (size_t)n_edges * row_bytes;
        const size_t block_span = (size_t)n_centres * cap * row_bytes;
        const char* a = static_cast<const char*>(src);
        const char* b = static_cast<const char*>(dst);
        const size_t sa = gather ? edge_span : block_span, sb = gather ? block_span : edge_span;
        if (a < b + sb && b < a + sa) return NGA_EINVAL;
    }
    const int vb = row_bytes % 16 == 0 ? 16 : row_bytes % 8 == 0 ? 8 : 4;
    GatherArgs A;
    A.row_ptr = row_ptr;
    A.order = order;
    A.n_centres = n_centres;
    A.n_edges = n_edges;
    A.cap = cap;
    A.vpr = (int)(row_bytes / vb);
    A.vpr_log2 = (A.vpr & (A.vpr - 1)) == 0 ? __builtin_ctz((unsigned)A.vpr) : -1;
    A.src = src;
    A.dst = dst;
    A.status = &static_cast<WsHeader*>(ws)->status;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)n_centres), block(kGatherThreads);
    if (gather) {
        if (vb == 16) hipLaunchKernelGGL(block_gather_kernel<v4f>, grid, block, 0, s, A);
        else if (vb == 8) hipLaunchKernelGGL(block_gather_kernel<v2f>, grid, block, 0, s, A);
        else hipLaunchKernelGGL(block_gather_kernel<float>, grid, block, 0, s, A);
    } else {
        if (vb == 16) hipLaunchKernelGGL(block_scatter_kernel<v4f>, grid, block, 0, s, A);
        else if (vb == 8) hipLaunchKernelGGL(block_scatter_kernel<v2f>, grid, block, 0, s, A);
        else hipLaunchKernelGGL(block_scatter_kernel<float>, grid, block, 0, s, A);
    }
    return last_launch_status();
}

}  // namespace

}  // namespace nga

extern "C" int block_gather(int dtype, const int64_t* row_ptr, const int32_t* order,
                            int64_t n_centres, int64_t n_edges, int32_t nnei_cap, int32_t c,
                            const void* x, void* block, void* ws, size_t ws_bytes, void* stream) {
    return nga::run_copy(true, dtype, row_ptr, order, n_centres, n_edges, nnei_cap, c, x, block,
                         ws, ws_bytes, stream);
}

extern "C" int block_scatter(int dtype, const int64_t* row_ptr, const int32_t* order,
                             int64_t n_centres, int64_t n_edges, int32_t nnei_cap, int32_t c,
                             const void* block, void* y, void* ws, size_t ws_bytes,
                             void* stream) {
    return nga::run_copy(false, dtype, row_ptr, order, n_centres, n_edges, nnei_cap, c, block, y,
                         ws, ws_bytes, stream);
}
