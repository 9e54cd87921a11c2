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

#include <algorithm>
#include <type_traits>

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

// Scores of the four-head kernel are kept in base-2 units in fp32 (R scaled by log2 e, so the
// softmax exponentials are single v_exp_f32), in natural units in fp64.  `lead` bounds how far
// a later chunk's score may exceed the running shift before the shift is raised: weights up
// to 2^30 (fp32) or e^20 (fp64) leave every sum far from overflow and lose no relative
// precision, and a centre's shift then rarely changes after its first chunk.
template <typename T>
struct Base2;
template <>
struct Base2<float> {
    static constexpr float scale = 1.4426950408889634f;
    static constexpr float lead = 30.0f;
    __device__ static float ex(float v) { return __builtin_amdgcn_exp2f(v); }
};
template <>
struct Base2<double> {
    static constexpr double scale = 1.0;
    static constexpr double lead = 20.0;
    __device__ static double ex(double v) { return exp(v); }
};

// A value all lanes hold alike, moved to scalar registers.
__device__ inline int64_t uniform64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

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

// Position of a work-group in its sequence of chunk tasks: centre i (rows r0 .. r0+n-1 of the
// CSR) and the chunk starting at its row j0.  i >= n_centres ends the sequence.
struct LocalTask {
    int64_t i, r0, n, j0;
};

// Lane value of the quad partner (this lane xor 1 or xor 2): a DPP quad permutation.
template <int X>
__device__ inline float quad_xor(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 X == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true));
}
template <int X>
__device__ inline double quad_xor(double v) {
    int2 b = __builtin_bit_cast(int2, v);
    b.x = __builtin_amdgcn_update_dpp(0, b.x, X == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true);
    b.y = __builtin_amdgcn_update_dpp(0, b.y, X == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true);
    return __builtin_bit_cast(double, b);
}

// The streaming pass for four heads and rows of CV 16-byte vectors (CV = 4, 8 or 16: c = 16,
// 32 or 64 in fp32, 8, 16 or 32 in fp64), as a persistent kernel.  Work-group b takes centres
// b, b + G, b + 2G, ... (G work-groups, as many as the device holds at once); its chunks of up
// to 64 rows follow one another across those centres, and the next chunk's loads are in
// flight, in registers, while the current one is processed.  Chunks alternate between two LDS
// buffers, each row is read from LDS once per step for all four heads, and a chunk takes two
// barriers:
//   scores    four threads per row (row tid / 4, quarter tid % 4 of its vectors) form partial
//             dot products against R_0 .. R_3; two DPP exchanges inside the quad leave each
//             lane with the full score of one head, whose weight exp(s - m_h) it computes and
//             stores.  The shift m_h is held by every thread: 0 at a centre's start, raised
//             only when a score passes it by more than `lead` (or lowered when a centre's first
//             chunk has no score within `lead` below it), in a rare step that takes the exact
//             maximum and rescales what was summed so far.
//   sums      thread (vector column t, row partition p) accumulates U_0 .. U_3 of column t over
//             rows p, p + NPART, ... of every chunk, all four heads from one read of the row;
//             at the centre's end the partitions, and the lanes' parts of each normaliser,
//             are summed through LDS.
template <typename T, int CV, bool ORD>
__global__ void __launch_bounds__(kLocalThreads) local_stream_h4_kernel(LocalArgs<T> A) {
    typedef typename Vec<T>::type V;
    constexpr int EV = Vec<T>::n;
    constexpr int H = 4;
    constexpr int CH = kLocalChunk;                // rows per chunk
    constexpr int SXV = CV + 1;                    // padded LDS row stride in vectors
    constexpr int QV = CV / 4;                     // vectors per quarter row (scores)
    constexpr int NPART = kLocalThreads / CV;      // row partitions of the weighted sums
    constexpr int PER = CH * CV / kLocalThreads;   // chunk vectors per thread
    static_assert(QV >= 1 && PER >= 1 && PER * kLocalThreads == CH * CV, "shape");
    static_assert(CH * H == kLocalThreads, "one thread per (row, head) score");
    __shared__ V sX[2][CH * SXV];
    __shared__ V sR[H * CV];
    __shared__ __align__(16) T sS[CH][H];          // weights (scores in the rescaling step)
    __shared__ T sM[H], sAl[H], sZ[4][H];
    __shared__ __align__(4) uint8_t sFlag[4];      // per wave: bit 0 a score above m + lead,
                                                   // bit 1 a score at or above m - lead

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t N = A.n_centres, G = gridDim.x;
    bool bad_index = false;

    // Task values are alike in all lanes; they are kept in scalar registers.
    auto first_chunk = [&](int64_t i) -> LocalTask {
        for (; i < N; i += G) {
            const int64_t r0 = uniform64(A.row_ptr[i]), r1 = uniform64(A.row_ptr[i + 1]);
            if (r0 < 0 || r1 < r0 || r1 > A.n_edges) {
                if (tid == 0) raise_bits(A.status, kBitCap);
                continue;
            }
            if (r1 > r0) return LocalTask{i, r0, r1 - r0, 0};
            if (tid < H * CV) reinterpret_cast<V*>(A.un + i * (H * CV * EV))[tid] = vsplat<V>(T(0));
        }
        return LocalTask{N, 0, 0, 0};
    };
    auto next_task = [&](const LocalTask& t) -> LocalTask {
        if (t.j0 + CH < t.n) return LocalTask{t.i, t.r0, t.n, t.j0 + CH};
        return first_chunk(t.i + G);
    };
    // Thread tid loads vector u of rows jr, jr + 256 / CV, ...; rows past the chunk's end
    // repeat its last row (the loads stay unconditional; those rows get weight 0).
    const int jr = tid / CV, u = tid % CV;
    V pre[PER], preR = vsplat<V>(T(0));
    auto fetch = [&](const LocalTask& t) {
        const int last = (int)(t.n - t.j0 < CH ? t.n - t.j0 : CH) - 1;
        if (ORD) {
            const int32_t* ord = A.order + (t.r0 + t.j0);
            const V* xv = reinterpret_cast<const V*>(A.x);
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int j = min(jr + q * (kLocalThreads / CV), last);
                int64_t row = ord[j];
                if (row < 0 || row >= A.n_edges) {
                    bad_index = true;
                    row = 0;
                }
                pre[q] = xv[row * CV + u];
            }
        } else {
            const V* xv = reinterpret_cast<const V*>(A.x) + (t.r0 + t.j0) * CV;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int j = min(jr + q * (kLocalThreads / CV), last);
                pre[q] = xv[j * CV + u];
            }
        }
        if (t.j0 == 0 && tid < H * CV) preR = reinterpret_cast<const V*>(A.r + t.i * (H * CV * EV))[tid];
    };

    LocalTask cur = first_chunk(blockIdx.x);
    if (cur.i >= N) {
        if (bad_index) raise_bits(A.status, kBitIndex);
        return;
    }
    fetch(cur);
    LocalTask nxt = next_task(cur);
    const int srow = tid >> 2, sq = tid & 3;             // scores: row, quarter
    const int hq = 2 * (sq & 1) + (sq >> 1);             // the head whose score this lane ends with
    const int ut = tid % CV, upart = tid / CV;           // sums: vector column, row partition
    T m[H];                                              // shifts, alike in every thread
    T zl = T(0);                                         // this lane's part of Z_hq
    V U[H];
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
        m[hh] = T(0);
        U[hh] = vsplat<V>(T(0));
    }
    int buf = 0;
    while (true) {
        const int rows = (int)(cur.n - cur.j0 < CH ? cur.n - cur.j0 : CH);
        const bool fresh = cur.j0 == 0;  // a centre's first chunk
#pragma unroll
        for (int q = 0; q < PER; ++q) sX[buf][(jr + q * (kLocalThreads / CV)) * SXV + u] = pre[q];
        if (fresh && tid < H * CV) sR[tid] = preR * Base2<T>::scale;
        if (nxt.i < N) fetch(nxt);
        __syncthreads();
        // Score of row srow for head hq, and its weight.
        const bool valid = srow < rows;
        T sv, p;
        {
            V xq[QV];
#pragma unroll
            for (int u2 = 0; u2 < QV; ++u2) xq[u2] = sX[buf][srow * SXV + sq * QV + u2];
            T sc[H];
#pragma unroll
            for (int hh = 0; hh < H; ++hh) {
                T v = T(0);
#pragma unroll
                for (int u2 = 0; u2 < QV; ++u2) {
                    const V rv = sR[hh * CV + sq * QV + u2];
#pragma unroll
                    for (int e = 0; e < EV; ++e) v = fma(xq[u2][e], rv[e], v);
                }
                sc[hh] = v;
            }
            // quad transpose-sum: after the xor-1 step lane bit 0 selects heads {0,1} or {2,3},
            // after the xor-2 step lane bit 1 selects one of the pair
            const bool b0 = sq & 1, b1 = sq & 2;
            const T k0 = b0 ? sc[2] : sc[0], k1 = b0 ? sc[3] : sc[1];
            const T g0 = b0 ? sc[0] : sc[2], g1 = b0 ? sc[1] : sc[3];
            const T t0 = k0 + quad_xor<1>(g0), t1 = k1 + quad_xor<1>(g1);
            const T kk = b1 ? t1 : t0, gg = b1 ? t0 : t1;
            sv = kk + quad_xor<2>(gg);
            T mh = m[0];
#pragma unroll
            for (int hh = 1; hh < H; ++hh) mh = hq == hh ? m[hh] : mh;
            p = valid ? Base2<T>::ex(sv - mh) : T(0);
            const bool over = valid && sv > mh + Base2<T>::lead;
            const bool near = valid && sv >= mh - Base2<T>::lead;
            const bool any_over = __any(over), any_near = __any(near);
            if (lane == 0) sFlag[wave] = (uint8_t)((any_over ? 1 : 0) | (any_near ? 2 : 0));
            sS[srow][hq] = p;
        }
        __syncthreads();
        {
            const uint32_t fl = *reinterpret_cast<const uint32_t*>(sFlag);
            if ((fl & 0x01010101u) != 0u || (fresh && (fl & 0x02020202u) == 0u)) {
                // Rare: new shifts from the exact maxima (over the chunk, and the old shift
                // after a centre's first chunk), and the sums so far rescaled.
                sS[srow][hq] = valid ? sv : T(-INFINITY);
                __syncthreads();
                if (lane < H) {
                    // lanes 0..3 of every wave find the same four maxima; wave 0 writes them
                    const int hh = lane;
                    T mc = T(-INFINITY);
                    for (int j = 0; j < rows; ++j) mc = sS[j][hh] > mc ? sS[j][hh] : mc;
                    T mold = m[0];
#pragma unroll
                    for (int h2 = 1; h2 < H; ++h2) mold = hh == h2 ? m[h2] : mold;
                    const T mnew = fresh ? mc : (mc > mold ? mc : mold);
                    if (wave == 0) {
                        sM[hh] = mnew;
                        sAl[hh] = fresh ? T(1) : Base2<T>::ex(mold - mnew);
                    }
                }
                __syncthreads();
#pragma unroll
                for (int hh = 0; hh < H; ++hh) {
                    m[hh] = sM[hh];
                    U[hh] = U[hh] * sAl[hh];
                }
                T mh = m[0], al = sAl[0];
#pragma unroll
                for (int hh = 1; hh < H; ++hh) {
                    mh = hq == hh ? m[hh] : mh;
                    al = hq == hh ? sAl[hh] : al;
                }
                zl *= al;
                p = valid ? Base2<T>::ex(sv - mh) : T(0);
                sS[srow][hq] = p;  // the maxima are taken: the scores are read no more
                __syncthreads();
            }
        }
        zl += p;
        // Weighted sums of column ut over rows upart, upart + NPART, ..., all heads at once.
#pragma unroll
        for (int r = 0; r < CH / NPART; ++r) {
            const int j = upart + r * NPART;
            const V xv = sX[buf][j * SXV + ut];
#pragma unroll
            for (int hh = 0; hh < H; ++hh) U[hh] += sS[j][hh] * xv;
        }
        if (cur.j0 + CH >= cur.n) {
            // The centre's last chunk: sum the row partitions and the normaliser parts, store
            // U_h / Z_h.  Shuffles first fold a wavefront's partitions down to four (none when
            // CV = 16), then the 16 that remain go through LDS, over the other chunk buffer,
            // which nothing reads until the next chunk is written there.
            {  // Z parts: lanes with equal tid % 4 hold the same head
                T zw = zl;
#pragma unroll
                for (int off = 32; off >= 4; off >>= 1) zw += __shfl_xor(zw, off, 64);
                if (lane < 4) sZ[wave][hq] = zw;
            }
#pragma unroll
            for (int off = 32; off >= 4 * CV; off >>= 1) {
#pragma unroll
                for (int hh = 0; hh < H; ++hh)
#pragma unroll
                    for (int e = 0; e < EV; ++e) U[hh][e] += __shfl_xor(U[hh][e], off, 64);
            }
            V* part = &sX[buf ^ 1][0];  // [16][H][CV] vectors; 64 CV <= CH (CV + 1)
            if (lane < 4 * CV) {
                const int pp = wave * 4 + lane / CV;
#pragma unroll
                for (int hh = 0; hh < H; ++hh) part[(pp * H + hh) * CV + ut] = U[hh];
            }
            __syncthreads();
            if (tid < H * CV) {
                const int hh = tid / CV, t = tid % CV;
                V acc = vsplat<V>(T(0));
#pragma unroll
                for (int pp = 0; pp < 16; ++pp) acc += part[(pp * H + hh) * CV + t];
                const T z = (sZ[0][hh] + sZ[1][hh]) + (sZ[2][hh] + sZ[3][hh]);
                reinterpret_cast<V*>(A.un + cur.i * (H * CV * EV))[tid] = acc * (T(1) / z);
            }
            zl = T(0);
#pragma unroll
            for (int hh = 0; hh < H; ++hh) {
                m[hh] = T(0);
                U[hh] = vsplat<V>(T(0));
            }
            // the partials' space is the next chunk's buffer: all threads must be done with it
            __syncthreads();
        }
        buf ^= 1;
        if (nxt.i >= N) break;
        cur = nxt;
        nxt = next_task(cur);
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

// Work-groups of a persistent kernel: as many as the current device holds at once (resident
// work-groups per compute unit for this kernel, from its registers and LDS, times the units).
// fp32, four heads of c = 64 channels: the streaming pass on the matrix cores, one wavefront
// per centre at a time (wavefront w of the grid takes centres w, w + W, ...; no work-group
// barriers), in blocks of 16 rows.  v_mfma_f32_4x4x1_16b_f32 forms 16 independent 4x4 outer
// products per instruction; block b of it takes A[i] from lane 4b + i and B[j] from lane
// 4b + j and accumulates D[i][j] in lane 4b + j, register i.
//   scores  block b = (row group b % 4, channel slice b / 4): lane L holds row L % 16 of the
//           16-row block and channels 16u + 4 (L / 16) + e (u, e < 4) of it, straight from its
//           16-byte global loads, against R of head L % 4 for the same channels (registers,
//           per centre); 16 products, then the four slices summed across lanes (xor 16, 32).
//           Lane L then owns the score of row 4 ((L / 4) % 4) + L / 16 for head L % 4.
//   weights exp2(s - m_h) with the lazily moved shift of local_stream_h4_kernel, per wavefront.
//   sums    block b = columns 4b .. 4b + 3: per row, A[i] = the row's weight for head i, B[j] =
//           the row's column 4b + j (a transposed copy of the block in the wavefront's LDS), so
//           lane L accumulates U_h[L] for the four heads in its four D registers.
#ifndef NGA_LOCAL_MFMA
#define NGA_LOCAL_MFMA 1
#endif
constexpr bool kLocalMfma = NGA_LOCAL_MFMA;
constexpr int kMfRows = 16;
#ifndef NGA_LOCAL_AHEAD
#define NGA_LOCAL_AHEAD 1
#endif
constexpr int kMfAhead = NGA_LOCAL_AHEAD;  // blocks whose loads are in flight
constexpr int kMfLd = 64 + 4;  // padded LDS row, floats

// LDS writes of this wavefront visible to its own later reads (no work-group barrier).
__device__ inline void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool ORD>
__global__ void __launch_bounds__(kLocalThreads) local_mfma_kernel(LocalArgs<float> A) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int C = 64, H = 4, RB = kMfRows;
    __shared__ __align__(16) float sXw[kLocalThreads / 64][RB * kMfLd];
    __shared__ __align__(16) float sPw[kLocalThreads / 64][H * RB];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float* sX = sXw[wave];
    float* sPT = sPw[wave];
    const int G = lane >> 4, r16 = lane & 15, hq = lane & 3;
    const int own_row = 4 * ((lane >> 2) & 3) + G;  // the row this lane's score belongs to
    const int64_t N = A.n_centres;
    const int64_t W = (int64_t)gridDim.x * (kLocalThreads / 64);
    bool bad_index = false;

    // the first non-empty centre at or after i on this wavefront's stride; empty ones get zeros
    auto first_block = [&](int64_t i) -> LocalTask {
        for (; i < N; i += W) {
            const int64_t r0 = uniform64(A.row_ptr[i]), r1 = uniform64(A.row_ptr[i + 1]);
            if (r0 < 0 || r1 < r0 || r1 > A.n_edges) {
                if (lane == 0) raise_bits(A.status, kBitCap);
                continue;
            }
            if (r1 > r0) return LocalTask{i, r0, r1 - r0, 0};
            float* un = A.un + i * (H * C);
#pragma unroll
            for (int h = 0; h < H; ++h) un[h * C + lane] = 0.f;
        }
        return LocalTask{N, 0, 0, 0};
    };
    auto next_block = [&](const LocalTask& t) -> LocalTask {
        if (t.j0 + RB < t.n) return LocalTask{t.i, t.r0, t.n, t.j0 + RB};
        return first_block(t.i + W);
    };
    // Blocks in flight ahead of the current one: lane L loads the 16-byte vectors 4u + L / 16 of
    // row L % 16 (the score operands as they stand); rows past the centre's end repeat its
    // last row (weight 0).
    f4 xa[4], xn[4], xm[4];
    auto fetch = [&](f4 (&dst)[4], const LocalTask& t) {
        const int rows = (int)(t.n - t.j0 < RB ? t.n - t.j0 : RB);
        const int j = r16 < rows - 1 ? r16 : rows - 1;
        int64_t row = t.r0 + t.j0 + j;
        if (ORD) {
            row = A.order[row];
            if (row < 0 || row >= A.n_edges) {
                bad_index = true;
                row = 0;
            }
        }
        const f4* xr = reinterpret_cast<const f4*>(A.x + row * C);
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = xr[4 * u + G];
    };

    LocalTask cur = first_block((int64_t)blockIdx.x * (kLocalThreads / 64) + wave);
    // two ahead: nxt is the block after cur, its loads issued already
    LocalTask nxt = (kMfAhead == 2 && cur.i < N) ? next_block(cur) : cur;
    if (cur.i < N) fetch(xa, cur);
    if (kMfAhead == 2 && nxt.i < N) fetch(xn, nxt);
    f4 rr[4];                          // R of head hq, channels 16u + 4G .. + 3, in base-2 units
    f4 U0 = {0.f, 0.f, 0.f, 0.f}, U1 = U0;  // U_h[lane] over even / odd rows
    float m = 0.f, zl = 0.f;           // head hq's shift; this lane's part of Z_hq
    while (cur.i < N) {
        LocalTask nn;  // the block whose loads are issued now
        if (kMfAhead == 2) {
            nn = nxt.i < N ? next_block(nxt) : nxt;
            if (nn.i < N) fetch(xm, nn);
        } else {
            nn = next_block(cur);
            if (nn.i < N) fetch(xn, nn);
        }
        const bool fresh = cur.j0 == 0;
        if (fresh) {
            const f4* rp = reinterpret_cast<const f4*>(A.r + cur.i * (H * C) + hq * C);
#pragma unroll
            for (int u = 0; u < 4; ++u) rr[u] = rp[4 * u + G] * Base2<float>::scale;
        }
        const int rows = (int)(cur.n - cur.j0 < RB ? cur.n - cur.j0 : RB);
        // scores: 16 products in two chains, then the four channel slices summed
        f4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = d0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[u][0], rr[u][0], d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[u][1], rr[u][1], d1, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[u][2], rr[u][2], d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[u][3], rr[u][3], d1, 0, 0, 0);
        }
        f4 d = d0 + d1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            d[e] += __shfl_xor(d[e], 16, 64);
            d[e] += __shfl_xor(d[e], 32, 64);
        }
        const float sv = G == 0 ? d[0] : (G == 1 ? d[1] : (G == 2 ? d[2] : d[3]));
        const bool valid = own_row < rows;
        // the shift: 0 at a centre's start, moved only when a score passes it by more than
        // `lead`, or when a centre's first block has no score within `lead` below it
        const bool over = valid && sv > m + Base2<float>::lead;
        const bool near = valid && sv >= m - Base2<float>::lead;
        // lanes L with L % 4 = h hold head h: a head with no score near its shift in a centre's
        // first block has its shift lowered (every head has row 0 there)
        const uint64_t nm = __ballot(near);
        const bool some_head_far = (nm & 0x1111111111111111ull) == 0 || (nm & 0x2222222222222222ull) == 0 ||
                                   (nm & 0x4444444444444444ull) == 0 || (nm & 0x8888888888888888ull) == 0;
        if (__any(over) || (fresh && some_head_far)) {
            float mc = valid ? sv : -INFINITY;
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) {
                const float o = __shfl_xor(mc, off, 64);
                mc = o > mc ? o : mc;
            }
            const float mnew = fresh ? mc : (mc > m ? mc : m);
            const float alpha = fresh ? 1.f : Base2<float>::ex(m - mnew);
            zl *= alpha;
            m = mnew;
            f4 al;
#pragma unroll
            for (int h = 0; h < H; ++h) al[h] = __shfl(alpha, h, 64);  // lane h holds head h
            U0 *= al;
            U1 *= al;
        }
        const float p = valid ? Base2<float>::ex(sv - m) : 0.f;
        zl += p;
        // the block and its weights into this wavefront's LDS, transposed for the sums
        sPT[hq * RB + own_row] = p;
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<f4*>(&sX[r16 * kMfLd + 16 * u + 4 * G]) = xa[u];
        wave_sync_lds();
        f4 pa[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) pa[q] = *reinterpret_cast<const f4*>(&sPT[hq * RB + 4 * q]);
#pragma unroll
        for (int r = 0; r < RB; r += 2) {
            U0 = __builtin_amdgcn_mfma_f32_4x4x1f32(pa[r / 4][r % 4], sX[r * kMfLd + lane], U0, 0, 0, 0);
            U1 = __builtin_amdgcn_mfma_f32_4x4x1f32(pa[r / 4][r % 4 + 1], sX[(r + 1) * kMfLd + lane], U1, 0, 0, 0);
        }
        wave_sync_lds();  // the next block rewrites the buffers
        if (cur.j0 + RB >= cur.n) {
            // the centre's end: Z_h from the lanes' parts (lanes with equal hq), U_h / Z_h
            float z = zl;
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) z += __shfl_xor(z, off, 64);
            const f4 U = U0 + U1;
            float* un = A.un + cur.i * (H * C);
#pragma unroll
            for (int h = 0; h < H; ++h) un[h * C + lane] = U[h] * (1.f / __shfl(z, h, 64));
            U0 = f4{0.f, 0.f, 0.f, 0.f};
            U1 = U0;
            m = 0.f;
            zl = 0.f;
        }
        if (kMfAhead == 2) {
            cur = nxt;
            nxt = nn;
        } else {
            cur = nn;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xa[u] = xn[u];
            if (kMfAhead == 2) xn[u] = xm[u];
        }
    }
    if (bad_index) raise_bits(A.status, kBitIndex);
}

template <bool ORD>
void launch_mfma_o(const LocalArgs<float>& a, hipStream_t s) {
    const void* k = reinterpret_cast<const void*>(&local_mfma_kernel<ORD>);
    // one wavefront per centre at most
    const int64_t groups = std::min<int64_t>((a.n_centres + 3) / 4, resident_groups(k, kLocalThreads));
    hipLaunchKernelGGL((local_mfma_kernel<ORD>), dim3((unsigned)(groups < 1 ? 1 : groups)),
                       dim3(kLocalThreads), 0, s, a);
}

template <typename T, int CV, bool ORD>
void launch_stream_h4_o(const LocalArgs<T>& a, hipStream_t s) {
    const void* k = reinterpret_cast<const void*>(&local_stream_h4_kernel<T, CV, ORD>);
    const dim3 grid((unsigned)std::min<int64_t>(a.n_centres, resident_groups(k, kLocalThreads)));
    hipLaunchKernelGGL((local_stream_h4_kernel<T, CV, ORD>), grid, dim3(kLocalThreads), 0, s, a);
}

template <typename T, int CV>
void launch_stream_h4(const LocalArgs<T>& a, hipStream_t s) {
    if (a.order) launch_stream_h4_o<T, CV, true>(a, s);
    else launch_stream_h4_o<T, CV, false>(a, s);
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
        const int cvec = c / Vec<T>::n;
        if (std::is_same<T, float>::value && heads == 4 && c == 64 && kLocalMfma) {
            if (order) launch_mfma_o<true>(reinterpret_cast<const LocalArgs<float>&>(a), s);
            else launch_mfma_o<false>(reinterpret_cast<const LocalArgs<float>&>(a), s);
        } else if (heads == 4 && (cvec == 4 || cvec == 8 || cvec == 16)) {
            if (cvec == 4) launch_stream_h4<T, 4>(a, s);
            else if (cvec == 8) launch_stream_h4<T, 8>(a, s);
            else launch_stream_h4<T, 16>(a, s);
        } else if (nv <= kLocalThreads && loads <= 4)
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
