// Fused per-centre block attention in fp32 on the fp32 matrix cores, 16-wide heads.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense ...", section
// "Proposed fix: block-dense attention on the graph": gather a centre's (nnei, c) block
// through the destination CSR, dense attention math with a mask for the ragged tail,
// scatter back to the edge axis.  Here one work-group runs a centre's whole layer stack:
// the block is gathered once into LDS, intermediate layers hand their output back through
// the same LDS rows, and only the last layer writes to HBM.
//
// Work-group = H wavefronts, wavefront h owns head h (columns 16h .. 16h+15).  Every
// contraction is v_mfma_f32_16x16x4_f32: fp32 operands, fp32 products, fp32 accumulation.
// Its operand / result layouts (A[i][k] from lane i + 16k, B[k][j] from lane j + 16k,
// D[i][j] in lane j + 16(i/4), register i%4) let every result feed the next contraction
// directly, by choosing the order in which each contraction walks its k index:
//   projections  Q^T = Wq_h^T X^T, K^T = Wk_h^T X^T, V = X Wv_h   (k = input channel)
//                with k(step kk, lane group g) = 16(kk/4) + 4g + kk%4, so a lane reads
//                float4s of its own row of the block;
//   scores       S^T = K Q^T, k = head channel 4g + r: A = K^T result register r,
//                B = Q^T result register r;  lane (g, i) then holds query i against keys
//                4g + r of every key tile;
//   softmax      row max / sum over a lane's registers and the 4 lane groups (2 shuffles);
//   values       O^T = V^T P^T, k = key 16t + 4g + r: A = V result register r,
//                B = P register r;
//   output       Y^T = Wo^T [O_0 .. O_{H-1}]^T, k = 16hh + 4g + r: B = head hh's O^T
//                register r, exchanged through LDS; lane (g, i) gets 4 consecutive output
//                channels of row i, one float4.
// K^T and V of every row tile stay in registers for the whole layer; Q^T is formed one
// query tile at a time.  Rows past the centre's length are zeros in LDS, their keys are
// masked to -inf and their outputs are never stored.
#include "block_attn_fused.h"

#include <algorithm>

namespace nga {

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ inline f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr float kLog2e = 1.4426950408889634f;

// Weights in operand order: for layer l, matrix m (q, k, v, o) and wavefront h, lane
// L = 16g + i holds KS = C/4 consecutive floats, element kk = W_m[k(kk, g)][16h + i].
__global__ void __launch_bounds__(256)
pack_f32_weights_kernel(const float* __restrict__ w, int C, int H, int layers,
                        float* __restrict__ packed) {
    const int KS = C / 4;
    const int64_t total = (int64_t)layers * 4 * C * C;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        int64_t rest = idx;
        const int kk = (int)(rest % KS); rest /= KS;
        const int lane = (int)(rest % 64); rest /= 64;
        const int h = (int)(rest % H); rest /= H;
        const int m = (int)(rest % 4); rest /= 4;
        const int l = (int)rest;
        const int g = lane >> 4, i = lane & 15;
        const int k = 16 * (kk >> 2) + 4 * g + (kk & 3);
        packed[idx] = w[(((int64_t)l * 4 + m) * C + k) * C + 16 * h + i];
    }
}

struct F32Args {
    const int64_t* row_ptr;
    const int32_t* order;
    const float* x;
    float* y;
    const float* w;  // packed operand-order weights
    int n_centres;
    int64_t n_edges;
    int nnei_cap;
    int layers;
    const float* ldt;  // smooth attention: ln D~ [layers][n_edges][H], or NULL
    uint32_t* status;
};

// Row stride (floats) of the LDS block: 4 floats of padding per row put the float4 reads of
// the 16 rows of a tile on distinct banks.
template <int H>
struct Lds {
    static constexpr int C = 16 * H;
    static constexpr int XS = C + 4;
};

// One layer of one centre whose block (NT row tiles) sits in sX.  K^T and V of every tile go
// to registers; then for each query tile, Q^T is formed from the block, the scores, softmax
// and values follow, the heads' outputs meet in LDS for the output projection, and the
// result is stored to y (last layer) or written back over the block rows it came from
// (earlier layers; those rows are no longer read in this layer).
//
// Softmax shift.  Any shift b_j >= max_k s_jk gives the same softmax; the exact row max costs
// a pass over the scores before the exponentials.  Instead each query row takes the
// Cauchy-Schwarz bound b_j = |q_j| max_k |k_k| (in the base-2 units of the scaled keys), which
// needs only the query's norm, and enters the score MFMAs as their initial accumulator, so the
// exponentials read s_jk - b_j straight from the MFMA results.  If the bound is so loose that a
// row's exponentials all underflow (Z < 2^-64; it takes a score range of some 64 binary orders
// of magnitude between the bound and the true max), the wave recomputes its tile with the exact
// max.
template <int H, int NT, bool SMOOTH>
__device__ __forceinline__ void centre_layer(const F32Args& A, const float* __restrict__ P,
                                             const int layer, const int64_t r0, const int n,
                                             const bool last,
                                             float (*__restrict__ sX)[Lds<H>::XS],
                                             f4 (*__restrict__ sO)[H][64], const int lane,
                                             const int h) {
    constexpr int C = 16 * H;
    constexpr int KS = C / 4;
    constexpr int MAT = H * 64 * KS;
    const int g = lane >> 4;
    const int li = lane & 15;
    const float c1 = kLog2e * 0.25f;  // log2(e) / sqrt(16): the softmax in base 2

    float wq[KS], wk[KS], wv[KS], wo[KS];
#pragma unroll
    for (int k4 = 0; k4 < KS / 4; ++k4) {
        const f4 a = *reinterpret_cast<const f4*>(P + 0 * MAT + 4 * k4);
        const f4 b = *reinterpret_cast<const f4*>(P + 1 * MAT + 4 * k4);
        const f4 c = *reinterpret_cast<const f4*>(P + 2 * MAT + 4 * k4);
        const f4 d = *reinterpret_cast<const f4*>(P + 3 * MAT + 4 * k4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wq[4 * k4 + i] = a[i];
            wk[4 * k4 + i] = b[i];
            wv[4 * k4 + i] = c[i];
            wo[4 * k4 + i] = d[i];
        }
    }

    // K^T (scaled by c1: scores come out in base-2 units) and V of every row tile, kept in
    // registers for the layer; kn2 = the largest squared key norm of this head.
    f4 kt[NT], vt[NT];
    float kn2 = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float xo[KS];
#pragma unroll
        for (int u = 0; u < C / 16; ++u) {
            const f4 v = *reinterpret_cast<const f4*>(&sX[16 * t + li][16 * u + 4 * g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) xo[4 * u + i] = v[i];
        }
        f4 k = {0.f, 0.f, 0.f, 0.f}, v = k;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            k = mfma4(wk[kk], xo[kk], k);
            v = mfma4(xo[kk], wv[kk], v);
        }
        k *= c1;
        kt[t] = k;
        vt[t] = v;
        // lane (g, i) holds channels 4g .. 4g+3 of key 16t + i
        float k2 = k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3];
        k2 += __shfl_xor(k2, 16, 64);
        k2 += __shfl_xor(k2, 32, 64);
        kn2 = fmaxf(kn2, k2);
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) kn2 = fmaxf(kn2, __shfl_xor(kn2, d, 64));
    const float kmax = sqrtf(kn2);

    for (int qt = 0; qt < NT; ++qt) {
        f4 q = {0.f, 0.f, 0.f, 0.f};
        {
            float xo[KS];
#pragma unroll
            for (int u = 0; u < C / 16; ++u) {
                const f4 v = *reinterpret_cast<const f4*>(&sX[16 * qt + li][16 * u + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) xo[4 * u + i] = v[i];
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) q = mfma4(wq[kk], xo[kk], q);
        }
        // lane (g, j) holds channels 4g .. 4g+3 of query j: its norm times kmax bounds every
        // score of row j.
        float q2 = q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3];
        q2 += __shfl_xor(q2, 16, 64);
        q2 += __shfl_xor(q2, 32, 64);
        float shift = sqrtf(q2) * kmax;
        const f4 init = {-shift, -shift, -shift, -shift};
        f4 s[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f4 acc = mfma4(kt[t][0], q[0], init);
#pragma unroll
            for (int r = 1; r < 4; ++r) acc = mfma4(kt[t][r], q[r], acc);
            s[t] = acc;
        }
        // NT = ceil(n / 16), so only the last key tile can hold keys past the row end.
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (16 * (NT - 1) + 4 * g + r >= n) s[NT - 1][r] = -INFINITY;
        float z = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[t][r]);
                s[t][r] = p;
                z += p;
            }
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        if (__builtin_expect(__any(z < 0x1p-64f), 0)) {
            // The bound left a row's weights (nearly) all underflowed: this tile again with
            // the exact row max as the shift.
            float m = -INFINITY;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) acc = mfma4(kt[t][r], q[r], acc);
                s[t] = acc;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * (NT - 1) + 4 * g + r >= n) s[NT - 1][r] = -INFINITY;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) m = fmaxf(m, s[t][r]);
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            shift = m;
            z = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(s[t][r] - m);
                    s[t][r] = p;
                    z += p;
                }
            z += __shfl_xor(z, 16, 64);
            z += __shfl_xor(z, 32, 64);
        }
        f4 osum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) osum = mfma4(vt[t][r], s[t][r], osum);
        f4 o;
        if constexpr (SMOOTH) {
            // sum_j e_j / D~ times the softmax = exp(s_j / sqrt(d) - ln D~): the weighted sum
            // (shifted by `shift` in base 2) times 2^(shift - log2(e) ln D~) in place of 1 / Z.
            const int aq = 16 * qt + li;
            float f = 0.f;
            if (aq < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + aq] : r0 + aq;
                if (row >= 0 && row < A.n_edges)
                    f = exp2f(shift - kLog2e * A.ldt[((int64_t)layer * A.n_edges + row) * H + h]);
            }
            o = osum * f;
        } else {
            o = osum * __builtin_amdgcn_rcpf(z);
        }

        const int buf = qt & 1;
        sO[buf][h][lane] = o;
        __syncthreads();  // every head's O of this tile is in LDS; every wave has read rows qt
        f4 yv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
            const f4 oo = sO[buf][hh][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) yv = mfma4(wo[4 * hh + r], oo[r], yv);
        }
        const int a = 16 * qt + li;
        if (last) {
            if (a < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
                if (row >= 0 && row < A.n_edges)
                    *reinterpret_cast<f4*>(A.y + row * C + 16 * h + 4 * g) = yv;
            }
        } else {
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f4*>(&sX[a][16 * h + 4 * g]) = a < n ? yv : zero;
        }
    }
}

template <int H, int TMAX, bool SMOOTH>
__global__ void __launch_bounds__(64 * H, 2) fused_f32_kernel(F32Args A) {
    constexpr int C = 16 * H;
    constexpr int KS = C / 4;
    constexpr int NTH = 64 * H;
    constexpr int CH = C / 4;  // float4 chunks per row
    constexpr int PER = (16 * TMAX * CH + NTH - 1) / NTH;
    __shared__ __align__(16) float sX[16 * TMAX][Lds<H>::XS];
    __shared__ f4 sO[2][H][64];

    const int lane = threadIdx.x & 63;
    const int h = threadIdx.x >> 6;

    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (A.row_ptr[0] != 0 || A.row_ptr[A.n_centres] > A.n_edges) raise_bits(A.status, kBitCap);
    }
    const int centre = blockIdx.x;
    const int64_t r0 = A.row_ptr[centre];
    const int64_t r1 = A.row_ptr[centre + 1];
    if (r1 == r0) return;
    // A decreasing row_ptr, a row outside [0, n_edges) or one longer than the cap is
    // reported and skipped.
    if (r1 < r0 || r1 - r0 > A.nnei_cap || r1 - r0 > 16 * TMAX || r0 < 0 || r1 > A.n_edges) {
        if (threadIdx.x == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int n = (int)(r1 - r0);
    const int nt = (n + 15) >> 4;
    bool bad_index = false;

    // Gather the block: rows a < n from x (through `order`), zeros up to the tile edge.
    // All loads of a thread are issued before any LDS write.
    {
        f4 v[PER];
        const int chunks = 16 * nt * CH;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = threadIdx.x + j * NTH;
            const int a = idx / CH, c4 = idx % CH;
            v[j] = f4{0.f, 0.f, 0.f, 0.f};
            if (idx < chunks && a < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
                if (row >= 0 && row < A.n_edges)
                    v[j] = *reinterpret_cast<const f4*>(A.x + row * C + 4 * c4);
                else
                    bad_index = true;
            }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = threadIdx.x + j * NTH;
            const int a = idx / CH, c4 = idx % CH;
            if (idx < chunks) *reinterpret_cast<f4*>(&sX[a][4 * c4]) = v[j];
        }
    }
    __syncthreads();

    for (int layer = 0; layer < A.layers; ++layer) {
        const float* P = A.w + (size_t)layer * 4 * C * C + ((size_t)h * 64 + lane) * KS;
        const bool last = layer == A.layers - 1;
#define NGA_CASE(T)                                                                       \
    case T:                                                                               \
        if constexpr (T <= TMAX)                                                          \
            centre_layer<H, T, SMOOTH>(A, P, layer, r0, n, last, sX, sO, lane, h);        \
        break;
        switch (nt) {
            NGA_CASE(1) NGA_CASE(2) NGA_CASE(3) NGA_CASE(4) NGA_CASE(5) NGA_CASE(6)
            NGA_CASE(7) NGA_CASE(8) NGA_CASE(9) NGA_CASE(10) NGA_CASE(11) NGA_CASE(12)
            default: break;
        }
#undef NGA_CASE
        __syncthreads();  // this layer's rows are complete before the next layer reads them
    }
    if (bad_index) raise_bits(A.status, kBitIndex);
}

template <int H, bool SMOOTH>
int launch_hs(int tmax, const F32Args& a, hipStream_t s) {
    // One work-group per centre: two stay resident per compute unit (LDS and registers) and
    // the next starts as soon as one retires.
    dim3 grid((unsigned)a.n_centres), block(64 * H);
    if (tmax <= 4)
        hipLaunchKernelGGL((fused_f32_kernel<H, 4, SMOOTH>), grid, block, 0, s, a);
    else if (tmax <= 8)
        hipLaunchKernelGGL((fused_f32_kernel<H, 8, SMOOTH>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((fused_f32_kernel<H, 12, SMOOTH>), grid, block, 0, s, a);
    return last_launch_status();
}

template <int H>
int launch_h(int tmax, const F32Args& a, hipStream_t s) {
    return a.ldt ? launch_hs<H, true>(tmax, a, s) : launch_hs<H, false>(tmax, a, s);
}

}  // namespace

bool f32_fused_supported(int32_t nnei_cap, int32_t c, int32_t heads) {
    if (heads != 1 && heads != 2 && heads != 4) return false;
    if (c != 16 * heads) return false;
    return nnei_cap >= 1 && nnei_cap <= 16 * 12;
}

size_t f32_fused_workspace_floats(int32_t c, int32_t layers) {
    return (size_t)layers * 4 * c * c;
}

int run_f32_fused(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                  int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
                  const float* weights, const float* x, const float* log_dtilde, float* y,
                  float* packed, uint32_t* status, hipStream_t s) {
    const int64_t total = (int64_t)layers * 4 * c * c;
    const unsigned pblocks = (unsigned)std::min<int64_t>((total + 255) / 256, 1024);
    hipLaunchKernelGGL(pack_f32_weights_kernel, dim3(pblocks), dim3(256), 0, s, weights, (int)c,
                       (int)heads, (int)layers, packed);
    int rc = last_launch_status();
    if (rc) return rc;
    F32Args a;
    a.row_ptr = row_ptr;
    a.order = order;
    a.x = x;
    a.y = y;
    a.w = packed;
    a.n_centres = (int)n_centres;
    a.n_edges = n_edges;
    a.nnei_cap = nnei_cap;
    a.layers = layers;
    a.ldt = log_dtilde;
    a.status = status;
    const int tmax = (nnei_cap + 15) / 16;
    switch (heads) {
        case 1: return launch_h<1>(tmax, a, s);
        case 2: return launch_h<2>(tmax, a, s);
        default: return launch_h<4>(tmax, a, s);
    }
}

}  // namespace nga
