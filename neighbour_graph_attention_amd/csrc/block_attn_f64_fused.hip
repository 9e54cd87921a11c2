// Fused per-centre fp64 block attention for narrow features (c <= 32, heads of 8 or 16,
// rows <= 64), every layer in one launch.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense ...", section
// "Proposed fix: block-dense attention on the graph": gather a centre's (nnei, c) block
// through the destination CSR, dense attention with a mask for the ragged tail, scatter back.
// Section "Measurements": the diamond runs are fp64.  With c = 32 and rows of 40, one layer
// of one centre is about a hundred 16x16x4 fp64 matrix-core products, so the three launches
// per layer of the wide path (row GEMM, per-head core, row GEMM) cost more in launches and
// HBM round trips than in arithmetic.  Here one work-group takes a centre through the whole
// layer stack: the block stays in LDS, intermediate layers write their output back into it,
// and only the last layer writes y.
//
// Work-group = H wavefronts, wavefront h owns head h.  v_mfma_f64_16x16x4_f64 takes
// A[i][k] from lane i + 16k, B[k][j] from lane j + 16k and leaves D[i][j] in lane
// j + 16(i%4), register i/4.  Lane (g, l) below means lane 16g + l.  With X[a][ch] the
// block rows and W[in][out] the weights (y = x W):
//   Q^T, K^T = W_h^T X^T  (A: W[4kc+g][hd+l], B: X[16t+l][4kc+g]) -> lane (g, l), register r:
//                          channel 4r+g of row 16t+l;
//   V = X W_h             (A: X[16t+l][4kc+g], the same LDS value, B: W[4kc+g][hd+l])
//                          -> lane (g, l), register r: channel l of row 16t+4r+g;
//   S^T = K Q^T           (A: K^T register r, B: Q^T register r, for channels 4r .. 4r+3)
//                          -> lane (g, l), register r: key 16kt+4r+g against query 16qt+l;
//   O^T = V^T P^T         (A: V register r, B: P^T register r, for keys 16kt+4r .. +3)
//                          -> lane (g, l), register r: channel 4r+g of query 16qt+l;
//   Y^T = Wo^T O^T        (A: Wo[4kc+g][16u+l], B: the O^T register of head (4kc+g)/d,
//                          read from LDS) -> lane (g, l), register r: output 16u+4r+g.
// Every product's result registers are the next product's operands as they stand; the
// heads meet once per layer, through LDS, for the output projection.
#include <type_traits>

#include "block_attn_f64.h"

namespace nga {

namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef double d2 __attribute__((ext_vector_type(2)));

__device__ inline d4 mfma64(double a, double b, d4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

constexpr int kFusedF64Tiles = 4;  // rows per centre up to 64

struct FusedF64Args {
    const int64_t* row_ptr;
    const int32_t* order;
    const double* x;
    double* y;
    const double* w;    // [layers][4][c][c]
    const double* ldt;  // smooth attention: ln D~ [layers][n_edges][heads], or NULL
    int n_centres;
    int64_t n_edges;
    int nnei_cap;
    int layers;
    uint32_t* status;
    double one;  // 1.0, a run-time value the compiler cannot fold (settle())
};

// A matrix-core product's result scaled by f, read first by this vector multiply in the
// block that issued the product.  The fp64 16x16x4 product writes its result some 19 wait
// states after issue, and the compiler's hazard pass inserts that wait only along the code
// as laid out; a later branch that skips a masked region (s_cbranch_execz) can reach the
// first reader sooner.  That happened here: the row scale's branchy smooth-attention block
// between the last P.V product and its reader was skipped, and on some boxes the multiply
// read one of the four result registers before the product had written it (every output
// row of the last query tile missed the last key group's weighted values).  The empty asm
// keeps the multiply where it is; every later use, behind whatever branches, reads the
// multiply's result, which is a plain vector register write.
__device__ __forceinline__ d4 settle(d4 v, double f) {
    double a0 = v[0] * f, a1 = v[1] * f, a2 = v[2] * f, a3 = v[3] * f;
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    return d4{a0, a1, a2, a3};
}

template <int H, int D>
struct F64Shape {
    static constexpr int C = H * D;
    static constexpr int CP = C + 1;        // LDS row stride (doubles)
    static constexpr int KC = C / 4;        // 4-channel chunks of a contraction over c
    static constexpr int RK = D / 4;        // registers of Q^T / K^T that hold the head
    static constexpr int UO = (C + 15) / 16;  // 16-wide output tiles
    // A head's O^T tile as the output projection reads it: registers r = 0 .. D/4 - 1 of
    // each lane (channels 4r + g); heads of 8 leave registers 2 and 3 zero, so they keep two.
    using OTile = typename std::conditional<D == 8, d2, d4>::type;
};

// One layer of one centre; rows 16*NT and beyond are absent, rows n .. 16*NT-1 are zero in sX.
// SM: smooth attention (ldt given); a separate instance keeps the general exponential and its
// constants out of the registers of the plain softmax.
template <int H, int D, int NT, bool SM>
__device__ __forceinline__ void layer_f64(const FusedF64Args& A, const double* __restrict__ W,
                                          const double* __restrict__ ldt, const int64_t r0,
                                          const int n, const bool last, double* __restrict__ sX,
                                          typename F64Shape<H, D>::OTile (
                                              *__restrict__ sO)[kFusedF64Tiles][64],
                                          const int lane, const int h) {
    using S = F64Shape<H, D>;
    constexpr int C = S::C, CP = S::CP, KC = S::KC, RK = S::RK, UO = S::UO;
    const int g = lane >> 4, l = lane & 15;
    const double scale = 1.0 / __builtin_sqrt((double)D);
    const double scale2 = scale * kLog2eF64;  // softmax exponents in base 2

    // Projections of head h.  Heads of 16: lane (g, l) holds W[4kc+g][hd+l] of Wq, Wk and Wv,
    // and Q^T, K^T, V take one product each.  Heads of 8 would leave half of every 16-row
    // Q^T and K^T tile empty, so Q^T and K^T share one: A rows 0..7 are Wq's head columns and
    // rows 8..15 Wk's, which puts Q^T channel 4r+g in registers r = 0, 1 and K^T channel
    // 4(r-2)+g in registers 2, 3 (V keeps 8 of its 16 columns).
    constexpr bool kStackQK = D == 8;
    double wq[KC], wk[KC], wv[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int idx = (4 * kc + g) * C + h * D + (kStackQK ? (l & 7) : l);
        const bool in_head = l < D;
        if constexpr (kStackQK) {
            wq[kc] = in_head ? W[idx] : W[C * C + idx];
            wk[kc] = 0.0;
        } else {
            wq[kc] = in_head ? W[idx] : 0.0;
            wk[kc] = in_head ? W[C * C + idx] : 0.0;
        }
        wv[kc] = in_head ? W[2 * C * C + idx] : 0.0;
    }
    d4 qT[NT], kT[NT], v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        d4 q = {0.0, 0.0, 0.0, 0.0}, k = q, vv = q;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const double xv = sX[(16 * t + l) * CP + 4 * kc + g];
            q = mfma64(wq[kc], xv, q);
            if constexpr (!kStackQK) k = mfma64(wk[kc], xv, k);
            vv = mfma64(xv, wv[kc], vv);
        }
        qT[t] = q;
        kT[t] = k;
        v[t] = vv;
    }

#pragma unroll
    for (int qt = 0; qt < NT; ++qt) {
        d4 s[NT];
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            d4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                if constexpr (kStackQK) acc = mfma64(qT[kt][2 + r], qT[qt][r], acc);
                else acc = mfma64(kT[kt][r], qT[qt][r], acc);
            }
            s[kt] = acc;
        }
        // NT = ceil(n / 16), so only keys of the last tile can lie past n.
        double m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (kt == NT - 1 && 16 * kt + 4 * r + g >= n) s[kt][r] = -INFINITY;
                m = fmax(m, s[kt][r]);
            }
        m = fmax(m, __shfl_xor(m, 16, 64));
        m = fmax(m, __shfl_xor(m, 32, 64));
        double z = 0.0;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool masked = kt == NT - 1 && 16 * kt + 4 * r + g >= n;
                const double p = exp2_nonpos(masked ? -4096.0 : (s[kt][r] - m) * scale2);
                s[kt][r] = p;
                z += p;
            }
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        // The row's scale, with all of its branches, before the products whose results it
        // multiplies: see settle() for why no branch may separate those products from their
        // first reader.  Smooth attention: sum_j e_j / D~ times the softmax =
        // exp(s_j - ln D~), i.e. the weighted sum times exp(m - ln D~) in place of 1/Z.
        double f = 1.0 / z;
        if constexpr (SM) {
            f = 0.0;
            const int a = 16 * qt + l;
            if (a < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
                if (row >= 0 && row < A.n_edges) f = exp(m * scale - ldt[row * H + h]);
            }
        }
        d4 o = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) o = mfma64(v[kt][r], s[kt][r], o);
        o = settle(o, f);
        if constexpr (D == 8) sO[h][qt][lane] = d2{o[0], o[1]};
        else sO[h][qt][lane] = o;
    }
    __syncthreads();

    // Y^T tile (output tile u, query tile qt) for the pairs of this wavefront.
    for (int pr = h; pr < UO * NT; pr += H) {
        const int u = pr / NT, qt = pr % NT;
        const int out = 16 * u + l;
        d4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int in = 4 * kc + g;  // input channel: head in / D, channel in % D
            const double wo = out < C ? W[3 * C * C + in * C + out] : 0.0;
            const double ov = sO[in / D][qt][lane][(in % D) >> 2];
            acc = mfma64(wo, ov, acc);
        }
        acc = settle(acc, A.one);
        const int a = 16 * qt + l;
        if (last) {
            if (a < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
                if (row >= 0 && row < A.n_edges) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int oc = 16 * u + 4 * r + g;
                        if (oc < C) A.y[row * C + oc] = acc[r];
                    }
                }
            }
        } else {
            // Every read of this layer's rows happened before the barrier above, so the
            // output goes straight back into them; rows past n stay zero.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int oc = 16 * u + 4 * r + g;
                if (oc < C) sX[a * CP + oc] = a < n ? acc[r] : 0.0;
            }
        }
    }
}

// NTM: the most 16-row tiles a centre of this launch can have.  Rows of up to 48 leave out
// the four-tile instance, whose registers would otherwise set the whole kernel's (four heads
// of 8, plain softmax: 142 instead of 183 VGPRs, three work-groups per compute unit instead
// of two).
template <int H, int D, int NTM, bool SM>
__global__ void __launch_bounds__(64 * H, 2) fused_f64_kernel(FusedF64Args A) {
    using S = F64Shape<H, D>;
    constexpr int C = S::C, CP = S::CP;
    __shared__ double sX[16 * kFusedF64Tiles * CP];
    __shared__ typename S::OTile sO[H][kFusedF64Tiles][64];
    const int lane = threadIdx.x & 63;
    const int h = threadIdx.x >> 6;

    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (A.row_ptr[0] != 0 || A.row_ptr[A.n_centres] > A.n_edges) raise_bits(A.status, kBitCap);
    }
    const int centre = blockIdx.x;
    const int64_t r0 = A.row_ptr[centre];
    const int64_t r1 = A.row_ptr[centre + 1];
    if (r1 == r0) return;
    if (r1 < r0 || r1 - r0 > A.nnei_cap || r1 - r0 > 16 * NTM || r0 < 0 ||
        r1 > A.n_edges) {
        if (threadIdx.x == 0) raise_bits(A.status, kBitCap);
        return;
    }
    const int n = (int)(r1 - r0);
    const int nt = (n + 15) >> 4;
    bool bad_index = false;
    for (int idx = threadIdx.x; idx < 16 * nt * C; idx += 64 * H) {
        const int a = idx / C, ch = idx % C;
        double val = 0.0;
        if (a < n) {
            const int64_t row = A.order ? (int64_t)A.order[r0 + a] : r0 + a;
            if (row >= 0 && row < A.n_edges)
                val = A.x[row * C + ch];
            else
                bad_index = true;
        }
        sX[a * CP + ch] = val;
    }
    __syncthreads();
    for (int layer = 0; layer < A.layers; ++layer) {
        const double* W = A.w + (size_t)layer * 4 * C * C;
        const double* ldt = A.ldt ? A.ldt + (size_t)layer * A.n_edges * H : nullptr;
        const bool last = layer == A.layers - 1;
        switch (nt) {
            case 1: layer_f64<H, D, 1, SM>(A, W, ldt, r0, n, last, sX, sO, lane, h); break;
            case 2: layer_f64<H, D, 2, SM>(A, W, ldt, r0, n, last, sX, sO, lane, h); break;
            case 3: layer_f64<H, D, 3, SM>(A, W, ldt, r0, n, last, sX, sO, lane, h); break;
            default:
                if constexpr (NTM >= 4)
                    layer_f64<H, D, 4, SM>(A, W, ldt, r0, n, last, sX, sO, lane, h);
                break;
        }
        __syncthreads();
    }
    if (bad_index) raise_bits(A.status, kBitIndex);
}

template <int H, int D, bool SM>
void launch_fused_f64_sm(const FusedF64Args& a, hipStream_t s) {
    if (a.nnei_cap <= 48)
        hipLaunchKernelGGL((fused_f64_kernel<H, D, 3, SM>), dim3((unsigned)a.n_centres),
                           dim3(64 * H), 0, s, a);
    else
        hipLaunchKernelGGL((fused_f64_kernel<H, D, 4, SM>), dim3((unsigned)a.n_centres),
                           dim3(64 * H), 0, s, a);
}

template <int H, int D>
void launch_fused_f64(const FusedF64Args& a, hipStream_t s) {
    if (a.ldt) launch_fused_f64_sm<H, D, true>(a, s);
    else launch_fused_f64_sm<H, D, false>(a, s);
}

}  // namespace

bool fused_f64_supported(int32_t nnei_cap, int32_t c, int32_t heads) {
    if (heads < 1 || c % heads != 0 || c > 32) return false;
    const int d = c / heads;
    if (d != 8 && d != 16) return false;
    return nnei_cap >= 1 && nnei_cap <= 16 * kFusedF64Tiles;
}

int run_fused_f64(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                  int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
                  const double* weights, const double* x, const double* log_dtilde, double* y,
                  uint32_t* status, hipStream_t s) {
    FusedF64Args a;
    a.row_ptr = row_ptr;
    a.order = order;
    a.x = x;
    a.y = y;
    a.w = weights;
    a.ldt = log_dtilde;
    a.n_centres = (int)n_centres;
    a.n_edges = n_edges;
    a.nnei_cap = nnei_cap;
    a.layers = layers;
    a.status = status;
    a.one = 1.0;
    const int d = c / heads;
    if (d == 8) {
        switch (heads) {
            case 1: launch_fused_f64<1, 8>(a, s); break;
            case 2: launch_fused_f64<2, 8>(a, s); break;
            case 3: launch_fused_f64<3, 8>(a, s); break;
            default: launch_fused_f64<4, 8>(a, s); break;
        }
    } else {
        if (heads == 1) launch_fused_f64<1, 16>(a, s);
        else launch_fused_f64<2, 16>(a, s);
    }
    return last_launch_status();
}

}  // namespace nga
