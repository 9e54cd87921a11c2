// Fused per-centre block attention, fp32 results, 16-wide heads, on the f16 matrix cores with
// every contraction operand carried as an f16 (hi, lo) pair.  This is the NGA_F32_SPLIT16
// arithmetic, asked for by that dtype only: NGA_F32 runs the fp32 matrix-core kernel of
// block_attn_f32.hip.
//
// deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than dense ...", section
// "Proposed fix: block-dense attention on the graph": gather a centre's (nnei, c) block
// through the destination CSR, dense attention math with a mask for the ragged tail,
// scatter back to the edge axis.  Here one work-group runs a centre's whole layer stack:
// the block is gathered once into LDS, intermediate layers hand their output back through
// the same LDS rows, and only the last layer writes to HBM.
//
// Work-group = H wavefronts, wavefront h owns head h (columns 16h .. 16h+15).
//
// Every contraction -- the projections Q, K, V, Y and the scores S and weighted values O --
// runs on the f16 matrix cores, v_mfma_f32_16x16x32_f16 with fp32 accumulation, on operands
// split into two f16 parts v = hi + lo after scaling by a power of two:
//   block rows      2^ex per centre and layer (max |x| 2^ex in [2^13, 2^14));
//   weights         2^e per matrix;
//   K               per head, from max |K| over the centre;
//   Q               per query (one lane row), from max |Q| over the head's channels;
//   V and O         per centre, from max |V| (every O row is a convex combination of V rows);
//   P               2^13 (P <= 1 before scaling), folded into the exponent argument.
// All four partial products go in: one MFMA takes [a_hi, a_lo] . [b_hi, b_lo], a second one
// [a_hi, a_lo] . [b_lo, b_hi].  The pair of parts carries 21 or more significant bits; parts
// below the f16 normal range (the matrix cores flush f16 subnormals) lie under 2^-27 of their
// scale's maximum; every product is exact in the fp32 accumulator.  A 16-deep contraction
// then costs two 16x16x32 f16 MFMAs (16 CU cycles at gfx950's dense f16 rate) where fp32
// needs four 16x16x4 MFMAs (64 CU cycles).
//
// Operand / result layouts of the f16 16x16x32 MFMA: A[i][k] from lane i + 16(k/8),
// element k%8; B[k][j] from lane j + 16(k/8), element k%8; D[i][j] in lane j + 16(i/4),
// register i%4.  With k = 8g + e standing for channel (or key) 4g + e%4, hi part for e < 4
// and lo part for e >= 4, each result is already the next contraction's operand:
//   projections  Q^T = Wq_h^T X^T, K^T = Wk_h^T X^T (A = weights, B = block rows),
//                V = X Wv_h (A = block rows, B = weights), 16-channel chunk u per MFMA pair:
//                lane (g, i) holds Q, K of row i, channels 4g .. 4g+3, and V of rows
//                4g .. 4g+3, channel i;
//   scores       S^T = K Q^T: A = K of key tile t, B = Q of the query tile, both split in
//                place;  lane (g, i) then holds query i against keys 4g .. 4g+3 of tile t;
//   softmax      row max / sum over a lane's registers and the 4 lane groups (2 shuffles);
//   values       O^T = V^T P^T: A = V of key tile t, B = P of tile t, split in place;
//   output       Y^T = Wo^T [O_0 .. O_{H-1}]^T: head hh's O^T (channels 4g .. 4g+3 of query
//                i in lane (g, i)), split and exchanged through LDS, is the B operand of the
//                MFMA pair hh;  lane (g, i) gets 4 consecutive output channels of row i.
// K and V of every key tile stay in registers, split, for the whole layer; Q is formed one
// query tile at a time.  Rows past the centre's length are zeros in LDS, their keys are
// masked to -inf and their outputs are never stored.
//
// On gfx950 a wavefront's own MFMA and VALU instructions do not overlap (an MFMA followed by
// independent VALU work costs the sum of the two); only another wavefront on the same SIMD can
// issue VALU work while an MFMA runs.  Here MFMA busy (~35%) and VALU busy (~75%) nearly add
// up to the kernel time, so every VALU instruction of the query loop counts: contractions
// accumulate in a single chain, 1/Z uses the hardware reciprocal, and the splits use packed
// conversions and mixed-precision FMAs.
#include "block_attn_fused.h"

#include <climits>

namespace nga {

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ inline f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ inline f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Power-of-two exponent e with max |v| * 2^e in [2^13, 2^14); 0 for v == 0 and for a
// non-finite maximum (the infinity then reaches the output as inf or NaN, as in fp32 math).
// Split parts of values within 2^16 of the maximum then stay normal f16 numbers (the matrix
// cores flush f16 subnormals), and the largest part stays far below the f16 maximum.
__device__ inline int scale_exponent(float vmax) {
    return vmax > 0.f && vmax <= 3.402823466e38f ? 13 - ilogbf(vmax) : 0;
}

constexpr float kLog2e = 1.4426950408889634f;

// f16 (hi, lo) pair of v: hi is v rounded to f16, lo the remainder v - hi (exact in f32) rounded
// to f16.  The empty asm pins v as one rounded f32 value: otherwise the compiler may fold the
// product that made v into each conversion on its own (mixed-precision FMA with the unrounded
// product), and at an f16 rounding tie the stored hi and the hi subtracted for lo then differ
// by one f16 ulp.
__device__ inline h2 split_f16(float v) {
    asm("" : "+v"(v));
    const _Float16 hi = (_Float16)v;
    return h2{hi, (_Float16)(v - (float)hi)};
}

// Weights split into f16 (hi, lo) parts after scaling each matrix by 2^e (max |W| 2^e in
// [2^13, 2^14)).  Operand of wavefront h, lane L = 16g + i, chunk u: 8 halves, the hi parts
// of W[16u + 4g + e][16h + i] for e = 0..3 followed by their lo parts.  One work-group per
// (layer, matrix); the exponent goes to expo[layer * 4 + m].
__global__ void __launch_bounds__(256)
pack_weights_kernel(const float* __restrict__ w, int C, int H, float* __restrict__ packed_f,
                    int* __restrict__ expo) {
    __shared__ float red[4];
    const int lm = blockIdx.x;
    const float* W = w + (size_t)lm * C * C;
    float mx = 0.f;
    for (int idx = threadIdx.x; idx < C * C; idx += 256) mx = fmaxf(mx, fabsf(W[idx]));
    for (int d = 32; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = scale_exponent(mx);
    if (threadIdx.x == 0) expo[lm] = e;
    h8* packed = reinterpret_cast<h8*>(packed_f) + (size_t)lm * H * 64 * (C / 16);
    const int total = H * 64 * (C / 16);
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int u = idx % (C / 16);
        const int lane = (idx / (C / 16)) % 64;
        const int h = idx / (C / 16) / 64;
        const int g = lane >> 4, i = lane & 15;
        h8 op;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const h2 p = split_f16(ldexpf(W[(size_t)(16 * u + 4 * g + q) * C + 16 * h + i], e));
            op[q] = p[0];
            op[4 + q] = p[1];
        }
        packed[idx] = op;
    }
}

struct FusedArgs {
    const int64_t* row_ptr;
    const int32_t* order;
    const float* x;
    float* y;
    const float* w;  // packed split weights
    const int* expo;
    int n_centres;
    int64_t n_edges;
    int nnei_cap;
    int layers;
    const float* ldt;  // smooth attention: ln D~ [layers][n_edges][H], or NULL
    uint32_t* status;
};

// Smooth attention rescales each (query, head) output by sum_j e_j / D~, so O is no longer a
// convex combination of V rows and max |V| no longer bounds it.  Its instances give every
// query row its own power-of-two scale instead, common to the row's heads: each head's O row
// is formed as (fraction in [1, 2) of the factor) * O, its magnitude ilogb(max |O|) plus the
// factor's power of two goes through LDS, and the largest over the heads fixes the shift that
// brings that row to [2^13, 2^14) before the split.  Y is shifted back by the same power.
constexpr int kNoMagnitude = INT_MIN / 2;

// LDS block row: 64 hi halves, 64 lo halves, 16 bytes of padding (272 bytes) -- or, between
// layers, the row's C floats.
// Slot of 8-byte chunk k (channels 4k .. 4k+3) in the hi and in the lo halves of block row a:
// rows 8..15 of every 16-row tile swap neighbouring chunks.  An operand read has lane
// (g, i) take chunk g (plus a multiple of 4) of row i; with the 272-byte row stride rows i and
// i+8 of a tile would otherwise fall on the same LDS banks.
__device__ inline int chunk_slot(int k, int a) { return k ^ ((a >> 3) & 1); }

template <int H>
struct Lds {
    static constexpr int C = 16 * H;
    static constexpr int RB = 4 * C + 16;  // row bytes
};

// [hi, lo] f16 operand of the four values w.  hi: the values rounded toward zero to f16 by
// the packed conversion; lo: w - hi (exact in fp32) rounded to f16.  Any hi works as long as
// lo is taken from that same hi.  The multiply by an opaque 1.0 lets the compiler form each lo
// half with one mixed-precision FMA reading fp32 w and one f16 half of hi.
__device__ inline h8 split4_unscaled(f4 w) {
    float one = 1.0f;
    asm("" : "+v"(one));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm("" : "+v"(w[i]));
    const h2 h01 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(w[0], w[1]));
    const h2 h23 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(w[2], w[3]));
    h8 r;
    r[0] = h01[0]; r[1] = h01[1]; r[2] = h23[0]; r[3] = h23[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[4 + i] = (_Float16)__builtin_fmaf(w[i], one, -(float)r[i]);
    return r;
}

// The same for the four values v * 2^e.
__device__ inline h8 split4(f4 v, int e) {
    f4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = ldexpf(v[i], e);
    return split4_unscaled(w);
}

__device__ inline h8 swap_halves(h8 v) {
    return __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
}

__device__ inline h8 dup_read(const unsigned char* p) {
    const h4 v = *reinterpret_cast<const h4*>(p);
    return h8{v[0], v[1], v[2], v[3], v[0], v[1], v[2], v[3]};
}

template <int H, int NT, bool SMOOTH>
__device__ __forceinline__ void centre_layer(const FusedArgs& A, const h8* __restrict__ P,
                                             const int layer, const int ex, const int64_t r0,
                                             const int n, const bool last,
                                             unsigned char* __restrict__ sX,
                                             h8 (*__restrict__ sO)[H][64],
                                             h8 (*__restrict__ sWoh)[64], float* red,
                                             int (*__restrict__ sMag)[16], const int lane,
                                             const int h) {
    constexpr int C = 16 * H;
    constexpr int U = C / 16;
    constexpr int RB = Lds<H>::RB;
    constexpr int MAT = H * 64 * U;  // h8 per packed matrix
    const int g = lane >> 4;
    const int li = lane & 15;
    // Byte offset of this lane's channels 4g .. 4g+3 within the hi (and lo) halves of its
    // block row 16t + li, chunks swizzled as chunk_slot.
    const int xo = 8 * chunk_slot(g, li);
    const int eq = A.expo[4 * layer + 0], ek = A.expo[4 * layer + 1];
    const int ev = A.expo[4 * layer + 2], eo = A.expo[4 * layer + 3];
    // K and Q leave the projections scaled by 2^(ex + ek) and 2^(ex + eq); values and outputs
    // by 2^(ex + ev) and 2^(ex + ev + eo).

    h8 wq[U], wk[U], wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        wq[u] = P[0 * MAT + u];
        wk[u] = P[1 * MAT + u];
        wv[u] = P[2 * MAT + u];
        sWoh[u][lane] = P[3 * MAT + u];
    }

    f4 kt[NT], vt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const unsigned char* row = sX + (16 * t + li) * RB;
        f4 k = {0.f, 0.f, 0.f, 0.f}, v = k;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const h8 xh = dup_read(row + 32 * u + xo);
            const h8 xl = dup_read(row + 2 * C + 32 * u + xo);
            k = mfma16(wk[u], xh, k);
            k = mfma16(wk[u], xl, k);
            v = mfma16(xh, wv[u], v);
            v = mfma16(xl, wv[u], v);
        }
        kt[t] = k;
        vt[t] = v;
    }
    // K rescaled per head (max |K| over the centre to [2^13, 2^14)) and split: lane (i, g) of
    // key tile t then holds [K_hi, K_lo] of key 16t + i, channels 4g .. 4g+3, which is the A
    // operand of S^T = K Q^T on the f16 cores.
    float kmax = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) kmax = fmaxf(kmax, fabsf(kt[t][r]));
    for (int d = 32; d > 0; d >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, d, 64));
    const int e_k = scale_exponent(kmax);
    h8 ka[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ka[t] = split4(kt[t], e_k);

    // O is a convex combination of V rows, so max |V| over the centre bounds it: the scale
    // that brings that bound to [2^13, 2^14) is shared by every head for the output projection.
    float vmax = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) vmax = fmaxf(vmax, fabsf(vt[t][r]));
    for (int d = 32; d > 0; d >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, d, 64));
    if (lane == 0) red[h] = vmax;
    __syncthreads();
    vmax = red[0];
#pragma unroll
    for (int w = 1; w < H; ++w) vmax = fmaxf(vmax, red[w]);
    const int e_o = scale_exponent(vmax);
    const float yscale = ldexpf(1.f, -(ex + ev + e_o + eo));
    // V at that scale, split: lane (i, g) of key tile t holds [V_hi, V_lo] of keys
    // 16t + 4g .. 16t + 4g + 3, channel i -- the A operand of O^T = V^T P^T.
    h8 va[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) va[t] = split4(vt[t], e_o);

    for (int qt = 0; qt < NT; ++qt) {
        f4 q = {0.f, 0.f, 0.f, 0.f};
        {
            const unsigned char* row = sX + (16 * qt + li) * RB;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const h8 xh = dup_read(row + 32 * u + xo);
                const h8 xl = dup_read(row + 2 * C + 32 * u + xo);
                q = mfma16(wq[u], xh, q);
                q = mfma16(wq[u], xl, q);
            }
        }
        // Q rescaled per query (lane (i, g) holds channels 4g .. 4g+3 of query i; the scale
        // is shared by the 4 lane groups) and split: the B operand of S^T = K Q^T.
        float qm = fmaxf(fmaxf(fabsf(q[0]), fabsf(q[1])), fmaxf(fabsf(q[2]), fabsf(q[3])));
        qm = fmaxf(qm, __shfl_xor(qm, 16, 64));
        qm = fmaxf(qm, __shfl_xor(qm, 32, 64));
        const int e_q = scale_exponent(qm);
        const h8 qa = split4(q, e_q);
        const h8 qb = swap_halves(qa);
        const float c1 = ldexpf(kLog2e * 0.25f, -(2 * ex + eq + ek + e_k + e_q));
        f4 s[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // [K_hi, K_lo] . [Q_hi, Q_lo] + [K_hi, K_lo] . [Q_lo, Q_hi]
            f4 acc = mfma16(ka[t], qa, f4{0.f, 0.f, 0.f, 0.f});
            s[t] = mfma16(ka[t], qb, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (16 * (NT - 1) + 4 * g + r >= n) s[NT - 1][r] = -INFINITY;
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, s[t][r]);
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        // P scaled by 2^13 (max P = 2^13) so that its split parts stay normal f16 numbers.
        const float mc = m * c1 - 13.f;
        float z = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[t][r] * c1 - mc);
                s[t][r] = p;
                z += p;
            }
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        f4 osum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // [V_hi, V_lo] . [P_hi, P_lo] + [V_hi, V_lo] . [P_lo, P_hi]
            const h8 pa = split4_unscaled(s[t]);
            osum = mfma16(va[t], pa, osum);
            osum = mfma16(va[t], swap_halves(pa), osum);
        }
        f4 o;
        int e_row = 0;  // smooth: the query row's shift, common to its heads
        if constexpr (SMOOTH) {
            // sum_j e_j / D~ times the softmax = exp(s_j - ln D~): in place of 1/Z the factor
            // 2^t, t = m c1 - 13 - log2(e) ln D~ (P carries 2^13 and the row max), taken as
            // 2^k * 2^(t - k) with k = floor(t).
            const int aq = 16 * qt + li;
            float frac = 0.f;
            int k = 0;
            if (aq < n) {
                const int64_t row = A.order ? (int64_t)A.order[r0 + aq] : r0 + aq;
                if (row >= 0 && row < A.n_edges) {
                    const float t = mc - kLog2e * A.ldt[((int64_t)layer * A.n_edges + row) * H + h];
                    const float kf = floorf(fminf(fmaxf(t, -4096.f), 4096.f));
                    frac = exp2f(t - kf);
                    k = (int)kf;
                }
            }
            o = osum * frac;
            float om = fmaxf(fmaxf(fabsf(o[0]), fabsf(o[1])), fmaxf(fabsf(o[2]), fabsf(o[3])));
            om = fmaxf(om, __shfl_xor(om, 16, 64));
            om = fmaxf(om, __shfl_xor(om, 32, 64));
            // A zero row has no magnitude; a non-finite one keeps its scale (the infinity or
            // NaN reaches y as in fp32 arithmetic).
            const int mag = om > 0.f && om <= 3.402823466e38f ? ilogbf(om) + k : kNoMagnitude;
            if (g == 0) sMag[h][li] = mag;
            __syncthreads();
            int top = sMag[0][li];
#pragma unroll
            for (int w = 1; w < H; ++w) top = max(top, sMag[w][li]);
            e_row = top == kNoMagnitude ? 0 : 13 - top;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = ldexpf(o[r], k + e_row);
        } else {
            o = osum * __builtin_amdgcn_rcpf(z);
        }

        h8 os;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const h2 p = split_f16(o[r]);
            os[r] = p[0];
            os[4 + r] = p[1];
        }
        const int buf = qt & 1;
        sO[buf][h][lane] = os;
        __syncthreads();
        f4 yv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
            const h8 oo = sO[buf][hh][lane];
            const h8 oh = h8{oo[0], oo[1], oo[2], oo[3], oo[0], oo[1], oo[2], oo[3]};
            const h8 ol = h8{oo[4], oo[5], oo[6], oo[7], oo[4], oo[5], oo[6], oo[7]};
            const h8 wo = sWoh[hh][lane];
            yv = mfma16(wo, oh, yv);
            yv = mfma16(wo, ol, yv);
        }
        if constexpr (SMOOTH) {
            const int back = -(ex + ev + e_o + eo) - e_row;
#pragma unroll
            for (int r = 0; r < 4; ++r) yv[r] = ldexpf(yv[r], back);
        } else {
            yv *= yscale;
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
            *reinterpret_cast<f4*>(sX + a * Lds<H>::RB + 4 * (16 * h + 4 * g)) = a < n ? yv : zero;
        }
    }
}

// Split the block's rows (held as floats in vals, PER float4 chunks per thread) into hi/lo
// halves at the block's power-of-two scale; returns the exponent.
template <int H, int PER>
__device__ inline int split_block(f4 (&vals)[PER], int chunks, unsigned char* sX, float* red) {
    constexpr int C = 16 * H;
    constexpr int CH = C / 4;
    constexpr int NTH = 64 * H;
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(vals[j][i]));
    for (int d = 32; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < H; ++w) mx = fmaxf(mx, red[w]);
    const int e = scale_exponent(mx);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int idx = threadIdx.x + j * NTH;
        if (idx >= chunks) continue;
        const int a = idx / CH, c4 = idx % CH;
        h4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h2 p = split_f16(ldexpf(vals[j][i], e));
            hi[i] = p[0];
            lo[i] = p[1];
        }
        unsigned char* row = sX + a * Lds<H>::RB;
        const int slot = chunk_slot(c4, a);
        *reinterpret_cast<h4*>(row + 8 * slot) = hi;
        *reinterpret_cast<h4*>(row + 2 * C + 8 * slot) = lo;
    }
    return e;
}

template <int H, int TMAX, bool SMOOTH>
__global__ void __launch_bounds__(64 * H, 2) fused_f32_split16_kernel(FusedArgs A) {
    constexpr int C = 16 * H;
    constexpr int U = C / 16;
    constexpr int NTH = 64 * H;
    constexpr int CH = C / 4;
    constexpr int PER = (16 * TMAX * CH + NTH - 1) / NTH;
    __shared__ __align__(16) unsigned char sX[16 * TMAX * Lds<H>::RB];
    __shared__ h8 sO[2][H][64];
    __shared__ h8 sWo[H][U][64];
    __shared__ float red[H];
    __shared__ int sMag[H][16];

    const int lane = threadIdx.x & 63;
    const int h = threadIdx.x >> 6;

    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (A.row_ptr[0] != 0 || A.row_ptr[A.n_centres] > A.n_edges) raise_bits(A.status, kBitCap);
    }
    bool bad_index = false;
    {
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
        const int chunks = 16 * nt * CH;
        f4 v[PER];
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
        int ex = split_block<H, PER>(v, chunks, sX, red);
        __syncthreads();

        for (int layer = 0; layer < A.layers; ++layer) {
            const h8* P = reinterpret_cast<const h8*>(A.w) + (size_t)layer * 4 * H * 64 * U +
                          ((size_t)h * 64 + lane) * U;
            const bool last = layer == A.layers - 1;
#define NGA_CASE(T)                                                                            \
    case T:                                                                                    \
        if constexpr (T <= TMAX)                                                               \
            centre_layer<H, T, SMOOTH>(A, P, layer, ex, r0, n, last, sX, sO, sWo[h], red, sMag, \
                                       lane, h);                                               \
        break;
            switch (nt) {
                NGA_CASE(1) NGA_CASE(2) NGA_CASE(3) NGA_CASE(4) NGA_CASE(5) NGA_CASE(6)
                NGA_CASE(7) NGA_CASE(8) NGA_CASE(9) NGA_CASE(10) NGA_CASE(11) NGA_CASE(12)
                default: break;
            }
#undef NGA_CASE
            __syncthreads();
            if (!last) {
                // The rows now hold this layer's output as floats: re-split for the next.
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const int idx = threadIdx.x + j * NTH;
                    const int a = idx / CH, c4 = idx % CH;
                    v[j] = f4{0.f, 0.f, 0.f, 0.f};
                    if (idx < chunks)
                        v[j] = *reinterpret_cast<const f4*>(sX + a * Lds<H>::RB + 16 * c4);
                }
                __syncthreads();
                ex = split_block<H, PER>(v, chunks, sX, red);
                __syncthreads();
            }
        }
    }
    if (bad_index) raise_bits(A.status, kBitIndex);
}

template <int H, bool SMOOTH>
int launch_hs(int tmax, const FusedArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_centres), block(64 * H);
    if (tmax <= 4)
        hipLaunchKernelGGL((fused_f32_split16_kernel<H, 4, SMOOTH>), grid, block, 0, s, a);
    else if (tmax <= 8)
        hipLaunchKernelGGL((fused_f32_split16_kernel<H, 8, SMOOTH>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((fused_f32_split16_kernel<H, 12, SMOOTH>), grid, block, 0, s, a);
    return last_launch_status();
}

template <int H>
int launch_h(int tmax, const FusedArgs& a, hipStream_t s) {
    return a.ldt ? launch_hs<H, true>(tmax, a, s) : launch_hs<H, false>(tmax, a, s);
}

}  // namespace

bool fused_supported(int dtype, int32_t nnei_cap, int32_t c, int32_t heads) {
    if (dtype != NGA_F32_SPLIT16) return false;
    if (heads < 1 || c != 16 * heads) return false;
    if (heads != 1 && heads != 2 && heads != 4) return false;
    return nnei_cap >= 1 && nnei_cap <= 16 * 12;
}

const char* fused_name(int dtype, int32_t c, int32_t heads) {
    (void)dtype; (void)c; (void)heads;
    return "fused_f32_split16";
}

size_t fused_workspace_floats(int32_t c, int32_t layers) { return (size_t)layers * 4 * c * c + 64 + 4 * layers; }

int run_fused(int dtype, const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
              int64_t n_edges, int32_t nnei_cap, int32_t c, int32_t heads, int32_t layers,
              const void* weights, const void* x, const void* log_dtilde, void* y, void* packed,
              uint32_t* status, hipStream_t s) {
    (void)dtype;
    float* pk = static_cast<float*>(packed);
    int* expo = reinterpret_cast<int*>(pk + (size_t)layers * 4 * c * c);
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)(layers * 4)), dim3(256), 0, s,
                       static_cast<const float*>(weights), (int)c, (int)heads, pk, expo);
    int rc = last_launch_status();
    if (rc) return rc;
    FusedArgs a;
    a.row_ptr = row_ptr;
    a.order = order;
    a.x = static_cast<const float*>(x);
    a.y = static_cast<float*>(y);
    a.w = pk;
    a.expo = expo;
    a.n_centres = (int)n_centres;
    a.n_edges = n_edges;
    a.nnei_cap = nnei_cap;
    a.layers = layers;
    a.ldt = static_cast<const float*>(log_dtilde);
    a.status = status;
    const int tmax = (nnei_cap + 15) / 16;
    switch (heads) {
        case 1: return launch_h<1>(tmax, a, s);
        case 2: return launch_h<2>(tmax, a, s);
        default: return launch_h<4>(tmax, a, s);
    }
}

}  // namespace nga
