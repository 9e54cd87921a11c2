// nl_build: O(N) cell-list neighbour rows under periodic boundaries.
//
// deepmd-kit issue "perf: DPA4 .pt2 LAMMPS (C++ AOTI) inference 3-6x slower than Python
// (ASE) ...", section "Root cause analysis": the fast path builds the neighbour list on the
// GPU with an O(N) cell list; its comments describe the GPU pipeline as distance
// computation, prefix-scan compaction and a dense list fill.  deepmd-kit issue
// "perf: NeighborGraph attention is 4-9x slower than dense ...", section "Measurements":
// each centre keeps its nsel nearest neighbours within rcut.
//
// Pipeline (all on the caller's stream):
//   1. clear per-cell counts
//   2. bin: validate each position, cell id, atomic slot within the cell
//   3. exclusive scan of cell counts -> cell offsets (scan.hip)
//   4. scatter atoms into cell order (positions copied bit for bit)
//      (steps 1-4 are one single-work-group launch for up to 8,192 atoms and 4,096 cells)
//   5. select: one work-group per (cell, split) with the cell's stencil merged into segments
//      in LDS; each wavefront takes one centre at a time (about four per work-group and
//      wavefront), reads the segments' cell-sorted positions with coalesced loads, evaluates
//      the fp64 distance of every candidate, compacts the accepted ones with ballot/mbcnt into
//      a per-wave LDS list, sorts them in registers (bitonic on 32-bit words: a distance
//      class of r2 above the list index, then runs of equal classes re-ranked by the full key
//      (r2, j, shift)) and writes the first min(sel, count) as the row.  Candidates are
//      read in rounds of three 64-wide chunks, per segment, or across segment ends when the
//      segments are short (small boxes, sparse cells).
//
// The distance is d = (x_j - x_i) + n*L per axis, r2 = (dx*dx + dy*dy) + dz*dz, in IEEE
// fp64 with contraction disabled in this file, so every accepted r2 is bit-identical to a
// plain evaluation of the same formula.
#pragma clang fp contract(off)

#include <mutex>

#include "nga_internal.h"

#include <algorithm>
#include <vector>

namespace nga {

namespace {

constexpr int kNlBlock = 256;
constexpr int kNlWaves = kNlBlock / 64;
constexpr int kMaxReach = 5;     // stencil reach (cells) per side
constexpr double kCellSlack = 1e-9;  // cells are at least rcut * (1 + slack) wide
constexpr int kMaxCellsPerAxis = 1024;
constexpr int64_t kTrimMinAtoms = 512;  // smaller systems keep whole-cell stencils

struct Geom {
    double L[3];
    double inv_h[3];
    double h[3];
    int nc[3];
    int reach[3];
    int stencil;
    int64_t ncells;
    int trim;  // > 0: cells of at least rcut / 2, per-centre stencils of reach `trim`
};

// Cells per axis: as many as keep the cell edge >= rcut * (1 + slack), capped so that the
// cell arrays stay O(N).  The stencil reach k covers every cell whose nearest point can be
// within rcut * (1 + slack): k = ceil(rcut * (1 + slack) / h).  Binning rounds positions
// to cells with an error of a few ulps of L, far below the slack, so no pair within rcut is
// missed.
//
// With `trim`, a single structure whose box holds at least five cells of edge rcut / 2 per
// axis is binned into those cells instead (reach 2, or 1 where capping made them wider), and
// selection takes each centre's own stencil: only the cells whose nearest point can be within
// rcut of that centre (select_trim_kernel).
bool make_geom_cells(int64_t n_atoms, const double* box, double rcut, double div, Geom* g);

bool make_geom(int64_t n_atoms, const double* box, double rcut, Geom* g, bool trim = false) {
    if (trim && make_geom_cells(n_atoms, box, rcut, 2.0, g)) {
        int k = 1;
        for (int a = 0; a < 3; ++a) k = std::max(k, g->reach[a]);
        bool ok = k <= 2;
        for (int a = 0; a < 3; ++a) ok = ok && g->nc[a] >= 2 * k + 1;
        if (ok && n_atoms >= kTrimMinAtoms) {
            g->trim = k;
            return true;
        }
    }
    if (!make_geom_cells(n_atoms, box, rcut, 1.0, g)) return false;
    g->trim = 0;
    return true;
}

// Cells of edge at least rcut * (1 + slack) / div per axis.
bool make_geom_cells(int64_t n_atoms, const double* box, double rcut, double div, Geom* g) {
    if (!box || !(std::isfinite(rcut) && rcut > 0.0) || n_atoms < 0 || n_atoms >= INT32_MAX)
        return false;
    const double rc = rcut * (1.0 + kCellSlack);
    int64_t cap = std::max<int64_t>(64, 2 * n_atoms);
    for (int a = 0; a < 3; ++a) {
        if (!finite_pos(box[a])) return false;
        if (box[a] / rcut > 1e7) return false;
        double q = std::floor(box[a] * div / rc);
        g->nc[a] = (int)std::max(1.0, std::min(q, (double)kMaxCellsPerAxis));
        g->L[a] = box[a];
    }
    while ((int64_t)g->nc[0] * g->nc[1] * g->nc[2] > cap) {
        int a = 0;
        for (int b = 1; b < 3; ++b)
            if (g->nc[b] > g->nc[a]) a = b;
        g->nc[a] = (g->nc[a] + 1) / 2;
    }
    g->stencil = 1;
    for (int a = 0; a < 3; ++a) {
        double h = g->L[a] / g->nc[a];
        g->h[a] = h;
        g->inv_h[a] = (double)g->nc[a] / g->L[a];
        int k = (int)std::ceil(rc / h);
        if (k < 1) k = 1;
        if (k > kMaxReach) return false;
        g->reach[a] = k;
        g->stencil *= 2 * k + 1;
    }
    g->ncells = (int64_t)g->nc[0] * g->nc[1] * g->nc[2];
    return true;
}

struct WsLayout {
    int32_t* cell_count;
    int64_t* tile_sums;
    int64_t* cell_start;
    int32_t* atom_cell;
    int32_t* atom_slot;
    // Cell-sorted atoms, 32 bytes each: x, y, z and the atom index (its integer bits in the
    // fourth double), so that a candidate is two 16-byte loads.
    double* sa;
    size_t bytes;
};

typedef double d2 __attribute__((ext_vector_type(2)));

// Atom i at sorted slot d of the cell-sorted array.
__device__ inline void store_sorted(double* __restrict__ sa, int64_t d, const double* pos,
                                    int64_t i) {
    d2* o = reinterpret_cast<d2*>(sa) + 2 * d;
    o[0] = d2{pos[3 * i + 0], pos[3 * i + 1]};
    o[1] = d2{pos[3 * i + 2], __longlong_as_double((long long)i)};
}

WsLayout carve(void* ws, int64_t n, const Geom& g) {
    Carver cv(ws);
    WsLayout w;
    w.cell_count = cv.take<int32_t>(g.ncells);
    w.tile_sums = cv.take<int64_t>(scan_tiles(g.ncells) + 1);
    w.cell_start = cv.take<int64_t>(g.ncells + 1);
    w.atom_cell = cv.take<int32_t>(n);
    w.atom_slot = cv.take<int32_t>(n);
    w.sa = cv.take<double>(4 * n);
    w.bytes = cv.off;
    return w;
}

__global__ void clear_i32_kernel(int32_t* a, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = 0;
}

__global__ void __launch_bounds__(256)
bin_kernel(const double* __restrict__ pos, int n, Geom g, int32_t* __restrict__ cell_count,
           int32_t* __restrict__ atom_cell, int32_t* __restrict__ atom_slot, uint32_t* status) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    int c[3];
    bool bad = false;
    for (int a = 0; a < 3; ++a) {
        double x = pos[3 * (int64_t)i + a];
        // NaN and +-inf fail one of the two comparisons.
        bool ok = (x >= 0.0) && (x < g.L[a]);
        bad |= !ok;
        int ci = ok ? (int)(x * g.inv_h[a]) : 0;
        c[a] = ci < g.nc[a] ? ci : g.nc[a] - 1;
    }
    if (bad) raise_bits(status, kBitBox);
    int cell = (c[2] * g.nc[1] + c[1]) * g.nc[0] + c[0];
    atom_cell[i] = cell;
    atom_slot[i] = atomicAdd(&cell_count[cell], 1);
}

// A structure of a batch: its geometry, first global cell and first atom.
struct BatchGeom {
    Geom g;
    int64_t cell_base;
    int64_t atom_base;
};

// Last b in [0, nb) with ptr[b] <= v (ptr[0] = 0 <= v, ptr non-decreasing).
__device__ inline int find_segment(const int64_t* ptr, int nb, int64_t v) {
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ptr[mid] <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// bin_kernel for a batch: atom i belongs to the structure whose atom range holds it, and its
// cell index is that structure's first cell plus its cell within the structure's box.
__global__ void __launch_bounds__(256)
bin_batch_kernel(const double* __restrict__ pos, int n, const BatchGeom* __restrict__ table,
                 const int64_t* __restrict__ atom_ptr, int n_structs,
                 int32_t* __restrict__ cell_count, int32_t* __restrict__ atom_cell,
                 int32_t* __restrict__ atom_slot, uint32_t* status) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int b = find_segment(atom_ptr, n_structs, i);
    const Geom& g = table[b].g;
    int c[3];
    bool bad = false;
    for (int a = 0; a < 3; ++a) {
        double x = pos[3 * (int64_t)i + a];
        bool ok = (x >= 0.0) && (x < g.L[a]);
        bad |= !ok;
        int ci = ok ? (int)(x * g.inv_h[a]) : 0;
        c[a] = ci < g.nc[a] ? ci : g.nc[a] - 1;
    }
    if (bad) raise_bits(status, kBitBox);
    int cell = (int)table[b].cell_base + (c[2] * g.nc[1] + c[1]) * g.nc[0] + c[0];
    atom_cell[i] = cell;
    atom_slot[i] = atomicAdd(&cell_count[cell], 1);
}

__global__ void __launch_bounds__(256)
scatter_kernel(const double* __restrict__ pos, int n, const int64_t* __restrict__ cell_start,
               const int32_t* __restrict__ atom_cell, const int32_t* __restrict__ atom_slot,
               double* __restrict__ sa) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    store_sorted(sa, cell_start[atom_cell[i]] + atom_slot[i], pos, i);
}

// Small systems: counting, the exclusive scan of the cell counts and the scatter in one
// work-group, with the counts in LDS, in place of five launches (clear, bin, two scan
// passes, scatter) that each cost more in launch latency than in work.  The order of atoms
// inside a cell differs from the multi-launch path, as it does between any two runs of that
// path's atomics; rows do not depend on it, since each row is sorted by its full key.
constexpr int kSmallThreads = 1024;
constexpr int kSmallPer = 8;                            // atoms per thread
constexpr int kSmallAtoms = kSmallThreads * kSmallPer;  // 8,192
constexpr int kSmallCells = 4096;

__global__ void __launch_bounds__(kSmallThreads)
bin_small_kernel(const double* __restrict__ pos, int n, Geom g, int64_t* __restrict__ cell_start,
                 double* __restrict__ sa, uint32_t* status) {
    __shared__ int32_t s_count[kSmallCells];
    __shared__ int32_t s_wave[kSmallThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nc = (int)g.ncells;
    for (int c = tid; c < nc; c += kSmallThreads) s_count[c] = 0;
    __syncthreads();

    int cell[kSmallPer], slot[kSmallPer];
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        const int i = tid + kSmallThreads * k;
        cell[k] = 0;
        slot[k] = 0;
        if (i < n) {
            int c[3];
            for (int a = 0; a < 3; ++a) {
                const double x = pos[3 * (int64_t)i + a];
                // NaN and +-inf fail one of the two comparisons.
                const bool ok = (x >= 0.0) && (x < g.L[a]);
                bad |= !ok;
                const int ci = ok ? (int)(x * g.inv_h[a]) : 0;
                c[a] = ci < g.nc[a] ? ci : g.nc[a] - 1;
            }
            cell[k] = (c[2] * g.nc[1] + c[1]) * g.nc[0] + c[0];
            slot[k] = atomicAdd(&s_count[cell[k]], 1);
        }
    }
    if (bad) raise_bits(status, kBitBox);
    __syncthreads();

    // Exclusive scan: thread t owns cells t*per .. t*per + per - 1.
    const int per = (nc + kSmallThreads - 1) / kSmallThreads;
    const int c0 = tid * per;
    int mine = 0;
    for (int j = 0; j < per; ++j)
        if (c0 + j < nc) mine += s_count[c0 + j];
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int run = incl - mine, total = 0;
    for (int w = 0; w < kSmallThreads / 64; ++w) {
        if (w < wave) run += s_wave[w];
        total += s_wave[w];
    }
    for (int j = 0; j < per; ++j) {
        if (c0 + j < nc) {
            const int cnt = s_count[c0 + j];
            cell_start[c0 + j] = run;
            s_count[c0 + j] = run;  // this thread's own cells only
            run += cnt;
        }
    }
    if (tid == 0) cell_start[nc] = total;
    __syncthreads();

#pragma unroll
    for (int k = 0; k < kSmallPer; ++k) {
        const int i = tid + kSmallThreads * k;
        if (i < n) store_sorted(sa, s_count[cell[k]] + slot[k], pos, i);
    }
}

// Image shift n packed 8 bits per axis with offset 128: code = (nx+128)<<16 | (ny+128)<<8 |
// (nz+128).  Ordering codes as integers orders shifts lexicographically (nx, ny, nz).
__device__ inline int pack_shift(int nx, int ny, int nz) {
    return ((nx + 128) << 16) | ((ny + 128) << 8) | (nz + 128);
}
__device__ inline int shift_x(int code) { return ((code >> 16) & 255) - 128; }
__device__ inline int shift_y(int code) { return ((code >> 8) & 255) - 128; }
__device__ inline int shift_z(int code) { return (code & 255) - 128; }

struct SelectArgs {
    Geom g;
    const BatchGeom* table;   // batch: per-structure geometry (g unused)
    const int64_t* cell_ptr;  // batch: first global cell per structure, [n_structs + 1]
    int n_structs;
    double rc2;
    int n;
    int sel;
    int nsplit;
    const int64_t* cell_start;
    const double* sa;  // cell-sorted atoms (WsLayout::sa)
    int32_t* nbr;
    int32_t* nbr_shift;
    int32_t* nnei;
    uint32_t* status;
};

struct Stencil {
    int cx, cy, cz;
};

// floor(r / nc) for nc > 0.
__device__ inline int floor_div(int r, int nc) { return r >= 0 ? r / nc : -((-r + nc - 1) / nc); }

// Stencil entry s of the cell (cx, cy, cz): neighbour cell and image shift.
__device__ inline void stencil_entry(int ncx, int ncy, int ncz, int kx, int ky, int kz,
                                     const Stencil& st, int s, int* wcell, int* code) {
    const int wx = 2 * kx + 1, wy = 2 * ky + 1;
    const int rx = st.cx + s % wx - kx;
    const int ry = st.cy + (s / wx) % wy - ky;
    const int rz = st.cz + s / (wx * wy) - kz;
    const int nx = floor_div(rx, ncx), ny = floor_div(ry, ncy), nz = floor_div(rz, ncz);
    *wcell = ((rz - nz * ncz) * ncy + (ry - ny * ncy)) * ncx + (rx - nx * ncx);
    *code = pack_shift(nx, ny, nz);
}

// Per-wavefront candidate list in LDS: r2 bit patterns, neighbour index, shift code, and the
// list index each sorted position came from.
struct WaveList {
    uint64_t r2[NGA_ROW_CAP];
    int32_t j[NGA_ROW_CAP];
    int32_t code[NGA_ROW_CAP];
    uint16_t pay[NGA_ROW_CAP];
};

// The list seen through an LDS pointer: where the sort is a called function rather than
// inlined, a plain reference would leave it generic (flat) memory accesses.
typedef __attribute__((address_space(3))) WaveList LdsList;
__device__ inline LdsList* lds(WaveList& L) { return (LdsList*)&L; }

__device__ inline uint64_t lo_key(const LdsList* L, int p) {
    return ((uint64_t)(uint32_t)L->j[p] << 24) | (uint64_t)(uint32_t)L->code[p];
}

// Sort words: a 23-bit distance class above the 9-bit list index of the candidate.
constexpr int kIndexBits = 9;
static_assert(NGA_ROW_CAP <= (1 << kIndexBits), "list index must fit the sort word");
constexpr uint32_t kIndexMask = (1u << kIndexBits) - 1;
constexpr double kClassMax = (double)((1u << (32 - kIndexBits)) - 2);

// Distance class of r2 in [0, rc2): floor(r2 * 2^23 / rc2), capped below the padding word's
// class.  Non-decreasing in r2, so ordering by class and then re-ranking each run of equal
// classes by the full key gives the full-key order.
__device__ inline uint32_t dist_class(uint64_t r2_bits, double qscale) {
    const double s = __longlong_as_double((long long)r2_bits) * qscale;
    return s < kClassMax ? (uint32_t)s : (uint32_t)kClassMax;
}

// v of lane (this lane xor lx), lx a power of two below 64: lane-local DPP moves within a quad
// for 1 and 2, an LDS-free swizzle within 32 lanes for 4 to 16, a permute for 32.  The sort
// below is a chain of such exchanges, so their latency adds up.
__device__ inline uint32_t xor_lanes(uint32_t v, int lx) {
    switch (lx) {
        case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
        case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
        case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (4 << 10) | 0x1F);
        case 8: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (8 << 10) | 0x1F);
        case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (16 << 10) | 0x1F);
        default: return __shfl_xor(v, lx, 64);
    }
}

// min(a, b) when c = 0, max(a, b) when c = ~0: the median of the three, one v_med3_u32.
__device__ inline uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
    return min(max(a, b), max(min(a, b), c));
}

// Bitonic sort of 64*NS 32-bit words held NS per lane (element e = lane*NS + q), ascending.
// Every compare-exchange is one median-of-three against a per-stage mask word that says
// whether this position keeps the smaller or the larger word.
template <int NS>
__device__ inline void bitonic_sort(uint32_t (&k)[NS], int lane) {
    constexpr int M = 64 * NS;
#pragma unroll
    for (int size = 2; size <= M; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride < NS) {
#pragma unroll
                for (int q = 0; q < NS; ++q) {
                    if (q & stride) continue;
                    const int o = q | stride;
                    // e & size: from q alone below NS, from the lane above
                    const bool ascending = size < NS ? (q & size) == 0 : ((lane * NS) & size) == 0;
                    const uint32_t keep = ascending ? 0u : ~0u;
                    const uint32_t a = k[q], b = k[o];
                    k[q] = med3u(a, b, keep);
                    k[o] = med3u(a, b, ~keep);
                }
            } else {
                const int lx = stride / NS;
                // e & size and e & stride come from the lane (size > stride >= NS)
                const bool ascending = ((lane * NS) & size) == 0;
                const bool lower = ((lane * NS) & stride) == 0;
                const uint32_t keep = lower == ascending ? 0u : ~0u;
#pragma unroll
                for (int q = 0; q < NS; ++q) k[q] = med3u(xor_lanes(k[q], lx), k[q], keep);
            }
        }
    }
}

__device__ inline void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Full key of list entry p, compared as (r2 bit pattern, j, shift code).
__device__ inline bool full_less(const LdsList* L, int a, int b) {
    if (L->r2[a] != L->r2[b]) return L->r2[a] < L->r2[b];
    return lo_key(L, a) < lo_key(L, b);
}

// Sort the wave's `count` candidates by (r2, j, shift) and write the first `keep` as row i.
// The bitonic network sorts one 32-bit word per candidate: its distance class (dist_class,
// qscale = 2^23 / rc2) above its list index.  Entries whose class equals a neighbour's are
// then re-ranked inside their run by the full key (runs are rare: classes are rc2 * 2^-23
// wide, so it takes r2 values within about 1e-5 A^2 of each other at rcut = 8 A, such as the
// exact ties of ideal lattices).
template <int NS>
__device__ void sort_and_write(LdsList* L, int count, int keep, int sel, double qscale,
                               int32_t* row, int32_t* rsh, int lane) {
    uint32_t k[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int e = lane * NS + q;
        k[q] = e < count ? (dist_class(L->r2[e], qscale) << kIndexBits) | (uint32_t)e : ~0u;
    }
    bitonic_sort<NS>(k, lane);

    const uint32_t prev_last = __shfl_up(k[NS - 1], 1, 64);
    bool tie = false;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int e = lane * NS + q;
        const uint32_t before = q > 0 ? k[q - 1] : prev_last;
        if (e > 0 && e < count && (before >> kIndexBits) == (k[q] >> kIndexBits)) tie = true;
    }
    int pos[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) pos[q] = lane * NS + q;
    if (__ballot(tie)) {
        // Publish the sorted list indices, then rank each entry of a run of equal classes by
        // the full key.
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int e = lane * NS + q;
            if (e < count) L->pay[e] = (uint16_t)(k[q] & kIndexMask);
        }
        wave_sync_lds();
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int e = lane * NS + q;
            if (e >= count) continue;
            const uint32_t cls = k[q] >> kIndexBits;
            const int me = (int)(k[q] & kIndexMask);
            int rs = e, re = e + 1;
            while (rs > 0 && dist_class(L->r2[L->pay[rs - 1]], qscale) == cls) --rs;
            while (re < count && dist_class(L->r2[L->pay[re]], qscale) == cls) ++re;
            if (re - rs == 1) continue;
            int rank = 0;
            for (int t = rs; t < re; ++t) rank += full_less(L, L->pay[t], me);
            pos[q] = rs + rank;
        }
    }

#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int e = lane * NS + q;
        if (e < count) {
            const int at = pos[q];
            if (at < keep) {
                const int p = (int)(k[q] & kIndexMask);
                const int code = L->code[p];
                row[at] = L->j[p];
                rsh[3 * at + 0] = shift_x(code);
                rsh[3 * at + 1] = shift_y(code);
                rsh[3 * at + 2] = shift_z(code);
            }
        } else if (e < sel) {
            row[e] = -1;
            rsh[3 * e + 0] = 0; rsh[3 * e + 1] = 0; rsh[3 * e + 2] = 0;
        }
    }
    for (int e = 64 * NS + lane; e < sel; e += 64) {
        row[e] = -1;
        rsh[3 * e + 0] = 0; rsh[3 * e + 1] = 0; rsh[3 * e + 2] = 0;
    }
}

// One work-group per (cell, split).  The cell's stencil (start, length, shift code per
// neighbour cell) goes to LDS once; then each wavefront takes one centre of the cell at a
// time and walks the stencil cells, reading their cell-sorted positions with coalesced
// loads, testing the pinned fp64 distance and compacting the accepted candidates into its
// LDS list with ballot / mbcnt.
// BATCH: the cells of several structures, each block finding its structure's geometry.
template <bool BATCH, bool FLAT>
__global__ void __launch_bounds__(kNlBlock)
select_kernel(SelectArgs A) {
    const int gcell = blockIdx.x;
    const int c0 = (int)A.cell_start[gcell];
    const int c1 = (int)A.cell_start[gcell + 1];
    if (c0 == c1 || (int)blockIdx.y * kNlWaves >= c1 - c0) return;  // uniform per block
    Geom g;
    int cbase = 0;
    if constexpr (BATCH) {
        const int b = find_segment(A.cell_ptr, A.n_structs, gcell);
        g = A.table[b].g;
        cbase = (int)A.cell_ptr[b];
    } else {
        g = A.g;
    }

    extern __shared__ __align__(16) unsigned char nl_smem[];
    WaveList* lists = reinterpret_cast<WaveList*>(nl_smem);
    int* s_start = reinterpret_cast<int*>(nl_smem + kNlWaves * sizeof(WaveList));
    int* s_len = s_start + g.stencil;
    int* s_code = s_len + g.stencil;

    const int ncx = g.nc[0], ncy = g.nc[1], ncz = g.nc[2];
    const int cell = gcell - cbase;
    Stencil st;
    st.cx = cell % ncx;
    st.cy = (cell / ncx) % ncy;
    st.cz = cell / (ncx * ncy);
    const int S = g.stencil;
    // Merge stencil cells that follow each other in memory with the same image shift (the
    // cells of one x-row away from the box edge) into one segment; empty cells drop out.
    __shared__ int s_nseg;
    if (S <= 64) {
        // One wavefront: entry e in lane e; a non-empty entry starts a segment unless the
        // previous non-empty entry has its shift and ends where it begins.
        if (threadIdx.x < 64) {
            const int e = threadIdx.x;
            int b = 0, l = 0, code = -1;
            if (e < S) {
                int w;
                stencil_entry(ncx, ncy, ncz, g.reach[0], g.reach[1], g.reach[2], st, e, &w,
                              &code);
                const int64_t b64 = A.cell_start[cbase + w];
                b = (int)b64;
                l = (int)(A.cell_start[cbase + w + 1] - b64);
            }
            const bool filled = l > 0;
            const uint64_t below = e == 0 ? 0ull : (~0ull >> (64 - e));
            const uint64_t fm = __ballot(filled);
            const uint64_t fb = fm & below;
            const int pe = fb ? 63 - __clzll(fb) : e;  // previous non-empty entry
            const int pb = __shfl(b, pe, 64), pl = __shfl(l, pe, 64), pc = __shfl(code, pe, 64);
            const bool head = filled && (fb == 0 || pc != code || pb + pl != b);
            const uint64_t hm = __ballot(head);
            // The segment headed here ends with the last non-empty entry before the next head.
            const uint64_t after = e == 63 ? 0ull : (hm & (~0ull << (e + 1)));
            const int nh = after ? __ffsll((long long)after) - 1 : 64;
            const uint64_t upto = fm & (nh == 64 ? ~0ull : ((1ull << nh) - 1));
            const int last = upto ? 63 - __clzll(upto) : e;
            const int end = __shfl(b + l, last, 64);
            if (head) {
                const int sid = __popcll(hm & below);
                s_start[sid] = b;
                s_len[sid] = end - b;
                s_code[sid] = code;
            }
            if (e == 0) s_nseg = __popcll(hm);
        }
    } else {
        for (int e = threadIdx.x; e < S; e += kNlBlock) {
            int w, code;
            stencil_entry(ncx, ncy, ncz, g.reach[0], g.reach[1], g.reach[2], st, e, &w, &code);
            const int64_t b = A.cell_start[cbase + w];
            s_start[e] = (int)b;
            s_len[e] = (int)(A.cell_start[cbase + w + 1] - b);
            s_code[e] = code;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int nseg = 0;
            for (int e = 0; e < S; ++e) {
                const int b = s_start[e], l = s_len[e], code = s_code[e];
                if (l == 0) continue;
                if (nseg > 0 && s_code[nseg - 1] == code &&
                    s_start[nseg - 1] + s_len[nseg - 1] == b) {
                    s_len[nseg - 1] += l;
                } else {
                    s_start[nseg] = b;
                    s_len[nseg] = l;
                    s_code[nseg] = code;
                    ++nseg;
                }
            }
            s_nseg = nseg;
        }
    }
    __syncthreads();
    const int nseg = s_nseg;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    WaveList& L = lists[wave];
    const int zero_code = (128 << 16) | (128 << 8) | 128;
    const double Lx = g.L[0], Ly = g.L[1], Lz = g.L[2];
    const double rc2 = A.rc2;
    const int sel = A.sel;
    const d2* __restrict__ sa2 = reinterpret_cast<const d2*>(A.sa);

    for (int li = blockIdx.y * kNlWaves + wave; li < c1 - c0; li += kNlWaves * A.nsplit) {
        const int ci = c0 + li;
        const d2 ci0 = sa2[2 * ci], ci1 = sa2[2 * ci + 1];
        const int i = (int)__double_as_longlong(ci1[1]);
        const double xi = ci0[0], yi = ci0[1], zi = ci1[0];
        int count = 0;
        if constexpr (FLAT) {
            // Short segments (small boxes, where most of the stencil is periodic images, or few
            // atoms per cell): rounds of three 64-candidate chunks taken across segment ends,
            // each chunk with its own image shift, instead of whole rounds per segment.
            int sc = 0, off = 0;
            while (sc < nseg) {  // uniform
                double cx[3], cy[3], cz[3];
                int cj[3], cl[3], cc[3];
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    cl[u] = 0;
                    cc[u] = zero_code;
                    if (sc < nseg) {  // uniform
                        const int len = s_len[sc];
                        cl[u] = len - off < 64 ? len - off : 64;
                        cc[u] = s_code[sc];
                        const int a = s_start[sc] + off + (lane < cl[u] ? lane : 0);
                        const d2 v0 = sa2[2 * a], v1 = sa2[2 * a + 1];
                        cx[u] = v0[0];
                        cy[u] = v0[1];
                        cz[u] = v1[0];
                        cj[u] = (int)__double_as_longlong(v1[1]);
                        off += 64;
                        if (off >= len) {
                            ++sc;
                            off = 0;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    if (cl[u] == 0) break;  // uniform
                    const int code = cc[u];
                    const double dx = (cx[u] - xi) + (double)shift_x(code) * Lx;
                    const double dy = (cy[u] - yi) + (double)shift_y(code) * Ly;
                    const double dz = (cz[u] - zi) + (double)shift_z(code) * Lz;
                    const double sxy = dx * dx + dy * dy;
                    const double r2 = sxy + dz * dz;
                    const int j = cj[u];
                    const bool accept =
                        lane < cl[u] && (r2 < rc2) && !(j == i && code == zero_code);
                    const uint64_t m = __ballot(accept);
                    const int slot = count + __popcll(m & lt_mask);
                    if (accept && slot < NGA_ROW_CAP) {
                        L.r2[slot] = (uint64_t)__double_as_longlong(r2);
                        L.j[slot] = j;
                        L.code[slot] = code;
                    }
                    count += __popcll(m);
                }
            }
        }
        for (int sc = 0; sc < (FLAT ? 0 : nseg); ++sc) {
            const int base = s_start[sc], len = s_len[sc], code = s_code[sc];
            const double nx = (double)shift_x(code) * Lx;
            const double ny = (double)shift_y(code) * Ly;
            const double nz = (double)shift_z(code) * Lz;
            // Three chunks of 64 candidates per round: every load is issued before the first
            // distance is evaluated.
            for (int t0 = 0; t0 < len; t0 += 3 * 64) {
                double cx[3], cy[3], cz[3];
                int cj[3];
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int t = t0 + 64 * u + lane;
                    const int a = base + (t < len ? t : 0);
                    const d2 v0 = sa2[2 * a], v1 = sa2[2 * a + 1];
                    cx[u] = v0[0];
                    cy[u] = v0[1];
                    cz[u] = v1[0];
                    cj[u] = (int)__double_as_longlong(v1[1]);
                }
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    if (t0 + 64 * u >= len) break;  // uniform
                    const int t = t0 + 64 * u + lane;
                    const double dx = (cx[u] - xi) + nx;
                    const double dy = (cy[u] - yi) + ny;
                    const double dz = (cz[u] - zi) + nz;
                    const double sxy = dx * dx + dy * dy;
                    const double r2 = sxy + dz * dz;
                    const int j = cj[u];
                    const bool accept = t < len && (r2 < rc2) && !(j == i && code == zero_code);
                    const uint64_t m = __ballot(accept);
                    const int slot = count + __popcll(m & lt_mask);
                    if (accept && slot < NGA_ROW_CAP) {
                        L.r2[slot] = (uint64_t)__double_as_longlong(r2);
                        L.j[slot] = j;
                        L.code[slot] = code;
                    }
                    count += __popcll(m);
                }
            }
        }
        wave_sync_lds();
        if (count > NGA_ROW_CAP) {
            if (lane == 0) raise_bits(A.status, kBitRowCap);
            count = 0;
        }
        const int keep = count < sel ? count : sel;
        int32_t* row = A.nbr + (int64_t)i * sel;
        int32_t* rsh = A.nbr_shift + (int64_t)i * sel * 3;
        const double qscale = 8388608.0 / rc2;
        if (count <= 64) sort_and_write<1>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        else if (count <= 128) sort_and_write<2>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        else if (count <= 256) sort_and_write<4>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        else sort_and_write<8>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        if (lane == 0) A.nnei[i] = keep;
        wave_sync_lds();
    }
}

// Exclusive prefix sum over the wavefront (and the total), with DPP moves only: shifts by 1,
// 2, 4 and 8 inside each row of 16 lanes (zero shifted in), then each row's running total
// broadcast into the next rows (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and
// 3).
__device__ inline int wave_excl_scan(int v, int lane, int* total) {
    (void)lane;
    int incl = v;
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xA, 0xF, false);  // row_bcast:15
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xC, 0xF, false);  // row_bcast:31
    *total = __builtin_amdgcn_readlane(incl, 63);
    return incl - v;
}

// Selection with per-centre stencils (Geom::trim = K, cells of about rcut / 2): a wavefront
// takes one centre at a time.  Lane r < (2K+1)^2 takes stencil row (dy, dz) = (r % (2K+1) - K,
// r / (2K+1) - K): from the centre's offset inside its own cell it finds the y and z gaps to
// that row and then the run dx = lo .. hi of the row's cells whose nearest point is within
// rcut (the gap grows with |dx|, so the run is contiguous).  A run is one stretch of the
// cell-sorted array, or two where it crosses the box's x face (with their own image shifts).
// The runs are concatenated into one list of candidate positions, read 64 to a chunk across
// run ends: a bitmap of run starts in LDS and the run counts before each 32-bit word give
// every lane its run.  Accepted candidates are compacted, sorted and written as in
// select_kernel.  Any gap below the true distance only admits extra candidates, which the
// exact r2 < rc2 test then rejects; so the run bounds take rc2 (1 + 1e-6).
constexpr int kTrimWindow = 1024;     // candidate positions per bitmap
constexpr int kTrimCentresPerGroup = 16;

struct TrimList {
    WaveList L;
    uint32_t bm[kTrimWindow / 32];
    int32_t pc[kTrimWindow / 32];
    int2 seg[2 * 25];  // per run: (first atom slot minus its first position, shift code)
};

// Gap along one axis, in cell widths, between a point at offset f in its cell and the cell d
// away.
__device__ inline double cell_gap(int d, double f) {
    return d > 0 ? (double)d - f : (d < 0 ? f + (double)(-d - 1) : 0.0);
}

template <int K, bool SMALL>
__global__ void __launch_bounds__(kNlBlock) select_trim_kernel(SelectArgs A) {
    constexpr int W = 2 * K + 1, R = W * W;
    static_assert(R <= 25, "reach");
    extern __shared__ __align__(16) unsigned char nl_smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    TrimList& T = reinterpret_cast<TrimList*>(nl_smem)[wave];
    WaveList& L = T.L;
    const Geom g = A.g;
    const int ncx = g.nc[0], ncy = g.nc[1], ncz = g.nc[2];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int zero_code = (128 << 16) | (128 << 8) | 128;
    const double rc2 = A.rc2, rc2s = A.rc2 * (1.0 + 1e-6);
    const int sel = A.sel;
    const d2* __restrict__ sa2 = reinterpret_cast<const d2*>(A.sa);
    const int64_t* __restrict__ cs = A.cell_start;
    // Work-groups go to the eight XCDs in turn; work-group b takes centre group
    // (b % 8) (G / 8) + b / 8, so that each XCD's L2 serves a contiguous run of centres whose
    // stencils overlap (the last G % 8 groups keep their own index).  1% faster at 65,536
    // atoms, rows unchanged.
    int grp = (int)blockIdx.x;
    {
        const int G = (int)gridDim.x, full = G / 8 * 8;
        if (grp < full) grp = (grp % 8) * (G / 8) + grp / 8;
    }
    const int c_end = (int)std::min<int64_t>((int64_t)A.n, ((int64_t)grp + 1) * kTrimCentresPerGroup);

    for (int ci = grp * kTrimCentresPerGroup + wave; ci < c_end; ci += kNlWaves) {
        const d2 ci0 = sa2[2 * ci], ci1 = sa2[2 * ci + 1];
        const int i = (int)__double_as_longlong(ci1[1]);
        const double xi = ci0[0], yi = ci0[1], zi = ci1[0];
        // the centre's cell, as binning found it, and its offset inside (clamped to [0, 1])
        int cc[3];
        double f[3];
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            const double x = a == 0 ? xi : (a == 1 ? yi : zi);
            const bool ok = (x >= 0.0) && (x < g.L[a]);
            int c = ok ? (int)(x * g.inv_h[a]) : 0;
            c = c < g.nc[a] ? c : g.nc[a] - 1;
            cc[a] = c;
            const double o = ok ? x * g.inv_h[a] - (double)c : 0.5;
            f[a] = o < 0.0 ? 0.0 : (o > 1.0 ? 1.0 : o);
        }
        // this lane's row runs
        int sA = 0, lA = 0, cdA = zero_code, sB = 0, lB = 0, cdB = zero_code;
        if (lane < R) {
            const int dy = lane % W - K, dz = lane / W - K;
            const double gy = cell_gap(dy, f[1]) * g.h[1], gz = cell_gap(dz, f[2]) * g.h[2];
            const double rem = rc2s - gy * gy - gz * gz;
            if (rem > 0.0) {
                int lo = 0, hi = 0;
#pragma unroll
                for (int d = 1; d <= K; ++d) {
                    const double gp = cell_gap(d, f[0]) * g.h[0], gm = cell_gap(-d, f[0]) * g.h[0];
                    if (gp * gp < rem) hi = d;
                    if (gm * gm < rem) lo = -d;
                }
                // the stencil spans fewer cells than the box (nc >= 2K+1): one wrap at most
                const int ry = cc[1] + dy, rz = cc[2] + dz;
                const int ny = ry < 0 ? -1 : (ry >= ncy ? 1 : 0);
                const int nz = rz < 0 ? -1 : (rz >= ncz ? 1 : 0);
                const int rowc = ((rz - nz * ncz) * ncy + (ry - ny * ncy)) * ncx;
                int a0 = cc[0] + lo, a1 = cc[0] + hi, b0 = 0, b1 = -1, nxb = 0;
                if (a0 < 0) {
                    b0 = a0 + ncx; b1 = ncx - 1; nxb = -1; a0 = 0;
                } else if (a1 >= ncx) {
                    b0 = 0; b1 = a1 - ncx; nxb = 1; a1 = ncx - 1;
                }
                sA = (int)cs[rowc + a0];
                lA = (int)cs[rowc + a1 + 1] - sA;
                cdA = pack_shift(0, ny, nz);
                if (b1 >= b0) {
                    sB = (int)cs[rowc + b0];
                    lB = (int)cs[rowc + b1 + 1] - sB;
                    cdB = pack_shift(nxb, ny, nz);
                }
            }
        }
        int nseg_all, total;
        const int sid = wave_excl_scan((lA > 0) + (lB > 0), lane, &nseg_all);
        const int base = wave_excl_scan(lA + lB, lane, &total);
        total = __builtin_amdgcn_readfirstlane(total);  // alike in all lanes
        if (lA > 0) T.seg[sid] = make_int2(sA - base, cdA);
        if (lB > 0) T.seg[sid + (lA > 0)] = make_int2(sB - (base + lA), cdB);
        int count = 0;
        for (int w0 = 0; w0 < total; w0 += kTrimWindow) {  // uniform; one window in practice
            if (lane < kTrimWindow / 32) T.bm[lane] = 0u;
            wave_sync_lds();
            const int bB = base + lA;
            if (lA > 0 && base >= w0 && base < w0 + kTrimWindow)
                atomicOr(&T.bm[(base - w0) >> 5], 1u << ((base - w0) & 31));
            if (lB > 0 && bB >= w0 && bB < w0 + kTrimWindow)
                atomicOr(&T.bm[(bB - w0) >> 5], 1u << ((bB - w0) & 31));
            const int before = __popcll(__ballot(lA > 0 && base < w0)) +
                               __popcll(__ballot(lB > 0 && bB < w0));
            wave_sync_lds();
            {
                const int bits = lane < kTrimWindow / 32 ? __popc(T.bm[lane]) : 0;
                int nb;
                const int ex = wave_excl_scan(bits, lane, &nb);
                if (lane < kTrimWindow / 32) T.pc[lane] = before + ex;
            }
            wave_sync_lds();
            const int wend = total < w0 + kTrimWindow ? total : w0 + kTrimWindow;
            // rounds of three 64-candidate chunks: every load is issued before the first
            // distance is evaluated
            for (int t0 = w0; t0 < wend; t0 += 3 * 64) {
                double cx[3], cy[3], cz[3];
                int cj[3], ccode[3];
                bool live[3];
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int t = t0 + 64 * u + lane;
                    live[u] = t < wend;
                    const int p = (live[u] ? t : w0) - w0;
                    const uint32_t word = T.bm[p >> 5];
                    const int b = p & 31;
                    const uint32_t upto = b == 31 ? word : (word & ((2u << b) - 1u));
                    const int owner = T.pc[p >> 5] + __popc(upto) - 1;
                    const int2 sg = T.seg[owner];
                    const int a = sg.x + (live[u] ? t : w0);
                    ccode[u] = sg.y;
                    const d2 v0 = sa2[2 * a], v1 = sa2[2 * a + 1];
                    cx[u] = v0[0];
                    cy[u] = v0[1];
                    cz[u] = v1[0];
                    cj[u] = (int)__double_as_longlong(v1[1]);
                }
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    if (t0 + 64 * u >= wend) break;  // uniform
                    const int code = ccode[u];
                    // n L is exact for n in {-1, 0, 1}, so the fused form rounds once, as
                    // the pinned (x_j - x_i) + n L does
                    const double dx = __builtin_fma((double)shift_x(code), g.L[0], cx[u] - xi);
                    const double dy = __builtin_fma((double)shift_y(code), g.L[1], cy[u] - yi);
                    const double dz = __builtin_fma((double)shift_z(code), g.L[2], cz[u] - zi);
                    const double sxy = dx * dx + dy * dy;
                    const double r2 = sxy + dz * dz;
                    const int j = cj[u];
                    const bool accept = live[u] && (r2 < rc2) && !(j == i && code == zero_code);
                    const uint64_t m = __ballot(accept);
                    const int slot = count + __popcll(m & lt_mask);
                    if (accept && slot < NGA_ROW_CAP) {
                        L.r2[slot] = (uint64_t)__double_as_longlong(r2);
                        L.j[slot] = j;
                        L.code[slot] = code;
                    }
                    count += __popcll(m);
                }
            }
            wave_sync_lds();  // the next window rewrites the bitmap
        }
        wave_sync_lds();
        if (count > NGA_ROW_CAP) {
            if (lane == 0) raise_bits(A.status, kBitRowCap);
            count = 0;
        }
        const int keep = count < sel ? count : sel;
        int32_t* row = A.nbr + (int64_t)i * sel;
        int32_t* rsh = A.nbr_shift + (int64_t)i * sel * 3;
        const double qscale = 8388608.0 / rc2;
        // two sort widths only: every instance inlined here costs registers in the whole
        // kernel.  SMALL: for rows of a few dozen candidates.
        if (SMALL && count <= 64) sort_and_write<1>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        else if (!SMALL && count <= 256) sort_and_write<4>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        else sort_and_write<8>(lds(L), count, keep, sel, qscale, row, rsh, lane);
        if (lane == 0) A.nnei[i] = keep;
        wave_sync_lds();
    }
}

// Work-groups per cell for select: about four centres per wavefront, which amortises each
// work-group's stencil set-up, unless that leaves fewer than kMinSelectGroups work-groups in
// all; then more, down to one centre per wavefront.
constexpr double kMinSelectGroups = 1024.0;
int select_splits(double per_cell, int64_t ncells) {
    double ns = std::ceil(per_cell / (4.0 * kNlWaves));
    if (ns * (double)ncells < kMinSelectGroups)
        ns = std::min(std::ceil(per_cell / kNlWaves), std::ceil(kMinSelectGroups / (double)ncells));
    return (int)std::max(1.0, std::min(ns, 4096.0));
}

size_t select_lds_bytes(const Geom& g) {
    return kNlWaves * sizeof(WaveList) + 3 * sizeof(int) * (size_t)g.stencil;
}

// Candidate rounds that cross segment ends pay off when segments are shorter than about a
// round and a half: a segment is about one x-row of stencil cells (a single cell when the box
// has one cell per row, whose images then come as separate segments).
bool short_segments(int64_t n, const Geom& g) {
    const double seg_est = (double)n / (double)g.ncells *
                           (double)std::min(g.nc[0], 2 * g.reach[0] + 1);
    return seg_est <= 96.0;
}

// ws: the scratch regions (carved after a 256-byte header); status: the word that collects
// device-detected errors (the workspace's own header word for nl_build).
int launch_nl(const double* pos, int64_t n, const Geom& g, double rcut, int32_t sel,
              int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* ws, uint32_t* status,
              hipStream_t s) {
    WsLayout w = carve(ws, n, g);
    const int ni = (int)n;
    int rc;
    if (n <= kSmallAtoms && g.ncells <= kSmallCells) {
        hipLaunchKernelGGL(bin_small_kernel, dim3(1), dim3(kSmallThreads), 0, s, pos, ni, g,
                           w.cell_start, w.sa, status);
        if ((rc = last_launch_status())) return rc;
    } else {
        hipLaunchKernelGGL(clear_i32_kernel, dim3((unsigned)((g.ncells + 255) / 256)), dim3(256),
                           0, s, w.cell_count, g.ncells);
        hipLaunchKernelGGL(bin_kernel, dim3((ni + 255) / 256), dim3(256), 0, s, pos, ni, g,
                           w.cell_count, w.atom_cell, w.atom_slot, status);
        if ((rc = last_launch_status())) return rc;
        if ((rc = scan_counts(w.cell_count, g.ncells, INT32_MAX, w.tile_sums, w.cell_start, s)))
            return rc;
        hipLaunchKernelGGL(scatter_kernel, dim3((ni + 255) / 256), dim3(256), 0, s, pos, ni,
                           w.cell_start, w.atom_cell, w.atom_slot, w.sa);
        if ((rc = last_launch_status())) return rc;
    }

    SelectArgs A;
    A.g = g;
    A.rc2 = rcut * rcut;
    A.n = ni;
    A.sel = sel;
    A.nsplit = select_splits((double)n / (double)g.ncells, g.ncells);
    A.cell_start = w.cell_start;
    A.sa = w.sa;
    A.nbr = nbr; A.nbr_shift = nbr_shift; A.nnei = nnei;
    A.status = status;
    A.table = nullptr;
    A.cell_ptr = nullptr;
    A.n_structs = 1;
    if (g.trim > 0) {
        const dim3 grid((unsigned)((n + kTrimCentresPerGroup - 1) / kTrimCentresPerGroup));
        const unsigned lds = (unsigned)(kNlWaves * sizeof(TrimList));
        // neighbours within rcut at the mean density
        const double vol = g.L[0] * g.L[1] * g.L[2];
        const double expect = (double)n / vol * 4.18879020478639 * rcut * rcut * rcut;
        const bool small = expect <= 48.0;
        if (g.trim == 1 && small)
            hipLaunchKernelGGL((select_trim_kernel<1, true>), grid, dim3(kNlBlock), lds, s, A);
        else if (g.trim == 1)
            hipLaunchKernelGGL((select_trim_kernel<1, false>), grid, dim3(kNlBlock), lds, s, A);
        else if (small)
            hipLaunchKernelGGL((select_trim_kernel<2, true>), grid, dim3(kNlBlock), lds, s, A);
        else
            hipLaunchKernelGGL((select_trim_kernel<2, false>), grid, dim3(kNlBlock), lds, s, A);
        return last_launch_status();
    }
    const bool flat = short_segments(n, g);
    if (flat)
        hipLaunchKernelGGL((select_kernel<false, true>), dim3((unsigned)g.ncells,
                           (unsigned)A.nsplit), dim3(kNlBlock), (unsigned)select_lds_bytes(g), s, A);
    else
        hipLaunchKernelGGL((select_kernel<false, false>), dim3((unsigned)g.ncells,
                           (unsigned)A.nsplit), dim3(kNlBlock), (unsigned)select_lds_bytes(g), s, A);
    return last_launch_status();
}

// ---------------------------------------------------------------------------------------
// Batches of structures: one launch sequence for many boxes.  The cells of all structures are
// numbered one after the other, so counting, scanning and scattering run unchanged over the
// whole batch; binning and selection look up each atom's / cell's structure.

struct BatchPlan {
    std::vector<BatchGeom> table;
    std::vector<int64_t> atom_ptr;  // [n_structs + 1]
    std::vector<int64_t> cell_ptr;  // [n_structs + 1]
    int64_t n_atoms = 0;
    int64_t n_cells = 0;
    int max_stencil = 1;
    int nsplit = 1;
    bool flat = true;  // every structure has short segments
};

bool plan_batch(int32_t n_structs, const int64_t* atom_ptr, const double* boxes, double rcut,
                BatchPlan* p) {
    if (n_structs < 1 || !atom_ptr || !boxes || atom_ptr[0] != 0) return false;
    p->table.resize(n_structs);
    p->atom_ptr.assign(atom_ptr, atom_ptr + n_structs + 1);
    p->cell_ptr.resize((size_t)n_structs + 1);
    p->cell_ptr[0] = 0;
    double max_per_cell = 0.0;
    for (int32_t b = 0; b < n_structs; ++b) {
        const int64_t nb = atom_ptr[b + 1] - atom_ptr[b];
        if (nb < 0) return false;
        Geom g;
        if (!make_geom(nb, boxes + 3 * (size_t)b, rcut, &g)) return false;
        p->table[b].g = g;
        p->table[b].cell_base = p->cell_ptr[b];
        p->table[b].atom_base = atom_ptr[b];
        p->cell_ptr[b + 1] = p->cell_ptr[b] + g.ncells;
        p->max_stencil = std::max(p->max_stencil, g.stencil);
        max_per_cell = std::max(max_per_cell, (double)nb / (double)g.ncells);
        p->flat = p->flat && short_segments(nb, g);
    }
    p->n_atoms = atom_ptr[n_structs];
    p->n_cells = p->cell_ptr[n_structs];
    if (p->n_atoms >= INT32_MAX || p->n_cells >= INT32_MAX) return false;
    p->nsplit = select_splits(max_per_cell, p->n_cells);
    return true;
}

struct BatchWs {
    WsLayout w;
    BatchGeom* table;
    int64_t* atom_ptr;
    int64_t* cell_ptr;
    size_t bytes;
};

BatchWs carve_batch(void* ws, const BatchPlan& p) {
    Geom all;
    all.ncells = p.n_cells;
    BatchWs b;
    b.w = carve(ws, p.n_atoms, all);
    Carver cv(ws);
    cv.off = b.w.bytes;
    b.table = cv.take<BatchGeom>(p.table.size());
    b.atom_ptr = cv.take<int64_t>(p.atom_ptr.size());
    b.cell_ptr = cv.take<int64_t>(p.cell_ptr.size());
    b.bytes = cv.off;
    return b;
}

int launch_nl_batch(const double* pos, const BatchPlan& p, double rcut, int32_t sel,
                    int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* ws, hipStream_t s) {
    BatchWs b = carve_batch(ws, p);
    const WsLayout& w = b.w;
    uint32_t* status = &static_cast<WsHeader*>(ws)->status;
    // The structure table is host data: upload it, and wait, so that nothing here outlives
    // the call.
    int rc = hip_status(hipMemcpyAsync(b.table, p.table.data(), p.table.size() * sizeof(BatchGeom),
                                       hipMemcpyHostToDevice, s));
    if (!rc) rc = hip_status(hipMemcpyAsync(b.atom_ptr, p.atom_ptr.data(),
                                            p.atom_ptr.size() * sizeof(int64_t),
                                            hipMemcpyHostToDevice, s));
    if (!rc) rc = hip_status(hipMemcpyAsync(b.cell_ptr, p.cell_ptr.data(),
                                            p.cell_ptr.size() * sizeof(int64_t),
                                            hipMemcpyHostToDevice, s));
    if (!rc) rc = hip_status(hipStreamSynchronize(s));
    if (rc) return rc;
    const int ni = (int)p.n_atoms;
    const int ns = (int)p.table.size();
    hipLaunchKernelGGL(clear_i32_kernel, dim3((unsigned)((p.n_cells + 255) / 256)), dim3(256), 0,
                       s, w.cell_count, p.n_cells);
    if (ni > 0)
        hipLaunchKernelGGL(bin_batch_kernel, dim3((ni + 255) / 256), dim3(256), 0, s, pos, ni,
                           b.table, b.atom_ptr, ns, w.cell_count, w.atom_cell, w.atom_slot,
                           status);
    if ((rc = last_launch_status())) return rc;
    if ((rc = scan_counts(w.cell_count, p.n_cells, INT32_MAX, w.tile_sums, w.cell_start, s)))
        return rc;
    if (ni == 0) return NGA_OK;
    hipLaunchKernelGGL(scatter_kernel, dim3((ni + 255) / 256), dim3(256), 0, s, pos, ni,
                       w.cell_start, w.atom_cell, w.atom_slot, w.sa);
    if ((rc = last_launch_status())) return rc;
    SelectArgs A;
    A.g = p.table[0].g;
    A.table = b.table;
    A.cell_ptr = b.cell_ptr;
    A.n_structs = ns;
    A.rc2 = rcut * rcut;
    A.n = ni;
    A.sel = sel;
    A.nsplit = p.nsplit;
    A.cell_start = w.cell_start;
    A.sa = w.sa;
    A.nbr = nbr; A.nbr_shift = nbr_shift; A.nnei = nnei;
    A.status = status;
    const size_t lds = kNlWaves * sizeof(WaveList) + 3 * sizeof(int) * (size_t)p.max_stencil;
    if (p.flat)
        hipLaunchKernelGGL((select_kernel<true, true>), dim3((unsigned)p.n_cells,
                           (unsigned)A.nsplit), dim3(kNlBlock), (unsigned)lds, s, A);
    else
        hipLaunchKernelGGL((select_kernel<true, false>), dim3((unsigned)p.n_cells,
                           (unsigned)A.nsplit), dim3(kNlBlock), (unsigned)lds, s, A);
    return last_launch_status();
}

// ---------------------------------------------------------------------------------------
// Reuse across steps ("ago > 0" in deepmd-kit issue "perf: DPA4 .pt2 LAMMPS (C++ AOTI)
// inference 3-6x slower ...", section "Proposed optimizations": keep what was built while
// the neighbour list is unchanged).  Candidate rows built once with a larger cutoff
// rcut + skin hold, while no atom has moved more than skin / 2, every pair within rcut; the
// rows of the current positions are then the candidates re-evaluated and re-ranked.

struct RefineArgs {
    const double* pos;
    int n;
    double L[3];
    double rc2;
    int sel;
    const int32_t* cnbr;
    const int32_t* cshift;
    const int32_t* cnnei;
    int csel;
    int32_t* nbr;
    int32_t* nbr_shift;
    int32_t* nnei;
    uint32_t* status;
};

// One wavefront per centre: the pinned fp64 distance of each candidate at the current
// positions, those within rcut compacted into the wave's LDS list with ballot / mbcnt, then
// the same ranking and row write as nl_build (sort_and_write), so that the row equals the one
// nl_build makes from the same positions whenever the candidates hold every pair within rcut.
constexpr int kRefineChunks = 4;

__global__ void __launch_bounds__(kNlBlock) refine_kernel(RefineArgs A) {
    __shared__ WaveList lists[kNlWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.x * kNlWaves + wave;
    if (i >= A.n) return;  // whole wavefronts; the kernel has no work-group barrier
    WaveList& L = lists[wave];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const double xi = A.pos[3 * (int64_t)i], yi = A.pos[3 * (int64_t)i + 1],
                 zi = A.pos[3 * (int64_t)i + 2];
    int cn = A.cnnei ? A.cnnei[i] : A.csel;
    cn = cn < 0 ? 0 : (cn > A.csel ? A.csel : cn);
    const int32_t* crow = A.cnbr + (int64_t)i * A.csel;
    const int32_t* csh = A.cshift + (int64_t)i * A.csel * 3;
    bool bad = false;
    int count = 0;
    // Rounds of kRefineChunks chunks of 64 candidates: every row entry, then every position
    // gather of the round is issued before the first distance is evaluated.
    for (int t0 = 0; t0 < cn; t0 += 64 * kRefineChunks) {
        int jj[kRefineChunks], sx[kRefineChunks], sy[kRefineChunks], sz[kRefineChunks];
        bool ok[kRefineChunks];
#pragma unroll
        for (int u = 0; u < kRefineChunks; ++u) {
            const int t = t0 + 64 * u + lane;
            jj[u] = -1;
            sx[u] = sy[u] = sz[u] = 0;
            if (t < cn) {
                jj[u] = crow[t];
                sx[u] = csh[3 * t];
                sy[u] = csh[3 * t + 1];
                sz[u] = csh[3 * t + 2];
            }
        }
        double px[kRefineChunks], py[kRefineChunks], pz[kRefineChunks];
#pragma unroll
        for (int u = 0; u < kRefineChunks; ++u) {
            const int j = jj[u];
            ok[u] = j >= 0 && j < A.n && sx[u] >= -127 && sx[u] <= 127 && sy[u] >= -127 &&
                    sy[u] <= 127 && sz[u] >= -127 && sz[u] <= 127;
            if (j >= 0 && !ok[u]) bad = true;
            const int64_t jp = ok[u] ? j : i;
            px[u] = A.pos[3 * jp];
            py[u] = A.pos[3 * jp + 1];
            pz[u] = A.pos[3 * jp + 2];
        }
#pragma unroll
        for (int u = 0; u < kRefineChunks; ++u) {
            if (t0 + 64 * u >= cn) break;  // uniform
            bool accept = false;
            double r2 = 0.0;
            if (ok[u]) {
                const double dx = (px[u] - xi) + (double)sx[u] * A.L[0];
                const double dy = (py[u] - yi) + (double)sy[u] * A.L[1];
                const double dz = (pz[u] - zi) + (double)sz[u] * A.L[2];
                const double sxy = dx * dx + dy * dy;
                r2 = sxy + dz * dz;
                accept = r2 < A.rc2 && !(jj[u] == i && sx[u] == 0 && sy[u] == 0 && sz[u] == 0);
            }
            const uint64_t m = __ballot(accept);
            const int slot = count + __popcll(m & lt_mask);
            if (accept) {
                L.r2[slot] = (uint64_t)__double_as_longlong(r2);
                L.j[slot] = jj[u];
                L.code[slot] = pack_shift(sx[u], sy[u], sz[u]);
            }
            count += __popcll(m);
        }
    }
    wave_sync_lds();
    const int keep = count < A.sel ? count : A.sel;
    int32_t* row = A.nbr + (int64_t)i * A.sel;
    int32_t* rsh = A.nbr_shift + (int64_t)i * A.sel * 3;
    const double qscale = 8388608.0 / A.rc2;
    if (count <= 64) sort_and_write<1>(lds(L), count, keep, A.sel, qscale, row, rsh, lane);
    else if (count <= 128) sort_and_write<2>(lds(L), count, keep, A.sel, qscale, row, rsh, lane);
    else if (count <= 256) sort_and_write<4>(lds(L), count, keep, A.sel, qscale, row, rsh, lane);
    else sort_and_write<8>(lds(L), count, keep, A.sel, qscale, row, rsh, lane);
    if (lane == 0) A.nnei[i] = keep;
    if (__ballot(bad) && lane == 0) raise_bits(A.status, kBitIndex);
}

__global__ void zero_f64_kernel(double* p) { *p = 0.0; }

// max over atoms of the plain distance |pos - pos_ref| (no minimum image), via an atomic max on
// the bit patterns (non-negative doubles order as their signed 64-bit patterns).  The cached
// candidate rows store image shifts taken at pos_ref, so an atom that was re-wrapped into the box
// since then must read as a displacement of about one box length, which forces a rebuild; a
// minimum-image distance would hide the wrap and let stale shifts drop its pairs.
__global__ void __launch_bounds__(256)
max_displacement_kernel(const double* __restrict__ pos, const double* __restrict__ ref, int n,
                        double* out) {
    double m = 0.0;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const double dx = pos[3 * (int64_t)i] - ref[3 * (int64_t)i];
        const double dy = pos[3 * (int64_t)i + 1] - ref[3 * (int64_t)i + 1];
        const double dz = pos[3 * (int64_t)i + 2] - ref[3 * (int64_t)i + 2];
        // A NaN distance must not read as "no displacement": it becomes +inf.
        double d = sqrt((dx * dx + dy * dy) + dz * dz);
        if (!(d <= 1.79769313486231570e308)) d = INFINITY;
        m = d > m ? d : m;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const double o = __shfl_xor(m, off, 64);
        m = o > m ? o : m;
    }
    if ((threadIdx.x & 63) == 0 && m > 0.0)
        atomicMax(reinterpret_cast<unsigned long long*>(out),
                  (unsigned long long)__double_as_longlong(m));
}

}  // namespace

}  // namespace nga

extern "C" size_t nl_build_batch_workspace_bytes(int32_t n_structs, const int64_t* h_atom_ptr,
                                                 const double* h_boxes, double rcut) {
    nga::BatchPlan p;
    if (!nga::plan_batch(n_structs, h_atom_ptr, h_boxes, rcut, &p)) return 0;
    return nga::carve_batch(nullptr, p).bytes;
}

extern "C" int nl_build_batch(const double* pos, int32_t n_structs, const int64_t* h_atom_ptr,
                              const double* h_boxes, double rcut, int32_t sel, int32_t* nbr,
                              int32_t* nbr_shift, int32_t* nnei, void* ws, size_t ws_bytes,
                              void* stream) {
    using namespace nga;
    BatchPlan p;
    if (!plan_batch(n_structs, h_atom_ptr, h_boxes, rcut, &p)) return NGA_EINVAL;
    if (sel < 1) return NGA_EINVAL;
    if (p.n_atoms > 0 && (!pos || !nbr || !nbr_shift || !nnei)) return NGA_EINVAL;
    if (!ws || ws_bytes < carve_batch(nullptr, p).bytes) return NGA_EWORKSPACE;
    if (p.n_atoms == 0) return NGA_OK;
    return launch_nl_batch(pos, p, rcut, sel, nbr, nbr_shift, nnei, ws,
                           static_cast<hipStream_t>(stream));
}

extern "C" int nl_refine(const double* pos, int64_t n_atoms, const double* h_box, double rcut,
                         int32_t sel, const int32_t* cand_nbr, const int32_t* cand_shift,
                         const int32_t* cand_nnei, int32_t cand_sel, const double* h_cand_box,
                         int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* ws,
                         size_t ws_bytes, void* stream) {
    using namespace nga;
    if (n_atoms < 0 || n_atoms >= INT32_MAX || !h_box || !h_cand_box || !(rcut > 0.0) ||
        !std::isfinite(rcut))
        return NGA_EINVAL;
    for (int a = 0; a < 3; ++a) {
        if (!finite_pos(h_box[a])) return NGA_EINVAL;
        if (h_cand_box[a] != h_box[a]) return NGA_EINVAL;  // candidates of another box: stale
    }
    if (sel < 1 || cand_sel < 1 || cand_sel > NGA_ROW_CAP) return NGA_EINVAL;
    if (n_atoms == 0) return NGA_OK;
    if (!pos || !cand_nbr || !cand_shift || !nbr || !nbr_shift || !nnei) return NGA_EINVAL;
    if (!ws || ws_bytes < sizeof(WsHeader)) return NGA_EWORKSPACE;
    RefineArgs A;
    A.pos = pos;
    A.n = (int)n_atoms;
    A.L[0] = h_box[0]; A.L[1] = h_box[1]; A.L[2] = h_box[2];
    A.rc2 = rcut * rcut;
    A.sel = sel;
    A.cnbr = cand_nbr; A.cshift = cand_shift; A.cnnei = cand_nnei; A.csel = cand_sel;
    A.nbr = nbr; A.nbr_shift = nbr_shift; A.nnei = nnei;
    A.status = &static_cast<WsHeader*>(ws)->status;
    const unsigned blocks = (unsigned)((n_atoms + kNlWaves - 1) / kNlWaves);
    hipLaunchKernelGGL(refine_kernel, dim3(blocks), dim3(kNlBlock), 0,
                       static_cast<hipStream_t>(stream), A);
    return last_launch_status();
}

extern "C" int nl_max_displacement(const double* pos, const double* pos_ref, int64_t n_atoms,
                                   const double* h_box, double* d_max, void* stream) {
    using namespace nga;
    if (n_atoms < 0 || n_atoms >= INT32_MAX || !h_box || !d_max) return NGA_EINVAL;
    for (int a = 0; a < 3; ++a)
        if (!finite_pos(h_box[a])) return NGA_EINVAL;
    if (n_atoms > 0 && (!pos || !pos_ref)) return NGA_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(zero_f64_kernel, dim3(1), dim3(1), 0, s, d_max);
    if (n_atoms > 0) {
        int64_t blocks = (n_atoms + 255) / 256;
        if (blocks > 1024) blocks = 1024;
        hipLaunchKernelGGL(max_displacement_kernel, dim3((unsigned)blocks), dim3(256), 0, s, pos,
                           pos_ref, (int)n_atoms, d_max);
    }
    return last_launch_status();
}

extern "C" size_t nl_build_workspace_bytes(int64_t n_atoms, const double* h_box, double rcut) {
    nga::Geom g;
    if (!nga::make_geom(n_atoms, h_box, rcut, &g, true)) return 0;
    return nga::carve(nullptr, n_atoms, g).bytes;
}

extern "C" int nl_build(const double* pos, int64_t n_atoms, const double* h_box, double rcut,
                        int32_t sel, int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* ws,
                        size_t ws_bytes, void* stream) {
    nga::Geom g;
    if (!nga::make_geom(n_atoms, h_box, rcut, &g, true)) return NGA_EINVAL;
    if (sel < 1) return NGA_EINVAL;
    if (n_atoms == 0) return NGA_OK;
    if (!pos || !nbr || !nbr_shift || !nnei) return NGA_EINVAL;
    if (!ws || ws_bytes < nga::carve(nullptr, n_atoms, g).bytes) return NGA_EWORKSPACE;
    return nga::launch_nl(pos, n_atoms, g, rcut, sel, nbr, nbr_shift, nnei, ws,
                          &static_cast<nga::WsHeader*>(ws)->status,
                          static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------
// nl_build_static: nl_build for callers that cannot allocate.  Its scratch (cell counts, the
// cell scan, per-atom cell and slot, the cell-sorted atoms) lives in this file-scope device
// array, one copy per GPU, held until the process ends.  In host code `scratch` only names
// the symbol: its device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept in scratch_dev; that address is what the kernels receive.  Every
// call on a GPU reuses that GPU's array, so calls that overlap on one GPU race; nothing in it
// has to start at zero (the counting kernels clear what they count into).
static __device__ __align__(256) unsigned char scratch[NGA_STATIC_SCRATCH_BYTES];

namespace nga {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NGA_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NGA_EHIP;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return NGA_OK;
}

}  // namespace
}  // namespace nga

extern "C" int nl_build_static(const double* pos, int64_t n_atoms, const double* h_box,
                               double rcut, int32_t sel, int32_t* nbr, int32_t* nbr_shift,
                               int32_t* nnei, void* status, void* stream) {
    nga::Geom g;
    if (!nga::make_geom(n_atoms, h_box, rcut, &g, true)) return NGA_EINVAL;
    if (sel < 1) return NGA_EINVAL;
    if (nga::carve(nullptr, n_atoms, g).bytes > (size_t)NGA_STATIC_SCRATCH_BYTES)
        return NGA_ETOOBIG;
    if (n_atoms == 0) return NGA_OK;
    if (!pos || !nbr || !nbr_shift || !nnei || !status) return NGA_EINVAL;
    void* ws = nullptr;
    if (int rc = nga::static_scratch(&ws)) return rc;
    return nga::launch_nl(pos, n_atoms, g, rcut, sel, nbr, nbr_shift, nnei, ws,
                          &static_cast<nga::WsHeader*>(status)->status,
                          static_cast<hipStream_t>(stream));
}
