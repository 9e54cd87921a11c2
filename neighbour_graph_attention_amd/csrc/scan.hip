// Device-wide exclusive scan of int32 counts into int64 offsets: out[0] = 0 and
// out[i+1] = sum of min(max(counts[j], 0), hi) over j <= i.  The clamp lets a caller scan
// neighbour counts (nnei, at most sel per row) without a separate counting pass.
//
// Up to kScanOnePassMax counts take one launch: each work-group scans its own tile of 8,192
// counts and adds the sum of every tile before it, which it reads itself (at most three
// tiles, 96 KB).  Longer inputs take two launches over tiles of 2,048: per-tile sums, then
// each tile adds the sums before it and scans its own counts; past four tiles that is
// faster than one work-group re-reading every earlier tile.  Used for cell
// offsets, CSR row offsets and pair offsets.
#include "nga_internal.h"

namespace nga {

namespace {

__device__ inline int32_t clamp_count(int32_t v, int32_t hi) {
    return v < 0 ? 0 : (v < hi ? v : hi);
}

__device__ inline int64_t wave_inclusive_scan(int64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int64_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

template <int B>
__device__ inline int64_t block_sum(int64_t v, int64_t* red) {
    v = wave_inclusive_scan(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 63) red[wave] = v;
    __syncthreads();
    int64_t t = 0;
    for (int w = 0; w < B / 64; ++w) t += red[w];
    __syncthreads();
    return t;
}

// Scans the I counts of thread t (tile[t*I .. t*I+I-1], already clamped) and writes
// out[base + t*I + k + 1] for the ones below n, starting from pre + everything before t.
template <int B, int I>
__device__ inline void scan_tile_and_write(const int32_t (&v)[I], int64_t pre, int64_t base,
                                           int64_t n, int64_t* wave_tot, int64_t* out) {
    int64_t mine = 0;
#pragma unroll
    for (int k = 0; k < I; ++k) mine += v[k];
    const int64_t incl = wave_inclusive_scan(mine);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int64_t run = pre + incl - mine;
    for (int w = 0; w < wave; ++w) run += wave_tot[w];
#pragma unroll
    for (int k = 0; k < I; ++k) {
        const int64_t i = base + (int64_t)threadIdx.x * I + k;
        run += v[k];
        if (i < n) out[i + 1] = run;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = 0;
}

constexpr int kOneBlock = 1024;
constexpr int kOneItems = 8;
constexpr int kOneTile = kOneBlock * kOneItems;  // 8,192
#ifndef NGA_SCAN_ONE_PASS_TILES
#define NGA_SCAN_ONE_PASS_TILES 4
#endif
constexpr int64_t kScanOnePassMax = NGA_SCAN_ONE_PASS_TILES * (int64_t)kOneTile;
constexpr int kPreUnroll = 8;  // int4 loads in flight per thread while summing earlier tiles

// One launch: work-group b scans counts [8192 b, 8192 (b+1)) and reads [0, 8192 b) for its
// offset.  With vec, counts is 16-byte aligned and read as int4s; otherwise one by one.
__global__ void __launch_bounds__(kOneBlock)
scan_one_pass_kernel(const int32_t* __restrict__ counts, int64_t n, int32_t hi, bool vec,
                     int64_t* __restrict__ out) {
    __shared__ int64_t red[kOneBlock / 64];
    __shared__ int64_t wave_tot[kOneBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kOneTile;
    const int4* c4 = reinterpret_cast<const int4*>(counts);

    // Sum of the earlier tiles: base is a multiple of 8,192, so every int4 below it is whole.
    int64_t pre = 0;
    if (!vec)
        for (int64_t i = threadIdx.x; i < base; i += kOneBlock) pre += clamp_count(counts[i], hi);
    for (int64_t q = threadIdx.x; vec && 4 * q < base; q += kPreUnroll * kOneBlock) {
        int4 a[kPreUnroll];
#pragma unroll
        for (int u = 0; u < kPreUnroll; ++u) {
            const int64_t qq = q + (int64_t)u * kOneBlock;
            a[u] = 4 * qq < base ? c4[qq] : int4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kPreUnroll; ++u)
            pre += (int64_t)clamp_count(a[u].x, hi) + clamp_count(a[u].y, hi) +
                   clamp_count(a[u].z, hi) + clamp_count(a[u].w, hi);
    }
    pre = block_sum<kOneBlock>(pre, red);

    int32_t v[kOneItems];
    const int64_t first = base + (int64_t)threadIdx.x * kOneItems;
    if (vec && first + kOneItems <= n) {
        const int4 a = c4[first / 4], b = c4[first / 4 + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int k = 0; k < kOneItems; ++k) v[k] = first + k < n ? counts[first + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < kOneItems; ++k) v[k] = clamp_count(v[k], hi);
    scan_tile_and_write<kOneBlock, kOneItems>(v, pre, base, n, wave_tot, out);
}

__global__ void __launch_bounds__(kScanBlock)
tile_sums_kernel(const int32_t* __restrict__ counts, int64_t n, int32_t hi,
                 int64_t* __restrict__ tile_sums) {
    __shared__ int64_t red[kScanBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int64_t s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + k * kScanBlock + threadIdx.x;
        if (i < n) s += clamp_count(counts[i], hi);
    }
    s = block_sum<kScanBlock>(s, red);
    if (threadIdx.x == 0) tile_sums[blockIdx.x] = s;
}

__global__ void __launch_bounds__(kScanBlock)
tile_scan_kernel(const int32_t* __restrict__ counts, int64_t n, int32_t hi,
                 const int64_t* __restrict__ tile_sums, int64_t* __restrict__ out) {
    __shared__ int64_t red[kScanBlock / 64];
    __shared__ int32_t tile[kScanTile];
    __shared__ int64_t wave_tot[kScanBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;

    // Offset of this tile: sum of all earlier tiles' sums.
    int64_t pre = 0;
    for (int64_t b = threadIdx.x; b < blockIdx.x; b += kScanBlock) pre += tile_sums[b];
    pre = block_sum<kScanBlock>(pre, red);

    // Coalesced loads into LDS, then each thread takes kScanItems consecutive counts.
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + k * kScanBlock + threadIdx.x;
        tile[k * kScanBlock + threadIdx.x] = i < n ? clamp_count(counts[i], hi) : 0;
    }
    __syncthreads();
    int32_t v[kScanItems];
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) v[k] = tile[threadIdx.x * kScanItems + k];
    scan_tile_and_write<kScanBlock, kScanItems>(v, pre, base, n, wave_tot, out);
}

}  // namespace

int scan_counts(const int32_t* counts, int64_t n, int32_t hi, int64_t* tile_sums, int64_t* out,
                hipStream_t s) {
    if (n <= kScanOnePassMax) {
        const int64_t blocks = n > 0 ? (n + kOneTile - 1) / kOneTile : 1;
        const bool vec = (reinterpret_cast<uintptr_t>(counts) & 15) == 0;
        hipLaunchKernelGGL(scan_one_pass_kernel, dim3((unsigned)blocks), dim3(kOneBlock), 0, s,
                           counts, n, hi, vec, out);
        return last_launch_status();
    }
    const int64_t nt = scan_tiles(n);
    hipLaunchKernelGGL(tile_sums_kernel, dim3((unsigned)nt), dim3(kScanBlock), 0, s, counts, n,
                       hi, tile_sums);
    int rc = last_launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(tile_scan_kernel, dim3((unsigned)nt), dim3(kScanBlock), 0, s, counts, n,
                       hi, tile_sums, out);
    return last_launch_status();
}

}  // namespace nga
