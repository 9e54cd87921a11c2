// Device-wide exclusive scan of int32 counts into int64 offsets, in two passes over
// tiles of kScanTile counts: per-tile sums, then each tile adds the sum of the tiles
// before it and scans its own counts.  Used for cell offsets and CSR row offsets.
#include "nga_internal.h"

namespace nga {

namespace {

__device__ inline int64_t wave_inclusive_scan(int64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int64_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

__device__ inline int64_t block_sum(int64_t v, int64_t* red) {
    v = wave_inclusive_scan(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 63) red[wave] = v;
    __syncthreads();
    int64_t t = 0;
    for (int w = 0; w < kScanBlock / 64; ++w) t += red[w];
    __syncthreads();
    return t;
}

__global__ void __launch_bounds__(kScanBlock)
tile_sums_kernel(const int32_t* __restrict__ counts, int64_t n, int64_t* __restrict__ tile_sums) {
    __shared__ int64_t red[kScanBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int64_t s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + k * kScanBlock + threadIdx.x;
        if (i < n) s += counts[i];
    }
    s = block_sum(s, red);
    if (threadIdx.x == 0) tile_sums[blockIdx.x] = s;
}

__global__ void __launch_bounds__(kScanBlock)
tile_scan_kernel(const int32_t* __restrict__ counts, int64_t n,
                 const int64_t* __restrict__ tile_sums, int64_t* __restrict__ out) {
    __shared__ int64_t red[kScanBlock / 64];
    __shared__ int32_t tile[kScanTile];
    __shared__ int64_t wave_tot[kScanBlock / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;

    // Offset of this tile: sum of all earlier tiles' sums.
    int64_t pre = 0;
    for (int64_t b = threadIdx.x; b < blockIdx.x; b += kScanBlock) pre += tile_sums[b];
    pre = block_sum(pre, red);

#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + k * kScanBlock + threadIdx.x;
        tile[k * kScanBlock + threadIdx.x] = i < n ? counts[i] : 0;
    }
    __syncthreads();
    int64_t mine = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) mine += tile[threadIdx.x * kScanItems + k];
    int64_t incl = wave_inclusive_scan(mine);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int64_t run = pre + incl - mine;
    for (int w = 0; w < wave; ++w) run += wave_tot[w];
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + threadIdx.x * kScanItems + k;
        run += tile[threadIdx.x * kScanItems + k];
        if (i < n) out[i + 1] = run;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = 0;
}

}  // namespace

int scan_counts_tile_sums(const int32_t* counts, int64_t n, int64_t* tile_sums, hipStream_t s) {
    const int64_t nt = scan_tiles(n);
    if (nt == 0) return NGA_OK;
    hipLaunchKernelGGL(tile_sums_kernel, dim3((unsigned)nt), dim3(kScanBlock), 0, s, counts, n,
                       tile_sums);
    return last_launch_status();
}

int scan_counts_finish(const int32_t* counts, int64_t n, const int64_t* tile_sums, int64_t* out,
                       hipStream_t s) {
    const int64_t nt = scan_tiles(n) > 0 ? scan_tiles(n) : 1;
    hipLaunchKernelGGL(tile_scan_kernel, dim3((unsigned)nt), dim3(kScanBlock), 0, s, counts, n,
                       tile_sums, out);
    return last_launch_status();
}

}  // namespace nga
