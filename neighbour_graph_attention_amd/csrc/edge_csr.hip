// edge_csr: padded neighbour rows -> destination CSR, on the device.
//
// deepmd-kit issue "perf: DPA4 .pt2 LAMMPS (C++ AOTI) inference 3-6x slower than Python
// (ASE) ...": the C++ path builds edge_index / edge_vec / edge_scatter_index / edge_mask with
// CPU loops (section "Root cause analysis", bottleneck 1); the fix its comments propose is
// to produce them on the device with a prefix-scan compaction.  deepmd-kit issue
// "perf: NeighborGraph attention is 4-9x slower than dense ...", section "Proposed fix":
// the destination CSR (destination_row_ptr) that the attention gathers through.
//
// Launches: the scan of the per-row edge counts into row_ptr (nnei clamped to [0, sel], or a
// counting pass over the slots when nnei is absent), and a fill where one wavefront compacts
// one row with ballot/mbcnt, keeping slot order.  With nnei given and up to 65,536 rows
// that is two launches in all.
#pragma clang fp contract(off)

#include "nga_internal.h"

namespace nga {

namespace {

struct CsrWs {
    int32_t* counts;
    int64_t* tile_sums;
    size_t bytes;
};

CsrWs carve_csr(void* ws, int64_t n) {
    Carver cv(ws);
    CsrWs w;
    w.counts = cv.take<int32_t>(n + 1);
    w.tile_sums = cv.take<int64_t>(scan_tiles(n) + 1);
    w.bytes = cv.off;
    return w;
}

// Edges of row i when no nnei is given: the slots with nbr >= 0, one wavefront per row.
__global__ void __launch_bounds__(256)
count_kernel(const int32_t* __restrict__ nbr, int n, int sel, int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int row = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
    if (row >= n) return;
    const int32_t* r = nbr + (int64_t)row * sel;
    int cnt = 0;
    for (int k = lane; k - lane < sel; k += 64) {
        bool valid = k < sel && r[k] >= 0;
        cnt += __popcll(__ballot(valid));
    }
    if (lane == 0) counts[row] = cnt;
}

struct FillArgs {
    const int32_t* nbr;
    const int32_t* nbr_shift;
    const int32_t* nnei;
    int n;
    int sel;
    const double* pos;
    double L[3];
    const int64_t* row_ptr;
    int32_t* col;
    int32_t* shift;
    int32_t* dst;
    double* edge_vec;
    int64_t e_cap;
    uint32_t* status;
};

__global__ void __launch_bounds__(256)
fill_kernel(FillArgs A) {
    const int lane = threadIdx.x & 63;
    const int row = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
    if (row >= A.n) return;
    if (row == 0 && lane == 0 && A.row_ptr[A.n] > A.e_cap) raise_bits(A.status, kBitCap);
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t* r = A.nbr + (int64_t)row * A.sel;
    const int32_t* rs = A.nbr_shift + (int64_t)row * A.sel * 3;
    int lim = A.sel;
    if (A.nnei) {
        int v = A.nnei[row];
        lim = v < 0 ? 0 : (v < A.sel ? v : A.sel);
    }
    int64_t base = A.row_ptr[row];
    bool bad_index = false;
    for (int k0 = 0; k0 < lim; k0 += 64) {
        const int k = k0 + lane;
        int j = -1;
        if (k < lim) j = r[k];
        const bool valid = (k < lim) && (A.nnei ? true : j >= 0);
        const uint64_t m = __ballot(valid);
        if (valid) {
            const int64_t e = base + __popcll(m & lt_mask);
            if (j < 0 || j >= A.n) {
                bad_index = true;
            }
            if (e < A.e_cap) {
                const int nx = rs[3 * k + 0], ny = rs[3 * k + 1], nz = rs[3 * k + 2];
                A.col[e] = j;
                A.shift[3 * e + 0] = nx;
                A.shift[3 * e + 1] = ny;
                A.shift[3 * e + 2] = nz;
                if (A.dst) A.dst[e] = row;
                if (A.edge_vec) {
                    const int jj = (j >= 0 && j < A.n) ? j : row;
                    const double* xj = A.pos + 3 * (int64_t)jj;
                    const double* xi = A.pos + 3 * (int64_t)row;
                    A.edge_vec[3 * e + 0] = (xj[0] - xi[0]) + (double)nx * A.L[0];
                    A.edge_vec[3 * e + 1] = (xj[1] - xi[1]) + (double)ny * A.L[1];
                    A.edge_vec[3 * e + 2] = (xj[2] - xi[2]) + (double)nz * A.L[2];
                }
            }
        }
        base += __popcll(m);
    }
    if (__ballot(bad_index) && lane == 0) raise_bits(A.status, kBitIndex);
}

__global__ void write_zero_kernel(int64_t* p) { p[0] = 0; }

}  // namespace

// First device error recorded in a workspace, highest priority first.
int status_from_bits(uint32_t bits) {
    if (bits & kBitBox) return NGA_EBOX;
    if (bits & kBitRowCap) return NGA_EROWCAP;
    if (bits & kBitCap) return NGA_ECAP;
    if (bits & kBitIndex) return NGA_EINDEX;
    return NGA_OK;
}

int read_and_clear_status(void* ws, hipStream_t s) {
    uint32_t bits = 0;
    WsHeader* h = static_cast<WsHeader*>(ws);
    hipError_t e = hipMemcpyAsync(&bits, &h->status, sizeof(bits), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return NGA_EHIP;
    if (bits) {
        uint32_t zero = 0;
        e = hipMemcpyAsync(&h->status, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return NGA_EHIP;
    }
    return status_from_bits(bits);
}

}  // namespace nga

extern "C" size_t edge_csr_workspace_bytes(int64_t n_atoms, int32_t sel) {
    if (n_atoms < 0 || n_atoms >= INT32_MAX || sel < 1) return 0;
    return nga::carve_csr(nullptr, n_atoms).bytes;
}

extern "C" int edge_csr(const int32_t* nbr, const int32_t* nbr_shift, const int32_t* nnei,
                        int64_t n_atoms, int32_t sel, const double* pos, const double* h_box,
                        int64_t* row_ptr, int32_t* col, int32_t* shift, int32_t* dst,
                        double* edge_vec, int64_t e_cap, int64_t* h_n_edges, void* ws,
                        size_t ws_bytes, void* stream) {
    using namespace nga;
    if (n_atoms < 0 || n_atoms >= INT32_MAX || sel < 1 || e_cap < 0) return NGA_EINVAL;
    if (!row_ptr) return NGA_EINVAL;
    if (n_atoms > 0 && (!nbr || !nbr_shift)) return NGA_EINVAL;
    if (e_cap > 0 && (!col || !shift)) return NGA_EINVAL;
    if (edge_vec) {
        if (!pos || !h_box) return NGA_EINVAL;
        for (int a = 0; a < 3; ++a)
            if (!finite_pos(h_box[a])) return NGA_EINVAL;
    }
    if (!ws || ws_bytes < carve_csr(nullptr, n_atoms).bytes) return NGA_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    CsrWs w = carve_csr(ws, n_atoms);
    const int n = (int)n_atoms;
    int rc;
    if (n == 0) {
        hipLaunchKernelGGL(write_zero_kernel, dim3(1), dim3(1), 0, s, row_ptr);
        if ((rc = last_launch_status())) return rc;
    } else {
        const unsigned blocks = (unsigned)(((int64_t)n * 64 + 255) / 256);
        // With nnei the scan clamps it to [0, sel] itself; without, count the valid slots.
        const int32_t* counts = nnei;
        if (!nnei) {
            hipLaunchKernelGGL(count_kernel, dim3(blocks), dim3(256), 0, s, nbr, n, sel,
                               w.counts);
            if ((rc = last_launch_status())) return rc;
            counts = w.counts;
        }
        if ((rc = scan_counts(counts, n, sel, w.tile_sums, row_ptr, s))) return rc;
        FillArgs A;
        A.nbr = nbr; A.nbr_shift = nbr_shift; A.nnei = nnei;
        A.n = n; A.sel = sel; A.pos = pos;
        for (int a = 0; a < 3; ++a) A.L[a] = edge_vec ? h_box[a] : 0.0;
        A.row_ptr = row_ptr; A.col = col; A.shift = shift; A.dst = dst; A.edge_vec = edge_vec;
        A.e_cap = e_cap;
        A.status = &static_cast<WsHeader*>(ws)->status;
        hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, s, A);
        if ((rc = last_launch_status())) return rc;
    }
    if (h_n_edges) {
        hipError_t e = hipMemcpyAsync(h_n_edges, row_ptr + n, sizeof(int64_t),
                                      hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return NGA_EHIP;
        return read_and_clear_status(ws, s);
    }
    return NGA_OK;
}
