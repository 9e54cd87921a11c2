// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "nga.h"

namespace nga {

// Device-detected error bits, OR-ed into the workspace status word.
enum : uint32_t {
    kBitBox = 1u << 0,
    kBitRowCap = 1u << 1,
    kBitCap = 1u << 2,
    kBitIndex = 1u << 3,
};

// Every workspace starts with this header.
struct WsHeader {
    uint32_t status;
    uint32_t pad0;
    int64_t aux[31];
};
static_assert(sizeof(WsHeader) == 256, "workspace header must be 256 bytes");

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive aligned regions out of a workspace.
struct Carver {
    char* base;
    size_t off;
    explicit Carver(void* b) : base(static_cast<char*>(b)), off(align_up(sizeof(WsHeader))) {}
    template <typename T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off = align_up(off + count * sizeof(T));
        return p;
    }
};

inline int hip_status(hipError_t e) { return e == hipSuccess ? NGA_OK : NGA_EHIP; }

// Launch error of the last kernel enqueued by this thread.
inline int last_launch_status() { return hip_status(hipGetLastError()); }

__device__ inline void raise_bits(uint32_t* status, uint32_t bits) { atomicOr(status, bits); }

inline bool finite_pos(double v) { return std::isfinite(v) && v > 0.0; }

// Exclusive scan of clamped int32 counts into int64 offsets (scan.hip):
// out[0] = 0, out[i+1] = sum over j <= i of min(max(counts[j], 0), hi).  tile_sums is
// scratch of scan_tiles(n) int64 (used only for long inputs).
constexpr int kScanBlock = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanBlock * kScanItems;
inline int64_t scan_tiles(int64_t n) { return (n + kScanTile - 1) / kScanTile; }
int scan_counts(const int32_t* counts, int64_t n, int32_t hi, int64_t* tile_sums, int64_t* out,
                hipStream_t s);

// Status word handling (edge_csr.hip).
int status_from_bits(uint32_t bits);
int read_and_clear_status(void* ws, hipStream_t s);

}  // namespace nga
