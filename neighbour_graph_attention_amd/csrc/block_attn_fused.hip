// Fused per-centre attention kernels.
#include "block_attn_fused.h"

namespace nga {

bool fused_supported(int, int32_t, int32_t, int32_t) { return false; }

const char* fused_name(int, int32_t, int32_t) { return "none"; }

int run_fused(int, const int64_t*, const int32_t*, int64_t, int64_t, int32_t, int32_t, int32_t,
              int32_t, const void*, const void*, void*, uint32_t*, hipStream_t) {
    return NGA_EINVAL;
}

}  // namespace nga
