// Status queries of the C ABI: nga_sync_status, nga_strerror.
#include "nga_internal.h"

extern "C" int nga_sync_status(void* ws, void* stream) {
    if (!ws) return NGA_EWORKSPACE;
    return nga::read_and_clear_status(ws, static_cast<hipStream_t>(stream));
}

extern "C" const char* nga_strerror(int status) {
    switch (status) {
        case NGA_OK: return "ok";
        case NGA_EINVAL: return "invalid argument";
        case NGA_EBOX: return "a position is not finite or lies outside [0, L)";
        case NGA_EROWCAP: return "a centre has more neighbours within rcut than the row capacity";
        case NGA_ECAP: return "edge count exceeds the capacity";
        case NGA_EDTYPE: return "unsupported dtype";
        case NGA_EWORKSPACE: return "workspace missing or too small";
        case NGA_EHIP: return "HIP runtime error";
        case NGA_EINDEX: return "an index in device data is out of range";
        case NGA_ETOOBIG:
            return "the problem needs more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}
