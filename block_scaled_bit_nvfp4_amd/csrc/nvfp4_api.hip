// nvfp4_api.hip -- status strings of the libnvfp4 C ABI.
#include "nvfp4_host.h"

NVFP4_API const char *nvfp4_strerror(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_EINVAL: return "invalid argument (null pointer, n out of range or bad tscale)";
        case NVFP4_ESHAPE: return "invalid shape (rows >= 1, cols >= 16 and a multiple of 16)";
        case NVFP4_EALIGN: return "misaligned pointer (16 bytes for inputs, natural for outputs)";
        case NVFP4_EWORKSPACE: return "workspace too small";
        case NVFP4_EHIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}
