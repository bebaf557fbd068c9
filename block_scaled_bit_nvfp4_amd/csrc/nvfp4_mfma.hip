// nvfp4_mfma.hip -- products with more than 8 activation columns.
// Interim form: column chunks of 8 on the VALU matvec (weights re-read once
// per chunk).
#include "nvfp4_host.h"

namespace nvfp4 {

template <bool ARGMAX>
int launch_valu(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, unsigned long long *amax_ws, int32_t *argmax_out, hipStream_t stream);

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream) {
    for (int c = 0; c < n; c += 8) {
        const int m = n - c < 8 ? n - c : 8;
        if (int st = launch_valu<false>(g, wq, ws, tscale, X + int64_t(c) * g.cols, m, Y + int64_t(c) * g.rows,
                                        nullptr, nullptr, stream))
            return st;
    }
    return NVFP4_OK;
}

}  // namespace nvfp4
