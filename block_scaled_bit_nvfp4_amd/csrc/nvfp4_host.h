// nvfp4_host.h -- host-side argument checks and launch helpers shared by the
// C-ABI entry points of libnvfp4.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"
#include "nvfp4_device.h"

#define NVFP4_API extern "C" __attribute__((visibility("default")))

namespace nvfp4 {

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// rows x cols must describe whole 16-element blocks and stay addressable with
// 64-bit offsets and 32-bit tile/block counts.
inline int check_shape(int64_t rows, int64_t cols) {
    if (rows < 1 || cols < 16 || cols % 16 != 0) return NVFP4_ESHAPE;
    if (rows > (int64_t(1) << 31) - 64 || cols > (int64_t(1) << 31) - 1024) return NVFP4_ESHAPE;
    if (rows > (int64_t(1) << 62) / cols) return NVFP4_ESHAPE;
    return NVFP4_OK;
}

// MXFP4 takes whole 32-element blocks.
inline int check_mx_shape(int64_t rows, int64_t cols) {
    if (int st = check_shape(rows, cols)) return st;
    return cols % kMxBlock == 0 ? NVFP4_OK : NVFP4_ESHAPE;
}

inline bool tscale_ok(float t) { return t > 0.0f && t <= 3.4028234663852886e38f; }

struct Geometry {
    int64_t rows, cols;
    int64_t kb;          // 16-element blocks per row
    int64_t tiles;       // 16-row tiles
    int64_t supertiles;  // 64-row super-tiles
    int64_t octets;      // octets of 8 blocks per row
    Geometry(int64_t r, int64_t c)
        : rows(r), cols(c), kb(c / kBlock), tiles(ceil_div(r, kTileRows)),
          supertiles(ceil_div(ceil_div(r, kTileRows), kSuperTiles)), octets(ceil_div(c / kBlock, kOctet)) {}
    size_t code_bytes() const { return size_t(supertiles) * size_t(octets) * kCodeRegion; }
    size_t scale_bytes() const { return size_t(supertiles) * size_t(octets) * kScaleRegion; }
    size_t mx_scale_bytes() const { return size_t(supertiles) * size_t(octets) * kMxScaleRegion; }
    size_t scale_bytes(int fmt) const { return fmt == kMxfp4 ? mx_scale_bytes() : scale_bytes(); }
};

// Workgroups of a one-dimensional launch over `units` items at `threads`
// per workgroup, or 0 when they would pass the largest grid (2^31 - 1
// workgroups); the entry points return NVFP4_ESHAPE for 0 before launching,
// so no grid is ever truncated.
inline unsigned grid_1d(int64_t units, int threads) {
    const int64_t g = ceil_div(units, threads);
    return g < 1 || g > int64_t(0x7FFFFFFF) ? 0u : unsigned(g);
}

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace nvfp4
