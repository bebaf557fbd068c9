// nvfp4_probe.hip -- the measured walls of libnvfp4_probe (see
// nvfp4_probe.h): a plain streaming read and a bare bf16 MFMA loop on
// gfx950.  A measurement aid; the product library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"
#include "nvfp4_probe.h"

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                              // loads in flight per thread
constexpr uint32_t kRound = kThreads * 16;              // bytes a workgroup's load instruction covers: 4 KiB
constexpr uint32_t kMagic = 0x9E3779B9u;

// Workgroup g reads its share [g * share, (g + 1) * share) of the buffer
// (share a multiple of 4 KiB) in rounds of eight loads per thread.  Its
// buffer resource spans only its share, clipped to the buffer's end, so the
// loads of the last round that pass either read zeros without touching
// memory.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint8_t *buf, uint64_t bytes, uint32_t share,
                                                               uint32_t *sink) {
    const uint64_t start = uint64_t(blockIdx.x) * share;
    const uint32_t mine = start >= bytes ? 0u : uint32_t(bytes - start < share ? bytes - start : share);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(buf + (start < bytes ? start : 0)),
                                                      (short)0, int(mine), 0x00020000);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint32_t off = threadIdx.x * 16u; off < mine; off += kRound * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * kRound, 0, 2));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    const uint32_t a = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (a == kMagic) sink[0] = a;
}

// The same read of `rbytes` bytes, then workgroup g stores its share
// [g * oshare, (g + 1) * oshare) of the `obytes`-byte output (oshare a
// multiple of 16) with 128-bit stores whose value comes from its loads, so
// they wait for them, as a product's outputs wait for its sums.
__global__ void __launch_bounds__(kThreads) stream_read_store_kernel(const uint8_t *buf, uint64_t rbytes, uint32_t rshare,
                                                                     uint8_t *out, uint64_t obytes, uint32_t oshare) {
    const uint64_t start = uint64_t(blockIdx.x) * rshare;
    const uint32_t mine = start >= rbytes ? 0u : uint32_t(rbytes - start < rshare ? rbytes - start : rshare);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(buf + (start < rbytes ? start : 0)),
                                                      (short)0, int(mine), 0x00020000);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint32_t off = threadIdx.x * 16u; off < mine; off += kRound * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * kRound, 0, 2));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    const uint64_t ostart = uint64_t(blockIdx.x) * oshare;
    const uint32_t omine = ostart >= obytes ? 0u : uint32_t(obytes - ostart < oshare ? obytes - ostart : oshare);
    for (uint32_t off = threadIdx.x * 16u; off + 16u <= omine; off += kRound)
        *reinterpret_cast<u32x4 *>(out + ostart + off) = acc;
}

__global__ void __launch_bounds__(1024) mfma_probe_kernel(int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float((lane + i) & 7) * 0.125f);
        b[i] = (__bf16)(float((lane * 3 + i) & 7) * 0.25f);
    }
    floatx4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (s == 1234.5f) sink[0] = s;
}

}  // namespace

PROBE_API int nvfp4_probe_stream_read(const void *buf, size_t bytes, int groups, uint32_t *sink,
                                      hipStream_t stream) {
    if (!buf || !sink || groups < 1 || groups > 65536) return NVFP4_EINVAL;
    if (bytes < 16 || bytes >= (size_t(1) << 31)) return NVFP4_ESHAPE;
    if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(sink) % 4) return NVFP4_EALIGN;
    const size_t per = (bytes + size_t(groups) - 1) / size_t(groups);
    const size_t share = (per + kRound - 1) / kRound * kRound;
    (void)hipGetLastError();
    hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(groups)), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t *>(buf), uint64_t(bytes), uint32_t(share), sink);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

PROBE_API int nvfp4_probe_stream_read_store(const void *buf, size_t rbytes, void *out, size_t obytes, int groups,
                                            hipStream_t stream) {
    if (!buf || !out || groups < 1 || groups > 65536) return NVFP4_EINVAL;
    if (rbytes < 16 || rbytes >= (size_t(1) << 31) || obytes < 16 || obytes >= (size_t(1) << 31) || obytes % 16)
        return NVFP4_ESHAPE;
    if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(out) % 16) return NVFP4_EALIGN;
    const size_t per = (rbytes + size_t(groups) - 1) / size_t(groups);
    const size_t rshare = (per + kRound - 1) / kRound * kRound;
    const size_t oper = (obytes + size_t(groups) - 1) / size_t(groups);
    const size_t oshare = (oper + 15) / 16 * 16;
    (void)hipGetLastError();
    hipLaunchKernelGGL(stream_read_store_kernel, dim3(unsigned(groups)), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t *>(buf), uint64_t(rbytes), uint32_t(rshare), static_cast<uint8_t *>(out),
                       uint64_t(obytes), uint32_t(oshare));
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

PROBE_API int nvfp4_probe_mfma_bf16(int groups, int waves, int iters, float *sink, hipStream_t stream) {
    if (!sink || groups < 1 || groups > 65536 || waves < 1 || waves > 16 || iters < 1) return NVFP4_EINVAL;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(unsigned(groups)), dim3(unsigned(64 * waves)), 0, stream, iters, sink);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}
