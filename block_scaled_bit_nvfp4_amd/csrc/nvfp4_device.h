// nvfp4_device.h -- layout constants and in-register decode helpers shared by
// the gfx950 kernels of libnvfp4.  Internal to the library.
//
// NVFP4 as used here: E2M1 4-bit element codes, one E4M3 ("FN") scale byte
// per 16 consecutive elements of a row, one fp32 tensor scale.  The pages name
// this the block-scaled FP4 weight format of their decode matvec (bw24 wiki,
// feature list, NVFP4 decode-path item) and place E2M1 as its element
// (qwentin README, "Why it's interesting").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Repacked ("split-plane") layout; the public definition is in nvfp4.h.
constexpr int kTileRows = 16;   // rows per tile
constexpr int kRowPairs = 8;    // row pairs per tile
constexpr int kLanes = 64;      // blocks per step (one per lane of a wave64)
constexpr int kBlock = 16;      // elements per scale block

typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Two E2M1 codes (byte `Byte` of `word`, element 2i in the low nibble) -> two
// exact bf16 values packed low/high.  v_cvt_scalef32_pk_bf16_fp4 with scale
// 1.0; every E2M1 value is a bf16 value, so the conversion is exact.
template <int Byte>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, Byte);
}

// E4M3 byte `Byte` of `word` -> exact fp32 (OCP E4M3 on gfx950: bias 7,
// subnormals kept, 0x7F/0xFF NaN).
template <int Byte>
__device__ __forceinline__ float e4m3_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8(word, Byte);
}

__device__ __forceinline__ float e4m3_f32_dyn(uint32_t word, int byte) {
    switch (byte & 3) {
        case 0: return e4m3_f32<0>(word);
        case 1: return e4m3_f32<1>(word);
        case 2: return e4m3_f32<2>(word);
        default: return e4m3_f32<3>(word);
    }
}

// Streaming 16-byte load of weight bytes that are read once per call: the
// nontemporal hint keeps them from displacing reused data in the caches.
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ uint32_t as_u32(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// acc + a.lo*b.lo + a.hi*b.hi in fp32 (v_dot2_f32_bf16).  Each product of an
// E2M1 value and a bf16 value is exact in fp32.
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

}  // namespace nvfp4
