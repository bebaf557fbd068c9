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
constexpr int kBlock = 16;                            // elements per scale block
constexpr int kTileRows = 16;                         // rows per tile
constexpr int kSuperTiles = 4;                        // tiles per super-tile
constexpr int kSuperRows = kTileRows * kSuperTiles;   // 64
constexpr int kOctet = 8;                             // blocks per octet
constexpr int kLanes = 64;
constexpr int kCodeChunk = kLanes * 16;               // one tile's octet of codes: 1 KiB
constexpr int kScaleChunk = kTileRows * kOctet;       // one tile's octet of scales: 128 B
constexpr int kCodeRegion = kSuperTiles * kCodeChunk;     // one super-tile's octet: 4 KiB
constexpr int kScaleRegion = kSuperTiles * kScaleChunk;   // 512 B

// The second block-scaled format, MXFP4: the same E2M1 codes and code plane,
// one E8M0 scale byte (2^(b - 127)) per 32 elements; its scale plane holds
// 4 bytes per row and octet (the octet's four 32-element blocks).
enum ScaleFormat { kNvfp4 = 0, kMxfp4 = 1 };
constexpr int kMxBlock = 32;
constexpr int kMxScaleChunk = kTileRows * 4;                 // one tile's octet of MX scales: 64 B
constexpr int kMxScaleRegion = kSuperTiles * kMxScaleChunk;  // 256 B

typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Two E2M1 codes (byte `Byte` of `word`, the even element in the low nibble)
// -> two exact bf16 values packed low/high.  v_cvt_scalef32_pk_bf16_fp4 with
// scale 1.0; every E2M1 value is a bf16 value, so the conversion is exact.
template <int Byte>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, Byte);
}

// Eight E2M1 codes (one 32-bit word, element 0 in the lowest nibble) -> the
// eight exact bf16 values of an MFMA operand, in element order.
__device__ __forceinline__ bf16x8 e2m1x8_bf16(uint32_t word) {
    const bf16x2 p0 = e2m1x2_bf16<0>(word), p1 = e2m1x2_bf16<1>(word);
    const bf16x2 p2 = e2m1x2_bf16<2>(word), p3 = e2m1x2_bf16<3>(word);
    bf16x8 o;
    o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
    o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
    return o;
}

// E4M3 byte `Byte` of `word` -> exact fp32 (OCP E4M3 on gfx950: bias 7,
// subnormals kept, 0x7F/0xFF NaN).
template <int Byte>
__device__ __forceinline__ float e4m3_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8(word, Byte);
}

// E4M3 bytes 2 hi, 2 hi + 1 of `word` -> two exact fp32 (one v_cvt_pk_f32_fp8).
__device__ __forceinline__ float2 e4m3x2_f32(uint32_t word, int hi) {
    const auto v = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true) : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    return float2{v[0], v[1]};
}

__device__ __forceinline__ float e4m3_f32_dyn(uint32_t word, int byte) {
    switch (byte & 3) {
        case 0: return e4m3_f32<0>(word);
        case 1: return e4m3_f32<1>(word);
        case 2: return e4m3_f32<2>(word);
        default: return e4m3_f32<3>(word);
    }
}

// E8M0 byte b -> fp32 2^(b - 127): b = 0 is the subnormal 2^-127, 0xFF NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t b) {
    b &= 0xFFu;
    return __uint_as_float(b == 0xFFu ? 0x7FC00000u : (b == 0u ? 0x00400000u : b << 23));
}

// Eight E2M1 codes (one word) times 2^(b - 127) -> the eight exact bf16
// values of an MFMA operand.  The scaled conversion multiplies by the power
// of two in its scale operand's exponent field, so the E8M0 byte goes there
// (b = 0 gives 2^-127 as well); every product e2m1 * 2^(b - 127) below
// bf16's overflow is a bf16 value.  For finite bytes (not 0xFF).
__device__ __forceinline__ bf16x8 e2m1x8_bf16_e8m0(uint32_t word, uint32_t b) {
    const float s = __uint_as_float((b & 0xFFu) << 23);
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 3);
    bf16x8 o;
    o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
    o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
    return o;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ uint32_t as_u32(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// One DPP step of a 64-bit maximum: each lane takes the larger of its value
// and the value of the lane CTRL names (quad permutation or row mirror).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_u64(unsigned long long v) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(v)), CTRL, 0xF, 0xF, false));
    const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, false));
    const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
    return o > v ? o : v;
}

// Maximum of a 64-bit value over the rows (16-lane groups) of each aligned
// group of G lanes (G = 32 or 64), for values already reduced within rows
// (or per lane class): permlane swaps, no LDS.
template <int G>
__device__ __forceinline__ unsigned long long rows_max_u64(unsigned long long v) {
    static_assert(G == 32 || G == 64, "row group of 32 or 64 lanes");
    // rows (x0 x1 x2 x3) -> (x0 x0 x2 x2) and (x1 x1 x3 x3)
    const auto l = __builtin_amdgcn_permlane16_swap(uint32_t(v), uint32_t(v), false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(uint32_t(v >> 32), uint32_t(v >> 32), false, false);
    unsigned long long a = (static_cast<unsigned long long>(h[0]) << 32) | l[0];
    unsigned long long b = (static_cast<unsigned long long>(h[1]) << 32) | l[1];
    v = a > b ? a : b;
    if constexpr (G == 64) {
        // (y0 y1 y2 y3) -> (y0 y1 y0 y1) and (y2 y3 y2 y3)
        const auto l2 = __builtin_amdgcn_permlane32_swap(uint32_t(v), uint32_t(v), false, false);
        const auto h2 = __builtin_amdgcn_permlane32_swap(uint32_t(v >> 32), uint32_t(v >> 32), false, false);
        a = (static_cast<unsigned long long>(h2[0]) << 32) | l2[0];
        b = (static_cast<unsigned long long>(h2[1]) << 32) | l2[1];
        v = a > b ? a : b;
    }
    return v;
}

// Maximum of a 64-bit value over each aligned group of G lanes (G = 16, 32 or
// 64), left in every lane of the group, without LDS: quad swaps, then the
// half-row and row mirrors (16 lanes), then permlane swaps across rows.
// Every lane of a group must be active.
template <int G>
__device__ __forceinline__ unsigned long long lanes_max_u64(unsigned long long v) {
    static_assert(G == 16 || G == 32 || G == 64, "lane group of 16, 32 or 64");
    v = dpp_max_u64<0xB1>(v);    // quad_perm [1,0,3,2]
    v = dpp_max_u64<0x4E>(v);    // quad_perm [2,3,0,1]
    v = dpp_max_u64<0x141>(v);   // row_half_mirror: quads 0|1 and 2|3 of a row
    v = dpp_max_u64<0x140>(v);   // row_mirror: the two halves of a row
    if constexpr (G >= 32) v = rows_max_u64<G>(v);
    return v;
}

// v holds item g in lane group g (lanes 16g .. 16g + 15); returns o[k] = item
// k in every lane.  One v_permlane32_swap and two v_permlane16_swap.
__device__ __forceinline__ void gather_lane_groups(uint32_t v, uint32_t (&o)[4]) {
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);      // (v0 v1 v0 v1), (v2 v3 v2 v3)
    const auto b0 = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);   // (v0 ...), (v1 ...)
    const auto b1 = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);   // (v2 ...), (v3 ...)
    o[0] = b0[0];
    o[1] = b0[1];
    o[2] = b1[0];
    o[3] = b1[1];
}

// Buffer loads: offsets past the resource's byte count read zeros without a
// memory access, which bounds every prefetch and ragged tail without a branch.
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kStream = 2;               // nontemporal: weight bytes are read once per call

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes), kRsrcWord3);
}

}  // namespace nvfp4
