// nvfp4_quant.hip -- quantise, repack and dequantise kernels (gfx950) and
// their C-ABI entry points.
//
// quantise: fp32 -> canonical NVFP4, the at-load re-encode of higher
//   precision weights (bw24 wiki, feature list, safetensors-loader item).
// repack:   canonical -> split-plane regions read by the products (bw24 wiki,
//   feature list, NVFP4 decode-path item; the loader's NVFP4 repack is
//   byte-exact, and so is this one).
// dequant:  repacked -> fp32 / bf16, a verification export of the decode.
#include "nvfp4_host.h"

namespace nvfp4 {

// ----------------------------------------------------------------- quantise

// Nearest E4M3 byte to q >= 0 (ties to even mantissa, saturating at 448,
// subnormal spacing 2^-9).  q / quantum is an exact power-of-two scaling, and
// rint() rounds half to even in the default rounding mode.
__device__ __forceinline__ uint32_t e4m3_rne(double q) {
    if (!(q > 0.0)) return 0u;
    if (q >= 448.0) return 0x7Eu;
    int e;
    (void)frexp(q, &e);            // q in [2^(e-1), 2^e)
    int E = e - 1;                  // unbiased exponent of q
    if (E < -6) {                   // subnormal range: m * 2^-9, m in [0, 8]
        double m = rint(ldexp(q, 9));
        return uint32_t(m);         // m == 8 encodes 2^-6 (0x08), still right
    }
    double m = rint(ldexp(q, 3 - E));   // in [8, 16]
    return uint32_t((E + 7) << 3) + uint32_t(m) - 8u;   // m == 16 carries into E
}

// E2M1 magnitude code of v >= 0, nearest with ties to the even code,
// saturating at 6.  Midpoints 0.25 .. 5 are exact; at a midpoint whose upper
// neighbour has the even code the comparison is >=, otherwise >.
__device__ __forceinline__ uint32_t e2m1_rne_mag(double v) {
    return uint32_t(v > 0.25) + uint32_t(v >= 0.75) + uint32_t(v > 1.25) + uint32_t(v >= 1.75) +
           uint32_t(v > 2.5) + uint32_t(v >= 3.5) + uint32_t(v > 5.0);
}

// Exact value of an E4M3 byte as fp64 (finite bytes only: the quantiser
// never produces 0x7F).
__device__ __forceinline__ double e4m3_f64(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    return e == 0 ? ldexp(double(m), -9) : ldexp(double(8u + m), int(e) - 10);
}

// One thread per 16-element block.
__global__ void __launch_bounds__(256) quantize_kernel(const float4 *__restrict__ W, int64_t nblocks,
                                                       float tscale, uint2 *__restrict__ codes,
                                                       uint8_t *__restrict__ scales) {
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    float w[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float4 f = W[i * 4 + v];
        w[4 * v + 0] = f.x; w[4 * v + 1] = f.y; w[4 * v + 2] = f.z; w[4 * v + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(w[k]));
    const double t = double(tscale);
    uint32_t sb = e4m3_rne(double(amax) / (6.0 * t));
    uint32_t out[2] = {0u, 0u};
    if (sb != 0u) {
        const double denom = e4m3_f64(sb) * t;     // exact: 4 x 24 significant bits
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            uint32_t c = e2m1_rne_mag(fabs(double(w[k])) / denom);
            c |= signbit(w[k]) ? 8u : 0u;
            out[k >> 3] |= c << (4 * (k & 7));
        }
    }
    codes[i] = make_uint2(out[0], out[1]);
    scales[i] = uint8_t(sb);
}

// MXFP4: one thread per 32-element block.  E = floor(log2(amax / tscale)) - 2
// (2 = the largest E2M1 exponent), clamped to [-127, 127] (amax = 0 gives
// -127), read exactly off the fp64 exponent of the quotient; the scale byte
// is E + 127 and each code the E2M1 nearest (ties to even, saturating at 6)
// to |w| / (2^E * tscale), decided on that exact fp64 quotient.
__global__ void __launch_bounds__(256) mx_quantize_kernel(const float4 *__restrict__ W, int64_t nblocks,
                                                          float tscale, uint4 *__restrict__ codes,
                                                          uint8_t *__restrict__ scales) {
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    float w[kMxBlock];
#pragma unroll
    for (int v = 0; v < kMxBlock / 4; ++v) {
        float4 f = W[i * (kMxBlock / 4) + v];
        w[4 * v + 0] = f.x; w[4 * v + 1] = f.y; w[4 * v + 2] = f.z; w[4 * v + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < kMxBlock; ++k) amax = fmaxf(amax, fabsf(w[k]));
    const double t = double(tscale);
    const double q = double(amax) / t;
    int E = -127;
    if (q > 0.0) {
        int e;
        (void)frexp(q, &e);        // q in [2^(e-1), 2^e)
        E = e - 3;
        E = E < -127 ? -127 : (E > 127 ? 127 : E);
    }
    const double denom = ldexp(1.0, E) * t;   // exact
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kMxBlock; ++k) {
        uint32_t c = e2m1_rne_mag(fabs(double(w[k])) / denom);
        c |= signbit(w[k]) ? 8u : 0u;
        out[k >> 3] |= c << (4 * (k & 7));
    }
    codes[i] = make_uint4(out[0], out[1], out[2], out[3]);
    scales[i] = uint8_t(E + 127);
}

// ------------------------------------------------------------------- repack

// Threads [0, code_units) write one 16-byte code entry (st, o, tt, lane)
// each; threads [code_units, code_units + scale_units) one scale entry
// (st, o, tt, r) each: 8 bytes (the octet's eight 16-element blocks) for
// NVFP4, 4 bytes (its four 32-element blocks) for MXFP4.  The code plane is
// the same for both formats.
template <int FMT>
__global__ void __launch_bounds__(256) repack_kernel(const uint8_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ scales, int64_t rows,
                                                     int64_t cols, int64_t octets, int64_t code_units,
                                                     int64_t scale_units, uint4 *__restrict__ wq,
                                                     void *__restrict__ ws) {
    int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t kb = cols / kBlock;
    if (u < code_units) {
        const int l = int(u % kLanes), tt = int((u / kLanes) % kSuperTiles);
        const int64_t rest = u / (kLanes * kSuperTiles), o = rest % octets, st = rest / octets;
        const int g = l >> 4, r = l & 15;
        const int64_t row = st * kSuperRows + tt * kTileRows + r;
        uint32_t v[4] = {0u, 0u, 0u, 0u};
        if (row < rows) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int64_t b = o * kOctet + 2 * d + (g >> 1);
                if (b < kb) v[d] = *reinterpret_cast<const uint32_t *>(codes + row * (cols / 2) + b * 8 + 4 * (g & 1));
            }
        }
        wq[u] = make_uint4(v[0], v[1], v[2], v[3]);
        return;
    }
    u -= code_units;
    if (u >= scale_units) return;
    const int r = int(u % kTileRows), tt = int((u / kTileRows) % kSuperTiles);
    const int64_t rest = u / (kTileRows * kSuperTiles), o = rest % octets, st = rest / octets;
    const int64_t row = st * kSuperRows + tt * kTileRows + r;
    if (FMT == kMxfp4) {
        const int64_t kbm = cols / kMxBlock;
        uint32_t v = 0u;
        if (row < rows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t b = o * 4 + i;
                if (b < kbm) v |= uint32_t(scales[row * kbm + b]) << (8 * i);
            }
        }
        static_cast<uint32_t *>(ws)[u] = v;
        return;
    }
    uint32_t v[2] = {0u, 0u};
    if (row < rows) {
#pragma unroll
        for (int i = 0; i < kOctet; ++i) {
            const int64_t b = o * kOctet + i;
            if (b < kb) v[i >> 2] |= uint32_t(scales[row * kb + b]) << (8 * (i & 3));
        }
    }
    static_cast<uint2 *>(ws)[u] = make_uint2(v[0], v[1]);
}

// ------------------------------------------------------------------ dequant

// One thread per 16-byte code entry: 4 half-blocks (8 elements) of one row.
__global__ void __launch_bounds__(256) dequant_kernel(const uint4 *__restrict__ wq,
                                                      const uint2 *__restrict__ ws, float tscale,
                                                      int64_t rows, int64_t cols, int64_t octets,
                                                      int64_t code_units, float *__restrict__ out_f32,
                                                      uint16_t *__restrict__ out_bf16) {
    const int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (u >= code_units) return;
    const int l = int(u % kLanes), tt = int((u / kLanes) % kSuperTiles);
    const int64_t rest = u / (kLanes * kSuperTiles), o = rest % octets, st = rest / octets;
    const int g = l >> 4, r = l & 15;
    const int64_t row = st * kSuperRows + tt * kTileRows + r;
    if (row >= rows) return;
    const uint4 c = wq[u];
    const uint2 sc = ws[(rest * kSuperTiles + tt) * kTileRows + r];
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int ib = 2 * d + (g >> 1);                 // block within the octet
        const int64_t b = o * kOctet + ib;
        if (b >= cols / kBlock) continue;
        const float s = e4m3_f32_dyn(ib < 4 ? sc.x : sc.y, ib & 3);
        const uint32_t pairs[4] = {as_u32(e2m1x2_bf16<0>(cw[d])), as_u32(e2m1x2_bf16<1>(cw[d])),
                                   as_u32(e2m1x2_bf16<2>(cw[d])), as_u32(e2m1x2_bf16<3>(cw[d]))};
        float v[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v[2 * p + 0] = __uint_as_float(pairs[p] << 16) * s;          // exact
            v[2 * p + 1] = __uint_as_float(pairs[p] & 0xFFFF0000u) * s;  // exact
        }
        const int64_t off = row * cols + b * kBlock + 8 * (g & 1);
        if (out_bf16) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (__float_as_uint(v[2 * e]) >> 16) | (__float_as_uint(v[2 * e + 1]) & 0xFFFF0000u);
            *reinterpret_cast<uint4 *>(out_bf16 + off) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if (out_f32) {
            float4 *dst = reinterpret_cast<float4 *>(out_f32 + off);
            dst[0] = make_float4(v[0] * tscale, v[1] * tscale, v[2] * tscale, v[3] * tscale);
            dst[1] = make_float4(v[4] * tscale, v[5] * tscale, v[6] * tscale, v[7] * tscale);
        }
    }
}

// MXFP4: one thread per 16-byte code entry; word d is 8 elements of the
// octet's 32-element block d, whose E8M0 scale is byte d of the row's scale
// entry.  e2m1 * 2^(b - 127) is exact in bf16 (below its overflow); the fp32
// output is e2m1 * 2^(b - 127) * tscale, rounded once.
__global__ void __launch_bounds__(256) mx_dequant_kernel(const uint4 *__restrict__ wq,
                                                         const uint32_t *__restrict__ ws, float tscale,
                                                         int64_t rows, int64_t cols, int64_t octets,
                                                         int64_t code_units, float *__restrict__ out_f32,
                                                         uint16_t *__restrict__ out_bf16) {
    const int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (u >= code_units) return;
    const int l = int(u % kLanes), tt = int((u / kLanes) % kSuperTiles);
    const int64_t rest = u / (kLanes * kSuperTiles), o = rest % octets, st = rest / octets;
    const int g = l >> 4, r = l & 15;
    const int64_t row = st * kSuperRows + tt * kTileRows + r;
    if (row >= rows) return;
    const uint4 c = wq[u];
    const uint32_t sc = ws[(rest * kSuperTiles + tt) * kTileRows + r];
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int64_t k0 = o * (kOctet * kBlock) + d * kMxBlock;
        if (k0 >= cols) continue;
        const uint32_t b = (sc >> (8 * d)) & 0xFFu;
        // The eight bf16 values as four 32-bit pairs (a whole-vector bit cast;
        // taking the vector's bf16 elements one by one loses all but one of
        // the conversions in this compiler).
        const u32x4 pairs = __builtin_bit_cast(u32x4, e2m1x8_bf16_e8m0(cw[d], b));
        const int64_t off = row * cols + k0 + 8 * g;
        uint32_t bits[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bits[2 * e] = b == 0xFFu ? 0x7FC0u : (pairs[e] & 0xFFFFu);
            bits[2 * e + 1] = b == 0xFFu ? 0x7FC0u : (pairs[e] >> 16);
        }
        if (out_bf16) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = bits[2 * e] | (bits[2 * e + 1] << 16);
            *reinterpret_cast<uint4 *>(out_bf16 + off) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if (out_f32) {
            // e2m1 * 2^(b - 127) * tscale in fp64 (exact), rounded once: the
            // bf16 value above may already be past fp32's range where the
            // product with tscale is not.
            const u32x4 plain = __builtin_bit_cast(u32x4, e2m1x8_bf16(cw[d]));
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t pb = e & 1 ? plain[e >> 1] & 0xFFFF0000u : plain[e >> 1] << 16;
                f[e] = b == 0xFFu ? __uint_as_float(0x7FC00000u)
                                  : float(ldexp(double(__uint_as_float(pb)), int(b) - 127) * double(tscale));
            }
            float4 *dst = reinterpret_cast<float4 *>(out_f32 + off);
            dst[0] = make_float4(f[0], f[1], f[2], f[3]);
            dst[1] = make_float4(f[4], f[5], f[6], f[7]);
        }
    }
}

}  // namespace nvfp4

using namespace nvfp4;

NVFP4_API size_t nvfp4_repacked_code_bytes(int64_t rows, int64_t cols) {
    return check_shape(rows, cols) == NVFP4_OK ? Geometry(rows, cols).code_bytes() : 0;
}

NVFP4_API size_t nvfp4_repacked_scale_bytes(int64_t rows, int64_t cols) {
    return check_shape(rows, cols) == NVFP4_OK ? Geometry(rows, cols).scale_bytes() : 0;
}

NVFP4_API int nvfp4_quantize(const float *W, int64_t rows, int64_t cols, float tscale,
                             uint8_t *codes, uint8_t *scales, hipStream_t stream) {
    if (!W || !codes || !scales || !tscale_ok(tscale)) return NVFP4_EINVAL;
    if (int st = check_shape(rows, cols)) return st;
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 16)) return NVFP4_EALIGN;
    const int64_t nblocks = rows * (cols / kBlock);
    const unsigned grid = grid_1d(nblocks, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(quantize_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(W), nblocks, tscale,
                       reinterpret_cast<uint2 *>(codes), scales);
    return launch_status();
}

NVFP4_API int nvfp4_repack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                           uint8_t *wq, uint8_t *ws, hipStream_t stream) {
    if (!codes || !scales || !wq || !ws) return NVFP4_EINVAL;
    if (int st = check_shape(rows, cols)) return st;
    if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(wq, 16) || !aligned(ws, 16))
        return NVFP4_EALIGN;
    const Geometry g(rows, cols);
    const int64_t code_units = int64_t(g.code_bytes() / 16), scale_units = int64_t(g.scale_bytes() / 8);
    const unsigned grid = grid_1d(code_units + scale_units, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(repack_kernel<kNvfp4>, dim3(grid), dim3(256),
                       0, stream, codes, scales, rows, cols, g.octets, code_units, scale_units,
                       reinterpret_cast<uint4 *>(wq), static_cast<void *>(ws));
    return launch_status();
}

NVFP4_API int nvfp4_dequant(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows,
                            int64_t cols, float *out_f32, uint16_t *out_bf16, hipStream_t stream) {
    if (!wq || !ws || (!out_f32 && !out_bf16) || !tscale_ok(tscale)) return NVFP4_EINVAL;
    if (int st = check_shape(rows, cols)) return st;
    if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(out_f32, 16) || !aligned(out_bf16, 16))
        return NVFP4_EALIGN;
    const Geometry g(rows, cols);
    const int64_t code_units = int64_t(g.code_bytes() / 16);
    const unsigned grid = grid_1d(code_units, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(wq), reinterpret_cast<const uint2 *>(ws), tscale,
                       rows, cols, g.octets, code_units, out_f32, out_bf16);
    return launch_status();
}

// ------------------------------------------------------------------ MXFP4

NVFP4_API size_t mxfp4_repacked_code_bytes(int64_t rows, int64_t cols) {
    return check_mx_shape(rows, cols) == NVFP4_OK ? Geometry(rows, cols).code_bytes() : 0;
}

NVFP4_API size_t mxfp4_repacked_scale_bytes(int64_t rows, int64_t cols) {
    return check_mx_shape(rows, cols) == NVFP4_OK ? Geometry(rows, cols).mx_scale_bytes() : 0;
}

NVFP4_API int mxfp4_quantize(const float *W, int64_t rows, int64_t cols, float tscale, uint8_t *codes,
                             uint8_t *scales, hipStream_t stream) {
    if (!W || !codes || !scales || !tscale_ok(tscale)) return NVFP4_EINVAL;
    if (int st = check_mx_shape(rows, cols)) return st;
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 16)) return NVFP4_EALIGN;
    const int64_t nblocks = rows * (cols / kMxBlock);
    const unsigned grid = grid_1d(nblocks, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mx_quantize_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(W), nblocks, tscale, reinterpret_cast<uint4 *>(codes),
                       scales);
    return launch_status();
}

NVFP4_API int mxfp4_repack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                           uint8_t *wq, uint8_t *ws, hipStream_t stream) {
    if (!codes || !scales || !wq || !ws) return NVFP4_EINVAL;
    if (int st = check_mx_shape(rows, cols)) return st;
    if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(wq, 16) || !aligned(ws, 16))
        return NVFP4_EALIGN;
    const Geometry g(rows, cols);
    const int64_t code_units = int64_t(g.code_bytes() / 16), scale_units = int64_t(g.mx_scale_bytes() / 4);
    const unsigned grid = grid_1d(code_units + scale_units, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(repack_kernel<kMxfp4>, dim3(grid), dim3(256),
                       0, stream, codes, scales, rows, cols, g.octets, code_units, scale_units,
                       reinterpret_cast<uint4 *>(wq), static_cast<void *>(ws));
    return launch_status();
}

NVFP4_API int mxfp4_dequant(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                            float *out_f32, uint16_t *out_bf16, hipStream_t stream) {
    if (!wq || !ws || (!out_f32 && !out_bf16) || !tscale_ok(tscale)) return NVFP4_EINVAL;
    if (int st = check_mx_shape(rows, cols)) return st;
    if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(out_f32, 16) || !aligned(out_bf16, 16))
        return NVFP4_EALIGN;
    const Geometry g(rows, cols);
    const int64_t code_units = int64_t(g.code_bytes() / 16);
    const unsigned grid = grid_1d(code_units, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mx_dequant_kernel, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(wq), reinterpret_cast<const uint32_t *>(ws), tscale, rows,
                       cols, g.octets, code_units, out_f32, out_bf16);
    return launch_status();
}
