// nvfp4_gemv.hip -- the NVFP4 x bf16 matrix-vector products on the VALU
// (n <= 8 columns), the argmax epilogue of the vocabulary projection, and the
// SwiGLU step between MLP matvecs; gfx950.
//
// Pages: bw24 wiki (GitHub), feature list -- the NVFP4 decode matvec over
// split-plane repacked weights, picked per matrix shape, and the batched K+1
// verify that reads each weight once for every column; bw24 wiki, exactness
// note after the gate list -- summation order is part of the contract;
// qwentin README (gitlite mirror), "How it works" -- dense-argmax descent over
// the draft tree and the persistent-MLP decode GEMV.
//
// Work decomposition.  One workgroup per 16-row tile; its `ksplit` waves
// take contiguous ranges of 64-block steps (the per-lane step is described in
// nvfp4_valu.h).  The reduction over lanes and waves has a fixed shape that
// depends only on (rows, cols), never on n or on timing.
#include "nvfp4_valu.h"

namespace nvfp4 {

template <int N, bool ARGMAX>
__global__ void __launch_bounds__(kLanes * kMaxKsplit)
gemv_valu_kernel(const uint4 *__restrict__ wq, const uint4 *__restrict__ ws, float tscale, int rows,
                 int kb, int steps, int ksplit, const uint16_t *__restrict__ X, int64_t x_stride,
                 float *__restrict__ Y, int64_t y_stride, unsigned long long *__restrict__ amax_ws,
                 int32_t *__restrict__ argmax_out) {
    __shared__ float red[kMaxKsplit][kTileRows][N];
    const int t = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int j0 = (steps * wave) / ksplit;
    const int j1 = (steps * (wave + 1)) / ksplit;

    Frag<N> f;
    clear(f);
    accumulate_steps<N>(f, wq, ws, X, x_stride, t, j0, j1, steps, kb, lane);

    wave_reduce<N>(f, lane);
    if ((lane & 3) == 0) {
        const int r = reduced_row(lane);
#pragma unroll
        for (int n = 0; n < N; ++n) red[wave][r][n] = f.acc[0][n];
    }
    __syncthreads();
    if (wave != 0) return;

    // lane = n * 16 + r covers the tile's outputs in two rounds for n > 4.
#pragma unroll
    for (int base = 0; base < kTileRows * N; base += kLanes) {
        const int idx = base + lane;
        const bool live = idx < kTileRows * N;
        const int n = live ? idx / kTileRows : 0;
        const int r = idx % kTileRows;
        float total = 0.0f;
        if (live) {
            total = red[0][r][n];
            for (int w = 1; w < ksplit; ++w) total += red[w][r][n];
        }
        const float y = total * tscale;
        const int row = t * kTileRows + r;
        const bool valid = live && row < rows;
        if (valid && Y) Y[n * y_stride + row] = y;
        if (ARGMAX) {
            unsigned long long key = valid ? argmax_key(y, uint32_t(row)) : 0ull;
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                const unsigned long long other = __shfl_xor(key, o);
                key = other > key ? other : key;
            }
            if (live && r == 0 && key != 0ull)
                __hip_atomic_fetch_max(amax_ws + n, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (ARGMAX) {
        // The last tile to finish turns the keys into row indices and returns
        // the workspace to all-zero for the next call.  The maxima are
        // order-independent, so the result does not depend on which tile is
        // last.  Keys and counter are touched only by device-scope atomics,
        // which are coherent across the XCDs' L2s without cache maintenance;
        // waiting for this wave's key atomics to complete before the counter
        // increment orders them (an agent-scope fence would write back and
        // invalidate L2 in every tile instead).
        unsigned int *counter = reinterpret_cast<unsigned int *>(amax_ws + kMaxValuN);
        __builtin_amdgcn_s_waitcnt(0);
        unsigned int prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __shfl(prev, 0);
        if (prev == gridDim.x - 1) {
            if (lane < N) {
                const unsigned long long k =
                    __hip_atomic_exchange(amax_ws + lane, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                argmax_out[lane] = int32_t(0xFFFFFFFFu - uint32_t(k));
            }
            if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------------ SwiGLU

// SiLU(g) * u in fp32 and its nearest-even bf16 bits; the one definition the
// separate SwiGLU kernel and the fused gate||up kernel share.
__device__ __forceinline__ float swiglu_f32(float g, float u) { return g * u / (1.0f + expf(-g)); }

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;     // finite v
}

__global__ void __launch_bounds__(256) swiglu_kernel(const float *__restrict__ gu, int64_t F, int64_t total,
                                                     uint16_t *__restrict__ h) {
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t n = i / F, c = i % F;
    h[i] = uint16_t(bf16_rne_bits(swiglu_f32(gu[n * 2 * F + c], gu[n * 2 * F + F + c])));
}

// The gate||up product with SwiGLU in its epilogue: one workgroup per pair
// (gate tile p, up tile p + F/16) of the stacked [2F][K] matrix, `ksplit`
// waves per tile with the k split the plain matvec uses for that matrix, so
// gu and h carry the bits of nvfp4_gemv followed by nvfp4_swiglu; the fp32
// gate/up values never travel through memory unless asked for.
// Up to 16 waves (k split 8) at one column, whose matvec fits 128 registers;
// up to 8 waves (k split 4) otherwise.
template <int N>
constexpr int swiglu_max_waves() { return N == 1 ? 2 * kMaxKsplit : kMaxKsplit; }

template <int N>
__global__ void __launch_bounds__(kLanes * swiglu_max_waves<N>())
gemv_swiglu_kernel(const uint4 *__restrict__ wq, const uint4 *__restrict__ ws, float tscale, int F, int kb,
                   int steps, int ksplit, const uint16_t *__restrict__ X, int64_t x_stride,
                   float *__restrict__ gu_out, uint16_t *__restrict__ h) {
    __shared__ float red[2 * kMaxKsplit][kTileRows][N];
    const int pair = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int half = wave / ksplit, part = wave % ksplit;       // half 0: gate, 1: up
    const int t = pair + half * (F / kTileRows);
    const int j0 = (steps * part) / ksplit;
    const int j1 = (steps * (part + 1)) / ksplit;

    Frag<N> f;
    clear(f);
    accumulate_steps<N>(f, wq, ws, X, x_stride, t, j0, j1, steps, kb, lane);
    wave_reduce<N>(f, lane);
    if ((lane & 3) == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) red[wave][reduced_row(lane)][n] = f.acc[0][n];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int idx = lane; idx < kTileRows * N; idx += kLanes) {
        const int n = idx / kTileRows, r = idx % kTileRows;
        float g = red[0][r][n], u = red[ksplit][r][n];
        for (int w = 1; w < ksplit; ++w) {
            g += red[w][r][n];
            u += red[ksplit + w][r][n];
        }
        g *= tscale;
        u *= tscale;
        const int row = pair * kTileRows + r;
        if (gu_out) {
            gu_out[int64_t(n) * 2 * F + row] = g;
            gu_out[int64_t(n) * 2 * F + F + row] = u;
        }
        h[int64_t(n) * F + row] = uint16_t(bf16_rne_bits(swiglu_f32(g, u)));
    }
}

// ------------------------------------------------------------------ dispatch

template <bool ARGMAX>
int launch_valu(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, unsigned long long *amax_ws, int32_t *argmax_out, hipStream_t stream) {
    const int ksplit = choose_ksplit(g.tiles, g.steps);
    const dim3 grid(unsigned(g.tiles)), block(unsigned(kLanes * ksplit));
    auto q = reinterpret_cast<const uint4 *>(wq);
    auto s = reinterpret_cast<const uint4 *>(ws);
    const int rows = int(g.rows), kb = int(g.kb), steps = int(g.steps);
    const int64_t xs = g.cols, ys = g.rows;
#define NVFP4_LAUNCH(NN)                                                                            \
    hipLaunchKernelGGL((gemv_valu_kernel<NN, ARGMAX>), grid, block, 0, stream, q, s, tscale, rows, kb, \
                       steps, ksplit, X, xs, Y, ys, amax_ws, argmax_out)
    switch (n) {
        case 1: NVFP4_LAUNCH(1); break;
        case 2: NVFP4_LAUNCH(2); break;
        case 3: NVFP4_LAUNCH(3); break;
        case 4: NVFP4_LAUNCH(4); break;
        case 5: NVFP4_LAUNCH(5); break;
        case 6: NVFP4_LAUNCH(6); break;
        case 7: NVFP4_LAUNCH(7); break;
        case 8: NVFP4_LAUNCH(8); break;
        default: return NVFP4_EINVAL;
    }
#undef NVFP4_LAUNCH
    return launch_status();
}

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream);

int launch_gemv_swiglu(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t hidden, int64_t F,
                       const uint16_t *X, int n, float *gu, uint16_t *h, hipStream_t stream) {
    const Geometry g(2 * F, hidden);
    const int ksplit = choose_ksplit(g.tiles, g.steps);
    const int max_waves = n == 1 ? swiglu_max_waves<1>() : swiglu_max_waves<2>();
    if (2 * ksplit > max_waves) {
        // Narrow MLPs (F < 4096) over a wide hidden dimension split k further
        // than one workgroup can hold for n > 1: the plain matvec into gu,
        // then the SwiGLU kernel, give the same bits.
        if (!gu) return NVFP4_ESHAPE;
        if (int st = launch_valu<false>(g, wq, ws, tscale, X, n, gu, nullptr, nullptr, stream)) return st;
        hipLaunchKernelGGL(swiglu_kernel, dim3(unsigned(ceil_div(F * n, 256))), dim3(256), 0, stream, gu, F,
                           F * n, h);
        return launch_status();
    }
    const dim3 grid(unsigned(F / kTileRows)), block(unsigned(kLanes * 2 * ksplit));
    auto q = reinterpret_cast<const uint4 *>(wq);
    auto s = reinterpret_cast<const uint4 *>(ws);
#define NVFP4_LAUNCH(NN)                                                                                   \
    hipLaunchKernelGGL(gemv_swiglu_kernel<NN>, grid, block, 0, stream, q, s, tscale, int(F), int(g.kb), \
                       int(g.steps), ksplit, X, int64_t(hidden), gu, h)
    switch (n) {
        case 1: NVFP4_LAUNCH(1); break;
        case 2: NVFP4_LAUNCH(2); break;
        case 3: NVFP4_LAUNCH(3); break;
        case 4: NVFP4_LAUNCH(4); break;
        case 5: NVFP4_LAUNCH(5); break;
        case 6: NVFP4_LAUNCH(6); break;
        case 7: NVFP4_LAUNCH(7); break;
        case 8: NVFP4_LAUNCH(8); break;
        default: return NVFP4_EINVAL;
    }
#undef NVFP4_LAUNCH
    return launch_status();
}

}  // namespace nvfp4

using namespace nvfp4;

static int check_product_args(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                              const uint16_t *X, int n) {
    if (!wq || !ws || !X || !tscale_ok(tscale) || n < 1 || n > NVFP4_MAX_N) return NVFP4_EINVAL;
    if (int st = check_shape(rows, cols)) return st;
    if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(X, 16)) return NVFP4_EALIGN;
    return NVFP4_OK;
}

NVFP4_API int nvfp4_gemv(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                         const uint16_t *X, int n, float *Y, hipStream_t stream) {
    if (!Y) return NVFP4_EINVAL;
    if (int st = check_product_args(wq, ws, tscale, rows, cols, X, n)) return st;
    if (!aligned(Y, 4)) return NVFP4_EALIGN;
    const Geometry g(rows, cols);
    (void)hipGetLastError();
    if (n <= kMaxValuN) return launch_valu<false>(g, wq, ws, tscale, X, n, Y, nullptr, nullptr, stream);
    return launch_mfma(g, wq, ws, tscale, X, n, Y, stream);
}

NVFP4_API size_t nvfp4_gemv_argmax_workspace_bytes(int n) {
    // kMaxValuN 64-bit keys and a 32-bit completion counter, whatever n.
    return (n >= 1 && n <= kMaxValuN) ? size_t(8) * (kMaxValuN + 1) : 0;
}

NVFP4_API int nvfp4_gemv_argmax(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows,
                                int64_t cols, const uint16_t *X, int n, float *logits, int32_t *argmax,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!argmax || !workspace) return NVFP4_EINVAL;
    if (int st = check_product_args(wq, ws, tscale, rows, cols, X, n)) return st;
    if (n > kMaxValuN) return NVFP4_EINVAL;
    if (!aligned(logits, 4) || !aligned(argmax, 4) || !aligned(workspace, 8)) return NVFP4_EALIGN;
    if (workspace_bytes < nvfp4_gemv_argmax_workspace_bytes(n)) return NVFP4_EWORKSPACE;
    if (rows > int64_t(0x7FFFFFFF)) return NVFP4_ESHAPE;
    const Geometry g(rows, cols);
    (void)hipGetLastError();
    return launch_valu<true>(g, wq, ws, tscale, X, n, logits, static_cast<unsigned long long *>(workspace),
                             argmax, stream);
}

NVFP4_API int nvfp4_gemv_swiglu(const uint8_t *wq_gu, const uint8_t *ws_gu, float tscale, int64_t hidden,
                                int64_t F, const uint16_t *X, int n, float *gu, uint16_t *h,
                                hipStream_t stream) {
    if (!h) return NVFP4_EINVAL;
    if (F < kTileRows || F % kTileRows != 0) return NVFP4_ESHAPE;
    if (int st = check_product_args(wq_gu, ws_gu, tscale, 2 * F, hidden, X, n)) return st;
    if (n > kMaxValuN) return NVFP4_EINVAL;
    if (!aligned(gu, 4) || !aligned(h, 2)) return NVFP4_EALIGN;
    (void)hipGetLastError();
    return launch_gemv_swiglu(wq_gu, ws_gu, tscale, hidden, F, X, n, gu, h, stream);
}

NVFP4_API int nvfp4_swiglu(const float *gu, int64_t F, int n, uint16_t *h, hipStream_t stream) {
    if (!gu || !h || n < 1 || n > NVFP4_MAX_N) return NVFP4_EINVAL;
    if (F < 1 || F > (int64_t(1) << 40)) return NVFP4_ESHAPE;
    if (!aligned(gu, 16) || !aligned(h, 4)) return NVFP4_EALIGN;
    const int64_t total = F * n;
    (void)hipGetLastError();
    hipLaunchKernelGGL(swiglu_kernel, dim3(unsigned(ceil_div(total, 256))), dim3(256), 0, stream, gu, F, total, h);
    return launch_status();
}
