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
// take contiguous ranges of 64-block steps.  Per step, lane l owns block
// 64j + l of all 16 rows: 8 code loads of 16 bytes (one per row pair, each
// wave load 8 full 128-byte lines), one 16-byte scale load, and 32 bytes of
// each activation column, all 128-bit and coalesced across the wave.  The 16 rows reuse the activation registers.
// Decode is one v_cvt_scalef32_pk_bf16_fp4 per 2 codes and one E4M3
// conversion per row-block, shared by all columns; each column then takes 8
// v_dot2_f32_bf16 per row-block (products exact in fp32) and one fp32 FMA by
// the block scale.  The reduction over lanes and waves has a fixed shape that
// depends only on (rows, cols), never on n or on timing.
#include "nvfp4_host.h"

namespace nvfp4 {

constexpr int kMaxValuN = 8;
constexpr int kMaxKsplit = 8;
constexpr int kPrefetchMaxN = 4;   // beyond this, double-buffered operands exceed the register file

// Argmax key: order-preserving map of an fp32 value (with -0 folded into +0)
// in the high word, the complement of the row index in the low word, so the
// unsigned maximum picks the largest value and, among equals, the lowest row.
__device__ __forceinline__ unsigned long long argmax_key(float y, uint32_t row) {
    uint32_t b = __float_as_uint(y == 0.0f ? 0.0f : y);
    uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<unsigned long long>(k) << 32) | (0xFFFFFFFFu - row);
}

template <int N>
struct Frag {
    float acc[kTileRows][N];
};

// acc[r][c] += s_r * sum over the block of e2m1 * x_c for the 16 rows of one
// (tile, step) entry held by this lane.
template <int N>
__device__ __forceinline__ void mac_step(Frag<N> &f, const uint4 (&c)[kRowPairs], const uint4 &sc,
                                         const uint32_t (&x)[N][8]) {
    const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
    for (int q = 0; q < kRowPairs; ++q) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 2 * q + h;
            const uint32_t d0 = h ? c[q].z : c[q].x;
            const uint32_t d1 = h ? c[q].w : c[q].y;
            bf16x2 p[8];
            p[0] = e2m1x2_bf16<0>(d0);
            p[1] = e2m1x2_bf16<1>(d0);
            p[2] = e2m1x2_bf16<2>(d0);
            p[3] = e2m1x2_bf16<3>(d0);
            p[4] = e2m1x2_bf16<0>(d1);
            p[5] = e2m1x2_bf16<1>(d1);
            p[6] = e2m1x2_bf16<2>(d1);
            p[7] = e2m1x2_bf16<3>(d1);
            float s;
            switch (r & 3) {
                case 0: s = e4m3_f32<0>(sw[r >> 2]); break;
                case 1: s = e4m3_f32<1>(sw[r >> 2]); break;
                case 2: s = e4m3_f32<2>(sw[r >> 2]); break;
                default: s = e4m3_f32<3>(sw[r >> 2]); break;
            }
            // Columns interleaved innermost: N independent dot2 chains.
            float part[N];
#pragma unroll
            for (int n = 0; n < N; ++n) part[n] = dot2(p[0], as_bf16x2(x[n][0]), 0.0f);
#pragma unroll
            for (int i = 1; i < 8; ++i)
#pragma unroll
                for (int n = 0; n < N; ++n) part[n] = dot2(p[i], as_bf16x2(x[n][i]), part[n]);
#pragma unroll
            for (int n = 0; n < N; ++n) f.acc[r][n] = __builtin_fmaf(s, part[n], f.acc[r][n]);
        }
    }
}

// ------------------------------------------------------- lane reduction

__device__ __forceinline__ void permlane32_swap(float &a, float &b) {
    // a <- {a[0..31], b[0..31]},  b <- {a[32..63], b[32..63]}
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void permlane16_swap(float &a, float &b) {
    // a <- {a.row0, b.row0, a.row2, b.row2},  b <- {a.row1, b.row1, a.row3, b.row3}
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

constexpr int kDppRowRor8 = 0x128;      // lane l reads lane (l + 8) mod 16 of its row: l ^ 8
constexpr int kDppHalfMirror = 0x141;   // lane l reads lane 7 - (l mod 8) of its half-row
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]

// Sum acc over the 64 lanes with a fixed tree.  Three exchange-and-halve
// rounds (lane bit 5 by v_permlane32_swap, bit 4 by v_permlane16_swap, bit 3
// by a DPP row rotate) and one more against the mirrored half-row leave each
// lane one row; two DPP quad rounds finish the sum.  Afterwards every lane l
// holds, for each column, the total of row l >> 2.  The tree is the same for
// every column and every launch.
template <int N>
__device__ __forceinline__ void wave_reduce(Frag<N> &f, int lane) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            permlane32_swap(f.acc[i][n], f.acc[i + 8][n]);
            f.acc[i][n] = f.acc[i][n] + f.acc[i + 8][n];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            permlane16_swap(f.acc[i][n], f.acc[i + 4][n]);
            f.acc[i][n] = f.acc[i][n] + f.acc[i + 4][n];
        }
    }
    const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
#pragma unroll
    for (int n = 0; n < N; ++n) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float lo = f.acc[i][n], hi = f.acc[i + 2][n];
            const float keep = b3 ? hi : lo, send = b3 ? lo : hi;
            f.acc[i][n] = keep + dpp<kDppRowRor8>(send);
        }
        {
            const float lo = f.acc[0][n], hi = f.acc[1][n];
            const float keep = b2 ? hi : lo, send = b2 ? lo : hi;
            f.acc[0][n] = keep + dpp<kDppHalfMirror>(send);
        }
        f.acc[0][n] = f.acc[0][n] + dpp<kDppQuadXor1>(f.acc[0][n]);
        f.acc[0][n] = f.acc[0][n] + dpp<kDppQuadXor2>(f.acc[0][n]);
    }
}

__device__ __forceinline__ int reduced_row(int lane) { return lane >> 2; }

// One step's operands for one lane: 8 code entries, the scale entry, and the
// activation pairs of its block for every column.
template <int N>
struct StepData {
    uint4 c[kRowPairs];
    uint4 sc;
    uint32_t x[N][8];
};

template <int N>
__device__ __forceinline__ void load_step(StepData<N> &d, const uint4 *__restrict__ wq,
                                          const uint4 *__restrict__ ws, const uint16_t *__restrict__ X,
                                          int64_t x_stride, int t, int j, int steps, int kb, int lane) {
    const int64_t entry = int64_t(t) * steps + j;
    // Entry (t, j, g, q, i) of block 8g + i: lanes 8g..8g+7 read 128
    // contiguous bytes per row pair.
    const uint4 *cp = wq + entry * (kRowPairs * kLanes) + (lane >> 3) * 64 + (lane & 7);
#pragma unroll
    for (int q = 0; q < kRowPairs; ++q) d.c[q] = load_stream(cp + q * 8);
    d.sc = load_stream(ws + entry * kLanes + lane);
    const int b = j * kLanes + lane;
    if (b < kb) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(X + n * x_stride + int64_t(b) * kBlock);
            const uint4 a = xp[0], bb = xp[1];
            d.x[n][0] = a.x; d.x[n][1] = a.y; d.x[n][2] = a.z; d.x[n][3] = a.w;
            d.x[n][4] = bb.x; d.x[n][5] = bb.y; d.x[n][6] = bb.z; d.x[n][7] = bb.w;
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n)
#pragma unroll
            for (int i = 0; i < 8; ++i) d.x[n][i] = 0u;
    }
}

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
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
#pragma unroll
        for (int n = 0; n < N; ++n) f.acc[r][n] = 0.0f;

    if constexpr (N <= kPrefetchMaxN) {
        // Software pipeline over two register buffers: the next step's loads
        // are in flight while this step's operands are decoded and multiplied.
        StepData<N> a, b;
        int j = j0;
        if (j < j1) load_step<N>(a, wq, ws, X, x_stride, t, j, steps, kb, lane);
        while (j < j1) {
            if (j + 1 < j1) load_step<N>(b, wq, ws, X, x_stride, t, j + 1, steps, kb, lane);
            mac_step<N>(f, a.c, a.sc, a.x);
            if (++j >= j1) break;
            if (j + 1 < j1) load_step<N>(a, wq, ws, X, x_stride, t, j + 1, steps, kb, lane);
            mac_step<N>(f, b.c, b.sc, b.x);
            ++j;
        }
    } else {
        // Wider column counts keep one step of operands in registers.
        for (int j = j0; j < j1; ++j) {
            StepData<N> cur;
            load_step<N>(cur, wq, ws, X, x_stride, t, j, steps, kb, lane);
            mac_step<N>(f, cur.c, cur.sc, cur.x);
        }
    }

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

__global__ void __launch_bounds__(256) swiglu_kernel(const float *__restrict__ gu, int64_t F, int64_t total,
                                                     uint16_t *__restrict__ h) {
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t n = i / F, c = i % F;
    const float g = gu[n * 2 * F + c];
    const float u = gu[n * 2 * F + F + c];
    const float v = g * u / (1.0f + expf(-g));
    const uint32_t b = __float_as_uint(v);
    h[i] = uint16_t((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);   // nearest-even (finite v)
}

// ------------------------------------------------------------------ dispatch

// Waves per tile: enough (tile, part) waves to give every CU several, never
// more parts than steps.  Depends only on the matrix shape.
inline int choose_ksplit(const Geometry &g) {
    const int64_t target_waves = 2048;
    int64_t k = ceil_div(target_waves, g.tiles);
    if (k > g.steps) k = g.steps;
    if (k > kMaxKsplit) k = kMaxKsplit;
    if (k < 1) k = 1;
    return int(k);
}

template <bool ARGMAX>
int launch_valu(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, unsigned long long *amax_ws, int32_t *argmax_out, hipStream_t stream) {
    const int ksplit = choose_ksplit(g);
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

NVFP4_API int nvfp4_swiglu(const float *gu, int64_t F, int n, uint16_t *h, hipStream_t stream) {
    if (!gu || !h || n < 1 || n > NVFP4_MAX_N) return NVFP4_EINVAL;
    if (F < 1 || F > (int64_t(1) << 40)) return NVFP4_ESHAPE;
    if (!aligned(gu, 16) || !aligned(h, 4)) return NVFP4_EALIGN;
    const int64_t total = F * n;
    (void)hipGetLastError();
    hipLaunchKernelGGL(swiglu_kernel, dim3(unsigned(ceil_div(total, 256))), dim3(256), 0, stream, gu, F, total, h);
    return launch_status();
}
