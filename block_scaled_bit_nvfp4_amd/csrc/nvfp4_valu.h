// nvfp4_valu.h -- the VALU matvec building blocks shared by the plain,
// argmax and fused-MLP kernels of libnvfp4.  Internal to the library.
//
// Per step, lane l of a wave owns block 64j + l of all 16 rows of a tile:
// 8 code loads of 16 bytes (one per row pair; each wave load is 8 full
// 128-byte lines), one 16-byte scale load, and 32 bytes of each activation
// column, all 128-bit and coalesced across the wave.  The 16 rows reuse the
// activation registers.  Decode is one v_cvt_scalef32_pk_bf16_fp4 per 2 codes
// and one E4M3 conversion per row-block, shared by all columns; each column
// then takes 8 v_dot2_f32_bf16 per row-block (products exact in fp32) and one
// fp32 FMA by the block scale.  The lane reduction has a fixed shape.
#pragma once

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

// f += this lane's share of tile t over steps [j0, j1).
template <int N>
__device__ __forceinline__ void accumulate_steps(Frag<N> &f, const uint4 *__restrict__ wq,
                                                 const uint4 *__restrict__ ws, const uint16_t *__restrict__ X,
                                                 int64_t x_stride, int t, int j0, int j1, int steps, int kb,
                                                 int lane) {
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

}

template <int N>
__device__ __forceinline__ void clear(Frag<N> &f) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r)
#pragma unroll
        for (int n = 0; n < N; ++n) f.acc[r][n] = 0.0f;
}

// Waves per tile: enough (tile, part) waves to give every CU several, never
// more parts than steps.  Depends only on the matrix shape.
inline int choose_ksplit(int64_t tiles, int64_t steps) {
    const int64_t target_waves = 2048;
    int64_t k = ceil_div(target_waves, tiles);
    if (k > steps) k = steps;
    if (k > kMaxKsplit) k = kMaxKsplit;
    if (k < 1) k = 1;
    return int(k);
}

}  // namespace nvfp4
