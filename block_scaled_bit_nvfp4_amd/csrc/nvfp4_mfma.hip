// nvfp4_mfma.hip -- the prefill-width product (more than 8 activation
// columns) as a dequant-to-bf16 MFMA contraction on gfx950.
//
// Pages: qwentin README (gitlite mirror), "How it works" and "Highlights":
// wide prefill turns the projections into one wide block-scaled GEMM that
// reads each weight once for N tokens; bw24 wiki, feature list: prefill runs a
// tensor-core GEMM beside the decode matvec.  Their kernels use NVIDIA
// block-scaled MMA instructions; gfx950's scaled MFMA takes power-of-two
// scales, which cannot hold an E4M3 x fp32 scale exactly, so the weights are
// decoded to bf16 values e2m1 * e4m3 (exact: at most 6 significant bits) and
// multiplied on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the tensor
// scale multiplies the result.
//
// Tiling.  A wave owns 64 weight rows x 64 activation columns (64 fp32
// accumulators per lane) over the whole K; a workgroup's four waves share one
// 64-column tile of X, staged through LDS in 128-deep k chunks (double
// buffered), and take four different 64-row units.  Weights never touch LDS:
// every lane loads whole 16-byte code entries of the repacked layout (two rows
// x one 16-element block) and decodes them in registers; a chunk is one group
// of 8 blocks, 1 KiB contiguous per tile.  The contraction is free to permute
// k and the output rows, so each 16-byte entry feeds four MFMA operands
// directly: MFMA (h, e) takes row 2q + h of the entry's row pair and elements
// 8e..8e+7 of its block, and lane group s of the wave (lanes 16s .. 16s + 15)
// takes blocks s and s + 4 of the group.  The activation operand is read from
// LDS with the same k mapping.  A lane's outputs come out as 8 consecutive
// rows of one column.
#include "nvfp4_host.h"

namespace nvfp4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmWaves = 4;         // waves per workgroup
constexpr int kGemmUnitTiles = 4;     // 16-row tiles per wave: 64 weight rows
constexpr int kGemmCols = 64;         // activation columns per workgroup
constexpr int kGemmColSub = kGemmCols / 16;
constexpr int kChunkBlocks = 8;       // a chunk is one group of 8 blocks
constexpr int kChunkK = kChunkBlocks * kBlock;
constexpr int kLdsRowBytes = kChunkK * 2 + 16;   // padded: 16-byte reads of
                                                 // neighbouring columns spread
                                                 // over the banks
constexpr int kBPasses = kGemmCols * (kChunkK / 8) / (kGemmWaves * kLanes);   // 16-byte X loads per thread
constexpr int kChunksPerIter = 2;     // chunks multiplied per iteration, and prefetched ahead

// Decode one 32-bit word of codes (8 elements of one row) with scale s into
// the bf16x8 MFMA operand.  e2m1 * s is exact in fp32 and in bf16.
__device__ __forceinline__ bf16x8_t decode_a(uint32_t word, float s) {
    bf16x8_t out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo, hi;
        switch (i) {
            case 0: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); lo = v[0]; hi = v[1]; break; }
            case 1: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); lo = v[0]; hi = v[1]; break; }
            case 2: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); lo = v[0]; hi = v[1]; break; }
            default: { auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); lo = v[0]; hi = v[1]; break; }
        }
        out[2 * i] = (__bf16)(lo * s);
        out[2 * i + 1] = (__bf16)(hi * s);
    }
    return out;
}

// One chunk of this lane's weights: [tile pair tp][half f] entries for
// blocks 4f + s of the group, and their two scale bytes (rows 2q, 2q + 1).
struct AFrag {
    uint4 code[2][2];
    uint32_t scale[2][2];
};

__global__ void __launch_bounds__(kGemmWaves * kLanes, 2)
gemm_mfma_kernel(const uint4 *__restrict__ wq, const uint8_t *__restrict__ ws, float tscale, int rows,
                 int tiles, int steps, int chunks, int K, const uint16_t *__restrict__ X, int n,
                 float *__restrict__ Y, int row_groups, int vec_store) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[kChunksPerIter][kGemmCols * kLdsRowBytes];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rg = blockIdx.x % row_groups;          // 4 row units per workgroup
    const int ct = blockIdx.x / row_groups;          // column tile
    const int unit = rg * kGemmWaves + wave;         // this wave's 64-row unit
    const int n0 = ct * kGemmCols;
    const int rho = lane & 15, sig = lane >> 4;
    const int q = rho & 7;

    // This lane's entry tiles: tile pair tp covers tiles unit*4 + 2tp, +1.
    int tl[2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) tl[tp] = unit * kGemmUnitTiles + 2 * tp + (rho >> 3);

    floatx4_t acc[2][2][kGemmColSub];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < kGemmColSub; ++c) acc[tp][h][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto load_a = [&](AFrag &a, int c) {
        const int j = c >> 3, grp = c & 7;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int i = 4 * f + sig;
                if (tl[tp] < tiles) {
                    const int64_t entry = int64_t(tl[tp]) * steps + j;
                    a.code[tp][f] = wq[entry * (kRowPairs * kLanes) + grp * 64 + q * 8 + i];
                    a.scale[tp][f] = *reinterpret_cast<const uint16_t *>(
                        ws + (entry * kLanes + grp * 8 + i) * 16 + 2 * q);
                } else {
                    a.code[tp][f] = make_uint4(0u, 0u, 0u, 0u);
                    a.scale[tp][f] = 0u;
                }
            }
        }
    };
    // X for chunk c (128 k) of this workgroup's columns: 16 bytes per thread
    // and pass.
    auto load_b = [&](uint4 *bst, int c) {
#pragma unroll
        for (int p = 0; p < kBPasses; ++p) {
            const int idx = threadIdx.x + p * kGemmWaves * kLanes;
            const int col = idx / (kChunkK / 8), part = idx % (kChunkK / 8);
            const int k = c * kChunkK + part * 8;
            bst[p] = make_uint4(0u, 0u, 0u, 0u);
            if (n0 + col < n && k < K)
                bst[p] = *reinterpret_cast<const uint4 *>(X + int64_t(n0 + col) * K + k);
        }
    };
    auto store_b = [&](const uint4 *bst, int buf) {
#pragma unroll
        for (int p = 0; p < kBPasses; ++p) {
            const int idx = threadIdx.x + p * kGemmWaves * kLanes;
            const int col = idx / (kChunkK / 8), part = idx % (kChunkK / 8);
            *reinterpret_cast<uint4 *>(&lds_b[buf][col * kLdsRowBytes + part * 16]) = bst[p];
        }
    };
    auto compute = [&](const AFrag &a, int buf) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            // Decode: operand (tp, h, e) from dword 2h + e of entry (tp, f).
            bf16x8_t afr[2][2][2];
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                const uint4 cw = a.code[tp][f];
                const uint32_t d[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float s = e4m3_f32_dyn(a.scale[tp][f], h);
#pragma unroll
                    for (int e = 0; e < 2; ++e) afr[tp][h][e] = decode_a(d[2 * h + e], s);
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
#pragma unroll
                for (int cs = 0; cs < kGemmColSub; ++cs) {
                    const int kk = f * 64 + sig * 16 + e * 8;     // element offset in the chunk
                    const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t *>(
                        &lds_b[buf][(cs * 16 + rho) * kLdsRowBytes + kk * 2]);
#pragma unroll
                    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            acc[tp][h][cs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[tp][h][e], bfr,
                                                                                     acc[tp][h][cs], 0, 0, 0);
                }
            }
        }
    };

    // An iteration multiplies kChunksPerIter chunks (one LDS buffer each)
    // while the next iteration's weights and activations are in flight in
    // registers.  `chunks` is a multiple of kChunksPerIter (trailing all-zero
    // chunks stay inside the padded planes and the activation guard), and the
    // last iteration re-requests its own chunks instead of branching, so the
    // loop body is straight-line.
    AFrag a_cur[kChunksPerIter], a_nxt[kChunksPerIter];
    uint4 b_nxt[kChunksPerIter * kBPasses];
#pragma unroll
    for (int i = 0; i < kChunksPerIter; ++i) {
        load_a(a_cur[i], i);
        load_b(b_nxt + i * kBPasses, i);
    }
#pragma unroll
    for (int i = 0; i < kChunksPerIter; ++i) store_b(b_nxt + i * kBPasses, i);
    __syncthreads();
    for (int c = 0; c < chunks; c += kChunksPerIter) {
        const int cn = c + kChunksPerIter < chunks ? c + kChunksPerIter : c;
#pragma unroll
        for (int i = 0; i < kChunksPerIter; ++i) {
            load_a(a_nxt[i], cn + i);
            load_b(b_nxt + i * kBPasses, cn + i);
        }
#pragma unroll
        for (int i = 0; i < kChunksPerIter; ++i) compute(a_cur[i], i);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kChunksPerIter; ++i) {
            store_b(b_nxt + i * kBPasses, i);
            a_cur[i] = a_nxt[i];
        }
        __syncthreads();
    }

    // Lane group s holds output slots 4s..4s+3 of every MFMA tile; slot p of
    // operand h is row 2 (p mod 8) + h of tile 2tp + (p >= 8), so the lane
    // holds rows 8 (s & 1) .. 8 (s & 1) + 7 of tile unit*4 + 2tp + (s >> 1).
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
        const int tile = unit * kGemmUnitTiles + 2 * tp + (sig >> 1);
        const int row0 = tile * kTileRows + (sig & 1) * 8;
#pragma unroll
        for (int cs = 0; cs < kGemmColSub; ++cs) {
            const int col = n0 + cs * 16 + rho;
            if (col >= n || row0 >= rows) continue;
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = acc[tp][0][cs][i] * tscale;
                v[2 * i + 1] = acc[tp][1][cs][i] * tscale;
            }
            float *dst = Y + int64_t(col) * rows + row0;
            if (vec_store && row0 + 8 <= rows) {
                reinterpret_cast<float4 *>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
                reinterpret_cast<float4 *>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (row0 + i < rows) dst[i] = v[i];
            }
        }
    }
}

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream) {
    const int64_t units = ceil_div(g.tiles, kGemmUnitTiles);
    const int64_t row_groups = ceil_div(units, kGemmWaves);
    const int64_t col_tiles = ceil_div(n, kGemmCols);
    // Chunks of one 8-block group, rounded up to whole iterations; the
    // planes' 64-block steps always cover them.
    const int64_t chunks = kChunksPerIter * ceil_div(g.kb, kChunkBlocks * kChunksPerIter);
    hipLaunchKernelGGL(gemm_mfma_kernel, dim3(unsigned(row_groups * col_tiles)), dim3(kGemmWaves * kLanes), 0,
                       stream, reinterpret_cast<const uint4 *>(wq), ws, tscale, int(g.rows), int(g.tiles),
                       int(g.steps), int(chunks), int(g.cols), X, n, Y, int(row_groups),
                       int(aligned(Y, 16) && g.rows % 4 == 0));
    return launch_status();
}

}  // namespace nvfp4
