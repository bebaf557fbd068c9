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
// Tiling.  A wave owns one 64-row super-tile x 64 activation columns (64
// fp32 accumulators per lane) over the whole K; a workgroup's four waves
// share one 64-column tile of X, staged through LDS in octet chunks of 128 k
// (double buffered), and take four different super-tiles.  Weights never
// touch LDS: per octet a lane loads its 16-byte code entry of each of the
// four tiles and its one 8-byte scale entry (spread to the other lane groups
// with v_permlane swaps), and decodes in registers: word d of a tile's entry
// is directly the A operand of k = 128o + 32d .. +31 (lane 16g + r: row r,
// elements 8g .. 8g + 7).  A lane's outputs come out as 4 consecutive rows of
// one column per tile.
#include "nvfp4_host.h"

namespace nvfp4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmWaves = 4;         // waves per workgroup
constexpr int kGemmCols = 64;         // activation columns per workgroup
constexpr int kGemmColSub = kGemmCols / 16;
constexpr int kChunkK = kOctet * kBlock;   // a chunk is one octet: 128 k
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

// One chunk (octet) of this lane's weights: its code entry of each tile of
// the super-tile and its scale entry (tile lane >> 4, row lane & 15).
struct AFrag {
    uint4 code[kSuperTiles];
    uint2 scale;
};

__global__ void __launch_bounds__(kGemmWaves * kLanes, 2)
gemm_mfma_kernel(const uint4 *__restrict__ wq, const uint2 *__restrict__ ws, float tscale, int rows,
                 int supertiles, int octets, int chunks, int K, const uint16_t *__restrict__ X, int n,
                 float *__restrict__ Y, int row_groups, int vec_store) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[kChunksPerIter][kGemmCols * kLdsRowBytes];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rg = blockIdx.x % row_groups;          // 4 super-tiles per workgroup
    const int ct = blockIdx.x / row_groups;          // column tile
    const int unit = rg * kGemmWaves + wave;         // this wave's super-tile
    const int n0 = ct * kGemmCols;
    const int rho = lane & 15, sig = lane >> 4;

    floatx4_t acc[kSuperTiles][kGemmColSub];
#pragma unroll
    for (int tt = 0; tt < kSuperTiles; ++tt)
#pragma unroll
        for (int c = 0; c < kGemmColSub; ++c) acc[tt][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto load_a = [&](AFrag &a, int c) {
        if (unit < supertiles && c < octets) {
            const int64_t region = int64_t(unit) * octets + c;
#pragma unroll
            for (int tt = 0; tt < kSuperTiles; ++tt) a.code[tt] = wq[(region * kSuperTiles + tt) * kLanes + lane];
            a.scale = ws[region * kLanes + lane];
        } else {
#pragma unroll
            for (int tt = 0; tt < kSuperTiles; ++tt) a.code[tt] = make_uint4(0u, 0u, 0u, 0u);
            a.scale = make_uint2(0u, 0u);
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
        // Scale words of row rho of every tile: blocks 0..3 and 4..7 of the octet.
        uint32_t s0[4], s1[4];
        gather_lane_groups(a.scale.x, s0);
        gather_lane_groups(a.scale.y, s1);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int ib = 2 * d + (sig >> 1);   // this lane's block of pair d
            bf16x8_t afr[kSuperTiles];
#pragma unroll
            for (int tt = 0; tt < kSuperTiles; ++tt) {
                const uint32_t sw = d < 2 ? s0[tt] : s1[tt];
                const float s = e4m3_f32<0>(sw >> (8 * (ib & 3)));
                const uint4 cw = a.code[tt];
                afr[tt] = decode_a(d == 0 ? cw.x : d == 1 ? cw.y : d == 2 ? cw.z : cw.w, s);
            }
#pragma unroll
            for (int cs = 0; cs < kGemmColSub; ++cs) {
                const int kk = 32 * d + 8 * sig;     // element offset in the chunk
                const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t *>(
                    &lds_b[buf][(cs * 16 + rho) * kLdsRowBytes + kk * 2]);
#pragma unroll
                for (int tt = 0; tt < kSuperTiles; ++tt)
                    acc[tt][cs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[tt], bfr, acc[tt][cs], 0, 0, 0);
            }
        }
    };

    // An iteration multiplies kChunksPerIter chunks (one LDS buffer each)
    // while the next iteration's weights and activations are in flight in
    // registers.  `chunks` is a multiple of kChunksPerIter (chunks past the
    // last octet read as zeros), and the last iteration re-requests its own
    // chunks instead of branching, so the loop body is straight-line.
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

    // Lane group s holds rows 4s .. 4s + 3 of each tile for column rho of
    // every column subtile.
#pragma unroll
    for (int tt = 0; tt < kSuperTiles; ++tt) {
        const int row0 = unit * kSuperRows + tt * kTileRows + 4 * sig;
#pragma unroll
        for (int cs = 0; cs < kGemmColSub; ++cs) {
            const int col = n0 + cs * 16 + rho;
            if (col >= n || row0 >= rows) continue;
            float *dst = Y + int64_t(col) * rows + row0;
            const floatx4_t v = acc[tt][cs] * tscale;
            if (vec_store && row0 + 4 <= rows) {
                *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < rows) dst[i] = v[i];
            }
        }
    }
}

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream) {
    const int64_t row_groups = ceil_div(g.supertiles, kGemmWaves);
    const int64_t col_tiles = ceil_div(n, kGemmCols);
    // Octet chunks rounded up to whole iterations; chunks past the last octet
    // read as zeros.
    const int64_t chunks = kChunksPerIter * ceil_div(g.octets, kChunksPerIter);
    hipLaunchKernelGGL(gemm_mfma_kernel, dim3(unsigned(row_groups * col_tiles)), dim3(kGemmWaves * kLanes), 0,
                       stream, reinterpret_cast<const uint4 *>(wq), reinterpret_cast<const uint2 *>(ws), tscale,
                       int(g.rows), int(g.supertiles), int(g.octets), int(chunks), int(g.cols), X, n, Y,
                       int(row_groups), int(aligned(Y, 16) && g.rows % 4 == 0));
    return launch_status();
}

}  // namespace nvfp4
