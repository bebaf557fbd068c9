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
// scale multiplies the result.  The same body, instantiated for MXFP4, reads
// one E8M0 byte per 32 elements and decodes e2m1 * 2^(b - 127) in the scaled
// conversion itself (exact for every finite byte).
//
// Tiling (the product shape; WideShape below gives the narrower shapes that
// serve 9..128 columns).  Two waves per SIMD, so that one wave's weight
// decode (VALU) runs while the other's MFMAs execute.  A workgroup of eight
// waves owns four 64-row super-tiles x 128 activation columns; wave w takes two tiles
// (32 rows) of super-tile w / 2 over all 128 columns (64 fp32 accumulators
// per lane, in AGPRs).  The workgroup's X tile (128 columns) is staged in
// LDS one octet (128 k) at a time through a ring of two buffers by
// direct-to-LDS buffer loads, XOR-swizzled by 16-byte chunk so that the
// B-operand reads of 16 neighbouring columns hit distinct banks; the weights
// go the same way into a ring of three stages, two octets ahead of the
// MFMAs, their loads spread over the slices of an octet.  Word d of a
// lane's 16-byte code entry of a tile is directly the A operand of
// k = 128o + 32d .. +31 (lane 16g + r: row r, elements
// 8g .. 8g + 7), decoded to exact bf16 in registers with its E4M3 scale.  A
// decoded A operand feeds eight MFMAs (the column subtiles); the next slice's
// A operands are decoded, and each B operand is re-read for the next slice,
// between the current slice's MFMAs.
//
// Balance.  When the super-tiles do not split evenly over the CUs (17408
// rows = 272 super-tiles against 256 CUs at N = 512), the row groups are cut
// back to a whole number of CU rounds and each workgroup also takes one of
// the remaining tiles, its eight waves one 16-column subtile each: every wave
// then carries the same MFMA work (2 x 128 + 16 tile-columns at N = 512).
// The extra tile's A operands are decoded once per workgroup: waves 0..3
// each decode one 32-k slice of the next octet (from their own copy of its
// raw bytes) into a two-octet LDS ring that every wave reads.  Each output's
// accumulation is the same MFMA chain whichever wave computes it, so the
// decomposition does not change any result bit.
//
// Workgroup order.  The column tiles of one row group are consecutive
// workgroups of one XCD (workgroup b runs on XCD b mod 8), so a row group's
// weights are fetched from HBM into that XCD's L2 once and re-read there by
// the other column tiles.
#include <mutex>
#include <type_traits>

#include "nvfp4_host.h"

namespace nvfp4 {

constexpr int kWideWaves = 8;                   // waves per workgroup
constexpr int kXColBytes = kOctet * kBlock * 2; // one column's octet: 128 bf16
constexpr int kXRing = 2;                       // octets of X in LDS
constexpr int kXDecoders = 4;                   // waves decoding the extra tile, one slice each
constexpr int kWXWave = kCodeChunk + 256;       // a decoder's raw extra tile: code, then 128 scale bytes
constexpr int kWRing = 3;                       // octets of weights in LDS
// The extra tile's decoded A operands of one octet: 4 slices x 64 lanes x
// 16 bytes, in a ring of two octets.
constexpr int kXABuf = 4 * kLanes * 16;
constexpr int kXARing = 2;

// The shape of a workgroup: eight waves, each taking WT tiles of the
// workgroup's SUP super-tiles over its CS 16-column subtiles of X.  The
// product shape (two tiles per wave, four super-tiles, 128 columns) is the
// one described above, with its extra tiles.  The narrower shapes (one tile
// per wave, two super-tiles: twice the workgroups for the same rows) take
// 128, 64 or 32 columns for products of 9 to 128 columns, where the product
// shape's workgroups would leave CUs idle and its 128-column tile would
// spend LDS reads and MFMAs on columns past n.  One weight decode feeds CS
// MFMAs in every shape; each output is the same MFMA chain over the same k
// order in every shape, so the shape changes no result bit.
template <int WT, int SUP, int CS>
struct WideShape {
    static constexpr int kWaveTiles = WT;
    static constexpr int kSupers = SUP;
    static constexpr int kSub = CS;                        // column subtiles per wave
    static constexpr int kCols = 16 * CS;                  // activation columns per workgroup
    static constexpr int kXBuf = kCols * kXColBytes;       // one octet of the X tile
    static constexpr int kXDmaPerWave = kXBuf / (kWideWaves * kLanes * 16);   // 16-byte lanes
    static constexpr bool kExtra = WT == 2 && SUP == 4 && CS == 8;             // the extra-tile balancing
    // One octet of the workgroup's weights in LDS: per wave its code chunks
    // and its tiles' scale bytes as two dword planes; then, with the extra
    // tile, for each of the waves that decode it (one 32-k slice each), its
    // own copy of the extra tile's code chunk and scale bytes.
    static constexpr int kWWave = WT * kCodeChunk + 2 * 256;
    static constexpr int kWXCode = kWideWaves * kWWave;
    static constexpr int kWStage = kWXCode + (kExtra ? kXDecoders * kWXWave : 0);
    static constexpr int kLds = kXRing * kXBuf + kWRing * kWStage + (kExtra ? kXARing * kXABuf : 0);
    static_assert(SUP * kSuperTiles / WT == kWideWaves, "eight waves per workgroup");
    static_assert(kXDmaPerWave >= 1 && kXDmaPerWave * kWideWaves * kLanes * 16 == kXBuf, "whole X staging rounds");
    static_assert(CS % WT == 0, "a wave's decodes fall between its column subtiles");
};
using ShapeProduct = WideShape<2, 4, 8>;   // wide products; 148 KiB of LDS
using ShapeMid128 = WideShape<1, 2, 8>;
using ShapeMid64 = WideShape<1, 2, 4>;
using ShapeMid32 = WideShape<1, 2, 2>;
enum WideShapeId { kShapeProduct = 0, kShapeMid128 = 1, kShapeMid64 = 2, kShapeMid32 = 3 };
constexpr int kXcds = 8;
// Longest rows of the wide product: a column tile of X and a super-tile's
// code stream stay below 2^31 bytes of buffer offset.
constexpr int64_t kMaxWideCols = int64_t(1) << 22;
// Largest scale plane of the wide product (addressed with 32-bit offsets).
constexpr int64_t kMaxWideScaleBytes = int64_t(1) << 31;

// Decode one 32-bit word of codes (8 elements of one row) with scale s into
// the bf16x8 MFMA operand.  e2m1 * s is exact in fp32 and in bf16.
__device__ __forceinline__ bf16x8 decode_scaled(uint32_t word, float s) {
    bf16x8 out;
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

// s_waitcnt immediate that waits until at most v vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left alone).
constexpr int vmcnt_only(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// The same, and every LDS operation of this wave done.
constexpr int vmcnt_lds(int v) { return (v & 0xF) | ((v >> 4) << 14) | (0x7 << 4); }

// LDS byte offset of 16-byte chunk j (k = 8j .. 8j + 7 of the octet) of
// column c of an X tile buffer.
__device__ __forceinline__ uint32_t xtile_offset(int c, int j) {
    return uint32_t(c * kXColBytes + ((j ^ (c & 15)) << 4));
}


// Host-chosen decomposition (a function of rows, cols, n and the CU count).
struct WideConfig {
    int shape;        // WideShapeId
    int col_groups;   // column tiles of X
    int row_groups;   // workgroups per column tile
    int extra;        // workgroups (per column tile) that also take one remaining tile (product shape)
    int64_t groups;   // launched workgroups (whole XCD rounds; the excess leaves at once)
};

// FMT kMxfp4: the scale plane holds a row's four E8M0 bytes per octet, and
// word d of a code entry (32-element block d of the octet) is decoded by the
// scaled conversion alone (the power of two goes into its scale operand).
template <int FMT, class S>
__device__ __forceinline__ void
wide_body(const uint8_t *__restrict__ wq, const uint8_t *__restrict__ ws, float tscale, int rows, int supertiles,
          int octets, int K, const uint16_t *__restrict__ X, int n, float *__restrict__ Y, int row_groups,
          int col_groups, int extra, int vec_store) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // X ring, then the weight ring
    asm volatile("" ::: "a0");   // lets the accumulators live in AGPRs
    constexpr int kWaveTiles = S::kWaveTiles, kWideSupers = S::kSupers, kWideCols = S::kCols, kWideSub = S::kSub;
    constexpr int kXBuf = S::kXBuf, kXDmaPerWave = S::kXDmaPerWave;
    constexpr int kWWave = S::kWWave, kWXCode = S::kWXCode, kWStage = S::kWStage;

    // Workgroup -> (row group, column tile): the column tiles of a row group
    // are consecutive workgroups of one XCD.
    const int b = blockIdx.x;
    const int q = b / kXcds;
    const int cg = q % col_groups;
    const int rg = (q / col_groups) * kXcds + b % kXcds;
    if (rg >= row_groups) return;   // the whole workgroup leaves before any barrier

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n0 = cg * kWideCols;
    const int c16 = lane & 15, g = lane >> 4;

    // This wave's tiles: kWaveTiles half .. kWaveTiles (half + 1) - 1 of
    // super-tile unit; a super-tile past the last reads zeros and stores
    // nothing.
    constexpr int kWavesPerSuper = kSuperTiles / kWaveTiles;
    const int unit = rg * kWideSupers + wave / kWavesPerSuper;
    const int half = wave % kWavesPerSuper;
    const bool has_unit = unit < supertiles;
    constexpr int SREGION = FMT == kMxfp4 ? kMxScaleRegion : kScaleRegion;
    constexpr int SCHUNK = FMT == kMxfp4 ? kMxScaleChunk : kScaleChunk;
    const int64_t ubase = int64_t(has_unit ? unit : 0) * octets;
    const auto crs = make_rsrc(wq + ubase * kCodeRegion + half * kWaveTiles * kCodeChunk,
                               has_unit ? uint32_t(octets) * kCodeRegion : 0u);
    const auto srs = make_rsrc(ws + ubase * SREGION + half * kWaveTiles * SCHUNK,
                               has_unit ? uint32_t(octets) * SREGION : 0u);
    // The extra tile of this workgroup (each wave takes column subtile wave).
    const int xtile = row_groups * kWideSupers * kSuperTiles + rg;
    const bool has_extra = S::kExtra && rg < extra && xtile < supertiles * kSuperTiles;
    const int64_t xbase = has_extra ? int64_t(xtile >> 2) * octets : 0;
    const auto xcrs = make_rsrc(wq + xbase * kCodeRegion + (xtile & 3) * kCodeChunk,
                                has_extra ? uint32_t(octets) * kCodeRegion : 0u);
    const auto xsrs = make_rsrc(ws + xbase * SREGION + (xtile & 3) * SCHUNK,
                                has_extra ? uint32_t(octets) * SREGION : 0u);
    // This workgroup's columns of X; columns past n read zeros.
    const int ncols = n - n0 < kWideCols ? n - n0 : kWideCols;
    const auto xrs = make_rsrc(X + int64_t(n0) * K, uint32_t(ncols) * uint32_t(K) * 2u);
    auto lds_ptr = [](uint8_t *p) { return (__attribute__((address_space(3))) void *)p; };

    // Direct-to-LDS staging: LDS chunk p = (wave * kXDmaPerWave + i) * 64 +
    // lane of a buffer holds column p >> 4, k-chunk (p & 15) ^ (column & 15).
    auto stage_x = [&](int o) {
        uint8_t *dst = xs + (o % kXRing) * kXBuf + wave * kXDmaPerWave * 1024;
#pragma unroll
        for (int i = 0; i < kXDmaPerWave; ++i) {
            const int p = (wave * kXDmaPerWave + i) * kLanes + lane;
            const int c = p >> 4, j = (p & 15) ^ (c & 15);
            const uint32_t off = (o * 128 + 8 * j < K) ? uint32_t(c * K + o * 128 + 8 * j) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, lds_ptr(dst + i * 1024), 16, off, 0, 0, 0);
        }
    };
    // Weights of octet o into ring stage o % 3: this wave's two code chunks
    // (lane l's 16 bytes of tile j at 1024 j + 16 l), its tiles' scale bytes
    // (NVFP4: 256 as low and high dwords of lanes 0 .. 31, lane 16 j + r
    // holding row r of tile j; MXFP4: 128 as one dword of those lanes), and
    // for a decoder wave its own copy of the extra tile's code chunk and
    // scale bytes.  Every load has its own source and destination, so the
    // compiler cannot merge two of them: the waits below count them.
    uint8_t *const wring = xs + kXRing * kXBuf;
    uint8_t *const xaring = wring + kWRing * kWStage;
    // Part 0: the code chunks; part 1: the own scale bytes; part 2: the
    // extra tile's bytes (decoder waves only).
    auto load_w_part = [&](int o, int part) {
        uint8_t *dst = wring + (o % kWRing) * kWStage;
        uint8_t *mine = dst + wave * kWWave;
        const uint32_t co = uint32_t(o) * kCodeRegion + uint32_t(lane) * 16u;
        if (part == 0) {
#pragma unroll
            for (int j = 0; j < kWaveTiles; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, lds_ptr(mine + j * kCodeChunk), 16, co + j * kCodeChunk,
                                                         0, 0, kStream);
        } else if (part == 1) {
        if constexpr (FMT == kMxfp4) {
            const uint32_t so = lane < 16 * kWaveTiles ? uint32_t(o) * SREGION + uint32_t(lane) * 4u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds_ptr(mine + kWaveTiles * kCodeChunk), 4, so, 0, 0, kStream);
        } else {
            const uint32_t so = lane < 16 * kWaveTiles ? uint32_t(o) * SREGION + uint32_t(lane) * 8u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds_ptr(mine + kWaveTiles * kCodeChunk), 4, so, 0, 0, kStream);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds_ptr(mine + kWaveTiles * kCodeChunk + 256), 4,
                                                     so == kOutOfRange ? so : so + 4, 0, 0, kStream);
        }
        } else if (S::kExtra && wave < kXDecoders) {
            uint8_t *xw = dst + kWXCode + wave * kWXWave;
            // the extra tile's 16 rows of scale bytes: 8 per row (NVFP4) or 4 (MXFP4)
            const int xlanes = FMT == kMxfp4 ? 16 : 32;
            const uint32_t xso = lane < xlanes ? uint32_t(o) * SREGION + uint32_t(lane) * 4u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xcrs, lds_ptr(xw), 16, co, 0, 0, kStream);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrs, lds_ptr(xw + kCodeChunk), 4, xso, 0, 0, kStream);
        }
    };
    auto load_w = [&](int o) {
        load_w_part(o, 0);
        load_w_part(o, 1);
        load_w_part(o, 2);
    };
    // Vector-memory operations of load_w: a decoder wave issues the extra
    // tile's two loads on top of its own.  (A wave's loads complete in
    // issue order; the waits below leave exactly the newest load_w
    // outstanding, so everything issued before it has landed in LDS.)
    constexpr int kWLoadsOwn = kWaveTiles + (FMT == kMxfp4 ? 1 : 2);
    constexpr int kWLoadsDec = kWLoadsOwn + (S::kExtra ? 2 : 0);
    const bool xdecoder = S::kExtra && wave < kXDecoders;   // issues the extra tile's loads (zeros when there is none)
    // A decoder wave turns slice d = wave of the extra tile's octet o into
    // exact bf16 A operands for every lane, from its own copy of the raw
    // bytes, into the extra ring (published by the next barrier).
    auto decode_extra = [&](int o) {
        const uint8_t *xw = wring + (o % kWRing) * kWStage + kWXCode + wave * kWXWave;
        const int d = wave;
        const uint32_t word = *reinterpret_cast<const uint32_t *>(xw + lane * 16 + d * 4);
        bf16x8 v;
        if constexpr (FMT == kMxfp4) {
            const uint32_t sw = *reinterpret_cast<const uint32_t *>(xw + kCodeChunk + c16 * 4);
            v = e2m1x8_bf16_e8m0(word, sw >> (8 * d));
        } else {
            const uint32_t sw = *reinterpret_cast<const uint32_t *>(xw + kCodeChunk + c16 * 8 + (d < 2 ? 0 : 4));
            v = decode_scaled(word, e4m3_f32<0>(sw >> (8 * ((2 * d + (g >> 1)) & 3))));
        }
        *reinterpret_cast<bf16x8 *>(xaring + (o % kXARing) * kXABuf + d * kLanes * 16 + lane * 16) = v;
    };

    floatx4 acc[kWaveTiles][kWideSub], xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < kWaveTiles; ++tt)
#pragma unroll
        for (int cs = 0; cs < kWideSub; ++cs) acc[tt][cs] = floatx4{0.f, 0.f, 0.f, 0.f};

    // B-operand chunk offsets of this lane for each 32-k slice d; the extra
    // tile's column subtile is this wave's.
    uint32_t boff[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) boff[d] = xtile_offset(c16, 4 * d + g);
    const uint32_t xboff = uint32_t(wave * 16 * kXColBytes);

    // wo >= 0: the weight loads of octet wo are issued in three parts at the
    // starts of slices 1, 2 and 3, after this octet's X loads and spread
    // between the MFMAs instead of in one burst after the barrier.
    auto compute = [&](int o, auto extra_c, int wo) {
        constexpr bool EXTRA = decltype(extra_c)::value;   // wave-uniform, fixed per workgroup
        const uint8_t *wst = wring + (o % kWRing) * kWStage;
        const uint8_t *mine = wst + wave * kWWave;
        u32x4 code[kWaveTiles];
#pragma unroll
        for (int tt = 0; tt < kWaveTiles; ++tt)
            code[tt] = *reinterpret_cast<const u32x4 *>(mine + tt * kCodeChunk + lane * 16);
        const uint32_t scl = *reinterpret_cast<const uint32_t *>(mine + kWaveTiles * kCodeChunk + lane * 4);
        uint32_t s0[4], s1[4] = {0u, 0u, 0u, 0u};   // scale words (blocks 0..3, 4..7) of row r of each tile
        gather_lane_groups(scl, s0);
        if constexpr (FMT != kMxfp4) {
            const uint32_t sch = *reinterpret_cast<const uint32_t *>(mine + kWaveTiles * kCodeChunk + 256 + lane * 4);
            gather_lane_groups(sch, s1);
        }
        const uint8_t *xb = xs + (o % kXRing) * kXBuf;
        const uint8_t *xab = xaring + (o % kXARing) * kXABuf + lane * 16;
        auto scale_of = [&](uint32_t w0, uint32_t w1, int d) {
            const int sh = 8 * ((2 * d + (g >> 1)) & 3);   // this lane's block of pair d
            return e4m3_f32<0>((d < 2 ? w0 : w1) >> sh);
        };
        auto decode = [&](int d, int tt) {
            if constexpr (FMT == kMxfp4) return e2m1x8_bf16_e8m0(code[tt][d], s0[tt] >> (8 * d));
            else return decode_scaled(code[tt][d], scale_of(s0[tt], s1[tt], d));
        };
        auto read_b = [&](int d, int cs) {
            return *reinterpret_cast<const bf16x8 *>(xb + cs * 16 * kXColBytes + boff[d]);
        };
        auto read_xb = [&](int d) { return *reinterpret_cast<const bf16x8 *>(xb + xboff + boff[d]); };
        auto read_xa = [&](int d) { return *reinterpret_cast<const bf16x8 *>(xab + d * kLanes * 16); };
        // Software pipeline over the four 32-k slices: a[d & 1] holds slice
        // d's A operands, slice d + 1's are decoded into the other half
        // between slice d's MFMAs, and each B operand is re-read for slice
        // d + 1 as soon as slice d's MFMAs have issued with it.  No branch
        // inside, so the scheduler can interleave decode and MFMAs.
        bf16x8 a[2][kWaveTiles], xa[2] = {}, bv[kWideSub], xbv = {};
#pragma unroll
        for (int cs = 0; cs < kWideSub; ++cs) bv[cs] = read_b(0, cs);
#pragma unroll
        for (int tt = 0; tt < kWaveTiles; ++tt) a[0][tt] = decode(0, tt);
        if (EXTRA) {
            xa[0] = read_xa(0);
            xbv = read_xb(0);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int cur = d & 1, nxt = cur ^ 1;
            // A decoder wave decodes its slice of the next octet's extra
            // tile here, between its own MFMAs, once that octet's weight
            // loads (issued an octet earlier, ahead of the X loads and the
            // first part of octet wo's) have landed.
            if (d == 2 && EXTRA && xdecoder && o + 1 < octets) {
                if (wo >= 0) __builtin_amdgcn_s_waitcnt(vmcnt_only(kXDmaPerWave + kWaveTiles));
                else __builtin_amdgcn_s_waitcnt(vmcnt_only(kXDmaPerWave));
                asm volatile("" ::: "memory");   // the raw bytes' LDS reads stay below the wait
                decode_extra(o + 1);
            }
            if (d >= 1 && wo >= 0) load_w_part(wo, d - 1);
            // Waves w and w + 4 share a SIMD, and at equal priority the older
            // (w) wins the issue arbitration and ends its octet early, leaving
            // w + 4 to finish alone.  w + 4 takes the higher priority for the
            // first two slices, which brings the two to the barrier together.
            if (wave >= kWideWaves / 2) {
                if (d <= 1) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
#pragma unroll
            for (int cs = 0; cs < kWideSub; ++cs) {
#pragma unroll
                for (int tt = 0; tt < kWaveTiles; ++tt)
                    acc[tt][cs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cur][tt], bv[cs], acc[tt][cs], 0, 0, 0);
                if (d < 3) bv[cs] = read_b(d + 1, cs);
                constexpr int kPer = kWideSub / kWaveTiles;   // subtiles between a wave's decodes
                if (d < 3 && cs % kPer == kPer - 1) a[nxt][cs / kPer] = decode(d + 1, cs / kPer);
            }
            if (EXTRA) {
                xacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[cur], xbv, xacc, 0, 0, 0);
                if (d < 3) {
                    xbv = read_xb(d + 1);
                    xa[nxt] = read_xa(d + 1);
                }
            }
        }
    };

    // Octet o is multiplied from X buffer o % 2 and weight stage o % 3.  At
    // octet o a wave issues octet o + 1's X loads, then (spread over the
    // slices) octet o + 2's weight loads, so at the start of octet o + 1 only
    // the latter may still be outstanding: the wait below leaves exactly
    // those outstanding (the wave's own load_w count), which finishes the
    // loads of the octet about to be used and their LDS writes, and the
    // barrier publishes every wave's loads and decoded extra operands and
    // frees the buffers restaged next (read at octet o - 1).  A bare barrier:
    // __syncthreads() would also drain every outstanding load (its fence),
    // emptying the rings; the memory clobber keeps the LDS accesses on their
    // side of it.  A decoder wave decodes octet o + 1's extra slice in the
    // middle of octet o's MFMAs (see compute), where its SIMD-mate's MFMAs
    // hide it.  The compiler barriers between the load groups keep the X and
    // weight loads in program order, which the counts rely on.
    auto fence = [] { asm volatile("" ::: "memory"); };
    auto run = [&](auto extra_c) {
        constexpr bool EXTRA = decltype(extra_c)::value;
        const bool decoder = EXTRA && xdecoder;
        load_w(0);
        fence();
        stage_x(0);
        fence();
        if (octets > 1) load_w(1);
        fence();
        if (decoder) {
            if (octets > 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(kWLoadsDec));
            else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            fence();   // the raw bytes' LDS reads stay below the wait
            decode_extra(0);
        }
        for (int o = 0; o < octets; ++o) {
            if (o + 1 < octets) {
                if (xdecoder) __builtin_amdgcn_s_waitcnt(vmcnt_lds(kWLoadsDec));
                else __builtin_amdgcn_s_waitcnt(vmcnt_lds(kWLoadsOwn));
            } else {
                __builtin_amdgcn_s_waitcnt(0);
            }
            asm volatile("s_barrier" ::: "memory");
            if (o + 1 < octets) stage_x(o + 1);
            fence();
            compute(o, extra_c, o + 2 < octets ? o + 2 : -1);
        }
    };
    if constexpr (S::kExtra) {
        if (has_extra) run(std::true_type{});
        else run(std::false_type{});
    } else {
        run(std::false_type{});
    }

    // Lane (g, c16) holds rows 4g .. 4g + 3 of a tile for column
    // cs * 16 + c16 of the column tile.
    auto store = [&](const floatx4 &a, int row0, int col) {
        const floatx4 v = a * tscale;
        float *dst = Y + int64_t(col) * rows + row0;
        if (vec_store) {   // rows % 4 == 0: a lane's four rows are all in range or all out
            if (col < n && row0 < rows) *reinterpret_cast<floatx4 *>(dst) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (col < n && row0 + i < rows) dst[i] = v[i];
        }
    };
    if (has_unit) {
#pragma unroll
        for (int tt = 0; tt < kWaveTiles; ++tt)
#pragma unroll
            for (int cs = 0; cs < kWideSub; ++cs)
                store(acc[tt][cs], unit * kSuperRows + (half * kWaveTiles + tt) * kTileRows + 4 * g,
                      n0 + cs * 16 + c16);
    }
    if (has_extra) store(xacc, xtile * kTileRows + 4 * g, n0 + wave * 16 + c16);
}

// Super-tiles per workgroup and columns per workgroup of each shape.
constexpr int kShapeSupers[4] = {ShapeProduct::kSupers, ShapeMid128::kSupers, ShapeMid64::kSupers, ShapeMid32::kSupers};
constexpr int kShapeCols[4] = {ShapeProduct::kCols, ShapeMid128::kCols, ShapeMid64::kCols, ShapeMid32::kCols};

// The shape for n columns: up to 32 and 64 columns the 32- and 64-column
// shapes (faster than the product shape on every matrix measured: 34816 x
// 5120 at 48 columns 55 against 72 us, the 151936 x 5120 head 147 against
// 226 us); up to 128 the 128-column narrow shape while its workgroups (two
// super-tiles each, one per CU for their 100 KiB of LDS) fit one round of
// the CUs, else the product shape (34816 x 5120 at 128 columns: two rounds
// of the narrow shape 98.9 us, one of the product shape 79.5 us).
inline int wide_shape(const Geometry &g, int n, int cus) {
    if (n > 128) return kShapeProduct;
    if (n > 64) return ceil_div(g.supertiles, int64_t(kShapeSupers[kShapeMid128])) <= cus ? kShapeMid128 : kShapeProduct;
    return n > 32 ? kShapeMid64 : kShapeMid32;
}

// The decomposition: workgroups of the shape's super-tiles per column tile.
// For the product shape, when those workgroups would overshoot a whole
// number of CU rounds by at most one tile per workgroup, the row groups are
// cut back to the whole rounds and the remaining tiles become the
// workgroups' extra tiles.
inline WideConfig wide_config(const Geometry &g, int n, int cus) {
    WideConfig c;
    c.shape = wide_shape(g, n, cus);
    const int supers = kShapeSupers[c.shape];
    c.col_groups = int(ceil_div(n, kShapeCols[c.shape]));
    c.row_groups = int(ceil_div(g.supertiles, int64_t(supers)));
    c.extra = 0;
    if (c.shape == kShapeProduct && cus > 0 && cus % c.col_groups == 0) {
        const int64_t per_round = cus / c.col_groups;                  // row groups per CU round
        const int64_t rounds = (g.supertiles / supers) / per_round;
        if (rounds >= 1) {
            const int64_t rg = rounds * per_round;
            const int64_t left_tiles = (g.supertiles - rg * supers) * kSuperTiles;
            if (left_tiles > 0 && left_tiles <= rg) {
                c.row_groups = int(rg);
                c.extra = int(left_tiles);
            }
        }
    }
    c.groups = int64_t(kXcds) * c.col_groups * ceil_div(c.row_groups, kXcds);
    return c;
}

// The two formats' kernels, one per shape.
template <class S>
__global__ void __launch_bounds__(kWideWaves * kLanes, 2)
wide_kernel_nvfp4(const uint8_t *__restrict__ wq, const uint8_t *__restrict__ ws, float tscale, int rows,
                  int supertiles, int octets, int K, const uint16_t *__restrict__ X, int n, float *__restrict__ Y,
                  int row_groups, int col_groups, int extra, int vec_store) {
    wide_body<kNvfp4, S>(wq, ws, tscale, rows, supertiles, octets, K, X, n, Y, row_groups, col_groups, extra, vec_store);
}

template <class S>
__global__ void __launch_bounds__(kWideWaves * kLanes, 2)
wide_kernel_mxfp4(const uint8_t *__restrict__ wq, const uint8_t *__restrict__ ws, float tscale, int rows,
                  int supertiles, int octets, int K, const uint16_t *__restrict__ X, int n, float *__restrict__ Y,
                  int row_groups, int col_groups, int extra, int vec_store) {
    wide_body<kMxfp4, S>(wq, ws, tscale, rows, supertiles, octets, K, X, n, Y, row_groups, col_groups, extra, vec_store);
}

// Per-device facts the wide launch needs, taken once per device on its first
// wide call (with that device current): the CU count, which the
// decomposition follows, and the dynamic-LDS attribute of every wide kernel
// whose rings are above the default limit (the product shape's 148 KiB).
// Later calls only look up the current device's index.
constexpr int kMaxDevices = 64;
struct WideDevice {
    std::once_flag once;
    int cus = 0;
    bool lds_ok = false;
};
static WideDevice g_wide_devices[kMaxDevices];

template <class S>
static bool set_wide_lds() {
    if (S::kLds <= 65536) return true;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(wide_kernel_nvfp4<S>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, S::kLds) == hipSuccess &&
           hipFuncSetAttribute(reinterpret_cast<const void *>(wide_kernel_mxfp4<S>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, S::kLds) == hipSuccess;
}

static const WideDevice *wide_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    WideDevice &w = g_wide_devices[dev];
    std::call_once(w.once, [&w, dev] {
        if (hipDeviceGetAttribute(&w.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) w.cus = 0;
        w.lds_ok = set_wide_lds<ShapeProduct>() && set_wide_lds<ShapeMid128>() && set_wide_lds<ShapeMid64>() &&
                   set_wide_lds<ShapeMid32>();
    });
    return &w;
}

// Estimated duration in microseconds of the wide product at n columns on
// this device, or a negative value when it cannot take the shape (or the
// device cannot be queried).  A workgroup of each shape spends about this
// long per octet of its rows, measured on 17408 x 5120, 4096 x 4096 and
// 5120 x 17408 with one round of workgroups: 1.6 us (product shape), 1.2
// (128-column narrow shape), 0.85 (64 columns) and 0.75 (32 columns); a
// launch adds about 2 us.
double wide_estimate_us(const Geometry &g, int n, int fmt) {
    if (g.cols > kMaxWideCols || int64_t(g.scale_bytes(fmt)) > kMaxWideScaleBytes) return -1.0;
    const WideDevice *wd = wide_device();
    if (!wd || wd->cus <= 0) return -1.0;
    static constexpr double kUsPerOctet[4] = {1.6, 1.2, 0.85, 0.75};
    const WideConfig c = wide_config(g, n, wd->cus);
    const int64_t active = int64_t(c.row_groups) * c.col_groups;
    const int64_t rounds = ceil_div(active, int64_t(wd->cus));
    return double(rounds) * double(g.octets) * kUsPerOctet[c.shape] + 2.0;
}

template <class S>
static void launch_wide_shape(int fmt, const WideConfig &c, const Geometry &g, const uint8_t *wq, const uint8_t *ws,
                              float tscale, const uint16_t *X, int n, float *Y, int vec, hipStream_t stream) {
    if (fmt == kMxfp4)
        hipLaunchKernelGGL(wide_kernel_mxfp4<S>, dim3(unsigned(c.groups)), dim3(kWideWaves * kLanes), S::kLds,
                           stream, wq, ws, tscale, int(g.rows), int(g.supertiles), int(g.octets), int(g.cols), X, n,
                           Y, c.row_groups, c.col_groups, c.extra, vec);
    else
        hipLaunchKernelGGL(wide_kernel_nvfp4<S>, dim3(unsigned(c.groups)), dim3(kWideWaves * kLanes), S::kLds,
                           stream, wq, ws, tscale, int(g.rows), int(g.supertiles), int(g.octets), int(g.cols), X, n,
                           Y, c.row_groups, c.col_groups, c.extra, vec);
}

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream, int fmt) {
    if (g.cols > kMaxWideCols || int64_t(g.scale_bytes(fmt)) > kMaxWideScaleBytes) return NVFP4_ESHAPE;
    const WideDevice *wd = wide_device();
    if (!wd || !wd->lds_ok) return NVFP4_EHIP;
    const WideConfig c = wide_config(g, n, wd->cus);
    if (c.groups > (int64_t(1) << 31) - 1) return NVFP4_ESHAPE;
    const int vec = int(aligned(Y, 16) && g.rows % 4 == 0);
    switch (c.shape) {
        case kShapeMid128: launch_wide_shape<ShapeMid128>(fmt, c, g, wq, ws, tscale, X, n, Y, vec, stream); break;
        case kShapeMid64: launch_wide_shape<ShapeMid64>(fmt, c, g, wq, ws, tscale, X, n, Y, vec, stream); break;
        case kShapeMid32: launch_wide_shape<ShapeMid32>(fmt, c, g, wq, ws, tscale, X, n, Y, vec, stream); break;
        default: launch_wide_shape<ShapeProduct>(fmt, c, g, wq, ws, tscale, X, n, Y, vec, stream); break;
    }
    return launch_status();
}

}  // namespace nvfp4
