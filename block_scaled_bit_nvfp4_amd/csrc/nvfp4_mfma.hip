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
// Tiling.  One wave per SIMD (the whole register file: accumulators in
// AGPRs, operand pipelines in VGPRs).  A wave owns one 64-row super-tile x
// 128 activation columns over the whole K; a workgroup's four waves share
// one 128-column tile of X, staged in LDS one octet (128 k) at a time through
// a ring of three buffers: direct-to-LDS buffer loads two octets ahead of
// the MFMAs, XOR-swizzled by 16-byte chunk so that the B-operand reads of 16
// neighbouring columns hit distinct banks.  Weights never touch LDS: per
// octet a lane loads its 16-byte code entry of each tile and one 8-byte scale
// entry (spread to the other lane groups with v_permlane swaps), two octets
// ahead, and decodes in registers: word d of a tile's entry is directly the A
// operand of k = 128o + 32d .. +31 (lane 16g + r: row r, elements
// 8g .. 8g + 7).  A decoded A operand feeds eight MFMAs (the column
// subtiles); the next slice's A operands are decoded, and each B operand is
// re-read for the next slice, between the current slice's MFMAs.
//
// Balance.  When the super-tiles do not split evenly over the CUs (17408
// rows = 272 super-tiles against 256 CUs at N = 512), the row groups are cut
// back to a whole number of CU rounds and each workgroup also takes one of
// the remaining tiles, its four waves one 32-column quarter each: every wave
// then carries exactly the same work (4 x 128 + 32 tile-columns at N = 512).
// Each output's accumulation is the same MFMA chain whichever wave computes
// it, so the decomposition does not change any result bit.
//
// Workgroup order.  The column tiles of one row group are consecutive
// workgroups of one XCD (workgroup b runs on XCD b mod 8), so a row group's
// weights are fetched from HBM into that XCD's L2 once and re-read there by
// the other column tiles.
#include <type_traits>

#include "nvfp4_host.h"

namespace nvfp4 {

constexpr int kWideWaves = 4;                   // waves (super-tiles) per workgroup
constexpr int kWideCols = 128;                  // activation columns per workgroup
constexpr int kWideSub = kWideCols / 16;        // column subtiles of an MFMA
constexpr int kExtraSub = kWideSub / kWideWaves;   // column subtiles of a wave's extra tile
constexpr int kXColBytes = kOctet * kBlock * 2; // one column's octet: 128 bf16
constexpr int kXBuf = kWideCols * kXColBytes;   // one octet of the X tile: 32 KiB
constexpr int kXRing = 2;                       // octets of X in LDS
constexpr int kXDmaPerWave = kXBuf / (kWideWaves * kLanes * 16);   // 16-byte lanes
// A wave's weights of one octet in LDS: the super-tile's four code chunks,
// the extra tile's code chunk, the super-tile's scale entry as two dword
// planes and the extra tile's 128 scale bytes.
constexpr int kWCode = 0, kWXCode = 4096, kWScaleLo = 5120, kWScaleHi = 5376, kWXScale = 5632;
constexpr int kWStage = 6144;
constexpr int kWRing = 3;                       // octets of weights in LDS
constexpr int kWideLds = kXRing * kXBuf + kWRing * kWideWaves * kWStage;   // 136 KiB
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

// LDS byte offset of 16-byte chunk j (k = 8j .. 8j + 7 of the octet) of
// column c of an X tile buffer.
__device__ __forceinline__ uint32_t xtile_offset(int c, int j) {
    return uint32_t(c * kXColBytes + ((j ^ (c & 15)) << 4));
}


// Host-chosen decomposition (a function of rows, cols, n and the CU count).
struct WideConfig {
    int col_groups;   // 128-column tiles of X
    int row_groups;   // workgroups per column tile, four super-tiles each
    int extra;        // workgroups (per column tile) that also take one remaining tile
    int64_t groups;   // launched workgroups (whole XCD rounds; the excess leaves at once)
};

__global__ void __launch_bounds__(kWideWaves * kLanes, 1)
wide_kernel(const uint8_t *__restrict__ wq, const uint8_t *__restrict__ ws, float tscale, int rows, int supertiles,
            int octets, int K, const uint16_t *__restrict__ X, int n, float *__restrict__ Y, int row_groups,
            int col_groups, int extra, int vec_store) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // X ring, then the weight rings
    asm volatile("" ::: "a0");   // lets the accumulators live in AGPRs

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

    // This wave's super-tile; one past the last reads zeros and stores nothing.
    const int unit = rg * kWideWaves + wave;
    const bool has_unit = unit < supertiles;
    const int64_t ubase = int64_t(has_unit ? unit : 0) * octets;
    const auto crs = make_rsrc(wq + ubase * kCodeRegion, has_unit ? uint32_t(octets) * kCodeRegion : 0u);
    const auto srs = make_rsrc(ws + ubase * kScaleRegion, has_unit ? uint32_t(octets) * kScaleRegion : 0u);
    // The extra tile of this workgroup (the same for its four waves, each
    // taking column subtiles 2 wave, 2 wave + 1 of it).
    const int xtile = row_groups * kWideWaves * kSuperTiles + rg;
    const bool has_extra = rg < extra && xtile < supertiles * kSuperTiles;
    const int64_t xbase = has_extra ? int64_t(xtile >> 2) * octets : 0;
    const auto xcrs = make_rsrc(wq + xbase * kCodeRegion + (xtile & 3) * kCodeChunk,
                                has_extra ? uint32_t(octets) * kCodeRegion : 0u);
    const auto xsrs = make_rsrc(ws + xbase * kScaleRegion + (xtile & 3) * kScaleChunk,
                                has_extra ? uint32_t(octets) * kScaleRegion : 0u);
    // This workgroup's columns of X; columns past n read zeros.
    const int ncols = n - n0 < kWideCols ? n - n0 : kWideCols;
    const auto xrs = make_rsrc(X + int64_t(n0) * K, uint32_t(ncols) * uint32_t(K) * 2u);

    // Direct-to-LDS staging: LDS chunk p = (wave * kXDmaPerWave + i) * 64 +
    // lane of a buffer holds column p >> 4, k-chunk (p & 15) ^ (column & 15).
    auto stage_x = [&](int o) {
        uint8_t *dst = xs + (o % kXRing) * kXBuf + wave * kXDmaPerWave * 1024;
#pragma unroll
        for (int i = 0; i < kXDmaPerWave; ++i) {
            const int p = (wave * kXDmaPerWave + i) * kLanes + lane;
            const int c = p >> 4, j = (p & 15) ^ (c & 15);
            const uint32_t off = (o * 128 + 8 * j < K) ? uint32_t(c * K + o * 128 + 8 * j) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void *)(dst + i * 1024),
                                                     16, off, 0, 0, 0);
        }
    };
    // Weights of octet o into this wave's ring stage o % 3 (direct-to-LDS).
    uint8_t *const wring = xs + kXRing * kXBuf + wave * kWRing * kWStage;
    auto lds_ptr = [](uint8_t *p) { return (__attribute__((address_space(3))) void *)p; };
    auto load_w = [&](int o) {
        uint8_t *dst = wring + (o % kWRing) * kWStage;
        const uint32_t co = uint32_t(o) * kCodeRegion + uint32_t(lane) * 16u;
#pragma unroll
        for (int tt = 0; tt < kSuperTiles; ++tt)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, lds_ptr(dst + kWCode + tt * kCodeChunk), 16, co + tt * kCodeChunk,
                                                     0, 0, kStream);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xcrs, lds_ptr(dst + kWXCode), 16, co, 0, 0, kStream);
        const uint32_t so = uint32_t(o) * kScaleRegion + uint32_t(lane) * 8u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds_ptr(dst + kWScaleLo), 4, so, 0, 0, kStream);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds_ptr(dst + kWScaleHi), 4, so + 4, 0, 0, kStream);
        const uint32_t xso = lane < 32 ? uint32_t(o) * kScaleRegion + uint32_t(lane) * 4u : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrs, lds_ptr(dst + kWXScale), 4, xso, 0, 0, kStream);
    };
    constexpr int kWLoads = kSuperTiles + 4;   // vector-memory operations of load_w

    floatx4 acc[kSuperTiles][kWideSub], xacc[kExtraSub];
#pragma unroll
    for (int tt = 0; tt < kSuperTiles; ++tt)
#pragma unroll
        for (int cs = 0; cs < kWideSub; ++cs) acc[tt][cs] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < kExtraSub; ++e) xacc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

    // B-operand chunk offsets of this lane for each 32-k slice d.
    uint32_t boff[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) boff[d] = xtile_offset(c16, 4 * d + g);

    // The extra tile's B operands: this wave's quarter, column subtiles
    // 2 wave and 2 wave + 1.
    const uint32_t xboff = uint32_t(kExtraSub * wave * 16 * kXColBytes);

    auto compute = [&](int o, auto extra_c) {
        constexpr bool EXTRA = decltype(extra_c)::value;   // wave-uniform, fixed per workgroup
        const uint8_t *wst = wring + (o % kWRing) * kWStage;
        u32x4 code[kSuperTiles], xcode = {};
#pragma unroll
        for (int tt = 0; tt < kSuperTiles; ++tt)
            code[tt] = *reinterpret_cast<const u32x4 *>(wst + kWCode + tt * kCodeChunk + lane * 16);
        const uint32_t scl = *reinterpret_cast<const uint32_t *>(wst + kWScaleLo + lane * 4);
        const uint32_t sch = *reinterpret_cast<const uint32_t *>(wst + kWScaleHi + lane * 4);
        uint32_t xs0 = 0, xs1 = 0;
        if (EXTRA) {
            xcode = *reinterpret_cast<const u32x4 *>(wst + kWXCode + lane * 16);
            xs0 = *reinterpret_cast<const uint32_t *>(wst + kWXScale + c16 * 8);
            xs1 = *reinterpret_cast<const uint32_t *>(wst + kWXScale + c16 * 8 + 4);
        }
        uint32_t s0[4], s1[4];   // scale words (blocks 0..3, 4..7) of row r of each tile
        gather_lane_groups(scl, s0);
        gather_lane_groups(sch, s1);
        const uint8_t *xb = xs + (o % kXRing) * kXBuf;
        auto scale_of = [&](uint32_t w0, uint32_t w1, int d) {
            const int sh = 8 * ((2 * d + (g >> 1)) & 3);   // this lane's block of pair d
            return e4m3_f32<0>((d < 2 ? w0 : w1) >> sh);
        };
        auto decode = [&](int d, int tt) { return decode_scaled(code[tt][d], scale_of(s0[tt], s1[tt], d)); };
        auto xdecode = [&](int d) { return decode_scaled(xcode[d], scale_of(xs0, xs1, d)); };
        auto read_b = [&](int d, int cs) {
            return *reinterpret_cast<const bf16x8 *>(xb + cs * 16 * kXColBytes + boff[d]);
        };
        auto read_xb = [&](int d, int e) {
            return *reinterpret_cast<const bf16x8 *>(xb + xboff + e * 16 * kXColBytes + boff[d]);
        };
        // Software pipeline over the four 32-k slices: slice d + 1's A
        // operands are decoded between slice d's MFMAs (one tile per two
        // column subtiles), and each B operand is re-read for slice d + 1 as
        // soon as slice d's MFMAs have issued with it.  No branch inside, so
        // the scheduler can interleave the decode with the MFMAs.
        // a[d & 1]: slice d's A operands; slice d + 1's go to the other half,
        // so no register copies between slices.
        bf16x8 a[2][kSuperTiles], xa[2] = {}, bv[kWideSub], xbv[kExtraSub];
#pragma unroll
        for (int cs = 0; cs < kWideSub; ++cs) bv[cs] = read_b(0, cs);
#pragma unroll
        for (int tt = 0; tt < kSuperTiles; ++tt) a[0][tt] = decode(0, tt);
        if (EXTRA) {
            xa[0] = xdecode(0);
#pragma unroll
            for (int e = 0; e < kExtraSub; ++e) xbv[e] = read_xb(0, e);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int cur = d & 1, nxt = cur ^ 1;
#pragma unroll
            for (int cs = 0; cs < kWideSub; ++cs) {
#pragma unroll
                for (int tt = 0; tt < kSuperTiles; ++tt)
                    acc[tt][cs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cur][tt], bv[cs], acc[tt][cs], 0, 0, 0);
                if (d < 3) bv[cs] = read_b(d + 1, cs);
                if (d < 3 && (cs & 1)) a[nxt][cs >> 1] = decode(d + 1, cs >> 1);
            }
            if (EXTRA) {
#pragma unroll
                for (int e = 0; e < kExtraSub; ++e) {
                    xacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[cur], xbv[e], xacc[e], 0, 0, 0);
                    if (d < 3) xbv[e] = read_xb(d + 1, e);
                }
                if (d < 3) xa[nxt] = xdecode(d + 1);
            }
        }
    };

    // Octet o is multiplied from X buffer o % 2 and weight stage o % 3.  At
    // octet o a wave issues octet o + 1's X loads, then octet o + 2's weight
    // loads, so at the start of octet o + 1 only the latter may still be
    // outstanding: the wait below finishes this wave's loads of the octet
    // about to be used, and the barrier publishes every wave's share of the
    // X tile and frees the buffers restaged next (read at octet o - 1).  A
    // bare barrier: __syncthreads() would also drain every outstanding load
    // (its fence), emptying the rings; the memory clobber keeps the LDS reads
    // below it.
    auto run = [&](auto extra_c) {
        load_w(0);
        stage_x(0);
        if (octets > 1) load_w(1);
        for (int o = 0; o < octets; ++o) {
            if (o + 1 < octets) __builtin_amdgcn_s_waitcnt(vmcnt_only(kWLoads));
            else __builtin_amdgcn_s_waitcnt(0);
            asm volatile("s_barrier" ::: "memory");
            if (o + 1 < octets) stage_x(o + 1);
            if (o + 2 < octets) load_w(o + 2);
            compute(o, extra_c);
        }
    };
    if (has_extra) run(std::true_type{});
    else run(std::false_type{});

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
        for (int tt = 0; tt < kSuperTiles; ++tt)
#pragma unroll
            for (int cs = 0; cs < kWideSub; ++cs)
                store(acc[tt][cs], unit * kSuperRows + tt * kTileRows + 4 * g, n0 + cs * 16 + c16);
    }
    if (has_extra) {
#pragma unroll
        for (int e = 0; e < kExtraSub; ++e)
            store(xacc[e], xtile * kTileRows + 4 * g, n0 + (kExtraSub * wave + e) * 16 + c16);
    }
}

// The decomposition: workgroups of four super-tiles per 128-column tile.
// When those workgroups would overshoot a whole number of CU rounds by at
// most one tile per workgroup, the row groups are cut back to the whole
// rounds and the remaining tiles become the workgroups' extra tiles.
inline WideConfig wide_config(const Geometry &g, int n, int cus) {
    WideConfig c;
    c.col_groups = int(ceil_div(n, kWideCols));
    c.row_groups = int(ceil_div(g.supertiles, kWideWaves));
    c.extra = 0;
    if (cus > 0 && cus % c.col_groups == 0) {
        const int64_t per_round = cus / c.col_groups;                  // row groups per CU round
        const int64_t rounds = (g.supertiles / kWideWaves) / per_round;
        if (rounds >= 1) {
            const int64_t rg = rounds * per_round;
            const int64_t left_tiles = (g.supertiles - rg * kWideWaves) * kSuperTiles;
            if (left_tiles > 0 && left_tiles <= rg) {
                c.row_groups = int(rg);
                c.extra = int(left_tiles);
            }
        }
    }
    c.groups = int64_t(kXcds) * c.col_groups * ceil_div(c.row_groups, kXcds);
    return c;
}

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream) {
    if (g.cols > kMaxWideCols || int64_t(g.scale_bytes()) > kMaxWideScaleBytes) return NVFP4_ESHAPE;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    const WideConfig c = wide_config(g, n, cus);
    if (c.groups > (int64_t(1) << 31) - 1) return NVFP4_ESHAPE;
    // The rings (136 KiB) are above the default dynamic-LDS limit.
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(wide_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kWideLds) != hipSuccess)
        return NVFP4_EHIP;
    hipLaunchKernelGGL(wide_kernel, dim3(unsigned(c.groups)), dim3(kWideWaves * kLanes), kWideLds, stream, wq,
                       ws, tscale, int(g.rows), int(g.supertiles), int(g.octets), int(g.cols), X, n, Y, c.row_groups,
                       c.col_groups, c.extra, int(aligned(Y, 16) && g.rows % 4 == 0));
    return launch_status();
}

}  // namespace nvfp4
