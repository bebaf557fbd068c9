// nvfp4_narrow.h -- the matrix-vector product for n <= 8 activation columns
// (decode and the batched speculative verify), shared by the plain, argmax
// and fused gate||up+SwiGLU kernels of libnvfp4.  Internal to the library.
//
// Each 16-element block's dot product runs on v_mfma_f32_16x16x32_bf16, the
// block scale and the running sum on the VALU:
//
//   B operand (32 k x 16 rows): lane l = 16g + r of a code entry holds 8 codes
//     of row r, elements 32p + 8g .. +7 of block pair p -- exactly one 32-bit
//     word of the repacked entry, decoded by four v_cvt_scalef32_pk_bf16_fp4
//     (exact).  Lane groups 0,1 carry the pair's even block, groups 2,3 its
//     odd block.
//   A operand (16 slots x 32 k): slot s holds activation column
//     c(s) = (s >> 2) + 4 ((s >> 1) & 1) restricted to block parity s & 1:
//     x values where the lane group's block has that parity, zeros elsewhere.
//   D (16 slots x 16 rows): lane (g, r) receives slots 4g .. 4g + 3 of row r,
//     i.e. the even- and odd-block partial sums of columns g and g + 4, each
//     the exact block dot product rounded by the MFMA's fp32 accumulation.
//   acc += e4m3(scale) * D, one fp32 FMA per block, in block order.
//
// Column c always sits in the same slots and lanes whatever n is, and the
// MFMA computes each output independently of the other slots, so column c of
// an n-column product equals the 1-column product bit for bit.  The work
// decomposition (tiles per workgroup, k split) depends only on the matrix
// shape, so results are also reproducible run to run.
//
// Memory: a workgroup owns `tww` tiles of one 64-row super-tile and splits the
// row's octets (8 blocks) over `ksplit` waves; each wave streams its octets
// with range-checked buffer loads, one octet ahead of the MFMAs: per tile one
// 16-byte code load (the tile's 1 KiB chunk), the scales of its rows, and one
// compact 16-byte activation load per four columns (for one column the
// activations and scales of four octets come in one load each, a group
// ahead).  Loads past the wave's last octet read zeros with no
// memory traffic, so the loop needs no branch around a load.
//
// A operands: the wave writes the octet's compact activations to its own LDS
// slot and reads each A operand back with one ds_read_b128 per 32-k slice:
// an active lane reads its column's 8 values, an inactive lane (slot of the
// other block parity, or a column >= n) reads a 256-byte run of zeros kept in
// the same wave-private region.  No workgroup barrier is involved: LDS
// operations of one wave complete in order.
#pragma once

#include <type_traits>

#include "nvfp4_host.h"

namespace nvfp4 {

constexpr int kMaxNarrowN = 8;
constexpr int kMaxKsplit = 16;
// Longest rows the narrow products take: a super-tile's code regions and the
// activations of 8 columns stay below 2^31 bytes of buffer offset.
constexpr int64_t kMaxNarrowCols = int64_t(1) << 26;

// Decomposition of a rows x cols product with n columns over workgroups.
// The waves per workgroup (the octet ranges, hence every row's summation
// order) are a function of the shape alone, so column c of an n-column
// product has the bits of the 1-column product; the tiles per workgroup also
// follow n.  Measured on the workload shapes (decode 4096 x 4096, the MLP's
// 34816 x 5120 and 5120 x 17408, the 17408 x 5120 verify matrix, the
// 151936 x 5120 vocabulary head and the 8192 x 4096 draft head, n = 1..8) and
// on 320..1024-tile sweeps at 4096 and 5120 columns: the narrow kernel keeps
// enough bytes in flight with eight waves of two tiles per workgroup, except
// that
//   - small matrices (<= 256 tiles) want one tile per workgroup and sixteen
//     waves, so that every CU gets a workgroup and each wave a short chain;
//     up to 512 tiles this still pays while each of the sixteen waves has at
//     most two octets (both loaded before the first is used);
//   - mid-size ones (512 < tiles <= 4096) run best with one tile and eight
//     waves, which also keeps the fused gate||up+SwiGLU workgroup (two sets of
//     waves) at two workgroups per CU.
// Other shapes between 256 and 512 tiles take two tiles per workgroup so that
// the workgroups (<= 256) stay one per CU instead of doubling up on some CUs.
// Past four columns a wave stages twice the activations per octet and runs
// twice the block products per tile; a workgroup of more tiles spreads that
// staging over more rows, so there the tiles per workgroup double (one to
// two, two to four) except for small matrices and the two-tile shapes
// between 256 and 512 tiles, where it leaves CUs idle: e.g. 8192 x 4096 at
// n = 8 takes 7.2 instead of 8.4 us, the vocabulary head 74 instead of 83 us.
// max_tww caps the tiles for kernels built only up to two (MXFP4).
struct NarrowConfig {
    int tww;      // tiles per workgroup: 1, 2 or 4
    int ksplit;   // waves per workgroup (octet ranges)
    int64_t groups;   // workgroups
};

inline NarrowConfig narrow_config(const Geometry &g, int n, int max_tww = 4) {
    NarrowConfig c;
    int k;
    const bool small = g.tiles <= 256, short_rows = g.tiles <= 512 && g.octets <= 2 * 16;
    if (small || short_rows) {
        c.tww = 1;
        k = 16;
    } else if (g.tiles <= 512 || g.tiles > 4096) {
        c.tww = 2;
        k = 8;
    } else {
        c.tww = 1;
        k = 8;
    }
    if (n > 4 && !small && (short_rows || g.tiles > 512)) c.tww *= 2;
    if (c.tww > max_tww) c.tww = max_tww;
    if (k > g.octets) k = int(g.octets);
    c.ksplit = k < 1 ? 1 : k;
    c.groups = g.supertiles * (kSuperTiles / c.tww);
    return c;
}

// The argmax products' decomposition: one key per workgroup and column goes
// to the finish launch, and at four columns a large matrix (more than 4096
// tiles) takes four tiles per workgroup, as it does past four columns: half
// the keys.  The 151936 x 5120 vocabulary head's call measured 75.3-76.0
// against 76.0-79.0 us (its product alone 1.6 us slower, the finish faster),
// the verify step with it 82.1-83.2 against 83.6-85.4 us; at one to three
// columns four tiles measured no better (one column: 72 against 70 us).
// Tiles per workgroup change no row's summation order, so the logits keep
// the bits of the plain product.
inline NarrowConfig argmax_config(const Geometry &g, int n) {
    NarrowConfig c = narrow_config(g, n);
    if (n == 4 && g.tiles > 4096 && c.tww < 4) {
        c.tww = 4;
        c.groups = g.supertiles;
    }
    return c;
}

// Octet range [o0, o1) of wave part p of ksplit over a row's octets.  The
// narrow products take at most kMaxNarrowCols columns (2^19 octets) and 16
// waves, so octets * (p + 1) < 2^23 and 32-bit unsigned division gives the
// exact quotients (a 64-bit one expands into a long emulated sequence ahead
// of the first load).
__device__ __forceinline__ int octet_bound(int octets, int p, int ksplit) {
    return int(uint32_t(octets) * uint32_t(p) / uint32_t(ksplit));
}
static_assert((kMaxNarrowCols / (kOctet * kBlock)) * kMaxKsplit < (int64_t(1) << 32), "octet bounds fit 32 bits");

// Bytes of LDS per wave of the narrow kernels: a 256-byte run of zeros, then
// one slot of compact activations (1 KiB per four columns).
constexpr int narrow_wave_lds_bytes(int n) { return 256 + (n > 4 ? 2 : 1) * 1024; }

// Dynamic LDS of a narrow workgroup: each wave's slot, then the partial sums
// of its tiles' rows for every column.  Kept within the default 64 KiB
// dynamic limit, so no launch needs a function attribute.
constexpr size_t narrow_lds_bytes(int waves, int n, int tww) {
    return size_t(waves) * (size_t(narrow_wave_lds_bytes(n)) + size_t(n) * tww * kTileRows * sizeof(float));
}
constexpr size_t kNarrowLdsLimit = 65536;

// Argmax key: order-preserving map of an fp32 value (with -0 folded into +0)
// in the high word, the complement of the row index in the low word, so the
// unsigned maximum picks the largest value and, among equals, the lowest row.
__device__ __forceinline__ unsigned long long argmax_key(float y, uint32_t row) {
    uint32_t b = __float_as_uint(y == 0.0f ? 0.0f : y);
    uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<unsigned long long>(k) << 32) | (0xFFFFFFFFu - row);
}

// NVFP4 scale entries of a workgroup's tiles come in one 8-byte load per
// lane when the tiles are two or four (lane 16 tt + r: row r of tile tt),
// spread to the lane groups with permlane swaps; otherwise one per tile.
template <int TWW, int FMT>
constexpr bool merged_scales() { return TWW == 4 || (TWW == 2 && FMT == kNvfp4); }
template <int TWW, int FMT>
constexpr int scale_loads() { return merged_scales<TWW, FMT>() ? 1 : TWW; }

// One octet of one wave's operands.  NVFP4 scale entries are 8 bytes per row
// (the octet's eight 16-element blocks), MXFP4 ones 4 bytes (its four
// 32-element blocks).
template <int FMT>
using ScaleWord = typename std::conditional<FMT == kMxfp4, uint32_t, u32x2>::type;

template <int NC, int TWW, int FMT = kNvfp4>
struct OctetData {
    u32x4 code[TWW];                            // lane's 16-byte code entry of each tile
    ScaleWord<FMT> scale[scale_loads<TWW, FMT>()];   // merged: lane 16tt + r holds tile tt row r; else row r of each tile
    u32x4 x[NC];                                // compact activations: lane 16c + 4p + q holds X[c][128o + 32p + 8q ..]
};

// acc[tt][h]: this wave's share (octets [o0, o1)) of rows 16 (tile) + r of
// tile tg * TWW + tt of super-tile st, for columns g + 4h (lane = 16g + r).
// `wl` is the wave's private LDS region of narrow_wave_lds_bytes(N) bytes.
// FMT kMxfp4: the scale plane holds the four E8M0 bytes of a row's octet; a
// 32-element slice p is one MX block, so both halves of its MFMA result take
// that block's scale.
template <int N, int TWW, int FMT = kNvfp4>
__device__ __forceinline__ void narrow_accumulate(const uint8_t *__restrict__ wq, const uint8_t *__restrict__ ws,
                                                  int64_t st, int tg, int o0, int o1, int octets, int kb,
                                                  const uint16_t *__restrict__ X, int K, int lane,
                                                  float (&acc)[TWW][N > 4 ? 2 : 1], uint8_t *wl) {
    constexpr int NC = N > 4 ? 2 : 1;
    constexpr int H = NC;
    const int g = lane >> 4, r = lane & 15;

    static_assert(FMT == kNvfp4 || TWW < 4, "MXFP4 products take one or two tiles per workgroup");
    constexpr int SREGION = FMT == kMxfp4 ? kMxScaleRegion : kScaleRegion;
    constexpr int SCHUNK = FMT == kMxfp4 ? kMxScaleChunk : kScaleChunk;
    constexpr int SROW = FMT == kMxfp4 ? 4 : 8;    // scale bytes per row and octet
    const auto crs = make_rsrc(wq + st * octets * int64_t(kCodeRegion), uint32_t(o1) * kCodeRegion);
    const auto srs = make_rsrc(ws + st * octets * int64_t(SREGION), uint32_t(o1) * SREGION);
    const auto xrs = make_rsrc(X, uint32_t(N) * uint32_t(K) * 2u);
    const uint32_t coff = uint32_t(lane * 16 + tg * TWW * kCodeChunk);
    const uint32_t soff = TWW == 4 ? uint32_t(lane * 8)
                          : merged_scales<TWW, FMT>() ? (lane < TWW * kTileRows ? uint32_t((tg * TWW * kTileRows + lane) * SROW)
                                                                               : kOutOfRange)
                                                      : uint32_t((tg * TWW * kTileRows + r) * SROW);

    // Compact activation load of this lane: column xc (+4), k = 128o + 32xp + 8xq.
    const int xc = lane >> 4, xp = (lane >> 2) & 3, xq = lane & 3;
    const int xblk = 2 * xp + (xq >> 1);   // its block within the octet
    uint32_t xvo[NC];
#pragma unroll
    for (int h = 0; h < NC; ++h) {
        const int c = xc + 4 * h;
        xvo[h] = c < N ? uint32_t((c * K + 32 * xp + 8 * xq) * 2) : kOutOfRange;
    }
    // LDS: [0, 256) zeros, then the slot: compact activations in lane order,
    // i.e. column c's 128 values of the octet at 256 (c & 3) + 1024 (c >> 2).
    reinterpret_cast<uint32_t *>(wl)[lane] = 0u;
    u32x4 *const xslot = reinterpret_cast<u32x4 *>(wl + 256);
    // A-operand role of this lane: slot r of k-group g, column cs.
    const int cs = (r >> 2) + 4 * ((r >> 1) & 1);
    const bool active = cs < N && (g >> 1) == (r & 1);
    const uint32_t aoff = active ? uint32_t(256 + (cs >> 2) * 1024 + (cs & 3) * 256 + 16 * g) : 0u;

    float part[TWW][H][2];
#pragma unroll
    for (int tt = 0; tt < TWW; ++tt)
#pragma unroll
        for (int h = 0; h < H; ++h) part[tt][h][0] = part[tt][h][1] = 0.0f;

    auto load = [&](OctetData<NC, TWW, FMT> &d, int o) {
        const uint32_t co = uint32_t(o) * kCodeRegion + coff, so = uint32_t(o) * SREGION + soff;
#pragma unroll
        for (int tt = 0; tt < TWW; ++tt)
            d.code[tt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, co + tt * kCodeChunk, 0, kStream));
#pragma unroll
        for (int tt = 0; tt < scale_loads<TWW, FMT>(); ++tt) {
            if constexpr (FMT == kMxfp4)
                d.scale[tt] = __builtin_amdgcn_raw_buffer_load_b32(srs, so + tt * SCHUNK, 0, kStream);
            else
                d.scale[tt] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, so + tt * SCHUNK, 0, kStream));
        }
#pragma unroll
        for (int h = 0; h < NC; ++h) {
            const uint32_t vo = (o * kOctet + xblk < kb) ? xvo[h] : kOutOfRange;   // ragged last octet
            d.x[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, uint32_t(o) * 256u, 0));
        }
    };

    auto compute = [&](const OctetData<NC, TWW, FMT> &d) {
#pragma unroll
        for (int h = 0; h < NC; ++h) xslot[h * kLanes + lane] = d.x[h];
        bf16x8 A[4];   // A operand of block pair p = 2-block slice 32p .. 32p + 31
#pragma unroll
        for (int p = 0; p < 4; ++p) A[p] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wl + aoff + 64 * p));
        uint32_t S[2][TWW];   // scale words (blocks 0..3, 4..7 of the octet) of each tile's row r
        if constexpr (FMT == kMxfp4) {
#pragma unroll
            for (int tt = 0; tt < TWW; ++tt) S[0][tt] = S[1][tt] = d.scale[tt];   // MX blocks 0..3
        } else if (merged_scales<TWW, FMT>()) {
            uint32_t t0[4], t1[4];
            gather_lane_groups(d.scale[0][0], t0);
            gather_lane_groups(d.scale[0][1], t1);
#pragma unroll
            for (int tt = 0; tt < TWW; ++tt) {
                S[0][tt] = t0[tt];
                S[1][tt] = t1[tt];
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TWW; ++tt) {
                S[0][tt] = d.scale[tt][0];
                S[1][tt] = d.scale[tt][1];
            }
        }
#pragma unroll
        for (int tt = 0; tt < TWW; ++tt) {
            // The tile's four MFMAs first, then the scale FMAs in block order:
            // no FMA waits on the MFMA issued just before it.
            floatx4 D[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
                D[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[p], e2m1x8_bf16(d.code[tt][p]),
                                                            floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float2 sc;
                if constexpr (FMT == kMxfp4) {
                    const float s = e8m0_f32(S[0][tt] >> (8 * p));   // MX block p holds both halves
                    sc = float2{s, s};
                } else {
                    sc = e4m3x2_f32(S[p >> 1][tt], p & 1);   // blocks 2p, 2p + 1
                }
                float &a0 = part[tt][0][p & 1];
                a0 = __builtin_fmaf(sc.x, D[p][0], a0);
                a0 = __builtin_fmaf(sc.y, D[p][1], a0);
                if (H == 2) {
                    float &a1 = part[tt][H - 1][p & 1];
                    a1 = __builtin_fmaf(sc.x, D[p][2], a1);
                    a1 = __builtin_fmaf(sc.y, D[p][3], a1);
                }
            }
        }
    };

    if constexpr (N == 1) {
        // One column: the activations and scales of four octets come in one
        // load each (per scale load 4 / TWW octets), a group ahead of use, so
        // an octet costs the wave its code loads alone.  Vector-memory
        // instructions, more than bytes, are what the small per-octet
        // activation and scale loads cost (the 5120 x 17408 down product 6 %
        // faster, 17408 x 5120 5 %, the 8192 x 4096 draft head 4 %; the same
        // bits as per-octet loads).  Lane 16j + 4p + q holds
        // X[128(ob + j) + 32p + 8q ..]; the group's 1 KiB goes to the slot,
        // where octet j's A operands are read at 256 j.  Scale load i: lane
        // 16 (TWW a + t) + r holds row r of tile t for octet ob + OPS i + a.
        constexpr int G = 4;             // octets per group
        constexpr int OPS = G / TWW;     // octets per scale load
        constexpr int SPG = TWW;         // scale loads per group
        static_assert(OPS * TWW == G, "a group's scale loads cover it");
        const uint32_t gxo = uint32_t((128 * xc + 32 * xp + 8 * xq) * 2);
        const int sa = lane / (kTileRows * TWW), stt = (lane >> 4) % TWW;
        const uint32_t gso = uint32_t(sa) * SREGION + uint32_t(((tg * TWW + stt) * kTileRows + r) * SROW);
        struct Group {
            u32x4 x;
            ScaleWord<FMT> s[SPG];
        };
        auto load_group = [&](Group &gd, int ob) {
            const uint32_t vo = ((ob + xc) * kOctet + xblk < kb) ? gxo : kOutOfRange;   // ragged last octet
            gd.x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, uint32_t(ob) * 256u, 0));
#pragma unroll
            for (int i = 0; i < SPG; ++i) {
                const uint32_t so = uint32_t(ob + OPS * i) * SREGION + gso;
                if constexpr (FMT == kMxfp4)
                    gd.s[i] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, kStream);
                else
                    gd.s[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, so, 0, kStream));
            }
        };
        auto load_codes = [&](u32x4 (&c)[TWW], int o) {
            const uint32_t co = uint32_t(o) * kCodeRegion + coff;
#pragma unroll
            for (int tt = 0; tt < TWW; ++tt)
                c[tt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, co + tt * kCodeChunk, 0, kStream));
        };
        // A scale load's words spread to every lane when its first octet comes
        // up: lo[k] (and hi for NVFP4's blocks 4..7) = the word of lane group k.
        uint32_t lo[4], hi[4];
        auto spread = [&](const Group &gd, int i) {
            if constexpr (FMT == kMxfp4) {
                gather_lane_groups(gd.s[i], lo);
            } else {
                gather_lane_groups(gd.s[i][0], lo);
                gather_lane_groups(gd.s[i][1], hi);
            }
        };
        auto compute_g = [&](const u32x4 (&c)[TWW], int j) {
            const uint32_t ao = active ? aoff + uint32_t(256 * j) : 0u;
            bf16x8 A[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) A[p] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(wl + ao + 64 * p));
#pragma unroll
            for (int tt = 0; tt < TWW; ++tt) {
                const int k = (j % OPS) * TWW + tt;
                const uint32_t s0 = lo[k], s1 = FMT == kMxfp4 ? lo[k] : hi[k];
                floatx4 D[4];
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    D[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[p], e2m1x8_bf16(c[tt][p]),
                                                                floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    float2 sc;
                    if constexpr (FMT == kMxfp4) {
                        const float sv = e8m0_f32(s0 >> (8 * p));
                        sc = float2{sv, sv};
                    } else {
                        sc = e4m3x2_f32(p >> 1 ? s1 : s0, p & 1);
                    }
                    float &a0 = part[tt][0][p & 1];
                    a0 = __builtin_fmaf(sc.x, D[p][0], a0);
                    a0 = __builtin_fmaf(sc.y, D[p][1], a0);
                }
            }
        };
        if (o0 < o1) {
            Group gd;
            u32x4 cb[2][TWW];
            load_group(gd, o0);
            load_codes(cb[0], o0);
            load_codes(cb[1], o0 + 1);
            int ob = o0;
            for (; ob + G <= o1; ob += G) {
#pragma unroll
                for (int j = 0; j < G; ++j) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (j == 0) xslot[lane] = gd.x;
                    if (j % OPS == 0) spread(gd, j / OPS);
                    __builtin_amdgcn_sched_barrier(0);
                    // the group's registers are free once its last scale
                    // load is spread: the next group's loads go out here
                    if (j == G - OPS) load_group(gd, ob + G);   // past o1 or the row end it reads zeros
                    __builtin_amdgcn_sched_barrier(0);
                    compute_g(cb[j & 1], j);
                    __builtin_amdgcn_sched_barrier(0);
                    load_codes(cb[j & 1], ob + j + 2);
                }
            }
            if (ob < o1) {   // one to three octets left, their data loaded
                xslot[lane] = gd.x;
#pragma unroll
                for (int j = 0; j < G - 1; ++j) {
                    if (ob + j < o1) {
                        if (j % OPS == 0) spread(gd, j / OPS);
                        compute_g(cb[j & 1], j);
                    }
                    if (j == 0 && ob + 2 < o1) load_codes(cb[0], ob + 2);
                }
            }
        }
    } else {
    // Two octets in flight: full iterations prefetch unconditionally (always
    // inside [o0, o1)); the tail covers the last one to three octets.
    OctetData<NC, TWW, FMT> buf[2];
    if (o0 < o1) {
        const int n = o1 - o0;
        load(buf[0], o0);
        const int full = (n - 1) / 2;   // iterations whose two prefetches stay in range
        int o = o0;
        for (int it = 0; it < full; ++it, o += 2) {
            load(buf[1], o + 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(buf[0]);
            __builtin_amdgcn_sched_barrier(0);
            load(buf[0], o + 2);
            __builtin_amdgcn_sched_barrier(0);
            compute(buf[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (o + 1 < o1) load(buf[1], o + 1);
        compute(buf[0]);
        if (o + 1 < o1) compute(buf[1]);
    }
    }
#pragma unroll
    for (int tt = 0; tt < TWW; ++tt)
#pragma unroll
        for (int h = 0; h < H; ++h) acc[tt][h] = part[tt][h][0] + part[tt][h][1];
}

}  // namespace nvfp4
