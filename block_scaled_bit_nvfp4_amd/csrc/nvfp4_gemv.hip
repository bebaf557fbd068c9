// nvfp4_gemv.hip -- the NVFP4 x bf16 matrix-vector products for n <= 8
// activation columns (the block dot products on MFMA, scales and sums on the
// VALU; see nvfp4_narrow.h), the argmax epilogue of the vocabulary
// projection, and the SwiGLU step between MLP products; gfx950.
//
// Pages: bw24 wiki (GitHub), feature list -- the NVFP4 decode matvec over
// split-plane repacked weights, picked per matrix shape, and the batched K+1
// verify that reads each weight once for every column; bw24 wiki, exactness
// note after the gate list -- summation order is part of the contract;
// qwentin README (gitlite mirror), "How it works" -- dense-argmax descent over
// the draft tree and the persistent-MLP decode GEMV.
//
// Work decomposition.  A workgroup owns `tww` 16-row tiles and `ksplit` waves
// that take contiguous octet ranges of the rows (nvfp4_narrow.h); the waves'
// partial sums meet in LDS and are added in wave order.  Everything depends
// only on (rows, cols), never on n or on timing.
#include <mutex>

#include "nvfp4_narrow.h"

namespace nvfp4 {

enum NarrowMode { kPlain = 0, kArgmax = 1, kSwiglu = 2 };

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

// ------------------------------------------------- the argmax workspace

// One argmax product's workspace: a finish header, then the keys
// [workgroups][N] of the product.  The header holds the split finish's
// counter (a 128-byte line of its own) and its workgroups' partial maxima
// [kFinishGroups][N].  The product's first workgroup zeroes the counter, so
// the workspace takes any contents and no clearing between calls.
constexpr int kFinishGroups = 16;                  // workgroups of the split finish
constexpr int kFinishCounterWords = 16;            // 128 bytes
constexpr int64_t kFinishHeaderWords = kFinishCounterWords + kFinishGroups * kMaxNarrowN;

__device__ __forceinline__ unsigned *finish_counter(unsigned long long *keys) {
    return reinterpret_cast<unsigned *>(keys - kFinishHeaderWords);
}

// ------------------------------------------------------------ the products

// The epilogue of the narrow products.  LDS: each wave's slot
// (narrow_wave_lds_bytes), then the waves' partial sums
// red[(wave * N + c) * SEG + row of the workgroup], SEG = TWW * 16 rows.
template <int N, int TWW>
__device__ __forceinline__ void store_partials(float *red, int wave, int lane, const float (&acc)[TWW][N > 4 ? 2 : 1]) {
    constexpr int SEG = TWW * kTileRows;
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int tt = 0; tt < TWW; ++tt)
#pragma unroll
        for (int hh = 0; hh < (N > 4 ? 2 : 1); ++hh) {
            const int c = g + 4 * hh;
            if (c < N) red[(wave * N + c) * SEG + tt * kTileRows + r] = acc[tt][hh];
        }
}

// After the barrier: the waves' partials of each (column, row) added in wave
// order, times tscale, stored to Y [N][rows] (when Y is not NULL); with keys
// not NULL, the workgroup's largest argmax key of each column goes to
// keys[c].  row0 is the workgroup's first row.
template <int N, int TWW>
__device__ __forceinline__ void finish_rows(const float *red, int ksplit, float tscale, int rows, int row0,
                                            float *__restrict__ Y, unsigned long long *__restrict__ keys) {
    constexpr int SEG = TWW * kTileRows;
    // Segments of SEG consecutive threads hold one column's rows; blockDim is
    // a multiple of 64 and SEG divides 64, so a segment never straddles a
    // wave or an iteration.
    for (int idx = threadIdx.x; idx < N * SEG; idx += blockDim.x) {
        // every wave's partial is read before the first add (clamped indices,
        // adds in wave order): one LDS round trip instead of one per batch
        const int c = idx / SEG, lr = idx % SEG;
        float part[kMaxKsplit];
#pragma unroll
        for (int w = 0; w < kMaxKsplit; ++w) part[w] = red[((w < ksplit ? w : 0) * N + c) * SEG + lr];
        float tot = part[0];
#pragma unroll
        for (int w = 1; w < kMaxKsplit; ++w)
            if (w < ksplit) tot += part[w];
        const float y = tot * tscale;
        const int row = row0 + lr;
        const bool valid = row < rows;
        if (valid && Y) Y[int64_t(c) * rows + row] = y;
        if (keys) {
            // the segment's SEG lanes are all active (SEG divides 64; keys is
            // the same for the whole workgroup)
            const unsigned long long key = lanes_max_u64<SEG>(valid ? argmax_key(y, uint32_t(row)) : 0ull);
            if (lr == 0) keys[c] = key;
        }
    }
}

// MODE kPlain:  Y[c][row] = tscale * sum.
// MODE kArgmax: as kPlain (Y may be NULL) plus, per column, the largest
//   argmax key of the workgroup's rows stored to amax_ws[blockIdx][c]
//   (amax_ws: the keys after the finish header, whose counter workgroup 0
//   zeroes); an argmax finish kernel, launched next on the stream, reduces
//   them.
// MODE kSwiglu: the workgroup's waves [0, ksplit) take gate rows, waves
//   [ksplit, 2 ksplit) the up rows up_st super-tiles further down (the same
//   positions of the stacked matrix); h[c][row] = bf16(SiLU(g) u) with
//   g, u = tscale * sum, and Y (when not NULL) receives g and u at the stacked
//   positions, so every bit equals the plain product followed by the SwiGLU
//   kernel.
template <int N, int TWW, int MODE, int FMT = kNvfp4>
__global__ void __launch_bounds__(kLanes * kMaxKsplit)
narrow_kernel(const uint8_t *__restrict__ wq, const uint8_t *__restrict__ ws, float tscale, int rows, int octets,
              int kb, int ksplit, const uint16_t *__restrict__ X, int K, float *__restrict__ Y,
              unsigned long long *__restrict__ amax_ws, int up_st, uint16_t *__restrict__ h) {
    // [waves][narrow_wave_lds_bytes(N)] activation slots, then the partial
    // sums [waves][N][SEG]
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int GPS = kSuperTiles / TWW;   // workgroups per super-tile
    constexpr int SEG = TWW * kTileRows;     // rows per workgroup
    constexpr int H = N > 4 ? 2 : 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int st = blockIdx.x / GPS, tg = blockIdx.x % GPS;
    const int half = MODE == kSwiglu ? wave / ksplit : 0;
    const int part = MODE == kSwiglu ? wave % ksplit : wave;
    const int o0 = octet_bound(octets, part, ksplit), o1 = octet_bound(octets, part + 1, ksplit);
    constexpr int WL = narrow_wave_lds_bytes(N);
    float *const red = reinterpret_cast<float *>(lds + int(blockDim.x >> 6) * WL);
    if (MODE == kArgmax && blockIdx.x == 0 && threadIdx.x == 0) *finish_counter(amax_ws) = 0u;

    float acc[TWW][H];
    narrow_accumulate<N, TWW, FMT>(wq, ws, int64_t(st) + (half ? up_st : 0), tg, o0, o1, octets, kb, X, K, lane,
                                   acc, lds + wave * WL);
    store_partials<N, TWW>(red, wave, lane, acc);
    __syncthreads();

    const int row0 = st * kSuperRows + tg * SEG;
    if (MODE == kSwiglu) {
        const int F = up_st * kSuperRows;
        for (int idx = threadIdx.x; idx < N * SEG; idx += blockDim.x) {
            // both halves' partials read before the first add (at most
            // kMaxKsplit / 2 waves per half), adds in wave order
            constexpr int KH = kMaxKsplit / 2;
            const int c = idx / SEG, lr = idx % SEG;
            float gp[KH], up[KH];
#pragma unroll
            for (int w = 0; w < KH; ++w) {
                const int ww = w < ksplit ? w : 0;
                gp[w] = red[(ww * N + c) * SEG + lr];
                up[w] = red[((ksplit + ww) * N + c) * SEG + lr];
            }
            float gs = gp[0], us = up[0];
#pragma unroll
            for (int w = 1; w < KH; ++w)
                if (w < ksplit) {
                    gs += gp[w];
                    us += up[w];
                }
            gs *= tscale;
            us *= tscale;
            const int row = row0 + lr;
            if (Y) {
                Y[int64_t(c) * 2 * F + row] = gs;
                Y[int64_t(c) * 2 * F + F + row] = us;
            }
            h[int64_t(c) * F + row] = uint16_t(bf16_rne_bits(swiglu_f32(gs, us)));
        }
        return;
    }

    finish_rows<N, TWW>(red, ksplit, tscale, rows, row0, Y,
                        MODE == kArgmax ? amax_ws + int64_t(blockIdx.x) * N : nullptr);
}

// ------------------------------------------------ several products, one launch

// Up to kMaxBatch independent products of one activation matrix in one
// launch (see nvfp4_gemv_batch): workgroups [group0, next group0) belong to a
// product, and each runs exactly the narrow_kernel workgroup of that product
// (the same waves, octet ranges and arithmetic), so every product has the
// bits of its own nvfp4_gemv or nvfp4_gemv_argmax call.
constexpr int kMaxBatch = 4;
struct BatchSegment {
    const uint8_t *wq, *ws;
    float *Y;                    // NULL: not stored
    unsigned long long *keys;    // NULL: no argmax; else the product's keys (after its finish header)
    float tscale;
    int rows;
};
struct BatchArgs {
    int group0[kMaxBatch];       // each product's first workgroup; unused entries past the last workgroup
    BatchSegment seg[kMaxBatch];
};

template <int N, int TWW>
__global__ void __launch_bounds__(kLanes * kMaxKsplit)
narrow_batch_kernel(BatchArgs args, int octets, int kb, int ksplit, const uint16_t *__restrict__ X, int K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int GPS = kSuperTiles / TWW;
    constexpr int SEG = TWW * kTileRows;
    constexpr int H = N > 4 ? 2 : 1;
    // The workgroup's product: the products' first workgroups and every
    // other scalar argument come in one round of argument loads, then the
    // product's fields in a second (a uniform index into the argument
    // segment, no copy of the array to registers).  The empty asm statements
    // keep the compiler from sinking loads into later, dependent rounds.
    asm volatile("" ::"s"(X), "s"(K), "s"(octets), "s"(kb), "s"(ksplit));
    int pi = 0, g0 = 0;   // group0[0] is 0
#pragma unroll
    for (int i = 1; i < kMaxBatch; ++i)
        if (int(blockIdx.x) >= args.group0[i]) {   // ascending: the last one passed is the product's
            pi = i;
            g0 = args.group0[i];
        }
    pi = __builtin_amdgcn_readfirstlane(pi);
    const BatchSegment seg = args.seg[pi];
    asm volatile("" ::"s"(seg.wq), "s"(seg.ws));
    const int b = int(blockIdx.x) - g0;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int st = b / GPS, tg = b % GPS;
    const int o0 = octet_bound(octets, wave, ksplit), o1 = octet_bound(octets, wave + 1, ksplit);
    constexpr int WL = narrow_wave_lds_bytes(N);
    float *const red = reinterpret_cast<float *>(lds + int(blockDim.x >> 6) * WL);
    if (seg.keys != nullptr && b == 0 && threadIdx.x == 0) *finish_counter(seg.keys) = 0u;
    float acc[TWW][H];
    narrow_accumulate<N, TWW, kNvfp4>(seg.wq, seg.ws, int64_t(st), tg, o0, o1, octets, kb, X, K, lane, acc,
                                      lds + wave * WL);
    store_partials<N, TWW>(red, wave, lane, acc);
    __syncthreads();
    finish_rows<N, TWW>(red, ksplit, seg.tscale, seg.rows, st * kSuperRows + tg * SEG, seg.Y,
                        seg.keys ? seg.keys + int64_t(b) * N : nullptr);
}

// Second launch of the argmax: the product's per-workgroup keys are complete
// (kernel boundary); the largest key of each column names its row.  The
// maximum is order-independent, so the result is exact and reproducible.
// The keys were just written from every XCD, so each read goes to memory,
// and one CU takes them in at only about 30 GB/s.  Up to 6144 keys (12288 at
// one or two columns; finish_split) one workgroup reads them all: every
// thread issues all its loads of a pass (up to 8 groups of N keys, or 32 keys
// of one column at N = 8) before it compares any of them, one or two memory
// round trips instead of one per loop iteration.  Above that,
// argmax_finish_split_kernel spreads the reads over kFinishGroups workgroups
// (on as many CUs).
constexpr int kFinishThreads = 1024;

template <int N>
__global__ void __launch_bounds__(kFinishThreads)
argmax_finish_kernel(const unsigned long long *__restrict__ keys, int groups, int32_t *__restrict__ argmax_out) {
    __shared__ unsigned long long part[kFinishThreads / kLanes][N];
    if constexpr (N == 8) {
        // Thread t reads keys t, t + 1024, ... of the flat [groups][8] array,
        // all of column t % 8, so consecutive lanes read consecutive keys
        // where the per-group loads below leave 64-byte gaps between lanes
        // (vocabulary head at N = 8: 83.5 against 86.2 us per call; at N = 1
        // and 4 the per-group loads measured faster).
        constexpr int U = 32;
        const int total = groups * N;
        unsigned long long m = 0ull;
        for (int j0 = 0; j0 < total; j0 += kFinishThreads * U) {
            unsigned long long k[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u * kFinishThreads + int(threadIdx.x);
                k[u] = j < total ? keys[j] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) m = k[u] > m ? k[u] : m;
        }
        // lanes l, l ^ 8, l ^ 16 and l ^ 32 share a column: row_ror:8 pairs
        // lane i of a row with lane i ^ 8, then the rows meet by permlanes
        m = rows_max_u64<kLanes>(dpp_max_u64<0x128>(m));
        if ((threadIdx.x & 63) < N) part[threadIdx.x >> 6][threadIdx.x & 63] = m;
        __syncthreads();
        if (threadIdx.x < N) {
            const int c = threadIdx.x;
            unsigned long long best = part[0][c];
#pragma unroll
            for (int w = 1; w < kFinishThreads / kLanes; ++w) best = part[w][c] > best ? part[w][c] : best;
            argmax_out[c] = int32_t(0xFFFFFFFFu - uint32_t(best));
        }
        return;
    }
    constexpr int U = N > 4 ? 4 : 8;   // groups per thread per pass (register budget)
    unsigned long long m[N];
#pragma unroll
    for (int c = 0; c < N; ++c) m[c] = 0ull;
    for (int g0 = 0; g0 < groups; g0 += kFinishThreads * U) {
        unsigned long long k[U][N];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u * kFinishThreads + int(threadIdx.x);
#pragma unroll
            for (int c = 0; c < N; ++c) k[u][c] = g < groups ? keys[int64_t(g) * N + c] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < N; ++c) m[c] = k[u][c] > m[c] ? k[u][c] : m[c];
    }
#pragma unroll
    for (int c = 0; c < N; ++c) {
        m[c] = lanes_max_u64<kLanes>(m[c]);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][c] = m[c];
    }
    __syncthreads();
    if (threadIdx.x < N) {
        const int c = threadIdx.x;
        unsigned long long best = part[0][c];
#pragma unroll
        for (int w = 1; w < kFinishThreads / kLanes; ++w) best = part[w][c] > best ? part[w][c] : best;
        argmax_out[c] = int32_t(0xFFFFFFFFu - uint32_t(best));
    }
}

// The split finish: workgroup w reduces its share of the groups to N
// partial maxima, stores them to the header and counts itself on the
// header's counter with an agent-scope release add; the workgroup that
// counts last takes an agent-scope acquire fence, reads the kFinishGroups x N
// parts and writes the indices.  The part stores come from threads 0 .. N - 1
// (N <= 8), all in the first wave, whose thread 0 also makes the release add:
// the release covers them as that wave's own earlier stores (the L2
// write-back and the wait for the wave's outstanding stores come before the
// add), whatever the workgroup barrier between them does or does not wait for.  On gfx950 the release is an L2 write-back
// and the acquire an L2 invalidate (the XCDs' L2s are not coherent); with
// the L2 holding only the parts, both measured within noise of leaving them
// out.  The product zeroed the counter.
constexpr int kSplitFinishThreads = 256;
static_assert(kMaxNarrowN <= kLanes, "the split finish's part stores come from its first wave");

template <int N>
__global__ void __launch_bounds__(kSplitFinishThreads)
argmax_finish_split_kernel(unsigned long long *__restrict__ keys, int groups, int32_t *__restrict__ argmax_out) {
    __shared__ unsigned long long part[kSplitFinishThreads / kLanes][N];
    __shared__ int last;
    unsigned long long *const parts = keys - kFinishHeaderWords + kFinishCounterWords;
    const int per = (groups + kFinishGroups - 1) / kFinishGroups;
    const int g_lo = int(blockIdx.x) * per;
    const int g_hi = groups - g_lo < per ? groups : g_lo + per;
    constexpr int U = N > 4 ? 2 : 4;   // groups per thread per pass
    unsigned long long m[N];
#pragma unroll
    for (int c = 0; c < N; ++c) m[c] = 0ull;
    for (int g0 = g_lo; g0 < g_hi; g0 += kSplitFinishThreads * U) {
        unsigned long long k[U][N];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u * kSplitFinishThreads + int(threadIdx.x);
#pragma unroll
            for (int c = 0; c < N; ++c) k[u][c] = g < g_hi ? keys[int64_t(g) * N + c] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < N; ++c) m[c] = k[u][c] > m[c] ? k[u][c] : m[c];
    }
#pragma unroll
    for (int c = 0; c < N; ++c) {
        m[c] = lanes_max_u64<kLanes>(m[c]);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][c] = m[c];
    }
    __syncthreads();
    if (threadIdx.x < N) {
        const int c = threadIdx.x;
        unsigned long long best = part[0][c];
#pragma unroll
        for (int w = 1; w < kSplitFinishThreads / kLanes; ++w) best = part[w][c] > best ? part[w][c] : best;
        parts[int(blockIdx.x) * N + c] = best;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool l = __hip_atomic_fetch_add(finish_counter(keys), 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
                       unsigned(kFinishGroups - 1);
        if (l) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        last = l;
    }
    __syncthreads();
    if (!last || threadIdx.x >= N) return;
    const int c = threadIdx.x;
    unsigned long long p[kFinishGroups];
#pragma unroll
    for (int w = 0; w < kFinishGroups; ++w) p[w] = parts[w * N + c];
    unsigned long long best = p[0];
#pragma unroll
    for (int w = 1; w < kFinishGroups; ++w) best = p[w] > best ? p[w] : best;
    argmax_out[c] = int32_t(0xFFFFFFFFu - uint32_t(best));
}

// ------------------------------------------------------------------ dispatch

template <int MODE, int TWW, int FMT = kNvfp4>
int launch_narrow_tww(const Geometry &g, const NarrowConfig &cfg, const uint8_t *wq, const uint8_t *ws,
                      float tscale, const uint16_t *X, int n, float *Y, unsigned long long *amax_ws,
                      int up_st, uint16_t *h, int waves, int64_t groups, hipStream_t stream) {
    const dim3 grid{unsigned(groups)}, block{unsigned(kLanes * waves)};
    const size_t lds = narrow_lds_bytes(waves, n, TWW);
    if (lds > kNarrowLdsLimit) return NVFP4_EINVAL;
    const int rows = int(g.rows), octets = int(g.octets), kb = int(g.kb), K = int(g.cols);
#define NVFP4_LAUNCH(NN)                                                                                      \
    hipLaunchKernelGGL((narrow_kernel<NN, TWW, MODE, FMT>), grid, block, lds, stream, wq, ws, tscale, rows, octets, \
                       kb, cfg.ksplit, X, K, Y, amax_ws, up_st, h)
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

template <int MODE>
int launch_narrow(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                  int n, float *Y, unsigned long long *amax_ws, hipStream_t stream) {
    const NarrowConfig cfg = MODE == kArgmax ? argmax_config(g, n) : narrow_config(g, n);
    switch (cfg.tww) {
        case 1: return launch_narrow_tww<MODE, 1>(g, cfg, wq, ws, tscale, X, n, Y, amax_ws, 0, nullptr, cfg.ksplit,
                                                 cfg.groups, stream);
        case 2: return launch_narrow_tww<MODE, 2>(g, cfg, wq, ws, tscale, X, n, Y, amax_ws, 0, nullptr, cfg.ksplit,
                                                 cfg.groups, stream);
        default: return launch_narrow_tww<MODE, 4>(g, cfg, wq, ws, tscale, X, n, Y, amax_ws, 0, nullptr,
                                                  cfg.ksplit, cfg.groups, stream);
    }
}

int launch_mfma(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                int n, float *Y, hipStream_t stream, int fmt = kNvfp4);
double wide_estimate_us(const Geometry &g, int n, int fmt);

// Products of 9..128 columns either as passes of the matvec over column
// chunks of at most eight (columns [8p, 8p + 8) of X and Y in pass p: each
// column then has the bits of its one-column product, and the weights are
// read once per pass), or as the wide product, whichever is estimated
// faster.  A pass costs about the read of the weights at 4 TB/s plus 2.5 us
// (17408 x 5120: 12.5-13.8 us, 4096 x 4096: 4.3-4.6 us, 5120 x 17408: 15 us
// measured); the wide product's estimate follows its shape and workgroup
// rounds (wide_estimate_us).  So 17408 x 5120 takes two passes up to 16
// columns (28 against 30 us) and the wide product from 17 (30.5 us at 32
// columns against 53 us in four passes), while 4096 x 4096 and 5120 x 17408
// keep passes to about 48 and 56 columns.  Returns the number of passes, 0
// for the wide product.
int narrow_passes(const Geometry &g, int n, int fmt) {
    if (n <= kMaxNarrowN || n > 16 * kMaxNarrowN || g.cols > kMaxNarrowCols) return 0;
    const int passes = int(ceil_div(n, kMaxNarrowN));
    const double pass_us = double(g.code_bytes() + g.scale_bytes(fmt)) / 4.0e6 + 2.5;
    const double wide_us = wide_estimate_us(g, n, fmt);
    return wide_us < 0.0 || double(passes) * pass_us <= wide_us ? passes : 0;
}

template <typename Launch>
int launch_passes(const Geometry &g, const uint16_t *X, int n, float *Y, Launch launch) {
    for (int c0 = 0; c0 < n; c0 += kMaxNarrowN) {
        const int w = n - c0 < kMaxNarrowN ? n - c0 : kMaxNarrowN;
        if (int st = launch(X + int64_t(c0) * g.cols, w, Y + int64_t(c0) * g.rows)) return st;
    }
    return NVFP4_OK;
}

// The MXFP4 matvec: the plain product's decomposition and kernel with the
// E8M0 scale plane, at most two tiles per workgroup.
int launch_narrow_mx(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale, const uint16_t *X,
                     int n, float *Y, hipStream_t stream) {
    const NarrowConfig cfg = narrow_config(g, n, 2);
    switch (cfg.tww) {
        case 1: return launch_narrow_tww<kPlain, 1, kMxfp4>(g, cfg, wq, ws, tscale, X, n, Y, nullptr, 0, nullptr,
                                                            cfg.ksplit, cfg.groups, stream);
        case 2: return launch_narrow_tww<kPlain, 2, kMxfp4>(g, cfg, wq, ws, tscale, X, n, Y, nullptr, 0, nullptr,
                                                            cfg.ksplit, cfg.groups, stream);
        default: return NVFP4_EINVAL;
    }
}

// True when the fused gate||up+SwiGLU kernel reproduces the stacked product's
// decomposition: the up rows start on a super-tile boundary and a workgroup
// can hold both halves' waves.
inline bool swiglu_fusable(const Geometry &stacked, int64_t F, int n) {
    return F % kSuperRows == 0 && 2 * narrow_config(stacked, n).ksplit <= kMaxKsplit;
}

int launch_gemv_swiglu(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t hidden, int64_t F,
                       const uint16_t *X, int n, float *gu, uint16_t *h, hipStream_t stream) {
    const Geometry g(2 * F, hidden);
    if (!swiglu_fusable(g, F, n)) {
        // The plain product into gu, then the SwiGLU kernel: the same bits.
        const unsigned grid = grid_1d(F * n, 256);
        if (!gu || !grid) return NVFP4_ESHAPE;
        if (int st = launch_narrow<kPlain>(g, wq, ws, tscale, X, n, gu, nullptr, stream)) return st;
        hipLaunchKernelGGL(swiglu_kernel, dim3(grid), dim3(256), 0, stream, gu, F,
                           F * n, h);
        return launch_status();
    }
    NarrowConfig cfg = narrow_config(g, n);
    // A workgroup holds both halves' waves; where their LDS would pass the
    // limit (four tiles at 16 waves past four columns) it takes fewer tiles,
    // which changes no row's summation order.
    while (cfg.tww > 1 && narrow_lds_bytes(2 * cfg.ksplit, n, cfg.tww) > kNarrowLdsLimit) {
        cfg.tww /= 2;
        cfg.groups = g.supertiles * (kSuperTiles / cfg.tww);
    }
    const int64_t groups = cfg.groups / 2;   // the gate half's workgroups
    const int up_st = int(F / kSuperRows);
    switch (cfg.tww) {
        case 1: return launch_narrow_tww<kSwiglu, 1>(g, cfg, wq, ws, tscale, X, n, gu, nullptr, up_st, h,
                                                    2 * cfg.ksplit, groups, stream);
        case 2: return launch_narrow_tww<kSwiglu, 2>(g, cfg, wq, ws, tscale, X, n, gu, nullptr, up_st, h,
                                                    2 * cfg.ksplit, groups, stream);
        default: return launch_narrow_tww<kSwiglu, 4>(g, cfg, wq, ws, tscale, X, n, gu, nullptr, up_st, h,
                                                     2 * cfg.ksplit, groups, stream);
    }
}

}  // namespace nvfp4

using namespace nvfp4;

static int check_product_args(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                              const uint16_t *X, int n) {
    if (!wq || !ws || !X || !tscale_ok(tscale) || n < 1 || n > NVFP4_MAX_N) return NVFP4_EINVAL;
    if (int st = check_shape(rows, cols)) return st;
    // The narrow products address a wave's weights and the activations with
    // 32-bit buffer offsets.
    if (n <= kMaxNarrowN && cols > kMaxNarrowCols) return NVFP4_ESHAPE;
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
    if (n <= kMaxNarrowN) return launch_narrow<kPlain>(g, wq, ws, tscale, X, n, Y, nullptr, stream);
    if (narrow_passes(g, n, kNvfp4))
        return launch_passes(g, X, n, Y, [&](const uint16_t *Xp, int w, float *Yp) {
            return launch_narrow<kPlain>(g, wq, ws, tscale, Xp, w, Yp, nullptr, stream);
        });
    return launch_mfma(g, wq, ws, tscale, X, n, Y, stream);
}

NVFP4_API size_t nvfp4_gemv_argmax_workspace_bytes(int64_t rows, int64_t cols, int n) {
    // The finish header, then one 64-bit key per workgroup and column.
    if (n < 1 || n > kMaxNarrowN || check_shape(rows, cols) != NVFP4_OK || cols > kMaxNarrowCols) return 0;
    return (size_t(kFinishHeaderWords) + size_t(argmax_config(Geometry(rows, cols), n).groups) * size_t(n)) *
           sizeof(unsigned long long);
}

// Whether the argmax finish of `groups` workgroups' keys of n columns runs
// split.  Measured on the vocabulary head (9496 keys either way): at four
// columns the split finish took 0.6 us less, at two 0.3 us more, where the
// one workgroup's loads take fewer instructions per key; at eight (18992
// keys) 1.8 us less.
inline bool finish_split(int64_t groups, int n) { return groups * n > (n <= 2 ? 12288 : 6144); }

// The argmax finish of `groups` workgroups' keys of n columns (keys: after
// the product's finish header).
static int launch_finish(int n, unsigned long long *keys, int groups, int32_t *argmax, hipStream_t stream) {
    const bool split = finish_split(groups, n);
#define NVFP4_FINISH(NN)                                                                                      \
    if (split)                                                                                              \
        hipLaunchKernelGGL(argmax_finish_split_kernel<NN>, dim3(kFinishGroups), dim3(kSplitFinishThreads), 0, \
                           stream, keys, groups, argmax);                                                   \
    else                                                                                                    \
        hipLaunchKernelGGL(argmax_finish_kernel<NN>, dim3(1), dim3(kFinishThreads), 0, stream, keys, groups, argmax)
    switch (n) {
        case 1: NVFP4_FINISH(1); break;
        case 2: NVFP4_FINISH(2); break;
        case 3: NVFP4_FINISH(3); break;
        case 4: NVFP4_FINISH(4); break;
        case 5: NVFP4_FINISH(5); break;
        case 6: NVFP4_FINISH(6); break;
        case 7: NVFP4_FINISH(7); break;
        default: NVFP4_FINISH(8); break;
    }
#undef NVFP4_FINISH
    return launch_status();
}

// The argmax's two launches in `workspace` (its finish header, then the
// keys); the arguments are already validated.
static int launch_gemv_argmax(const Geometry &g, const uint8_t *wq, const uint8_t *ws, float tscale,
                              const uint16_t *X, int n, float *logits, int32_t *argmax,
                              unsigned long long *workspace, hipStream_t stream) {
    unsigned long long *const keys = workspace + kFinishHeaderWords;
    (void)hipGetLastError();
    if (int st = launch_narrow<kArgmax>(g, wq, ws, tscale, X, n, logits, keys, stream)) return st;
    return launch_finish(n, keys, int(argmax_config(g, n).groups), argmax, stream);
}

static int check_argmax_args(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                             const uint16_t *X, int n, float *logits, int32_t *argmax) {
    if (!argmax) return NVFP4_EINVAL;
    if (int st = check_product_args(wq, ws, tscale, rows, cols, X, n)) return st;
    if (n > kMaxNarrowN) return NVFP4_EINVAL;
    if (!aligned(logits, 4) || !aligned(argmax, 4)) return NVFP4_EALIGN;
    return NVFP4_OK;
}

NVFP4_API int nvfp4_gemv_argmax(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows,
                                int64_t cols, const uint16_t *X, int n, float *logits, int32_t *argmax,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!workspace) return NVFP4_EINVAL;
    if (int st = check_argmax_args(wq, ws, tscale, rows, cols, X, n, logits, argmax)) return st;
    if (!aligned(workspace, 8)) return NVFP4_EALIGN;
    if (workspace_bytes < nvfp4_gemv_argmax_workspace_bytes(rows, cols, n)) return NVFP4_EWORKSPACE;
    return launch_gemv_argmax(Geometry(rows, cols), wq, ws, tscale, X, n, logits, argmax,
                              static_cast<unsigned long long *>(workspace), stream);
}

// ------------------------------------------- the argmax without a workspace

// The key workspace of nvfp4_gemv_argmax_noalloc: one static array per GPU,
// loaded with the library's code object and held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address); it passes the address that
// hipGetSymbolAddress gives on that device, looked up once per device on the
// entry point's first call there, with that device current.
static __device__ __align__(256) unsigned long long scratch[NVFP4_ARGMAX_SCRATCH_BYTES / sizeof(unsigned long long)];

namespace {
constexpr int kMaxScratchDevices = 64;
struct ScratchDevice {
    std::once_flag once;
    unsigned long long *ptr = nullptr;
};
ScratchDevice g_scratch[kMaxScratchDevices];

unsigned long long *scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    ScratchDevice &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) d.ptr = static_cast<unsigned long long *>(p);
    });
    return d.ptr;
}
}  // namespace

NVFP4_API int nvfp4_gemv_argmax_noalloc(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows,
                                        int64_t cols, const uint16_t *X, int n, float *logits, int32_t *argmax,
                                        hipStream_t stream) {
    if (int st = check_argmax_args(wq, ws, tscale, rows, cols, X, n, logits, argmax)) return st;
    if (nvfp4_gemv_argmax_workspace_bytes(rows, cols, n) > NVFP4_ARGMAX_SCRATCH_BYTES) return NVFP4_EWORKSPACE;
    unsigned long long *const ptr = scratch_on_current_device();
    if (!ptr) return NVFP4_EHIP;
    return launch_gemv_argmax(Geometry(rows, cols), wq, ws, tscale, X, n, logits, argmax, ptr, stream);
}

NVFP4_API int nvfp4_gemv_swiglu(const uint8_t *wq_gu, const uint8_t *ws_gu, float tscale, int64_t hidden,
                                int64_t F, const uint16_t *X, int n, float *gu, uint16_t *h,
                                hipStream_t stream) {
    if (!h) return NVFP4_EINVAL;
    if (F < kTileRows || F % kTileRows != 0) return NVFP4_ESHAPE;
    if (int st = check_product_args(wq_gu, ws_gu, tscale, 2 * F, hidden, X, n)) return st;
    if (n > kMaxNarrowN) return NVFP4_EINVAL;
    if (!aligned(gu, 4) || !aligned(h, 2)) return NVFP4_EALIGN;
    (void)hipGetLastError();
    return launch_gemv_swiglu(wq_gu, ws_gu, tscale, hidden, F, X, n, gu, h, stream);
}

NVFP4_API int nvfp4_swiglu(const float *gu, int64_t F, int n, uint16_t *h, hipStream_t stream) {
    if (!gu || !h || n < 1 || n > NVFP4_MAX_N) return NVFP4_EINVAL;
    if (F < 1 || F > (int64_t(1) << 40)) return NVFP4_ESHAPE;
    if (!aligned(gu, 16) || !aligned(h, 4)) return NVFP4_EALIGN;
    const int64_t total = F * n;
    const unsigned grid = grid_1d(total, 256);
    if (!grid) return NVFP4_ESHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(swiglu_kernel, dim3(grid), dim3(256), 0, stream, gu, F, total, h);
    return launch_status();
}

// ------------------------------------------------------------------ MXFP4

NVFP4_API int mxfp4_gemv(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                         const uint16_t *X, int n, float *Y, hipStream_t stream) {
    if (!Y) return NVFP4_EINVAL;
    if (int st = check_product_args(wq, ws, tscale, rows, cols, X, n)) return st;
    if (int st = check_mx_shape(rows, cols)) return st;
    if (!aligned(Y, 4)) return NVFP4_EALIGN;
    const Geometry g(rows, cols);
    (void)hipGetLastError();
    if (n <= kMaxNarrowN) return launch_narrow_mx(g, wq, ws, tscale, X, n, Y, stream);
    if (narrow_passes(g, n, kMxfp4))
        return launch_passes(g, X, n, Y, [&](const uint16_t *Xp, int w, float *Yp) {
            return launch_narrow_mx(g, wq, ws, tscale, Xp, w, Yp, stream);
        });
    return launch_mfma(g, wq, ws, tscale, X, n, Y, stream, kMxfp4);
}

// --------------------------------------------------- several products, one launch

namespace {

// How nvfp4_gemv_batch runs a batch: one launch of narrow_batch_kernel when
// every product's own decomposition splits a row over the same number of
// waves (then each product's bits are those of its own call, whatever the
// tiles per workgroup), with the largest of the products' tiles per
// workgroup; otherwise each product's own launch.  The argmax products'
// workspaces (finish header, then keys) follow one another.
struct BatchPlan {
    bool fused;
    int ksplit, tww;
    int64_t groups[kMaxBatch];      // workgroups of each product
    int64_t key_offset[kMaxBatch];  // first key of each argmax product, after its finish header (words)
    int64_t keys;                   // 64-bit words in all: each argmax product's header and keys
    int64_t total_groups;
};

BatchPlan plan_batch(const nvfp4_product *p, int count, int64_t cols, int n) {
    BatchPlan b{};
    b.fused = count > 1;
    for (int i = 0; i < count; ++i) {
        const Geometry g(p[i].rows, cols);
        const NarrowConfig c = p[i].argmax ? argmax_config(g, n) : narrow_config(g, n);
        if (i == 0) {
            b.ksplit = c.ksplit;
            b.tww = c.tww;
        }
        if (c.ksplit != b.ksplit) b.fused = false;
        if (c.tww > b.tww) b.tww = c.tww;
    }
    for (int i = 0; i < count; ++i) {
        const Geometry g(p[i].rows, cols);
        b.groups[i] = b.fused ? g.supertiles * (kSuperTiles / b.tww)
                              : (p[i].argmax ? argmax_config(g, n) : narrow_config(g, n)).groups;
        b.key_offset[i] = b.keys + kFinishHeaderWords;
        if (p[i].argmax) b.keys += kFinishHeaderWords + b.groups[i] * n;
        b.total_groups += b.groups[i];
    }
    return b;
}

int check_batch(const nvfp4_product *p, int count, int64_t cols, int n) {
    if (!p || count < 1 || count > kMaxBatch || n < 1 || n > kMaxNarrowN) return NVFP4_EINVAL;
    if (int st = check_shape(1, cols)) return st;
    if (cols > kMaxNarrowCols) return NVFP4_ESHAPE;
    for (int i = 0; i < count; ++i) {
        const nvfp4_product &q = p[i];
        if (!q.wq || !q.ws || !tscale_ok(q.tscale) || (!q.y && !q.argmax)) return NVFP4_EINVAL;
        if (int st = check_shape(q.rows, cols)) return st;
        if (!aligned(q.wq, 16) || !aligned(q.ws, 16) || !aligned(q.y, 4) || !aligned(q.argmax, 4)) return NVFP4_EALIGN;
    }
    return NVFP4_OK;
}

}  // namespace

NVFP4_API size_t nvfp4_gemv_batch_workspace_bytes(const nvfp4_product *products, int count, int64_t cols, int n) {
    if (check_batch(products, count, cols, n) != NVFP4_OK) return 0;
    return size_t(plan_batch(products, count, cols, n).keys) * sizeof(unsigned long long);
}

NVFP4_API int nvfp4_gemv_batch(const nvfp4_product *products, int count, int64_t cols, const uint16_t *X, int n,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!X) return NVFP4_EINVAL;
    if (int st = check_batch(products, count, cols, n)) return st;
    if (!aligned(X, 16)) return NVFP4_EALIGN;
    const BatchPlan b = plan_batch(products, count, cols, n);
    if (b.keys > 0) {
        if (!workspace) return NVFP4_EINVAL;
        if (!aligned(workspace, 8)) return NVFP4_EALIGN;
        if (workspace_bytes < size_t(b.keys) * sizeof(unsigned long long)) return NVFP4_EWORKSPACE;
    }
    if (b.total_groups > (int64_t(1) << 31) - 1) return NVFP4_ESHAPE;
    auto *keys = static_cast<unsigned long long *>(workspace);
    (void)hipGetLastError();
    if (b.fused) {
        BatchArgs a{};
        int64_t g0 = 0;
        for (int i = 0; i < count; ++i) {
            const nvfp4_product &q = products[i];
            a.group0[i] = int(g0);
            a.seg[i] = BatchSegment{q.wq, q.ws, q.y, q.argmax ? keys + b.key_offset[i] : nullptr, q.tscale,
                                    int(q.rows)};
            g0 += b.groups[i];
        }
        for (int i = count; i < kMaxBatch; ++i) a.group0[i] = int(g0);   // past the grid: never selected
        const Geometry g(1, cols);
        const size_t lds = narrow_lds_bytes(b.ksplit, n, b.tww);
        if (lds > kNarrowLdsLimit) return NVFP4_EINVAL;
        const dim3 grid{unsigned(b.total_groups)}, block{unsigned(kLanes * b.ksplit)};
        const int octets = int(g.octets), kb = int(g.kb), K = int(cols);
#define NVFP4_BATCH(NN, TT) \
    hipLaunchKernelGGL((narrow_batch_kernel<NN, TT>), grid, block, lds, stream, a, octets, kb, b.ksplit, X, K)
#define NVFP4_BATCH_N(TT)                    \
    switch (n) {                            \
        case 1: NVFP4_BATCH(1, TT); break;  \
        case 2: NVFP4_BATCH(2, TT); break;  \
        case 3: NVFP4_BATCH(3, TT); break;  \
        case 4: NVFP4_BATCH(4, TT); break;  \
        case 5: NVFP4_BATCH(5, TT); break;  \
        case 6: NVFP4_BATCH(6, TT); break;  \
        case 7: NVFP4_BATCH(7, TT); break;  \
        default: NVFP4_BATCH(8, TT); break; \
    }
        switch (b.tww) {
            case 1: NVFP4_BATCH_N(1); break;
            case 2: NVFP4_BATCH_N(2); break;
            default: NVFP4_BATCH_N(4); break;
        }
#undef NVFP4_BATCH_N
#undef NVFP4_BATCH
        if (int st = launch_status()) return st;
    } else {
        for (int i = 0; i < count; ++i) {
            const nvfp4_product &q = products[i];
            const Geometry g(q.rows, cols);
            const int st = q.argmax ? launch_narrow<kArgmax>(g, q.wq, q.ws, q.tscale, X, n, q.y, keys + b.key_offset[i], stream)
                                    : launch_narrow<kPlain>(g, q.wq, q.ws, q.tscale, X, n, q.y, nullptr, stream);
            if (st) return st;
        }
    }
    for (int i = 0; i < count; ++i)
        if (products[i].argmax)
            if (int st = launch_finish(n, keys + b.key_offset[i], int(b.groups[i]), products[i].argmax, stream))
                return st;
    return NVFP4_OK;
}
