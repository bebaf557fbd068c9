/*
 * nvfp4.h -- C ABI of libnvfp4: NVFP4 weight x bf16 activation matrix-vector
 * products on AMD Instinct MI355X (gfx950).
 *
 * The method (pages this library follows):
 *   - bw24 wiki (GitHub) and bw24 README (wpnews page "Bw24 - from scratch
 *     rust+CUDA inference, every kernel tuned for sm_120a"), feature list,
 *     NVFP4 decode-path item: decode multiplies block-scaled FP4 weights by
 *     the activation vector in a matvec fed by a "split-plane" repack of the
 *     weights, a wider GEMM serves prefill, and the kernel is picked per
 *     matrix shape; the MTP item: the K+1 draft tokens of a speculative round
 *     are verified in one batched forward, so every weight is read once for
 *     all K+1 columns.
 *   - bw24 wiki, correctness gates and the exactness note after them: the
 *     order of floating-point summation is part of the contract, and a
 *     prefill-argmax vs decode-argmax gate precedes any timing.
 *   - qwentin README (gitlite mirror), "Why it's interesting": NVFP4's
 *     element is E2M1; "How it works": the speculative verify reads each
 *     weight once for the whole tree, wide prefill reads it once for N
 *     tokens, and the draft tree descends by a dense argmax.
 *
 * Format.  NVFP4 = E2M1 element codes (bias 1, values 0, .5, 1, 1.5, 2, 3, 4,
 * 6 and their negatives), one E4M3 scale byte per 16 consecutive elements of
 * a row (OCP "FN": bias 7, subnormals, max 448, NaN only at 0x7F/0xFF), and
 * one fp32 tensor scale:  w_hat[r][k] = e2m1(code) * e4m3(scale) * tscale.
 *
 * Canonical layout (input of nvfp4_repack, output of nvfp4_quantize):
 *   codes  uint8 [rows][cols/2]:  element k of a row sits in byte k/2, in the
 *                                 low nibble when k is even, high when odd;
 *   scales uint8 [rows][cols/16]: scale of elements 16b..16b+15 at [r][b].
 *
 * Repacked layout (what the products read; "split-plane": codes and scales
 * are two separate planes).  Rows are grouped in tiles of 16 and tiles in
 * super-tiles of 4 (64 rows); the 16-element blocks of a row in octets of 8.
 * Let T = ceil(rows/16), ST = ceil(T/4), KB = cols/16, O = ceil(KB/8).
 *   code plane  uint8 [ST][O][4][64][16]: entry (st, o, tt, l), l = 16g + r
 *       (g = 0..3, r = 0..15), belongs to row 64st + 16tt + r; its bytes
 *       4d..4d+3 (d = 0..3) are the canonical code bytes of elements
 *       8h..8h+7 of block 8o + 2d + (g >> 1) of that row, h = g & 1 -- so
 *       word d of the entry holds elements 32(4o + d) + 8g .. +7 of the row;
 *   scale plane uint8 [ST][O][4][16][8]: entry (st, o, tt, r) byte i is the
 *       scale of block 8o + i of row 64st + 16tt + r;
 *   positions past the last row or block hold 0.
 * One tile's octet is a 1 KiB code chunk that a 64-lane wavefront reads with
 * one 128-bit load per lane, and its 16 rows' scales are 128 contiguous
 * bytes; each 32-bit word of a code entry is directly the weight operand of
 * one 16x16x32 MFMA (row r, elements 8g..8g+7 of a 32-element k slice), for
 * the matvec and the wide contraction alike.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device memory owned by the caller; the library
 *     allocates nothing, and the only state it keeps between calls are facts
 *     it looks up once per device (the CU count, the wide kernels' LDS limit,
 *     the address of nvfp4_gemv_argmax_noalloc's array).  Inputs must not be
 *     modified, and outputs not read, until the call's work on `stream` is
 *     done.  `stream` may be NULL (the null stream).
 *   - Calls are asynchronous and stream-ordered: arguments are validated on
 *     the host, kernels are enqueued on `stream`, and the call returns
 *     without waiting.  No host synchronisation, no device allocation.
 *   - Pointers to weights, activations and fp32 matrices must be 16-byte
 *     aligned (NVFP4_EALIGN otherwise).
 *   - NVFP4 rows are any whole number of 16-element blocks (cols % 16 == 0,
 *     MXFP4: cols % 32 == 0): the repacked planes zero-pad the last octet,
 *     and every kernel range-checks its activation loads, so no row length
 *     beyond whole scale blocks is required.
 *   - Activations X are bf16 bit patterns [n][cols] row-major; outputs Y are
 *     fp32 [n][rows] row-major (column c of the product is X[c], Y[c]).
 *   - Return value: NVFP4_OK or a negative NVFP4_E* code; nvfp4_strerror
 *     names it.  On an error nothing has been enqueued, except for
 *     NVFP4_EHIP (a launch failed; earlier launches of the call may have run).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OK 0
#define NVFP4_EINVAL (-1)     /* null pointer, n out of range, tscale not finite and > 0 */
#define NVFP4_ESHAPE (-2)     /* rows < 1, cols < 16, cols % 16 != 0, or a size overflows */
#define NVFP4_EALIGN (-3)     /* a pointer is not 16-byte aligned (2-/4-byte for outputs) */
#define NVFP4_EWORKSPACE (-4) /* workspace smaller than nvfp4_gemv_argmax_workspace_bytes */
#define NVFP4_EHIP (-5)       /* a kernel launch failed (e.g. no gfx950 device) */

/* Largest n accepted by the products (columns of X). */
#define NVFP4_MAX_N 65536

/* Human-readable name of a status code; a static string, never NULL. */
const char *nvfp4_strerror(int status);

/* Sizes in bytes of the repacked code and scale planes for a rows x cols
 * matrix (rows padded to 64, blocks to 8): ST * O * 4096 and ST * O * 512,
 * or 0 for an invalid shape. */
size_t nvfp4_repacked_code_bytes(int64_t rows, int64_t cols);
size_t nvfp4_repacked_scale_bytes(int64_t rows, int64_t cols);

/* Quantise fp32 W [rows][cols] (finite values) to canonical NVFP4.
 * Per 16-element block: scale = E4M3 nearest-even of amax / (6 * tscale),
 * saturating at 448; each code = sign bit of w | E2M1 nearest-even of
 * |w| / (scale * tscale), saturating at 6; a block whose scale is 0 gets all
 * zero codes.  The rounding decisions are exact (taken on fp64 quotients).
 * The pages re-encode higher-precision checkpoints to NVFP4 at load (bw24
 * wiki, feature list, safetensors-loader item); the rule above is the
 * common amax/6 block scaling.  codes [rows][cols/2], scales [rows][cols/16]. */
int nvfp4_quantize(const float *W, int64_t rows, int64_t cols, float tscale,
                   uint8_t *codes, uint8_t *scales, hipStream_t stream);

/* Canonical (codes, scales) -> repacked (wq, ws), a pure byte permutation
 * plus zero padding (bw24 wiki, feature list: "split-plane repack" of the
 * NVFP4 decode path; its safetensors loader repacks NVFP4 byte-exactly).
 * wq holds nvfp4_repacked_code_bytes(rows, cols) bytes, ws
 * nvfp4_repacked_scale_bytes(rows, cols); every byte of both is written. */
int nvfp4_repack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                 uint8_t *wq, uint8_t *ws, hipStream_t stream);

/* Dequantise a repacked matrix to canonical row-major outputs (either may be
 * NULL, not both):
 *   out_f32  [rows][cols] fp32: e2m1 * e4m3 * tscale rounded once to fp32;
 *   out_bf16 [rows][cols] bf16 bits: e2m1 * e4m3 (tensor scale excluded),
 *            exact because the product has at most 6 significant bits.
 * NaN scale bytes give NaN.  A verification export of the decode the
 * products use. */
int nvfp4_dequant(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                  float *out_f32, uint16_t *out_bf16, hipStream_t stream);

/* Y[c][r] = tscale * sum_k e2m1(code[r][k]) * e4m3(scale[r][k/16]) * X[c][k]
 * for c < n, r < rows (bw24 wiki, feature list: the NVFP4 decode matvec and
 * the batched K+1 verify; qwentin README, "How it works": each weight read
 * once for all columns; wide prefill for large n).
 * Products are exact in fp32 and accumulate in fp32 in a fixed order that
 * depends only on (rows, cols, n) and the device's CU count: results are
 * bitwise reproducible run to run; wherever the matvec runs, column c
 * equals, bit for bit, the n = 1 product of X[c], and wherever the MFMA
 * contraction runs, the same column of any wider contraction (bw24 wiki,
 * exactness note: summation order is part of the contract).  n <= 8 runs
 * the matvec (block dot products on MFMA, block scales and the running sum
 * in fp32 on the VALU; cols <= 2^26, else NVFP4_ESHAPE).  9 <= n <= 128
 * runs either the matvec in passes of up to eight columns (columns 0..7,
 * then 8..15, ...) or a dequant-to-bf16 MFMA tile contraction, whichever a
 * cost model of the two on the device's CU count estimates faster (the
 * contraction takes rows of at most 2^22 elements, the passes 2^26);
 * n > 128 runs the contraction (cols <= 2^22, else NVFP4_ESHAPE).
 * 1 <= n <= NVFP4_MAX_N.
 * X [n][cols] bf16 bits, Y [n][rows]. */
int nvfp4_gemv(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
               const uint16_t *X, int n, float *Y, hipStream_t stream);

/* Workspace bytes nvfp4_gemv_argmax needs for a rows x cols matrix and n
 * columns: a 1152-byte header for the finish, then one 64-bit key per
 * workgroup of the product and column (at most 4 bytes per row, rows rounded
 * up to a multiple of 64); 0 for an invalid shape or n out of 1..8.  It
 * takes the matrix shape as well as n because the product's workgroup count
 * follows the shape; a caller that sizes one workspace for every call of a
 * model uses its largest matrix and n = 8 (the header plus 4 bytes per row
 * bound that for every n). */
size_t nvfp4_gemv_argmax_workspace_bytes(int64_t rows, int64_t cols, int n);

/* nvfp4_gemv for 1 <= n <= 8 plus, per column c, argmax[c] = the lowest row
 * index of the largest Y[c][r] (-0 and +0 compare equal) -- the vocabulary
 * projection with the greedy token (bw24 wiki: prefill-argmax vs
 * decode-argmax gate; qwentin README, "How it works": dense-argmax descent).
 * Two launches: the product, whose workgroups each store, per column, the
 * largest (order-preserving value key, complemented row) of their rows to the
 * workspace, then a finish that reduces those keys to row indices: one
 * workgroup, or, above 6144 keys (12288 for n <= 2), 16 workgroups whose
 * partial maxima meet in the workspace header, where the last of them to
 * count itself on an atomic counter (zeroed by the product) reduces them.
 * A maximum does not depend on the order of its operands, so the result is
 * exact and the same on every run.
 * logits [n][rows] may be NULL (not stored).  workspace: device memory of at
 * least nvfp4_gemv_argmax_workspace_bytes(rows, cols, n) bytes, 8-byte
 * aligned, any contents; the call overwrites it.  Calls sharing a workspace
 * must not run concurrently. */
int nvfp4_gemv_argmax(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows,
                      int64_t cols, const uint16_t *X, int n, float *logits, int32_t *argmax,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Largest workspace nvfp4_gemv_argmax_noalloc serves: 1 MiB, enough for
 * every n <= 8 up to 262144 rows (at most 256 KiB and the header there) and,
 * at n = 8, for up to 1047424 rows of more than 4096 16-row tiles. */
#define NVFP4_ARGMAX_SCRATCH_BYTES (1u << 20)

/* nvfp4_gemv_argmax without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The keys
 * go to a static device array of NVFP4_ARGMAX_SCRATCH_BYTES that the library
 * holds on each GPU until the process ends (its address is looked up once per
 * device, on the first call there).  Same kernels, same results, bit for
 * bit, as nvfp4_gemv_argmax.  NVFP4_EWORKSPACE when
 * nvfp4_gemv_argmax_workspace_bytes(rows, cols, n) exceeds that size;
 * NVFP4_EHIP if the array's address cannot be found.  Every call on one GPU
 * shares its array: calls that may overlap on one GPU (several streams, or
 * several host threads) race and must be serialised by the caller.  The
 * array needs no clearing: each call writes every key it reads and zeroes
 * the finish's counter before the finish counts on it. */
int nvfp4_gemv_argmax_noalloc(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows,
                              int64_t cols, const uint16_t *X, int n, float *logits, int32_t *argmax,
                              hipStream_t stream);

/* ---------------------------------------------------- a batch of products
 * Several independent products of one activation matrix X [n][cols] in one
 * launch: the bw24 wiki's MTP item verifies K+1 draft tokens in one batched
 * forward, whose products of one input (the vocabulary head beside another
 * projection of the same hidden state, or the projections that share a
 * layer's input) need not wait for one another.  Product i computes
 * y = W_i X as nvfp4_gemv does (y may be NULL when argmax is set), and, with
 * argmax set, the per-column greedy index as nvfp4_gemv_argmax does.  Every
 * product's outputs are bit for bit those of its own call. */
typedef struct nvfp4_product {
    const uint8_t *wq;     /* repacked code plane (16-byte aligned) */
    const uint8_t *ws;     /* repacked scale plane (16-byte aligned) */
    float tscale;          /* fp32 tensor scale, finite and > 0 */
    int64_t rows;          /* output rows of W_i */
    float *y;              /* fp32 [n][rows], 4-byte aligned; NULL: not stored (argmax set) */
    int32_t *argmax;       /* NULL: a plain product; else int32 [n] greedy rows */
} nvfp4_product;

/* Largest batch of nvfp4_gemv_batch. */
#define NVFP4_MAX_BATCH 4

/* Workspace bytes of nvfp4_gemv_batch: each argmax product's finish header
 * (1152 bytes) and keys, one 64-bit key per workgroup and column (0 when no
 * product has argmax set, or for invalid arguments). */
size_t nvfp4_gemv_batch_workspace_bytes(const nvfp4_product *products, int count, int64_t cols, int n);

/* The products of `count` (1..NVFP4_MAX_BATCH) matrices of `cols` columns
 * with the same X (bf16 bits [n][cols], 1 <= n <= 8): one product launch
 * when the matrices' own decompositions split a row over the same number of
 * waves (true for the 17408 x 5120 matrix beside the 151936 x 5120
 * vocabulary head), else one launch per product; then one argmax finish per
 * argmax product.  workspace: nvfp4_gemv_batch_workspace_bytes bytes,
 * 8-byte aligned, any contents (NULL allowed when no argmax is asked).
 * The products' outputs must not overlap one another, X, the planes or the
 * workspace (the launches write them concurrently).  Errors as nvfp4_gemv /
 * nvfp4_gemv_argmax; NVFP4_EINVAL also for a count out of range or a
 * product with neither y nor argmax. */
int nvfp4_gemv_batch(const nvfp4_product *products, int count, int64_t cols, const uint16_t *X, int n,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* SwiGLU between the MLP matvecs: gu fp32 [n][2F] holds the stacked gate
 * (columns 0..F-1) and up (F..2F-1) outputs; h [n][F] bf16 bits =
 * bf16_nearest_even(g * u / (1 + exp(-g))) computed in fp32 (the pages'
 * persistent-MLP decode GEMV, qwentin README "How it works", runs this
 * step between its gate/up and down products).  1 <= n <= NVFP4_MAX_N,
 * F >= 1; gu 16-byte aligned, h 4-byte aligned. */
int nvfp4_swiglu(const float *gu, int64_t F, int n, uint16_t *h, hipStream_t stream);

/* The gate||up product of a decode MLP with SwiGLU in its epilogue, one
 * launch: for the stacked [2F][hidden] matrix (gate rows 0..F-1, up rows
 * F..2F-1), h[c][i] = bf16_nearest_even(SiLU(g) * u) in fp32 with
 * g = Y[c][i], u = Y[c][F + i] of nvfp4_gemv on that matrix.  gu, when not
 * NULL, receives Y itself (fp32 [n][2F]); h is bf16 [n][F].  Both are bit for
 * bit what nvfp4_gemv followed by nvfp4_swiglu give (the pages'
 * persistent-MLP decode GEMV, qwentin README "How it works", also keeps the
 * MLP's intermediate out of memory).  1 <= n <= 8; F a multiple of 16;
 * gu 4-byte and h 2-byte aligned.  One launch when F is a multiple of 64 and
 * the stacked product splits each row over at most 8 waves (true for the
 * 27B-class MLP, F = 17408, hidden = 5120); other shapes run the plain
 * product into gu (then required, else NVFP4_ESHAPE) and the SwiGLU kernel,
 * with the same bits. */
int nvfp4_gemv_swiglu(const uint8_t *wq_gu, const uint8_t *ws_gu, float tscale, int64_t hidden,
                      int64_t F, const uint16_t *X, int n, float *gu, uint16_t *h, hipStream_t stream);

/* ------------------------------------------------------------------ MXFP4
 * The second block-scaled format on the same layout and kernels: E2M1 codes
 * with one power-of-two E8M0 scale byte per 32 elements of a row, the
 * "E8M0-style" scale the pages set beside NVFP4 (bw24 wiki, feature list;
 * qwentin README, "Why it's interesting"), read as the OCP Microscaling
 * MXFP4 format.  Canonical layout: codes [rows][cols/2] (nibble order as
 * NVFP4), scales [rows][cols/32] (byte b means 2^(b - 127), 0xFF NaN);
 * cols % 32 == 0 (else NVFP4_ESHAPE).  Repacked layout: the NVFP4 code
 * plane of the same codes, and a scale plane [ST][O][4 tiles][16 rows][4 B]
 * whose entry (st, o, tt, r) byte i is the scale of 32-element block 4o + i
 * of row 64 st + 16 tt + r (zero past the matrix).  The fp32 tensor scale is
 * a multiplier as for NVFP4.  Error codes and conventions as above. */

/* Sizes of the repacked MXFP4 planes (0 for an invalid shape). */
size_t mxfp4_repacked_code_bytes(int64_t rows, int64_t cols);
size_t mxfp4_repacked_scale_bytes(int64_t rows, int64_t cols);

/* Quantise fp32 W [rows][cols] to canonical MXFP4.  Per 32-element block:
 * E = floor(log2(amax / tscale)) - 2, clamped to [-127, 127] (amax = 0 gives
 * -127), scale byte E + 127; code = sign bit of w | E2M1 nearest-even of
 * |w| / (2^E tscale), saturating at 6.  Decisions are exact (fp64). */
int mxfp4_quantize(const float *W, int64_t rows, int64_t cols, float tscale, uint8_t *codes,
                   uint8_t *scales, hipStream_t stream);

/* Canonical MXFP4 -> repacked (a byte permutation plus zero padding). */
int mxfp4_repack(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, uint8_t *wq,
                 uint8_t *ws, hipStream_t stream);

/* Dequantise repacked MXFP4: out_f32 = e2m1 * 2^(b - 127) * tscale rounded
 * once to fp32; out_bf16 = e2m1 * 2^(b - 127) (exact, infinite past bf16's
 * range); NaN scale bytes give NaN.  Either output may be NULL, not both. */
int mxfp4_dequant(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
                  float *out_f32, uint16_t *out_bf16, hipStream_t stream);

/* nvfp4_gemv for MXFP4 weights: the same products (n <= 8 the matvec with
 * each 32-element block's dot product on MFMA and its scale in fp32; 9..128
 * columns in passes of it or the dequant-to-bf16 MFMA contraction by the
 * same cost model as nvfp4_gemv; past 128 the contraction, decoding with one
 * scaled conversion per two elements), the same fixed summation order and
 * column identity.  Domain: the sums run in fp32 (the wide product's decoded
 * weights in bf16, the same exponent range) before the tensor scale, so a
 * weight whose e2m1 * 2^(b - 127) passes fp32's range (scale bytes 253 and
 * 254 with |e2m1| >= 4 resp. >= 2) makes its outputs infinite or NaN even
 * where tscale < 1 would bring the exact result back into range.  Subnormal
 * scales (bytes 0 and 1) are exact in both products. */
int mxfp4_gemv(const uint8_t *wq, const uint8_t *ws, float tscale, int64_t rows, int64_t cols,
               const uint16_t *X, int n, float *Y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
