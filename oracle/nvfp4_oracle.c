/*
 * nvfp4_oracle.c -- plain, slow fp64 CPU oracle for the NVFP4 weight x bf16
 * activation matrix-vector path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: every constant below is written out here from the format's
 * definition.
 *
 * Sources.  The pages this method comes from name the format but never spell
 * it out:
 *   - bw24 wiki (GitHub), feature list, "NVFP4 (W4) decode path" item:
 *     block-scaled FP4 weights read by a matvec for decode and by a wider
 *     GEMM for prefill; the same list appears in the bw24 README (wpnews page
 *     "Bw24 - from scratch rust+CUDA inference, every kernel tuned for
 *     sm_120a").
 *   - qwentin README (gitlite mirror), "Why it's interesting": its E2M1 4-bit
 *     weight mode sits in the NVFP4 quality class, i.e. the NVFP4 element is
 *     E2M1.
 *   - bw24 README / wiki, "FP8 (e4m3)" KV option and the qwentin README's
 *     "E4M3 V" cache: the FP8 flavour these engines use is E4M3.
 * The format this oracle implements is therefore: E2M1 4-bit element codes,
 * one E4M3 scale byte per 16 consecutive elements of a row, and one fp32
 * tensor scale.  Every reading the pages leave open (OCP "FN" E4M3, nibble
 * order, rounding, saturation, signed zero) is stated at the function that
 * takes it.
 *
 * Arithmetic.  Every E2M1, E4M3, bf16 and fp32 value is a dyadic rational
 * that fp64 holds exactly, and so is every product w_hat * x used here
 * (E2M1: 2 significant bits, E4M3: 4, fp32 tensor scale: 24, bf16: 8 -- at
 * most 38 bits).  Rounding happens only in the fp64 sums and where a
 * function says so.
 *
 * Row-parallel loops use OpenMP over output rows only; each row's k-sum is a
 * single sequential loop, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the row-parallel loops below use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of the row-parallel loops (timing only: every output is
 * one sequential k-sum, so results do not depend on the count). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- decode -- */

/* E2M1 code (4 bits) -> exact value.  Bit 3 sign, bits 2..1 exponent (bias 1),
 * bit 0 mantissa; exponent field 0 is subnormal (0 or 0.5).  No inf, no NaN.
 * Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * m;
    else
        mag = (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -mag : mag;
}

/* E4M3 byte -> exact value, OCP "FN" variant: bit 7 sign, bits 6..3 exponent
 * (bias 7), bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6); the
 * only NaNs are 0x7F and 0xFF; no infinities; largest finite 448 (0x7E). */
double oracle_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double mag;
    if ((byte & 0x7F) == 0x7F)
        return NAN;
    if (e == 0)
        mag = (m / 8.0) * ldexp(1.0, -6);
    else
        mag = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* bf16 bit pattern -> exact value (the fp32 whose upper half it is). */
double oracle_bf16_value(uint16_t u)
{
    uint32_t bits = (uint32_t)u << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------- encode -- */

/* Round a non-negative value q to the nearest E4M3 "FN" value, ties to the
 * even mantissa code, saturating at 448 and never producing NaN; subnormals
 * are kept.  Returns the byte (sign bit 0).
 *
 * Written as a search: walk the 127 finite non-negative codes in increasing
 * value order and pick the nearest, a tie going to the even code.  The
 * comparison uses midpoints between neighbours, which are exact in fp64. */
uint8_t oracle_e4m3_encode(double q)
{
    int best = 0;
    if (!(q > 0.0))
        return 0;
    if (q >= 448.0)
        return 0x7E;
    for (int c = 0; c < 0x7E; ++c) {
        double lo = oracle_e4m3_value(c);
        double hi = oracle_e4m3_value(c + 1);
        double mid = 0.5 * (lo + hi);          /* exact: both dyadic, 5 bits */
        if (q < mid) { best = c; break; }
        if (q == mid) { best = (c % 2 == 0) ? c : c + 1; break; }
        best = c + 1;
    }
    return (uint8_t)best;
}

/* Round a non-negative magnitude v to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}
 * with ties to the even code and saturation at 6.  Returns the 3-bit
 * magnitude code.  Midpoints between neighbours (0.25, 0.75, 1.25, 1.75, 2.5,
 * 3.5, 5) are exact in fp64. */
int oracle_e2m1_encode_mag(double v)
{
    for (int c = 0; c < 7; ++c) {
        double lo = oracle_e2m1_value(c);
        double hi = oracle_e2m1_value(c + 1);
        double mid = 0.5 * (lo + hi);
        if (v < mid) return c;
        if (v == mid) return (c % 2 == 0) ? c : c + 1;
    }
    return 7;
}

/* Quantise an fp32 matrix W[R][K] (row-major, K % 16 == 0) to NVFP4 in the
 * canonical layout:
 *   codes  [R][K/2]  byte k/2 of a row holds element k in its low nibble when
 *                    k is even and in its high nibble when k is odd;
 *   scales [R][K/16] one E4M3 byte per 16-element block, row-major.
 * Per block b of a row:  s_b = E4M3_RNE(amax_b / (6 * tscale))  (saturating
 * at 448), then  code_i = sign(w_i) | E2M1_RNE(|w_i| / (s_b * tscale)).
 * A block whose scale rounds to 0 gets all-zero codes.  The sign bit of a
 * code copies the sign bit of w (so a negative w rounding to 0 gives code 8).
 *
 * Decisions are taken on fp64 quotients.  fp64 is enough to make them
 * exactly: a quotient of two values with at most 24+3 and 24+4 significant
 * bits that is not exactly on a rounding midpoint lies at least 2^-32
 * relatively away from it, far more than one fp64 rounding (2^-53). */
void oracle_quantize(const float *W, int64_t R, int64_t K, float tscale,
                     uint8_t *codes, uint8_t *scales)
{
    int64_t KB = K / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            const float *w = W + r * K + b * 16;
            double amax = 0.0;
            for (int i = 0; i < 16; ++i) {
                double a = fabs((double)w[i]);
                if (a > amax) amax = a;
            }
            uint8_t sb = oracle_e4m3_encode(amax / (6.0 * (double)tscale));
            scales[r * KB + b] = sb;
            double denom = oracle_e4m3_value(sb) * (double)tscale;
            for (int i = 0; i < 16; i += 2) {
                int c[2];
                for (int h = 0; h < 2; ++h) {
                    if (sb == 0) { c[h] = 0; continue; }
                    double v = fabs((double)w[i + h]) / denom;
                    c[h] = oracle_e2m1_encode_mag(v) | (signbit(w[i + h]) ? 8 : 0);
                }
                codes[r * (K / 2) + b * 8 + i / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* ------------------------------------------------------- dequant / gemv -- */

/* Exact dequantised value of element (r, k): e2m1(code) * e4m3(scale) * tscale. */
static double w_hat(const uint8_t *codes, const uint8_t *scales, float tscale,
                    int64_t K, int64_t r, int64_t k)
{
    uint8_t byte = codes[r * (K / 2) + k / 2];
    int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
    return oracle_e2m1_value(code) * oracle_e4m3_value(scales[r * (K / 16) + k / 16])
           * (double)tscale;
}

/* out[r][k] = exact w_hat (fp64 holds it exactly). */
void oracle_dequant(const uint8_t *codes, const uint8_t *scales, float tscale,
                    int64_t R, int64_t K, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = w_hat(codes, scales, tscale, K, r, k);
}

/* Matrix-vector product for a list of output rows.
 *   X    bf16 bit patterns [N][K] row-major (column n of the product is X[n]);
 *   rows the nrows output rows to compute (each in [0, R));
 *   Y    [N][nrows]:  Y[n][i] = sum_k w_hat[rows[i]][k] * x_n[k], fp64, k ascending;
 *   S    [N][nrows]:  S[n][i] = sum_k |w_hat[rows[i]][k] * x_n[k]|  (the
 *        magnitude sum that scales the parity tolerance); may be NULL. */
void oracle_gemv_rows(const uint8_t *codes, const uint8_t *scales, float tscale,
                      int64_t R, int64_t K, const uint16_t *X, int64_t N,
                      const int64_t *rows, int64_t nrows, double *Y, double *S)
{
    (void)R;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        for (int64_t n = 0; n < N; ++n) {
            double y = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = w_hat(codes, scales, tscale, K, r, k)
                           * oracle_bf16_value(X[n * K + k]);
                y += p;
                s += fabs(p);
            }
            Y[n * nrows + i] = y;
            if (S) S[n * nrows + i] = s;
        }
    }
}

/* ---------------------------------------------------------------- swiglu -- */

/* SiLU(gate) * up in fp64 for gate||up rows stacked as gu[N][2F] (gate in
 * columns 0..F-1, up in F..2F-1):  h[n][i] = g * u / (1 + exp(-g)). */
void oracle_swiglu(const float *gu, int64_t F, int64_t N, double *h)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < F; ++i) {
            double g = gu[n * 2 * F + i];
            double u = gu[n * 2 * F + F + i];
            h[n * F + i] = g * u / (1.0 + exp(-g));
        }
}

/* fp64 -> bf16 bit pattern, round to nearest, ties to even (finite input,
 * result within bf16 range).  Written on the value: find the bf16 grid
 * spacing at v and round v / spacing with rint (fp64 default mode is
 * round-to-nearest-even; the division by a power of two is exact). */
uint16_t oracle_bf16_rne(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    int e;
    frexp(a, &e);                       /* a = f * 2^e, f in [0.5, 1) */
    int ulp_exp = e - 8;                /* bf16 has 8 significant bits */
    if (ulp_exp < -133) ulp_exp = -133; /* subnormal spacing 2^-133 */
    double q = rint(ldexp(a, -ulp_exp));
    double r = ldexp(q, ulp_exp);
    float f = (float)r;                 /* exact: r is a bf16 value */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t out = (uint16_t)(bits >> 16);
    return signbit(v) ? (uint16_t)(out | 0x8000) : out;
}

/* ---------------------------------------------------------------- repack -- */

/* Reference of the library's repacked ("split-plane") layout, written from
 * its published definition, not from the library's code.  The definition:
 *   rows are grouped in tiles of 16 and tiles in super-tiles of 4 (64
 *   rows); the 16-element blocks of a row are grouped in octets of 8;
 *   T = ceil(R/16), ST = ceil(T/4), KB = K/16, O = ceil(KB/8);
 *   code plane  [ST][O][4][64][16 bytes]: entry (st, o, tt, l), with
 *     l = 16g + r (g = 0..3, r = 0..15), belongs to row 64st + 16tt + r; its
 *     bytes 4d..4d+3 (d = 0..3) are the 4 canonical code bytes holding
 *     elements 8h..8h+7 of block b = 8o + 2d + (g >> 1) of that row, with
 *     h = g & 1;
 *   scale plane [ST][O][4][16][8 bytes]: entry (st, o, tt, r) byte i is the
 *     scale of block 8o + i of row 64st + 16tt + r;
 *   positions past the last row or block hold 0.
 * The inverse is checked separately. */
void oracle_repack(const uint8_t *codes, const uint8_t *scales, int64_t R, int64_t K,
                   uint8_t *wq, uint8_t *ws)
{
    int64_t KB = K / 16;
    int64_t T = (R + 15) / 16;
    int64_t ST = (T + 3) / 4;
    int64_t O = (KB + 7) / 8;
    memset(wq, 0, (size_t)(ST * O * 4 * 64 * 16));
    memset(ws, 0, (size_t)(ST * O * 4 * 16 * 8));
    for (int64_t row = 0; row < R; ++row) {
        int64_t st = row / 64, tt = (row % 64) / 16, r = row % 16;
        for (int64_t b = 0; b < KB; ++b) {
            int64_t o = b / 8, ib = b % 8;     /* octet, block within the octet */
            int64_t d = ib / 2, par = ib % 2;  /* block pair, parity within it */
            for (int64_t h = 0; h < 2; ++h) {
                int64_t g = 2 * par + h, l = 16 * g + r;
                uint8_t *dst = wq + (((st * O + o) * 4 + tt) * 64 + l) * 16 + 4 * d;
                memcpy(dst, codes + row * (K / 2) + 8 * b + 4 * h, 4);
            }
            ws[(((st * O + o) * 4 + tt) * 16 + r) * 8 + ib] = scales[row * KB + b];
        }
    }
}

/* ============================================================== MXFP4 -- */
/*
 * The second block-scaled format on the same skeleton: E2M1 element codes
 * with one power-of-two scale per 32 consecutive elements of a row, the
 * "E8M0-style" scale the pages set beside NVFP4 (bw24 wiki, feature list:
 * the E2M1 weight class; qwentin README, "Why it's interesting").  The
 * pages do not define it; the plainest reading is the OCP Microscaling (MX)
 * MXFP4 format, which this part implements:
 *   element  E2M1 code, as above;
 *   scale    E8M0 byte b: 2^(b - 127); b = 0xFF is NaN; no sign, no zero;
 *   block    32 consecutive elements of a row; canonical layout
 *            codes [R][K/2] (nibble order as NVFP4), scales [R][K/32];
 *   tensor   one fp32 multiplier, as for NVFP4 (1.0 in every workload).
 */

/* E8M0 byte -> exact value 2^(b - 127); 0xFF is NaN. */
double oracle_e8m0_value(int byte)
{
    if ((byte & 0xFF) == 0xFF)
        return NAN;
    return ldexp(1.0, (byte & 0xFF) - 127);
}

/* Quantise an fp32 matrix W[R][K] (row-major, K % 32 == 0) to MXFP4 in the
 * canonical layout.  Per 32-element block of a row, following the MX
 * definition's conversion of a vector to one shared scale:
 *   q = amax / tscale;  E = floor(log2 q) - 2  (2 = the largest exponent of
 *   an E2M1 value, 6 = 1.5 * 2^2), clamped to [-127, 127]; q = 0 gives
 *   E = -127;  scale byte = E + 127;
 *   code_i = sign(w_i) | E2M1_RNE(|w_i| / (2^E * tscale))  (ties to even,
 *   saturating at 6: a block's largest element lies in [4, 8) * 2^E, so
 *   values above 6 * 2^E clip to 6).
 * floor(log2 q) is read exactly off the fp64 exponent of q (frexp); q is a
 * quotient of two fp32 values, so it is exactly a power of two or at least
 * 2^-24 relatively away from one, and fp64 keeps that side.  The element
 * quotient is decided as in oracle_quantize. */
void oracle_mx_quantize(const float *W, int64_t R, int64_t K, float tscale,
                        uint8_t *codes, uint8_t *scales)
{
    int64_t KB = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            const float *w = W + r * K + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                double a = fabs((double)w[i]);
                if (a > amax) amax = a;
            }
            double q = amax / (double)tscale;
            int E;
            if (q > 0.0) {
                int e;
                frexp(q, &e);            /* q = f * 2^e, f in [0.5, 1): floor(log2 q) = e - 1 */
                E = (e - 1) - 2;
                if (E < -127) E = -127;
                if (E > 127) E = 127;
            } else {
                E = -127;
            }
            scales[r * KB + b] = (uint8_t)(E + 127);
            double denom = ldexp(1.0, E) * (double)tscale;
            for (int i = 0; i < 32; i += 2) {
                int c[2];
                for (int h = 0; h < 2; ++h) {
                    double v = fabs((double)w[i + h]) / denom;
                    c[h] = oracle_e2m1_encode_mag(v) | (signbit(w[i + h]) ? 8 : 0);
                }
                codes[r * (K / 2) + b * 16 + i / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* Exact dequantised MXFP4 element (r, k): e2m1(code) * e8m0(scale) * tscale. */
static double mx_w_hat(const uint8_t *codes, const uint8_t *scales, float tscale,
                       int64_t K, int64_t r, int64_t k)
{
    uint8_t byte = codes[r * (K / 2) + k / 2];
    int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
    return oracle_e2m1_value(code) * oracle_e8m0_value(scales[r * (K / 32) + k / 32])
           * (double)tscale;
}

void oracle_mx_dequant(const uint8_t *codes, const uint8_t *scales, float tscale,
                       int64_t R, int64_t K, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = mx_w_hat(codes, scales, tscale, K, r, k);
}

/* As oracle_gemv_rows, for MXFP4 weights. */
void oracle_mx_gemv_rows(const uint8_t *codes, const uint8_t *scales, float tscale,
                         int64_t R, int64_t K, const uint16_t *X, int64_t N,
                         const int64_t *rows, int64_t nrows, double *Y, double *S)
{
    (void)R;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        for (int64_t n = 0; n < N; ++n) {
            double y = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = mx_w_hat(codes, scales, tscale, K, r, k)
                           * oracle_bf16_value(X[n * K + k]);
                y += p;
                s += fabs(p);
            }
            Y[n * nrows + i] = y;
            if (S) S[n * nrows + i] = s;
        }
    }
}

/* Reference of the library's MXFP4 repacked layout, from its published
 * definition: the code plane is the NVFP4 code plane of the same codes
 * (tiles of 16 rows, super-tiles of 4 tiles, octets of 128 elements; entry
 * (st, o, tt, l = 16g + r) bytes 4d..4d+3 hold elements
 * 32(4o + d) + 8g .. +7 of row 64st + 16tt + r, i.e. the code bytes
 * 16(4o + d) + 4g .. +3 of that row); the scale plane is
 * [ST][O][4][16][4 bytes]: entry (st, o, tt, r) byte i is the scale of
 * 32-element block 4o + i of that row; O = ceil(K / 128); positions past
 * the last row or block hold 0. */
void oracle_mx_repack(const uint8_t *codes, const uint8_t *scales, int64_t R, int64_t K,
                      uint8_t *wq, uint8_t *ws)
{
    int64_t KB = K / 32;
    int64_t T = (R + 15) / 16;
    int64_t ST = (T + 3) / 4;
    int64_t O = (K + 127) / 128;
    memset(wq, 0, (size_t)(ST * O * 4 * 64 * 16));
    memset(ws, 0, (size_t)(ST * O * 4 * 16 * 4));
    for (int64_t row = 0; row < R; ++row) {
        int64_t st = row / 64, tt = (row % 64) / 16, r = row % 16;
        for (int64_t j = 0; j < K / 32; ++j) {          /* 32-element slice */
            int64_t o = j / 4, d = j % 4;
            for (int64_t g = 0; g < 4; ++g) {
                int64_t l = 16 * g + r;
                uint8_t *dst = wq + (((st * O + o) * 4 + tt) * 64 + l) * 16 + 4 * d;
                memcpy(dst, codes + row * (K / 2) + 16 * j + 4 * g, 4);
            }
        }
        for (int64_t b = 0; b < KB; ++b)
            ws[(((st * O + b / 4) * 4 + tt) * 16 + r) * 4 + b % 4] = scales[row * KB + b];
    }
}
