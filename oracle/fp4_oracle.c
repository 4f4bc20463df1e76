/*
 * fp4_oracle.c -- the CPU oracle for block-wise microscaling FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, loop-by-loop statement
 * of what the quantization path computes.  It is built into liboracle.so and
 * called by the tests, by the package smoke check and by the benchmark's
 * cpu_baseline leg.  The product path (the HIP library) never links, loads or
 * calls it, and shares no header, table or helper with it.
 *
 * Sources (web pages summarising three papers):
 *   [DIAG]  "Diagnosing FP4 inference: a layer-wise and block-wise sensitivity
 *           analysis of NVFP4 and MXFP4" -- technical summary, section 2
 *           (Metodologia / Methodology): MXFP4 = 32-element blocks sharing an
 *           8-bit exponent over E2M1 elements; NVFP4 = 16-element blocks with
 *           dynamic scaling and "max" calibration; weights are quantized on the
 *           fly and dequantized for the compute.
 *   [MRGPTQ] "Bridging the Gap Between Promise and Performance for Microscaling
 *           FP4 Quantization" -- Sommario tecnico section 1 (RTN; E8M0
 *           power-of-two scales for MXFP4, E4M3 scales for NVFP4), section 2
 *           (dead zone of E8M0 scales; rotation spreads the block maximum),
 *           section 3 item 1 (block-wise Hadamard rotations).
 *   [FINER] "Is finer better? Limits of micro-scaling formats in LLMs" --
 *           Metodologia, Framework Teorico (three error sources: non-maximum
 *           elements, the block maximum, zero-rounding of the whole block;
 *           smallest non-zero UE4M3 scale 2^-9), Contributi Chiave item 3
 *           (UE5M3: smallest non-zero scale 2^-17, no per-tensor scale),
 *           Risultati (UE4M3-S = UE4M3 with a per-tensor scale).
 *
 * Where the pages leave a step open, the reading taken here is stated at the
 * function that takes it.  Every reading is one of:
 *   R1  E2M1 magnitudes are {0, .5, 1, 1.5, 2, 3, 4, 6}; round to nearest, an
 *       exact tie goes to the even 3-bit code, values past 6 saturate to 6,
 *       and the sign bit is kept even when the magnitude rounds to 0.
 *   R2  MXFP4 exponent E = floor(log2 m) - 2 (2 = largest E2M1 exponent),
 *       clamped to [-127, 127]; all-zero block -> E = -127 (byte 0x00).
 *   R3  UE4M3 scale: s = m / (6 g) in binary32, rounded to nearest UE4M3 value
 *       (ties to the even code), saturating at 448; d = s_hat * g in binary32;
 *       element y = x / d in binary32.  Dynamic per-tensor scale
 *       g = amax / (6 * 448) in binary32 (1 if that is 0).
 *   R4  Blocks run along a row (consecutive elements of the contiguous
 *       dimension).  Packing: element 2j in the low nibble of byte j.
 *   R5  Rotation: Sylvester-ordered Walsh-Hadamard butterfly in binary32,
 *       stages h = 1, 2, 4, ... in that order, then multiply by RN32(n^-1/2).
 *   R6  Error terms in binary64: block max m = max |x_i|, i* = lowest index
 *       attaining it; a Z-block has m > 0 and every dequantized value 0 (all
 *       its squared error is zero-rounding error); otherwise the i* squared
 *       error is the max-element term and the rest is the non-max term.
 *       Per-block MSE = SSE/b (absolute) or SSE/sum(x^2) (relative).
 *   R7  UE5M3 (unsigned, 5 exponent bits, 3 mantissa bits, bias 15): values
 *       j*2^-17 (e = 0) and (1 + j/8)*2^(e-15) (e = 1..30); exponent 31 is
 *       reserved; largest value 1.875 * 2^15 = 61440.
 *   R8  Scale search: the max-based code and its neighbours within a radius,
 *       scored by block SSE, visited nearest first, replaced only when better
 *       by more than a relative 2^-40 (see oracle_quantize_search).
 *   R9  Per-row dynamic scale (activations, one row per token): g_r =
 *       RN32(amax_r / 2688) from the row's own (rotated) maximum, 1 when that
 *       is 0; the row is then quantized exactly as under a given g = g_r.
 *   R10 FP4 GEMM: C = A_hat B_hat^T from the exactly dequantized MXFP4 operands,
 *       summed in binary64 (see oracle_gemm_mxfp4).
 *   R11 NVFP4 GEMM: the same product of two NVFP4 operands (blocks of 16,
 *       UE4M3 scale bytes, a per-tensor g each), taken on their dequantized
 *       binary32 values x_hat = RN32(v * RN32(s_hat * g)) -- the values
 *       oracle_dequantize returns -- and summed in binary64 (see
 *       oracle_gemm_nvfp4).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* Format identifiers; the same numeric values as the library's public enum
 * (an interface both sides follow, not shared code). */
#define FMT_MXFP4 0 /* E8M0 scale, block 32 */
#define FMT_UE4M3 1 /* NVFP4-style UE4M3 scale, any block size */
#define FMT_UE5M3 2 /* UE5M3 scale, no per-tensor scale */

#define GMODE_NONE 0
#define GMODE_DYNAMIC 1
#define GMODE_GIVEN 2
#define GMODE_ROW 3

#define MSE_ABS 0
#define MSE_REL 1

/* ------------------------------------------------------------------------ */
/* R1: E2M1 element code.  [DIAG] section 2 names E2M1; [MRGPTQ] section 1  */
/* names round-to-nearest.                                                  */
/* ------------------------------------------------------------------------ */

static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* 3-bit magnitude code of |y| (y exact).  Nearest grid value; on an exact tie
 * between two neighbours the even code wins; everything at or past 6 maps to 6. */
int oracle_e2m1_magnitude(double a)
{
    if (a < 0.0) a = -a;
    if (a >= 6.0) return 7; /* saturate (the nearest grid value is 6) */
    int best = 0;
    double best_dist = a; /* distance to grid value 0 */
    for (int k = 1; k < 8; ++k) {
        double dist = fabs(a - E2M1_MAGNITUDE[k]); /* exact: a < 6, a has 24 bits */
        if (dist < best_dist || (dist == best_dist && (k % 2) == 0)) {
            best = k;
            best_dist = dist;
        }
    }
    return best;
}

/* Full 4-bit code of the value y: sign bit (taken from y, so -0 -> 0x8) over
 * the magnitude code. */
int oracle_e2m1_code(double y)
{
    int sign = signbit(y) ? 1 : 0;
    return (sign << 3) | oracle_e2m1_magnitude(y);
}

/* Value of a 4-bit code. */
double oracle_e2m1_value(int code)
{
    double v = E2M1_MAGNITUDE[code & 7];
    return (code & 8) ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* R2: MXFP4 shared exponent (E8M0).  [MRGPTQ] section 1: power-of-two      */
/* scales; [DIAG] section 2: a shared 8-bit exponent per 32 elements.       */
/* ------------------------------------------------------------------------ */

int oracle_e8m0_exponent(float m)
{
    if (!(m > 0.0f)) return -127;
    int k;
    (void)frexp((double)m, &k); /* m = f * 2^k with f in [1/2, 1) */
    int e = (k - 1) - 2;        /* floor(log2 m) minus the top E2M1 exponent */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------------ */
/* R3: UE4M3 block scales.  [MRGPTQ] section 1 (E4M3 scales); [FINER]      */
/* Framework Teorico (unsigned E4M3, smallest non-zero value 2^-9).         */
/* ------------------------------------------------------------------------ */

/* Value of a UE4M3 byte 0x00..0x7E (sign bit always clear, 0x7F is NaN). */
double oracle_ue4m3_value(int byte)
{
    int e = (byte >> 3) & 15, j = byte & 7;
    if (e == 0) return ldexp((double)j, -9);
    return ldexp(1.0 + j / 8.0, e - 7);
}

/* Nearest UE4M3 value to s >= 0 by enumeration of all 127 finite codes; an
 * exact tie goes to the even code; anything past 448 saturates to 448. */
int oracle_ue4m3_byte(float s)
{
    double sv = (double)s;
    if (sv >= 448.0) return 0x7E; /* saturate (the nearest value is 448) */
    int best = 0;
    double best_dist = fabs(sv - oracle_ue4m3_value(0));
    for (int c = 1; c <= 0x7E; ++c) {
        double dist = fabs(sv - oracle_ue4m3_value(c));
        if (dist < best_dist || (dist == best_dist && (c % 2) == 0)) {
            best = c;
            best_dist = dist;
        }
    }
    return best;
}

/* R7: UE5M3 values, [FINER] Contributi Chiave item 3. */
double oracle_ue5m3_value(int byte)
{
    int e = (byte >> 3) & 31, j = byte & 7;
    if (e == 0) return ldexp((double)j, -17);
    return ldexp(1.0 + j / 8.0, e - 15);
}

/* Nearest UE5M3 value (codes 0x00..0xF7), ties to the even code, saturating
 * at 61440. */
int oracle_ue5m3_byte(float s)
{
    double sv = (double)s;
    if (sv >= 61440.0) return 0xF7; /* saturate (the nearest value is 61440) */
    int best = 0;
    double best_dist = fabs(sv - oracle_ue5m3_value(0));
    for (int c = 1; c <= 0xF7; ++c) {
        double dist = fabs(sv - oracle_ue5m3_value(c));
        if (dist < best_dist || (dist == best_dist && (c % 2) == 0)) {
            best = c;
            best_dist = dist;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------ */
/* R5: block Hadamard rotation, [MRGPTQ] section 3 item 1 and section 2.    */
/* ------------------------------------------------------------------------ */

/* RN32(n^-1/2) for n = 16 (exactly 1/4) and n = 32. */
static float hadamard_norm(int n)
{
    return (float)(1.0 / sqrt((double)n));
}

/* In-place normalised Sylvester Walsh-Hadamard transform of n = 16 or 32
 * binary32 values: butterfly stages h = 1, 2, 4, ..., n/2 in that order, then
 * one multiplication by RN32(n^-1/2).  The map is its own inverse. */
void oracle_hadamard_block(float* a, int n)
{
    for (int h = 1; h < n; h *= 2) {
        for (int i = 0; i < n; ++i) {
            if (i & h) continue;
            float u = a[i], v = a[i + h];
            a[i] = u + v;
            a[i + h] = u - v;
        }
    }
    float c = hadamard_norm(n);
    for (int i = 0; i < n; ++i) a[i] = a[i] * c;
}

/* Rotate every block of every row: x is rows x cols row-major. */
int oracle_hadamard(const float* x, int64_t rows, int64_t cols, int n, float* out)
{
    if (n != 16 && n != 32) return ORACLE_BAD_ARG;
    if (cols % n != 0) return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c0 = 0; c0 < cols; c0 += n) {
            float blk[32];
            for (int i = 0; i < n; ++i) blk[i] = x[r * cols + c0 + i];
            oracle_hadamard_block(blk, n);
            for (int i = 0; i < n; ++i) out[r * cols + c0 + i] = blk[i];
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-block quantization.                                                  */
/* ------------------------------------------------------------------------ */

/* Scale description of one block: the byte stored, the exponent (MXFP4) or
 * the decode scale d (UE4M3/UE5M3). */
typedef struct {
    int byte;
    int exponent; /* MXFP4 only */
    float d;      /* UE4M3 / UE5M3 only: RN32(s_hat * g) */
} block_scale;

static float block_absmax(const float* x, int b)
{
    float m = 0.0f;
    for (int i = 0; i < b; ++i) {
        float a = fabsf(x[i]);
        if (a > m) m = a;
    }
    return m;
}

static block_scale scale_for_block(int fmt, float m, float g)
{
    block_scale s = {0, 0, 0.0f};
    if (fmt == FMT_MXFP4) {
        s.exponent = oracle_e8m0_exponent(m);
        s.byte = s.exponent + 127;
    } else if (fmt == FMT_UE4M3) {
        float D = 6.0f * g;      /* maps the block max onto the top E2M1 value */
        float sv = m / D;        /* binary32 division */
        s.byte = oracle_ue4m3_byte(sv);
        s.d = (float)oracle_ue4m3_value(s.byte) * g;
    } else { /* FMT_UE5M3: g is 1 by construction of the format */
        float D = 6.0f * g;
        float sv = m / D;
        s.byte = oracle_ue5m3_byte(sv);
        s.d = (float)oracle_ue5m3_value(s.byte) * g;
    }
    return s;
}

static block_scale scale_from_byte(int fmt, int byte, float g)
{
    block_scale s = {byte, 0, 0.0f};
    if (fmt == FMT_MXFP4) {
        s.exponent = byte - 127;
    } else if (fmt == FMT_UE4M3) {
        s.d = (float)oracle_ue4m3_value(byte) * g;
    } else {
        s.d = (float)oracle_ue5m3_value(byte) * g;
    }
    return s;
}

/* Code of one element x under the block's scale. */
static int element_code(int fmt, float x, block_scale s)
{
    if (fmt == FMT_MXFP4) {
        double y = ldexp((double)x, -s.exponent); /* exact: power-of-two scale */
        return oracle_e2m1_code(y);
    }
    if (s.d == 0.0f) /* zero scale: every magnitude is 0, sign kept */
        return signbit(x) ? 8 : 0;
    float y = x / s.d; /* binary32 division */
    return oracle_e2m1_code((double)y);
}

/* Dequantized value of one code (binary32). */
static float element_value(int fmt, int code, block_scale s)
{
    double v = oracle_e2m1_value(code);
    if (fmt == FMT_MXFP4) return (float)ldexp(v, s.exponent); /* exact */
    float vf = (float)v;
    return vf * s.d; /* binary32 product */
}

/* R6: error terms of one block.  x are the (rotated, if rotating) values the
 * codes were taken from; xh their dequantized values.  Adds into acc[0..3] =
 * {non-max, max-element, zero-rounding, sum x^2}, cnt[0..1] = {blocks,
 * zero-rounded blocks}; returns the block's MSE as binary32. */
static float block_error(const float* x, const float* xh, int b, int mse_kind,
                         double* acc, int64_t* cnt)
{
    float m = block_absmax(x, b);
    int istar = 0;
    for (int i = 0; i < b; ++i) {
        if (fabsf(x[i]) == m) { istar = i; break; }
    }
    int all_zero = 1;
    for (int i = 0; i < b; ++i)
        if (xh[i] != 0.0f) all_zero = 0;
    int zero_block = (m > 0.0f) && all_zero;

    double sse = 0.0, nonmax = 0.0, sumsq = 0.0;
    for (int i = 0; i < b; ++i) {
        double e = (double)x[i] - (double)xh[i];
        sse += e * e;
        if (i != istar) nonmax += e * e;
        sumsq += (double)x[i] * (double)x[i];
    }
    double emax = (double)x[istar] - (double)xh[istar];
    if (acc) {
        if (zero_block) {
            acc[2] += sse;
        } else {
            acc[0] += nonmax;
            acc[1] += emax * emax;
        }
        acc[3] += sumsq;
    }
    if (cnt) {
        cnt[0] += 1;
        cnt[1] += zero_block;
    }
    if (mse_kind == MSE_REL) return sumsq > 0.0 ? (float)(sse / sumsq) : 0.0f;
    return (float)(sse / (double)b);
}

/* Largest |x| over the whole tensor (over the rotated blocks when rotating). */
float oracle_tensor_amax(const float* x, int64_t rows, int64_t cols, int rotate)
{
    float amax = 0.0f;
    if (rotate == 0) {
        for (int64_t i = 0; i < rows * cols; ++i)
            if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
        return amax;
    }
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c0 = 0; c0 < cols; c0 += rotate) {
            float blk[32];
            for (int i = 0; i < rotate; ++i) blk[i] = x[r * cols + c0 + i];
            oracle_hadamard_block(blk, rotate);
            for (int i = 0; i < rotate; ++i)
                if (fabsf(blk[i]) > amax) amax = fabsf(blk[i]);
        }
    }
    return amax;
}

/* R3: per-tensor scale for the dynamic mode ([FINER] Risultati, UE4M3-S). */
float oracle_dynamic_g(float amax)
{
    float g = amax / 2688.0f; /* 2688 = 6 * 448 */
    if (!(g > 0.0f)) g = 1.0f;
    return g;
}

static int valid_shape(int fmt, int block, int64_t rows, int64_t cols, int rotate)
{
    if (rows < 0 || cols < 0) return 0;
    if (fmt == FMT_MXFP4 && block != 32) return 0;
    if (block != 8 && block != 16 && block != 32 && block != 64 && block != 128 && block != 256)
        return 0;
    if (cols % block != 0) return 0;
    if (rotate != 0 && rotate != block) return 0;
    if (rotate != 0 && rotate != 16 && rotate != 32) return 0;
    return 1;
}

/*
 * Quantize a rows x cols row-major tensor in blocks of `block` along each row.
 *   fmt      FMT_MXFP4 (block must be 32), FMT_UE4M3 or FMT_UE5M3
 *   gmode    per-tensor scale for UE4M3: NONE (1), DYNAMIC (from amax, written
 *            to *g), GIVEN (read from *g).  UE5M3 and MXFP4 use none.
 *   rotate   0, or the Hadamard size (must equal block, 16 or 32)
 *   codes    rows*cols/2 bytes, element 2j in the low nibble of byte j
 *   scales   rows*cols/block bytes
 *   block_mse (may be NULL) rows*cols/block floats
 *   acc      (may be NULL) 4 doubles {non-max, max, zero-rounding, sum x^2}
 *   cnt      (may be NULL) 2 int64 {blocks, zero-rounded blocks}
 */
int oracle_quantize(const float* x, int64_t rows, int64_t cols, int fmt, int block,
                    int gmode, float* g, int rotate, uint8_t* codes, uint8_t* scales,
                    float* block_mse, int mse_kind, double* acc, int64_t* cnt)
{
    if (!valid_shape(fmt, block, rows, cols, rotate)) return ORACLE_BAD_ARG;
    if (fmt != FMT_UE4M3 && gmode != GMODE_NONE) return ORACLE_BAD_ARG;
    if (gmode == GMODE_ROW) {
        /* R9: every row under its own dynamic scale, written to g[row]. */
        if (!g) return ORACLE_BAD_ARG;
        if (acc) memset(acc, 0, 4 * sizeof(double));
        if (cnt) memset(cnt, 0, 2 * sizeof(int64_t));
        int64_t nblk_row = cols / block;
        for (int64_t r = 0; r < rows; ++r) {
            double racc[4];
            int64_t rcnt[2];
            g[r] = oracle_dynamic_g(oracle_tensor_amax(x + r * cols, 1, cols, rotate));
            int rc = oracle_quantize(x + r * cols, 1, cols, fmt, block, GMODE_GIVEN, g + r, rotate,
                                     codes + r * cols / 2, scales + r * nblk_row,
                                     block_mse ? block_mse + r * nblk_row : NULL, mse_kind,
                                     racc, rcnt);
            if (rc) return rc;
            if (acc) for (int k = 0; k < 4; ++k) acc[k] += racc[k];
            if (cnt) for (int k = 0; k < 2; ++k) cnt[k] += rcnt[k];
        }
        return ORACLE_OK;
    }
    float gv = 1.0f;
    if (fmt == FMT_UE4M3) {
        if (gmode == GMODE_DYNAMIC) {
            gv = oracle_dynamic_g(oracle_tensor_amax(x, rows, cols, rotate));
            if (g) *g = gv;
        } else if (gmode == GMODE_GIVEN) {
            if (!g) return ORACLE_BAD_ARG;
            gv = *g;
        }
    }
    if (acc) memset(acc, 0, 4 * sizeof(double));
    if (cnt) memset(cnt, 0, 2 * sizeof(int64_t));
    int64_t nblk_row = cols / block;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < nblk_row; ++k) {
            const float* src = x + r * cols + k * block;
            float v[256], xh[256];
            int cd[256];
            for (int i = 0; i < block; ++i) v[i] = src[i];
            if (rotate) oracle_hadamard_block(v, rotate);
            block_scale s = scale_for_block(fmt, block_absmax(v, block), gv);
            for (int i = 0; i < block; ++i) {
                cd[i] = element_code(fmt, v[i], s);
                xh[i] = element_value(fmt, cd[i], s);
            }
            scales[r * nblk_row + k] = (uint8_t)s.byte;
            for (int i = 0; i < block; i += 2) {
                int64_t byte_idx = (r * cols + k * block + i) / 2;
                codes[byte_idx] = (uint8_t)(cd[i] | (cd[i + 1] << 4));
            }
            float mse = block_error(v, xh, block, mse_kind, acc, cnt);
            if (block_mse) block_mse[r * nblk_row + k] = mse;
        }
    }
    return ORACLE_OK;
}

/*
 * Scale search ([MRGPTQ] Sommario tecnico section 3 item 2: scales chosen to
 * minimise the reconstruction MSE instead of the max-based scale; the page
 * gives no search procedure).  Reading R8:
 *   - Candidates are the max-based scale code c0 (the one oracle_quantize
 *     picks) and its neighbours c0 + j, 0 < |j| <= radius, that lie in the
 *     format's code range: MXFP4 bytes 0..254, UE4M3 0..0x7E, UE5M3 0..0xF7.
 *     Consecutive bytes are consecutive scale values in all three formats.
 *   - Each candidate is scored by its block SSE in binary64, with the
 *     elements coded and dequantized exactly as oracle_quantize does under
 *     that scale code.
 *   - Candidates are visited in the order j = 0, -1, +1, -2, +2, ...; one
 *     replaces the best so far only when its SSE is below
 *     best - best * 2^-40.  Near-ties therefore keep the code closest to c0
 *     (the smaller code first), and the choice does not hinge on the last
 *     bits of a sum.
 *   - The chosen code's codes, dequantized values and error split are the
 *     outputs, as in oracle_quantize.  The per-tensor scale g is found as
 *     there; no search over g.
 */
static double block_sse_under(int fmt, const float* v, int b, block_scale s, int* cd, float* xh)
{
    double sse = 0.0;
    for (int i = 0; i < b; ++i) {
        cd[i] = element_code(fmt, v[i], s);
        xh[i] = element_value(fmt, cd[i], s);
        double e = (double)v[i] - (double)xh[i];
        sse += e * e;
    }
    return sse;
}

int oracle_quantize_search(const float* x, int64_t rows, int64_t cols, int fmt, int block,
                           int gmode, float* g, int rotate, int radius, uint8_t* codes,
                           uint8_t* scales, float* block_mse, int mse_kind, double* acc,
                           int64_t* cnt)
{
    if (!valid_shape(fmt, block, rows, cols, rotate)) return ORACLE_BAD_ARG;
    if (fmt != FMT_UE4M3 && gmode != GMODE_NONE) return ORACLE_BAD_ARG;
    if (radius < 0 || radius > 8) return ORACLE_BAD_ARG;
    float gv = 1.0f;
    if (fmt == FMT_UE4M3) {
        if (gmode == GMODE_DYNAMIC) {
            gv = oracle_dynamic_g(oracle_tensor_amax(x, rows, cols, rotate));
            if (g) *g = gv;
        } else if (gmode == GMODE_GIVEN) {
            if (!g) return ORACLE_BAD_ARG;
            gv = *g;
        }
    }
    const int max_byte = fmt == FMT_MXFP4 ? 254 : (fmt == FMT_UE4M3 ? 0x7E : 0xF7);
    if (acc) memset(acc, 0, 4 * sizeof(double));
    if (cnt) memset(cnt, 0, 2 * sizeof(int64_t));
    int64_t nblk_row = cols / block;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < nblk_row; ++k) {
            const float* src = x + r * cols + k * block;
            float v[256], xh[256], best_xh[256];
            int cd[256], best_cd[256];
            for (int i = 0; i < block; ++i) v[i] = src[i];
            if (rotate) oracle_hadamard_block(v, rotate);
            int c0 = scale_for_block(fmt, block_absmax(v, block), gv).byte;
            int best_byte = c0;
            double best_sse = 0.0;
            for (int t = 0; t <= 2 * radius; ++t) {
                int j = t == 0 ? 0 : ((t & 1) ? -(t + 1) / 2 : t / 2);
                int byte = c0 + j;
                if (byte < 0 || byte > max_byte) continue;
                double sse = block_sse_under(fmt, v, block, scale_from_byte(fmt, byte, gv), cd, xh);
                if (t == 0 || sse < best_sse - best_sse * 0x1p-40) {
                    best_sse = sse;
                    best_byte = byte;
                    memcpy(best_cd, cd, sizeof(int) * (size_t)block);
                    memcpy(best_xh, xh, sizeof(float) * (size_t)block);
                }
            }
            scales[r * nblk_row + k] = (uint8_t)best_byte;
            for (int i = 0; i < block; i += 2) {
                int64_t byte_idx = (r * cols + k * block + i) / 2;
                codes[byte_idx] = (uint8_t)(best_cd[i] | (best_cd[i + 1] << 4));
            }
            float mse = block_error(v, best_xh, block, mse_kind, acc, cnt);
            if (block_mse) block_mse[r * nblk_row + k] = mse;
        }
    }
    return ORACLE_OK;
}

/*
 * Product of two MXFP4 matrices ([MRGPTQ] Sommario tecnico section 3 item 4
 * and section 4: the FP4 GEMM that consumes the packed codes and scales).
 * A (M x K) and B (N x K) are given as codes and E8M0 scale bytes in the
 * layout oracle_quantize writes (blocks of 32 along K); the result is
 * C = A_hat * B_hat^T in binary64 from the exactly dequantized values, C row
 * major M x N.  (Every dequantized value v * 2^E is exact in binary64, so
 * the only rounding is in the sums.)  R10: the product is taken on the
 * dequantized operands; the pages give no accumulation order or precision.
 */
int oracle_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                      const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, double* c)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t ea = m * K + k, eb = n * K + k;
                int ca = (a_codes[ea / 2] >> ((ea % 2) * 4)) & 15;
                int cb = (b_codes[eb / 2] >> ((eb % 2) * 4)) & 15;
                double va = ldexp(oracle_e2m1_value(ca), (int)a_scales[m * (K / 32) + k / 32] - 127);
                double vb = ldexp(oracle_e2m1_value(cb), (int)b_scales[n * (K / 32) + k / 32] - 127);
                sum += va * vb;
            }
            c[m * N + n] = sum;
        }
    }
    return ORACLE_OK;
}

/*
 * R11: product of two NVFP4 matrices (the FP4 GEMM of [MRGPTQ] Sommario
 * tecnico section 3 item 4 and section 4, for the NVFP4 format of [DIAG]
 * section 2).  A (M x K) and B (N x K) are codes and UE4M3 scale bytes per 16
 * elements along K, as oracle_quantize writes them for block 16, with
 * per-tensor scales ga and gb; each element is dequantized exactly as
 * oracle_dequantize does (binary32: d = RN32(s_hat * g), x_hat = RN32(v * d)),
 * and C = A_hat * B_hat^T is summed in binary64, row major M x N.
 */
int oracle_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, float ga,
                      const uint8_t* b_codes, const uint8_t* b_scales, float gb, int64_t M,
                      int64_t N, int64_t K, double* c)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t ea = m * K + k, eb = n * K + k;
                int ca = (a_codes[ea / 2] >> ((ea % 2) * 4)) & 15;
                int cb = (b_codes[eb / 2] >> ((eb % 2) * 4)) & 15;
                block_scale sa = scale_from_byte(FMT_UE4M3, a_scales[m * (K / 16) + k / 16], ga);
                block_scale sb = scale_from_byte(FMT_UE4M3, b_scales[n * (K / 16) + k / 16], gb);
                sum += (double)element_value(FMT_UE4M3, ca, sa) * (double)element_value(FMT_UE4M3, cb, sb);
            }
            c[m * N + n] = sum;
        }
    }
    return ORACLE_OK;
}

/* Dequantize codes back to binary32 in the original domain: with rotation the
 * dequantized block is rotated again (the transform is its own inverse). */
int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int fmt, int block,
                      float g, int64_t rows, int64_t cols, int rotate, float* out)
{
    if (!valid_shape(fmt, block, rows, cols, rotate)) return ORACLE_BAD_ARG;
    int64_t nblk_row = cols / block;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < nblk_row; ++k) {
            block_scale s = scale_from_byte(fmt, scales[r * nblk_row + k], g);
            float xh[256];
            for (int i = 0; i < block; ++i) {
                int64_t e = r * cols + k * block + i;
                int code = (codes[e / 2] >> ((e % 2) * 4)) & 15;
                xh[i] = element_value(fmt, code, s);
            }
            if (rotate) oracle_hadamard_block(xh, rotate);
            for (int i = 0; i < block; ++i) out[r * cols + k * block + i] = xh[i];
        }
    }
    return ORACLE_OK;
}

/* Error terms of stored codes against x (rotated first when rotating). */
int oracle_block_mse(const float* x, const uint8_t* codes, const uint8_t* scales, int fmt,
                     int block, float g, int64_t rows, int64_t cols, int rotate,
                     float* block_mse, int mse_kind, double* acc, int64_t* cnt)
{
    if (!valid_shape(fmt, block, rows, cols, rotate)) return ORACLE_BAD_ARG;
    if (acc) memset(acc, 0, 4 * sizeof(double));
    if (cnt) memset(cnt, 0, 2 * sizeof(int64_t));
    int64_t nblk_row = cols / block;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < nblk_row; ++k) {
            block_scale s = scale_from_byte(fmt, scales[r * nblk_row + k], g);
            float v[256], xh[256];
            for (int i = 0; i < block; ++i) {
                int64_t e = r * cols + k * block + i;
                v[i] = x[e];
                int code = (codes[e / 2] >> ((e % 2) * 4)) & 15;
                xh[i] = element_value(fmt, code, s);
            }
            if (rotate) oracle_hadamard_block(v, rotate);
            float mse = block_error(v, xh, block, mse_kind, acc, cnt);
            if (block_mse) block_mse[r * nblk_row + k] = mse;
        }
    }
    return ORACLE_OK;
}

/* Binary32 -> bfloat16 bits, round to nearest, ties to an even bf16 mantissa:
 * the two bf16 neighbours of |v| are compared by exact distance.  Past the
 * largest finite bf16 the upper neighbour is 2^128 (infinity after rounding),
 * as in IEEE rounding with an unbounded exponent. */
uint16_t oracle_to_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint32_t sign = u & 0x80000000u, mag = u & 0x7FFFFFFFu;
    uint32_t lo = mag & 0xFFFF0000u;
    if (lo == mag) return (uint16_t)(u >> 16);
    uint32_t hi = lo + 0x10000u; /* next bf16 magnitude */
    float flo, fhi, fmag;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    memcpy(&fmag, &mag, 4);
    double dhi_val = ((hi >> 23) == 0xFFu) ? ldexp(1.0, 128) : (double)fhi;
    double dlo = (double)fmag - (double)flo, dhi = dhi_val - (double)fmag;
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1u) ? hi : lo;
    return (uint16_t)((sign | pick) >> 16);
}

void oracle_to_bf16_array(const float* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_to_bf16(v[i]);
}

/* Array forms of the scalar rules, for exhaustive checks. */
void oracle_e2m1_codes(const double* y, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_code(y[i]);
}

void oracle_e8m0_exponents(const float* m, int64_t n, int32_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e8m0_exponent(m[i]);
}

void oracle_ue4m3_bytes(const float* s, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_ue4m3_byte(s[i]);
}

void oracle_ue5m3_bytes(const float* s, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_ue5m3_byte(s[i]);
}
