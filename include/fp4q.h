/*
 * fp4q.h -- C ABI of the MI355X (gfx950) microscaling FP4 quantization library.
 *
 * The library quantizes row-major matrices to 4-bit E2M1 codes in blocks of b
 * consecutive elements along each row, each block sharing one 8-bit scale:
 *
 *   MXFP4  b = 32, E8M0 power-of-two scale (a shared 8-bit exponent).
 *          Source: "Diagnosing FP4 inference: a layer-wise and block-wise
 *          sensitivity analysis of NVFP4 and MXFP4", technical summary section 2
 *          (32-element blocks, shared 8-bit exponent, E2M1 elements);
 *          "Bridging the Gap Between Promise and Performance for Microscaling
 *          FP4 Quantization", Sommario tecnico section 1 (E8M0 power-of-two
 *          scales, round-to-nearest).
 *   NVFP4  b = 16, unsigned E4M3 (UE4M3) scale under an FP32 per-tensor scale g.
 *          Same pages: 16-element blocks, dynamic "max" scaling, E4M3 scales;
 *          "Is finer better? Limits of micro-scaling formats in LLMs",
 *          Framework Teorico (UE4M3, smallest non-zero scale 2^-9) and
 *          Risultati (UE4M3-S: UE4M3 with per-tensor scaling).
 *   UE4M3 / UE5M3 at b in {8, 16, 32, 64, 128, 256}: the block-size sweep and
 *          the UE5M3 scale (smallest non-zero scale 2^-17, no per-tensor scale)
 *          of "Is finer better?", Metodologia and Contributi Chiave item 3.
 *
 * An optional block-diagonal Hadamard rotation of size 16 or 32 (equal to the
 * block) precedes quantization ("Bridging the Gap...", Sommario tecnico
 * section 3 item 1 and section 2).  The error of each block is split into the
 * three sources of "Is finer better?", Framework Teorico: non-maximum elements,
 * the block maximum, and zero-rounding of a whole block.
 *
 * Rules the pages leave open, as this library implements them:
 *   - E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}: nearest value, an exact tie
 *     goes to the even 3-bit code, past 6 saturates to 6; the code's sign bit is
 *     the input's sign (so -0 and small negatives give 0x8).
 *   - MXFP4 scale exponent E = floor(log2 m) - 2, clamped to [-127, 127], where
 *     m is the block's largest magnitude; byte = E + 127 (0x00 for an all-zero
 *     block); codes are those of x * 2^-E.
 *   - UE4M3 scale: D = RN32(6 g); s = RN32(m / D); the byte is s rounded to
 *     the nearest UE4M3 value (ties to even, saturating at 448, E4M3 bit
 *     pattern with a clear sign bit); d = RN32(s_hat * g); codes are those of
 *     RN32(x / d), or sign-only zeros when s_hat = 0.  UE5M3 is the same with
 *     bias 15, values down to 2^-17 and up to 61440, and g = 1.
 *   - Dynamic per-tensor scale: g = RN32(amax / 2688) over the (rotated)
 *     tensor, g = 1 when that is 0.
 *   - Rotation: normalised Sylvester Walsh-Hadamard transform in binary32,
 *     butterfly stages h = 1, 2, 4, ... in that order, then one multiply by
 *     RN32(n^-1/2).  Quantization, amax and errors act on rotated values.
 *   - Packing: byte j of a row's codes holds element 2j in its low nibble and
 *     element 2j+1 in its high nibble.  Scales are one byte per block, row-major
 *     (rows x cols/b).  Per-block MSE is one float per block, same layout.
 *   - Errors: e = x - x_hat; block SSE; m = max |x|, i* = the lowest index
 *     attaining m.  A zero-rounded block has m > 0 and every x_hat = 0: its SSE
 *     is the zero-rounding term.  Otherwise e_{i*}^2 is the max-element term
 *     and the rest of the SSE the non-max term.  Per-block MSE is SSE/b (ABS)
 *     or SSE/sum(x^2) (REL, 0 when sum(x^2) = 0).
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library allocates nothing.  Inputs and outputs are contiguous row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every
 *     call is asynchronous; outputs are valid once the stream has reached the
 *     call.  Calls may be captured into a HIP graph.
 *   - A call returns a status at once.  Arguments are checked before anything is
 *     launched: on an error nothing is launched or written, and fp4q_last_error()
 *     (thread-local) holds a description.  No C++ exception crosses the ABI.
 *   - rows * cols == 0 is valid: codes/scales/block_mse are untouched, *stats
 *     is set to zeros and, in the dynamic mode, *g to 1 (with FP4Q_G_ROW,
 *     g[0..rows) to 1).
 *   - NaN and infinite inputs are outside the contract: codes are unspecified
 *     for them; nothing faults.  With rotation, inputs must also keep the
 *     binary32 butterfly finite, which |x| < 2^100 guarantees.
 *   - Workspace: calls that take `ws` need fp4q_workspace_bytes() bytes of
 *     device memory (256-byte aligned, any initial contents).  One workspace
 *     serves any number of calls in stream order, but only one call at a time:
 *     calls that overlap on one workspace race.
 *   - Results are deterministic: the same inputs give bit-identical outputs,
 *     including the floating-point sums in fp4q_stats.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 2

typedef enum {
    FP4Q_OK = 0,
    FP4Q_ERR_ARG = 1,       /* a required pointer is NULL or an enum is out of range */
    FP4Q_ERR_SHAPE = 2,     /* negative size, cols % block != 0, bad block/rotation,
                               more than (2^31 - 1) * 512 elements */
    FP4Q_ERR_ALIGN = 3,     /* a pointer violates the alignment stated below */
    FP4Q_ERR_WORKSPACE = 4, /* ws missing or smaller than fp4q_workspace_bytes() */
    FP4Q_ERR_HIP = 5        /* the HIP runtime reported an error at launch */
} fp4q_status;

typedef enum { FP4Q_BF16 = 0, FP4Q_F32 = 1 } fp4q_dtype;

typedef enum {
    FP4Q_FMT_MXFP4 = 0, /* E8M0 scales, block 32 */
    FP4Q_FMT_UE4M3 = 1, /* UE4M3 scales (NVFP4 at block 16), with per-tensor g */
    FP4Q_FMT_UE5M3 = 2  /* UE5M3 scales, no per-tensor scale (g = 1) */
} fp4q_format;

typedef enum {
    FP4Q_G_NONE = 0,    /* g = 1 */
    FP4Q_G_DYNAMIC = 1, /* g = RN32(amax / 2688), written to *g (device) */
    FP4Q_G_GIVEN = 2,   /* g read from *g (device); must be positive and finite */
    FP4Q_G_ROW = 3      /* one dynamic scale per row (per token of an activation
                           matrix): g_r = RN32(amax_r / 2688) over row r (rotated
                           when rotating), 1 when 0, written to g[0..rows);
                           UE4M3 only.  One kernel launch; no workspace unless
                           stats are wanted. */
} fp4q_gmode;

typedef enum { FP4Q_MSE_ABS = 0, FP4Q_MSE_REL = 1 } fp4q_mse_kind;

/* Tensor-level error terms (device memory, written by the call). */
typedef struct {
    double sse_nonmax;     /* sum of squared errors of non-maximum elements */
    double sse_max;        /* sum of squared errors of the block maxima */
    double sse_zero;       /* squared error of zero-rounded blocks (whole blocks) */
    double sum_x2;         /* sum of x^2 (rotated values when rotating); within
                              (4 + log2(b / 8)) 2^-24 of its exact value,
                              relatively (a quantize pass sums the exact squares
                              of bf16 input without rotation per block in
                              binary32) */
    int64_t n_blocks;      /* rows * cols / block */
    int64_t n_zero_blocks; /* number of zero-rounded blocks */
} fp4q_stats;

/*
 * MXFP4 quantization (block 32, E8M0 scales), fused with dequantization and the
 * error split.
 *   x          device, rows x cols, dtype xt (FP4Q_BF16 or FP4Q_F32); 16-byte aligned
 *   rotate     0 or 32 (block Hadamard before quantization)
 *   codes      device out, rows x cols/2 bytes; 16-byte aligned
 *   scales     device out, rows x cols/32 bytes (E8M0 byte = E + 127)
 *   block_mse  device out or NULL, rows x cols/32 floats (kind mse_kind); 4-byte aligned
 *   stats      device out or NULL; 8-byte aligned
 *   ws         device workspace (see Conventions); needed when stats != NULL
 * cols must be a multiple of 32.  With block_mse and stats both NULL only codes
 * and scales are produced.
 */
fp4q_status mxfp4_quantize(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t rotate,
                           uint8_t* codes, uint8_t* scales, float* block_mse, int32_t mse_kind,
                           fp4q_stats* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * UE4M3 / UE5M3 block quantization (NVFP4 at block 16), fused as above.
 *   block      8, 16, 32, 64, 128 or 256; cols must be a multiple of it
 *   scale_fmt  FP4Q_FMT_UE4M3 or FP4Q_FMT_UE5M3 (UE5M3 requires gmode NONE)
 *   gmode      fp4q_gmode; g is a device pointer to one float, written in the
 *              dynamic mode and read in the given mode (may be NULL for NONE);
 *              with FP4Q_G_ROW it points to rows floats, all written (may be
 *              NULL when rows is 0)
 *   rotate     0, or equal to block when block is 16 or 32
 *   ws         needed when stats != NULL or gmode == DYNAMIC
 * Other arguments as for mxfp4_quantize; scales are rows x cols/block bytes.
 */
fp4q_status nvfp4_quantize(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t block,
                           int32_t scale_fmt, int32_t gmode, float* g, int32_t rotate,
                           uint8_t* codes, uint8_t* scales, float* block_mse, int32_t mse_kind,
                           fp4q_stats* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * One tensor in both formats ("Diagnosing FP4 inference", technical summary
 * section 2: each layer's tensors quantized to NVFP4 and to MXFP4 and their
 * errors compared): mxfp4_quantize (no rotation) and nvfp4_quantize with UE4M3
 * scales under the dynamic per-tensor scale (no rotation), as one call.  The
 * MXFP4 pass reads every element anyway, so it also takes the tensor maximum,
 * and the NVFP4 pass uses it: the tensor is read twice instead of three times
 * (no separate amax pass).
 *   mx_*       outputs of the MXFP4 pass, as for mxfp4_quantize (block 32)
 *   nv_block   block of the NVFP4 pass (8 ... 256, dividing cols)
 *   g          device out, one float: the per-tensor scale RN32(amax / 2688)
 *              (1 when amax is 0), as nvfp4_quantize writes in the dynamic mode
 *   nv_*       outputs of the NVFP4 pass, as for nvfp4_quantize
 *   mse_kind   kind of both per-block MSE outputs
 *   ws         fp4q_workspace_bytes() bytes, always needed
 * Every output equals the two separate calls' outputs bit for bit, except the
 * NVFP4 pass's sum_x2 term when nv_block_mse is NULL or mse_kind is
 * FP4Q_MSE_ABS: the separate dynamic call sums it in its amax pass (binary64),
 * this call in its NVFP4 pass (per block in binary32 for bf16 input, within
 * (4 + log2(nv_block / 8)) 2^-24 relatively; else binary64, equal to rounding).
 * Errors as for the two calls; nothing is launched
 * unless both calls' arguments are valid.
 */
fp4q_status fp4_quantize_mx_nv(const void* x, int32_t xt, int64_t rows, int64_t cols,
                               uint8_t* mx_codes, uint8_t* mx_scales, float* mx_block_mse,
                               fp4q_stats* mx_stats, int32_t nv_block, float* g, uint8_t* nv_codes,
                               uint8_t* nv_scales, float* nv_block_mse, fp4q_stats* nv_stats,
                               int32_t mse_kind, void* ws, size_t ws_bytes, void* stream);

/* One tensor of a batched fp4_quantize_mx_nv call: its device input and the
 * outputs of both passes, laid out as for fp4_quantize_mx_nv. */
typedef struct {
    const void* x;             /* device, rows x cols, 16-byte aligned */
    int64_t rows, cols;
    uint8_t* mx_codes;         /* MXFP4 pass, as for mxfp4_quantize */
    uint8_t* mx_scales;
    float* mx_block_mse;
    fp4q_stats* mx_stats;
    float* g;                  /* device out: the NVFP4 per-tensor scale */
    uint8_t* nv_codes;         /* NVFP4 pass, as for nvfp4_quantize */
    uint8_t* nv_scales;
    float* nv_block_mse;
    fp4q_stats* nv_stats;
} fp4q_mx_nv_tensor;

#define FP4Q_MAX_BATCH 16

/*
 * fp4_quantize_mx_nv for up to FP4Q_MAX_BATCH tensors (say, one layer's
 * projections) in one launch per pass: the grid is split between the tensors,
 * each tensor's workgroups sweeping only its own elements, so small tensors
 * share a launch instead of paying one each.
 *   tensors    host array of n_tensors descriptors (1 <= n_tensors <= 16);
 *              shapes may differ
 *   xt         dtype of every tensor's x
 *   nv_block   16 or 32
 *   mse_kind   kind of every per-block MSE output
 *   ws         fp4q_workspace_bytes() bytes, always needed
 * Each format's block_mse must be given for every tensor or for none, and
 * likewise its stats.  Every code byte, scale byte, per-block MSE and g equals
 * the single-tensor call's; the tensor terms equal it to rounding (a tensor's
 * partial sums follow its share of the grid).  Errors as for
 * fp4_quantize_mx_nv, with the failing tensor's index in the message;
 * nothing is launched unless every tensor's arguments are valid.
 */
fp4q_status fp4_quantize_mx_nv_batch(const fp4q_mx_nv_tensor* tensors, int32_t n_tensors,
                                     int32_t xt, int32_t nv_block, int32_t mse_kind, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * Quantization with a per-block scale search ("Bridging the Gap...", Sommario
 * tecnico section 3 item 2: scales chosen to minimise the reconstruction MSE
 * rather than taken from the block maximum).  The page gives no procedure; this
 * library's reading:
 *   - candidates are the max-based scale code c0 (the code mxfp4_quantize /
 *     nvfp4_quantize would write) and c0 + j for 0 < |j| <= radius, within the
 *     format's codes (MXFP4 0..254, UE4M3 0..0x7E, UE5M3 0..0xF7);
 *   - each is scored by the block's sum of squared errors in binary64, with
 *     codes and dequantized values formed exactly as the plain calls do under
 *     that code;
 *   - candidates are visited as j = 0, -1, +1, -2, +2, ...; one replaces the
 *     best so far only when its SSE is below best - best * 2^-40, so near-ties
 *     keep the code closest to c0;
 *   - codes, scales, block_mse and stats are those of the chosen code.
 * The per-tensor scale g (UE4M3) is found as in nvfp4_quantize; it is not
 * searched.  radius 0 gives exactly the plain calls' results.
 *   fmt, block  FP4Q_FMT_MXFP4 (block 32, gmode NONE), UE4M3 or UE5M3 (block
 *               8..256; UE5M3 with gmode NONE)
 *   radius      0..FP4Q_SEARCH_MAX_RADIUS
 * Other arguments and the workspace rule as for nvfp4_quantize.  The search
 * costs about 2 * radius + 1 times the arithmetic of a plain call.
 */
#define FP4Q_SEARCH_MAX_RADIUS 8
fp4q_status fp4_quantize_search(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t fmt,
                                int32_t block, int32_t gmode, float* g, int32_t rotate,
                                int32_t radius, uint8_t* codes, uint8_t* scales, float* block_mse,
                                int32_t mse_kind, fp4q_stats* stats, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Dequantization of stored codes and scales ("Diagnosing FP4 inference",
 * section 2: weights are dequantized for the compute).  x_hat = v * 2^E (MXFP4,
 * exact) or RN32(v * d) with d = RN32(s_hat * g); with rotate the block
 * Hadamard is applied to x_hat, returning to the original domain.
 *   codes, scales  device, as written by the quantize calls; codes 4-byte aligned
 *   fmt, block     FP4Q_FMT_MXFP4 (block 32) / UE4M3 / UE5M3 (block 8..256)
 *   g              device pointer to g for UE4M3 (NULL means g = 1); ignored otherwise
 *   out            device out, rows x cols of dtype ot (F32, or BF16 rounded to
 *                  nearest even); 16-byte aligned
 */
fp4q_status fp4_dequantize(const uint8_t* codes, const uint8_t* scales, int32_t fmt, int32_t block,
                           const float* g, int64_t rows, int64_t cols, int32_t rotate, void* out,
                           int32_t ot, void* stream);

/*
 * Error split of stored codes against x (rotated first when rotate != 0), by
 * the same definitions as the fused quantize calls: for codes and scales they
 * wrote, block_mse and the block counts are bit-identical to theirs and the
 * tensor terms equal theirs up to the order of summation.  The max-element
 * term uses the lowest index attaining the block maximum, so codes need not
 * come from this library.  ws is needed when stats != NULL.
 */
fp4q_status fp4_block_mse(const void* x, int32_t xt, const uint8_t* codes, const uint8_t* scales,
                          int32_t fmt, int32_t block, const float* g, int64_t rows, int64_t cols,
                          int32_t rotate, float* block_mse, int32_t mse_kind, fp4q_stats* stats,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Block-diagonal normalised Hadamard rotation ("Bridging the Gap...", Sommario
 * tecnico section 3 item 1), n = 16 or 32, cols % n == 0.  out is device
 * binary32, 16-byte aligned.  The transform is its own inverse up to rounding.
 */
fp4q_status hadamard_block_rotate(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t n,
                                  float* out, void* stream);

/*
 * MXFP4 matrix product on the gfx950 scaled matrix cores ("Bridging the
 * Gap...", Sommario tecnico section 3 item 4 and section 4: the FP4 GEMM that
 * consumes the packed codes and scales).  C = A_hat * B_hat^T, where A (M x K)
 * and B (N x K) are MXFP4 matrices exactly as mxfp4_quantize writes them
 * (codes rows x K/2 bytes, E8M0 scales rows x K/32 bytes, blocks of 32 along
 * K; without rotation, or with the same rotation applied to both, since the
 * block Hadamard is orthogonal along K).  For activations times weights, A is
 * tokens x in-features and B out-features x in-features.
 *   a_codes, b_codes    device, 16-byte aligned
 *   a_scales, b_scales  device, any alignment
 *   M, N, K             K % 32 == 0, K <= 2^23, M < 2^31, N * sizeof(out
 *                       element) < 2^23; M or N == 0 is a no-op; K == 0
 *                       writes zeros
 *   c                   device out, M x N row-major, ct = FP4Q_F32 or FP4Q_BF16
 *                       (round to nearest even); aligned to its element
 *   ws, ws_bytes        device scratch of at least
 *                       fp4_gemm_workspace_bytes(M, N, K) bytes, 16-byte
 *                       aligned (not needed when M, N or K is 0): the scales
 *                       repacked in matrix-core order and, for products with
 *                       too few 256 x 256 tiles to fill the chip (small M),
 *                       the binary32 partial products of K ranges.  Owned by
 *                       the caller; calls that overlap in time need distinct
 *                       workspaces.
 * Decode-sized products (M <= 32, K % 128 == 0, both scale arrays 4-byte
 * aligned) run a kernel that streams B once, 32 rows of B per wave, with the
 * same arithmetic contract below; other shapes run the 256 x 256 tile kernel.
 * Products of E2M1 values and E8M0 scales are exact; the matrix cores add them
 * in binary32 in 64-element steps (partial products of K ranges are added in
 * binary64 and rounded once), so C differs from the exact product by rounding
 * of order (K/64 + 1) * 2^-24 of sum |a| |b|.  Results are the same on every
 * run for a given shape.  Errors: FP4Q_ERR_SHAPE
 * (sizes), FP4Q_ERR_ARG (NULL operand or c, bad ct), FP4Q_ERR_ALIGN,
 * FP4Q_ERR_WORKSPACE, FP4Q_ERR_HIP (launch failure); nothing is launched on
 * an error other than FP4Q_ERR_HIP.
 */
fp4q_status fp4_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                           int32_t ct, void* ws, size_t ws_bytes, void* stream);

/*
 * NVFP4 matrix product ("Bridging the Gap...", Sommario tecnico section 3
 * item 4 and section 4, for the NVFP4 format of "Diagnosing FP4 inference",
 * section 2).  C = A_hat * B_hat^T, where A (M x K) and B (N x K) are NVFP4
 * matrices exactly as nvfp4_quantize writes them with block 16 and UE4M3
 * scales (codes rows x K/2 bytes, scale bytes rows x K/16), each with its
 * per-tensor scale g.  The matrix cores' block scales are powers of two, so
 * each element's E2M1 value times its block scale (exact in bf16) goes
 * through bf16 matrix instructions, and a_g * b_g is applied to the binary32
 * result.
 *   a_codes, b_codes    device, 16-byte aligned
 *   a_scales, b_scales  device, 4-byte aligned
 *   a_g, b_g            device binary32 per-tensor scales (as nvfp4_quantize
 *                       writes or reads them); NULL means 1
 *   M, N, K             K % 64 == 0, K <= 2^23, M < 2^31, N * sizeof(out
 *                       element) < 2^23; M or N == 0 is a no-op; K == 0
 *                       writes zeros
 *   c, ct               as for fp4_gemm_mxfp4
 *   ws, ws_bytes        device scratch of at least
 *                       fp4_gemm_nvfp4_workspace_bytes(M, N, K) bytes (0 for
 *                       most shapes; then ws may be NULL), 16-byte aligned:
 *                       binary32 partial products of K ranges for products
 *                       with too few 256 x 256 tiles or few rows of B.
 *                       Owned by the caller.
 * Products of at most 32 rows of A run a kernel that streams B once, 32 rows
 * of B per wave; others run the 256 x 256 tile kernel; the contract below is
 * the same for both.
 * Against the exact product of the dequantized operands (x_hat = RN32(v *
 * RN32(s_hat * g)), as fp4_dequantize writes them), C differs by rounding of
 * order (K/16 + 8) * 2^-23 of sum |a_hat| |b_hat|: binary32 accumulation in
 * 16-element steps, partial products added in binary64, and the roundings of
 * the dequantized values and of the per-tensor scales.  Results are the same
 * on every run for a given shape.  Errors as for fp4_gemm_mxfp4.
 */
fp4q_status fp4_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g,
                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_g, int64_t M,
                           int64_t N, int64_t K, void* c, int32_t ct, void* ws, size_t ws_bytes,
                           void* stream);

/* Workspace bytes fp4_gemm_nvfp4 needs for an M x N x K product: 4 * M * N per
 * K range when K is split (a function of M, N and K only); 0 otherwise. */
size_t fp4_gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Workspace bytes fp4_gemm_mxfp4 needs for an M x N x K product: 256 *
 * (ceil(M/32) + ceil(N/32)) * ceil(K/256), rounded up to 256, plus
 * 4 * M * N per K range when K is split (the larger of the two kernels'
 * range counts, so a function of M, N and K only, whatever the alignment of
 * the scale arrays); 0 when M, N or K is 0. */
size_t fp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Workspace size in bytes for any call on a rows x cols tensor (a constant
 * upper bound in this version). */
size_t fp4q_workspace_bytes(int64_t rows, int64_t cols, int32_t block);

/* Description of the last error returned on the calling thread ("" if none). */
const char* fp4q_last_error(void);

/* FP4Q_ABI_VERSION of the loaded library. */
int32_t fp4q_abi_version(void);

/* nvfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, outputs and errors without `ws`/`ws_bytes`.  The
 * workspace is instead a static device array inside the library
 * (fp4q_workspace_bytes() bytes, about 0.8 MB, a fixed maximum that every
 * tensor size fits), one per device, kept until the process ends; its device
 * address is looked up once per device (FP4Q_ERR_HIP if that fails).  Nothing
 * is allocated.  All calls on one device share that array, so calls that
 * overlap on one device (e.g. on two streams) race; calls in stream order do
 * not. */
fp4q_status nvfp4_quantize_noalloc(const void* x, int32_t xt, int64_t rows, int64_t cols,
                                   int32_t block, int32_t scale_fmt, int32_t gmode, float* g,
                                   int32_t rotate, uint8_t* codes, uint8_t* scales, float* block_mse,
                                   int32_t mse_kind, fp4q_stats* stats, void* stream);

/* Launch timing, for benchmarks and profiling (no counterpart on the pages).
 * events: 2 * n_pairs HIP events (hipEvent_t passed as void*), created and
 * owned by the caller (with timing enabled to read durations).  From this call
 * on, every kernel the library launches from the calling thread records
 * events[2i] on its stream just before itself and events[2i + 1] just after,
 * for i = 0, 1, ... in launch order, until n_pairs launches have been
 * recorded.  A quantize call launches, in order: the amax pass (dynamic
 * per-tensor scale only), the quantize kernel, and the reduction of the tensor
 * terms (stats only).  n_pairs = 0 or events = NULL stops recording.  The
 * array and the events must stay valid while recording is on; nothing is
 * allocated.  Errors: FP4Q_ERR_ARG for n_pairs < 0. */
fp4q_status fp4q_profile_events(void* const* events, int32_t n_pairs);

/* Kernel launches recorded on the calling thread since the last
 * fp4q_profile_events call. */
int32_t fp4q_profile_count(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
