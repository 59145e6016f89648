/*
 * kq.h - C ABI of libkq, the MI355X (gfx950) KroQuant online activation
 * quantizer.
 *
 * What it computes.  KroQuant (arXiv 2607.21446; read from the Pith review
 * page, "What carries the argument", core claim, and the referee report on
 * Sec. 3.2 Eqs. (4)-(6); and the AIssential summary page) quantizes the input
 * X[tokens][d] of a DiT linear layer to W4A4's activation side as follows:
 *   1. every 32-channel block j of a row is multiplied on the right by its
 *      own invertible 32x32 matrix K(j) = G1 (x) G2 (x) G3 (x) G4 (x) G5, a
 *      Kronecker product of five 2x2 unit-determinant LU factors
 *      G = [[1,0],[l,1]] [[a,b],[0,1/a]] = [[a, b], [l a, l b + 1/a]]
 *      (three scalars per factor, 15 per block); y = x K(j) in the
 *      row-vector convention of the review's Eq. (1);
 *   2. each transformed block of 32 is quantized to MXFP4 (OCP Microscaling
 *      Formats v1.0, the review's reference [10]): one E8M0 scale byte
 *      e + 127 with e = floor(log2 amax) - 2 (amax = 0 -> byte 0; clamped to
 *      [-127, 127]), and 32 E2M1 codes of y / 2^e rounded to nearest with
 *      ties to the even code and saturation at +-6; bit 3 of a code is the
 *      sign of y.
 * The pages compare this quantizer with a per-channel (SmoothQuant) scale and
 * a fixed Hadamard transform at the same block size (review, "If this is
 * right"; original abstract); those two, and a plain MXFP4 quantizer, are
 * here too with the same output format.
 *
 * Layouts (all row-major, little-endian):
 *   X         bf16 bit patterns [tokens][d], d a positive multiple of 32.
 *   K_params  fp32 [nb][5][3] (nb = d/32): (l, a, b) of G1 .. G5 for block j
 *             at K_params + j * params_block_stride (stride 15, or 0 for one
 *             K shared by every block).  a must be nonzero and finite.
 *   K_f32     fp32 [nb][32][32], K[r][c] (r = input channel, c = output).
 *   K_bf16    bf16 bit patterns [nb][n_split][32][32], TRANSPOSED: entry
 *             [j][s][c][r]; the terms hi = bf16(K), mid = bf16(K - hi),
 *             lo = bf16(K - hi - mid), each rounded to nearest even.  With
 *             three terms hi + mid + lo equals the fp32 K exactly.
 *   codes     uint8 [tokens][d/2]; byte q of block j holds the codes of
 *             channels 32j+2q (low nibble) and 32j+2q+1 (high nibble).
 *   scales    uint8 [tokens][d/32], E8M0 (2^(byte-127)).
 *   ch_mult   fp32 [d] per-channel multipliers (SmoothQuant: 1/s_c).
 *   Y         fp32 [tokens][d], the values the quantizer rounded.
 *
 * Numerics.  The transform runs in fp32 (fp32 butterfly stages, or MFMA bf16
 * products of X with a three-term bf16 split of K); the per-element error
 * against the exact sum is below 1e-5 of the block amax.  Whenever a
 * block's amax lands within 2^-16 (relative) of a power of two, the columns
 * that decide the scale are recomputed exactly (fp64 sum of exact products,
 * the fp32 K), so the E8M0 scales equal those of an exact evaluation.  An
 * E2M1 code can differ from the exact evaluation's only where y / 2^e lies
 * within that error of a rounding midpoint.  Plain and SmoothQuant
 * front-ends are exact.
 *
 * Ownership and streams.  The caller owns every buffer (device memory, e.g.
 * PyTorch tensors).  The library allocates nothing, frees nothing, keeps no
 * pointer after returning and never synchronizes: each call only enqueues
 * kernels on `stream` (NULL = the null stream) and returns.  Outputs must not
 * overlap inputs.  Reentrant and thread-safe; the only shared state is a
 * per-device cache of the compute-unit count, filled on first use.
 *
 * Errors.  Argument checks run before any HIP call and write nothing:
 *   KQ_ERR_NULL    a required pointer is NULL while tokens > 0;
 *   KQ_ERR_SHAPE   d <= 0, d % 32 != 0, d > 2^24, tokens < 0, tokens >= 2^28,
 *                  tokens * d >= 2^40,
 *                  nb <= 0, n_split not in 1..3, a stride other than 15 / 0;
 *   KQ_ERR_ALIGN   X, codes, Y, K_bf16, ch_mult not 16-byte aligned, or
 *                  K_params / K_f32 not 4-byte aligned;
 *   KQ_ERR_VARIANT unknown variant, or a variant whose inputs are missing
 *                  (KQ_MFMA_DENSE needs K_bf16; the others need K_params);
 *   KQ_ERR_ALIAS   an output range overlaps an input range or another output.
 * tokens == 0 returns KQ_OK without touching the GPU.  A failed launch
 * returns KQ_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronization, as for any asynchronous HIP work.  No C++ exception
 * crosses this boundary.
 *
 * Interface notes (where these calls go beyond the plain form
 * kq_quantize(X, d, K_params, codes, scales, stream)):
 *   - every quantizing entry point takes `tokens`, the row count of X;
 *   - kq_quantize_ex takes no term count for K_bf16: KQ_MFMA_DENSE always
 *     reads the three-term split.  One bf16 term keeps 8 significant bits of
 *     each entry of K and two keep 16, so the transform error is bounded
 *     only by about 2^-9 or 2^-17 of sum_r |x_r K_rc|, which is above 1e-5
 *     of the block amax as soon as that sum exceeds 1.3 times the amax (as
 *     it does for most blocks); only three terms (the fp32 K exactly) keep
 *     the error within 1e-5 for every K.  kq_build_blocks still writes 1 to
 *     3 terms for other consumers;
 *   - kq_transform_f32 is one diagnostic entry for every front-end: it takes
 *     the front-end, the parameter stride, K_bf16 and ch_mult, and writes the
 *     codes and scales beside Y, so that each quantizing entry point's own
 *     kernel (plus a Y store) is what a test checks, codes included;
 *   - KQ_ERR_ALIAS: overlapping ranges are rejected with their own status
 *     rather than left undefined, since with an overlap the result would
 *     depend on the order in which the workgroups run.
 */
#ifndef KQ_H
#define KQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  KQ_OK = 0,
  KQ_ERR_NULL = 1,
  KQ_ERR_SHAPE = 2,
  KQ_ERR_ALIGN = 3,
  KQ_ERR_VARIANT = 4,
  KQ_ERR_HIP = 5,
  KQ_ERR_ALIAS = 6
} kq_status;

/* How K is applied.  AUTO picks per shape: a kq_tune result if one was recorded, else the rule in kq_auto_variant. */
typedef enum {
  KQ_AUTO = 0,
  KQ_MFMA_DENSE = 1, /* MFMA bf16 contraction with prebuilt K_bf16 (three-term split) */
  KQ_MFMA_OTF = 2,   /* MFMA bf16 contraction, K rebuilt in-kernel from the 15 scalars */
  KQ_BUTTERFLY = 3   /* five fp32 butterfly stages (two shears each, then the product of the
                        diagonals) from the 15 scalars, one block per lane, no MFMA */
} kq_variant;

/* Front-ends of kq_transform_f32. */
typedef enum { KQ_FRONT_KRON = 0, KQ_FRONT_PLAIN = 1, KQ_FRONT_SMOOTH = 2, KQ_FRONT_HADAMARD = 3 } kq_front;

/* ABI version of this header (bumped on any signature or layout change). */
#define KQ_ABI_VERSION 6
int kq_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* kq_status_str(kq_status status);

/*
 * Dense blocks from the 15 scalars per block (the "precomputed dense blocks"
 * kernel variant of the review, "What carries the argument").  For each of
 * nb blocks, with parameters at K_params + 15 j: K = G1 (x) ... (x) G5 with
 * every entry the product, in fp64 and in factor order, of one entry of each
 * factor (G1 on bit 4 of the row and column index, G5 on bit 0), then
 * rounded once to fp32.  Writes K_f32 [nb][32][32] if non-NULL and the
 * transposed bf16 split K_bf16 [nb][n_split][32][32] if non-NULL
 * (1 <= n_split <= 3).  At least one output must be non-NULL.
 */
kq_status kq_build_blocks(const float* K_params, int64_t nb, float* K_f32, uint16_t* K_bf16, int n_split,
                          hipStream_t stream);

/*
 * The online quantizer: codes and scales of X K for every block, with K
 * built from K_params (stride 15).  Equivalent to kq_quantize_ex(X, tokens,
 * d, K_params, 15, NULL, KQ_AUTO, out_codes, out_scales, stream).
 */
kq_status kq_quantize(const uint16_t* X, int64_t tokens, int64_t d, const float* K_params, uint8_t* out_codes,
                      uint8_t* out_scales, hipStream_t stream);

/*
 * As kq_quantize, choosing how K is applied.  params_block_stride is 15 (one
 * parameter set per block) or 0 (block 0's parameters, and K_bf16's block 0,
 * for every block).  K_bf16 (three-term split from kq_build_blocks, layout
 * above) is required by KQ_MFMA_DENSE and ignored by the other variants;
 * K_params is required by every variant except KQ_MFMA_DENSE.  KQ_AUTO uses
 * KQ_BUTTERFLY when K_params is given and KQ_MFMA_DENSE when only K_bf16 is
 * (unless kq_tune recorded another choice for the shape).
 */
kq_status kq_quantize_ex(const uint16_t* X, int64_t tokens, int64_t d, const float* K_params,
                         int64_t params_block_stride, const uint16_t* K_bf16, kq_variant variant,
                         uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream);

/*
 * The variant KQ_AUTO resolves to for a call with this shape, given whether
 * K_params and K_bf16 are supplied (nonzero = supplied): the same rule the
 * entry points apply (a KQ_VARIANT override, else a kq_tune record, else
 * KQ_BUTTERFLY with K_params, KQ_MFMA_DENSE with K_bf16 alone).  Returns
 * KQ_AUTO when no variant can serve the call (neither input supplied).  Pure
 * host logic, no HIP call.
 *
 * Two environment variables, read once at the first call, exist for
 * measurement and change no result: KQ_VARIANT (mfma_dense, mfma_otf or
 * butterfly) replaces KQ_AUTO's choice wherever the supplied inputs allow
 * that variant, and KQ_WG_PER_CU (1 .. 64) caps the workgroups per compute
 * unit that every grid of the library is sized for.  Other values are ignored.
 */
kq_variant kq_auto_variant(int64_t tokens, int64_t d, int has_params, int has_split);

/* Plain MXFP4: y = x. */
kq_status kq_mx_quantize(const uint16_t* X, int64_t tokens, int64_t d, uint8_t* out_codes, uint8_t* out_scales,
                         hipStream_t stream);

/*
 * SmoothQuant front-end then MXFP4: y = fp32(x * ch_mult[c]) (one rounding),
 * the activation side of X diag(s)^-1 with ch_mult = 1/s (SmoothQuant, the
 * handbook page "Quantization: where diffusion differs from an LLM",
 * SmoothQuant section; the per-channel scaling baseline of the review).
 */
kq_status kq_smooth_quantize(const uint16_t* X, int64_t tokens, int64_t d, const float* ch_mult,
                             uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream);

/*
 * Fixed block-Hadamard front-end then MXFP4: y[c] = fp32(sum_r x[r] H[r][c] /
 * sqrt(32)) with H[r][c] = (-1)^popcount(r & c) (natural-order Walsh-
 * Hadamard, orthonormal), the "fixed Hadamard at the same block size" of the
 * review's significance paragraph.
 */
kq_status kq_hadamard_quantize(const uint16_t* X, int64_t tokens, int64_t d, uint8_t* out_codes,
                               uint8_t* out_scales, hipStream_t stream);

/*
 * Block-Hadamard front-end of size `block` (32, 64, 128, 256 or 512; d a
 * multiple of it) then MXFP4 over blocks of 32: y[c] = fp32(sum_r x[r]
 * H[r][c] / sqrt(block)) within each block of `block` channels, the "larger
 * block sizes" a fixed Hadamard needs (Pith review, original abstract).
 * block = 32 is kq_hadamard_quantize.  Other sizes -> KQ_ERR_SHAPE.
 */
kq_status kq_hadamard_quantize_ex(const uint16_t* X, int64_t tokens, int64_t d, int block, uint8_t* out_codes,
                                  uint8_t* out_scales, hipStream_t stream);

/*
 * 16-wide KroQuant blocks with four factors (a block-size / factor-count
 * variant, 12 scalars per 16 channels at K_params16 + 12 b, (l, a, b) of
 * G1 .. G4, G1 on bit 3 of the 16-index): written as block-diagonal 32x32
 * blocks diag(K_{2j}, K_{2j+1}) in the layouts of kq_build_blocks (K_f32
 * [nb16/2][32][32], K_bf16 [nb16/2][n_split][32][32] transposed), each entry
 * the fp64 product in factor order rounded once to fp32, zeros off the
 * diagonal blocks.  Quantize with kq_quantize_ex(..., K_bf16, KQ_MFMA_DENSE).
 * nb16 must be even (KQ_ERR_SHAPE otherwise); errors as kq_build_blocks.
 */
kq_status kq_build_blocks16(const float* K_params16, int64_t nb16, float* K_f32, uint16_t* K_bf16, int n_split,
                            hipStream_t stream);

/*
 * Per-shape tuning of KQ_AUTO (opt-in).  Times the variant the built-in rule
 * picks and every variant the supplied inputs allow (KQ_MFMA_OTF and
 * KQ_BUTTERFLY need K_params with stride 15, KQ_MFMA_DENSE needs K_bf16), the
 * MFMA variants each with fourteen grid shapes (seven sizes of the second
 * part of the grid, the share of row tiles left to workgroups that start as
 * others finish and the tiles each of those takes, times a first part sized
 * for the resident workgroups per CU or for one; outputs do not depend on the
 * grid shape), on the caller's buffers: three interleaved rounds of 3 warm-up
 * launches and `reps` timed launches per candidate (1 <= reps <= 1000, else
 * KQ_ERR_SHAPE), timed with events on `stream`, each candidate scored by its
 * median round.  The fastest candidate is recorded if it is at least 3%
 * faster than the built-in rule's, else the rule's choice is (the timing
 * reuses one set of buffers, which can stay in the last-level cache; the
 * margin keeps a pick that only wins warm from replacing the rule).  The
 * record is keyed by (tokens, d, which inputs are supplied), process-wide:
 * later KQ_AUTO calls with that key use its variant (kq_auto_variant reports
 * it; a KQ_VARIANT environment override still wins), and later kq_quantize /
 * kq_quantize_ex calls with that key, stride 15 and that variant use its grid
 * shape.  On return out_codes / out_scales hold the recorded variant's result
 * and *chosen (if not NULL) the variant.  This is the one entry point that
 * blocks: it synchronizes on its timing event.  Neither input ->
 * KQ_ERR_VARIANT; other errors as kq_quantize_ex; a failed launch or event ->
 * KQ_ERR_HIP.
 */
kq_status kq_tune(const uint16_t* X, int64_t tokens, int64_t d, const float* K_params, const uint16_t* K_bf16,
                  uint8_t* out_codes, uint8_t* out_scales, int reps, kq_variant* chosen, hipStream_t stream);

/* Forget every choice kq_tune recorded (KQ_AUTO falls back to its default rule). */
void kq_tune_reset(void);

/*
 * Diagnostic entry (tests): runs the same kernels as the entries above and
 * also stores Y, the fp32 values each code was rounded from.  front selects
 * the front-end; variant, K_params, params_block_stride and K_bf16 apply to
 * KQ_FRONT_KRON as in kq_quantize_ex, ch_mult to KQ_FRONT_SMOOTH.
 */
kq_status kq_transform_f32(int front, const uint16_t* X, int64_t tokens, int64_t d, const float* K_params,
                           int64_t params_block_stride, const uint16_t* K_bf16, kq_variant variant,
                           const float* ch_mult, float* Y, uint8_t* out_codes, uint8_t* out_scales,
                           hipStream_t stream);

/*
 * LayerNorm statistics per row, for the AdaLN producer step below (the
 * normalisation without affine parameters that precedes a DiT linear
 * layer's AdaLN modulation; the Pith review's summary gives AdaLN as the
 * reason the transform runs online, its ledger lists LayerNorm / AdaLN as
 * normalisations that do not commute with it).  For each row t:
 *   mean = sum_c x / d, var = sum_c (x - mean)^2 / d   (fp64 sums),
 *   rstd = 1 / sqrt(var + eps)                         (fp64),
 * stored as fp32 row_stats[2t] = mean, row_stats[2t+1] = rstd.  The fp64
 * summation order is unspecified: results can differ from a sequential
 * evaluation by one fp32 ulp, rarely.  Errors as above; eps < 0 or not finite
 * -> KQ_ERR_SHAPE; X 16-byte and row_stats 8-byte aligned.
 */
kq_status kq_row_stats(const uint16_t* X, int64_t tokens, int64_t d, float eps, float* row_stats,
                       hipStream_t stream);

/*
 * The quantizer with the AdaLN producer step fused in front of the transform
 * (one read of X instead of a modulation kernel's read + write followed by
 * the quantizer's read).  Each element, in fp32, one IEEE operation each and
 * in this order (no contraction):
 *   v = x;
 *   v = (v - mean_t) * rstd_t                 if row_stats != NULL ([tokens][2], above);
 *   v = v * (1 + mod_scale[s][c])             if mod_scale != NULL;
 *   v = v + mod_shift[s][c]                   if mod_shift != NULL;
 * with s = t / tokens_per_sample and mod_scale, mod_shift fp32
 * [ceil(tokens / tokens_per_sample)][d]; v is rounded to bf16 (nearest even)
 * and then transformed and quantized exactly as kq_quantize_ex would
 * transform and quantize that bf16 matrix (the handbook page "Quantization:
 * where diffusion differs from an LLM" describes AdaLN as timestep-dependent
 * per-channel scales and shifts; the form v (1 + scale) + shift is the DiT
 * one).  tokens_per_sample must be a multiple of 32 or at least tokens
 * (KQ_ERR_SHAPE otherwise).  Variants as kq_quantize_ex, with the same
 * inputs and the same rule for KQ_AUTO: every variant applies the producer
 * step, and the codes and scales equal those kq_quantize_ex gives with that
 * variant on the modulated bf16 matrix, bit for bit.
 * row_stats must be 8-byte aligned, mod_scale / mod_shift 16-byte aligned
 * (KQ_ERR_ALIGN otherwise).
 */
kq_status kq_quantize_adaln(const uint16_t* X, int64_t tokens, int64_t d, const float* row_stats,
                            const float* mod_scale, const float* mod_shift, int64_t tokens_per_sample,
                            const float* K_params, int64_t params_block_stride, const uint16_t* K_bf16,
                            kq_variant variant, uint8_t* out_codes, uint8_t* out_scales, hipStream_t stream);

/*
 * Blocks of the offline weight fold (Pith review, circularity check:
 * Eq. (1), A T (W T^-T)^T = A W^T): as kq_build_blocks, for
 * K^-T = (G1^-1)^T (x) ... (x) (G5^-1)^T with G^-1 = [[l b + 1/a, -b],
 * [-l a, a]] (each entry the fp64 product in factor order, rounded once to
 * fp32; same layouts and errors).  The folded, quantized weight is then
 * kq_quantize_ex(W, N_out, K_in, NULL, 15, K_bf16 of these blocks,
 * KQ_MFMA_DENSE, w_codes, w_scales, stream) for a bf16 weight W [N_out][K_in]
 * (rows = output features), i.e. every weight row times T^-T, quantized to
 * MXFP4 along K_in.
 */
kq_status kq_build_blocks_inverse_t(const float* K_params, int64_t nb, float* K_f32, uint16_t* K_bf16, int n_split,
                                    hipStream_t stream);

/*
 * W4A4 GEMM on the scaled FP4 matrix cores: Y[m][n] = sum_k a[m][k] b[n][k]
 * with a = E2M1(code) * 2^(scale - 127) from A (codes [M][K/2], scales
 * [M][K/32], the layout kq_quantize writes) and b likewise from B [N][K]
 * (a folded weight from kq_build_blocks_inverse_t + kq_quantize_ex).  Each
 * product is exact; sums are fp32 (per element error below K 2^-24 sum|a b|
 * in practice).  Writes Y_f32 [M][N] fp32 and/or Y_bf16 [M][N] bf16 (nearest
 * even), either may be NULL but not both.  K a positive multiple of 32
 * (<= 2^24), M <= 2^23, N <= 2^22, else KQ_ERR_SHAPE; codes 16-byte aligned;
 * outputs must not overlap inputs.  M == 0 or N == 0 returns KQ_OK.
 */
kq_status kq_gemm_mx(const uint8_t* A_codes, const uint8_t* A_scales, int64_t M, const uint8_t* B_codes,
                     const uint8_t* B_scales, int64_t N, int64_t K, float* Y_f32, uint16_t* Y_bf16,
                     hipStream_t stream);

/*
 * Measurement entry (not a quantizer): moves exactly the traffic of
 * kq_quantize's default kernel on X [tokens][d] (every bf16 of X read once in
 * 4 KB units of 64 consecutive 32-channel blocks, one 16-byte record per
 * block written to out_codes [tokens][d/2] and one byte per block to
 * out_scales [tokens][d/32], each wave's units in the same order, through the
 * same wave-private LDS round trip; the grid is sized for the probe's own
 * occupancy, one resident round of waves) with no arithmetic:
 * the outputs hold an XOR digest of the input, not codes.  Its rate is the
 * ceiling this access pattern reaches on the device, against which the
 * quantizers' rates are reported (the Pith review's Fig. 3 reports the
 * quantizer's effective HBM bandwidth).  Errors as kq_mx_quantize.
 */
kq_status kq_stream_probe(const uint16_t* X, int64_t tokens, int64_t d, uint8_t* out_codes, uint8_t* out_scales,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KQ_H */
