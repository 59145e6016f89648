/*
 * CPU oracle for the KroQuant online activation quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code with the HIP library.
 *
 * Plain, single-threaded, fp64 where the arithmetic is floating point.  The
 * method (KroQuant, arXiv 2607.21446, as read from the Pith review page,
 * "What carries the argument", referee report on Sec. 3.2 Eqs. (4)-(6), and
 * the original abstract):
 *   - a block-diagonal transform T applied to the activations, one 32x32
 *     block K(j) per 32 channels, K = G1 (x) G2 (x) G3 (x) G4 (x) G5;
 *   - each G_k a 2x2 unit-determinant LU factor with three scalars;
 *   - the transformed activations quantized to MXFP4 (E2M1 elements, one
 *     E8M0 scale per 32 elements; OCP Microscaling Formats v1.0, reference
 *     [10] of the same page).
 * Readings of points the pages leave open are listed next to each function.
 */
#ifndef KQ_ORACLE_H
#define KQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { KQO_KRON = 0, KQO_PLAIN = 1, KQO_SMOOTH = 2, KQO_HADAMARD = 3 };

/* G = L U with L = [[1,0],[l,1]], U = [[a,b],[0,1/a]], row-major G[0..3]. */
void kqo_factor(float l, float a, float b, double G[4]);
/* Closed-form inverse [[l b + 1/a, -b], [-l a, a]] of the factor above. */
void kqo_factor_inverse(float l, float a, float b, double Gi[4]);
/* K = G1 (x) ... (x) G5 from the index bits: K[r][c] = prod_k G_k[bit(r)][bit(c)]. */
void kqo_kron_dense(const float P[15], double K[1024]);
/* The same K, built by pushing each unit row vector through 5 butterfly stages. */
void kqo_kron_butterfly(const float P[15], double K[1024]);
/* (G1^-1) (x) ... (x) (G5^-1). */
void kqo_kron_inverse(const float P[15], double Kinv[1024]);
/* K rounded to fp32, row-major [r][c] (row r = input channel, c = output channel). */
void kqo_block_f32(const float P[15], float K32[1024]);
/*
 * Dense blocks for nb blocks, params read at P + j*pstride (pstride 15 or 0).
 * K32: [nb][32 r][32 c] fp32 (may be NULL).
 * Kbf: [nb][n_split][32 c][32 r] bf16 bit patterns, transposed, the terms
 *      hi = bf16(K32), mid = bf16(K32 - hi), lo = bf16(K32 - hi - mid) (may be NULL).
 */
void kqo_build_blocks(const float* P, int64_t nb, int64_t pstride, float* K32, uint16_t* Kbf, int n_split);

/*
 * Blocks for the offline weight fold (Pith review, circularity check:
 * Eq. (1), A T (W T^-T)^T = A W^T).  For the linear layer y = x W^T each row
 * of W is multiplied on the right by K(j)^-T, block by block, where
 * K^-T = (G1^-1)^T (x) ... (x) (G5^-1)^T.  Entry [r][c] of block j is the
 * product, in fp64 and factor order, of G_k^-1[bit(c)][bit(r)] over the five
 * factors, rounded once to fp32 (K32 [nb][32 r][32 c]); the bf16 split Kbf as
 * in kqo_build_blocks.  Either output may be NULL.
 */
void kqo_build_blocks_inverse_t(const float* P, int64_t nb, int64_t pstride, float* K32, uint16_t* Kbf,
                                int n_split);

/*
 * The KroQuant front-end with given fp32 blocks (K32 [nb][32 r][32 c], block j
 * at K32 + j * kstride, kstride 1024 or 0) in place of the 15 scalars; same
 * arithmetic and outputs as kqo_quantize_rows with KQO_KRON.  Returns 0 or 1.
 */
int kqo_quantize_rows_blocks(const uint16_t* X, int64_t T, int64_t d, const float* K32, int64_t kstride,
                             int64_t row0, int64_t row1, uint8_t* codes, uint8_t* scales, float* y32, double* yhat);

/*
 * Fixed block-Hadamard front-end of size B (a power of two, 32 <= B <= 512,
 * d % B == 0), the "larger block sizes" of the comparison (Pith review,
 * original abstract; the fixed Hadamard at the block size of the significance
 * paragraph is B = 32):
 *   y[c] = RNE_fp32((sum_r x[r] (-1)^popcount(r & c)) / sqrt(B))
 * over each B-channel block (fp64 sum in input order, one division), then
 * MXFP4 over blocks of 32 as for every front-end.  B = 32 equals the
 * KQO_HADAMARD front-end of kqo_quantize_rows.  Returns 0, or 1 on bad args.
 */
int kqo_quantize_rows_hadamard(const uint16_t* X, int64_t T, int64_t d, int B, int64_t row0, int64_t row1,
                               uint8_t* codes, uint8_t* scales, float* y32, double* yhat);

/*
 * 16-wide KroQuant blocks with four factors (a block-size / factor-count
 * variant; Pith review, "What carries the argument" and minor comments): for
 * each 16-channel block b the 16x16 matrix G1 (x) G2 (x) G3 (x) G4 (G1 on bit
 * 3 of the index, 12 scalars at P + 12 b), each entry the fp64 product in
 * factor order rounded once to fp32.  Written as block-diagonal 32x32 fp32
 * blocks diag(K_{2j}, K_{2j+1}) into K32 [nb16/2][32][32] (zeros elsewhere),
 * ready for kqo_quantize_rows_blocks; nb16 must be even.
 */
void kqo_build_blocks16(const float* P, int64_t nb16, float* K32);

/* MXFP4 dequantization: out[t][c] = E2M1(code) * 2^(scale - 127) in fp64 ([n][d]). */
void kqo_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t d, double* out);

/* E2M1 magnitude index (0..7) of |v| under round-to-nearest-even with saturation. */
int kqo_e2m1_index(double m);
/* E8M0 scale byte for a block amax: floor(log2 amax) - 2 + 127 clamped to [0, 254]; amax == 0 -> 0. */
uint8_t kqo_e8m0(float amax);
/* Quantize one block of 32 fp32 values: 16 packed code bytes + 1 scale byte. */
void kqo_quantize_block(const float y[32], uint8_t codes[16], uint8_t* scale);

/*
 * Whole path for rows [row0, row1) of X[T][d] (bf16 bits):
 *   front = KQO_KRON     y = x K(j), params at P + j*pstride
 *           KQO_PLAIN    y = x
 *           KQO_SMOOTH   y = fp32(x * m[c])
 *           KQO_HADAMARD y = fp32((x H32)[c] / sqrt(32)), H32[r][c] = (-1)^popcount(r & c)
 * Outputs are written for the requested rows only, starting at row 0 of each
 * output: codes [(row1-row0)][d/2], scales [(row1-row0)][d/32], and when not
 * NULL y32 (the fp32 values that were quantized) and yhat (the fp64 value
 * before the final rounding).  Returns 0, or 1 on bad arguments.
 */
int kqo_quantize_rows(int front, const uint16_t* X, int64_t T, int64_t d, const float* P, int64_t pstride,
                      const float* m, int64_t row0, int64_t row1, uint8_t* codes, uint8_t* scales, float* y32,
                      double* yhat);

/* MXFP4 of given fp32 values Y[n][d] (steps after the transform only). */
int kqo_quantize_f32_rows(const float* Y, int64_t n, int64_t d, uint8_t* codes, uint8_t* scales);

/*
 * Producer step in front of the quantizer (AdaLN: the Pith review's summary
 * gives AdaLN as the reason the transform must run online, and its ledger
 * lists LayerNorm / AdaLN as normalisations that do not commute with it; the
 * handbook page "Quantization: where diffusion differs from an LLM" describes
 * AdaLN as timestep-dependent per-channel scales and shifts).
 *
 * kqo_row_stats: LayerNorm statistics without affine parameters, per row:
 *   mean = (sum_c x) / d, var = (sum_c (x - mean)^2) / d, both summed in fp64
 *   in channel order; rstd = 1 / sqrt(var + eps) in fp64; stored as the fp32
 *   pair (mean, rstd) at stats[2t], stats[2t+1].  Returns 0, or 1 on bad args.
 */
int kqo_row_stats(const uint16_t* X, int64_t T, int64_t d, double eps, float* stats);
/*
 * kqo_adaln_rows: the modulated activation, per element in fp32, one IEEE
 * operation each and in this order (no contraction):
 *   v = x                                  (bf16 -> fp32, exact)
 *   v = (v - mean_t) * rstd_t              if stats != NULL
 *   v = v * (1 + scale[s][c])              if mscale != NULL; (1 + scale) is one fp32 add
 *   v = v + shift[s][c]                    if mshift != NULL
 * with s = t / tokens_per_sample (scale, shift: fp32 [n_samples][d]), then
 * rounded to bf16 (nearest even) into Xmod [T][d].  Returns 0, or 1.
 */
int kqo_adaln_rows(const uint16_t* X, int64_t T, int64_t d, const float* stats, const float* mscale,
                   const float* mshift, int64_t tokens_per_sample, uint16_t* Xmod);

/* Fast Walsh-Hadamard transform of 32 values in place (natural order, unnormalized). */
void kqo_fwht32(double v[32]);
/* Determinant of an n x n fp64 matrix by LU with partial pivoting. */
double kqo_det(const double* A, int n);

#ifdef __cplusplus
}
#endif
#endif
