/*
 * CPU oracle for the KroQuant online activation quantizer.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
 * See kq_oracle.h for the method summary and its sources.
 *
 * Built with -O2 -ffp-contract=off, no fast-math: every fp64 operation below
 * is one IEEE round-to-nearest-even operation, in the order written.
 */
#include "kq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

static float bf16_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/*
 * One Kronecker factor (Pith review, referee report on Sec. 3.2 Eq. (6):
 * G_k = L_k U_k, unit-determinant LU form, three scalars per factor).
 * Reading: L = [[1,0],[l,1]], U = [[a,b],[0,1/a]] (determinant +1; the
 * review's quoted U with -1/a would give determinant -1).  Expanded:
 * G = [[a, b], [l a, l b + 1/a]].
 */
void kqo_factor(float l, float a, float b, double G[4]) {
  const double L = l, A = a, B = b;
  const double inv_a = 1.0 / A;
  G[0] = A;
  G[1] = B;
  G[2] = L * A;
  G[3] = L * B + inv_a;
}

/* G^-1 = U^-1 L^-1 = [[1/a, -b], [0, a]] [[1,0],[-l,1]] = [[1/a + l b, -b], [-l a, a]]. */
void kqo_factor_inverse(float l, float a, float b, double Gi[4]) {
  const double L = l, A = a, B = b;
  Gi[0] = L * B + 1.0 / A;
  Gi[1] = -B;
  Gi[2] = -(L * A);
  Gi[3] = A;
}

/* Bit of index i that factor k (0-based, k = 0 is G1) acts on: G1 on the most significant of 5 bits. */
static int kbit(int i, int k) { return (i >> (4 - k)) & 1; }

/*
 * K = G1 (x) G2 (x) G3 (x) G4 (x) G5 (Pith review, "What carries the
 * argument" and core claim: a 32x32 block is the Kronecker product of five
 * 2x2 factors).  Standard Kronecker index order: G1 on bit 4 of the row and
 * column index, G5 on bit 0.  The entry is the product of one entry of each
 * factor, multiplied left to right (G1 first).
 */
void kqo_kron_dense(const float P[15], double K[1024]) {
  double G[5][4];
  for (int k = 0; k < 5; ++k) kqo_factor(P[3 * k], P[3 * k + 1], P[3 * k + 2], G[k]);
  for (int r = 0; r < 32; ++r)
    for (int c = 0; c < 32; ++c) {
      double p = G[0][2 * kbit(r, 0) + kbit(c, 0)];
      for (int k = 1; k < 5; ++k) p = p * G[k][2 * kbit(r, k) + kbit(c, k)];
      K[r * 32 + c] = p;
    }
}

/*
 * Row r of K is e_r K.  Multiplying a row vector by G1 (x) ... (x) G5 is the
 * same as applying each factor to the index bit it owns, one stage per
 * factor (mixed-product property): for every pair (v0, v1) of entries whose
 * indices differ only in that bit, (v0, v1) <- (v0, v1) G.
 */
void kqo_kron_butterfly(const float P[15], double K[1024]) {
  double G[5][4];
  for (int k = 0; k < 5; ++k) kqo_factor(P[3 * k], P[3 * k + 1], P[3 * k + 2], G[k]);
  for (int r = 0; r < 32; ++r) {
    double v[32];
    for (int c = 0; c < 32; ++c) v[c] = (c == r) ? 1.0 : 0.0;
    for (int k = 0; k < 5; ++k) {
      const int bit = 1 << (4 - k);
      for (int c0 = 0; c0 < 32; ++c0) {
        if (c0 & bit) continue;
        const int c1 = c0 | bit;
        const double v0 = v[c0], v1 = v[c1];
        v[c0] = v0 * G[k][0] + v1 * G[k][2];
        v[c1] = v0 * G[k][1] + v1 * G[k][3];
      }
    }
    for (int c = 0; c < 32; ++c) K[r * 32 + c] = v[c];
  }
}

/* (G1 (x) ... (x) G5)^-1 = G1^-1 (x) ... (x) G5^-1 (Pith review, axiom ledger). */
void kqo_kron_inverse(const float P[15], double Kinv[1024]) {
  double G[5][4];
  for (int k = 0; k < 5; ++k) kqo_factor_inverse(P[3 * k], P[3 * k + 1], P[3 * k + 2], G[k]);
  for (int r = 0; r < 32; ++r)
    for (int c = 0; c < 32; ++c) {
      double p = G[0][2 * kbit(r, 0) + kbit(c, 0)];
      for (int k = 1; k < 5; ++k) p = p * G[k][2 * kbit(r, k) + kbit(c, k)];
      Kinv[r * 32 + c] = p;
    }
}

/*
 * Reading: the dense block a kernel multiplies by is K rounded once to fp32
 * (the "precomputed dense blocks" kernel variant of the Pith review,
 * "What carries the argument").
 */
void kqo_block_f32(const float P[15], float K32[1024]) {
  double K[1024];
  kqo_kron_dense(P, K);
  for (int i = 0; i < 1024; ++i) K32[i] = (float)K[i];
}

void kqo_build_blocks(const float* P, int64_t nb, int64_t pstride, float* K32, uint16_t* Kbf, int n_split) {
  for (int64_t j = 0; j < nb; ++j) {
    float k32[1024];
    kqo_block_f32(P + j * pstride, k32);
    if (K32) memcpy(K32 + j * 1024, k32, sizeof k32);
    if (Kbf) {
      for (int r = 0; r < 32; ++r)
        for (int c = 0; c < 32; ++c) {
          float rest = k32[r * 32 + c];
          for (int s = 0; s < n_split; ++s) {
            const uint16_t h = f32_to_bf16_rne(rest);
            Kbf[((j * n_split + s) * 32 + c) * 32 + r] = h;
            rest = rest - bf16_to_f32(h);
          }
        }
    }
  }
}

/*
 * E2M1 element (OCP MX v1.0, FP4 E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
 * at codes 0..7).  Round to nearest; a value exactly halfway goes to the
 * even code; anything above 6 saturates to 6.  Written as the count of grid
 * midpoints that m lies above, where "above" is strict at a midpoint whose
 * lower neighbour has the even code and inclusive where the upper one does.
 */
int kqo_e2m1_index(double m) {
  return (m > 0.25) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5) + (m > 5.0);
}

/*
 * E8M0 shared scale (OCP MX v1.0): X = 2^(floor(log2 amax) - emax_elem) with
 * emax_elem = 2 for E2M1, stored biased by 127.  floor(log2 amax) is taken
 * exactly from the binary exponent (frexp), never from a log.  Readings: an
 * all-zero block gets the smallest scale (byte 0); the result is clamped to
 * [-127, 127], which finite fp32 inputs never reach at the top.
 */
uint8_t kqo_e8m0(float amax) {
  if (amax == 0.0f) return 0;
  int E;
  (void)frexp((double)amax, &E); /* amax = f * 2^E, f in [0.5, 1) -> floor(log2 amax) = E - 1 */
  int e = (E - 1) - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return (uint8_t)(e + 127);
}

void kqo_quantize_block(const float y[32], uint8_t codes[16], uint8_t* scale) {
  float amax = 0.0f;
  for (int c = 0; c < 32; ++c) {
    const float a = fabsf(y[c]);
    if (a > amax) amax = a;
  }
  const uint8_t sb = kqo_e8m0(amax);
  const int e = (int)sb - 127;
  int code[32];
  for (int c = 0; c < 32; ++c) {
    const double v = ldexp((double)y[c], -e); /* exact: a power-of-two scaling in fp64 */
    const int idx = kqo_e2m1_index(fabs(v));
    code[c] = idx | (signbit(y[c]) ? 8 : 0);
  }
  for (int q = 0; q < 16; ++q) codes[q] = (uint8_t)(code[2 * q] | (code[2 * q + 1] << 4));
  *scale = sb;
}

static int popcount5(int v) {
  int n = 0;
  for (int i = 0; i < 5; ++i) n += (v >> i) & 1;
  return n;
}

void kqo_fwht32(double v[32]) {
  for (int h = 1; h < 32; h <<= 1)
    for (int i = 0; i < 32; i += 2 * h)
      for (int k = i; k < i + h; ++k) {
        const double a = v[k], b = v[k + h];
        v[k] = a + b;
        v[k + h] = a - b;
      }
}

double kqo_det(const double* A, int n) {
  double* M = (double*)malloc(sizeof(double) * (size_t)(n * n));
  if (!M) return NAN;
  memcpy(M, A, sizeof(double) * (size_t)(n * n));
  double det = 1.0;
  for (int k = 0; k < n; ++k) {
    int p = k;
    for (int i = k + 1; i < n; ++i)
      if (fabs(M[i * n + k]) > fabs(M[p * n + k])) p = i;
    if (M[p * n + k] == 0.0) { free(M); return 0.0; }
    if (p != k) {
      for (int j = 0; j < n; ++j) { double t = M[k * n + j]; M[k * n + j] = M[p * n + j]; M[p * n + j] = t; }
      det = -det;
    }
    det *= M[k * n + k];
    for (int i = k + 1; i < n; ++i) {
      const double f = M[i * n + k] / M[k * n + k];
      for (int j = k; j < n; ++j) M[i * n + j] -= f * M[k * n + j];
    }
  }
  free(M);
  return det;
}

/*
 * The online path for rows [row0, row1).  Row-vector convention from Eq. (1)
 * as the review quotes it, A T (W T^-T)^T = A W^T: activations are multiplied
 * on the right, y = x K, y[c] = sum_r x[r] K[r][c].  The sum runs in fp64 from
 * +0 in order r = 0..31; every product of a bf16 and an fp32 value is exact in
 * fp64.  The value quantized is that sum rounded once to fp32.
 */
int kqo_quantize_rows(int front, const uint16_t* X, int64_t T, int64_t d, const float* P, int64_t pstride,
                      const float* m, int64_t row0, int64_t row1, uint8_t* codes, uint8_t* scales, float* y32,
                      double* yhat) {
  if (!X || d <= 0 || d % 32 != 0 || T < 0 || row0 < 0 || row1 > T || row0 > row1 || !codes || !scales) return 1;
  if (front == KQO_KRON && (!P || (pstride != 0 && pstride != 15))) return 1;
  if (front == KQO_SMOOTH && !m) return 1;
  if (front < KQO_KRON || front > KQO_HADAMARD) return 1;
  const int64_t nb = d / 32;
  float* K32 = NULL;
  if (front == KQO_KRON) {
    const int64_t nk = pstride == 0 ? 1 : nb;
    K32 = (float*)malloc(sizeof(float) * 1024 * (size_t)nk);
    if (!K32) return 1;
    for (int64_t j = 0; j < nk; ++j) kqo_block_f32(P + j * pstride, K32 + j * 1024);
  }
  const double sqrt32 = sqrt(32.0);
  for (int64_t t = row0; t < row1; ++t) {
    const int64_t ro = t - row0;
    for (int64_t j = 0; j < nb; ++j) {
      double x[32], yh[32];
      float y[32];
      for (int r = 0; r < 32; ++r) x[r] = bf16_to_f64(X[t * d + 32 * j + r]);
      if (front == KQO_KRON) {
        const float* K = K32 + (pstride == 0 ? 0 : j) * 1024;
        for (int c = 0; c < 32; ++c) {
          double s = 0.0;
          for (int r = 0; r < 32; ++r) s = s + x[r] * (double)K[r * 32 + c];
          yh[c] = s;
          y[c] = (float)s;
        }
      } else if (front == KQO_PLAIN) {
        for (int c = 0; c < 32; ++c) { yh[c] = x[c]; y[c] = (float)x[c]; }
      } else if (front == KQO_SMOOTH) {
        for (int c = 0; c < 32; ++c) {
          yh[c] = x[c] * (double)m[32 * j + c];
          y[c] = (float)yh[c];
        }
      } else {
        for (int c = 0; c < 32; ++c) {
          double s = 0.0;
          for (int r = 0; r < 32; ++r) s = s + ((popcount5(r & c) & 1) ? -x[r] : x[r]);
          yh[c] = s / sqrt32;
          y[c] = (float)yh[c];
        }
      }
      kqo_quantize_block(y, codes + ro * (d / 2) + 16 * j, scales + ro * nb + j);
      if (y32) memcpy(y32 + ro * d + 32 * j, y, sizeof y);
      if (yhat) memcpy(yhat + ro * d + 32 * j, yh, sizeof yh);
    }
  }
  free(K32);
  return 0;
}

int kqo_quantize_f32_rows(const float* Y, int64_t n, int64_t d, uint8_t* codes, uint8_t* scales) {
  if (!Y || !codes || !scales || n < 0 || d <= 0 || d % 32 != 0) return 1;
  const int64_t nb = d / 32;
  for (int64_t t = 0; t < n; ++t)
    for (int64_t j = 0; j < nb; ++j) kqo_quantize_block(Y + t * d + 32 * j, codes + t * (d / 2) + 16 * j, scales + t * nb + j);
  return 0;
}

/*
 * LayerNorm statistics (see kq_oracle.h): two passes over the row in fp64,
 * channel order, then one fp64 division and square root for rstd.
 */
int kqo_row_stats(const uint16_t* X, int64_t T, int64_t d, double eps, float* stats) {
  if (!X || !stats || T < 0 || d <= 0 || !(eps >= 0.0)) return 1;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* x = X + t * d;
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += bf16_to_f64(x[c]);
    const double mean = s / (double)d;
    double q = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      const double u = bf16_to_f64(x[c]) - mean;
      q += u * u;
    }
    const double var = q / (double)d;
    stats[2 * t] = (float)mean;
    stats[2 * t + 1] = (float)(1.0 / sqrt(var + eps));
  }
  return 0;
}

/* The modulated activation (see kq_oracle.h): fp32 steps in the stated order. */
int kqo_adaln_rows(const uint16_t* X, int64_t T, int64_t d, const float* stats, const float* mscale,
                   const float* mshift, int64_t tokens_per_sample, uint16_t* Xmod) {
  if (!X || !Xmod || T < 0 || d <= 0 || tokens_per_sample <= 0) return 1;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t s = t / tokens_per_sample;
    for (int64_t c = 0; c < d; ++c) {
      float v = bf16_to_f32(X[t * d + c]);
      if (stats) {
        const float centred = v - stats[2 * t];
        v = centred * stats[2 * t + 1];
      }
      if (mscale) {
        const float one_plus = 1.0f + mscale[s * d + c];
        v = v * one_plus;
      }
      if (mshift) v = v + mshift[s * d + c];
      Xmod[t * d + c] = f32_to_bf16_rne(v);
    }
  }
  return 0;
}

/* The bf16 split of one fp32 block into n_split terms, stored transposed ([s][c][r]). */
static void split_block(const float k32[1024], uint16_t* Kbf_block, int n_split) {
  for (int r = 0; r < 32; ++r)
    for (int c = 0; c < 32; ++c) {
      float rest = k32[r * 32 + c];
      for (int s = 0; s < n_split; ++s) {
        const uint16_t h = f32_to_bf16_rne(rest);
        Kbf_block[(s * 32 + c) * 32 + r] = h;
        rest = rest - bf16_to_f32(h);
      }
    }
}

void kqo_build_blocks_inverse_t(const float* P, int64_t nb, int64_t pstride, float* K32, uint16_t* Kbf,
                                int n_split) {
  for (int64_t j = 0; j < nb; ++j) {
    double Kinv[1024];
    kqo_kron_inverse(P + j * pstride, Kinv);
    float k32[1024];
    for (int r = 0; r < 32; ++r)
      for (int c = 0; c < 32; ++c) k32[r * 32 + c] = (float)Kinv[c * 32 + r];  /* transpose */
    if (K32) memcpy(K32 + j * 1024, k32, sizeof k32);
    if (Kbf) split_block(k32, Kbf + j * (int64_t)n_split * 1024, n_split);
  }
}

/* E2M1 magnitudes by index and the E8M0 scale (OCP MX v1.0). */
void kqo_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t d, double* out) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  for (int64_t t = 0; t < n; ++t)
    for (int64_t c = 0; c < d; ++c) {
      const uint8_t byte = codes[t * (d / 2) + c / 2];
      const int code = (c & 1) ? (byte >> 4) : (byte & 15);
      const double v = mag[code & 7] * ldexp(1.0, (int)scales[t * (d / 32) + c / 32] - 127);
      out[t * d + c] = (code & 8) ? -v : v;
    }
}

/*
 * The KroQuant front-end with the fp32 blocks given instead of their 15
 * scalars (K32 [nb][32 r][32 c], block j at K32 + j * kstride, kstride 1024
 * or 0): y = RNE_fp32(sum_r x[r] K[r][c]) with the fp64 sum of exact
 * products, then MXFP4, exactly as kqo_quantize_rows does for KQO_KRON.  Used
 * for the weight fold with the blocks of kqo_build_blocks_inverse_t.
 */
int kqo_quantize_rows_blocks(const uint16_t* X, int64_t T, int64_t d, const float* K32, int64_t kstride,
                             int64_t row0, int64_t row1, uint8_t* codes, uint8_t* scales, float* y32, double* yhat) {
  if (!X || !K32 || d <= 0 || d % 32 != 0 || T < 0 || row0 < 0 || row1 > T || row0 > row1 || !codes || !scales ||
      (kstride != 0 && kstride != 1024))
    return 1;
  const int64_t nb = d / 32;
  for (int64_t t = row0; t < row1; ++t) {
    const int64_t ro = t - row0;
    for (int64_t j = 0; j < nb; ++j) {
      double x[32], yh[32];
      float y[32];
      for (int r = 0; r < 32; ++r) x[r] = bf16_to_f64(X[t * d + 32 * j + r]);
      const float* K = K32 + j * kstride;
      for (int cc = 0; cc < 32; ++cc) {
        double s = 0.0;
        for (int r = 0; r < 32; ++r) s = s + x[r] * (double)K[r * 32 + cc];
        yh[cc] = s;
        y[cc] = (float)s;
      }
      kqo_quantize_block(y, codes + ro * (d / 2) + 16 * j, scales + ro * nb + j);
      if (y32) memcpy(y32 + ro * d + 32 * j, y, sizeof y);
      if (yhat) memcpy(yhat + ro * d + 32 * j, yh, sizeof yh);
    }
  }
  return 0;
}

int kqo_quantize_rows_hadamard(const uint16_t* X, int64_t T, int64_t d, int B, int64_t row0, int64_t row1,
                               uint8_t* codes, uint8_t* scales, float* y32, double* yhat) {
  if (!X || !codes || !scales || B < 32 || B > 512 || (B & (B - 1)) || d <= 0 || d % B != 0 || T < 0 || row0 < 0 ||
      row1 > T || row0 > row1)
    return 1;
  const double sqrtB = sqrt((double)B);
  const int64_t nb = d / 32;
  double* yh = (double*)malloc(sizeof(double) * (size_t)d);
  float* y = (float*)malloc(sizeof(float) * (size_t)d);
  if (!yh || !y) { free(yh); free(y); return 1; }
  for (int64_t t = row0; t < row1; ++t) {
    const int64_t ro = t - row0;
    for (int64_t b0 = 0; b0 < d; b0 += B) {
      for (int c = 0; c < B; ++c) {
        double s = 0.0;
        for (int r = 0; r < B; ++r) {
          const double x = bf16_to_f64(X[t * d + b0 + r]);
          s = s + ((__builtin_popcount((unsigned)(r & c)) & 1) ? -x : x);
        }
        yh[b0 + c] = s / sqrtB;
        y[b0 + c] = (float)yh[b0 + c];
      }
    }
    for (int64_t j = 0; j < nb; ++j) kqo_quantize_block(y + 32 * j, codes + ro * (d / 2) + 16 * j, scales + ro * nb + j);
    if (y32) memcpy(y32 + ro * d, y, sizeof(float) * (size_t)d);
    if (yhat) memcpy(yhat + ro * d, yh, sizeof(double) * (size_t)d);
  }
  free(yh);
  free(y);
  return 0;
}

void kqo_build_blocks16(const float* P, int64_t nb16, float* K32) {
  for (int64_t j = 0; j < nb16 / 2; ++j) {
    float* K = K32 + j * 1024;
    for (int i = 0; i < 1024; ++i) K[i] = 0.0f;
    for (int h = 0; h < 2; ++h) {
      double G[4][4];
      const float* p = P + (2 * j + h) * 12;
      for (int k = 0; k < 4; ++k) kqo_factor(p[3 * k], p[3 * k + 1], p[3 * k + 2], G[k]);
      for (int r = 0; r < 16; ++r)
        for (int cc = 0; cc < 16; ++cc) {
          double v = G[0][2 * ((r >> 3) & 1) + ((cc >> 3) & 1)];
          for (int k = 1; k < 4; ++k) v = v * G[k][2 * ((r >> (3 - k)) & 1) + ((cc >> (3 - k)) & 1)];
          K[(16 * h + r) * 32 + 16 * h + cc] = (float)v;
        }
    }
  }
}
