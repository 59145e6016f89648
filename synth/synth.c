/*
 * Seeded synthetic inputs for the KroQuant activation quantizer.
 *
 * This file builds inputs only: bf16 activation matrices shaped like the DiT
 * linear-layer inputs the KroQuant paper measures (PixArt-Sigma, SANA and
 * FLUX.1-schnell widths; Pith review of arXiv 2607.21446, "Summary" and
 * Table 1 setting), per-block transform parameters drawn around the
 * identity, and SmoothQuant-style channel multipliers.  It contains none of
 * the quantizer's arithmetic.  The CPU oracle and the HIP library both read
 * the buffers it writes; neither links this file.
 *
 * Random numbers come from a counter-based generator: every value is a pure
 * function of (seed, stream, index), so a buffer is the same whatever the
 * thread count, and any element can be regenerated alone.
 *   u64(seed, stream, i) = mix64(seed*PHI + stream*C2 + i)
 *   mix64 = the SplitMix64 output function (Steele, Lea, Flood, "Fast
 *           splittable pseudorandom number generators", OOPSLA 2014).
 *   uniform in (0,1) = ((u64 >> 11) + 0.5) * 2^-53
 *   normal = Box-Muller cosine branch on uniforms (2k, 2k+1) of a stream.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static const uint64_t PHI = 0x9E3779B97F4A7C15ull;
static const uint64_t C2 = 0xD1B54A32D192ED03ull;

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t i) {
  return mix64(seed * PHI + stream * C2 + i);
}

double synth_uniform(uint64_t seed, uint64_t stream, uint64_t i) {
  return ((double)(synth_u64(seed, stream, i) >> 11) + 0.5) * 0x1.0p-53;
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t k) {
  double u1 = synth_uniform(seed, stream, 2 * k);
  double u2 = synth_uniform(seed, stream, 2 * k + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* float -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* Stream numbering: (matrix_id << 8) | purpose. */
enum {
  S_BASE0 = 1, S_BASE1 = 2, S_BASE2 = 3, S_BASE3 = 4, /* up to four normals per element */
  S_TOKEN = 5, S_OUTLIER = 6, S_ZERO = 7,
  S_PL = 10, S_PA = 11, S_PB = 12
};

/* base value kinds */
enum { BASE_NORMAL = 0, BASE_GELU = 1, BASE_STUDENT_T3 = 2 };

typedef struct {
  uint16_t* X;
  int64_t T, d;
  uint64_t seed, mid;
  int kind;
  double token_sigma;
  const double* chan_mult; /* [d] */
  double zero_frac;
  int64_t row0, row1;
} job_t;

static void* run_rows(void* arg) {
  job_t* j = (job_t*)arg;
  const uint64_t sb = j->mid << 8;
  const int64_t nb = j->d / 32;
  for (int64_t t = j->row0; t < j->row1; ++t) {
    double tok = 1.0;
    if (j->token_sigma > 0.0) tok = 1.0 + j->token_sigma * synth_normal(j->seed, sb | S_TOKEN, (uint64_t)t);
    for (int64_t c = 0; c < j->d; ++c) {
      uint64_t i = (uint64_t)(t * j->d + c);
      double v;
      if (j->kind == BASE_NORMAL) {
        v = synth_normal(j->seed, sb | S_BASE0, i);
      } else if (j->kind == BASE_GELU) {
        double z0 = synth_normal(j->seed, sb | S_BASE0, i);
        double z1 = synth_normal(j->seed, sb | S_BASE1, i);
        v = (z0 > 0.0 ? z0 : 0.0) + 0.05 * z1;
      } else {
        double z0 = synth_normal(j->seed, sb | S_BASE0, i);
        double z1 = synth_normal(j->seed, sb | S_BASE1, i);
        double z2 = synth_normal(j->seed, sb | S_BASE2, i);
        double z3 = synth_normal(j->seed, sb | S_BASE3, i);
        v = z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
      }
      v *= tok * j->chan_mult[c];
      j->X[t * j->d + c] = f32_to_bf16((float)v);
    }
    if (j->zero_frac > 0.0) {
      for (int64_t b = 0; b < nb; ++b) {
        if (synth_uniform(j->seed, sb | S_ZERO, (uint64_t)(t * nb + b)) < j->zero_frac)
          memset(j->X + t * j->d + 32 * b, 0, 64);
      }
    }
  }
  return NULL;
}

/*
 * Fill X[T][d] (bf16 bits).  n_outliers channels, chosen uniformly without
 * replacement (partial Fisher-Yates), are multiplied by outlier_mult; the
 * chosen channel indices are written to outliers_out (may be NULL).  Every
 * row is scaled by (1 + token_sigma * N(0,1)) when token_sigma > 0.  With
 * zero_frac > 0, each 32-channel group of a row is zeroed with that
 * probability.  Returns 0 on success.
 */
int synth_matrix(uint16_t* X, int64_t T, int64_t d, uint64_t seed, uint64_t matrix_id, int kind,
                 int64_t n_outliers, double outlier_mult, double token_sigma, double zero_frac,
                 int n_threads, int64_t* outliers_out) {
  if (!X || T < 0 || d <= 0 || d % 32 != 0 || n_outliers < 0 || n_outliers > d) return 1;
  double* mult = (double*)malloc(sizeof(double) * (size_t)d);
  int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)d);
  if (!mult || !perm) { free(mult); free(perm); return 2; }
  for (int64_t c = 0; c < d; ++c) { mult[c] = 1.0; perm[c] = c; }
  const uint64_t sb = matrix_id << 8;
  for (int64_t k = 0; k < n_outliers; ++k) {
    int64_t r = k + (int64_t)(synth_u64(seed, sb | S_OUTLIER, (uint64_t)k) % (uint64_t)(d - k));
    int64_t tmp = perm[k]; perm[k] = perm[r]; perm[r] = tmp;
    mult[perm[k]] = outlier_mult;
    if (outliers_out) outliers_out[k] = perm[k];
  }
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 64) n_threads = 64;
  if ((int64_t)n_threads > T) n_threads = T > 0 ? (int)T : 1;
  pthread_t th[64];
  int created[64];
  job_t jobs[64];
  int64_t per = (T + n_threads - 1) / n_threads;
  for (int i = 0; i < n_threads; ++i) {
    int64_t r0 = i * per, r1 = (i + 1) * per < T ? (i + 1) * per : T;
    jobs[i] = (job_t){X, T, d, seed, matrix_id, kind, token_sigma, mult, zero_frac, r0, r1};
    created[i] = 0;
    if (r0 >= r1) continue;
    if (n_threads > 1 && pthread_create(&th[i], NULL, run_rows, &jobs[i]) == 0) created[i] = 1;
    else run_rows(&jobs[i]);
  }
  for (int i = 0; i < n_threads; ++i)
    if (created[i]) pthread_join(th[i], NULL);
  free(mult);
  free(perm);
  return 0;
}

/*
 * Per-block transform parameters, layout [nb][5][3] with (l, a, b) per
 * factor, factor 1 first: l, b ~ N(0, sigma_lb), a = exp(N(0, sigma_a)).
 * special_blocks = 1 sets block 0 to the identity factors (l=0, a=1, b=0)
 * and block 1 to the Hadamard-like factors (l=1, a=1/sqrt2, b=-1/sqrt2).
 */
int synth_params(float* P, int64_t nb, uint64_t seed, uint64_t matrix_id, double sigma_lb,
                 double sigma_a, int special_blocks) {
  if (!P || nb <= 0) return 1;
  const uint64_t sb = matrix_id << 8;
  for (int64_t j = 0; j < nb; ++j) {
    for (int k = 0; k < 5; ++k) {
      uint64_t i = (uint64_t)(j * 5 + k);
      double l = sigma_lb * synth_normal(seed, sb | S_PL, i);
      double a = exp(sigma_a * synth_normal(seed, sb | S_PA, i));
      double b = sigma_lb * synth_normal(seed, sb | S_PB, i);
      if (special_blocks && j == 0) { l = 0.0; a = 1.0; b = 0.0; }
      if (special_blocks && j == 1) { l = 1.0; a = 0.70710678118654752440; b = -0.70710678118654752440; }
      P[(j * 5 + k) * 3 + 0] = (float)l;
      P[(j * 5 + k) * 3 + 1] = (float)a;
      P[(j * 5 + k) * 3 + 2] = (float)b;
    }
  }
  return 0;
}

/*
 * SmoothQuant-style channel multipliers m_c = 1 / s_c with
 * s_c = max_t |X[t,c]|^0.5 (migration strength 0.5, weight term 1); a column
 * that is all zero gets m_c = 1.  The multipliers only need a realistic
 * spread: the kernel's cost does not depend on their values.
 */
int synth_smooth_mult(const uint16_t* X, int64_t T, int64_t d, float* m) {
  if (!X || !m || d <= 0) return 1;
  float* amax = (float*)calloc((size_t)d, sizeof(float));
  if (!amax) return 2;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < d; ++c) {
      uint32_t b = (uint32_t)(X[t * d + c] & 0x7FFFu) << 16;
      float f;
      memcpy(&f, &b, 4);
      if (f > amax[c]) amax[c] = f;
    }
  for (int64_t c = 0; c < d; ++c) m[c] = amax[c] > 0.0f ? (float)(1.0 / sqrt((double)amax[c])) : 1.0f;
  free(amax);
  return 0;
}

/*
 * AdaLN modulation vectors, fp32 [n_samples][d] each: scale = sigma * N(0,1)
 * with every channel in `amplified` (a uniform sample of round(frac * d)
 * channels, the same for every sample) raised by `amp`, and shift =
 * sigma * N(0,1).  AdaLN multiplies timestep-dependent scales onto the
 * activations and amplifies a few channels many times over (handbook page
 * "Quantization: where diffusion differs from an LLM", differences list).
 */
int synth_adaln(float* scale, float* shift, int64_t n_samples, int64_t d, uint64_t seed, uint64_t matrix_id,
                double sigma, double frac, double amp) {
  if (!scale || !shift || n_samples <= 0 || d <= 0) return 1;
  const uint64_t base = matrix_id << 8;
  for (int64_t i = 0; i < n_samples * d; ++i) {
    scale[i] = (float)(sigma * synth_normal(seed, base | 20u, (uint64_t)i));
    shift[i] = (float)(sigma * synth_normal(seed, base | 21u, (uint64_t)i));
  }
  const int64_t k = (int64_t)(frac * (double)d + 0.5);
  if (k <= 0) return 0;
  int64_t* idx = (int64_t*)malloc((size_t)d * sizeof(int64_t));
  if (!idx) return 2;
  for (int64_t c = 0; c < d; ++c) idx[c] = c;
  for (int64_t c = 0; c < k && c < d; ++c) {  // partial Fisher-Yates
    const int64_t r = c + (int64_t)(synth_uniform(seed, base | 22u, (uint64_t)c) * (double)(d - c));
    const int64_t tmp = idx[c];
    idx[c] = idx[r < d ? r : d - 1];
    idx[r < d ? r : d - 1] = tmp;
  }
  for (int64_t s = 0; s < n_samples; ++s)
    for (int64_t c = 0; c < k && c < d; ++c) scale[s * d + idx[c]] += (float)amp;
  free(idx);
  return 0;
}
