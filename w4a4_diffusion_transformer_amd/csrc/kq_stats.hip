// LayerNorm row statistics for the AdaLN producer step in front of the
// quantizer (gfx950).
//
// The normalisation in front of a DiT linear layer's AdaLN modulation is a
// LayerNorm without affine parameters; the Pith review's summary gives AdaLN
// as the reason KroQuant's transform runs online, and its ledger lists
// LayerNorm and AdaLN among the normalisations that do not commute with it.
// Per row: mean = sum(x) / d and var = sum((x - mean)^2) / d, both summed in
// fp64, rstd = 1 / sqrt(var + eps) in fp64, stored as the fp32 pair
// (mean, rstd).  The sums are exact or nearly so in fp64 (bf16 inputs), so
// the fp32 results agree with a sequential evaluation except, rarely, by one
// ulp.  Rows held in registers take sum (x - mean)^2 as sum x^2 - mean sum x
// from one pass when that is accurate to about 2^-40 (below), else in a
// second pass.
//
// Rows up to 8192 channels: one wave per row, no LDS and no barriers; lane
// l holds the row's 16-byte pieces l, l + 64, ... in registers (4, 8, 12 or
// 16 of them), so the row is read from HBM once, and both sums are reduced
// with wave shuffles.  Rows up to 16384 channels: one four-wave workgroup
// per row, the row again held in registers, the sums reduced across the
// waves through LDS.  Longer rows:
// the same workgroup shape in two passes over memory.  Rows are grid-strided
// over a launch sized to fill the GPU once.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ double piece_sum(u32x4 v) {
#pragma clang fp contract(off)
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += (double)bf16_lo(v[k]) + (double)bf16_hi(v[k]);
  return s;
}

// Sum of squares of a piece's 8 values (each square exact in fp64).
__device__ __forceinline__ double piece_sumsq(u32x4 v) {
#pragma clang fp contract(off)
  double q = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double u0 = (double)bf16_lo(v[k]), u1 = (double)bf16_hi(v[k]);
    q += u0 * u0;
    q += u1 * u1;
  }
  return q;
}

__device__ __forceinline__ double piece_sq(u32x4 v, double mean) {
#pragma clang fp contract(off)
  double q = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double u0 = (double)bf16_lo(v[k]) - mean;
    const double u1 = (double)bf16_hi(v[k]) - mean;
    q += u0 * u0;
    q += u1 * u1;
  }
  return q;
}

// Sum over the WPR waves of one row (WPR > 1: the whole workgroup is one row).
template <int WPR>
__device__ __forceinline__ double row_sum(double v, double* red) {
  v = wave_sum(v);
  if constexpr (WPR > 1) {
    const int w = threadIdx.x >> 6;
    __syncthreads();  // red[] may still be read from the previous reduction
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = 0.0;
#pragma unroll
    for (int i = 0; i < WPR; ++i) v += red[i];
  }
  return v;
}

// Both sums of a row at once (one exchange through LDS for WPR > 1).
template <int WPR>
__device__ __forceinline__ void row_sum2(double& a, double& b, double* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  if constexpr (WPR > 1) {
    const int w = threadIdx.x >> 6;
    __syncthreads();  // red[] may still be read from the previous reduction
    if ((threadIdx.x & 63) == 0) {
      red[w] = a;
      red[kWaves + w] = b;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
#pragma unroll
    for (int i = 0; i < WPR; ++i) {
      a += red[i];
      b += red[kWaves + i];
    }
  }
}

// WPR waves per row (1: each wave its own row; kWaves: the workgroup), MAXP
// register-resident 16-byte pieces per thread (0: two passes over memory).
template <int WPR, int MAXP>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(const uint16_t* __restrict__ X, int T, int d,
                                                             double eps, float* __restrict__ stats) {
#pragma clang fp contract(off)
  __shared__ double red[2 * kWaves];
  constexpr int kRowThreads = 64 * WPR, kRowsPerStep = kWaves / WPR;
  const int t = threadIdx.x % kRowThreads;
  const int slot = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kRowThreads));
  const int npieces = d >> 3;  // 8 bf16 per 16-byte piece
  const int step = gridDim.x * kRowsPerStep;
  for (int row = blockIdx.x * kRowsPerStep + slot; row < T; row += step) {
    const auto rx = rsrc_uniform(X + (int64_t)row * d, (int64_t)d * 2);  // pieces past the row read as zero
    double s = 0.0, qs = 0.0, mean;
    if constexpr (MAXP > 0) {
      // all of the row's loads first (the scheduler would otherwise hold some
      // back behind the sums of the first pieces, a memory round trip each);
      // pieces wholly past the row are neither loaded nor summed
      u32x4 v[MAXP];
#pragma unroll
      for (int k = 0; k < MAXP; ++k) {
        const int p = t + kRowThreads * k;
        v[k] = u32x4{0u, 0u, 0u, 0u};
        if (kRowThreads * k < npieces)  // uniform
          v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, p < npieces ? (uint32_t)(16 * p) : kOut, 0, kNT);
      }
      __builtin_amdgcn_sched_barrier(0);
      // One pass over the registers: S = sum x and Q = sum x^2 (pieces past
      // the row are zero), then sum (x - mean)^2 = Q - S mean.  That
      // difference carries an error of a few units in 2^-52 of Q, so it is
      // used only while Q <= 2^12 (Q - S mean): then var is accurate to
      // about 2^-40 and its fp32 rstd rounds as the two-pass value's does
      // except within that distance of a tie.  Other rows (a mean far larger
      // than the spread) take the two-pass sum from the registers.
      double q1 = 0.0;
#pragma unroll
      for (int k = 0; k < MAXP; ++k) {
        if (kRowThreads * k < npieces) {  // uniform
          s += piece_sum(v[k]);
          q1 += piece_sumsq(v[k]);
        }
      }
      double S = s, Q = q1;
      row_sum2<WPR>(S, Q, red);
      mean = S / (double)d;
      const double m2 = Q - S * mean;
      if (m2 * 0x1p12 >= Q) {  // uniform over the row
        const double var = m2 / (double)d;
        if (t == 0) {
          stats[2 * (int64_t)row] = (float)mean;
          stats[2 * (int64_t)row + 1] = (float)(1.0 / sqrt(var + eps));
        }
        continue;
      }
      // (the values are converted again here: an empty asm on the raw
      // pieces keeps the compiler from holding all their fp64 conversions
      // in registers across the test above, which would cost occupancy)
#pragma unroll
      for (int k = 0; k < MAXP; ++k) asm volatile("" : "+v"(v[k]));
#pragma unroll
      for (int k = 0; k < MAXP; ++k)
        if (t + kRowThreads * k < npieces) qs += piece_sq(v[k], mean);
    } else {
#pragma unroll 4
      for (int p = t; p < npieces; p += kRowThreads)
        s += piece_sum(__builtin_amdgcn_raw_buffer_load_b128(rx, 16 * p, 0, 0));
      mean = row_sum<WPR>(s, red) / (double)d;
#pragma unroll 4
      for (int p = t; p < npieces; p += kRowThreads)
        qs += piece_sq(__builtin_amdgcn_raw_buffer_load_b128(rx, 16 * p, 0, 0), mean);
    }
    const double var = row_sum<WPR>(qs, red) / (double)d;
    if (t == 0) {
      stats[2 * (int64_t)row] = (float)mean;
      stats[2 * (int64_t)row + 1] = (float)(1.0 / sqrt(var + eps));
    }
  }
}

}  // namespace

hipError_t launch_row_stats(const uint16_t* X, int T, int d, double eps, float* stats, hipStream_t stream) {
  const int pieces = d / 8;  // 16-byte pieces per row
  const void* fn;
  int rows_per_wg;
  if (pieces <= 64 * 4) {
    fn = (const void*)&row_stats_kernel<1, 4>;
    rows_per_wg = kWaves;
  } else if (pieces <= 64 * 8) {
    fn = (const void*)&row_stats_kernel<1, 8>;
    rows_per_wg = kWaves;
  } else if (pieces <= 64 * 12) {
    fn = (const void*)&row_stats_kernel<1, 12>;
    rows_per_wg = kWaves;
  } else if (pieces <= 64 * 16) {
    fn = (const void*)&row_stats_kernel<1, 16>;
    rows_per_wg = kWaves;
  } else if (pieces <= kThreads * 8) {
    fn = (const void*)&row_stats_kernel<kWaves, 8>;
    rows_per_wg = 1;
  } else {
    fn = (const void*)&row_stats_kernel<kWaves, 0>;
    rows_per_wg = 1;
  }
  const int64_t slots = (int64_t)cu_count() * resident_per_cu(fn, kThreads);
  const int64_t need = ((int64_t)T + rows_per_wg - 1) / rows_per_wg;
  const int grid = (int)(need < slots ? need : slots);
  if (grid == 0) return hipSuccess;
  void* kargs[] = {&X, &T, &d, &eps, &stats};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace kq
