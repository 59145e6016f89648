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
// ulp.
//
// One workgroup per row (grid-strided): two passes over the row, the second
// served mostly from L2, block reductions through LDS.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red[] may still be read from the previous reduction
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) s += red[i];
  return s;
}

__global__ __launch_bounds__(kThreads) void row_stats_kernel(const uint16_t* __restrict__ X, int T, int d,
                                                             double eps, float* __restrict__ stats) {
#pragma clang fp contract(off)
  __shared__ double red[kThreads / 64];
  const int npieces = d >> 3;  // 8 bf16 per 16-byte piece
  for (int row = blockIdx.x; row < T; row += gridDim.x) {
    const u32x4* x = reinterpret_cast<const u32x4*>(X + (int64_t)row * d);
    double s = 0.0;
    for (int p = threadIdx.x; p < npieces; p += kThreads) {
      const u32x4 v = x[p];
#pragma unroll
      for (int k = 0; k < 4; ++k) s += (double)bf16_lo(v[k]) + (double)bf16_hi(v[k]);
    }
    const double mean = block_sum(s, red) / (double)d;
    double qs = 0.0;
    for (int p = threadIdx.x; p < npieces; p += kThreads) {
      const u32x4 v = x[p];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double u0 = (double)bf16_lo(v[k]) - mean;
        const double u1 = (double)bf16_hi(v[k]) - mean;
        qs += u0 * u0;
        qs += u1 * u1;
      }
    }
    const double var = block_sum(qs, red) / (double)d;
    if (threadIdx.x == 0) {
      stats[2 * (int64_t)row] = (float)mean;
      stats[2 * (int64_t)row + 1] = (float)(1.0 / sqrt(var + eps));
    }
  }
}

}  // namespace

hipError_t launch_row_stats(const uint16_t* X, int T, int d, double eps, float* stats, hipStream_t stream) {
  const int grid = T < 4096 ? T : 4096;
  void* kargs[] = {&X, &T, &d, &eps, &stats};
  return hipLaunchKernel((const void*)&row_stats_kernel, dim3(grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace kq
