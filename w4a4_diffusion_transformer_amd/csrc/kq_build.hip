// Dense blocks from the 15 scalars per block (KroQuant's "precomputed dense
// blocks" kernel variant; Pith review, "What carries the argument").
// One thread per entry K[j][r][c]: the product, in fp64 and in factor order,
// of one entry of each factor G1 .. G5 (G1 on bit 4 of r and c), rounded once
// to fp32; optionally split into bf16 terms hi, mid, lo (each rounded to
// nearest even from the running remainder) stored transposed, [j][s][c][r].
//
// With inverse_t the block is K^-T = (G1^-1)^T (x) ... (x) (G5^-1)^T, the
// right factor of the offline weight fold W T^-T (Pith review, circularity
// check: Eq. (1)).  G^-1 = [[l b + 1/a, -b], [-l a, a]], so G^-T is G with
// its diagonal swapped and its off-diagonal entries negated and swapped;
// negation is exact, so these entries carry the same fp64 roundings as G's.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

__device__ __forceinline__ Factor inverse_transpose(Factor g) { return Factor{g.g11, -g.g10, -g.g01, g.g00}; }

__global__ __launch_bounds__(256) void build_kernel(const float* __restrict__ P, int nb, float* __restrict__ K32,
                                                    uint16_t* __restrict__ Kbf, int n_split, int inverse_t) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nb * 1024) return;
  const int j = (int)(idx >> 10), r = (int)((idx >> 5) & 31), c = (int)(idx & 31);
  Factors F = factors_f64(P + (int64_t)j * 15);
  if (inverse_t)
    F = Factors{inverse_transpose(F.f1), inverse_transpose(F.f2), inverse_transpose(F.f3), inverse_transpose(F.f4),
                inverse_transpose(F.f5)};
  const float k = k32_entry(F, r, c);
  if (K32) K32[idx] = k;
  if (Kbf) {
    float rest = k;
    for (int s = 0; s < n_split; ++s) {
      const __bf16 h = (__bf16)rest;
      Kbf[(((int64_t)j * n_split + s) * 32 + c) * 32 + r] = __builtin_bit_cast(uint16_t, h);
      rest = rest - (float)h;
    }
  }
}

// 16-wide blocks with four factors, as block-diagonal 32x32 blocks: entry
// [r][c] of block j is zero unless r and c lie in the same half h; then it is
// the fp64 product in factor order of G1 .. G4 of 16-wide block 2 j + h (G1 on
// bit 3 of r & 15 and c & 15), rounded once to fp32.
__global__ __launch_bounds__(256) void build16_kernel(const float* __restrict__ P, int nb, float* __restrict__ K32,
                                                      uint16_t* __restrict__ Kbf, int n_split) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nb * 1024) return;
  const int j = (int)(idx >> 10), r = (int)((idx >> 5) & 31), c = (int)(idx & 31);
  float k = 0.0f;
  if ((r >> 4) == (c >> 4)) {
    const float* p = P + (int64_t)(2 * j + (r >> 4)) * 12;
    const Factor f1 = factor_f64(p), f2 = factor_f64(p + 3), f3 = factor_f64(p + 6), f4 = factor_f64(p + 9);
    double v = pick(f1, (r >> 3) & 1, (c >> 3) & 1);
    v = v * pick(f2, (r >> 2) & 1, (c >> 2) & 1);
    v = v * pick(f3, (r >> 1) & 1, (c >> 1) & 1);
    v = v * pick(f4, r & 1, c & 1);
    k = (float)v;
  }
  if (K32) K32[idx] = k;
  if (Kbf) {
    float rest = k;
    for (int s = 0; s < n_split; ++s) {
      const __bf16 h = (__bf16)rest;
      Kbf[(((int64_t)j * n_split + s) * 32 + c) * 32 + r] = __builtin_bit_cast(uint16_t, h);
      rest = rest - (float)h;
    }
  }
}

}  // namespace

hipError_t launch_build16(const float* P16, int nb, float* K32, uint16_t* Kbf, int n_split, hipStream_t stream) {
  const int64_t n = (int64_t)nb * 1024;
  const int grid = (int)((n + 255) / 256);
  void* kargs[] = {&P16, &nb, &K32, &Kbf, &n_split};
  return hipLaunchKernel((const void*)&build16_kernel, dim3(grid), dim3(256), kargs, 0, stream);
}

hipError_t launch_build(const float* P, int nb, float* K32, uint16_t* Kbf, int n_split, int inverse_t,
                        hipStream_t stream) {
  const int64_t n = (int64_t)nb * 1024;
  const int grid = (int)((n + 255) / 256);
  void* kargs[] = {&P, &nb, &K32, &Kbf, &n_split, &inverse_t};
  return hipLaunchKernel((const void*)&build_kernel, dim3(grid), dim3(256), kargs, 0, stream);
}

}  // namespace kq
