// Dense blocks from the 15 scalars per block (KroQuant's "precomputed dense
// blocks" kernel variant; Pith review, "What carries the argument").
// One thread per entry K[j][r][c]: the product, in fp64 and in factor order,
// of one entry of each factor G1 .. G5 (G1 on bit 4 of r and c), rounded once
// to fp32; optionally split into bf16 terms hi, mid, lo (each rounded to
// nearest even from the running remainder) stored transposed, [j][s][c][r].
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

__global__ __launch_bounds__(256) void build_kernel(const float* __restrict__ P, int nb, float* __restrict__ K32,
                                                    uint16_t* __restrict__ Kbf, int n_split) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nb * 1024) return;
  const int j = (int)(idx >> 10), r = (int)((idx >> 5) & 31), c = (int)(idx & 31);
  const Factors F = factors_f64(P + (int64_t)j * 15);
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

}  // namespace

hipError_t launch_build(const float* P, int nb, float* K32, uint16_t* Kbf, int n_split, hipStream_t stream) {
  const int64_t n = (int64_t)nb * 1024;
  const int grid = (int)((n + 255) / 256);
  void* kargs[] = {&P, &nb, &K32, &Kbf, &n_split};
  return hipLaunchKernel((const void*)&build_kernel, dim3(grid), dim3(256), kargs, 0, stream);
}

}  // namespace kq
