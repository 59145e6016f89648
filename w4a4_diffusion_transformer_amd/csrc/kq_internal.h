// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

enum { KSRC_PARAMS = 0, KSRC_SPLIT = 1 };

// Shared work decomposition: a wave owns blocks (2 pair, 2 pair + 1) and rows
// [chunk * rows_per_chunk, ...); work item w = chunk * npairs + pair.
struct MfmaArgs {
  const uint16_t* X;
  int T, d, nb;
  const float* P;  // [nb][15] or one set (pstride 0)
  int pstride;
  const uint16_t* Kbf;  // [nb][3][32][32] transposed split
  int kstride;          // 3072 or 0
  uint8_t* codes;
  uint8_t* scales;
  float* Y;  // diagnostic output or nullptr
  int npairs, rows_per_chunk, nwork;
};

struct QuadArgs {
  const uint16_t* X;
  int T, d, nb;
  const float* P;
  int pstride;
  const float* m;  // channel multipliers (SmoothQuant front-end)
  uint8_t* codes;
  uint8_t* scales;
  float* Y;
  int npairs, rows_per_chunk, nwork;
};

hipError_t launch_mfma(int ksrc, bool store_y, const MfmaArgs& args, hipStream_t stream);
hipError_t launch_quad(int front, bool store_y, const QuadArgs& args, hipStream_t stream);
hipError_t launch_build(const float* P, int nb, float* K32, uint16_t* Kbf, int n_split, hipStream_t stream);

}  // namespace kq
