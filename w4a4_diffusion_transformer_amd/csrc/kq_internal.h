// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

enum { KSRC_PARAMS = 0, KSRC_SPLIT = 1 };

// Tile decomposition of the MFMA kernels: a workgroup of eight waves owns a
// column group of 8 blocks (512 B of each bf16 row; each wave one block,
// whose K operands stay in its registers) and processes tiles of 32 rows.
// The grid has two parts.  The first w1 = ngroups * nchunks workgroups fill
// the GPU once: workgroup (group g, chunk c) takes row tiles c, c + nchunks,
// ... below r1.  The rest take the tiles from r1 on, n2 consecutive tiles
// each; the hardware dispatcher starts them on whichever compute units
// finish their first-part work first, which evens out the finish times.
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
  // AdaLN producer step (the MOD kernels): row (mean, rstd) pairs or nullptr,
  // per-sample fp32 scale and shift [samples][d] or nullptr, rows per sample
  const float* stats;
  const float* mscale;
  const float* mshift;
  int tps;
  int ngroups, nchunks;
  int w1, r1, n2;  // second part of the grid: see above
  // requested grid shape: size of the second part (percent of the tiles,
  // tiles per workgroup) and workgroups per CU the first part is sized for;
  // -1: the built-in rule.  The results do not depend on it, only the time.
  int req_tail_pct = -1, req_n2 = -1, req_wg_per_cu = -1;
};

// Row-segment decomposition of the vector-ALU kernels: a workgroup of four
// waves owns a column group of 16 blocks (1 KB of each bf16 row); each lane
// owns one fixed 16-byte piece (8 channels) of it, so every wave instruction
// reads 1 KB and writes 256 code bytes and 16 scale bytes, all contiguous.
// Rows go in blocks of four (one per wave); workgroup (group g, chunk c)
// takes row blocks c, c + nchunks, c + 2 nchunks, ...
struct QuadArgs {
  const uint16_t* X;
  int T, d, nb;
  const float* P;
  int pstride;
  const float* m;  // channel multipliers (SmoothQuant front-end)
  uint8_t* codes;
  uint8_t* scales;
  float* Y;
  int ngroups, nchunks;
};

// Block-per-lane decomposition of the vector-ALU kernels: X as a flat
// sequence of 64-byte blocks, a wave per unit of 64 consecutive blocks (one
// per lane, staged through a wave-private LDS region), each wave visiting
// units a whole number of rows apart so that each lane keeps one block
// column.  Set by launch_flat: nblocks, xbytes, units, phases, chunks.
struct FlatArgs {
  const uint16_t* X;
  int T, nb;
  const float* P;
  int pstride;
  const float* m;  // channel multipliers (SmoothQuant front-end)
  uint8_t* codes;
  uint8_t* scales;
  float* Y;
  // FRONT_ADALN: per-row (mean, rstd) [T][2] (null: 0, 1), (1 + scale) and shift vectors
  // [samples][d] (null: scale 0, shift -0), rows per sample (>= T: one sample)
  const float* stats = nullptr;
  const float* mscale = nullptr;
  const float* mshift = nullptr;
  int64_t tps = 0;
  int64_t nblocks, xbytes, units;
  int phases, chunks;
  int rows_step;      // set by launch_flat: rows between a lane's consecutive blocks
  int req_waves = 0;  // requested total waves (tuning; 0: one resident round)
  int hlog = 5;       // FRONT_HADAMARD_WIDE: log2 of the Hadamard block (6 .. 9)
  float hscale = 0.0f;  // and 1 / sqrt(block) in fp32
};

// Compute units of the current device (cached per device).
int cu_count();
// Workgroups of `fn` (block_threads threads, no dynamic LDS) resident per
// compute unit, from the occupancy calculator, cached per kernel and device;
// capped by the KQ_WG_PER_CU tuning override when set.
int resident_per_cu(const void* fn, int block_threads);
// Row chunks so that ngroups x nchunks workgroups fill the machine exactly
// once (no second, partial round), with at least one row tile per chunk.
int chunks_one_round(const void* fn, int block_threads, int ngroups, int ntiles, int wg_per_cu_cap = 0);

hipError_t launch_mfma(int ksrc, bool store_y, bool mod, const MfmaArgs& args, hipStream_t stream);
hipError_t launch_quad(int front, bool store_y, const QuadArgs& args, hipStream_t stream);
hipError_t launch_flat(int front, bool store_y, const FlatArgs& args, hipStream_t stream);
// W4A4 GEMM: Y [M][N] = deq(A) deq(B)^T, A [M][K] and B [N][K] in MXFP4
// (codes [rows][K/2], E8M0 scales [rows][K/32]); either output may be null.
struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int M, N, K;
  float* y_f32;
  uint16_t* y_bf16;
  int full_tiles;  // set by launch_gemm: tiles computed whole; the rest in two halves
};

hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream);
hipError_t launch_row_stats(const uint16_t* X, int T, int d, double eps, float* stats, hipStream_t stream);
hipError_t launch_build(const float* P, int nb, float* K32, uint16_t* Kbf, int n_split, int inverse_t,
                        hipStream_t stream);
hipError_t launch_build16(const float* P16, int nb, float* K32, uint16_t* Kbf, int n_split, hipStream_t stream);

}  // namespace kq
