// W4A4 consumer: Y = deq(A) deq(B)^T on the gfx950 scaled FP4 matrix cores.
//
// A [M][K] and B [N][K] are MXFP4 in the quantizer's output format (codes
// [rows][K/2], even element in the low nibble; E8M0 scales [rows][K/32]):
// A the quantized activation X T, B the quantized folded weight W T^-T, so
// that Y approximates X W^T (Pith review, circularity check: Eq. (1); the
// W4A4 MXFP4 GEMM the quantizer feeds).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1: lane l holds 32
// consecutive K values (16 bytes) of row l % 16 at K offset 32 (l / 16) -
// exactly one MX block - plus that block's E8M0 byte as its scale operand;
// the result lane l holds D[4 (l / 16) + i][l % 16], i = 0..3 (verified on
// MI355X against a CPU evaluation).  Products of E2M1 values and power-of-two
// scales are exact; sums are fp32.
//
// Workgroup: 4 waves (2 x 2), a 128 x 128 tile of Y, each wave 64 x 64
// (4 x 4 MFMA tiles).  Per K step of 128: the A and B tiles (128 rows x 64 B
// each) and their scale bytes are staged through double-buffered LDS (row
// stride 80 B: the 16 rows an MFMA fragment reads fall on distinct banks);
// the next step's global loads are in flight during the current step's
// MFMAs; one barrier per step.  Rows past M or N and K blocks past K read as
// zero codes (buffer range / masked offsets), which contribute nothing.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kThreads = 256;
constexpr int kBM = 128, kBN = 128;  // tile of Y
constexpr int kStride = 80;          // LDS bytes per staged row (64 B of codes + 16 B pad)
constexpr int kTileBytes = kBM * kStride;

__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][kTileBytes];
  __shared__ uint8_t as_lds[2][kBM * 4];
  __shared__ uint8_t bs_lds[2][kBN * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int K = g.K, kbytes = K >> 1, kblocks = K >> 5;
  const int nsteps = (K + 127) >> 7;
  const int mrows = min(kBM, g.M - m0), nrows = min(kBN, g.N - n0);

  // Per-workgroup descriptors over this tile's rows (reads past them give zero).
  const auto ra = rsrc_uniform(g.a_codes + (int64_t)m0 * kbytes, (int64_t)mrows * kbytes);
  const auto rb = rsrc_uniform(g.b_codes + (int64_t)n0 * kbytes, (int64_t)nrows * kbytes);
  const auto ras = rsrc_uniform(g.a_scales + (int64_t)m0 * kblocks, (int64_t)mrows * kblocks);
  const auto rbs = rsrc_uniform(g.b_scales + (int64_t)n0 * kblocks, (int64_t)nrows * kblocks);

  // Code pieces this thread moves per step: 2 of A, 2 of B (row p / 4, 16-byte chunk p % 4).
  int prow[2], pchk[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = tid + kThreads * k;
    prow[k] = p >> 2;
    pchk[k] = p & 3;
  }
  // Scale bytes: threads 0..127 move row tid of A, 128..255 row tid - 128 of B (4 blocks each).
  const int srow = tid & 127;
  const bool s_is_a = wv < 2;  // waves 0, 1 (wave-uniform, so the descriptor choice stays scalar)

  u32x4 ra_reg[2], rb_reg[2];
  unsigned s_reg;
  auto gload = [&](int ks) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool kin = ks * 128 + 32 * pchk[k] < K;
      const uint32_t off = kin ? (uint32_t)(prow[k] * kbytes + ks * 64 + 16 * pchk[k]) : kOut;
      ra_reg[k] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      rb_reg[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    }
    unsigned v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool kin = 4 * ks + b < kblocks;
      const uint32_t off = kin ? (uint32_t)(srow * kblocks + 4 * ks + b) : kOut;
      const unsigned byte = __builtin_amdgcn_raw_buffer_load_b8(s_is_a ? ras : rbs, off, 0, 0);
      v |= (byte & 0xFFu) << (8 * b);
    }
    s_reg = v;
  };
  auto lwrite = [&](int buf) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      *reinterpret_cast<u32x4*>(&a_lds[buf][prow[k] * kStride + 16 * pchk[k]]) = ra_reg[k];
      *reinterpret_cast<u32x4*>(&b_lds[buf][prow[k] * kStride + 16 * pchk[k]]) = rb_reg[k];
    }
    *reinterpret_cast<unsigned*>(s_is_a ? &as_lds[buf][srow * 4] : &bs_lds[buf][srow * 4]) = s_reg;
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fg = lane >> 4;  // fragment row within 16, K block within the step
  auto compute = [&](int buf) {
    i32x8 af[4], bf[4];
    int sa[4], sb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ar = 64 * wm + 16 * t + fr, br = 64 * wn + 16 * t + fr;
      const u32x4 va = *reinterpret_cast<const u32x4*>(&a_lds[buf][ar * kStride + 16 * fg]);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(&b_lds[buf][br * kStride + 16 * fg]);
      af[t] = i32x8{(int)va[0], (int)va[1], (int)va[2], (int)va[3], 0, 0, 0, 0};
      bf[t] = i32x8{(int)vb[0], (int)vb[1], (int)vb[2], (int)vb[3], 0, 0, 0, 0};
      sa[t] = as_lds[buf][ar * 4 + fg];
      sb[t] = bs_lds[buf][br * 4 + fg];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                      sb[j]);
  };

  gload(0);
  lwrite(0);
  __syncthreads();
  for (int ks = 0; ks < nsteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nsteps) gload(ks + 1);  // workgroup-uniform
    compute(buf);
    if (ks + 1 < nsteps) lwrite(buf ^ 1);
    __syncthreads();
  }

  // Y rows m0 + 64 wm + 16 i + 4 fg + r, columns n0 + 64 wn + 16 j + fr.
  const int64_t N = g.N;
  if (g.y_f32) {
    const auto ry = rsrc_uniform(g.y_f32 + (int64_t)m0 * N, (int64_t)mrows * N * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 64 * wn + 16 * j + fr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 64 * wm + 16 * i + 4 * fg + r;
          const uint32_t off = col < nrows ? (uint32_t)((row * N + n0 + col) * 4) : kOut;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ry, off, 0, 0);
        }
      }
  }
  if (g.y_bf16) {
    const auto ry = rsrc_uniform(g.y_bf16 + (int64_t)m0 * N, (int64_t)mrows * N * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 64 * wn + 16 * j + fr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 64 * wm + 16 * i + 4 * fg + r;
          const uint32_t off = col < nrows ? (uint32_t)((row * N + n0 + col) * 2) : kOut;
          const __bf16 h = (__bf16)acc[i][j][r];
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), ry, off, 0, 0);
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream) {
  GemmArgs g = args;
  const dim3 grid((unsigned)((g.N + kBN - 1) / kBN), (unsigned)((g.M + kBM - 1) / kBM));
  void* kargs[] = {&g};
  return hipLaunchKernel((const void*)&gemm_kernel, grid, dim3(kThreads), kargs, 0, stream);
}

}  // namespace kq
