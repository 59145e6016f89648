// KroQuant block transform on the matrix cores, fused with the MXFP4
// quantizer (gfx950).
//
// y = x K(j) for every 32-channel block j (KroQuant, Pith review: "a single
// tensor-core GEMM per block"; Eq. (1) row-vector convention) computed as
// Y^T = K^T X^T with v_mfma_f32_16x16x32_bf16: M = 16 output channels,
// N = 16 tokens, K = the block's 32 input channels in one instruction.  X is
// bf16 already, so each lane's B operand is a 16-byte load straight from the
// activation row (no LDS staging, no conversion).  K is fp32; three bf16
// terms hi + mid + lo represent it exactly and the three products are
// accumulated in fp32 (smallest term first).
//
// Work decomposition: a wave owns a pair of adjacent blocks (its K operands
// stay in registers, 48 VGPRs) and streams a chunk of rows through it, 16
// tokens per step with loads kept two steps ahead.  Output channels are
// permuted across the MFMA rows so that each lane ends up with 8 consecutive
// channels of one token: lane (t = l & 15, q = l >> 4) holds channels
// 8q .. 8q+7 of token t, four code bytes stored with one dword store.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;  // waves per workgroup
constexpr int kDepth = 3;  // row steps in flight per wave (current + 2 ahead)

// Output channel held by MFMA row m of half h.
__device__ __forceinline__ int out_channel(int h, int m) { return 8 * (m >> 2) + 4 * h + (m & 3); }

template <int KSRC>
__device__ __forceinline__ void setup_a(bf16x8 A[2][3], int j, const float* __restrict__ P, int pstride,
                                        const uint16_t* __restrict__ Kbf, int kstride, int lane) {
  const int m = lane & 15, q = lane >> 4;
  if constexpr (KSRC == KSRC_PARAMS) {
    double G[5][4];
    factors_f64(P + (int64_t)j * pstride, G);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = out_channel(h, m);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float k = k32_entry(G, 8 * q + i, c);
        const __bf16 hi = (__bf16)k;
        const float r1 = k - (float)hi;
        const __bf16 mid = (__bf16)r1;
        const __bf16 lo = (__bf16)(r1 - (float)mid);
        A[h][0][i] = hi;
        A[h][1][i] = mid;
        A[h][2][i] = lo;
      }
    }
  } else {
    const uint16_t* kb = Kbf + (int64_t)j * kstride;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = out_channel(h, m);
#pragma unroll
      for (int s = 0; s < 3; ++s)
        A[h][s] = *reinterpret_cast<const bf16x8*>(kb + (s * 32 + c) * 32 + 8 * q);
    }
  }
}

template <int KSRC, bool STORE_Y>
__global__ __launch_bounds__(64 * kWaves) void mfma_kernel(MfmaArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int w = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wv;
  if (w >= a.nwork) return;
  const int pair = w % a.npairs, chunk = w / a.npairs;
  const int j0 = 2 * pair;
  const bool has1 = j0 + 1 < a.nb;
  const int t_begin = chunk * a.rows_per_chunk;
  const int t_end = min(a.T, t_begin + a.rows_per_chunk);
  const int ntiles = (t_end - t_begin + 15) >> 4;
  const int tl = lane & 15, q = lane >> 4;

  bf16x8 A[2][2][3];
  setup_a<KSRC>(A[0], j0, a.P, a.pstride, a.Kbf, a.kstride, lane);
  if (has1) setup_a<KSRC>(A[1], j0 + 1, a.P, a.pstride, a.Kbf, a.kstride, lane);

  const int64_t d = a.d;
  // this lane's 16 bytes of block j0 in row t: X + t*d + 32*j0 + 8q
  const uint16_t* xbase = a.X + 32 * j0 + 8 * q;
  u32x4 buf[kDepth][2];

  auto load = [&](int tile, u32x4 (&b)[2]) {
    const int t = t_begin + 16 * tile + tl;
    if (t < t_end) {
      const uint16_t* p = xbase + (int64_t)t * d;
      b[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      b[1] = has1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 32)) : u32x4{0, 0, 0, 0};
    } else {
      b[0] = u32x4{0, 0, 0, 0};
      b[1] = u32x4{0, 0, 0, 0};
    }
  };

  auto compute = [&](int tile, const u32x4 (&b)[2]) {
    const int t = t_begin + 16 * tile + tl;
    const bool valid = t < t_end;
    const int tc = valid ? t : t_begin;  // in-bounds row for the exact path (never used for invalid rows)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      if (bb == 1 && !has1) break;
      const int j = j0 + bb;
      const bf16x8 xb = __builtin_bit_cast(bf16x8, b[bb]);
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[bb][0][2], xb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[bb][1][2], xb, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[bb][0][1], xb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[bb][1][1], xb, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[bb][0][0], xb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[bb][1][0], xb, acc1, 0, 0, 0);
      float y[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
      const uint16_t* xblk = a.X + (int64_t)tc * d + 32 * j;
      unsigned word, byte;
      if constexpr (KSRC == KSRC_PARAMS) {
        mx_epilogue<LAYOUT_MFMA, true>(y, xblk, q, ExactFromParams{a.P + (int64_t)j * a.pstride}, word, byte);
      } else {
        mx_epilogue<LAYOUT_MFMA, true>(y, xblk, q, ExactFromSplit{a.Kbf + (int64_t)j * a.kstride}, word, byte);
      }
      if (valid) {
        uint8_t* crow = a.codes + (int64_t)t * (d >> 1);
        *reinterpret_cast<unsigned*>(crow + 16 * j + 4 * q) = word;
        if (q == bb) a.scales[(int64_t)t * a.nb + j] = (uint8_t)byte;
        if constexpr (STORE_Y) {
          float* yr = a.Y + (int64_t)t * d + 32 * j + 8 * q;
          *reinterpret_cast<f32x4*>(yr) = f32x4{y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4*>(yr + 4) = f32x4{y[4], y[5], y[6], y[7]};
        }
      }
    }
  };

#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k)
    if (k < ntiles) load(k, buf[k]);
  for (int it = 0; it < ntiles; it += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int tile = it + k;
      if (tile < ntiles) {
        const int pf = tile + kDepth - 1;
        if (pf < ntiles) load(pf, buf[(k + kDepth - 1) % kDepth]);
        compute(tile, buf[k]);
      }
    }
  }
}

}  // namespace

hipError_t launch_mfma(int ksrc, bool store_y, const MfmaArgs& args, hipStream_t stream) {
  const int64_t waves = args.nwork;
  const int grid = (int)((waves + kWaves - 1) / kWaves);
  MfmaArgs a = args;
  void* kargs[] = {&a};
  const void* fn;
  if (ksrc == KSRC_PARAMS)
    fn = store_y ? (const void*)&mfma_kernel<KSRC_PARAMS, true> : (const void*)&mfma_kernel<KSRC_PARAMS, false>;
  else
    fn = store_y ? (const void*)&mfma_kernel<KSRC_SPLIT, true> : (const void*)&mfma_kernel<KSRC_SPLIT, false>;
  return hipLaunchKernel(fn, dim3(grid), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace kq
