// KroQuant block transform on the matrix cores, fused with the MXFP4
// quantizer (gfx950).
//
// y = x K(j) for every 32-channel block j (KroQuant, Pith review: the block
// transform runs as "a single tensor-core GEMM per block"; row-vector
// convention of Eq. (1)) computed as Y^T = K^T X^T with
// v_mfma_f32_16x16x32_bf16: M = 16 output channels, N = 16 tokens, K = the
// block's 32 input channels in one instruction.  X is bf16 already; K is
// fp32, represented exactly by three bf16 terms hi + mid + lo whose products
// are accumulated in fp32 (smallest term first).
//
// Memory: HBM streaming needs every wave instruction to touch whole row
// segments, but the MFMA operand layout wants 16 tokens x 16 bytes.  So a
// workgroup (4 waves, 8 blocks = 512 B of each row) stages each 16-row tile
// through LDS: row segments are loaded from HBM into a padded LDS tile, each
// wave reads its two blocks back in operand layout, and the code words and
// scale bytes go through a second LDS tile so that they leave as contiguous
// 128-byte code segments per row.  Double buffers, one barrier per tile,
// global loads kept two tiles ahead.  Output channels are permuted across
// the MFMA rows so that each lane ends up with 8 consecutive channels of one
// token: lane (t = l & 15, q = l >> 4) holds channels 8q .. 8q+7 of token t.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kCB = 2 * kWaves;        // blocks per workgroup column group
constexpr int kRows = 16;              // rows per tile (MFMA N)
constexpr int kPieces = kRows * kCB * 4;           // 16-byte pieces of X per tile
constexpr int kPPT = kPieces / (64 * kWaves);      // pieces per thread per tile
constexpr int kAhead = 2;                          // tiles of global loads in flight beyond the current
constexpr int kInStride = kCB * 64 + 16;           // LDS bytes per input row (16 B pad: conflict-free reads)
constexpr int kOutStride = kCB * 16 + 16;          // LDS bytes per code row (stride 4 mod 64 dwords)
constexpr int kInBytes = kRows * kInStride;
constexpr int kOutBytes = kRows * kOutStride;
constexpr int kScaleBytes = kRows * kCB;
static_assert(kPPT * 64 * kWaves == kPieces, "tile pieces must split evenly over the workgroup");

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
  __shared__ __attribute__((aligned(16))) uint8_t lds_in[2][kInBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_out[2][kOutBytes];
  __shared__ uint8_t lds_sc[2][kScaleBytes];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int g = wg % a.ngroups, c = wg / a.ngroups;
  const int jg = kCB * g;                      // first block of the column group
  const int nvalid = min(kCB, a.nb - jg);      // blocks present in this group
  const int64_t d = a.d;
  const int ntile_rows = (a.T + kRows - 1) / kRows;
  const int nsteps = c < ntile_rows ? (ntile_rows - 1 - c) / a.nchunks + 1 : 0;
  auto row0_of = [&](int s) { return kRows * (c + s * a.nchunks); };

  // this wave's two blocks
  const int jb0 = jg + 2 * wv;
  const bool has0 = 2 * wv < nvalid, has1 = 2 * wv + 1 < nvalid;
  bf16x8 A[2][2][3];  // K^T operands: [block][output half][term hi, mid, lo]

  // global -> LDS pieces of a tile: piece p = tid + 256 k, row p / (4 kCB), 16-byte column p % (4 kCB)
  u32x4 pre[kAhead][kPPT];
  auto gload = [&](int s, u32x4 (&r)[kPPT]) {
    const int r0 = row0_of(s);
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
      const int p = tid + 64 * kWaves * k;
      const int row = r0 + p / (4 * kCB), col = p % (4 * kCB);
      const bool ok = row < a.T && (col >> 2) < nvalid;
      r[k] = ok ? __builtin_nontemporal_load(
                      reinterpret_cast<const u32x4*>(a.X + (int64_t)row * d + 32 * jg + 8 * col))
                : u32x4{0, 0, 0, 0};
    }
  };
  auto lwrite = [&](int buf, const u32x4 (&r)[kPPT]) {
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
      const int p = tid + 64 * kWaves * k;
      const int row = p / (4 * kCB), col = p % (4 * kCB);
      *reinterpret_cast<u32x4*>(&lds_in[buf][row * kInStride + 16 * col]) = r[k];
    }
  };
  // LDS -> global: 16 rows x (16 nvalid) code bytes, 16 rows x nvalid scale bytes
  auto gstore = [&](int s, int buf) {
    const int r0 = row0_of(s);
    for (int p = tid; p < kRows * kCB; p += 64 * kWaves) {
      const int row = p / kCB, col = p % kCB;
      if (r0 + row < a.T && col < nvalid) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&lds_out[buf][row * kOutStride + 16 * col]);
        *reinterpret_cast<u32x4*>(a.codes + (int64_t)(r0 + row) * (d >> 1) + 16 * (jg + col)) = v;
        a.scales[(int64_t)(r0 + row) * a.nb + jg + col] = lds_sc[buf][row * kCB + col];
      }
    }
  };

  const int tl = lane & 15, q = lane >> 4;
  auto compute = [&](int s, int buf) {
    const int r0 = row0_of(s);
    const int t = r0 + tl;
    const bool valid = t < a.T;
    const int tc = valid ? t : r0;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      if (!(bb == 0 ? has0 : has1)) break;
      const int jl = 2 * wv + bb, j = jg + jl;
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(&lds_in[buf][tl * kInStride + 64 * jl + 16 * q]);
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
      *reinterpret_cast<unsigned*>(&lds_out[buf][tl * kOutStride + 16 * jl + 4 * q]) = word;
      if (q == 0) lds_sc[buf][tl * kCB + jl] = (uint8_t)byte;
      if constexpr (STORE_Y) {
        if (valid) {
          float* yr = a.Y + (int64_t)t * d + 32 * j + 8 * q;
          *reinterpret_cast<f32x4*>(yr) = f32x4{y[0], y[1], y[2], y[3]};
          *reinterpret_cast<f32x4*>(yr + 4) = f32x4{y[4], y[5], y[6], y[7]};
        }
      }
    }
  };

#pragma unroll
  for (int k = 0; k < kAhead; ++k)
    if (k < nsteps) gload(k, pre[k]);
  // K operands after the first loads are in flight, so the setup overlaps them
  if (has0) setup_a<KSRC>(A[0], jb0, a.P, a.pstride, a.Kbf, a.kstride, lane);
  if (has1) setup_a<KSRC>(A[1], jb0 + 1, a.P, a.pstride, a.Kbf, a.kstride, lane);
  for (int it = 0; it < nsteps; it += kAhead) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      const int s = it + k;
      if (s < nsteps) {
        const int buf = s & 1;
        lwrite(buf, pre[k]);
        if (s + kAhead < nsteps) gload(s + kAhead, pre[k]);
        __syncthreads();
        if (s > 0) gstore(s - 1, buf ^ 1);
        compute(s, buf);
      }
    }
  }
  __syncthreads();
  if (nsteps > 0) gstore(nsteps - 1, (nsteps - 1) & 1);
}

}  // namespace

hipError_t launch_mfma(int ksrc, bool store_y, const MfmaArgs& args, hipStream_t stream) {
  const void* fn;
  if (ksrc == KSRC_PARAMS)
    fn = store_y ? (const void*)&mfma_kernel<KSRC_PARAMS, true> : (const void*)&mfma_kernel<KSRC_PARAMS, false>;
  else
    fn = store_y ? (const void*)&mfma_kernel<KSRC_SPLIT, true> : (const void*)&mfma_kernel<KSRC_SPLIT, false>;
  MfmaArgs a = args;
  a.ngroups = (a.nb + kCB - 1) / kCB;
  a.nchunks = chunks_one_round(fn, 64 * kWaves, a.ngroups, (a.T + kRows - 1) / kRows);
  void* kargs[] = {&a};
  return hipLaunchKernel(fn, dim3(a.ngroups * a.nchunks), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace kq
