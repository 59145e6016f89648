// Vector-ALU front-ends fused with the MXFP4 quantizer (gfx950):
//   FRONT_KRON      y = x K(j) as five fp32 2x2 butterfly stages, one per
//                   Kronecker factor (K = G1 (x) ... (x) G5: multiplying a row
//                   vector by it applies each G_k to the index bit it owns;
//                   KroQuant's on-the-fly "15 scalars" kernel variant, Pith
//                   review, "What carries the argument");
//   FRONT_PLAIN     y = x;
//   FRONT_SMOOTH    y = x * m[c] (SmoothQuant per-channel scale);
//   FRONT_HADAMARD  y = (x H32)[c] / sqrt(32), fast Walsh-Hadamard butterflies.
//
// Lane layout: four adjacent lanes hold one token's 32-channel block, lane
// q = l & 3 owning channels 8q .. 8q+7, so a wave's 16-byte loads cover 16
// rows x 64 contiguous bytes per block.  Stages on channel bits 0-2 stay in
// registers; bits 3 and 4 pair lane l with l^1 and l^2, exchanged with DPP
// quad permutes.  A wave owns two adjacent blocks and streams rows, 16
// tokens per step, loads kept two steps ahead.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;
constexpr int kDepth = 3;

// Per-lane coefficients of one block for the butterfly front-end.
struct Coef {
  float g[3][4];  // G5, G4, G3 (channel bits 0, 1, 2): full 2x2, row-major
  float cs[2];    // G2 (bit 3), G1 (bit 4): weight of this lane's own value
  float cp[2];    //                          weight of the partner lane's value
};

__device__ __forceinline__ void setup_coef(Coef& cf, const float* __restrict__ p15, int q) {
  double G[5][4];
  factors_f64(p15, G);
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) cf.g[s][e] = (float)G[4 - s][e];
  // cross-lane factor k acting on channel bit (4 - k); this lane's bit value is beta
  const int beta3 = q & 1, beta4 = q >> 1;
  // y_own = x_own G[beta][beta] + x_partner G[1 - beta][beta]
  cf.cs[0] = (float)G[1][2 * beta3 + beta3];
  cf.cp[0] = (float)G[1][2 * (1 - beta3) + beta3];
  cf.cs[1] = (float)G[0][2 * beta4 + beta4];
  cf.cp[1] = (float)G[0][2 * (1 - beta4) + beta4];
}

// (v[i], v[i | bit]) <- (v[i], v[i | bit]) G for every pair differing in `bit`.
template <int BIT>
__device__ __forceinline__ void stage_in_reg(float v[8], const float g[4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i & BIT) continue;
    const float x0 = v[i], x1 = v[i | BIT];
    v[i] = fmaf(x1, g[2], x0 * g[0]);
    v[i | BIT] = fmaf(x1, g[3], x0 * g[1]);
  }
}

template <int XOR>
__device__ __forceinline__ float partner(float v) {
  if constexpr (XOR == 1) return dpp_quad_xor1(v);
  else return dpp_quad_xor2(v);
}

template <int XOR>
__device__ __forceinline__ void stage_cross(float v[8], float cs, float cp) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], cs, partner<XOR>(v[i]) * cp);
}

// Walsh-Hadamard butterflies: (a, b) -> (a + b, a - b).
template <int BIT>
__device__ __forceinline__ void wht_in_reg(float v[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i & BIT) continue;
    const float a = v[i], b = v[i | BIT];
    v[i] = a + b;
    v[i | BIT] = a - b;
  }
}

// Lane with bit value beta: beta = 0 keeps own + partner, beta = 1 partner - own.
template <int XOR>
__device__ __forceinline__ void wht_cross(float v[8], float sgn) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], sgn, partner<XOR>(v[i]));
}

__device__ __forceinline__ void unpack8(const u32x4& w, float v[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16_lo(w[k]);
    v[2 * k + 1] = bf16_hi(w[k]);
  }
}

struct NoExact {
  __device__ float operator()(const uint16_t*, int) const { return 0.0f; }
};

template <int FRONT, bool STORE_Y>
__global__ __launch_bounds__(64 * kWaves) void quad_kernel(QuadArgs a) {
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
  const int tl = lane >> 2, q = lane & 3;

  Coef cf[2];
  float mult[2][8];
  if constexpr (FRONT == FRONT_KRON) {
    setup_coef(cf[0], a.P + (int64_t)j0 * a.pstride, q);
    if (has1) setup_coef(cf[1], a.P + (int64_t)(j0 + 1) * a.pstride, q);
  }
  if constexpr (FRONT == FRONT_SMOOTH) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      if (bb == 1 && !has1) break;
      const f32x4* mp = reinterpret_cast<const f32x4*>(a.m + 32 * (j0 + bb) + 8 * q);
      const f32x4 m0 = mp[0], m1 = mp[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mult[bb][i] = m0[i];
        mult[bb][4 + i] = m1[i];
      }
    }
  }
  const float sgn3 = (q & 1) ? -1.0f : 1.0f, sgn4 = (q >> 1) ? -1.0f : 1.0f;
  constexpr float kInvSqrt32 = 0.17677669529663688110f;

  const int64_t d = a.d;
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
    const int tc = valid ? t : t_begin;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      if (bb == 1 && !has1) break;
      const int j = j0 + bb;
      float y[8];
      unpack8(b[bb], y);
      if constexpr (FRONT == FRONT_KRON) {
        stage_in_reg<1>(y, cf[bb].g[0]);
        stage_in_reg<2>(y, cf[bb].g[1]);
        stage_in_reg<4>(y, cf[bb].g[2]);
        stage_cross<1>(y, cf[bb].cs[0], cf[bb].cp[0]);
        stage_cross<2>(y, cf[bb].cs[1], cf[bb].cp[1]);
      } else if constexpr (FRONT == FRONT_SMOOTH) {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] *= mult[bb][i];
      } else if constexpr (FRONT == FRONT_HADAMARD) {
        wht_in_reg<1>(y);
        wht_in_reg<2>(y);
        wht_in_reg<4>(y);
        wht_cross<1>(y, sgn3);
        wht_cross<2>(y, sgn4);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] *= kInvSqrt32;
      }
      const uint16_t* xblk = a.X + (int64_t)tc * d + 32 * j;
      unsigned word, byte;
      if constexpr (FRONT == FRONT_KRON) {
        mx_epilogue<LAYOUT_QUAD, true>(y, xblk, q, ExactFromParams{a.P + (int64_t)j * a.pstride}, word, byte);
      } else if constexpr (FRONT == FRONT_HADAMARD) {
        mx_epilogue<LAYOUT_QUAD, true>(y, xblk, q, ExactHadamard{}, word, byte);
      } else {
        mx_epilogue<LAYOUT_QUAD, false>(y, xblk, q, NoExact{}, word, byte);
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

template <int FRONT>
const void* pick(bool store_y) {
  return store_y ? (const void*)&quad_kernel<FRONT, true> : (const void*)&quad_kernel<FRONT, false>;
}

}  // namespace

hipError_t launch_quad(int front, bool store_y, const QuadArgs& args, hipStream_t stream) {
  const int grid = (int)(((int64_t)args.nwork + kWaves - 1) / kWaves);
  QuadArgs a = args;
  void* kargs[] = {&a};
  const void* fn = nullptr;
  switch (front) {
    case FRONT_KRON: fn = pick<FRONT_KRON>(store_y); break;
    case FRONT_PLAIN: fn = pick<FRONT_PLAIN>(store_y); break;
    case FRONT_SMOOTH: fn = pick<FRONT_SMOOTH>(store_y); break;
    case FRONT_HADAMARD: fn = pick<FRONT_HADAMARD>(store_y); break;
    default: return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, dim3(grid), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace kq
