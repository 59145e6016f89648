// Vector-ALU front-ends fused with the MXFP4 quantizer (gfx950):
//   FRONT_KRON      y = x K(j) as five fp32 2x2 butterfly stages, one per
//                   Kronecker factor (K = G1 (x) ... (x) G5: multiplying a row
//                   vector by it applies each G_k to the index bit it owns;
//                   KroQuant's on-the-fly "15 scalars" kernel variant, Pith
//                   review, "What carries the argument");
//   FRONT_PLAIN     y = x;
//   FRONT_SMOOTH    y = x * m[c] (SmoothQuant per-channel scale);
//   FRONT_HADAMARD  y = (x H_B)[c] / sqrt(B), fast Walsh-Hadamard butterflies
//                   over blocks of B = 32 .. 512 channels (stages on channel
//                   bits 5 and up pair lanes 4, 8, 16, 32 apart).
//
// Lane layout: a wave covers 1 KB of one bf16 row (16 blocks); lane l owns
// the fixed 16-byte piece l, i.e. channels 8q .. 8q+7 (q = l & 3) of block
// l >> 2 of its column group, for every row it visits.  Loads (1 KB), code
// stores (256 B) and scale stores (16 B) of a wave instruction are therefore
// contiguous, and each lane keeps the coefficients of a single block in
// registers.  Stages on channel bits 0-2 stay in registers; bits 3 and 4
// pair lane l with l^1 and l^2 (the four lanes of a block), exchanged with
// DPP quad permutes.  Rows stream with loads kept several rows ahead.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;  // waves per workgroup, one row each per step
constexpr int kDepth = 6;  // rows in flight per wave (current + 5 ahead)

// Per-lane coefficients of one block for the butterfly front-end.
struct Coef {
  float g[3][4];  // G5, G4, G3 (channel bits 0, 1, 2): full 2x2, row-major
  float cs[2];    // G2 (bit 3), G1 (bit 4): weight of this lane's own value
  float cp[2];    //                          weight of the partner lane's value
};

__device__ __forceinline__ void set_full(float g[4], const Factor& f) {
  g[0] = (float)f.g00;
  g[1] = (float)f.g01;
  g[2] = (float)f.g10;
  g[3] = (float)f.g11;
}

// A cross-lane stage: this lane's channel has bit value beta for the factor:
// y_own = x_own G[beta][beta] + x_partner G[1 - beta][beta].
__device__ __forceinline__ void set_cross(float& cs, float& cp, const Factor& f, int beta) {
  cs = (float)(beta ? f.g11 : f.g00);
  cp = (float)(beta ? f.g01 : f.g10);
}

__device__ __forceinline__ void setup_coef(Coef& cf, const float* __restrict__ p15, int q, double* g_out) {
  const Factors F = factors_f64(p15);
  if (g_out) store_factors(F, g_out);  // for the exact path
  set_full(cf.g[0], F.f5);             // channel bit 0
  set_full(cf.g[1], F.f4);             // bit 1
  set_full(cf.g[2], F.f3);             // bit 2
  set_cross(cf.cs[0], cf.cp[0], F.f2, q & 1);   // bit 3: lanes l, l^1
  set_cross(cf.cs[1], cf.cp[1], F.f1, q >> 1);  // bit 4: lanes l, l^2
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
  __shared__ double lds_g[FRONT == FRONT_KRON ? 16 : 1][20];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int g = wg % a.ngroups, c = wg / a.ngroups;
  const int j = 16 * g + (lane >> 2), q = lane & 3;
  const bool live = j < a.nb;  // the last column group may be partial
  const int jc = live ? j : a.nb - 1;

  Coef cf;
  float mult[8];
  if constexpr (FRONT == FRONT_KRON) {
    setup_coef(cf, a.P + (int64_t)jc * a.pstride, q, wv == 0 && q == 0 ? lds_g[lane >> 2] : nullptr);
    __syncthreads();
  }
  if constexpr (FRONT == FRONT_SMOOTH) {
    const f32x4* mp = reinterpret_cast<const f32x4*>(a.m + 32 * jc + 8 * q);
    const f32x4 m0 = mp[0], m1 = mp[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mult[i] = m0[i];
      mult[4 + i] = m1[i];
    }
  }
  const float sgn3 = (q & 1) ? -1.0f : 1.0f, sgn4 = (q >> 1) ? -1.0f : 1.0f;

  const int64_t d = a.d;
  const int nrb = (a.T + kWaves - 1) / kWaves;  // row blocks of kWaves rows
  const int nsteps = c < nrb ? (nrb - 1 - c) / a.nchunks + 1 : 0;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);  // the wave's row is wave-uniform
  // this lane's byte offsets within a row (kOut: nothing to move)
  const uint32_t xoff = live ? (uint32_t)(64 * j + 16 * q) : kOut;
  const uint32_t coff = live ? (uint32_t)(16 * j + 4 * q) : kOut;
  const uint32_t soff = live && q == 0 ? (uint32_t)j : kOut;
  u32x4 buf[kDepth];

  // Wave-uniform cursors advanced by a constant per step (the wave's next
  // row to load, and the row being computed and stored).  Rows past the end
  // read zeros and their stores are dropped by the buffer range check, so
  // every step issues the same memory instructions.
  const int step_rows = kWaves * a.nchunks;
  const int xrow_bytes = 2 * a.d, crow_bytes = a.d >> 1, srow_bytes = a.nb;
  const int row0 = kWaves * c + wvu;
  int lleft = a.T - row0;  // rows from the load cursor to the end (negative past it)
  const uint8_t* lx = reinterpret_cast<const uint8_t*>(a.X) + (int64_t)row0 * xrow_bytes;
  const int64_t lstep = (int64_t)step_rows * xrow_bytes;
  auto load = [&](int, u32x4& b) {
    b = __builtin_amdgcn_raw_buffer_load_b128(rsrc(lx, lleft > 0 ? xrow_bytes : 0), xoff, 0, kNT);
    lleft -= step_rows;
    lx += lstep;
  };
  int cleft = a.T - row0;  // the same for the row being computed and stored
  int64_t crow = row0;
  const uint16_t* cx = a.X + (int64_t)row0 * d;
  uint8_t* cc = a.codes + (int64_t)row0 * crow_bytes;
  uint8_t* cs = a.scales + (int64_t)row0 * srow_bytes;
  const int64_t cxstep = (int64_t)step_rows * d, ccstep = (int64_t)step_rows * crow_bytes,
                csstep = (int64_t)step_rows * srow_bytes;

  auto compute = [&](int, const u32x4& b) {
    const bool in = cleft > 0;
    float y[8];
    unpack8(b, y);
    if constexpr (FRONT == FRONT_KRON) {
      stage_in_reg<1>(y, cf.g[0]);
      stage_in_reg<2>(y, cf.g[1]);
      stage_in_reg<4>(y, cf.g[2]);
      stage_cross<1>(y, cf.cs[0], cf.cp[0]);
      stage_cross<2>(y, cf.cs[1], cf.cp[1]);
    } else if constexpr (FRONT == FRONT_SMOOTH) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] *= mult[i];
    } else if constexpr (FRONT == FRONT_HADAMARD) {
      wht_in_reg<1>(y);
      wht_in_reg<2>(y);
      wht_in_reg<4>(y);
      wht_cross<1>(y, sgn3);
      wht_cross<2>(y, sgn4);
      // channel bits 5 .. hlog-1 (blocks of 64 .. 512): bit b of the channel is bit b-3 of the lane
#pragma unroll 1
      for (int bt = 5; bt < a.hlog; ++bt) {
        const int m = 1 << (bt - 3);
        const float sgn = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = fmaf(y[i], sgn, __shfl_xor(y[i], m, 64));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] *= a.hscale;
    }
    // rows past the end hold zeros (amax 0): the exact path never runs for them
    const uint16_t* xblk = (in ? cx : a.X) + 32 * jc;
    unsigned word, byte;
    if constexpr (FRONT == FRONT_KRON) {
      mx_epilogue<LAYOUT_QUAD, true>(y, xblk, q, ExactFromFactors{lds_g[lane >> 2]}, word, byte);
    } else if constexpr (FRONT == FRONT_HADAMARD) {
      const int hb = 1 << a.hlog;
      const int off = (32 * jc) & (hb - 1);
      mx_epilogue<LAYOUT_QUAD, true>(y, xblk, q, ExactHadamardB{xblk - off, hb, off}, word, byte);
    } else {
      mx_epilogue<LAYOUT_QUAD, false>(y, xblk, q, NoExact{}, word, byte);
    }
    __builtin_amdgcn_raw_buffer_store_b32(word, rsrc(cc, in ? crow_bytes : 0), coff, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, rsrc(cs, in ? srow_bytes : 0), soff, 0, 0);
    if constexpr (STORE_Y) {
      if (live && in) {
        float* yr = a.Y + crow * d + 32 * j + 8 * q;
        *reinterpret_cast<f32x4*>(yr) = f32x4{y[0], y[1], y[2], y[3]};
        *reinterpret_cast<f32x4*>(yr + 4) = f32x4{y[4], y[5], y[6], y[7]};
      }
    }
    cleft -= step_rows;
    crow += step_rows;
    cx += cxstep;
    cc += ccstep;
    cs += csstep;
  };

#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k) load(k, buf[k]);
  for (int it = 0; it < nsteps; it += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int s = it + k;
      if (s < nsteps) {
        load(s + kDepth - 1, buf[(k + kDepth - 1) % kDepth]);
        compute(s, buf[k]);
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
  const void* fn = nullptr;
  switch (front) {
    case FRONT_KRON: fn = pick<FRONT_KRON>(store_y); break;
    case FRONT_PLAIN: fn = pick<FRONT_PLAIN>(store_y); break;
    case FRONT_SMOOTH: fn = pick<FRONT_SMOOTH>(store_y); break;
    case FRONT_HADAMARD: fn = pick<FRONT_HADAMARD>(store_y); break;
    default: return hipErrorInvalidValue;
  }
  QuadArgs a = args;
  a.ngroups = (a.nb + 15) / 16;
  a.nchunks = chunks_one_round(fn, 64 * kWaves, a.ngroups, (a.T + kWaves - 1) / kWaves);
  void* kargs[] = {&a};
  return hipLaunchKernel(fn, dim3(a.ngroups * a.nchunks), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace kq
