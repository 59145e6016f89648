// Vector-ALU comparison front-ends fused with the MXFP4 quantizer (gfx950),
// row layout:
//   FRONT_PLAIN     y = x;
//   FRONT_SMOOTH    y = x * m[c] (SmoothQuant per-channel scale).
// The library runs SmoothQuant here below 2^24 elements, where its 8
// multipliers per lane cost less setup than the block-per-lane kernel's 32
// (kq_flat.hip holds every other front-end).
//
// Lane layout: a wave covers 1 KB of one bf16 row (16 blocks); lane l owns
// the fixed 16-byte piece l, i.e. channels 8q .. 8q+7 (q = l & 3) of block
// l >> 2 of its column group, for every row it visits.  Loads (1 KB), code
// stores (256 B) and scale stores (16 B) of a wave instruction are therefore
// contiguous, and each lane keeps the multipliers of a single block in
// registers.  Rows stream with loads kept several rows ahead.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;  // waves per workgroup, one row each per step
constexpr int kDepth = 6;  // rows in flight per wave (current + 5 ahead)

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
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int g = wg % a.ngroups, c = wg / a.ngroups;
  const int j = 16 * g + (lane >> 2), q = lane & 3;
  const bool live = j < a.nb;  // the last column group may be partial
  const int jc = live ? j : a.nb - 1;

  float mult[8];
  if constexpr (FRONT == FRONT_SMOOTH) {
    const f32x4* mp = reinterpret_cast<const f32x4*>(a.m + 32 * jc + 8 * q);
    const f32x4 m0 = mp[0], m1 = mp[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mult[i] = m0[i];
      mult[4 + i] = m1[i];
    }
  }

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
    if constexpr (FRONT == FRONT_SMOOTH) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] *= mult[i];
    }
    // (plain and SmoothQuant values are exact in fp32: no exact-scale path)
    const uint16_t* xblk = (in ? cx : a.X) + 32 * jc;
    unsigned word, byte;
    mx_epilogue<LAYOUT_QUAD, false>(y, xblk, q, NoExact{}, word, byte);
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
    case FRONT_PLAIN: fn = pick<FRONT_PLAIN>(store_y); break;
    case FRONT_SMOOTH: fn = pick<FRONT_SMOOTH>(store_y); break;
    default: return hipErrorInvalidValue;
  }
  QuadArgs a = args;
  a.ngroups = (a.nb + 15) / 16;
  a.nchunks = chunks_one_round(fn, 64 * kWaves, a.ngroups, (a.T + kWaves - 1) / kWaves);
  void* kargs[] = {&a};
  return hipLaunchKernel(fn, dim3(a.ngroups * a.nchunks), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace kq
