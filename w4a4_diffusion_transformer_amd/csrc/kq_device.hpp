// Device-side building blocks shared by the libkq kernels (gfx950 only).
//
// Every kernel maps one 32-channel block of one token onto a group of four
// lanes; each lane owns 8 consecutive channels (8q .. 8q+7, q = 0..3) of the
// block.  Two lane layouts exist:
//   LAYOUT_MFMA  the lane order of a 16x16x32 MFMA result: lanes l, l^16,
//                l^32, l^48 share a token (q = lane >> 4);
//   LAYOUT_QUAD  four adjacent lanes share a token (q = lane & 3).
// The MXFP4 epilogue (block amax, E8M0 byte, E2M1 codes) is the same for
// both, only the cross-lane reduction differs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

enum { FRONT_KRON = 0, FRONT_PLAIN = 1, FRONT_SMOOTH = 2, FRONT_HADAMARD = 3 };
// Measurement only: the quantizer's memory traffic with no arithmetic.
enum { FRONT_PROBE = 4 };
// KroQuant with the AdaLN producer step in front of the transform (block-per-lane kernel).
enum { FRONT_ADALN = 5 };
// Block-Hadamard of 64 .. 512 channels (block-per-lane kernel; FRONT_HADAMARD is B = 32).
enum { FRONT_HADAMARD_WIDE = 6 };
enum { LAYOUT_MFMA = 0, LAYOUT_QUAD = 1 };

// Half-width of the window around a power of two inside which a block's
// scale is decided by exact arithmetic: 2^-16 relative, above the transform's
// worst-case fp32 error (1e-5 of the block amax) with margin.
constexpr unsigned kNearLoMant = 1u << 7;              // amax in [2^n, 2^n (1 + 2^-16))
constexpr unsigned kNearHiMant = (1u << 23) - (1u << 8);  // amax in [2^(n+1) (1 - 2^-16), 2^(n+1))

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- factors

// One Kronecker factor in fp64: G = [[1,0],[l,1]] [[a,b],[0,1/a]]
// = [[a, b], [l a, l b + 1/a]] (KroQuant, Sec. 3.2 Eq. (6) as the Pith review
// quotes it, with the determinant +1 form of U).  l a and l b are exact in
// fp64; 1/a and the final sum are single correctly rounded operations.
struct Factor {
  double g00, g01, g10, g11;
};

// The five factors of a block, G1 first.  Named members, not an array, so
// that lane-dependent entry selection stays in registers.
struct Factors {
  Factor f1, f2, f3, f4, f5;
};

__device__ __forceinline__ Factor factor_f64(const float* p) {
  const double L = p[0], A = p[1], B = p[2];
  const double inv_a = 1.0 / A;
  return Factor{A, B, L * A, L * B + inv_a};
}

__device__ __forceinline__ Factors factors_f64(const float* __restrict__ p15) {
  return Factors{factor_f64(p15), factor_f64(p15 + 3), factor_f64(p15 + 6), factor_f64(p15 + 9),
                 factor_f64(p15 + 12)};
}

// Entry [rb][cb] of a factor, rb and cb in {0, 1}.
__device__ __forceinline__ double pick(Factor g, int rb, int cb) {
  const double top = cb ? g.g01 : g.g00;
  const double bottom = cb ? g.g11 : g.g10;
  return rb ? bottom : top;
}

// K[r][c] of K = G1 (x) ... (x) G5 (G1 on bit 4 of r and c, G5 on bit 0): the
// product of one entry per factor, multiplied in factor order in fp64, then
// rounded once to fp32.
__device__ __forceinline__ float k32_entry(Factors F, int r, int c) {
  double p = pick(F.f1, (r >> 4) & 1, (c >> 4) & 1);
  p = p * pick(F.f2, (r >> 3) & 1, (c >> 3) & 1);
  p = p * pick(F.f3, (r >> 2) & 1, (c >> 2) & 1);
  p = p * pick(F.f4, (r >> 1) & 1, (c >> 1) & 1);
  p = p * pick(F.f5, r & 1, c & 1);
  return (float)p;
}

// The factors as 20 doubles (G1 first, each row-major), for staging in LDS.
__device__ __forceinline__ void store_factor(Factor f, double* out) {
  out[0] = f.g00;
  out[1] = f.g01;
  out[2] = f.g10;
  out[3] = f.g11;
}

__device__ __forceinline__ void store_factors(Factors F, double* out) {
  store_factor(F.f1, out);
  store_factor(F.f2, out + 4);
  store_factor(F.f3, out + 8);
  store_factor(F.f4, out + 12);
  store_factor(F.f5, out + 16);
}

// ---------------------------------------------------------------- cross-lane

__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Maximum over the four lanes that hold one token's block (v >= 0).
template <int LAYOUT>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LAYOUT == LAYOUT_QUAD) {
    v = fmaxf(v, dpp_quad_xor1(v));
    v = fmaxf(v, dpp_quad_xor2(v));
    return v;
  } else {
    unsigned u = __float_as_uint(v);
    auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // lanes l and l^16
    v = fmaxf(v, fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1])));
    u = __float_as_uint(v);
    auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // lanes l and l^32
    return fmaxf(v, fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1])));
  }
}

__device__ __forceinline__ float local_absmax8(const float y[8]) {
  float a = fmaxf(fabsf(y[0]), fabsf(y[1]));
  a = fmaxf(a, fmaxf(fabsf(y[2]), fabsf(y[3])));
  a = fmaxf(a, fmaxf(fabsf(y[4]), fabsf(y[5])));
  return fmaxf(a, fmaxf(fabsf(y[6]), fabsf(y[7])));
}

// ---------------------------------------------------------------- exact columns

// Exact value of output channel c of one block, as a correctly rounded fp32:
// the fp64 sum, from +0 in input order r = 0..31, of the exact products
// x[r] K[r][c] (bf16 times fp32 is exact in fp64), rounded once, with K the
// fp32 block (each entry the fp64 product of one entry per factor, rounded).
// The five factors come in fp64 (20 doubles, G1 first, each row-major),
// staged in LDS by the kernel's setup.
struct ExactFromFactors {
  const double* G;
  __device__ float operator()(const uint16_t* __restrict__ xblk, int c) const {
    double s = 0.0;
#pragma unroll 1
    for (int r = 0; r < 32; ++r) {
      double p = G[2 * ((r >> 4) & 1) + ((c >> 4) & 1)];
#pragma unroll
      for (int k = 1; k < 5; ++k) p = p * G[4 * k + 2 * ((r >> (4 - k)) & 1) + ((c >> (4 - k)) & 1)];
      const double x = (double)__uint_as_float((unsigned)xblk[r] << 16);
      s = fma(x, (double)(float)p, s);
    }
    return (float)s;
  }
};

// Same, with K read back from the three-term bf16 split [3][32 c][32 r]:
// (hi + mid) + lo is the fp32 K exactly.
struct ExactFromSplit {
  const uint16_t* kblk;  // this block's [3][32][32]
  __device__ float operator()(const uint16_t* __restrict__ xblk, int c) const {
    double s = 0.0;
#pragma unroll 1
    for (int r = 0; r < 32; ++r) {
      const float hi = __uint_as_float((unsigned)kblk[(0 * 32 + c) * 32 + r] << 16);
      const float mid = __uint_as_float((unsigned)kblk[(1 * 32 + c) * 32 + r] << 16);
      const float lo = __uint_as_float((unsigned)kblk[(2 * 32 + c) * 32 + r] << 16);
      const float k = (hi + mid) + lo;
      const double x = (double)__uint_as_float((unsigned)xblk[r] << 16);
      s = fma(x, (double)k, s);
    }
    return (float)s;
  }
};

// ---------------------------------------------------------------- epilogue
//
// MXFP4 for one lane's 8 values of a block whose four lanes hold one token:
//   amax  = max |y| over the block's 32 values (block_amax, group reduction);
//   byte  = max(exponent_field(amax) - 2, 0) = floor(log2 amax) - 2 + 127,
//           clamped at 0 (amax = 0 and subnormal amax give 0; finite fp32
//           never reaches the upper clamp)  (e8m0_byte);
//   codes = E2M1(y / 2^(byte - 127)) rounded to nearest, ties to the even
//           code, saturating at 6  (pack_fp4).  The gfx950 scaled fp4
//           convert divides by 2^(exponent field of its scale operand - 127),
//           reading field 0 as 2^-127, and rounds exactly like this rule: on
//           MI355X it matched for every finite fp32 input at scale 1 and for
//           every scale byte over 3.4e10 sampled values and all bf16 inputs.
//           So the scale operand is the float whose bit pattern is byte << 23.
//
// Transform front-ends (sums of products) first settle blocks whose amax is
// within 2^-16 of a power of two (near_pow2): the columns that could cross
// it are recomputed exactly (settle), so the scale equals the exact
// evaluation's.  An all-zero block of a transform gets +0 codes (the exact
// sum of zeros is +0).

template <int LAYOUT>
__device__ __forceinline__ float block_amax(const float y[8]) {
  return group_max<LAYOUT>(local_absmax8(y));
}

__device__ __forceinline__ bool near_pow2(float amax) {
  const unsigned ab = __float_as_uint(amax);
  const unsigned ex = ab >> 23, mant = ab & 0x7FFFFFu;
  return ex >= 2u && (mant < kNearLoMant || mant >= kNearHiMant);
}

// Replace every value of a near block that could reach the straddled power
// of two by its exact value.  Call with the whole wave (not under divergence
// between the lanes of a block); lanes whose block is not near keep y.
template <class Exact>
__device__ __forceinline__ void settle(float y[8], float amax, const uint16_t* __restrict__ xblk, int q,
                                       const Exact& exact) {
  if (near_pow2(amax)) {
    const unsigned ab = __float_as_uint(amax);
    const unsigned ex = ab >> 23, mant = ab & 0x7FFFFFu;
    // the power of two being straddled, and the smallest |y| that could reach it
    const unsigned pe = mant < kNearLoMant ? ex : ex + 1u;
    const float thr = __uint_as_float(pe << 23) * (1.0f - 0x1p-14f);
#pragma unroll 1
    for (int i = 0; i < 8; ++i)
      if (fabsf(y[i]) >= thr) y[i] = exact(xblk, 8 * q + i);
  }
}

__device__ __forceinline__ unsigned e8m0_byte(float amax) {
  const unsigned ex = __float_as_uint(amax) >> 23;
  return __builtin_elementwise_sub_sat(ex, 2u);  // max(ex - 2, 0): one clamped subtract
}

__device__ __forceinline__ unsigned pack_fp4(const float y[8], unsigned byte) {
  const float scale = __uint_as_float(byte << 23);
  // Each convert writes one byte of w and keeps the other three; the four
  // together write all of them, so w may start from any value: y[0]'s bits
  // (dead after this call on the common path) spare a register clear.
  unsigned w = __float_as_uint(y[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], scale, 3);
  return w;
}

// The whole epilogue for one block per lane group.
template <int LAYOUT, bool TRANSFORM, class Exact>
__device__ __forceinline__ void mx_epilogue(float y[8], const uint16_t* __restrict__ xblk, int q,
                                            const Exact& exact, unsigned& word, unsigned& byte) {
  float amax = block_amax<LAYOUT>(y);
  if constexpr (TRANSFORM) {
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(near_pow2(amax)) != 0, 0)) {
      settle(y, amax, xblk, q, exact);
      amax = block_amax<LAYOUT>(y);
    }
  }
  byte = e8m0_byte(amax);
  word = pack_fp4(y, byte);
  if constexpr (TRANSFORM) {
    if (amax == 0.0f) word = 0u;
  }
}

// ---------------------------------------------------------------- buffers

constexpr uint32_t kOut = 0xFFFFFFF0u;   // buffer offset past every range: load 0 / store dropped
constexpr int kMaxRecords = 0x7FFFFFFF;  // range cap; in-range offsets stay below 32 d <= 2^29
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family descriptor word 3)
constexpr int kNT = 2;                   // cache-policy bit of a buffer access: non-temporal (streamed once)
constexpr int kSC1 = 16;                 // cache-policy bit of a buffer access: device scope

// Raw buffer descriptor over [base, base + bytes): loads at or past `bytes`
// return zero and stores there are dropped (the hardware range check), so a
// streaming loop can issue the same memory instructions for full and partial
// tiles and the compiler can count outstanding loads exactly.  `base` must be
// wave-uniform (the descriptor lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= kMaxRecords ? kMaxRecords : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcFlags);
}

// Same, with every descriptor field moved to scalar registers.  Where the
// compiler evaluates a cursor's clamp in vector registers it cannot prove the
// descriptor uniform and wraps each buffer access in a loop over the
// distinct descriptors of the wave; reading the fields through readfirstlane
// (they are uniform by construction) removes those loops.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void* base, int64_t bytes) {
  const int n = __builtin_amdgcn_readfirstlane(bytes <= 0 ? 0 : (bytes >= kMaxRecords ? kMaxRecords : (int)bytes));
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t hi = (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo), (short)0, n, kRsrcFlags);
}

// ---------------------------------------------------------------- scheduling

// Workgroups are handed to the 8 XCDs round-robin.  Renumber them so that
// consecutive logical workgroups (adjacent columns of the same rows, which
// share output cache lines) run on the same XCD and its L2.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int per = G >> 3, rem = G & 7, x = b & 7;
  return x * per + (x < rem ? x : rem) + (b >> 3);
}

}  // namespace kq
