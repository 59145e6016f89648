// Block-per-lane front-ends fused with the MXFP4 quantizer (gfx950).
//
// The activation X[T][d] is, in memory, a flat sequence of T * d/32 blocks
// of 64 bytes (32 bf16 channels), and the codes and scales are flat
// sequences of 16-byte and 1-byte block records in the same order.  A wave
// takes a unit of 64 consecutive blocks (4 KB of X) at a time: four 1 KB
// loads, each contiguous, land in a wave-private LDS region and are read
// back so that lane i holds all 32 channels of block i of the unit.  The
// whole transform, the block amax, the E8M0 byte and the E2M1 codes then
// stay inside one lane, and the lane's 16 code bytes and its scale byte are
// stored as one contiguous 1 KB + 64 B per wave.  The waves of a workgroup
// never share unit data; only FRONT_ADALN shares its modulation vectors,
// once, at setup.
//
// A wave visits units u0, u0 + P C, u0 + 2 P C, ... with P = nb / gcd(64, nb)
// units spanning a whole number of rows, so lane i always holds the same
// block column j = (64 u0 + i) mod nb and keeps that block's coefficients in
// registers for all of its units.  (FRONT_ADALN on a batch of several
// samples: u0, u0 + P, u0 + 2P, ..., a contiguous band of rows.)
//
// FRONT_KRON: y = x K(j), K = G1 (x) ... (x) G5 (KroQuant; Pith review,
// "What carries the argument": the on-the-fly kernel that builds each block
// from its 15 scalars).  Each factor
//   G = [[1,0],[l,1]] [[a,b],[0,1/a]] = [[1,0],[l,1]] [[1,ab],[0,1]] diag(a,1/a)
// splits into two shears and a diagonal.  By the mixed-product property
// K = (L1 (x) ... (x) L5)(S1 (x) ... (x) S5)(D1 (x) ... (x) D5), and stages
// acting on different channel bits commute, so for a row vector
//   x K = [per factor k, on its bit p: x[c] += l x[c|p], then x[c|p] += ab x[c]
//          for every c with bit p clear]  then  y[c] = x[c] * prod_k D_k[bit_k(c)],
// five butterfly stages of one fused multiply-add per element, and one
// multiply by the product of the five diagonals.  All in fp32; the error
// against the exact sum stays well below 1e-5 of the block amax.
// FRONT_PLAIN: y = x.  FRONT_SMOOTH: y = x * m[c].  FRONT_HADAMARD: the
// 32-point Walsh-Hadamard butterflies, then / sqrt(32).  FRONT_HADAMARD_WIDE:
// blocks of B = 64 .. 512 channels, i.e. of B / 32 consecutive lanes (a
// unit's 64 blocks start on a multiple of B / 32 and rows hold whole
// Hadamard blocks): the 32-point stages in the lane, then one stage per
// channel bit 5 .. log2 B - 1 between lanes 1, 2, 4, 8 apart (swizzles),
// then / sqrt(B).  FRONT_ADALN: the
// AdaLN producer step, then KRON (below, at modulate32).  FRONT_PROBE: the
// same loads, LDS round trip and stores with no arithmetic (a bandwidth
// ceiling for this access pattern; its outputs are a digest, not codes).
#include <type_traits>

#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int kWaves = 4;             // waves per workgroup (independent)
constexpr int kDepth = 2;             // units of loads in flight per wave
constexpr int kUnitBlocks = 64;       // one block per lane
constexpr int kUnitBytes = 64 * 64;   // bf16 bytes of a unit
constexpr int kUnitCodes = 64 * 16;   // code bytes of a unit

// Position (in 16-byte chunks) of quarter qq of block b of a unit in the
// wave's LDS region.  The quarter index is XOR-swizzled with bits 2-3 of the
// block so that the 1 KB writes (16 lanes: blocks 4k .. 4k+3, all quarters)
// and the block reads (16 lanes: blocks 16k .. 16k+15, one quarter each)
// both touch every 4-byte bank of a 256-byte line once.
__device__ __forceinline__ int chunk_pos(int b, int qq) { return 4 * b + (qq ^ ((b >> 2) & 3)); }

// Two chains of three-input maxima (v_max3_f32 with |.| on its inputs): 16
// instructions for the 32 values.
__device__ __forceinline__ float absmax32(const float y[32]) {
  float m0 = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fabsf(y[2]));
  float m1 = fmaxf(fmaxf(fabsf(y[16]), fabsf(y[17])), fabsf(y[18]));
#pragma unroll
  for (int c = 3; c < 15; c += 2) m0 = fmaxf(fmaxf(m0, fabsf(y[c])), fabsf(y[c + 1]));
#pragma unroll
  for (int c = 19; c < 31; c += 2) m1 = fmaxf(fmaxf(m1, fabsf(y[c])), fabsf(y[c + 1]));
  m0 = fmaxf(fmaxf(m0, fabsf(y[15])), fabsf(y[31]));
  return fmaxf(m0, m1);
}

// Maximum over the 32 lanes of each half of the wave (DPP within rows of
// 16, then a swap between rows).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float max32(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror: lane i <-> 7 - i
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror: lane i <-> 15 - i
  const unsigned u = __float_as_uint(v);
  const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 0 <-> 1, 2 <-> 3
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// v of lane ^ M (M < 32), by a bit-mode swizzle within 32 lanes.  The
// exchange then runs on the LDS pipe, not the VALU, which the stages keep
// busy: 1-5% faster at B >= 128 than DPP quad permutes for M = 1, 2 (and
// row rotations for M = 8), measured on MI355X, outputs identical.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

// The AdaLN producer step of one block (the handbook page "Quantization:
// where diffusion differs from an LLM" gives AdaLN as timestep-dependent
// per-channel scales and shifts; the form v (1 + scale) + shift is the
// DiT one): per value, in fp32 and in this order with no contraction,
// v = ((x - mean) * rstd) * opa + sh, rounded to bf16 (nearest even).  An
// absent input is an identity operand (mean +0, rstd 1, opa 1, sh -0), which
// leaves v exactly x, signed zeros included.  y[c] receives the bf16 value
// as fp32; w (if not null) the bf16 pairs, even channel in the low half.
// The rounding converts the pair (+0, v): the bf16 lands in the high half of
// a word whose low half is zero, so the word is already the fp32 value (one
// convert per value and no shift back).
__device__ __forceinline__ void modulate32(const u32x4 x[4], float mean, float rstd, const float opa[32],
                                           const float sh[32], float y[32], u32x4* w) {
#pragma clang fp contract(off)
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      unsigned pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 8 * qq + 2 * e + h;
        float v = h ? bf16_hi(x[qq][e]) : bf16_lo(x[qq][e]);
        v = v - mean;
        v = v * rstd;
        v = v * opa[c];
        v = v + sh[c];
        const unsigned word = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{0.0f, v}, bf16x2));
        y[c] = __uint_as_float(word);
        pair |= h ? word : word >> 16;
      }
      if (w) w[qq][e] = pair;
    }
}

// Exact quantization of block b of the staged unit, by the whole wave: a
// block whose fp32 amax lies within 2^-16 of a power of two, where the
// transform's rounding could decide the scale (rare).  Lane c (mod 32)
// computes output channel c exactly, as the fp64 sum from +0 in input order
// of the exact products x[r] K32[r][c] (KRON) or of (-1)^popcount(r & c) x[r]
// then divided by sqrt(32) (HADAMARD), rounded once to fp32.  K32[r][c] is
// the fp64 product, in factor order, of one entry per factor (G1 on bit 4),
// rounded to fp32, with G = [[a, b], [l a, l b + 1/a]] in fp64 from the
// block's 15 scalars p15 (kept in LDS by the kernel's setup; the quotients
// 1/a are formed here, so that the common path carries no fp64 division).
// The 32 products of a column are summed in one dependent chain, which sets
// most of this path's time: splitting the products between the two
// half-waves (fewer fp64 instructions, same chain) was no faster.
// The block is then quantized from these values: res receives its four code
// words and its scale byte, ys (if not null) the 32 values.  Everything after
// the first reads runs in registers, so that a wave meeting such a block is
// held up only briefly.  The KroQuant fronts inline it (as a call it cost
// the kernel 20 more registers and 0.5-2% of its time);
// the Hadamard front calls it (inlined there, up to 5% slower at the small
// matrices).
template <int FRONT>
__device__ __forceinline__ void exact_block(const uint8_t* stage, int b, const float* p15, int lane,
                                            unsigned* res, float* ys) {
  const int c = lane & 31;
  u32x4 w[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) w[qq] = *reinterpret_cast<const u32x4*>(stage + 16 * chunk_pos(b, qq));
  auto x_of = [&](int r) {
    const unsigned v = w[r >> 3][(r >> 1) & 3];
    return (double)((r & 1) ? bf16_hi(v) : bf16_lo(v));
  };
  double s = 0.0;
  if constexpr (FRONT == FRONT_KRON) {
    // Lane k < 5 forms the two computed entries of factor k, l a and
    // l b + 1/a (l b is exact in fp64: one rounding), so that the wave runs
    // one fp64 division instead of five; every lane then takes the entries
    // of its column c from lanes 0 .. 4.
    const int kk = lane < 5 ? lane : 0;
    const double Lk = p15[3 * kk], Ak = p15[3 * kk + 1], Bk = p15[3 * kk + 2];
    const double q0 = Lk * Ak, q1 = fma(Lk, Bk, 1.0 / Ak);
    auto from_lane = [](double v, int k) {
      const uint64_t u = __builtin_bit_cast(uint64_t, v);
      const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, k);
      const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), k);
      return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    };
    double e0[5], e1[5];  // entries G_k[0][bit] and G_k[1][bit] of column c's bit of each factor
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const bool bit = (c >> (4 - k)) & 1;
      e0[k] = (double)(bit ? p15[3 * k + 2] : p15[3 * k + 1]);
      e1[k] = bit ? from_lane(q1, k) : from_lane(q0, k);
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      double p = ((r >> 4) & 1) ? e1[0] : e0[0];
      p = p * (((r >> 3) & 1) ? e1[1] : e0[1]);
      p = p * (((r >> 2) & 1) ? e1[2] : e0[2]);
      p = p * (((r >> 1) & 1) ? e1[3] : e0[3]);
      p = p * ((r & 1) ? e1[4] : e0[4]);
      s = fma(x_of(r), (double)(float)p, s);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 32; ++r) s = s + ((__popc(r & c) & 1) ? -x_of(r) : x_of(r));
  }
  const float y = FRONT == FRONT_KRON ? (float)s : (float)(s / 5.6568542494923801952067548968387923142786875015078);
  const unsigned byte = e8m0_byte(max32(fabsf(y)));
  // channels 2q, 2q + 1 -> code byte q (even channel in the low nibble)
  const float y1 = dpp_f<0xB1>(y);
  const unsigned pair = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, y1, __uint_as_float(byte << 23), 0) & 0xFFu;
  if (lane < 32 && !(c & 1)) reinterpret_cast<uint8_t*>(res)[c >> 1] = (uint8_t)pair;
  if (lane == 0) res[4] = byte;
  if (ys && lane < 32) ys[c] = y;
}

// Whether a KRON block whose fp32 amax lies within 2^-16 of a power of two
// (near_pow2) can have its exact amax on the other side of it.  The fp32
// transform of a block is within 27.2 u N_A max|x| of the exact sum (u =
// 2^-24; N_A = prod_k max row sum of |D_k||U_k||L_k| = [[|a|, |a||l|],
// [|b|, (1 + |a b||l|) / |a|]]: the rounding bound of the five shear pairs,
// the coefficient a b and the diagonal), and the exact amax rounds to fp32
// within 1.1 u amax; so only a block whose amax is within that distance of
// the power of two (times 1.01, which covers this evaluation's own
// roundings) needs its exact values.  Blocks outside the range where the
// bound holds as stated (amax below 2^-100, where products may be
// subnormal; a power of two at the top of the fp32 range; non-finite
// values) always answer yes.  The block's bf16 words are read from the
// stage; p15: its 15 scalars.
__device__ __forceinline__ bool straddle_possible(float amax, const uint8_t* stage, int lane, const float* p15) {
  // largest bf16 magnitude of the block: packed 16-bit maxima of the words
  // with their sign bits cleared (integer order is magnitude order); one
  // quarter at a time, so that the path needs few registers
  typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
  u16x2 m = {0, 0};
#pragma unroll 1
  for (int qq = 0; qq < 4; ++qq) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(stage + 16 * chunk_pos(lane, qq));
#pragma unroll
    for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, x[e] & 0x7FFF7FFFu));
  }
  const float mx = fmaxf(__uint_as_float((unsigned)m[0] << 16), __uint_as_float((unsigned)m[1] << 16));
  // (the reciprocal's ulp, like every rounding here, is inside the 1.01 margin)
  float na = 1.0f;
#pragma unroll 1
  for (int k = 0; k < 5; ++k) {
    const float l = fabsf(p15[3 * k]), a = fabsf(p15[3 * k + 1]), b = fabsf(p15[3 * k + 2]);
    na *= fmaxf(a * (1.0f + l), b + (1.0f + a * b * l) * __builtin_amdgcn_rcpf(a));
  }
  const float err = (27.2f * na * mx + 1.1f * amax) * 0x1p-24f * 1.01f;
  const unsigned ab = __float_as_uint(amax);
  const unsigned pe = (ab & 0x7FFFFFu) < kNearLoMant ? ab >> 23 : (ab >> 23) + 1u;  // the power of two's exponent field
  if (pe >= 255u || !(amax >= 0x1p-100f)) return true;
  return !(fabsf(amax - __uint_as_float(pe << 23)) > err);  // a NaN err answers yes
}

template <int FRONT>
__device__ __attribute__((noinline)) void exact_block_call(const uint8_t* stage, int b, const float* p15, int lane,
                                                           unsigned* res, float* ys) {
  exact_block<FRONT>(stage, b, p15, lane, res, ys);
}

// The exact path of FRONT_HADAMARD_WIDE: block b of the staged unit, one
// of the B / 32 blocks (lanes) of its Hadamard block.  Lane c (mod 32)
// computes the block's channel c as the fp64 sum, from +0 in input order,
// of (-1)^popcount(r & col) x[r] over the Hadamard block's B inputs (col:
// the channel's index in the Hadamard block), divided once by sqrt(B) and
// rounded to fp32; then as exact_block.
__device__ __attribute__((noinline)) void exact_block_wide(const uint8_t* stage, int b, int hlog, int lane,
                                                           unsigned* res, float* ys) {
  const int c = lane & 31;
  const int g = 1 << (hlog - 5);
  const int b0 = b & ~(g - 1);
  const int col = 32 * (b - b0) + c;
  double s = 0.0;
#pragma unroll 1
  for (int k = 0; k < g; ++k)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(stage + 16 * chunk_pos(b0 + k, qq));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 32 * k + 8 * qq + e;
        const double x = (double)((e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]));
        s = s + ((__popc(r & col) & 1) ? -x : x);
      }
    }
  // sqrt(B) for B = 64, 128, 256, 512, each correctly rounded
  const double sq = hlog == 6 ? 8.0
                    : hlog == 7 ? 11.313708498984760390413509793677584628557375003016
                    : hlog == 8 ? 16.0
                                : 22.627416997969520780827019587355169257114750006031;
  const float y = (float)(s / sq);
  const unsigned byte = e8m0_byte(max32(fabsf(y)));
  const float y1 = dpp_f<0xB1>(y);
  const unsigned pair = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, y1, __uint_as_float(byte << 23), 0) & 0xFFu;
  if (lane < 32 && !(c & 1)) reinterpret_cast<uint8_t*>(res)[c >> 1] = (uint8_t)pair;
  if (lane == 0) res[4] = byte;
  if (ys && lane < 32) ys[c] = y;
}

// The same values by the fp64 fast Walsh-Hadamard transform, when it is
// provably the same: every input is a bf16, an integer multiple of 2^(e' -
// 134) with e' = max(e, 1) its exponent field, so every partial sum of the
// Hadamard block is an integer multiple of 2^(min e' - 134) of magnitude below
// B 2^(max e' - 126); when max e' - min e' <= 45 - log2 B (nonzero inputs, no
// infinity or NaN) those integers fit in 53 bits, every sum is exact in fp64,
// and the butterflies give exactly the sequential sum.  Layout: lane l holds
// inputs 8 l .. 8 l + 7 of the Hadamard block (in-lane stages on bits 0-2,
// then stages between lanes 1, 2, 4, 8, 16, 32 apart), so block b's values are
// on lanes 4 (b - b0) .. + 3, which quantize them as the exact path's result.
// Returns false (nothing written) when the exponent range is too wide.
__device__ __attribute__((noinline)) bool exact_block_wide_fast(const uint8_t* stage, int b, int hlog, int lane,
                                                                unsigned* res) {
  const int g = 1 << (hlog - 5);
  const int b0 = b & ~(g - 1);
  const bool in = lane < 4 * g;
  const u32x4 w = in ? *reinterpret_cast<const u32x4*>(stage + 16 * chunk_pos(b0 + (lane >> 2), lane & 3))
                     : u32x4{0u, 0u, 0u, 0u};
  int emax = 0, emin = 255;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const unsigned h = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
    if (h & 0x7FFFu) {
      const int e = max((int)((h >> 7) & 0xFFu), 1);
      emax = max(emax, e);
      emin = min(emin, e);
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    emax = max(emax, __shfl_xor(emax, m, 64));
    emin = min(emin, __shfl_xor(emin, m, 64));
  }
  if (emax == 255 || emax - emin > 45 - hlog) return false;  // uniform
  double v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (double)((k & 1) ? bf16_hi(w[k >> 1]) : bf16_lo(w[k >> 1]));
#pragma unroll
  for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (!(k & bit)) {
        const double a0 = v[k], a1 = v[k | bit];
        v[k] = a0 + a1;
        v[k | bit] = a0 - a1;
      }
  for (int m = 1; m < 4 * g; m <<= 1) {  // uniform
    const bool hi = lane & m;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double o = __shfl_xor(v[k], m, 64);
      v[k] = hi ? o - v[k] : v[k] + o;
    }
  }
  // sqrt(B), correctly rounded, as the sequential path divides by it
  const double sq = hlog == 6 ? 8.0
                    : hlog == 7 ? 11.313708498984760390413509793677584628557375003016
                    : hlog == 8 ? 16.0
                                : 22.627416997969520780827019587355169257114750006031;
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = (float)(v[k] / sq);
  // block b: lanes 4 (b - b0) .. + 3, channels 8 (lane & 3) .. + 7
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(y[k]));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  const unsigned byte = e8m0_byte(a);
  const unsigned word = pack_fp4(y, byte);
  if ((lane >> 2) == b - b0) {
    res[lane & 3] = word;
    if ((lane & 3) == 0) res[4] = byte;
  }
  return true;
}

// CPOL: the cache policy of the code and scale stores (0, or kSC1: device
// scope, below at launch_flat).
template <int FRONT, bool STORE_Y, int CPOL>
__global__ __launch_bounds__(64 * kWaves) void flat_kernel(FlatArgs a) {
  __shared__ __attribute__((aligned(256))) uint8_t lds_x[kWaves][kUnitBytes];
  constexpr bool kKron = FRONT == FRONT_KRON || FRONT == FRONT_ADALN;  // fronts with KroQuant's transform
  __shared__ float lds_p[kKron ? kWaves : 1][64][15];                  // exact path: each lane's 15 scalars
  constexpr bool kHad = FRONT == FRONT_HADAMARD || FRONT == FRONT_HADAMARD_WIDE;
  constexpr bool kSum = kKron || kHad;                                 // fronts with an exact path
  __shared__ unsigned lds_res[kSum ? kWaves : 1][64][5];   // exact path: code words and byte per lane
  __shared__ float lds_ys[kSum && STORE_Y ? kWaves : 1][32];  // exact path: the values (diagnostic Y)

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned nph = (unsigned)a.phases;
  const unsigned units = (unsigned)a.units;
  // Wave -> (phase, chunk); unit indices stay below 2^29 (tokens * d <
  // 2^40), so the index arithmetic is 32-bit.  Most fronts: consecutive
  // waves take consecutive phases (the four waves of a workgroup stream
  // adjacent units), and no wave waits for another.  ADALN: the four waves
  // of a workgroup share one phase (consecutive chunks), so that they share
  // one copy of the modulation vectors of its 64 block columns (two
  // workgroup barriers at setup, which a wave without units joins too).
  int ph, chk, n;
  unsigned u0, ustep;
  unsigned wg_u0 = 0;  // ADALN: first unit of the workgroup's wave 0 (units if it has none)
  const bool contiguous = FRONT == FRONT_ADALN && a.tps < a.T;  // uniform
  if constexpr (FRONT == FRONT_ADALN) {
    ph = (int)(blockIdx.x % nph);
    chk = (int)(blockIdx.x / nph) * kWaves + wv;
    if ((unsigned)ph >= units) return;  // uniform over the workgroup
    // This wave's units: u0, u0 + ustep, ... (n of them).  Several samples:
    // a contiguous run of the phase's units, so that a wave's rows seldom
    // change sample.  One sample: chunk c of the phase starts at unit
    // ph + P c and steps over the whole resident round.  A chunk past the
    // last has no units and starts at unit `units` (its loads fetch nothing).
    auto run_start = [&](unsigned c, int& cnt_out) -> unsigned {
      const unsigned C = (unsigned)a.chunks;
      if (c >= C) {
        cnt_out = 0;
        return units;
      }
      if (contiguous) {
        const unsigned cnt = (units - 1 - (unsigned)ph) / nph + 1;
        const unsigned cq = cnt / C, cr = cnt % C;
        cnt_out = (int)(cq + (c < cr ? 1u : 0u));
        return cnt_out ? (unsigned)ph + nph * (c * cq + (c < cr ? c : cr)) : units;
      }
      const unsigned u = (unsigned)ph + nph * c;
      cnt_out = u < units ? (int)((units - 1 - u) / (nph * C)) + 1 : 0;
      return cnt_out ? u : units;
    };
    u0 = run_start((unsigned)chk, n);
    ustep = contiguous ? nph : nph * (unsigned)a.chunks;
    int cnt0;
    wg_u0 = run_start((unsigned)(chk - wv), cnt0);
  } else {
    const unsigned gw = (unsigned)__builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + wv);
    if (gw >= nph * (unsigned)a.chunks) return;  // wave-uniform; nothing below synchronizes the workgroup
    ph = (int)(gw % nph);
    chk = (int)(gw / nph);
    u0 = (unsigned)ph + (unsigned)a.phases * (unsigned)chk;  // first unit
    ustep = (unsigned)a.phases * (unsigned)a.chunks;         // units between this wave's units
    if (u0 >= units) return;
    n = (int)((units - 1 - u0) / ustep) + 1;
  }
  // this lane's block column, for every unit: (64 ph + lane) mod nb
  const unsigned nb = (unsigned)a.nb;
  const unsigned j0 = (64u * (unsigned)ph) % nb;  // wave-uniform
  const int j = (int)(nb >= 64 ? (j0 + lane >= nb ? j0 + lane - nb : j0 + lane) : (j0 + lane) % nb);
  uint8_t* stage = lds_x[wv];

  // ---- per-lane coefficients of block column j
  float sl[5], ss[5], dg[32];  // KRON: shear l, shear a b (G1 .. G5), product of the diagonals
  float mult[32];              // SMOOTH
  if constexpr (kKron) {
    const float* p = a.P + (int64_t)j * a.pstride;
    float da[5], ia[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      sl[k] = p[3 * k];
      const float av = p[3 * k + 1], bv = p[3 * k + 2];
      lds_p[wv][lane][3 * k] = sl[k];  // for the exact path
      lds_p[wv][lane][3 * k + 1] = av;
      lds_p[wv][lane][3 * k + 2] = bv;
      ss[k] = av * bv;
      da[k] = av;
      ia[k] = 1.0f / av;
    }
    // dg[c] = prod_k (bit (4 - k) of c ? 1/a_k : a_k), G1 first
    float h2[4], h3[8], h4[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) h2[c] = ((c >> 1) ? ia[0] : da[0]) * ((c & 1) ? ia[1] : da[1]);
#pragma unroll
    for (int c = 0; c < 8; ++c) h3[c] = h2[c >> 1] * ((c & 1) ? ia[2] : da[2]);
#pragma unroll
    for (int c = 0; c < 16; ++c) h4[c] = h3[c >> 1] * ((c & 1) ? ia[3] : da[3]);
#pragma unroll
    for (int c = 0; c < 32; ++c) dg[c] = h4[c >> 1] * ((c & 1) ? ia[4] : da[4]);
  }
  if constexpr (FRONT == FRONT_SMOOTH) {
    const f32x4* mp = reinterpret_cast<const f32x4*>(a.m + 32 * (int64_t)j);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = mp[k];
#pragma unroll
      for (int i = 0; i < 4; ++i) mult[4 * k + i] = v[i];
    }
  }

  // ---- ADALN: the row of this lane's block in the unit being loaded and in
  // the one being computed (each unit step advances it by rows_step), and
  // the lane's (1 + scale, shift) for its 32 channels of sample cur_s
  unsigned lrow = 0, crow = 0;
  int cur_s = -1;
  float opa[32], sh[32];
  // ADALN: loads (1 + scale, shift) for this lane's 32 channels of sample smp
  auto load_mod = [&](int smp) {
    const int64_t off = (int64_t)smp * (32 * (int64_t)a.nb) + 32 * j;
    if (a.mscale) {  // uniform
      const f32x4* mp = reinterpret_cast<const f32x4*>(a.mscale + off);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const f32x4 v = mp[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) opa[4 * k + i] = 1.0f + v[i];
      }
    }
    if (a.mshift) {  // uniform
      const f32x4* hp = reinterpret_cast<const f32x4*>(a.mshift + off);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const f32x4 v = hp[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) sh[4 * k + i] = v[i];
      }
    }
    cur_s = smp;
  };
  f32x4 mq[4];  // ADALN: this wave's quarter of the workgroup's (scale, shift) slices, as loaded
  int smp0 = 0;
  if constexpr (FRONT == FRONT_ADALN) {
    lrow = crow = (unsigned)((64ull * u0 + (unsigned)lane) / (unsigned)a.nb);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      opa[c] = 1.0f;
      sh[c] = -0.0f;
    }
    // The sample of the workgroup's first row, for every lane of its four
    // waves: the (scale, shift) slices of the phase's 64 block columns, read
    // with coalesced loads (eight 128-byte slices per instruction, a quarter
    // of them by each wave) before the unit loads go out, and passed to
    // their lanes through the workgroup's stages after.  Lanes whose rows
    // lie in another sample load their own when they reach them.
    if (contiguous && wg_u0 < units) smp0 = (int)((64ull * wg_u0 / nb) / (unsigned)a.tps);
    const float* src = wv < 2 ? a.mscale : a.mshift;  // wave-uniform
    if (src) {
      const int64_t base = (int64_t)smp0 * (32 * (int64_t)a.nb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned bo = 32u * (unsigned)(wv & 1) + 8u * (unsigned)i + ((unsigned)lane >> 3);
        mq[i] = *reinterpret_cast<const f32x4*>(src + base + 32 * (int64_t)((j0 + bo) % nb) + 4 * (lane & 7));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const auto rst = rsrc_uniform(a.stats, FRONT == FRONT_ADALN && a.stats ? (int64_t)a.T * 8 : 0);
  u32x2 pst[kDepth];  // ADALN: (mean, rstd) of the rows of the units in flight

  // ---- wave-uniform cursors: the next unit to load, the unit being stored
  const int64_t lstep = (int64_t)ustep * kUnitBytes;
  const uint8_t* lx = reinterpret_cast<const uint8_t*>(a.X) + (int64_t)u0 * kUnitBytes;
  int64_t lleft = a.xbytes - (int64_t)u0 * kUnitBytes;  // bytes from the load cursor to the end of X
  auto clamp_bytes = [](int64_t left, int unit) { return left <= 0 ? 0 : (left >= unit ? unit : (int)left); };
  u32x4 pre[kDepth][4];
  // The loads issued after a wave's last unit fetch nothing.  With the
  // interleaved order they lie past the end of X; ADALN's contiguous runs
  // would otherwise read the start of the next wave's run a second time, so
  // that front counts its loads.
  int loads_left = n;
  auto load = [&](int slot) {
    bool mine = true;
    if constexpr (FRONT == FRONT_ADALN) mine = loads_left-- > 0;  // uniform
    const auto rx = rsrc_uniform(lx, mine ? clamp_bytes(lleft, kUnitBytes) : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pre[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(1024 * i + 16 * lane), 0, kNT);
    if constexpr (FRONT == FRONT_ADALN) {
      // rows past the end (the last unit's tail) read zeros
      pst[slot] = __builtin_amdgcn_raw_buffer_load_b64(rst, mine && lrow < (unsigned)a.T ? 8 * lrow : kOut, 0, 0);
      lrow += (unsigned)a.rows_step;
    }
    lx += lstep;
    lleft -= lstep;
  };
  int64_t ub = (int64_t)u0 * kUnitBlocks;  // first block of the unit being computed
  const int64_t bstep = (int64_t)ustep * kUnitBlocks;

  auto compute = [&](int slot) {
    // stage: 1 KB load i holds 16-byte chunk 64 i + lane = quarter (lane & 3) of block 16 i + lane / 4
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(stage + 16 * chunk_pos(16 * i + (lane >> 2), lane & 3)) = pre[slot][i];
    const u32x2 cst = FRONT == FRONT_ADALN ? pst[slot] : u32x2{0u, 0u};  // this unit's row statistics
    load(slot);  // the slot is free again: the loads of unit + kDepth go out now
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    u32x4 w[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) w[qq] = *reinterpret_cast<const u32x4*>(stage + 16 * chunk_pos(lane, qq));
    float y[32];
    unsigned byte;
    u32x4 cw;
    float mean = 0.0f, rstd = 1.0f;  // ADALN: this block's row statistics
    if constexpr (FRONT == FRONT_PROBE) {
      cw = w[0] ^ w[1] ^ w[2] ^ w[3];
      byte = cw[0] & 0xFFu;
    } else {
      if constexpr (FRONT == FRONT_ADALN) {
        // a new sample for some lane: those lanes load its (1 + scale, shift)
        // (a few times per wave at most; rows past the end keep theirs)
        const bool live = crow < (unsigned)a.T;
        const int smp = a.tps >= a.T ? 0 : (int)(crow / (unsigned)a.tps);
        const bool chg = live && smp != cur_s;
        if (__builtin_amdgcn_ballot_w64(chg) != 0) {
          if (chg) load_mod(smp);
          // wait here, on this rare path, so that no use of the vectors on
          // the common path waits for them (such a wait would also drain the
          // next units' loads, which are older than nothing)
          __builtin_amdgcn_s_waitcnt(0);
        }
        if (a.stats) {  // uniform
          mean = __uint_as_float(cst[0]);
          rstd = __uint_as_float(cst[1]);
        }
        modulate32(w, mean, rstd, opa, sh, y, nullptr);
        crow += (unsigned)a.rows_step;
      } else {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[8 * qq + 2 * e] = bf16_lo(w[qq][e]);
            y[8 * qq + 2 * e + 1] = bf16_hi(w[qq][e]);
          }
      }

      if constexpr (kKron) {
#pragma unroll
        for (int k = 4; k >= 0; --k) {  // G5 (bit 0) first; the stages of different bits commute
          const int bit = 1 << (4 - k);
#pragma unroll
          for (int c = 0; c < 32; ++c)
            if (!(c & bit)) y[c] = fmaf(sl[k], y[c | bit], y[c]);
#pragma unroll
          for (int c = 0; c < 32; ++c)
            if (!(c & bit)) y[c | bit] = fmaf(ss[k], y[c], y[c | bit]);
        }
#pragma unroll
        for (int c = 0; c < 32; ++c) y[c] *= dg[c];
      } else if constexpr (FRONT == FRONT_SMOOTH) {
#pragma unroll
        for (int c = 0; c < 32; ++c) y[c] *= mult[c];
      } else if constexpr (FRONT == FRONT_HADAMARD) {
#pragma unroll
        for (int bit = 1; bit < 32; bit <<= 1)
#pragma unroll
          for (int c = 0; c < 32; ++c)
            if (!(c & bit)) {
              const float u = y[c], v = y[c | bit];
              y[c] = u + v;
              y[c | bit] = u - v;
            }
#pragma unroll
        for (int c = 0; c < 32; ++c) y[c] *= 0.17677669529663688110021109052621225982120698f;  // 1/sqrt(32)
      } else if constexpr (FRONT == FRONT_HADAMARD_WIDE) {
#pragma unroll
        for (int bit = 1; bit < 32; bit <<= 1)
#pragma unroll
          for (int c = 0; c < 32; ++c)
            if (!(c & bit)) {
              const float u = y[c], v = y[c | bit];
              y[c] = u + v;
              y[c | bit] = u - v;
            }
        // channel bits 5 .. hlog - 1: the lane with the bit clear keeps own + partner, the other
        // partner - own
        auto cross = [&](auto m_) {
          constexpr int M = decltype(m_)::value;
          const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
          for (int c = 0; c < 32; ++c) y[c] = fmaf(y[c], sgn, lane_xor<M>(y[c]));
        };
        cross(std::integral_constant<int, 1>{});
        if (a.hlog > 6) cross(std::integral_constant<int, 2>{});  // uniform
        if (a.hlog > 7) cross(std::integral_constant<int, 4>{});
        if (a.hlog > 8) cross(std::integral_constant<int, 8>{});
        const float hs = a.hscale;
#pragma unroll
        for (int c = 0; c < 32; ++c) y[c] *= hs;
      }

      const float amax = absmax32(y);
      byte = e8m0_byte(amax);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) cw[qq] = pack_fp4(&y[8 * qq], byte);
      if constexpr (kSum) {
        // Two rare cases share one test on the common path.  An all-zero
        // block of a sum gives +0 codes (its values may be -0).  Blocks whose
        // amax is within 2^-16 of a power of two are quantized again from
        // exact values, one at a time by the whole wave, after the packing
        // above (so that y need not stay in registers along this path).
        const bool zero = amax == 0.0f;
        bool near = near_pow2(amax);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(zero || near) != 0, 0)) {
          if (zero) cw = u32x4{0u, 0u, 0u, 0u};
          if constexpr (FRONT == FRONT_KRON) {
            // most near blocks are far enough from the power of two for the
            // transform's error bound to settle them (about 3 in 4 on the
            // DiT workloads); the rest take the exact path
            if (near) near = straddle_possible(amax, stage, lane, lds_p[wv][lane]);
          }
          const uint64_t nearm = __builtin_amdgcn_ballot_w64(near);
          if (nearm != 0) {
            if constexpr (FRONT == FRONT_ADALN) {
              // the exact path reads its block from the stage: every lane
              // writes its modulated bf16 values back there first
              u32x4 x[4], mw[4];
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) x[qq] = *reinterpret_cast<const u32x4*>(stage + 16 * chunk_pos(lane, qq));
              modulate32(x, mean, rstd, opa, sh, y, mw);
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<u32x4*>(stage + 16 * chunk_pos(lane, qq)) = mw[qq];
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
              __builtin_amdgcn_wave_barrier();
            }
            for (uint64_t m = nearm; m; m &= m - 1) {
              const int L = __builtin_ctzll(m);
              if constexpr (kKron)
                exact_block<FRONT_KRON>(stage, L, lds_p[wv][L], lane, lds_res[wv][L],
                                        STORE_Y ? lds_ys[STORE_Y ? wv : 0] : nullptr);
              else if constexpr (FRONT == FRONT_HADAMARD_WIDE) {
                if (STORE_Y || !exact_block_wide_fast(stage, L, a.hlog, lane, lds_res[wv][L]))
                  exact_block_wide(stage, L, a.hlog, lane, lds_res[wv][L], STORE_Y ? lds_ys[STORE_Y ? wv : 0] : nullptr);
              }
              else
                exact_block_call<FRONT>(stage, L, lds_p[0][L], lane, lds_res[wv][L],
                                        STORE_Y ? lds_ys[STORE_Y ? wv : 0] : nullptr);
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
              __builtin_amdgcn_wave_barrier();
              if constexpr (STORE_Y) {
                if (lane == L) {
#pragma unroll
                  for (int c = 0; c < 32; ++c) y[c] = lds_ys[wv][c];
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
              }
            }
            if (near) {
              const unsigned* r = lds_res[wv][lane];
              cw = u32x4{r[0], r[1], r[2], r[3]};
              byte = r[4];
            }
          }
        }
      }
    }
    const auto rc = rsrc_uniform(a.codes + ub * 16, clamp_bytes(a.nblocks * 16 - ub * 16, kUnitCodes));
    const auto rs = rsrc_uniform(a.scales + ub, clamp_bytes(a.nblocks - ub, kUnitBlocks));
    __builtin_amdgcn_raw_buffer_store_b128(cw, rc, (uint32_t)(16 * lane), 0, CPOL);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, rs, (uint32_t)lane, 0, CPOL);
    if constexpr (STORE_Y) {
      const auto ry = rsrc_uniform(a.Y + ub * 32, clamp_bytes((a.nblocks - ub) * 128, kUnitBlocks * 128));
#pragma unroll
      for (int k = 0; k < 8; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{y[4 * k], y[4 * k + 1], y[4 * k + 2],
                                                                                 y[4 * k + 3]}),
                                               ry, (uint32_t)(128 * lane + 16 * k), 0, 0);
    }
    ub += bstep;
  };

  // in unit order (the scheduler would otherwise be free to issue the second
  // unit's loads first, and every wait for the first unit would then drain both)
#pragma unroll
  for (int s = 0; s < kDepth; ++s) {
    load(s);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FRONT == FRONT_ADALN) {
    // The slices to their lanes through the four stages (16 KB, free until
    // the first unit): piece q (16 bytes) of slice b of vector t (scale,
    // shift) at piece 512 t + 8 b + (q ^ ((b >> 1) & 7)), XOR-swizzled by
    // slice pair so that the writes (two slices per 16 lanes) and the reads
    // (16 slices per 16 lanes) touch every bank once.
    uint8_t* mods = &lds_x[0][0];
    if (wv < 2 ? a.mscale != nullptr : a.mshift != nullptr) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bo = 32 * (wv & 1) + 8 * i + (lane >> 3), q = lane & 7;
        *reinterpret_cast<f32x4*>(mods + 16 * (512 * (wv >> 1) + 8 * bo + (q ^ ((bo >> 1) & 7)))) = mq[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 0 ? a.mscale == nullptr : a.mshift == nullptr) continue;  // uniform
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 r = *reinterpret_cast<const f32x4*>(mods + 16 * (512 * t + 8 * lane + (q ^ ((lane >> 1) & 7))));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (t == 0)
            opa[4 * q + e] = 1.0f + r[e];
          else
            sh[4 * q + e] = r[e];
        }
      }
    }
    cur_s = smp0;
    __syncthreads();  // every wave holds its vectors before any stage takes a unit
    if (n == 0) return;
  }
  for (int k0 = 0; k0 < n; k0 += kDepth) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s)
      if (k0 + s < n) compute(s);
  }
}

// The diagnostic form that also stores y keeps the default store policy.
template <int FRONT, int CPOL>
const void* pick(bool store_y) {
  return store_y ? (const void*)&flat_kernel<FRONT, true, 0> : (const void*)&flat_kernel<FRONT, false, CPOL>;
}

int gcd64(int nb) {
  int g = 64;
  while (nb % g) g >>= 1;
  return g;
}

}  // namespace

// Store policy, measured on MI355X (same process, identical outputs):
// device-scope stores take 2-7% off the fronts with arithmetic (KroQuant,
// AdaLN, Hadamard) at every DiT matrix and 2% at 453 MB.  The fronts with
// little or none (plain, SmoothQuant, probe) gain 2-5% with them from about
// 64 MiB of X and lose 1-7% below, so they switch there.
constexpr int64_t kScopeSwitchBytes = 64ll << 20;

hipError_t launch_flat(int front, bool store_y, const FlatArgs& args, hipStream_t stream) {
  const void* fn = nullptr;
  const bool big = (int64_t)args.T * args.nb * 64 >= kScopeSwitchBytes;
  switch (front) {
    case FRONT_KRON: fn = pick<FRONT_KRON, kSC1>(store_y); break;
    case FRONT_PLAIN: fn = big ? pick<FRONT_PLAIN, kSC1>(store_y) : pick<FRONT_PLAIN, 0>(store_y); break;
    case FRONT_SMOOTH: fn = big ? pick<FRONT_SMOOTH, kSC1>(store_y) : pick<FRONT_SMOOTH, 0>(store_y); break;
    case FRONT_HADAMARD: fn = pick<FRONT_HADAMARD, kSC1>(store_y); break;
    case FRONT_HADAMARD_WIDE: fn = pick<FRONT_HADAMARD_WIDE, kSC1>(store_y); break;
    case FRONT_PROBE:
      fn = big ? (const void*)&flat_kernel<FRONT_PROBE, false, kSC1> : (const void*)&flat_kernel<FRONT_PROBE, false, 0>;
      break;
    case FRONT_ADALN:
      if (store_y) return hipErrorInvalidValue;
      fn = (const void*)&flat_kernel<FRONT_ADALN, false, kSC1>;
      break;
    default: return hipErrorInvalidValue;
  }
  FlatArgs a = args;
  a.nblocks = (int64_t)a.T * a.nb;
  a.xbytes = a.nblocks * 64;
  a.units = (a.nblocks + kUnitBlocks - 1) / kUnitBlocks;
  a.phases = a.nb / gcd64(a.nb);
  const int64_t per_phase = (a.units + a.phases - 1) / a.phases;
  // one resident round of waves: every wave then owns about the same number of units
  const int64_t slots = (int64_t)cu_count() * resident_per_cu(fn, 64 * kWaves) * kWaves;
  int64_t chunks = a.req_waves > 0 ? (int64_t)a.req_waves / a.phases : slots / a.phases;
  const bool adaln = front == FRONT_ADALN;
  if (adaln && chunks >= kWaves) chunks -= chunks % kWaves;  // whole workgroups per phase
  if (chunks > per_phase) chunks = per_phase;
  if (chunks < 1) chunks = 1;
  a.chunks = (int)chunks;
  // consecutive units of a wave are phases x chunks units = chunks x 64 / gcd(64, nb) rows
  // apart, or phases units = 64 / gcd(64, nb) rows for a contiguous run (ADALN, several samples)
  a.rows_step = (int)((adaln && a.tps < a.T ? 1 : chunks) * (64 / gcd64(a.nb)));
  // ADALN: a workgroup per phase and four chunks; otherwise four consecutive waves
  const int64_t groups = adaln ? a.phases * ((chunks + kWaves - 1) / kWaves)
                               : (a.phases * chunks + kWaves - 1) / kWaves;
  void* kargs[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)groups), dim3(64 * kWaves), kargs, 0, stream);
}

}  // namespace kq
