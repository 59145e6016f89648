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
// workgroup (8 waves, one block each: 512 B of each row) stages each 32-row
// tile through LDS: row segments are loaded from HBM into a padded LDS tile,
// each wave reads its block back in operand layout (two 16-token MFMA
// groups), and the code words and scale bytes go through a second LDS tile
// so that they leave as contiguous 128-byte code segments per row.  Double
// buffers, one barrier per tile, global loads kept two (or three) tiles
// ahead; all global accesses go through buffer descriptors with
// wave-uniform cursors advanced by a constant per tile (few scalar
// instructions per tile).  Output channels are permuted across the MFMA
// rows so that each lane ends up with 8 consecutive channels of one token:
// lane (t = l & 15, q = l >> 4) holds channels 8q .. 8q+7 of token t.
#include "kq_device.hpp"
#include "kq_internal.h"

#include <algorithm>

namespace kq {

namespace {

constexpr int kWaves = 8;                          // waves per workgroup
constexpr int kCB = kWaves;                        // blocks per column group (512 B of a row), one per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kRT = 2;                             // 16-row MFMA sub-tiles per tile
constexpr int kRows = 16 * kRT;                    // rows per tile
constexpr int kPieces = kRows * kCB * 4;           // 16-byte pieces of X per tile
constexpr int kPPT = kPieces / kThreads;           // pieces per thread per tile
// LDS bytes per input row: 528 = 132 dwords, 4 banks apart mod 64, so the
// block reads (16 lanes on 16 rows, 16 bytes each) touch every bank once.
constexpr int kInStride = kCB * 64 + 16;
// LDS bytes per code row: 144 = 36 dwords.  The 4-byte code writes (16 rows
// x 4 lanes) touch every bank once; the 16-byte reads of the row segments
// (8 lanes on each of two rows) do not: the two rows' 32-dword spans start
// 36 dwords apart and share banks 0-3 mod 64.  The counters show bank
// conflicts for this kernel (about 1.5 cycles per LDS instruction), none
// for the block-per-lane kernel.  A dense 128-byte row with the chunk index
// XOR-swizzled by row pair (both accesses then touch every bank once)
// removed a quarter of those cycles and changed no timing: the rest come
// from elsewhere, and none of them is on the kernel's critical path.
constexpr int kOutStride = kCB * 16 + 16;
constexpr int kInBytes = kRows * kInStride;
constexpr int kOutBytes = kRows * kOutStride;
constexpr int kScaleBytes = kRows * kCB;
constexpr int kOPT = (kRows * kCB + kThreads - 1) / kThreads;  // output pieces per thread
static_assert(kPPT * kThreads == kPieces, "tile pieces must split evenly over the workgroup");

// Output channel held by MFMA row m of half h.
__device__ __forceinline__ int out_channel(int h, int m) { return 8 * (m >> 2) + 4 * h + (m & 3); }

// Two fp32 values rounded to bf16 (nearest even), packed (first in the low half).
__device__ __forceinline__ unsigned bf16_pair(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// The 15 scalars of one block, (l, a, b) of G1 .. G5.
struct Params15 {
  float v[15];
};

// K^T operands of one block for this lane: A[h][s] holds the 8 entries
// K[8q .. 8q+7][out_channel(h, m)] (q = lane >> 4, m = lane & 15) of term s.
//
// From the 15 scalars: lanes 0 .. 4 each build one factor in fp64 (lane k
// factor G(k+1)) and stage it in LDS, where the exact path also finds the
// five; every lane then reads the factor entries of its output channel and
// forms its 8 entries as products in factor order, sharing the partial
// products of the leading factors (the rounding sequence of each entry is
// that of kq_build_blocks), rounds them to fp32 and splits them into three
// bf16 terms, each rounded to nearest-even from the fp32 entry.
template <int KSRC>
__device__ __forceinline__ void setup_a(bf16x8 A[2][3], const Params15& pv, const uint16_t* __restrict__ kblk,
                                        int lane, double* __restrict__ g_lds) {
  const int m = lane & 15, q = lane >> 4;
  if constexpr (KSRC == KSRC_PARAMS) {
    if (lane < 5) {
      // this lane's factor scalars, written into lanes 1 .. 4 from the
      // wave-uniform set (lane 0 keeps G1's)
      float f3[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        int v = __float_as_int(pv.v[i]);
#pragma unroll
        for (int k = 1; k < 5; ++k) {
          const int src = __builtin_amdgcn_readfirstlane(__float_as_int(pv.v[3 * k + i]));  // uniform
          asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(src), "i"(k));
        }
        f3[i] = __int_as_float(v);
      }
      store_factor(factor_f64(f3), g_lds + 4 * lane);
    }
    // LDS accesses of one wave complete in issue order; the fence keeps the
    // compiler from moving the reads above the writes of other lanes.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = out_channel(h, m);
      // entry [rb][bit of c] of factor k, k = 0 .. 4 (G1 .. G5)
      auto e = [&](int k, int rb) { return g_lds[4 * k + 2 * rb + ((c >> (4 - k)) & 1)]; };
      const double p12 = e(0, q >> 1) * e(1, q & 1);
      const double p3[2] = {p12 * e(2, 0), p12 * e(2, 1)};
      double p4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p4[u] = p3[u >> 1] * e(3, u & 1);
      const double g5[2] = {e(4, 0), e(4, 1)};
      u32x4 t[3];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // entries 2u, 2u + 1: one packed pair per term
        float k0 = (float)(p4[u] * g5[0]), k1 = (float)(p4[u] * g5[1]);
        // opaque copies: the bf16 roundings below must start from the fp32
        // entries (the compiler would otherwise round the fp64 products to
        // bf16 directly, through a longer round-to-odd sequence)
        asm("" : "+v"(k0), "+v"(k1));
        const unsigned hi = bf16_pair(k0, k1);
        const float r0 = k0 - __uint_as_float(hi << 16), r1 = k1 - __uint_as_float(hi & 0xFFFF0000u);
        const unsigned mid = bf16_pair(r0, r1);
        const unsigned lo = bf16_pair(r0 - __uint_as_float(mid << 16), r1 - __uint_as_float(mid & 0xFFFF0000u));
        t[0][u] = hi;
        t[1][u] = mid;
        t[2][u] = lo;
      }
#pragma unroll
      for (int s = 0; s < 3; ++s) A[h][s] = __builtin_bit_cast(bf16x8, t[s]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = out_channel(h, m);
#pragma unroll
      for (int s = 0; s < 3; ++s)
        A[h][s] = *reinterpret_cast<const bf16x8*>(kblk + (s * 32 + c) * 32 + 8 * q);
    }
  }
}

// AdaLN producer step on this lane's 8 bf16 values of one token, in fp32,
// one IEEE operation each and in this order (no contraction): centre and
// scale by the row statistics, times (1 + scale[c]), plus shift[c]; then
// rounded to bf16 (nearest even).  The transform then sees exactly the bf16
// activation an unfused LayerNorm + modulation kernel would have written.
// A step whose input is absent gets an identity operand instead of a branch
// (mean +0, rstd 1, scale factor 1, shift -0: x - 0, x * 1 and x + (-0) are
// x exactly, signed zeros included), so the four operations run
// unconditionally (as selects, the skipped steps had cost three more
// instructions per value).
__device__ __forceinline__ bf16x8 modulate8(bf16x8 x, float mean, float rstd, const float opa[8],
                                            const float sh[8]) {
#pragma clang fp contract(off)
  bf16x8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = (float)x[i];
    v = v - mean;
    v = v * rstd;
    v = v * opa[i];
    v = v + sh[i];
    out[i] = (__bf16)v;
  }
  return out;
}

// AHEAD: tiles of global loads in flight beyond the current one (2, or 3 for
// the K-from-scalars kernel when a workgroup has few tiles: more of its
// loads then overlap the K setup).
template <int KSRC, bool STORE_Y, bool MOD, int AHEAD>
__global__ __launch_bounds__(kThreads) void mfma_kernel(MfmaArgs a) {
  constexpr int kAhead = AHEAD;
  __shared__ __attribute__((aligned(16))) uint8_t lds_in[2][kInBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_out[2][kOutBytes];
  __shared__ uint8_t lds_sc[2][kScaleBytes];
  __shared__ double lds_g[kCB][20];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntile_rows = (a.T + kRows - 1) / kRows;
  // Work of this workgroup: column group g, nsteps row tiles starting at row
  // row_first, step_rows apart, all below row_end.
  int g, row_first, step_rows, nsteps, row_end;
  if ((int)blockIdx.x < a.w1) {
    const int wg = xcd_remap(blockIdx.x, a.w1);
    const int c = wg / a.ngroups;
    const int lim = min(a.r1, ntile_rows);
    g = wg % a.ngroups;
    nsteps = c < lim ? (lim - 1 - c) / a.nchunks + 1 : 0;
    row_first = kRows * c;
    step_rows = kRows * a.nchunks;
    row_end = min(a.T, kRows * lim);
  } else {
    const int wg = xcd_remap((int)blockIdx.x - a.w1, (int)gridDim.x - a.w1);
    const int t0 = a.r1 + (wg / a.ngroups) * a.n2;
    g = wg % a.ngroups;
    nsteps = max(0, min(a.n2, ntile_rows - t0));
    row_first = kRows * t0;
    step_rows = kRows;
    row_end = min(a.T, kRows * (t0 + nsteps));
  }
  const int jg = kCB * g;
  const int nvalid = min(kCB, a.nb - jg);
  const int64_t d = a.d;

  const bool mine = wv < nvalid;  // this wave's block exists
  // The block's scalars are requested first, and unconditionally (a clamped
  // block for waves without one), so that no wait for them lands in front of
  // the first X loads.
  Params15 pv;
  if constexpr (KSRC == KSRC_PARAMS) {
    const float* p = a.P + (int64_t)min(jg + wv, a.nb - 1) * a.pstride;
#pragma unroll
    for (int i = 0; i < 15; ++i) pv.v[i] = p[i];
  }
  bf16x8 A[2][3];                 // K^T operands: [output half][term hi, mid, lo]

  uint32_t xoff[kPPT];
  int lin[kPPT];
#pragma unroll
  for (int k = 0; k < kPPT; ++k) {
    const int p = tid + kThreads * k;
    const int row = p / (4 * kCB), col = p % (4 * kCB);
    xoff[k] = (col >> 2) < nvalid ? (uint32_t)(row * d * 2 + 64 * jg + 16 * col) : kOut;
    lin[k] = row * kInStride + 16 * col;
  }
  uint32_t coff[kOPT], soff[kOPT];
  int lout[kOPT], lsc[kOPT];
#pragma unroll
  for (int k = 0; k < kOPT; ++k) {
    const int i = tid + kThreads * k;
    const int ii = i % (kRows * kCB);
    const int orow = ii / kCB, ocol = ii % kCB;
    const bool omine = i < kRows * kCB && ocol < nvalid;
    coff[k] = omine ? (uint32_t)(orow * (d >> 1) + 16 * (jg + ocol)) : kOut;
    soff[k] = omine ? (uint32_t)(orow * a.nb + jg + ocol) : kOut;
    lout[k] = orow * kOutStride + 16 * ocol;
    lsc[k] = orow * kCB + ocol;
  }

  u32x4 pre[kAhead][kPPT];
  // MOD: (mean, rstd) of rows 16 rt + tl of the tiles in flight, loaded with
  // their X (a zero-range descriptor when there are no statistics).
  u32x2 pst[kAhead][kRT];
  u32x2 cst[kRT];
  // Wave-uniform cursors, advanced by a constant per tile: the next tile to
  // load and the next tile to write out.  `left` counts the rows from a
  // cursor to row_end (negative past it); range sizes are clamped to one
  // tile, so rows past the end read zeros / drop stores, and the loads
  // issued ahead of the last tile fetch nothing.
  const int xrow_bytes = 2 * a.d, crow_bytes = a.d >> 1, srow_bytes = a.nb;
  auto rows_in = [](int left) { return left <= 0 ? 0 : (left >= kRows ? kRows : left); };

  int lleft = row_end - row_first;
  const uint8_t* lx = reinterpret_cast<const uint8_t*>(a.X) + (int64_t)row_first * xrow_bytes;
  const int64_t lstep = (int64_t)step_rows * xrow_bytes;
  const uint8_t* lst = reinterpret_cast<const uint8_t*>(a.stats) + (int64_t)row_first * 8;
  const int tl = lane & 15, q = lane >> 4;
  auto gload_next = [&](int slot) {
    const auto rx = rsrc_uniform(lx, rows_in(lleft) * xrow_bytes);
#pragma unroll
    for (int k = 0; k < kPPT; ++k) pre[slot][k] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[k], 0, kNT);
    if constexpr (MOD) {
      const auto rst = rsrc_uniform(lst, a.stats ? rows_in(lleft) * 8 : 0);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        pst[slot][rt] = __builtin_amdgcn_raw_buffer_load_b64(rst, (uint32_t)(16 * rt + tl) * 8u, 0, 0);
      lst += (int64_t)step_rows * 8;
    }
    lleft -= step_rows;
    lx += lstep;
  };
  auto lwrite = [&](int buf, int slot) {
#pragma unroll
    for (int k = 0; k < kPPT; ++k) *reinterpret_cast<u32x4*>(&lds_in[buf][lin[k]]) = pre[slot][k];
    if constexpr (MOD) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) cst[rt] = pst[slot][rt];
    }
  };
  int sleft = row_end - row_first;
  uint8_t* sc = a.codes + (int64_t)row_first * crow_bytes;
  uint8_t* ss = a.scales + (int64_t)row_first * srow_bytes;
  const int64_t cstep = (int64_t)step_rows * crow_bytes, sstep = (int64_t)step_rows * srow_bytes;
  auto gstore_next = [&](int buf) {
    const int n = rows_in(sleft);
    const auto rc = rsrc_uniform(sc, n * crow_bytes);
    const auto rs = rsrc_uniform(ss, n * srow_bytes);
#pragma unroll
    for (int k = 0; k < kOPT; ++k) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&lds_out[buf][lout[k]]);
      __builtin_amdgcn_raw_buffer_store_b128(v, rc, coff[k], 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8(lds_sc[buf][lsc[k]], rs, soff[k], 0, 0);
    }
    sleft -= step_rows;
    sc += cstep;
    ss += sstep;
  };

  int crow = row_first;  // first row of the tile being computed
  // MOD: this lane's (1 + scale, shift) for its 8 channels, of sample cur_s
  float opa[8], sh[8];
  int cur_s = -1;
  auto compute = [&](int buf) {
    if (!mine) return;  // wave-uniform
    const int jl = wv, j = jg + jl;
    if constexpr (MOD) {
      // tiles never straddle samples (tokens_per_sample is a multiple of the tile rows, or covers all rows)
      const int smp = crow / a.tps;
      if (smp != cur_s) {  // wave-uniform; a few times per workgroup at most
        cur_s = smp;
        // four 16-byte loads under one wait: the wait also drains the X
        // tiles in flight (the load counter retires in order), so it must
        // come once per sample change, not once per value
        const int64_t off = (int64_t)smp * a.d + 32 * j + 8 * q;
        f32x4 m0 = {0.f, 0.f, 0.f, 0.f}, m1 = m0, h0 = {-0.f, -0.f, -0.f, -0.f}, h1 = h0;
        if (a.mscale) {  // uniform
          m0 = *reinterpret_cast<const f32x4*>(a.mscale + off);
          m1 = *reinterpret_cast<const f32x4*>(a.mscale + off + 4);
        }
        if (a.mshift) {  // uniform
          h0 = *reinterpret_cast<const f32x4*>(a.mshift + off);
          h1 = *reinterpret_cast<const f32x4*>(a.mshift + off + 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          opa[i] = 1.0f + m0[i];
          opa[4 + i] = 1.0f + m1[i];
          sh[i] = h0[i];
          sh[4 + i] = h1[i];
        }
      }
    }
    // all MFMAs of the tile first, so their latency overlaps the epilogues
    float y[kRT][8];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int tr = 16 * rt + tl;
      bf16x8 xb = *reinterpret_cast<const bf16x8*>(&lds_in[buf][tr * kInStride + 64 * jl + 16 * q]);
      if constexpr (MOD) {
        const bool norm = a.stats != nullptr;  // uniform
        xb = modulate8(xb, norm ? __uint_as_float(cst[rt][0]) : 0.0f, norm ? __uint_as_float(cst[rt][1]) : 1.0f,
                       opa, sh);
        // the exact path reads the block back from this tile
        *reinterpret_cast<bf16x8*>(&lds_in[buf][tr * kInStride + 64 * jl + 16 * q]) = xb;
      }
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][2], xb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][2], xb, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][1], xb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][1], xb, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][0], xb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][0], xb, acc1, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[rt][i] = acc0[i];
        y[rt][4 + i] = acc1[i];
      }
    }
    float amax[kRT];
    bool near = false;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      amax[rt] = block_amax<LAYOUT_MFMA>(y[rt]);
      near = near || near_pow2(amax[rt]);
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(near) != 0, 0)) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        // the exact path reads this token's block back from the LDS tile
        const uint16_t* xblk = reinterpret_cast<const uint16_t*>(&lds_in[buf][(16 * rt + tl) * kInStride + 64 * jl]);
        if constexpr (KSRC == KSRC_PARAMS) {
          settle(y[rt], amax[rt], xblk, q, ExactFromFactors{lds_g[jl]});
        } else {
          settle(y[rt], amax[rt], xblk, q, ExactFromSplit{a.Kbf + (int64_t)j * a.kstride});
        }
        amax[rt] = block_amax<LAYOUT_MFMA>(y[rt]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int tr = 16 * rt + tl;
      const unsigned byte = e8m0_byte(amax[rt]);
      const unsigned word = amax[rt] == 0.0f ? 0u : pack_fp4(y[rt], byte);
      *reinterpret_cast<unsigned*>(&lds_out[buf][tr * kOutStride + 16 * jl + 4 * q]) = word;
      if (q == 0) lds_sc[buf][tr * kCB + jl] = (uint8_t)byte;
      if constexpr (STORE_Y) {
        if (crow + tr < a.T) {
          float* yr = a.Y + (int64_t)(crow + tr) * a.d + 32 * j + 8 * q;
          *reinterpret_cast<f32x4*>(yr) = f32x4{y[rt][0], y[rt][1], y[rt][2], y[rt][3]};
          *reinterpret_cast<f32x4*>(yr + 4) = f32x4{y[rt][4], y[rt][5], y[rt][6], y[rt][7]};
        }
      }
    }
  };

  // The first tile's loads go out before the K setup, which overlaps them;
  // the loads of the next tiles follow the setup, so that at the start of the
  // kernel (every workgroup issuing at once) the first tiles arrive early.
  gload_next(0);
  if (mine) setup_a<KSRC>(A, pv, KSRC == KSRC_SPLIT ? a.Kbf + (int64_t)(jg + wv) * a.kstride : nullptr, lane, lds_g[wv]);
#pragma unroll
  for (int k = 1; k < kAhead; ++k) gload_next(k);

  // Per tile s: stage tile s into LDS, fetch tile s + kAhead, barrier, write
  // out tile s - 1, compute tile s.  Every memory instruction is issued
  // unconditionally (out-of-range ones are no-ops), so the loads of the next
  // kAhead tiles stay in flight across the barrier.  Tile 0 is peeled: it has
  // no predecessor to write out.
  if (nsteps == 0) return;  // workgroup-uniform
  lwrite(0, 0);
  gload_next(0);
  __syncthreads();
  compute(0);
  crow += step_rows;
  for (int it = 1; it < nsteps; it += kAhead) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      const int s = it + k;
      if (s < nsteps) {
        const int buf = s & 1;
        lwrite(buf, (1 + k) % kAhead);
        gload_next((1 + k) % kAhead);
        __syncthreads();
        gstore_next(buf ^ 1);
        compute(buf);
        crow += step_rows;
      }
    }
  }
  __syncthreads();
  gstore_next((nsteps - 1) & 1);
}

}  // namespace

hipError_t launch_mfma(int ksrc, bool store_y, bool mod, const MfmaArgs& args, hipStream_t stream) {
  const void* fn;
  const void* fn3 = nullptr;  // the three-ahead form, where there is one
  if (mod) {
    if (store_y) return hipErrorInvalidValue;
    fn = ksrc == KSRC_PARAMS ? (const void*)&mfma_kernel<KSRC_PARAMS, false, true, 2>
                             : (const void*)&mfma_kernel<KSRC_SPLIT, false, true, 2>;
  } else if (ksrc == KSRC_PARAMS) {
    fn = store_y ? (const void*)&mfma_kernel<KSRC_PARAMS, true, false, 2>
                 : (const void*)&mfma_kernel<KSRC_PARAMS, false, false, 2>;
    fn3 = store_y ? (const void*)&mfma_kernel<KSRC_PARAMS, true, false, 3>
                  : (const void*)&mfma_kernel<KSRC_PARAMS, false, false, 3>;
  } else {
    fn = store_y ? (const void*)&mfma_kernel<KSRC_SPLIT, true, false, 2>
                 : (const void*)&mfma_kernel<KSRC_SPLIT, false, false, 2>;
  }
  MfmaArgs a = args;
  const int nt = (a.T + kRows - 1) / kRows;
  a.ngroups = (a.nb + kCB - 1) / kCB;
  a.nchunks = chunks_one_round(fn, kThreads, a.ngroups, nt, a.req_wg_per_cu);
  // Second part of the grid (tiles from r1 on, n2 per workgroup), sized by
  // the tiles a first-part workgroup would otherwise take (measured on
  // MI355X: finish times of equal first-part workgroups spread by up to a
  // fifth of the kernel, with the slow ones tied to address ranges).
  const int per = (nt + a.nchunks - 1) / a.nchunks;
  // (at 24 or more tiles per workgroup, 12% in runs of 3 measured 0.9-1.5% faster on the stress
  // matrix than 18% in runs of 6, in two sweeps with non-overlapping ranges; below 8, single
  // tiles measured 6-8% faster than runs of 2 at PixArt X1 and SANA X1, two sweeps, equal at
  // FLUX X1)
  const int tail_pct = a.req_tail_pct >= 0 ? std::min(a.req_tail_pct, 50) : (per >= 8 ? 12 : 6);
  a.n2 = a.req_n2 > 0 ? std::min(a.req_n2, 64) : (per >= 24 ? 3 : (per >= 8 ? 4 : 1));
  const int n1 = std::max(1, (int)((int64_t)nt * (100 - tail_pct) / (100 * (int64_t)a.nchunks)));
  a.r1 = (int)std::min<int64_t>(nt, (int64_t)n1 * a.nchunks);
  a.w1 = a.ngroups * a.nchunks;
  int64_t w2 = (int64_t)a.ngroups * ((nt - a.r1 + a.n2 - 1) / a.n2);
  // a launch holds fewer than 2^32 work-items: longer runs where a requested
  // split would exceed that (matrices of some 10^11 elements)
  while ((a.w1 + w2) * kThreads >= (int64_t(1) << 32)) {
    a.n2 *= 2;
    w2 = (int64_t)a.ngroups * ((nt - a.r1 + a.n2 - 1) / a.n2);
  }
  // Three tiles ahead when a first-part workgroup has at most four tiles
  // (measured on MI355X: 9% faster at FLUX X1, 16% at PixArt X1; 1-4% slower
  // with more tiles per workgroup).  Both forms fit two workgroups per CU.
  if (fn3 && per <= 4) fn = fn3;
  void* kargs[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)(a.w1 + w2)), dim3(kThreads), kargs, 0, stream);
}

}  // namespace kq
