// W4A4 consumer: Y = deq(A) deq(B)^T on the gfx950 scaled FP4 matrix cores.
//
// A [M][K] and B [N][K] are MXFP4 in the quantizer's output format (codes
// [rows][K/2], even element in the low nibble; E8M0 scales [rows][K/32]):
// A the quantized activation X T, B the quantized folded weight W T^-T, so
// that Y approximates X W^T (Pith review, circularity check: Eq. (1); the
// W4A4 MXFP4 GEMM the quantizer feeds).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1: lane l holds 32
// consecutive K values (16 bytes) of row l % 32 at K offset 32 (l / 32) -
// one MX block - and takes that block's E8M0 byte from its scale register
// (its low byte); result register r of lane l
// is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] (verified on MI355X against a
// CPU evaluation).  Products of E2M1 values and power-of-two scales are
// exact; sums are fp32.
//
// Workgroup: 8 waves (2 along M x 4 along N), a 256 x 256 tile of Y, each
// wave 128 x 64 (4 x 2 MFMA tiles of 32 x 32), or, for the tiles of a
// partial last round of the GPU, a 128 x 256 half tile (waves of 64 x 64).
// K advances 128 per stage.
// The A and B stage tiles (256 rows x 64 B each) go from global memory
// straight into LDS (buffer loads with the LDS bit), in a ring of four
// stages: three are in flight while one is multiplied.  Scale bytes go the
// same way, 16 K blocks (four stages) of a row per 16-byte load, into a ring
// of two such groups.  Rows of a staged tile are 64 B; the 16-byte chunk c
// of row r sits at position c ^ ((r / 4) % 4), so that the 16 rows one
// fragment read touches at a fixed chunk fall on distinct banks.  Rows past
// M or N and K blocks past K load as zero codes (buffer range /
// out-of-range offsets), which add nothing.
#include "kq_device.hpp"
#include "kq_internal.h"

namespace kq {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 512;
constexpr int kBM = 256, kBN = 256;  // tile of Y
constexpr int kStages = 4;           // LDS ring
constexpr int kRowB = 64;            // bytes per staged row (128 K values)
constexpr int kTileB = kBM * kRowB;  // 16 KB per operand per stage
constexpr int kGroupM = 4;           // M tiles per group of the tile order
constexpr int kScB = kBM * 16;       // scale bytes per operand per group of 4 stages: [row][16 K blocks]

// Loads into LDS issued as asm, so that the compiler inserts no waits of its
// own for them; the loop waits explicitly (s_waitcnt vmcnt) before the
// barrier that publishes a stage.  Lane i writes LDS bytes m0 + size * i.
__device__ __forceinline__ void dma_b128(u32x4 desc, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 1\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "{m0}"(lds), "v"(voff), "s"(desc)
               : "memory");
}
// An FP4 operand: the instruction reads only the first four registers of
// the eight-register operand when the format is E2M1, so the rest is left
// undefined (no moves to fill it).
__device__ __forceinline__ i32x8 fp4_operand(u32x4 v) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  const i32x4 w = __builtin_bit_cast(i32x4, v);
  return __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
}

// Raw buffer descriptor words over [base, base + bytes), in scalar registers.
__device__ __forceinline__ u32x4 desc_uniform(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= kMaxRecords ? kMaxRecords : (int)bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 dsc;
  dsc[0] = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  dsc[1] = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32)) & 0xFFFFu;
  dsc[2] = (unsigned)__builtin_amdgcn_readfirstlane(n);
  dsc[3] = (unsigned)kRsrcFlags;
  return dsc;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier with no implied wait (each wave has waited for its own
// loads into LDS); the empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// One output tile of 64 MI rows x 256 columns at (m0, n0): MI = 4 is the
// whole 256 x 256 tile, MI = 2 half of one (see launch_gemm).  Each wave
// computes 32 MI rows x 64 columns (MI x 2 MFMA tiles of 32 x 32).
template <int MI>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int m0, int n0, uint8_t (&a_st)[kStages][kTileB],
                                          uint8_t (&b_st)[kStages][kTileB], uint8_t (&as_st)[2][kScB],
                                          uint8_t (&bs_st)[2][kScB]) {
  constexpr int BM = 64 * MI;   // rows of the tile
  constexpr int NA = MI / 2;    // 16-row groups of A each wave stages per stage
  constexpr int kOps = NA + 2;  // code loads per wave and stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int K = g.K, kbytes = K >> 1, kblocks = K >> 5;
  const int nsteps = (K + 127) >> 7;
  const int mrows = min(BM, g.M - m0), nrows = min(kBN, g.N - n0);

  // Code loads of one stage: this wave moves the NA 16-row groups NA wv ..
  // of A and the groups 2 wv, 2 wv + 1 of B (lane l -> row l / 4 of the
  // group, LDS position l % 4, holding chunk (l % 4) ^ ((l / 16) % 4)).
  // Scale loads, once per group of 4 stages: wave w < 4 moves the 16 scale
  // bytes (K blocks of the 4 stages) of A rows 64 w .. 64 w + 63 (none past
  // the tile: a zero range), wave w >= 4 those of B rows 64 (w - 4) ..; one
  // 16-byte load per lane and row (byte offsets need no alignment for these
  // loads: checked on MI355X).  The code descriptors cover only the rows a
  // load may touch; the scale descriptors run to the end of the scale
  // tensor, since a row's last 16-byte piece reaches into the next row.  A
  // dword that crosses the end of a range reads as zero (range checks are
  // per dword: checked on MI355X), so when K / 32 is not a multiple of 4 the
  // final (K / 32) % 4 scale bytes of the last row of A and of B are read
  // here with ordinary loads and patched in at the last stage.
  u32x4 da[NA], db[2], dsc;
  const int cchunk = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    const int G = NA * wv + k;
    const int ra = min(16, max(0, mrows - 16 * G));
    da[k] = desc_uniform(g.a_codes + (int64_t)(m0 + 16 * G) * kbytes, (int64_t)ra * kbytes);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int G = 2 * wv + k;
    const int rb = min(16, max(0, nrows - 16 * G));
    db[k] = desc_uniform(g.b_codes + (int64_t)(n0 + 16 * G) * kbytes, (int64_t)rb * kbytes);
  }
  {
    const bool sa_side = wv < 4;  // wave-uniform
    const int r0 = 64 * (wv & 3);
    const int rs = sa_side ? (r0 < BM ? max(0, g.M - m0 - r0) : 0)  // rows to the end of the tensor
                           : max(0, g.N - n0 - r0);
    dsc = sa_side ? desc_uniform(g.a_scales + (int64_t)(m0 + min(r0, BM)) * kblocks, (int64_t)rs * kblocks)
                  : desc_uniform(g.b_scales + (int64_t)(n0 + r0) * kblocks, (int64_t)rs * kblocks);
  }
  const int kfull = kblocks & ~3, kr = kblocks & 3;
  unsigned pa = 0, pb = 0;  // final partial scale dwords of rows M - 1 and N - 1
  if (kr != 0 && m0 + BM >= g.M) {
    const uint8_t* p = g.a_scales + (int64_t)(g.M - 1) * kblocks + kfull;
    for (int j = 0; j < kr; ++j) pa |= (unsigned)p[j] << (8 * j);
  }
  if (kr != 0 && n0 + kBN >= g.N) {
    const uint8_t* p = g.b_scales + (int64_t)(g.N - 1) * kblocks + kfull;
    for (int j = 0; j < kr; ++j) pb |= (unsigned)p[j] << (8 * j);
  }
  const uint32_t crow_off = (uint32_t)((lane >> 2) * kbytes);
  const uint32_t srow_off = (uint32_t)(lane * kblocks);

  // Vector memory operations this wave issues for stage ks: kOps code loads
  // (parts 0 .. NA - 1 of A, NA and NA + 1 of B), plus the scale load of the
  // stage group when ks opens one (part NA + 2); part -1 issues them all.
  auto issue = [&](int ks, int slot, bool opens_group, int part) {
    const bool cin = ks * 128 + 32 * cchunk < K;
    const uint32_t co = cin ? crow_off + (uint32_t)(64 * ks + 16 * cchunk) : kOut;
#pragma unroll
    for (int k = 0; k < NA; ++k)
      if (part < 0 || part == k) dma_b128(da[k], co, lds_addr(&a_st[slot][1024 * (NA * wv + k)]));
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (part < 0 || part == NA + k) dma_b128(db[k], co, lds_addr(&b_st[slot][1024 * (2 * wv + k)]));
    if (opens_group && (part < 0 || part == NA + 2)) {  // ks % 4 == 0
      const int p = ks >> 2;
      const uint32_t so = 16 * p < kblocks ? srow_off + (uint32_t)(16 * p) : kOut;
      uint8_t* dst = wv < 4 ? &as_st[p & 1][16 * 64 * (wv & 3)] : &bs_st[p & 1][16 * 64 * (wv & 3)];
      dma_b128(dsc, so, lds_addr(dst));
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment rows of this lane and its K half within a 64-K sub-step.
  const int fr = lane & 31, fh = lane >> 5;
  // Scale rows of the current stage group (16 bytes: 4 per stage) of this
  // lane's A rows 32 MI wm + 32 i + fr and B rows 64 wn + 32 j + fr, read
  // once per group as whole rows (16-byte reads at a 16-byte lane stride are
  // free of bank conflicts; 4-byte reads at that stride are not).
  u32x4 ra[MI], rb[2];
  // Stage ks = 4 n + k (k = ks % 4, a constant: the stage loop is unrolled by
  // four) from ring slot k.  next(part) issues one part of a later stage's
  // loads; compute calls it between its MFMAs.
  auto compute = [&](int ks, int k, auto&& next) {
    const uint8_t* as = a_st[k];
    const uint8_t* bs = b_st[k];
    // scale bytes of K blocks 4 ks + fh (sub-step 0: byte 0 after the shift)
    // and 4 ks + 2 + fh (sub-step 1: byte 2, picked with op_sel); blocks past
    // K (whose codes load as zero) get the neutral byte 127; only the last
    // stage can be a tail stage, and only when K / 32 is not a multiple of 4
    const int grp = (ks >> 2) & 1;
    const bool tail = 4 * ks + 4 > kblocks;  // uniform
    auto fix = [&](unsigned w, bool last_row, unsigned patch) {
      if (tail && last_row) w = patch;
      w >>= 8 * fh;
      if (tail) {
        if (4 * ks + fh >= kblocks) w = (w & ~0xFFu) | 127u;
        if (4 * ks + 2 + fh >= kblocks) w = (w & ~0xFF0000u) | (127u << 16);
      }
      return (int)w;
    };
    // Every LDS read of the stage is issued before the first MFMA, each into
    // registers of its own, so the reads overlap one another and the MFMAs
    // wait only for the operands they take.
    u32x4 va[2][MI], vb[2][2];
    if (k == 0) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
        ra[i] = *reinterpret_cast<const u32x4*>(&as_st[grp][16 * (32 * MI * wm + 32 * i + fr)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) rb[j] = *reinterpret_cast<const u32x4*>(&bs_st[grp][16 * (64 * wn + 32 * j + fr)]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 2 * s + fh;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int R = 32 * MI * wm + 32 * i + fr;
        va[s][i] = *reinterpret_cast<const u32x4*>(&as[64 * R + 16 * (c ^ ((R >> 2) & 3))]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int R = 64 * wn + 32 * j + fr;
        vb[s][j] = *reinterpret_cast<const u32x4*>(&bs[64 * R + 16 * (c ^ ((R >> 2) & 3))]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    int sa[MI], sb[2];
#pragma unroll
    for (int i = 0; i < MI; ++i) sa[i] = fix(ra[i][k], m0 + 32 * MI * wm + 32 * i + fr == g.M - 1, pa);
#pragma unroll
    for (int j = 0; j < 2; ++j) sb[j] = fix(rb[j][k], n0 + 64 * wn + 32 * j + fr == g.N - 1, pb);
    // The loads of stage ks + 3 go out one at a time, each after a second
    // MFMA, instead of as one burst after the barrier (1-2% faster at the
    // FLUX shapes, measured on MI355X).
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int idx = (s * MI + i) * 2 + j;  // MFMA number, a constant
          if (idx % 2 == 1 && idx / 2 < kOps + 1) {
            __builtin_amdgcn_sched_barrier(0);
            next(idx / 2);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(va[0][i]), fp4_operand(vb[0][j]),
                                                                        acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(va[1][i]), fp4_operand(vb[1][j]),
                                                                        acc[i][j], 4, 4, 2, sa[i], 2, sb[j]);
        }
  };

  // Stages 0 .. 2 in flight; per stage ks: wait until this wave's loads of
  // stage ks have landed (the loads of stages ks + 1 and ks + 2 may stay
  // outstanding), barrier, multiply stage ks while loading stage ks + 3 into
  // the slot stage ks - 1 used (every wave is past it).  Stages past the end
  // load nothing but zeros.
  issue(0, 0, true, -1);
  issue(1, 1, false, -1);
  issue(2, 2, false, -1);
  // loads issued after stage ks's: those of stages ks + 1 and ks + 2 (2 kOps
  // code loads), plus the scale load of stage ks + 1 or ks + 2 when one of
  // them opens a stage group (k = 3, 2)
  constexpr int w01 = 2 * kOps, w23 = 2 * kOps + 1;
  static_assert(2 * (kOps + 1) <= 4 * MI, "every load of a stage goes out between its MFMAs");
  static_assert(w23 < 16, "vmcnt field");
  for (int ks0 = 0; ks0 < nsteps; ks0 += 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ks = ks0 + k;
      if (ks < nsteps) {  // uniform
        if (k >= 2)
          __builtin_amdgcn_s_waitcnt(w23 | 0x70 | 0xF00);
        else
          __builtin_amdgcn_s_waitcnt(w01 | 0x70 | 0xF00);
        lds_barrier();
        compute(ks, k, [&](int part) { issue(ks + 3, (k + 3) & 3, k == 1, part); });
      }
    }
  }
  // no load into LDS may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);

  // Y rows m0 + 32 MI wm + 32 i + 8 (r / 4) + 4 fh + r % 4, columns n0 + 64 wn + 32 j + fr; one
  // descriptor per 32-row band (ranges stay far below 2^31 bytes for any N).  Device-scope
  // stores: 1-9% faster than the default policy at the DiT shapes (MI355X), non-temporal ones
  // no faster.
  const int64_t N = g.N;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int band = 32 * MI * wm + 32 * i;
    const int brows = min(32, max(0, mrows - band));
    const int64_t base = (int64_t)(m0 + band) * N;
    if (g.y_f32) {
      const auto ry = rsrc_uniform(g.y_f32 + base, (int64_t)brows * N * 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = 64 * wn + 32 * j + fr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * fh + (r & 3);
          const uint32_t off = col < nrows ? (uint32_t)((row * N + n0 + col) * 4) : kOut;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ry, off, 0, kSC1);
        }
      }
    }
    if (g.y_bf16) {
      const auto ry = rsrc_uniform(g.y_bf16 + base, (int64_t)brows * N * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = 64 * wn + 32 * j + fr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * fh + (r & 3);
          const uint32_t off = col < nrows ? (uint32_t)((row * N + n0 + col) * 2) : kOut;
          const __bf16 h = (__bf16)acc[i][j][r];
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), ry, off, 0, kSC1);
        }
      }
    }
  }
}

// Tiles of Y (256 x 256) are numbered in groups of kGroupM M tiles, column
// by column.  Workgroups below full_tiles each compute one whole tile; the
// tiles from full_tiles on (the last, partial round of the GPU) are each
// computed as two 128-row halves by two workgroups, so that round takes
// about half as long.  Each kind is spread over the eight XCDs (workgroups
// are dealt to them in turn) so that XCD x takes the x-th eighth of its
// range of the order, and the workgroups running at once on one XCD share A
// rows and B rows in its L2.
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t a_st[kStages][kTileB];
  __shared__ __attribute__((aligned(1024))) uint8_t b_st[kStages][kTileB];
  __shared__ __attribute__((aligned(256))) uint8_t as_st[2][kScB];  // by parity of the stage group
  __shared__ __attribute__((aligned(256))) uint8_t bs_st[2][kScB];

  const int gm = (g.M + kBM - 1) / kBM, gn = (g.N + kBN - 1) / kBN;
  const int b = (int)blockIdx.x;
  const bool whole = b < g.full_tiles;  // workgroup-uniform
  int t, half = 0;
  if (whole) {
    t = xcd_remap(b, g.full_tiles);
  } else {
    // full_tiles is a multiple of 8, so block b - full_tiles sits on XCD (b - full_tiles) % 8
    const int u = xcd_remap(b - g.full_tiles, 2 * (gm * gn - g.full_tiles));
    t = g.full_tiles + (u >> 1);
    half = u & 1;
  }
  const int per_group = kGroupM * gn;
  const int grp = t / per_group, first = grp * kGroupM;
  const int rows = min(kGroupM, gm - first);
  const int w = t - grp * per_group;
  const int tm = first + w % rows, tn = w / rows;
  if (whole)
    gemm_tile<4>(g, tm * kBM, tn * kBN, a_st, b_st, as_st, bs_st);
  else
    gemm_tile<2>(g, tm * kBM + 128 * half, tn * kBN, a_st, b_st, as_st, bs_st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream) {
  GemmArgs g = args;
  // Wave quantisation: with `slots` workgroups resident at once, the tiles
  // past the last whole multiple of `slots` run as a partial last round.
  // When that round fills at most half the slots, its tiles are computed as
  // two halves each (twice the workgroups, each half the work).
  const int64_t tiles = (int64_t)((g.N + kBN - 1) / kBN) * ((g.M + kBM - 1) / kBM);
  const int64_t slots = (int64_t)cu_count() * resident_per_cu((const void*)&gemm_kernel, kThreads);
  const int64_t rem = tiles % slots;
  const bool split = rem > 0 && 2 * rem <= slots && (tiles - rem) % 8 == 0;
  g.full_tiles = (int)(split ? tiles - rem : tiles);
  const dim3 grid((unsigned)(split ? tiles + rem : tiles));
  void* kargs[] = {&g};
  return hipLaunchKernel((const void*)&gemm_kernel, grid, dim3(kThreads), kargs, 0, stream);
}

}  // namespace kq
