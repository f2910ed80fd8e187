// rkl_tile.h -- bf16 / fp16 MFMA tile engine for gfx950 (CDNA4).
//
// A workgroup tile C[BM, BN] (fp32) is the product of two operand tiles that
// arrive in LDS by direct-to-LDS DMA:  C[m, n] = sum_k A[m, k] * B[n, k].
// Each wave owns a sub-tile made of 32 x 32 blocks computed with
// v_mfma_f32_32x32x16_bf16 (or _f16); the kernels set the wave count and
// the wave layout.
//
// Operands may be K-major in memory (k contiguous: hidden states, LM-head
// weights, dz rows when the contraction runs over the vocabulary) or MN-major
// (m or n contiguous: the fp16 weight copy when the contraction runs over
// the vocabulary, dz and the fp16 copy of h_s when it runs over tokens).
// K-major tiles land as k-contiguous rows and every MFMA fragment is one
// 16-byte LDS read; MN-major tiles land as they are in memory and are read
// back with gfx950's transposing LDS read (two per fragment).
//
// The fused kernels' LDS rows are 128 bytes (64 bf16).  The 16-byte chunk c
// of row r lives at chunk c ^ ((r ^ (r >> 3)) & 7): fragment reads by 8
// consecutive lanes (8 consecutive rows, one chunk) spread over all banks,
// and one direct-to-LDS wave instruction (8 rows of 128 bytes) reads 8 whole
// 128-byte row segments from global memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rkl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // default workgroup size (4 waves) of the tile helpers
constexpr int kKT = 64;             // k extent of one staged tile
constexpr int kLdsRow = kKT * 2;    // bytes per LDS row

__device__ __forceinline__ int lds_off(int r, int chunk) {
  return r * kLdsRow + ((chunk ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// ---------------------------------------------------------------------------
// One 64-deep stage of MFMAs for a wave: FM x FN blocks of 32 x 32.
// arow0/brow0: first LDS row of this wave's A / B sub-tile.
// ---------------------------------------------------------------------------
// ELEM = bf16x8 (bf16 products) or f16x8 (fp16 products); fp32 accumulation.
template <typename ELEM>
__device__ __forceinline__ f32x16 mfma32(ELEM a, ELEM b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<bf16x8>(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<f16x8>(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Per-lane LDS offsets of the MFMA fragments of a swizzled K-major tile.
// Rows step by 32 between fragments, which flips bit 2 of the swizzle only,
// so for a tile row block starting at a multiple of 64 the fragment of
// 32-row block f at 16-deep step ks sits at
//   block base + p[ks ^ 2 (f & 1)] + 4096 f,
//   p[k] = (lane % 32) * 128 + 16 * ((2k + lane / 32) ^ (lane % 8) ^ (lane / 8 % 4)),
// the same four offsets for every block and both operands (this equals
// lds_off(row0 + 32 f + lane % 32, 2 ks + lane / 32) for row0 % 64 == 0).
struct FragLanes {
  uint32_t p[4];
  __device__ __forceinline__ void init(int lane) {
    const int lx = (lane & 7) ^ ((lane >> 3) & 3);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = (uint32_t)((lane & 31) * kLdsRow + (((2 * k + (lane >> 5)) ^ lx) << 4));
  }
};

// One MFMA fragment (B fragments first: the fm-major MFMA order needs every
// b before the second a).  f < FN: b[f]; else a[f - FN].  ldsA / ldsB point
// at this wave's row block (a multiple of 64 rows into the tile).
template <typename ELEM, int FM, int FN>
__device__ __forceinline__ void load_frag(ELEM (&a)[FM], ELEM (&b)[FN], const char* ldsA, const char* ldsB,
                                          const FragLanes& fl, int ks, int f) {
  if (f < FN)
    b[f] = *reinterpret_cast<const ELEM*>(ldsB + fl.p[ks ^ ((f & 1) << 1)] + f * 32 * kLdsRow);
  else
    a[f - FN] = *reinterpret_cast<const ELEM*>(ldsA + fl.p[ks ^ (((f - FN) & 1) << 1)] + (f - FN) * 32 * kLdsRow);
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;
}

template <int BM, int BN>
struct Stages {
  static constexpr int kA = BM * kLdsRow;
  static constexpr int kB = BN * kLdsRow;
  static constexpr int kStage = kA + kB;
};

constexpr int share_lo(int total, int slots, int i) { return (total * i) / slots; }

// ---------------------------------------------------------------------------
// Direct-to-LDS loads (gfx950 global_load_lds_dwordx4: each lane's 16 bytes
// land at the wave-uniform LDS address in M0 + 16 * lane, no VGPRs).  The
// global address is a wave-uniform 64-bit base in SGPRs plus a per-lane
// 32-bit offset; the issue paths below keep everything that depends on the
// k-tile or the block in the scalar base, so the per-lane part is a few
// full-rate integer ops.
// ---------------------------------------------------------------------------
#define RKL_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)RKL_LDS_PTR(p); }

__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t gp = (uint64_t)(uintptr_t)sbase;
  // (readfirstlane returns int: go through uint32_t so nothing is sign-extended)
  const uint32_t g_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(gp >> 32));
  const uint32_t g_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gp);
  const uint64_t g = ((uint64_t)g_hi << 32) | (uint64_t)g_lo;
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  // M0 is only ever written right before the instruction that reads it on
  // gfx9+, so setting it here does not disturb compiler-generated code.
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(g), "s"(l) : "memory", "m0");
}

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4]
// (left at 7 = no wait), lgkmcnt [11:8].
constexpr int waitcnt_imm(int vmcnt, int lgkmcnt) {
  return (vmcnt & 0xF) | ((vmcnt >> 4) << 14) | (7 << 4) | ((lgkmcnt & 0xF) << 8);
}

// Barrier that also publishes the DMA of the stage about to be read: this
// wave's LDS traffic done and at most `keep` DMA instructions (the stage after
// it) still in flight.  The compiler sees the waitcnt (builtin) and so knows
// which DMA stores are complete; the asm barrier keeps LDS accesses in place.
template <int keep>
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(keep, 0));
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One k-tile of the DMA pipeline: MFMAs of the tile in stage `cur`, its
// fragments one step ahead, the ND DMA instructions of the tile two ahead
// (issue(q), q < ND, into stage `pre`) spread evenly over all 32 MFMA slots
// (a burst of them fills the memory pipeline's queue and stalls the MFMAs
// behind it), and between steps 2 and 3 the barrier, after which step 3 reads
// the first fragments of the next tile from `nxt`.  The barrier lets exactly
// the kBefore DMAs of the tile two ahead issued so far stay in flight: every
// older one -- all of the next tile's -- has landed.  The caller's prologue
// issues two whole tiles and waits with ND in flight.
// MASKB: before its MFMAs, each 16-deep step zeroes the B fragments fn whose
// bit in `keep` is clear (this lane's token column fn is left out).
template <int BM, int BN, typename ELEM, int FM, int FN, int ND, bool MASKB = false, class Issue>
__device__ __forceinline__ void dma_iter(f32x16 (&acc)[FM][FN], ELEM (&a)[2][FM], ELEM (&b)[2][FN], Issue issue,
                                         const char* __restrict__ cur, const char* __restrict__ nxt,
                                         const FragLanes& fl, int arow0, int brow0, uint32_t keep = 0) {
  constexpr int M = FM * FN, R = FM + FN;
  constexpr int kA = BM * kLdsRow;
  constexpr int kBefore = share_lo(ND, 4 * M, 3 * M);   // DMAs of this call issued before its barrier
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks == 3) dma_barrier<kBefore>();
    const int fb = ks & 1, nb = fb ^ 1;
    if (MASKB) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        if (!((keep >> fn) & 1u)) b[fb][fn] = ELEM{};
    }
    const char* src = ks == 3 ? nxt : cur;
    const int nks = (ks + 1) & 3;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int fm = m / FN, fn = m % FN;
      acc[fm][fn] = mfma32<ELEM>(a[fb][fm], b[fb][fn], acc[fm][fn]);
      if (m < R)
        load_frag<ELEM, FM, FN>(a[nb], b[nb], src + arow0 * kLdsRow, src + kA + brow0 * kLdsRow, fl, nks, m);
#pragma unroll
      for (int q = share_lo(ND, 4 * M, ks * M + m); q < share_lo(ND, 4 * M, ks * M + m + 1); ++q) issue(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// K-major operand tile (R rows x 64 k) into the swizzled layout.  A wave
// instruction fills one 1 KB block = 8 LDS rows of 128 bytes; lane l covers
// LDS row 8*blk + l/8, physical chunk l%8, so it loads logical chunk
// (l%8) ^ swizzle(row) of that row: the swizzled layout comes out of the DMA
// as is.
template <int R, int NW = kThreads / 64>
struct DmaRows {
  static constexpr int kPerWave = R * kLdsRow / 1024 / NW;
  static_assert(kPerWave >= 1, "tile too small");
  // byte offset of this lane's 16 bytes for DMA instruction q, relative to
  // (row 0, k-tile start); rows past nrows (nrows >= 1) repeat row nrows-1:
  // such rows only meet outputs that are discarded or zero padding of the
  // other operand.
  __device__ __forceinline__ static uint32_t lane_off(int q, uint32_t ld2, int nrows, int lane, int wave) {
    const int blk = wave * kPerWave + q;
    const int lr = lane >> 3;
    const int row = min(8 * blk + lr, nrows - 1);
    return __umul24((uint32_t)row, ld2) + ((uint32_t)((lane & 7) ^ ((lr ^ blk) & 7)) << 4);
  }
};

// ---------------------------------------------------------------------------
// MN-major tiles (64 k-rows, each R consecutive m or n) through the DMA, read
// back with gfx950's transposing LDS read ds_read_b64_tr_b16.  Within each
// group of 16 lanes that instruction returns to lane i, slot r, element i%4
// of the 8 bytes addressed by lane 4r + i/4.  So if lane j of a group points
// at row k0 + j/4, columns m0 + 4(j%4) .. +3, lane i receives rows
// k0..k0+3 of column m0 + i: four consecutive k of one m, as an MFMA operand
// wants.  Two such reads give the 8 k values of a 32x32x16 operand.
// Layout: row k holds R elements (R/8 chunks of 16 bytes); logical chunk c
// sits at physical chunk c ^ 4(k & 3), so the 8 rows x 4 chunks that one
// transposing read touches fall on distinct bank groups twice at most.
// ---------------------------------------------------------------------------
template <int R, int NW = kThreads / 64, int KT = kKT>
struct MN {
  static_assert(R >= 128 && R % 128 == 0, "MN-major tiles need >= 128 columns");
  static_assert(KT == 32 || KT == 64, "32- or 64-deep k-tiles");
  static constexpr int kKTile = KT;
  static constexpr int kRowBytes = R * 2;
  static constexpr int kBytes = KT * kRowBytes;
  static constexpr int kPerWave = kBytes / 1024 / NW;
  __device__ __forceinline__ static int lds_pos(int k, int chunk) {
    return k * kRowBytes + ((chunk ^ ((k & 3) << 2)) << 4);
  }
  static constexpr int kRowsPerBlk = 1024 / kRowBytes;
  static constexpr int kLanesPerRow = kRowBytes / 16;
  // DMA state of one operand: base = element (k 0, mn 0) of this tile's
  // column block in a row-major [K, ld] matrix; off[q] = this lane's byte
  // offset for DMA instruction q within a k-tile.  Columns past nmn (nmn >= 8,
  // a multiple of 8) repeat the last 8-column group: every caller discards
  // such outputs.
  const uint16_t* base;
  uint32_t ld2;
  uint32_t off[kPerWave];
  __device__ __forceinline__ void init(const uint16_t* b, int ld, int nmn, int lane, int wave) {
    base = b;
    ld2 = 2u * (uint32_t)ld;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int blk = wave * kPerWave + q;
      const int kl = blk * kRowsPerBlk + lane / kLanesPerRow;
      const int c = (lane % kLanesPerRow) ^ ((kl & 3) << 2);
      off[q] = __umul24((uint32_t)kl, ld2) + 2u * (uint32_t)min(c * 8, nmn - 8);
    }
  }
  __device__ __forceinline__ void issue(int kt, uint32_t dst, int q, int wave) const {
    dma16(base + (int64_t)kt * KT * (ld2 >> 1), off[q], dst + (uint32_t)((wave * kPerWave + q) * 1024));
  }
  // Same, for a k-tile that runs past the kvalid valid k rows: rows past it
  // repeat row kvalid-1 (callers pair them with zero padding of the other
  // operand).
  __device__ __forceinline__ void issue_clamped(int kt, uint32_t dst, int q, int wave, int lane, int kvalid) const {
    const int blk = wave * kPerWave + q;
    const int kl = blk * kRowsPerBlk + lane / kLanesPerRow;
    const int row = min(kt * KT + kl, kvalid - 1) - kt * KT;
    const uint32_t voff = off[q] - __umul24((uint32_t)kl, ld2) + __umul24((uint32_t)row, ld2);
    dma16(base + (int64_t)kt * KT * (ld2 >> 1), voff, dst + (uint32_t)((wave * kPerWave + q) * 1024));
  }
  // MFMA operand for columns mn0 + 0..31 (lane%32), k = 16 ks + 8 (lane/32) .. +7
  template <typename ELEM>
  __device__ __forceinline__ static ELEM frag(const char* lds, int mn0, int ks, int lane) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const int j = lane & 15;
    const int m = mn0 + (((lane >> 4) & 1) << 4) + ((j & 3) << 2);
    const int k = 16 * ks + ((lane >> 5) << 3) + (j >> 2);
    const int chunk = m >> 3, within = (m & 7) * 2;
    const char* p0 = lds + lds_pos(k, chunk) + within;
    const char* p1 = lds + lds_pos(k + 4, chunk) + within;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)RKL_LDS_PTR(p0));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)RKL_LDS_PTR(p1));
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 v = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(ELEM, v);
  }
};

// K-major tiles for the generic GEMM: R rows x KT k.
//   KT = 64: rows of 128 bytes, chunk c of row r at c ^ ((r ^ r/8) % 8) (the
//            fused kernels' layout, lds_off);
//   KT = 32: rows of 64 bytes, chunk c of row r at c ^ (r/4 % 4): the 16 lanes
//            of a quarter of a ds_read_b128 (rows r0..r0+15, one chunk) then
//            cover all 64 banks once.  A DMA instruction fills 16 rows, lane l
//            row l/4, physical chunk l%4.
template <int R, int NW = kThreads / 64, int KT = kKT>
struct KM {
  static_assert(KT == 32 || KT == 64, "32- or 64-deep k-tiles");
  static constexpr int kKTile = KT;
  static constexpr int kRowB = KT * 2;
  static constexpr int kBytes = R * kRowB;
  static constexpr int kPerWave = kBytes / 1024 / NW;
  static_assert(kPerWave >= 1, "tile too small");
  // DMA state: base = element (row 0, k 0) of this tile's row block in a
  // row-major [rows, ld] matrix, nrows valid rows from there (rows past it
  // repeat row nrows-1: such rows only meet outputs that are discarded).
  const uint16_t* base;
  uint32_t off[kPerWave];
  __device__ __forceinline__ void init(const uint16_t* b, int ld, int nrows, int lane, int wave) {
    base = b;
    if constexpr (KT == 64) {
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) off[q] = DmaRows<R, NW>::lane_off(q, 2u * (uint32_t)ld, nrows, lane, wave);
    } else {
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) {
        const int row = min(16 * (wave * kPerWave + q) + (lane >> 2), nrows - 1);
        off[q] = __umul24((uint32_t)row, 2u * (uint32_t)ld) + ((uint32_t)((lane & 3) ^ ((row >> 2) & 3)) << 4);
      }
    }
  }
  __device__ __forceinline__ void issue(int kt, uint32_t dst, int q, int wave) const {
    dma16(base + kt * KT, off[q], dst + (uint32_t)((wave * kPerWave + q) * 1024));
  }
  template <typename ELEM>
  __device__ __forceinline__ static ELEM frag(const char* lds, int row0, int ks, int lane) {
    if constexpr (KT == 64) {
      return *reinterpret_cast<const ELEM*>(lds + lds_off(row0 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
      const int r = row0 + (lane & 31);
      return *reinterpret_cast<const ELEM*>(lds + r * 64 + (((ks * 2 + (lane >> 5)) ^ ((r >> 2) & 3)) << 4));
    }
  }
};

// bf16 fragment -> fp16 fragment (exact for values in fp16's normal range)
__device__ __forceinline__ f16x8 bf16_to_f16(bf16x8 x) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __builtin_bit_cast(float, u[e] << 16);
    const float hi = __builtin_bit_cast(float, u[e] & 0xFFFF0000u);
    o[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return __builtin_bit_cast(f16x8, o);
}

// ---------------------------------------------------------------------------
// Generic GEMM main loop, both operands through the DMA, NST LDS stages:
//   C[m, n] += sum_k A(m, k) B(n, k)   (fp32 accumulators)
// TA / TB are KM (K-major, swizzled rows) or MN (MN-major, read transposed)
// with the same k-tile depth KT = 16 KS.  Iteration kt: MFMAs of tile kt
// from stage kt % NST with the fragments one step ahead; the DMA of tile
// kt + NST - 1 into stage (kt - 1) % NST spread over steps 0 .. DSTEPS-1;
// before the last step a barrier that waits for tile kt + 1 (the NST - 2
// later tiles' DMA stays in flight), after which the last step reads the
// first fragments of tile kt + 1.  Stage (kt - 1) % NST was last read before
// the previous iteration's barrier, so a DMA never races a read.  Past the
// last tile the DMA repeats tile nk - 1 into stages that are no longer read.
// CVT_B converts B fragments from bf16 to fp16.
// ---------------------------------------------------------------------------
template <class TA, class TB, typename ELEM, bool CVT_B, int NST, bool RAGGED_B = false, int DSTEPS = 3, int FM,
          int FN>
__device__ __forceinline__ void gemm_loop(f32x16 (&acc)[FM][FN], int nk, char* lds, const TA& ta, const TB& tb,
                                          int kvalid_b, int tid, int arow0, int brow0) {
  static_assert(TA::kKTile == TB::kKTile, "both operands use one k-tile depth");
  constexpr int KS = TA::kKTile / 16;
  static_assert(NST >= 2 && NST <= 6, "two to six stages");
  static_assert((NST - 2) * (TA::kPerWave + TB::kPerWave) <= 63, "wait count fits vmcnt");
  static_assert(DSTEPS >= 1 && DSTEPS <= KS - 1, "the DMA is issued before the barrier of the last step");
  constexpr int kStage = TA::kBytes + TB::kBytes;
  constexpr int NA = TA::kPerWave, NB = TB::kPerWave, ND = NA + NB;
  constexpr int M = FM * FN, R = FM + FN;
  static_assert(R <= M, "fragment reads must fit the MFMA slots");
  using BRAW = typename std::conditional<CVT_B, bf16x8, ELEM>::type;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto fragA = [&](const char* st, int fm, int ks) { return TA::template frag<ELEM>(st, arow0 + fm * 32, ks, lane); };
  auto fragB = [&](const char* st, int fn, int ks) {
    const BRAW r = TB::template frag<BRAW>(st + TA::kBytes, brow0 + fn * 32, ks, lane);
    if constexpr (CVT_B) return bf16_to_f16(r);
    else return r;
  };
  const uint32_t lbase = lds_addr(lds);
  // RAGGED_B: B's last k-tile runs past its kvalid_b valid k rows (MN-major B)
  auto issue_tile = [&](int t, uint32_t st, int q) {
    if (q < NA) {
      ta.issue(t, st, q, wave);
    } else {
      if constexpr (RAGGED_B) {
        if (t == nk - 1) tb.issue_clamped(t, st + (uint32_t)TA::kBytes, q - NA, wave, lane, kvalid_b);
        else tb.issue(t, st + (uint32_t)TA::kBytes, q - NA, wave);
      } else {
        tb.issue(t, st + (uint32_t)TA::kBytes, q - NA, wave);
      }
    }
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
#pragma unroll
    for (int q = 0; q < ND; ++q) issue_tile(min(t, nk - 1), lbase + (uint32_t)(t * kStage), q);
  dma_barrier<(NST - 2) * ND>();
  ELEM a[2][FM], b[2][FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) b[0][fn] = fragB(lds, fn, 0);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) a[0][fm] = fragA(lds, fm, 0);
  int scur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int snxt = scur + 1 == NST ? 0 : scur + 1;
    const int spre = scur == 0 ? NST - 1 : scur - 1;   // (kt + NST - 1) % NST
    const char* cur = lds + scur * kStage;
    const char* nxt = lds + snxt * kStage;
    const uint32_t pre = lbase + (uint32_t)(spre * kStage);
    const int kn = min(kt + NST - 1, nk - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks == KS - 1) dma_barrier<(NST - 2) * ND>();
      const int fb = ks & 1, nb = fb ^ 1;
      const char* src = ks == KS - 1 ? nxt : cur;
      const int nks = ks == KS - 1 ? 0 : ks + 1;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int fm = m / FN, fn = m % FN;
        acc[fm][fn] = mfma32<ELEM>(a[fb][fm], b[fb][fn], acc[fm][fn]);
        if (m < FN) b[nb][m] = fragB(src, m, nks);
        else if (m < R) a[nb][m - FN] = fragA(src, m - FN, nks);
        if (ks < DSTEPS) {
#pragma unroll
          for (int q = share_lo(ND, DSTEPS * M, ks * M + m); q < share_lo(ND, DSTEPS * M, ks * M + m + 1); ++q)
            issue_tile(kn, pre, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    scur = snxt;
  }
  dma_barrier<0>();
}

// C-fragment coordinates of a 32x32 MFMA block: lane holds column (lane & 31)
// and rows 8*(i/4) + 4*(lane/32) + (i%4), i = 0..15.
__device__ __forceinline__ int frag_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Work-group order for the 8 XCDs of an MI355X: hardware hands consecutive
// workgroup ids to XCDs round robin; this maps them so that each XCD receives
// one contiguous range of logical tiles (tiles that share operands then share
// that XCD's L2).
__device__ __forceinline__ int xcd_logical(int lin, int total) {
  const int xcd = lin & 7, idx = lin >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Workgroup order for L2 reuse in the fused kernels.  Logical ids walk
// panels of GS vocabulary runs x all ntok token tiles; inside a panel,
// rectangles of GS runs x TG token tiles are consecutive, so the workgroups
// resident on one XCD at a time share both their weight k-slices (across
// token tiles) and their hidden-state k-slices (across vocabulary runs).
// A bijection of [0, nrun * ntok) for any GS, TG >= 1 (ragged last panel
// and last token group included).
__device__ __forceinline__ void panel_order(int logical, int nrun, int ntok, int GS, int TG, int& run, int& tt) {
  const int panel = logical / (GS * ntok);
  const int rem = logical - panel * GS * ntok;
  const int gs = min(GS, nrun - panel * GS);
  const int tg = rem / (gs * TG);
  const int r2 = rem - tg * gs * TG;
  run = panel * GS + r2 % gs;
  tt = tg * TG + r2 / gs;
}

}  // namespace rkl
