// rkl_tile.h -- bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup = 256 threads = 4 wave64s arranged 2 x 2.  A workgroup tile
// C[BM, BN] (fp32) is the product of two operand tiles that both arrive in
// LDS as "rows x 64 k" bf16 blocks:  C[m, n] = sum_k A[m, k] * B[n, k].
// Each wave owns a (BM/2) x (BN/2) sub-tile made of 32 x 32 blocks computed
// with v_mfma_f32_32x32x16_bf16.
//
// Operands may be K-major in memory (k contiguous: hidden states, LM-head
// weights, dz rows) or MN-major (m or n contiguous: the weight when the
// contraction runs over the vocabulary, dz when it runs over tokens).  The
// MN-major loader transposes 4 x 8 blocks in registers so that LDS always
// holds k-contiguous rows and every MFMA fragment is one 16-byte LDS read.
//
// LDS rows are 128 bytes (64 bf16).  The 16-byte chunk c of row r lives at
// chunk c ^ ((r ^ (r >> 3)) & 7): fragment reads by 8 consecutive lanes
// (8 consecutive rows, one chunk) and the transposing 8-byte writes both
// spread over all banks, and one direct-to-LDS wave instruction (8 rows of
// 128 bytes) reads 8 whole 128-byte row segments from global memory.
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

constexpr int kThreads = 256;
constexpr int kKT = 64;             // k extent of one staged tile
constexpr int kLdsRow = kKT * 2;    // bytes per LDS row

__device__ __forceinline__ int lds_off(int r, int chunk) {
  return r * kLdsRow + ((chunk ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// ---------------------------------------------------------------------------
// K-major operand: R rows (m or n), 64 consecutive k per row in memory.
// load_one(kt, i) / store_one(i) issue instruction i of k-tile kt, so the k
// loop can place each one between MFMAs.
// ---------------------------------------------------------------------------
template <int R>
struct KLoader {
  static constexpr int kPer = R * 8 / kThreads;
  static_assert(kPer >= 1 && (R * 8) % kThreads == 0, "tile too small");
  static constexpr int kVmem = kPer, kDsWrite = kPer;   // instructions per stage
  u32x4 v[kPer];
  const uint16_t* base;
  int64_t ld;
  int nrows;

  // src -> element (row 0, k 0) of the operand; rows >= nrows (nrows >= 1)
  // repeat row nrows-1: such rows only ever meet outputs that are discarded,
  // or zero padding of the other operand, so no branch or zero fill is needed.
  __device__ __forceinline__ void init(const uint16_t* src, int64_t ld_, int nrows_) {
    base = src; ld = ld_; nrows = nrows_;
  }
  __device__ __forceinline__ void load_one(int kt, int i, int tid) {
    const int c = tid + i * kThreads;
    const int r = min(c >> 3, nrows - 1), ch = c & 7;
    v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * ld + kt * kKT + ch * 8);
  }
  __device__ __forceinline__ void store_one(char* lds, int i, int tid) const {
    const int c = tid + i * kThreads;
    *reinterpret_cast<u32x4*>(lds + lds_off(c >> 3, c & 7)) = v[i];
  }
};

// ---------------------------------------------------------------------------
// MN-major operand: k-rows in memory, each holding consecutive m (or n).
// Thread work unit = 4 k x 8 mn; lanes 0-7 read one 128-byte row segment.
// ---------------------------------------------------------------------------
template <int R, bool TO_F16 = false>
struct MLoader {
  static constexpr int kBlocks = (kKT / 4) * (R / 8);
  static constexpr int kPer = kBlocks / kThreads;
  static_assert(kPer >= 1 && kBlocks % kThreads == 0, "tile too small");
  static constexpr int kVmem = 4 * kPer, kDsWrite = 8 * kPer;
  u32x4 v[kPer][4];
  const uint16_t* base;
  int64_t ld;
  int kvalid, nmn;

  __device__ __forceinline__ static void decode(int blk, int& bk, int& bm) {
    constexpr int MH = R / 64;
    const int rest = blk >> 4;
    bm = (blk & 7) + 8 * (rest % MH);
    bk = ((blk >> 3) & 1) + 2 * (rest / MH);
  }
  // src -> element (k 0, mn 0).  k rows >= kvalid and mn >= nmn (kvalid >= 1,
  // nmn >= 8, nmn % 8 == 0) repeat the last valid row / 8-column group: every
  // caller pairs such k rows with zero padding of the other operand and
  // discards such mn outputs.
  __device__ __forceinline__ void init(const uint16_t* src, int64_t ld_, int kvalid_, int nmn_) {
    base = src; ld = ld_; kvalid = kvalid_; nmn = nmn_;
  }
  __device__ __forceinline__ void load_one(int kt, int i, int tid) {
    const int blk = i >> 2, rr = i & 3;
    int bk, bm;
    decode(tid + blk * kThreads, bk, bm);
    const int col = min(8 * bm, nmn - 8);
    const int k = min(kt * kKT + 4 * bk + rr, kvalid - 1);
    v[blk][rr] = *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + col);
  }
  __device__ __forceinline__ void store_one(char* lds, int i, int tid) const {
    const int blk = i >> 3, j = i & 7;
    int bk, bm;
    decode(tid + blk * kThreads, bk, bm);
    const int r = 8 * bm + j;
    u32x2 out;
    if (TO_F16) {
      // bf16 -> fp32 is a shift; fp32 -> fp16 is exact for bf16 values in
      // fp16's normal range (only the rounding of tiny values depends on the
      // truncating pack)
      const int sh = (j & 1) ? 0 : 16;
      const uint32_t msk = (j & 1) ? 0xFFFF0000u : 0xFFFFFFFFu;
      const float f0 = __builtin_bit_cast(float, (v[blk][0][j >> 1] << sh) & msk);
      const float f1 = __builtin_bit_cast(float, (v[blk][1][j >> 1] << sh) & msk);
      const float f2 = __builtin_bit_cast(float, (v[blk][2][j >> 1] << sh) & msk);
      const float f3 = __builtin_bit_cast(float, (v[blk][3][j >> 1] << sh) & msk);
      out = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f2, f3))};
    } else {
      const int sh = (j & 1) * 16;
      const uint32_t e0 = (v[blk][0][j >> 1] >> sh) & 0xFFFFu;
      const uint32_t e1 = (v[blk][1][j >> 1] >> sh) & 0xFFFFu;
      const uint32_t e2 = (v[blk][2][j >> 1] >> sh) & 0xFFFFu;
      const uint32_t e3 = (v[blk][3][j >> 1] >> sh) & 0xFFFFu;
      out = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    }
    *reinterpret_cast<u32x2*>(lds + lds_off(r, bk >> 1) + (bk & 1) * 8) = out;
  }
};

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

// One MFMA fragment (B fragments first: the fm-major MFMA order needs every
// b before the second a).  f < FN: b[f]; else a[f - FN].
template <typename ELEM, int FM, int FN>
__device__ __forceinline__ void load_frag(ELEM (&a)[FM], ELEM (&b)[FN], const char* ldsA, const char* ldsB,
                                          int arow0, int brow0, int lane, int ks, int f) {
  const int chunk = ks * 2 + (lane >> 5);
  if (f < FN)
    b[f] = *reinterpret_cast<const ELEM*>(ldsB + lds_off(brow0 + f * 32 + (lane & 31), chunk));
  else
    a[f - FN] = *reinterpret_cast<const ELEM*>(ldsA + lds_off(arow0 + (f - FN) * 32 + (lane & 31), chunk));
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
  static constexpr int kBytes = 2 * kStage;
};

// Wait for this wave's LDS traffic, then the workgroup barrier.  Unlike
// __syncthreads() it does not drain outstanding global loads (the prefetch of
// the tile after next stays in flight); the memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

constexpr int share_lo(int total, int slots, int i) { return (total * i) / slots; }

// ---------------------------------------------------------------------------
// k loop over 64-deep tiles: two LDS stages, staging registers one tile
// ahead, fragment registers one 16-deep step ahead.  Iteration kt, in the
// order the instructions are issued (each MFMA followed by its extras; the
// order is pinned with scheduling barriers):
//   step 0: MFMAs of (kt, 0) | fragments (kt, 1) | LDS writes of tile kt+1
//   step 1: MFMAs of (kt, 1) | fragments (kt, 2) | global loads of tile kt+2
//   step 2: MFMAs of (kt, 2) | fragments (kt, 3)
//   barrier (LDS only)
//   step 3: MFMAs of (kt, 3) | fragments (kt+1, 0) from the other stage
// The barrier sits between steps 2 and 3: by then every wave has written
// stage (kt+1)&1 and read its last fragments of stage kt&1, so step 3 can
// already read tile kt+1 and iteration kt+1 can overwrite stage kt&1.  The
// 8 MFMAs of step 3 cover the latency of those reads.  Tiles past the end are
// clamped to the last one (never consumed), so the body is branch free.
// ---------------------------------------------------------------------------
template <int BM, int BN, typename ELEM = bf16x8, int FM, int FN, class LA, class LB>
__device__ __forceinline__ void kloop(f32x16 (&acc)[FM][FN], LA& la, LB& lb, int nk, char* lds, int tid,
                                      int arow0, int brow0) {
  using St = Stages<BM, BN>;
  static_assert(kKT / 16 == 4, "the schedule assumes 4 MFMA steps per tile");
  constexpr int M = FM * FN, R = FM + FN;
  constexpr int NW = LA::kDsWrite + LB::kDsWrite, NV = LA::kVmem + LB::kVmem;
  static_assert(R <= M, "fragment reads must fit the MFMA slots");
  const int lane = tid & 63;

#pragma unroll
  for (int i = 0; i < LA::kVmem; ++i) la.load_one(0, i, tid);
#pragma unroll
  for (int i = 0; i < LB::kVmem; ++i) lb.load_one(0, i, tid);
#pragma unroll
  for (int i = 0; i < LA::kDsWrite; ++i) la.store_one(lds, i, tid);
#pragma unroll
  for (int i = 0; i < LB::kDsWrite; ++i) lb.store_one(lds + St::kA, i, tid);
  {
    const int k1 = min(1, nk - 1);
#pragma unroll
    for (int i = 0; i < LA::kVmem; ++i) la.load_one(k1, i, tid);
#pragma unroll
    for (int i = 0; i < LB::kVmem; ++i) lb.load_one(k1, i, tid);
  }
  lds_barrier();
  ELEM a[2][FM], b[2][FN];
#pragma unroll
  for (int f = 0; f < R; ++f) load_frag<ELEM, FM, FN>(a[0], b[0], lds, lds + St::kA, arow0, brow0, lane, 0, f);

  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * St::kStage;
    char* nxt = lds + ((kt + 1) & 1) * St::kStage;
    const int kpre = min(kt + 2, nk - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks == 3) lds_barrier();
      const int fb = ks & 1, nb = fb ^ 1;
      const char* src = ks == 3 ? nxt : cur;
      const int nks = (ks + 1) & 3;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int fm = m / FN, fn = m % FN;
        acc[fm][fn] = mfma32<ELEM>(a[fb][fm], b[fb][fn], acc[fm][fn]);
        if (m < R) load_frag<ELEM, FM, FN>(a[nb], b[nb], src, src + St::kA, arow0, brow0, lane, nks, m);
        if (ks == 0) {
#pragma unroll
          for (int w = share_lo(NW, M, m); w < share_lo(NW, M, m + 1); ++w) {
            if (w < LA::kDsWrite) la.store_one(nxt, w, tid);
            else lb.store_one(nxt + St::kA, w - LA::kDsWrite, tid);
          }
        }
        if (ks == 1) {
#pragma unroll
          for (int q = share_lo(NV, M, m); q < share_lo(NV, M, m + 1); ++q) {
            if (q < LA::kVmem) la.load_one(kpre, q, tid);
            else lb.load_one(kpre, q - LA::kVmem, tid);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  lds_barrier();
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loads for K-major operands (gfx950 global_load_lds_dwordx4:
// each lane's 16 bytes land at the wave's LDS block + 16 * lane, no VGPRs).
// A wave instruction fills one 1 KB block = 8 LDS rows of 128 bytes; lane l
// covers LDS row 8*blk + l/8, physical chunk l%8, so it loads logical chunk
// (l%8) ^ swizzle(row) of that row: the swizzled layout comes out of the DMA
// as is.  Rows past nrows repeat row nrows-1 (see KLoader).
// ---------------------------------------------------------------------------
#define RKL_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

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
// (issue(q), q < ND, into stage `pre`) spread over step 0, and between steps
// 2 and 3 the barrier after which step 3 reads the first fragments of the
// next tile from stage `nxt`.
template <int BM, int BN, typename ELEM, int FM, int FN, int ND, class Issue>
__device__ __forceinline__ void dma_iter(f32x16 (&acc)[FM][FN], ELEM (&a)[2][FM], ELEM (&b)[2][FN], Issue issue,
                                         const char* __restrict__ cur, const char* __restrict__ nxt, int lane,
                                         int arow0, int brow0) {
  constexpr int M = FM * FN, R = FM + FN;
  constexpr int kA = BM * kLdsRow;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks == 3) dma_barrier<ND>();
    const int fb = ks & 1, nb = fb ^ 1;
    const char* src = ks == 3 ? nxt : cur;
    const int nks = (ks + 1) & 3;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int fm = m / FN, fn = m % FN;
      acc[fm][fn] = mfma32<ELEM>(a[fb][fm], b[fb][fn], acc[fm][fn]);
      if (m < R) load_frag<ELEM, FM, FN>(a[nb], b[nb], src, src + kA, arow0, brow0, lane, nks, m);
      if (ks == 0) {
#pragma unroll
        for (int q = share_lo(ND, M, m); q < share_lo(ND, M, m + 1); ++q) issue(q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// DMA of one K-major operand tile (R rows x 64 k) into the swizzled layout;
// per-lane addresses are computed at issue time.
template <int R>
struct DmaRows {
  static constexpr int kPerWave = R * kLdsRow / 1024 / (kThreads / 64);
  static_assert(kPerWave >= 1, "tile too small");
  __device__ __forceinline__ static void issue(const uint16_t* base, int64_t ld, int nrows, int kt, char* dst, int i,
                                               int lane, int wave) {
    const int blk = wave * kPerWave + i;
    const int row = 8 * blk + (lane >> 3);
    const int chunk = (lane & 7) ^ (((lane >> 3) ^ blk) & 7);
    const uint32_t off = (uint32_t)(((int64_t)min(row, nrows - 1) * ld + chunk * 8) * 2);
    // base, kt and dst are wave-uniform: keep them in SGPRs
    const uint64_t gp = (uint64_t)(uintptr_t)(base + kt * kKT);
    // (readfirstlane returns int: go through uint32_t so nothing is sign-extended)
    const uint32_t g_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(gp >> 32));
    const uint32_t g_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gp);
    const uint64_t g = ((uint64_t)g_hi << 32) | (uint64_t)g_lo;
    const uint32_t lds =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)RKL_LDS_PTR(dst + blk * 1024));
    // M0 is only ever written right before the instruction that reads it on
    // gfx9+, so setting it here does not disturb compiler-generated code.
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(g), "s"(lds)
                 : "memory", "m0");
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
template <int R>
struct MN {
  static_assert(R >= 128 && R % 128 == 0, "MN-major tiles need >= 128 columns");
  static constexpr int kRowBytes = R * 2;
  static constexpr int kBytes = kKT * kRowBytes;
  static constexpr int kPerWave = kBytes / 1024 / (kThreads / 64);
  __device__ __forceinline__ static int off(int k, int chunk) {
    return k * kRowBytes + ((chunk ^ ((k & 3) << 2)) << 4);
  }
  // DMA instruction i of k-tile kt: 1 KB block blk covers rows (blk*1024)/rowbytes ..
  __device__ __forceinline__ static void issue(const uint16_t* base, int64_t ld, int kvalid, int nmn, int kt,
                                               char* dst, int i, int lane, int wave) {
    constexpr int kLanesPerRow = kRowBytes / 16;   // chunks per row
    const int blk = wave * kPerWave + i;
    const int byte = blk * 1024 + lane * 16;
    const int k = byte / kRowBytes;
    const int pc = (byte % kRowBytes) >> 4;
    const int c = pc ^ ((k & 3) << 2);
    (void)kLanesPerRow;
    const int row = min(kt * kKT + k, kvalid - 1);
    const int col = min(c * 8, nmn - 8);
    const uint32_t goff = (uint32_t)(((int64_t)row * ld + col) * 2);
    const uint64_t gp = (uint64_t)(uintptr_t)base;
    const uint32_t g_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(gp >> 32));
    const uint32_t g_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gp);
    const uint64_t g = ((uint64_t)g_hi << 32) | (uint64_t)g_lo;
    const uint32_t lds =
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)RKL_LDS_PTR(dst + blk * 1024));
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(goff), "s"(g), "s"(lds)
                 : "memory", "m0");
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
    const char* p0 = lds + off(k, chunk) + within;
    const char* p1 = lds + off(k + 4, chunk) + within;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)RKL_LDS_PTR(p0));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)RKL_LDS_PTR(p1));
    typedef short s8 __attribute__((ext_vector_type(8)));
    const s8 v = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(ELEM, v);
  }
};

// K-major tiles (R rows x 64 k, swizzled rows of 128 bytes) for the generic GEMM.
template <int R>
struct KM {
  static constexpr int kBytes = R * kLdsRow;
  static constexpr int kPerWave = DmaRows<R>::kPerWave;
  __device__ __forceinline__ static void issue(const uint16_t* base, int64_t ld, int nrows, int kt, char* dst, int i,
                                               int lane, int wave) {
    DmaRows<R>::issue(base, ld, nrows, kt, dst, i, lane, wave);
  }
  template <typename ELEM>
  __device__ __forceinline__ static ELEM frag(const char* lds, int row0, int ks, int lane) {
    return *reinterpret_cast<const ELEM*>(lds + lds_off(row0 + (lane & 31), ks * 2 + (lane >> 5)));
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
// TA / TB are KM<rows> (K-major, swizzled rows) or MN<cols> (MN-major, read
// transposed).  Iteration kt: MFMAs of tile kt from stage kt % NST with the
// fragments one step ahead; the DMA of tile kt + NST - 1 into stage
// (kt - 1) % NST during step 0; between steps 2 and 3 a barrier that waits
// for tile kt + 1 (the DMA groups of the later tiles stay in flight), after
// which step 3 reads the first fragments of tile kt + 1.  Stage (kt - 1) %
// NST was last read before the previous iteration's barrier, so a DMA never
// races a read.  Past the last tile the DMA repeats tile nk - 1 into stages
// that are no longer read.  CVT_B converts B fragments from bf16 to fp16.
// ---------------------------------------------------------------------------
template <class TA, class TB, typename ELEM, bool CVT_B, int NST, int FM, int FN, class IssueA, class IssueB>
__device__ __forceinline__ void gemm_loop(f32x16 (&acc)[FM][FN], int nk, char* lds, IssueA issueA, IssueB issueB,
                                          int tid, int arow0, int brow0) {
  static_assert(NST == 2 || NST == 3, "two or three stages");
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
  auto issue_tile = [&](int t, char* st, int q) {
    if (q < NA) issueA(t, st, q, lane, wave);
    else issueB(t, st + TA::kBytes, q - NA, lane, wave);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
#pragma unroll
    for (int q = 0; q < ND; ++q) issue_tile(min(t, nk - 1), lds + t * kStage, q);
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
    char* pre = lds + spre * kStage;
    const int kn = min(kt + NST - 1, nk - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks == 3) dma_barrier<(NST - 2) * ND>();
      const int fb = ks & 1, nb = fb ^ 1;
      const char* src = ks == 3 ? nxt : cur;
      const int nks = (ks + 1) & 3;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int fm = m / FN, fn = m % FN;
        acc[fm][fn] = mfma32<ELEM>(a[fb][fm], b[fb][fn], acc[fm][fn]);
        if (m < FN) b[nb][m] = fragB(src, m, nks);
        else if (m < R) a[nb][m - FN] = fragA(src, m - FN, nks);
        if (ks == 0) {
#pragma unroll
          for (int q = share_lo(ND, M, m); q < share_lo(ND, M, m + 1); ++q) issue_tile(kn, pre, q);
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
