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
// spread over all banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// ---------------------------------------------------------------------------
template <int R>
struct KLoader {
  static constexpr int kPer = R * 8 / kThreads;
  static_assert(kPer >= 1 && (R * 8) % kThreads == 0, "tile too small");
  u32x4 v[kPer];

  // src -> element (row 0, k0) of the tile; rows >= nrows read as zero.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3, ch = c & 7;
      if (r < nrows)
        v[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * ld + ch * 8);
      else
        v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(lds + lds_off(c >> 3, c & 7)) = v[i];
    }
  }
};

// ---------------------------------------------------------------------------
// MN-major operand: 64 k-rows in memory, each holding R consecutive m (or n).
// Thread work unit = 4 k x 8 mn; lanes 0-7 read one 128-byte row segment.
// ---------------------------------------------------------------------------
template <int R, bool TO_F16 = false>
struct MLoader {
  static constexpr int kBlocks = (kKT / 4) * (R / 8);
  static constexpr int kPer = kBlocks / kThreads;
  static_assert(kPer >= 1 && kBlocks % kThreads == 0, "tile too small");
  u32x4 v[kPer][4];

  __device__ __forceinline__ static void decode(int blk, int& bk, int& bm) {
    constexpr int MH = R / 64;
    const int rest = blk >> 4;
    bm = (blk & 7) + 8 * (rest % MH);
    bk = ((blk >> 3) & 1) + 2 * (rest / MH);
  }
  // src -> element (k0, mn0); k rows >= nk and mn >= nmn (nmn % 8 == 0) read as zero.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int nk, int nmn, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int bk, bm;
      decode(tid + i * kThreads, bk, bm);
      const bool mn_ok = 8 * bm < nmn;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int k = 4 * bk + rr;
        if (mn_ok && k < nk)
          v[i][rr] = *reinterpret_cast<const u32x4*>(src + (int64_t)k * ld + 8 * bm);
        else
          v[i][rr] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int bk, bm;
      decode(tid + i * kThreads, bk, bm);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * bm + j;
        u32x2 out;
        if (TO_F16) {
          // bf16 -> fp32 is a shift; fp32 -> fp16 is exact for bf16 values in
          // fp16's normal range (only the rounding of tiny values depends on
          // the truncating pack)
          const int sh = (j & 1) ? 0 : 16;
          const uint32_t msk = (j & 1) ? 0xFFFF0000u : 0xFFFFFFFFu;
          const float f0 = __builtin_bit_cast(float, (v[i][0][j >> 1] << sh) & msk);
          const float f1 = __builtin_bit_cast(float, (v[i][1][j >> 1] << sh) & msk);
          const float f2 = __builtin_bit_cast(float, (v[i][2][j >> 1] << sh) & msk);
          const float f3 = __builtin_bit_cast(float, (v[i][3][j >> 1] << sh) & msk);
          out = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f2, f3))};
        } else {
          const int sh = (j & 1) * 16;
          const uint32_t e0 = (v[i][0][j >> 1] >> sh) & 0xFFFFu;
          const uint32_t e1 = (v[i][1][j >> 1] >> sh) & 0xFFFFu;
          const uint32_t e2 = (v[i][2][j >> 1] >> sh) & 0xFFFFu;
          const uint32_t e3 = (v[i][3][j >> 1] >> sh) & 0xFFFFu;
          out = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
        }
        *reinterpret_cast<u32x2*>(lds + lds_off(r, bk >> 1) + (bk & 1) * 8) = out;
      }
    }
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

template <typename ELEM, int FM, int FN>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[FM][FN], const char* ldsA, const char* ldsB,
                                          int arow0, int brow0, int lane) {
#pragma unroll
  for (int ks = 0; ks < kKT / 16; ++ks) {
    const int chunk = ks * 2 + (lane >> 5);
    ELEM a[FM], b[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      a[fm] = *reinterpret_cast<const ELEM*>(ldsA + lds_off(arow0 + fm * 32 + (lane & 31), chunk));
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      b[fn] = *reinterpret_cast<const ELEM*>(ldsB + lds_off(brow0 + fn * 32 + (lane & 31), chunk));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = mfma32<ELEM>(a[fm], b[fn], acc[fm][fn]);
  }
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

// ---------------------------------------------------------------------------
// Double-buffered k loop.  fetch(kt) issues the global loads of k-tile kt into
// the loaders' registers; the loaders then write LDS stage (kt & 1).  One
// barrier per k-tile: stage kt+1 is written only after every wave has left
// stage kt-1 (the barrier at the end of iteration kt-1).
//   lds layout: [stage 0: A (BM rows), B (BN rows)] [stage 1: A, B]
// Leaves LDS free to reuse (ends with a barrier).
// ---------------------------------------------------------------------------
template <int BM, int BN>
struct Stages {
  static constexpr int kA = BM * kLdsRow;
  static constexpr int kB = BN * kLdsRow;
  static constexpr int kStage = kA + kB;
  static constexpr int kBytes = 2 * kStage;
};

template <int BM, int BN, typename ELEM = bf16x8, int FM, int FN, class LA, class LB, class Fetch>
__device__ __forceinline__ void kloop(f32x16 (&acc)[FM][FN], LA& la, LB& lb, Fetch fetch, int nk, char* lds,
                                      int tid, int arow0, int brow0) {
  using St = Stages<BM, BN>;
  const int lane = tid & 63;
  fetch(0);
  la.store(lds, tid);
  lb.store(lds + St::kA, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * St::kStage;
    char* nxt = lds + ((kt + 1) & 1) * St::kStage;
    const bool more = kt + 1 < nk;
    if (more) fetch(kt + 1);
    mma_stage<ELEM, FM, FN>(acc, cur, cur + St::kA, arow0, brow0, lane);
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + St::kA, tid);
    }
    __syncthreads();
  }
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

}  // namespace rkl
