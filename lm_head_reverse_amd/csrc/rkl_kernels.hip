// rkl_kernels.hip -- HIP kernels for gfx950 of the fused LM-head projection +
// full-vocabulary reverse KL (forward, backward) and loss-mask compaction.
//
// Method (NeMo-RL pull request "add full-vocabulary on-policy distillation to
// SingleController"): summary -- L = sum_v p_s (log p_s - log p_t) per token;
// implementation notes -- dL/dz_s = p_s (w - L), w = log p_s - log p_t, with
// the log-softmaxes recomputed in the backward.  Compaction (slime pull
// request "compact actor logits before projection", summary): only the
// loss-masked rows are projected and scalars are scattered back.
//
// Orientation: every projection tile is computed as C[v, t] = W[v, :] . h[t, :]
// (vocabulary along MFMA rows, tokens along MFMA columns).  In the 32x32 MFMA
// output layout one lane then holds one token and 16 vocabulary entries per
// block, so the online log-sum-exp / KL statistics of a token live in that
// lane's registers for the whole sweep of a vocabulary split; lanes l and
// l^32 (the two row halves) merge when the split ends, then the waves that
// share tokens merge through LDS.
#include "rkl_tile.h"
#include "rkl_internal.h"

#include <hip/hip_ext.h>

#include <tuple>
#include <type_traits>

namespace rkl {

constexpr float kL2E = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // "no value seen yet" running max; exp2 of it underflows to 0

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge of two partial (max, sum of exp(z - max), sum of exp(z - max) * d) triples.
// The sums are written as explicit fmas: left to the compiler, s f1 + s2 f2
// may be contracted one way for the student's sum and the other way for the
// teacher's, and identical logits would then no longer give bit-identical
// log-normalisers (nor a loss of exactly zero).
__device__ __forceinline__ void merge3(float& m, float& s, float& a, float m2, float s2, float a2) {
  const float M = fmaxf(m, m2);
  const float f1 = ex2((m - M) * kL2E), f2 = ex2((m2 - M) * kL2E);
  s = fmaf(s, f1, s2 * f2);
  a = fmaf(a, f1, a2 * f2);
  m = M;
}
__device__ __forceinline__ void merge2(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float f1 = ex2((m - M) * kL2E), f2 = ex2((m2 - M) * kL2E);
  s = fmaf(s, f1, s2 * f2);
  m = M;
}

// ===========================================================================
// Fused forward: per (run of vocabulary splits, token tile) workgroup, sweep
// the splits' vocabulary tiles; for each tile form z_s (and z_t) in registers
// with MFMA and fold them into per-lane online statistics, written out per
// split
//   m_s, S_s = sum e^{z_s - m_s}, A = sum e^{z_s - m_s} (z_s - z_t), m_t, S_t.
// Nothing of size [N, V] is written.
// ===========================================================================
constexpr int FBM = 256;   // vocabulary rows per tile
constexpr int FBN = 128;   // tokens per tile
using FwdStages = Stages<FBM, FBN>;

// Wave layout of the fused kernels: NW waves as NW/2 rows (vocabulary) x 2
// columns (tokens) over the 256 x 128 tile; each wave holds FM x FN 32x32
// blocks of z_s and of z_t.  Built with eight waves (kFusedWaves) for the two
// projections: 64 x 64 per wave, 128 accumulator registers, two waves per
// SIMD (one can issue MFMAs while the other waits on LDS or the DMA); four
// waves at 128 x 64 would read a quarter fewer fragments per MFMA but need
// 256 accumulator registers per wave, which spill.  With one projection the
// four-wave layout holds 128 and is built (kFusedWavesOne) for the
// log-probability / entropy forward (-0.6 %) and the top-k estimator's dz
// (-2.5 %); the log-probability / entropy dz (its entropy term needs a few
// registers more) spills with four and keeps eight.
template <int NW>
struct Fused {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kWM = NW / 2;
  static constexpr int FM = FBM / kWM / 32, FN = FBN / 2 / 32;
  static constexpr int kA = DmaRows<FBM, NW>::kPerWave, kB = DmaRows<FBN, NW>::kPerWave, ND = kA + kB;
  static constexpr int kRedFloats = (kWM - 1) * 2 * FN * 32 * 5;
};

// Fold one tile's values of token column fn into the running statistics, one
// 32x32 block (16 values per side) at a time: block max, rescale of the
// running sums, then the block's exponentials.  Student and teacher go
// through the same operations, so identical logits give identical
// statistics (and A = 0 exactly).
template <bool TAIL, int FM, int FN>
__device__ __forceinline__ void fold_tile(const f32x16 (&zs)[FM][FN], const f32x16 (&zt)[FM][FN], int fn,
                                          int vrow, int V, float& ms, float& ss, float& aa, float& mt, float& st) {
  // vrow = vocabulary index of fragment row 0 for this lane (block fm = 0)
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    float tms = kNegBig, tmt = kNegBig;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !TAIL || (vrow + fm * 32 + 8 * (i >> 2) + (i & 3) < V);
      if (ok) {
        tms = fmaxf(tms, zs[fm][fn][i]);
        tmt = fmaxf(tmt, zt[fm][fn][i]);
      }
    }
    const float nms = fmaxf(ms, tms), nmt = fmaxf(mt, tmt);
    const float fs = ex2((ms - nms) * kL2E), ft = ex2((mt - nmt) * kL2E);
    const float cs = nms * kL2E, ct = nmt * kL2E;
    float ps0 = 0.f, ps1 = 0.f, pt0 = 0.f, pt1 = 0.f, pa0 = 0.f, pa1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !TAIL || (vrow + fm * 32 + 8 * (i >> 2) + (i & 3) < V);
      if (ok) {
        const float x = zs[fm][fn][i], y = zt[fm][fn][i];
        const float es = ex2(fmaf(x, kL2E, -cs));
        const float et = ex2(fmaf(y, kL2E, -ct));
        if (i & 1) {
          ps1 += es; pt1 += et; pa1 = fmaf(es, x - y, pa1);
        } else {
          ps0 += es; pt0 += et; pa0 = fmaf(es, x - y, pa0);
        }
      }
    }
    ss = fmaf(ss, fs, ps0 + ps1);
    aa = fmaf(aa, fs, pa0 + pa1);
    st = fmaf(st, ft, pt0 + pt1);
    ms = nms;
    mt = nmt;
    // one block at a time: keeps the accumulator reads of later blocks from
    // being hoisted (which would need more registers than the wave has)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Log-probability / entropy fold of one tile's token column fn: running
// m, S = sum e^{z - m}, B = sum e^{z - m} z (B rescales like S), and zy = the
// logit of the row's sampled token yv when this lane holds it (kNegBig
// otherwise, so a max merges it).  lse = m + log S, the entropy is
// lse - B / S and log p(y) = zy - lse (slime page, summary: log-probability
// and entropy of the compacted rows).
template <bool TAIL, int FM, int FN>
__device__ __forceinline__ void fold_lpe(const f32x16 (&zs)[FM][FN], int fn, int vrow, int V, int yv, float& ms,
                                         float& ss, float& bb, float& zy) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    float tms = kNegBig;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = !TAIL || (vrow + fm * 32 + 8 * (i >> 2) + (i & 3) < V);
      if (ok) tms = fmaxf(tms, zs[fm][fn][i]);
    }
    const float nms = fmaxf(ms, tms);
    const float fs = ex2((ms - nms) * kL2E);
    const float cs = nms * kL2E;
    float ps0 = 0.f, ps1 = 0.f, pb0 = 0.f, pb1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = vrow + fm * 32 + 8 * (i >> 2) + (i & 3);
      const bool ok = !TAIL || v < V;
      if (ok) {
        const float x = zs[fm][fn][i];
        const float es = ex2(fmaf(x, kL2E, -cs));
        if (i & 1) {
          ps1 += es; pb1 = fmaf(es, x, pb1);
        } else {
          ps0 += es; pb0 = fmaf(es, x, pb0);
        }
        if (v == yv) zy = x;
      }
    }
    ss = fmaf(ss, fs, ps0 + ps1);
    bb = fmaf(bb, fs, pb0 + pb1);
    ms = nms;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The z_t row of each of this lane's token columns: token n reads row
// z_rows[n] (row n without an index), clamped to [0, nrows); token columns
// past N read the row of token N-1 (their results are discarded).
template <int FN>
__device__ __forceinline__ void zt_rows(const int32_t* __restrict__ z_rows, int nrows, int N, int ncol,
                                        int (&zr)[FN]) {
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int n = min(ncol + fn * 32, N - 1);
    zr[fn] = z_rows ? min(max(z_rows[n], 0), nrows - 1) : n;
  }
}

// Teacher logits read into the accumulator layout (teacher-logits payload).
// zr[fn] = the z_t row of this lane's token column fn (zt_rows).  A full
// vocabulary tile (TAIL false) loads without conditions, from one row
// pointer per token column and immediate offsets; the last tile clamps each
// column index to V-1 and zeroes what lies past V.
// only >= 0 loads token column `only` alone.
template <bool VEC4, bool TAIL, int FM, int FN>
__device__ __forceinline__ void load_zt(f32x16 (&zt)[FM][FN], const float* __restrict__ z_t, int V, int vrow,
                                        const int (&zr)[FN], int only = -1) {
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    if (only >= 0 && fn != only) continue;
    const float* row = z_t + (int64_t)zr[fn] * V;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v = vrow + fm * 32 + 8 * g;
        if (VEC4) {
          // V % 4 == 0: a group of four is wholly inside or wholly past V
          float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
          if (!TAIL || v < V) q = *reinterpret_cast<const float4*>(row + v);
          zt[fm][fn][4 * g + 0] = q.x; zt[fm][fn][4 * g + 1] = q.y;
          zt[fm][fn][4 * g + 2] = q.z; zt[fm][fn][4 * g + 3] = q.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (TAIL) {
              const float x = row[min(v + e, V - 1)];
              zt[fm][fn][4 * g + e] = v + e < V ? x : 0.f;
            } else {
              zt[fm][fn][4 * g + e] = row[v + e];
            }
          }
          // the tail's clamped addresses four at a time (all at once would
          // hold 64 addresses in registers)
          if (TAIL) __builtin_amdgcn_sched_barrier(0);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Dual-projection stream.  A workgroup owns one 128-token tile and a run of
// 256-row vocabulary tiles ("jobs").  For each job it computes z_s (Hs/64
// k-tiles) and, with a hidden-state teacher, z_t (Ht/64 k-tiles), then calls
// the epilogue.  All k-tiles of all jobs form one stream through a 3-stage
// LDS ring fed by DMA two k-tiles ahead, so neither the switch between the
// projections nor the next job restarts the pipeline, and an epilogue
// overlaps the loads of the next job's first tiles.
// ---------------------------------------------------------------------------
// Bit 31 of a tile's teacher set: some row of the tile names no valid teacher.
constexpr uint32_t kTeacherOutOfRange = 1u << 31;

struct DualOps {
  const uint16_t* W[2];
  const uint16_t* h[2];
  int H[2];
  int nk[2];        // k-tiles per projection; nk[1] = 0 when the teacher is given as logits
  int V, N, n0, v0;  // v0: first row of job 0
  // Teacher passes of every job: one per set bit k of tset, projecting with
  // the weight at W[1] + k * wt_stride (one teacher: tset = 1, stride 0).
  uint32_t tset;
  int64_t wt_stride;
};

struct StreamPos {
  int job, phase, kt, tk;   // tk: teacher of a teacher pass (phase 1)
};

template <bool MULTI>
__device__ __forceinline__ void stream_advance(StreamPos& q, const DualOps& o) {
  if (++q.kt == (q.phase ? o.nk[1] : o.nk[0])) {
    q.kt = 0;
    if (!MULTI) {
      if (q.phase == 0 && o.nk[1] > 0) {
        q.phase = 1;
      } else {
        q.phase = 0;
        ++q.job;
      }
      return;
    }
    // the next teacher pass of this job: the next teacher bit of tset
    const uint32_t ts = o.tset & ~kTeacherOutOfRange;
    const uint32_t rest = q.phase == 0 ? ts : (ts & ~((2u << q.tk) - 1u));
    if (o.nk[1] > 0 && rest != 0) {
      q.phase = 1;
      q.tk = __builtin_ctz(rest);
    } else {
      q.phase = 0;
      ++q.job;
    }
  }
}

// No per-k-tile work besides the MFMAs.
struct NoTileHook {
  __device__ __forceinline__ void operator()(const char*, int, int) const {}
};

// epi(job, stage) runs after each job's last k-tile; `stage` is an LDS stage
// it may use as scratch (it must end with a workgroup barrier if it does,
// since the next k-tile's DMA writes it).
// hook(stage, job, kt) runs after each student k-tile: `stage` still holds
// that tile, and every wave has passed the barrier after which the tile is
// complete.  The next k-tile's DMA writes `stage`, so a hook that reads it
// must end with a workgroup barrier whenever it reads.
// tkl[fn] = teacher of this lane's token column fn (read only when tset has
// several bits: a teacher pass then zeroes, in every B fragment, the token
// columns of the other teachers, so each column accumulates exactly its own
// teacher's products -- the sum is the same as in a pass over that teacher
// alone, bit for bit).
template <int NW, bool MULTI = false, class Epi, class Hook = NoTileHook>
__device__ __forceinline__ void dual_stream(const DualOps& o, int njobs, char* lds,
                                            f32x16 (&zs)[Fused<NW>::FM][Fused<NW>::FN],
                                            f32x16 (&zt)[Fused<NW>::FM][Fused<NW>::FN], int tid, int arow0, int brow0,
                                            const int (&tkl)[Fused<NW>::FN], Epi epi, Hook hook = Hook{}) {
  using F = Fused<NW>;
  constexpr int FFM = F::FM, FFN = F::FN, kStreamA = F::kA, kStreamB = F::kB, kStreamND = F::ND;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // MULTI = false: one teacher (o.tset and o.wt_stride unused)
  const uint32_t tset = o.tset & ~kTeacherOutOfRange;
  const int passes = o.nk[1] > 0 ? (MULTI ? __builtin_popcount(tset) : 1) : 0;
  const bool mixed = MULTI && (passes > 1 || (o.tset & kTeacherOutOfRange) != 0);
  const int total = njobs * (o.nk[0] + passes * o.nk[1]);
  const uint32_t lbase = lds_addr(lds);
  // stage rotation as byte offsets: reads use lds + offset, the DMA lbase + offset
  int ocur = 0, onxt = FwdStages::kStage, opre = 2 * FwdStages::kStage;
  StreamPos dp{0, 0, 0, 0};
  int dissued = 0;
  // Per-lane DMA offsets of the current stream segment (one job's student or
  // teacher k-tiles), relative to the segment's tile base at k-tile 0, with
  // the ragged-tail clamp folded in (rows past the end repeat the last row).
  // They only change when the stream enters a new segment, so each DMA is
  // an SGPR base plus a table entry.
  uint32_t offA[kStreamA], offB[kStreamB];
  const uint16_t* segA = o.W[0];
  const uint16_t* segB = o.h[0];
  auto seg_setup = [&]() {
    const bool t = dp.phase != 0;
    const int ld = t ? o.H[1] : o.H[0];
    const int v0 = o.v0 + dp.job * FBM;
    segA = (t ? o.W[1] + (MULTI ? (int64_t)dp.tk * o.wt_stride : 0) : o.W[0]) + (int64_t)v0 * ld;
    segB = (t ? o.h[1] : o.h[0]) + (int64_t)o.n0 * ld;
    const int nA = o.V - v0, nB = o.N - o.n0;
    const uint32_t ld2 = 2u * (uint32_t)ld;
#pragma unroll
    for (int q = 0; q < kStreamA; ++q) offA[q] = DmaRows<FBM, NW>::lane_off(q, ld2, nA, lane, wave);
#pragma unroll
    for (int q = 0; q < kStreamB; ++q) offB[q] = DmaRows<FBN, NW>::lane_off(q, ld2, nB, lane, wave);
  };
  seg_setup();
  // DMA instruction q of stream position dp into the stage at LDS address dst;
  // past the end it repeats the last position (loads that are never consumed)
  auto dma_all = [&](uint32_t dst, int q) {
    if (q < kStreamA)
      dma16(segA + dp.kt * kKT, offA[q], dst + (uint32_t)((wave * kStreamA + q) * 1024));
    else
      dma16(segB + dp.kt * kKT, offB[q - kStreamA],
            dst + (uint32_t)(FwdStages::kA + (wave * kStreamB + q - kStreamA) * 1024));
  };
  auto dma_next = [&]() {
    if (dissued + 1 < total) {
      stream_advance<MULTI>(dp, o);
      if (dp.kt == 0) seg_setup();
    }
    ++dissued;
  };
#pragma unroll
  for (int q = 0; q < kStreamND; ++q) dma_all(lbase + (uint32_t)ocur, q);
  dma_next();
#pragma unroll
  for (int q = 0; q < kStreamND; ++q) dma_all(lbase + (uint32_t)onxt, q);
  dma_next();
  dma_barrier<kStreamND>();
  FragLanes fl;
  fl.init(lane);
  bf16x8 a[2][FFM], b[2][FFN];
#pragma unroll
  for (int f = 0; f < FFM + FFN; ++f)
    load_frag<bf16x8, FFM, FFN>(a[0], b[0], lds + arow0 * kLdsRow, lds + FwdStages::kA + brow0 * kLdsRow, fl, 0, f);

  auto step = [&](f32x16 (&acc)[FFM][FFN], auto maskb, uint32_t keep) {
    const uint32_t target = lbase + (uint32_t)opre;
    dma_iter<FBM, FBN, bf16x8, FFM, FFN, kStreamND, decltype(maskb)::value>(
        acc, a, b, [&](int q) { dma_all(target, q); }, lds + ocur, lds + onxt, fl, arow0, brow0, keep);
    dma_next();
    const int t = ocur;
    ocur = onxt;
    onxt = opre;
    opre = t;
  };
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  for (int job = 0; job < njobs; ++job) {
    zero_acc(zs);
    for (int kt = 0; kt < o.nk[0]; ++kt) {
      const char* consumed = lds + ocur;
      step(zs, Plain{}, 0u);
      hook(consumed, job, kt);
    }
    // per-row teachers: a tile whose rows all have ids outside [0, K) runs no
    // teacher pass, and its teacher logits are the zeros set here
    if (MULTI || passes > 0) {
      zero_acc(zt);
      if (!MULTI) {
        for (int kt = 0; kt < o.nk[1]; ++kt) step(zt, Plain{}, 0u);
      } else {
        for (uint32_t rest = tset; rest != 0; rest &= rest - 1) {
          const int k = __builtin_ctz(rest);
          uint32_t keep = ~0u;   // bit fn: token column fn belongs to teacher k
          if (mixed) {
#pragma unroll
            for (int fn = 0; fn < FFN; ++fn) keep &= ~((uint32_t)(tkl[fn] != k) << fn);
          }
          for (int kt = 0; kt < o.nk[1]; ++kt) step(zt, Masked{}, keep);
        }
      }
    }
    // the stage just consumed is free until the next k-tile's DMA
    epi(job, lds + opre);
  }
  dma_barrier<0>();
}

// Teachers of a 128-token tile (reverse KL with a teacher chosen per row):
// tkl[fn] = teacher of this lane's token column fn (-1 past N), and the
// returned bitmask holds every teacher id in [0, K) (K <= 31) of the tile's
// rows, plus bit 31 when one of its rows has an id outside [0, K).  Such a
// row selects no teacher: every pass over its tile is masked and leaves its
// teacher logits at 0 (no memory is addressed with the id).  Without per-row
// teachers (teacher NULL): one teacher, bitmask 1.  Every thread of the
// workgroup must call it.
template <int FN>
__device__ __forceinline__ uint32_t tile_teachers(const int32_t* __restrict__ teacher, int K, int N, int n0, int brow0,
                                                  int lane, int (&tkl)[FN], uint32_t* tset_lds) {
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) tkl[fn] = 0;
  if (!teacher) return 1u;
  uint32_t bits = 0;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int n = n0 + brow0 + fn * 32 + (lane & 31);
    tkl[fn] = n < N ? teacher[n] : -1;
    if (tkl[fn] >= 0 && tkl[fn] < K)
      bits |= 1u << tkl[fn];
    else if (n < N)
      bits |= kTeacherOutOfRange;
  }
  if (threadIdx.x == 0) *tset_lds = 0u;
  __syncthreads();
  if (bits) atomicOr(tset_lds, bits);
  __syncthreads();
  return *tset_lds;
}

// MODE 0: hidden teacher; 1: teacher logits; 2: log-probability / entropy
// (one projection; the statistics slots hold m, S, B, zy, 0); 3: hidden
// teacher chosen per row (as 0, with one teacher pass per teacher present in
// the token tile).
template <int MODE, bool VEC4, int NW>
__global__ __launch_bounds__(Fused<NW>::kThreads, 1) void fwd_tiles(FwdParams p) {
  using F = Fused<NW>;
  constexpr int FFM = F::FM, FFN = F::FN;
  __shared__ __attribute__((aligned(1024))) char lds[3 * FwdStages::kStage];
  __shared__ __attribute__((aligned(16))) float red[F::kRedFloats];
  __shared__ uint32_t tset_lds;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  // a workgroup takes splits [split0, split1) of token tile tt: their
  // vocabulary tiles form one stream, and each split's statistics are
  // written when its last tile is folded (the split plan, and so every
  // result bit, does not depend on how splits are grouped)
  const int ngroup = (p.nsplit + p.splits_per_wg - 1) / p.splits_per_wg;
  const int logical = xcd_logical(blockIdx.x, ngroup * p.ntok);
  int grp, tt;
  panel_order(logical, ngroup, p.ntok, p.order_gs, p.order_tg, grp, tt);
  const int n0 = tt * FBN;
  const int ntv = (p.V + FBM - 1) / FBM;
  const int split0 = grp * p.splits_per_wg;
  const int vt0 = split0 * p.tiles_per_split;
  const int vt1 = min(min(split0 + p.splits_per_wg, p.nsplit) * p.tiles_per_split, ntv);

  const int arow0 = wm * (FBM / F::kWM), brow0 = wn * (FBN / 2);
  float ms[FFN], ss[FFN], aa[FFN], mt[FFN], st[FFN];
  auto reset = [&]() {
#pragma unroll
    for (int fn = 0; fn < FFN; ++fn) { ms[fn] = kNegBig; ss[fn] = 0.f; aa[fn] = 0.f; mt[fn] = kNegBig; st[fn] = 0.f; }
  };
  reset();

  // One split's statistics: merge the two row halves of each 32x32 block
  // (lanes l and l^32), then the waves that hold the same tokens (wm = 1 ..
  // kWM-1 into wm = 0, in that order, through LDS), and write the partial.
  // Every thread calls it; the barriers wait for LDS only, so the DMA of the
  // next tiles stays in flight.
  auto flush = [&](int split) {
#pragma unroll
    for (int fn = 0; fn < FFN; ++fn) {
      const float oms = __shfl_xor(ms[fn], 32), oss = __shfl_xor(ss[fn], 32), oaa = __shfl_xor(aa[fn], 32);
      const float omt = __shfl_xor(mt[fn], 32), ost = __shfl_xor(st[fn], 32);
      merge3(ms[fn], ss[fn], aa[fn], oms, oss, oaa);
      merge2(mt[fn], st[fn], omt, ost);
    }
    if (wm > 0 && lane < 32) {
#pragma unroll
      for (int fn = 0; fn < FFN; ++fn) {
        float* q = red + ((((wm - 1) * 2 + wn) * FFN + fn) * 32 + lane) * 5;
        q[0] = ms[fn]; q[1] = ss[fn]; q[2] = aa[fn]; q[3] = mt[fn]; q[4] = st[fn];
      }
    }
    dma_barrier<63>();
    if (wm == 0 && lane < 32) {
#pragma unroll
      for (int fn = 0; fn < FFN; ++fn) {
#pragma unroll
        for (int r = 1; r < F::kWM; ++r) {
          const float* q = red + ((((r - 1) * 2 + wn) * FFN + fn) * 32 + lane) * 5;
          merge3(ms[fn], ss[fn], aa[fn], q[0], q[1], q[2]);
          merge2(mt[fn], st[fn], q[3], q[4]);
        }
        const int n = n0 + brow0 + fn * 32 + lane;
        if (n < p.N) {
          float* P = p.partial + (int64_t)split * 5 * p.N + n;
          P[0] = ms[fn];
          P[(int64_t)1 * p.N] = ss[fn];
          P[(int64_t)2 * p.N] = aa[fn];
          P[(int64_t)3 * p.N] = mt[fn];
          P[(int64_t)4 * p.N] = st[fn];
        }
      }
    }
    // red is written again by the next split's flush
    dma_barrier<63>();
    reset();
  };

  f32x16 zs[FFM][FFN], zt[FFM][FFN];
  const int lrow = 4 * (lane >> 5);
  DualOps o;
  o.W[0] = p.W_s; o.h[0] = p.h_s; o.H[0] = p.Hs; o.nk[0] = p.Hs / kKT;
  o.W[1] = p.W_t; o.h[1] = p.h_t; o.H[1] = p.Ht; o.nk[1] = (MODE == 0 || MODE == 3) ? p.Ht / kKT : 0;
  o.V = p.V; o.N = p.N; o.n0 = n0; o.v0 = vt0 * FBM;
  int tkl[FFN];
  o.tset = tile_teachers<FFN>(MODE == 3 ? p.teacher : nullptr, p.K, p.N, n0, brow0, lane, tkl, &tset_lds);
  o.wt_stride = p.wt_stride;
  int yv[FFN];   // sampled token of this lane's token columns (MODE 2)
#pragma unroll
  for (int fn = 0; fn < FFN; ++fn) {
    const int n = n0 + brow0 + fn * 32 + (lane & 31);
    yv[fn] = (MODE == 2 && n < p.N) ? p.y[n] : -1;
  }
  int zr[FFN];   // z_t row of this lane's token columns (MODE 1)
  if (MODE == 1) zt_rows<FFN>(p.z_rows, p.z_nrows, p.N, n0 + brow0 + (lane & 31), zr);

  dual_stream<NW, MODE == 3>(o, vt1 - vt0, lds, zs, zt, tid, arow0, brow0, tkl, [&](int job, char*) {
    const int v0 = (vt0 + job) * FBM;
    const int vrow = v0 + arow0 + lrow;
    if (v0 + FBM <= p.V) {
      // teacher logits: the next token column's loads are in flight while
      // this one folds (with V % 4 != 0 all at once: the unaligned rows need
      // more registers)
      if (MODE == 1) load_zt<VEC4, false>(zt, p.z_t, p.V, vrow, zr, VEC4 ? 0 : -1);
#pragma unroll
      for (int fn = 0; fn < FFN; ++fn) {
        if (MODE == 1 && VEC4 && fn + 1 < FFN)
          load_zt<VEC4, false>(zt, p.z_t, p.V, vrow, zr, fn + 1);
        if (MODE == 2)
          fold_lpe<false>(zs, fn, vrow, p.V, yv[fn], ms[fn], ss[fn], aa[fn], mt[fn]);
        else
          fold_tile<false>(zs, zt, fn, vrow, p.V, ms[fn], ss[fn], aa[fn], mt[fn], st[fn]);
      }
    } else {
      // the last vocabulary tile: teacher logits one token column at a time
      // (its clamped loads need an address per entry)
#pragma unroll
      for (int fn = 0; fn < FFN; ++fn) {
        if (MODE == 1) load_zt<VEC4, true>(zt, p.z_t, p.V, vrow, zr, fn);
        if (MODE == 2)
          fold_lpe<true>(zs, fn, vrow, p.V, yv[fn], ms[fn], ss[fn], aa[fn], mt[fn]);
        else
          fold_tile<true>(zs, zt, fn, vrow, p.V, ms[fn], ss[fn], aa[fn], mt[fn], st[fn]);
      }
    }
    // the split's last tile (or the vocabulary's): its statistics are complete
    const int vt = vt0 + job;
    if ((vt + 1) % p.tiles_per_split == 0 || vt + 1 == vt1) flush(vt / p.tiles_per_split);
  });
}

// Split combine.  Reverse KL: lse = m + log S per side, L = A / S_s -
// (lse_s - lse_t), stats (lse_s, lse_t, L, log p_max).  Log-probability /
// entropy (LPE): lse = m + log S, H = lse - B / S, log p(y) = zy - lse, stats
// (lse, H, log p(y), log p_max).  32 rows per workgroup; the 8 thread groups
// each merge every 8th split (coalesced over rows), then group 0 merges the 8
// results in a fixed order, so the result depends on V (the split plan) only,
// never on N.  KIND 0: reverse KL; 1: LPE; 2: no finalisation -- the merged
// (m_s, S_s, A, m_t, S_t) of all splits go to out0 as five planes of N (one
// vocabulary shard's contribution, to be merged with the other shards').
constexpr int kCombRows = 32, kCombWays = 8;
enum CombineKind : int { kCombineKL = 0, kCombineLPE = 1, kCombineMerged = 2 };

template <int KIND>
__global__ __launch_bounds__(256) void fwd_combine(const float* __restrict__ partial, int nsplit, int N,
                                                   const uint8_t* __restrict__ row_mask, float* __restrict__ out0,
                                                   float* __restrict__ out1, float* __restrict__ stats) {
  __shared__ float red[kCombWays][5][kCombRows];
  const int r = threadIdx.x % kCombRows, j = threadIdx.x / kCombRows;
  const int n = blockIdx.x * kCombRows + r;
  float ms = kNegBig, ss = 0.f, aa = 0.f, mt = kNegBig, st = 0.f;
  if (n < N) {
    for (int s = j; s < nsplit; s += kCombWays) {
      const float* P = partial + (int64_t)s * 5 * N + n;
      merge3(ms, ss, aa, P[0], P[(int64_t)N], P[(int64_t)2 * N]);
      merge2(mt, st, P[(int64_t)3 * N], P[(int64_t)4 * N]);
    }
  }
  red[j][0][r] = ms; red[j][1][r] = ss; red[j][2][r] = aa; red[j][3][r] = mt; red[j][4][r] = st;
  __syncthreads();
  if (j != 0 || n >= N) return;
#pragma unroll
  for (int q = 1; q < kCombWays; ++q) {
    merge3(ms, ss, aa, red[q][0][r], red[q][1][r], red[q][2][r]);
    merge2(mt, st, red[q][3][r], red[q][4][r]);
  }
  if (KIND == kCombineMerged) {
    out0[n] = ms;
    out0[(int64_t)N + n] = ss;
    out0[(int64_t)2 * N + n] = aa;
    out0[(int64_t)3 * N + n] = mt;
    out0[(int64_t)4 * N + n] = st;
    return;
  }
  const float log_ss = logf(ss);
  const bool dead = row_mask && row_mask[n] == 0;
  float lse_s = ms + log_ss;
  float lpmax = -log_ss;   // log of the largest student probability
  if (KIND == kCombineLPE) {
    float H = lse_s - aa / ss;
    float lpy = mt - lse_s;
    if (dead) { lse_s = 0.f; H = 0.f; lpy = 0.f; lpmax = 0.f; }
    out0[n] = lpy;
    if (out1) out1[n] = H;
    stats[4 * (int64_t)n + 0] = lse_s;
    stats[4 * (int64_t)n + 1] = H;
    stats[4 * (int64_t)n + 2] = lpy;
    stats[4 * (int64_t)n + 3] = lpmax;
  } else {
    float lse_t = mt + logf(st);
    float L = aa / ss - (lse_s - lse_t);
    if (dead) { L = 0.f; lse_s = 0.f; lse_t = 0.f; lpmax = 0.f; }
    out0[n] = L;
    stats[4 * (int64_t)n + 0] = lse_s;
    stats[4 * (int64_t)n + 1] = lse_t;
    stats[4 * (int64_t)n + 2] = L;
    stats[4 * (int64_t)n + 3] = lpmax;
  }
}

// ===========================================================================
// Backward, step 0: dz scale.  dz = g p_s (w - L) is stored as fp16(s * dz)
// (11-bit significand; bf16's 8 bits alone can use up the gradient tolerance
// when one vocabulary entry dominates a row).  s is the power of two that
// puts the largest g * p_s over live rows -- |g| exp(lpmax), lpmax = log of
// a row's largest student probability, from the forward -- in [16, 32): the
// bulk of dz then sits in fp16's normal range, and |w - L| up to ~2000 still
// fits below fp16's maximum (larger values saturate).  dh and dW are
// multiplied by 1/s (exact).
// Log-probability / entropy: |dz_v| <= 2 |g_lp| + |g_H| (p_v |log p_v| +
// p_v H) <= 2 |g_lp| + |g_H| (1 + H), so that bound takes the place of
// g * p_max: s * dz stays below 32.
// ===========================================================================
template <int MODE>
__global__ __launch_bounds__(1024) void grad_scale(const float* __restrict__ grad, const float* __restrict__ grad_h,
                                                   const uint8_t* __restrict__ row_mask,
                                                   const float* __restrict__ stats, int N, int nchunks,
                                                   uint32_t* __restrict__ scales) {
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  float m = 0.f;
  for (int n = tid; n < N; n += 1024) {
    const bool live = !row_mask || row_mask[n] != 0;
    if (!live) continue;
    const float g = grad ? fabsf(grad[n]) : 1.0f;
    if (MODE == kModeLogprobEntropy) {
      const float gh = grad_h ? fabsf(grad_h[n]) : 0.0f;
      m = fmaxf(m, 2.0f * g + gh * (1.0f + fabsf(stats[4 * (int64_t)n + 1])));
    } else if (MODE == kModeTopK) {
      m = fmaxf(m, g * stats[4 * (int64_t)n + 3]);   // the row's bound on |dz| / |g|
    } else {
      m = fmaxf(m, g * expf(stats[4 * (int64_t)n + 3]));
    }
  }
  red[tid] = m;
  // the magnitude records the later kernels take atomic maxima into
  if (tid == 0) scales[kScaleHmag] = 0u;
  for (int c = tid; c < nchunks; c += 1024) scales[kScaleWmag + c] = 0u;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  if (tid == 0) {
    int e = 0;
    if (red[0] > 0.f) frexpf(red[0], &e);     // max in [2^(e-1), 2^e)
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    scales[kScaleS] = __builtin_bit_cast(uint32_t, ldexpf(1.0f, 5 - e));
    scales[kScaleKs] = (uint32_t)(5 - e);
  }
}

// e with |x| in [2^(e-1), 2^e) for the bf16 magnitude bits m (bits & 0x7fff)
// of a nonzero finite value.
__device__ __forceinline__ int bf16_mag_exp(uint32_t m) {
  const int E = (int)(m >> 7);
  if (E > 0) return E - 126;
  return (32 - __clz((int)(m & 0x7fu))) - 133;   // subnormal: 0.f x 2^-126
}
__device__ __forceinline__ int clamp_shift(int k) { return k < -kMaxExpShift ? -kMaxExpShift : (k > kMaxExpShift ? kMaxExpShift : k); }
// 2^kh for h16: the largest |h_s| into [2^14, 2^15).
__device__ __forceinline__ int h_scale_exp(uint32_t m) { return m ? clamp_shift(15 - bf16_mag_exp(m)) : 0; }
// 2^kw for the W_s copy: 1 while the largest |W_s| is in [2^-10, 2^15) (no
// overflow, and everything within 2^-4 of fp16's normal range at the top),
// else as for h16.
__device__ __forceinline__ int w_scale_exp(uint32_t m) {
  if (m == 0) return 0;
  const int e = bf16_mag_exp(m);
  return (e >= -9 && e <= 15) ? 0 : clamp_shift(15 - e);
}
// Largest bf16 magnitude among the 8 values of a 16-byte piece.
__device__ __forceinline__ uint32_t bf16x8_absmax(u32x4 x) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max(x[e] & 0x7fffu, (x[e] >> 16) & 0x7fffu));
  return m;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  return m;
}

// scales[kScaleHmag] = largest bf16 magnitude among n values (n % 8 == 0 not
// required; 16-byte pieces, then a tail).
__global__ __launch_bounds__(256) void absmax_bf16(const uint16_t* __restrict__ h, int64_t n,
                                                   uint32_t* __restrict__ scales) {
  uint32_t m = 0;
  const int64_t n8 = n / 8;
  const u32x4* h8 = reinterpret_cast<const u32x4*>(h);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256)
    m = max(m, bf16x8_absmax(h8[i]));
  for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = max(m, (uint32_t)h[i] & 0x7fffu);
  // one atomic per workgroup (atomics on one address serialise in L2)
  __shared__ uint32_t wmax[4];
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (m) atomicMax(scales + kScaleHmag, m);
  }
}

// s * dz of this lane's accumulator elements, rounded to fp16 and packed in
// pairs.  Lane l (l < 32) holds rows {0-3, 8-11, 16-19, 24-27} of each 32-row
// block, lane l + 32 rows {4-7, 12-15, 20-23, 28-31}, same token; one
// permlane32 swap per dword leaves lane l with rows 0-7 and 16-23, lane l + 32
// with rows 8-15 and 24-31: runs of 8 consecutive vocabulary entries,
// pk[fm][fn][run] = 4 dwords.  The arithmetic is branch-free: entries past V
// (TAIL, the last vocabulary tile only) and dead token columns become zero by
// selection, so a dead row stays exactly zero whatever its logits are.
// vrow = vocabulary index of this lane's row 0 in block fm = 0; elem(z_s,
// z_t, fn, v) gives s * dz of one entry (v = its vocabulary index).
// col(fn) runs before token column fn is packed (the teacher-logits payload
// loads the next column's logits there).
struct NoColHook {
  __device__ __forceinline__ void operator()(int) const {}
};

template <bool TAIL, int FM, int FN, class Elem, class Col = NoColHook>
__device__ __forceinline__ void dz_pack(const f32x16 (&zs)[FM][FN], const f32x16 (&zt)[FM][FN],
                                        uint32_t (&pk)[FM][FN][2][4], const bool (&live)[FN], int vrow, int V,
                                        Elem elem, Col col = Col{}) {
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    col(fn);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      uint32_t w[4][2];   // [gq][dword]
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = zs[fm][fn][4 * gq + e];
          const float bb = zt[fm][fn][4 * gq + e];
          // (the tail copy reads its input through an empty asm so that the
          // compiler cannot merge the two copies' arithmetic above the branch
          // that selects them -- that computes every entry at once and spills)
          if (TAIL) asm volatile("" : "+v"(a));
          const int v = vrow + fm * 32 + 8 * gq + e;
          float d = elem(a, bb, fn, v);
          d = __builtin_amdgcn_fmed3f(d, -65504.f, 65504.f);
          if (TAIL) d = v < V ? d : 0.f;
          dv[e] = d;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // both halves rounded to nearest in one packed conversion
          const uint32_t x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{dv[2 * h], dv[2 * h + 1]}, f16x2));
          w[gq][h] = live[fn] ? x : 0u;
        }
        // four entries at a time: keeps the register peak down
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const auto r = __builtin_amdgcn_permlane32_swap(w[2 * pr][d], w[2 * pr + 1][d], false, false);
          w[2 * pr][d] = r[0];
          w[2 * pr + 1][d] = r[1];
        }
        pk[fm][fn][pr][0] = w[2 * pr][0];
        pk[fm][fn][pr][1] = w[2 * pr][1];
        pk[fm][fn][pr][2] = w[2 * pr + 1][0];
        pk[fm][fn][pr][3] = w[2 * pr + 1][1];
      }
    }
  }
}

// ===========================================================================
// Backward, step 1: recompute z_s, z_t for one (vocabulary tile, token tile)
// of the current chunk and write s * dz, dz = g p_s ((z_s - z_t) - (lse_s -
// lse_t + L)), rounded to fp16 into the chunk workspace dz[N, ldz]
// (column = v - c0).  Columns in [width, kpad) are written as zero; rows with
// row_mask 0 are zero.  MODE 2 recomputes the one projection and writes the
// log-probability / entropy gradient instead (see the per-token constants).
// ===========================================================================
template <int MODE, bool VEC4, int NW, bool LATE = false>
__global__ __launch_bounds__(Fused<NW>::kThreads, 1) void bwd_dz_tiles(BwdParams p) {
  using F = Fused<NW>;
  constexpr int FFM = F::FM, FFN = F::FN;
  __shared__ __attribute__((aligned(1024))) char lds[3 * FwdStages::kStage];
  __shared__ uint32_t tset_lds;
  __shared__ uint32_t wmag_lds[F::kThreads / 64];   // per wave: largest |W_s| bits it converted
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int logical = xcd_logical(blockIdx.x, p.ngroups * p.ntok);
  int grp, tt;
  panel_order(logical, p.ngroups, p.ntok, p.order_gs, p.order_tg, grp, tt);
  const int vt0 = grp * p.tiles_per_group;
  const int vt1 = min(vt0 + p.tiles_per_group, p.ntv);
  const int n0 = tt * FBN;
  const int arow0 = wm * (FBM / F::kWM), brow0 = wn * (FBN / 2);
  const int lrow = 4 * (lane >> 5);

  // per-token constants of this lane's token columns.  Reverse KL:
  //   s dz = gs p ((z_s - z_t) - cst),  gs = s g, cst = lse_s - lse_t + L;
  // log-probability / entropy (MODE 2), lp = z - lse:
  //   s dz = gs (1[v = y] - p) - ge p (lp + H) = -p (ge z + cst) + 1[v = y] gs,
  //   gs = s g_lp, ge = s g_H, cst = gs + ge (H - lse);
  // top-k estimator (MODE 4): the same form with ge = 0, cst = s g c and the
  // spike gs = s g sp from the forward's stats (lse, c, sp, bound).
  // css = lse_s log2(e): p = 2^(z log2(e) - css).
  bool live[FFN];
  float gs[FFN], ge[FFN], cst[FFN], css[FFN];
  int yv[FFN];
#pragma unroll
  for (int fn = 0; fn < FFN; ++fn) {
    const int n = n0 + brow0 + fn * 32 + (lane & 31);
    live[fn] = n < p.N && (!p.row_mask || p.row_mask[n] != 0);
    const int nc = min(n, p.N - 1);
    const float lse_s = p.stats[4 * (int64_t)nc + 0];
    gs[fn] = (p.grad ? p.grad[nc] : 1.0f) * __builtin_bit_cast(float, p.scales[kScaleS]);
    css[fn] = lse_s * kL2E;
    if (MODE == 2) {
      const float H = p.stats[4 * (int64_t)nc + 1];
      ge[fn] = (p.grad_h ? p.grad_h[nc] : 0.0f) * __builtin_bit_cast(float, p.scales[kScaleS]);
      cst[fn] = gs[fn] + ge[fn] * (H - lse_s);
      yv[fn] = p.y[nc];
    } else if (MODE == 4) {
      // top-k estimator, the dense part and the tail's spike (the support's
      // own terms are added by topk_dz_add): s dz = -p (gs c) + 1[v = y] gs sp
      cst[fn] = gs[fn] * p.stats[4 * (int64_t)nc + 1];
      gs[fn] *= p.stats[4 * (int64_t)nc + 2];
      ge[fn] = 0.f;
      yv[fn] = p.y[nc];
    } else {
      const float lse_t = p.stats[4 * (int64_t)nc + 1];
      const float L = p.stats[4 * (int64_t)nc + 2];
      cst[fn] = (lse_s - lse_t) + L;
      ge[fn] = 0.f;
      yv[fn] = -1;
    }
  }

  int zr[FFN];   // z_t row of this lane's token columns (MODE 1)
  if (MODE == 1) zt_rows<FFN>(p.z_rows, p.z_nrows, p.N, n0 + brow0 + (lane & 31), zr);

  f32x16 zs[FFM][FFN], zt[FFM][FFN];
  DualOps o;
  o.W[0] = p.W_s; o.h[0] = p.h_s; o.H[0] = p.Hs; o.nk[0] = p.Hs / kKT;
  o.W[1] = p.W_t; o.h[1] = p.h_t; o.H[1] = p.Ht; o.nk[1] = (MODE == 0 || MODE == 3) ? p.Ht / kKT : 0;
  o.V = p.V; o.N = p.N; o.n0 = n0; o.v0 = p.c0 + vt0 * FBM;
  int tkl[FFN];
  o.tset = tile_teachers<FFN>(MODE == 3 ? p.teacher : nullptr, p.K, p.N, n0, brow0, lane, tkl, &tset_lds);
  o.wt_stride = p.wt_stride;

  // fp16 copy of this workgroup's share of the W_s chunk for the dh GEMM:
  // of each vocabulary tile's Hs/64 student k-tiles, token tile tt converts
  // those with kt = tt (mod ntok), so every (tile, k-tile) is written once.
  // Rows past V hold the clamped copies of row V-1 the DMA brought in.  The
  // copy is unscaled; the largest magnitude converted goes to the chunk's
  // record, from which w_rescale decides whether the copy must be made again
  // with a scale: each wave keeps its running maximum in LDS, and the
  // workgroup takes one atomic maximum at its end (atomics on one address
  // serialise in L2: one per wave and conversion -- eight per job at 512
  // rows -- capped the kernel near 1.9 ms whatever N).
  //
  // When the workgroup converts at most one k-tile and runs one job (late_w16),
  // it converts it after the stream instead: the k-tile's W_s rows are loaded
  // again into the free LDS ring while the dz math runs, and the copy's stores
  // go out with the dz stores.  Mid-stream, the next k-step's barrier waits
  // for the copy's stores (a store and the DMA count in the one vector-memory
  // counter), about 3 us per workgroup; at the end their wait overlaps the dz
  // stores'.  The same bits either way.
  if (lane == 0) wmag_lds[w] = 0u;
  auto convert_rows = [&](const char* stage, int job, int kt) {
    // thread tid converts rows r = i * kThreads / 8 + tid / 8, 16-byte piece
    // tid % 8: a wave-uniform base plus a 32-bit lane offset
    const int c = tid & 7;
    const uint32_t loff = (uint32_t)(tid >> 3) * (uint32_t)p.Hs + (uint32_t)(c * 8);
    uint32_t mag = 0;
#pragma unroll
    for (int i = 0; i < FBM * 8 / F::kThreads; ++i) {
      const int r = i * (F::kThreads / 8) + (tid >> 3);
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + lds_off(r, c));
      mag = max(mag, bf16x8_absmax(x));
      uint16_t* rb = p.w16 + ((int64_t)(vt0 + job) * FBM + i * (F::kThreads / 8)) * p.Hs + kt * kKT;
      *reinterpret_cast<f16x8*>(rb + loff) = bf16_to_f16(__builtin_bit_cast(bf16x8, x));
    }
    mag = wave_max_u32(mag);
    if (lane == 0) wmag_lds[w] = max(wmag_lds[w], mag);   // this wave's slot only
  };
  constexpr bool late = LATE;
  auto convert_w = [&](const char* stage, int job, int kt) {
    if (late || kt % p.ntok != tt % p.ntok) return;
    convert_rows(stage, job, kt);
    // the next k-tile's DMA writes this stage: every wave's reads first
    // (the condition above is the same for the whole workgroup)
    dma_barrier<63>();
  };

  dual_stream<NW, MODE == 3>(o, vt1 - vt0, lds, zs, zt, tid, arow0, brow0, tkl, [&](int job, char* stage) {
    const int v0 = p.c0 + (vt0 + job) * FBM;
    const int hi = lane >> 5;
    const bool last = vt0 + job + 1 == vt1;
    // the late copy's k-tile and where it lands: after the dz tile's 64 KB
    const int kt_late = tt % p.ntok;
    const bool conv_late = late && last && kt_late < p.Hs / kKT;
    constexpr int kLateOff = FBN * FBM * 2;
    static_assert(kLateOff + FBM * kLdsRow <= 3 * FwdStages::kStage, "the late copy fits beside the dz tile");
    if (conv_late) {
      dma_barrier<0>();   // the stream's trailing DMAs landed: the whole ring is free
      const int wave = __builtin_amdgcn_readfirstlane(w);
      const uint16_t* src = p.W_s + (int64_t)v0 * p.Hs + kt_late * kKT;
      const uint32_t dst = lds_addr(lds) + (uint32_t)kLateOff;
#pragma unroll
      for (int q = 0; q < F::kA; ++q) {
        dma16(src, DmaRows<FBM, NW>::lane_off(q, 2u * (uint32_t)p.Hs, p.V - v0, lane, wave),
              dst + (uint32_t)((wave * F::kA + q) * 1024));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    uint32_t pk[FFM][FFN][2][4];   // [fm][fn][run][dword]
    auto kl = [&](float a, float bb, int fn, int) {
      return gs[fn] * ex2(fmaf(a, kL2E, -css[fn])) * ((a - bb) - cst[fn]);
    };
    auto lpe = [&](float a, float, int fn, int v) {
      const float d = -ex2(fmaf(a, kL2E, -css[fn])) * fmaf(ge[fn], a, cst[fn]);
      return v == yv[fn] ? d + gs[fn] : d;
    };
    if (MODE == 2 || MODE == 4) {
      // (one projection: lpe ignores its second operand, so z_s stands in for it)
      if (v0 + FBM <= p.V)
        dz_pack<false>(zs, zs, pk, live, v0 + arow0 + lrow, p.V, lpe);
      else
        dz_pack<true>(zs, zs, pk, live, v0 + arow0 + lrow, p.V, lpe);
    } else if (MODE != 1) {
      if (v0 + FBM <= p.V)
        dz_pack<false>(zs, zt, pk, live, v0 + arow0 + lrow, p.V, kl);
      else
        dz_pack<true>(zs, zt, pk, live, v0 + arow0 + lrow, p.V, kl);
    } else {
      // teacher logits, one token column at a time: the next column's loads
      // are in flight while this one is packed
      const int vr = v0 + arow0 + lrow;
      if (v0 + FBM <= p.V) {
        load_zt<VEC4, false>(zt, p.z_t, p.V, vr, zr, 0);
        dz_pack<false>(zs, zt, pk, live, vr, p.V, kl, [&](int fn) {
          if (fn + 1 < FFN) load_zt<VEC4, false>(zt, p.z_t, p.V, vr, zr, fn + 1);
        });
      } else {
        dz_pack<true>(zs, zt, pk, live, vr, p.V, kl,
                      [&](int fn) { load_zt<VEC4, true>(zt, p.z_t, p.V, vr, zr, fn); });
      }
    }
    // Stores go through LDS: the waves holding a round's tokens write a
    // [tokens][256 vocabulary] fp16 tile (16-byte chunk c of row t at chunk
    // c ^ (t % 32), so neither side has bank conflicts), then every thread
    // stores 16-byte pieces of whole rows: 512 contiguous bytes per token
    // row instead of 32 rows per store instruction.  Mid-stream only the
    // free stage (48 KB) can hold the tile: two rounds of 64 tokens.  After
    // the stream's last k-tile every stage is free once its DMAs have
    // landed: one round of all 128 tokens, every wave writing at once.
    auto store = [&](char* buf, auto rounds) {
      constexpr int NR = decltype(rounds)::value, TPR = FBN / NR;
#pragma unroll
      for (int round = 0; round < NR; ++round) {
        if (NR == 1 || wn == round) {
#pragma unroll
          for (int fn = 0; fn < FFN; ++fn) {
            const int tl = (NR == 1 ? brow0 : 0) + fn * 32 + (lane & 31);   // token within the round
#pragma unroll
            for (int fm = 0; fm < FFM; ++fm)
#pragma unroll
              for (int pr = 0; pr < 2; ++pr) {
                const int c = (arow0 + fm * 32 + 16 * pr + 8 * hi) >> 3;
                *reinterpret_cast<u32x4*>(buf + tl * 512 + ((c ^ (tl & 31)) << 4)) =
                    u32x4{pk[fm][fn][pr][0], pk[fm][fn][pr][1], pk[fm][fn][pr][2], pk[fm][fn][pr][3]};
              }
          }
        }
        // (the late copy's rows must have landed as well)
        if (conv_late)
          dma_barrier<0>();
        else
          dma_barrier<63>();
        // thread tid stores token row tr = it * kThreads / 32 + tid / 32 of
        // the round, columns col .. col + 7: a wave-uniform row base plus a
        // 32-bit lane offset (tid / 32) * ldz + (tid % 32) * 8 (no 64-bit
        // per-lane addresses live across the main loop)
        const int c = tid & 31;
        const int col = v0 - p.c0 + c * 8;
        const uint32_t loff = (uint32_t)(tid >> 5) * (uint32_t)p.ldz + (uint32_t)(c * 8);
#pragma unroll
        for (int it = 0; it < TPR * 32 / F::kThreads; ++it) {
          const int tr = it * (F::kThreads / 32) + (tid >> 5);
          const u32x4 x = *reinterpret_cast<const u32x4*>(buf + tr * 512 + ((c ^ (tr & 31)) << 4));
          uint16_t* rb = p.dz + (int64_t)(n0 + round * TPR + it * (F::kThreads / 32)) * p.ldz + (v0 - p.c0);
          if (col < p.kpad) *reinterpret_cast<u32x4*>(rb + loff) = x;
        }
        // buf is written again by the next round or the next k-tile's DMA
        // (after the last job nothing writes LDS again)
        if (NR > 1) dma_barrier<63>();
      }
    };
    static_assert(FBN * FBM * 2 <= 3 * FwdStages::kStage, "one round needs the whole tile in the LDS ring");
    if (last) {
      if (!conv_late) dma_barrier<0>();   // every DMA landed, every fragment read done: the whole ring is free
      store(lds, std::integral_constant<int, 1>{});
      if (conv_late) {
        __builtin_amdgcn_sched_barrier(0);   // the dz stores' registers first
        convert_rows(lds + kLateOff, job, kt_late);
      }
    } else {
      store(stage, std::integral_constant<int, 2>{});
    }
  }, convert_w);
  // the stream ended with a workgroup barrier: every wave's slot is final
  if (tid == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < F::kThreads / 64; ++i) m = max(m, wmag_lds[i]);
    if (m) atomicMax(p.wmag, m);
  }
}

// h_s [N, H] bf16 -> h16 [hrows, H] fp16 = fp16(2^kh h_s) (2^kh from the
// recorded largest |h_s|: exact except for values more than 2^29 below the
// largest, which fall to fp16 subnormals), zero rows for tokens in [N, hrows).
// Same layout as h_s: the dW GEMM reads it as its MN-major operand.
__global__ __launch_bounds__(256) void convert_h(const uint16_t* __restrict__ h, int N, int H,
                                                   const uint32_t* __restrict__ scales, uint16_t* __restrict__ h16,
                                                   int hrows) {
  const int kh = h_scale_exp(scales[kScaleHmag]);
  const int64_t n8 = (int64_t)hrows * H / 8, live8 = (int64_t)N * H / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    u32x4 o = u32x4{0u, 0u, 0u, 0u};
    if (i < live8) {
      const u32x4 x = reinterpret_cast<const u32x4*>(h)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = ldexpf(__builtin_bit_cast(float, x[e] << 16), kh);
        const float hi = ldexpf(__builtin_bit_cast(float, x[e] & 0xFFFF0000u), kh);
        o[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
      }
    }
    reinterpret_cast<u32x4*>(h16)[i] = o;
  }
}

// The fp16 copy of one chunk's W_s rows again, as fp16(2^kw W_s), when the
// largest magnitude the dz kernel recorded for the chunk lies outside the
// band where the unscaled copy is exact and finite (kw != 0); rows from
// `rows` to ntv * 256 are zero (their dz columns are zero).  Otherwise every
// workgroup returns at once.
__global__ __launch_bounds__(256) void w_rescale(const uint16_t* __restrict__ W, int rows, int total_rows, int H,
                                                 const uint32_t* __restrict__ wmag, uint16_t* __restrict__ w16) {
  const int kw = w_scale_exp(*wmag);
  if (kw == 0) return;
  const int64_t n8 = (int64_t)total_rows * H / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i * 8 / H;
    u32x4 o = u32x4{0u, 0u, 0u, 0u};
    if (row < rows) {
      const u32x4 x = reinterpret_cast<const u32x4*>(W)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = ldexpf(__builtin_bit_cast(float, x[e] << 16), kw);
        const float hi = ldexpf(__builtin_bit_cast(float, x[e] & 0xffff0000u), kw);
        o[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
      }
    }
    reinterpret_cast<u32x4*>(w16)[i] = o;
  }
}

// ===========================================================================
// Backward, step 2: dW_s[c0 + m, n] (+)= (1/s) sum_t dz[t, m] h_s[t, n]
// A = dz and B = h16 = the scaled fp16 copy of h_s, both MN-major (token rows,
// vocabulary / hidden units contiguous; read transposed): every DMA
// instruction loads two 512-byte row segments.  (With B as a transposed,
// K-major copy, the 32-deep k-tiles made 64-byte row segments, which the
// CU's vector-memory path serves at half the rate: 5 % slower.)  256 x 256
// tiles in 32-deep k-tiles through four LDS stages (128 KB): the DMA runs
// three k-tiles ahead.  (Three 64-deep stages of a 256 x 256 tile would need
// 192 KB; with two, memory latency showed.)
// ===========================================================================
constexpr int WBM = kDwTileM, WBN = kDwTileN, WKT = 32, WNST = 4, WDSTEPS = 1;

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void dw_gemm(DwParams p) {
  // NW = 8 (kDwWaves): waves 4 (m) x 2 (n), 64 x 128 each
  constexpr int WGN = 2, WGM = NW / WGN;
  using TA = MN<WBM, NW, WKT>;
  using TB = MN<WBN, NW, WKT>;
  __shared__ __attribute__((aligned(1024))) char lds[WNST * (TA::kBytes + TB::kBytes)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w / WGN, wn = w % WGN;
  const int logical = xcd_logical(blockIdx.x, p.ntm * p.ntn);
  const int tm = logical / p.ntn, tn = logical - tm * p.ntn;
  const int m0 = tm * WBM, n0 = tn * WBN;
  constexpr int FM = WBM / WGM / 32, FN = WBN / WGN / 32;
  f32x16 acc[FM][FN];
  zero_acc(acc);
  // A: dz rows are tokens (k, zero-padded to the workspace's row count >=
  // hrows), columns vocabulary (m); B: h16 rows are tokens (k, zero past N),
  // columns hidden units (n)
  TA ta;
  ta.init(p.dz + m0, p.ldz, p.kpad - m0, lane, __builtin_amdgcn_readfirstlane(w));
  TB tb;
  tb.init(p.h16 + n0, p.H, p.H - n0, lane, __builtin_amdgcn_readfirstlane(w));
  gemm_loop<TA, TB, f16x8, false, WNST, false, WDSTEPS>(acc, p.hrows / WKT, lds, ta, tb, 0, tid, wm * (WBM / WGM),
                                                       wn * (WBN / WGN));
  // undo both operand scales at once (exact: a power of two)
  const int unscale = -((int)p.scales[kScaleKs] + h_scale_exp(p.scales[kScaleHmag]));
  // Stores through LDS (free since gemm_loop's last barrier), in two rounds:
  // round r takes blocks fn = 2r, 2r + 1 of every wave, i.e. the tile's
  // columns wn * 128 + 64 r .. + 63 for both wn: a [256 rows][128] fp32 image
  // (128 KB), 16-byte chunk q of row t at chunk q ^ 8 ((t / 4) % 2) (the two
  // half-waves of a write, rows t and t + 4, then use different banks).  Then
  // every thread stores 16-byte pieces: 16 lanes cover 64 contiguous columns
  // of a row (256 bytes), where register-order stores would write one 4-byte
  // value per lane.
  static_assert(WBM * 128 * 4 <= WNST * (TA::kBytes + TB::kBytes) && FN == 4, "one round is half the tile");
  constexpr int kRowB = 128 * 4;
  auto chunk_at = [](int t, int q) { return q ^ (((t >> 2) & 1) << 3); };
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int fn = 2 * r + j;
      const int col = wn * 64 + j * 32 + (lane & 31);   // column within the round's image
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = wm * (WBM / WGM) + fm * 32 + frag_row(i, lane);
          *reinterpret_cast<float*>(lds + t * kRowB + (chunk_at(t, col >> 2) << 4) + (col & 3) * 4) =
              ldexpf(acc[fm][fn][i], unscale);
        }
    }
    dma_barrier<63>();
    // piece = (row, wn half): 16 threads x 16 bytes
#pragma unroll 4
    for (int it = 0; it < WBM * 2 * 16 / (64 * NW); ++it) {
      const int piece = it * (64 * NW / 16) + (tid >> 4);
      const int t = piece >> 1, half = piece & 1, q = half * 16 + (tid & 15);
      const int m = m0 + t, n = n0 + half * 128 + 64 * r + (tid & 15) * 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(lds + t * kRowB + (chunk_at(t, q) << 4));
      if (m < p.width && n < p.H) {
        f32x4* o = reinterpret_cast<f32x4*>(p.dW + (int64_t)m * p.H + n);
        *o = p.accumulate ? *o + v : v;
      }
    }
    if (r == 0) dma_barrier<63>();   // round 1 writes the image again
  }
}

// ===========================================================================
// Backward, step 3: dh_s[m, n] (+)= (1/s) sum_v dz[m, v] W_s[c0 + v, n]
// A = dz (K-major rows), B = the fp16 copy of the W_s chunk (MN-major:
// vocabulary rows, hidden contiguous; read transposed).  256 x 128 tiles,
// three LDS stages.  The sum over v runs in segments that end at multiples
// of kDhSegment (absolute column): each segment's fp32 sum is added to the
// running total in order.  Chunks that start on segment boundaries thus give
// the same bits whatever their width (a chunk's total leaves through memory,
// scaled by the power of two 1/s, which commutes with the additions), so dh
// does not depend on N through the chunk plan.  With fewer tiles than CUs
// (small N) each (tile, segment) is a workgroup of its own that writes its
// segment sum, and dh_reduce adds them in the same order: the same bits.
// ===========================================================================
constexpr int HBM = kDhTileM, HBN = kDhTileN, HKT = 64, HNST = 3, HDSTEPS = 3;

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void dh_gemm(DhParams p) {
  // NW = 4 (kDhWaves): waves 2 x 2, 128 x 64 each
  constexpr int HGM = NW / 2, HGN = 2;
  using TA = KM<HBM, NW, HKT>;
  using TB = MN<HBN, NW, HKT>;
  __shared__ __attribute__((aligned(1024))) char lds[HNST * (TA::kBytes + TB::kBytes)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w / HGN, wn = w % HGN;
  // workgroup order: panels of p.panel column tiles, all row tiles of a
  // panel consecutive (each XCD takes a contiguous run of them); split by
  // segment, the segment is the slowest index
  const int ntiles = p.ntm * p.ntn;
  const int logical0 = xcd_logical(blockIdx.x, ntiles * (p.partial ? p.nseg : 1));
  const int seg = logical0 / ntiles, logical = logical0 - seg * ntiles;
  const int per = p.panel * p.ntm, panel = logical / per, r = logical - panel * per;
  const int width = min(p.panel, p.ntn - panel * p.panel);
  const int tm = r / width, tn = panel * p.panel + (r - (r / width) * width);
  const int m0 = tm * HBM, n0 = tn * HBN;
  constexpr int FM = HBM / HGM / 32, FN = HBN / HGN / 32;
  f32x16 acc[FM][FN], tot[FM][FN];
  // A: dz rows are tokens (m; npad zero-padded rows), columns vocabulary (k,
  // zero past the chunk width); B: the fp16 copy of the W_s chunk, rows
  // vocabulary (k; the copy covers every k-tile), columns hidden units (n).
  // the two operand scales, undone at once at the end (exact: a power of two)
  const int unscale = -((int)p.scales[kScaleKs] + w_scale_exp(*p.wmag));
  // Adding into dh from earlier chunks: the running total starts from dh's
  // value in this chunk's scale (exact), so each segment is added to the
  // total one at a time, in order, whatever the chunk plan.
  const bool carry = p.accumulate && !p.partial;
  if (carry) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * (HBN / HGN) + fn * 32 + (lane & 31);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + wm * (HBM / HGM) + fm * 32 + frag_row(i, lane);
          tot[fm][fn][i] = (m < p.N && n < p.H) ? ldexpf(p.dh[(int64_t)m * p.H + n], -unscale) : 0.f;
        }
    }
  }
  // Segment sg of the chunk: its columns between absolute multiples of
  // kDhSegment (chunk-relative [k0, k1); the first one starts at the chunk).
  const int s0 = p.partial ? seg : 0, s1 = p.partial ? seg + 1 : p.nseg;
  for (int sg = s0; sg < s1; ++sg) {
    const int a = (p.c0 / kDhSegment + sg) * kDhSegment;
    const int k0 = max(a, p.c0) - p.c0, k1 = min(p.kpad, a + kDhSegment - p.c0);
    zero_acc(acc);
    TA ta;
    ta.init(p.dz + (int64_t)m0 * p.ldz + k0, p.ldz, p.npad - m0, lane, __builtin_amdgcn_readfirstlane(w));
    TB tb;
    tb.init(p.w16 + (int64_t)k0 * p.H + n0, p.H, p.H - n0, lane, __builtin_amdgcn_readfirstlane(w));
    gemm_loop<TA, TB, f16x8, false, HNST, false, HDSTEPS>(acc, (k1 - k0) / HKT, lds, ta, tb, 0, tid,
                                                         wm * (HBM / HGM), wn * (HBN / HGN));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          tot[fm][fn][i] = (sg == s0 && !carry) ? acc[fm][fn][i] : tot[fm][fn][i] + acc[fm][fn][i];
  }
  if (p.partial) {   // this segment's raw sum; dh_reduce adds the segments in order
    float* P = p.partial + (int64_t)seg * p.N * p.H;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * (HBN / HGN) + fn * 32 + (lane & 31);
      if (n >= p.H) continue;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + wm * (HBM / HGM) + fm * 32 + frag_row(i, lane);
          if (m < p.N) P[(int64_t)m * p.H + n] = tot[fm][fn][i];
        }
    }
    return;
  }
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int n = n0 + wn * (HBN / HGN) + fn * 32 + (lane & 31);
    if (n >= p.H) continue;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * (HBM / HGM) + fm * 32 + frag_row(i, lane);
        if (m < p.N) p.dh[(int64_t)m * p.H + n] = ldexpf(tot[fm][fn][i], unscale);
      }
  }
}

// The segment sums of a split dh GEMM, added in segment order to the running
// total (dh of the earlier chunks, in this chunk's scale, or the first
// segment) -- the order the one-workgroup-per-tile GEMM adds them in -- and
// unscaled into dh.
__global__ __launch_bounds__(256) void dh_reduce(DhParams p) {
  const int unscale = -((int)p.scales[kScaleKs] + w_scale_exp(*p.wmag));
  const int64_t n4 = (int64_t)p.N * p.H / 4, plane = (int64_t)p.N * p.H;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4* o = reinterpret_cast<float4*>(p.dh) + i;
    float4 t = reinterpret_cast<const float4*>(p.partial)[i];
    if (p.accumulate) {   // the running total starts from dh in this chunk's scale
      const float4 e = *o;
      t = make_float4(ldexpf(e.x, -unscale) + t.x, ldexpf(e.y, -unscale) + t.y, ldexpf(e.z, -unscale) + t.z,
                      ldexpf(e.w, -unscale) + t.w);
    }
    for (int sg = 1; sg < p.nseg; ++sg) {
      const float4 q = reinterpret_cast<const float4*>(p.partial + sg * plane)[i];
      t.x = t.x + q.x; t.y = t.y + q.y; t.z = t.z + q.z; t.w = t.w + q.w;
    }
    *o = make_float4(ldexpf(t.x, unscale), ldexpf(t.y, unscale), ldexpf(t.z, unscale), ldexpf(t.w, unscale));
  }
}

// ===========================================================================
// Both sides given as fp32 logits: one workgroup per row streams z_s, z_t.
// ===========================================================================
// merged != NULL: write the row's (m_s, S_s, A, m_t, S_t) to merged as five
// planes of N (one vocabulary shard's partial) instead of finalising.
__global__ __launch_bounds__(256) void fwd_rows_logits(const float* __restrict__ z_s, const float* __restrict__ z_t,
                                                       const int32_t* __restrict__ z_rows, int z_nrows, int N, int V,
                                                       const uint8_t* __restrict__ row_mask,
                                                       float* __restrict__ loss, float* __restrict__ stats,
                                                       float* __restrict__ merged) {
  __shared__ float red[5][256];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int64_t r = z_rows ? min(max(z_rows[n], 0), z_nrows - 1) : n;   // row of z_s and z_t
  const float* rs = z_s + r * V;
  const float* rt = z_t + r * V;
  float ms = kNegBig, ss = 0.f, aa = 0.f, mt = kNegBig, st = 0.f;
  for (int v0 = 0; v0 < V; v0 += 4 * 256) {
    float a[4], b[4];
    bool ok[4];
    float tms = kNegBig, tmt = kNegBig;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + e * 256 + tid;
      ok[e] = v < V;
      a[e] = ok[e] ? rs[v] : 0.f;
      b[e] = ok[e] ? rt[v] : 0.f;
      if (ok[e]) { tms = fmaxf(tms, a[e]); tmt = fmaxf(tmt, b[e]); }
    }
    const float nms = fmaxf(ms, tms), nmt = fmaxf(mt, tmt);
    const float cs = nms * kL2E, ct = nmt * kL2E;
    float ps = 0.f, pt = 0.f, pa = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[e]) {
        const float es = ex2(fmaf(a[e], kL2E, -cs));
        const float et = ex2(fmaf(b[e], kL2E, -ct));
        ps += es;
        pt += et;
        pa = fmaf(es, a[e] - b[e], pa);
      }
    const float fs = ex2((ms - nms) * kL2E), ft = ex2((mt - nmt) * kL2E);
    ss = fmaf(ss, fs, ps);
    aa = fmaf(aa, fs, pa);
    st = fmaf(st, ft, pt);
    ms = nms;
    mt = nmt;
  }
  red[0][tid] = ms; red[1][tid] = ss; red[2][tid] = aa; red[3][tid] = mt; red[4][tid] = st;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      float m1 = red[0][tid], s1 = red[1][tid], a1 = red[2][tid], m2 = red[3][tid], s2 = red[4][tid];
      merge3(m1, s1, a1, red[0][tid + off], red[1][tid + off], red[2][tid + off]);
      merge2(m2, s2, red[3][tid + off], red[4][tid + off]);
      red[0][tid] = m1; red[1][tid] = s1; red[2][tid] = a1; red[3][tid] = m2; red[4][tid] = s2;
    }
    __syncthreads();
  }
  if (tid == 0 && merged) {
#pragma unroll
    for (int c = 0; c < 5; ++c) merged[(int64_t)c * N + n] = red[c][0];
    return;
  }
  if (tid == 0) {
    const float log_ss = logf(red[1][0]);
    float lse_s = red[0][0] + log_ss;
    float lse_t = red[3][0] + logf(red[4][0]);
    float L = red[2][0] / red[1][0] - (lse_s - lse_t);
    float lpmax = -log_ss;
    if (row_mask && row_mask[n] == 0) { L = 0.f; lse_s = 0.f; lse_t = 0.f; lpmax = 0.f; }
    loss[n] = L;
    stats[4 * (int64_t)n + 0] = lse_s;
    stats[4 * (int64_t)n + 1] = lse_t;
    stats[4 * (int64_t)n + 2] = L;
    stats[4 * (int64_t)n + 3] = lpmax;
  }
}

__global__ __launch_bounds__(256) void bwd_rows_logits(const float* __restrict__ z_s, const float* __restrict__ z_t,
                                                       const int32_t* __restrict__ z_rows, int z_nrows, int N, int V,
                                                       const uint8_t* __restrict__ row_mask,
                                                       const float* __restrict__ grad, const float* __restrict__ stats,
                                                       float* __restrict__ dz) {
  const int n = blockIdx.x;
  const int v = blockIdx.y * 256 + threadIdx.x;
  if (v >= V) return;
  const bool live = !row_mask || row_mask[n] != 0;
  float d = 0.f;
  if (live) {
    const float lse_s = stats[4 * (int64_t)n + 0], lse_t = stats[4 * (int64_t)n + 1], L = stats[4 * (int64_t)n + 2];
    const float g = grad ? grad[n] : 1.0f;
    const int64_t r = z_rows ? min(max(z_rows[n], 0), z_nrows - 1) : n;   // row of z_s and z_t
    const float a = z_s[r * V + v], b = z_t[r * V + v];
    d = g * ex2(fmaf(a, kL2E, -(lse_s * kL2E))) * ((a - b) - ((lse_s - lse_t) + L));
  }
  dz[(int64_t)n * V + v] = d;
}

// ===========================================================================
// Top-k estimator of the reverse KL (NeMo-RL page, summary: the K = V limit
// of the top-k estimator, whose score-function tail vanishes once the
// support spans the vocabulary).  Per row t, support ids S[t, 0..K) (ids
// outside [0, V) are skipped), teacher log-probabilities lpt_S on them and
// lpt_y at the sampled token y, f = log p_s - log p_t:
//   L_hat = sum_{j in S} p_j f_j + [y not in S] f_y,
//   dz_j  = g (-p_j c + [j in S] p_j (f_j + 1) + [j = y, y not in S] sp),
//   c = sum_{j in S} p_j (f_j + 1) + [y not in S] sp,   sp = f_y + 1.
// The student logits on the support come from wave-wide dot products of the
// row of h with the support's rows of W, kTopkBatch support ids at a time so
// that their row loads are in flight together (fp32; each lane accumulates
// its slice in a fixed order, then a fixed butterfly: the backward
// recomputes exactly the forward's values).
// ===========================================================================
constexpr int kTopkBatch = 8;

// z[b] = h . W[j[b]] for the ids of one batch (ids outside [0, V) read row 0;
// their values are not used).
__device__ __forceinline__ void wave_dots_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                               const int (&j)[kTopkBatch], int V, int H, int lane,
                                               float (&z)[kTopkBatch]) {
  const uint16_t* row[kTopkBatch];
#pragma unroll
  for (int b = 0; b < kTopkBatch; ++b) {
    z[b] = 0.f;
    row[b] = W + (int64_t)((j[b] >= 0 && j[b] < V) ? j[b] : 0) * H;
  }
  for (int c = lane * 8; c < H; c += 512) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(h + c);
    u32x4 w[kTopkBatch];
#pragma unroll
    for (int b = 0; b < kTopkBatch; ++b) w[b] = *reinterpret_cast<const u32x4*>(row[b] + c);
#pragma unroll
    for (int b = 0; b < kTopkBatch; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[b] = fmaf(__builtin_bit_cast(float, x[e] << 16), __builtin_bit_cast(float, w[b][e] << 16), z[b]);
        z[b] = fmaf(__builtin_bit_cast(float, x[e] & 0xffff0000u), __builtin_bit_cast(float, w[b][e] & 0xffff0000u),
                    z[b]);
      }
  }
#pragma unroll
  for (int b = 0; b < kTopkBatch; ++b)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z[b] += __shfl_xor(z[b], o);
}

// The support ids k0 .. k0 + kTopkBatch - 1 of row t (-1 past K).
__device__ __forceinline__ void topk_batch_ids(const int32_t* __restrict__ S, int64_t t, int K, int k0,
                                               int (&j)[kTopkBatch]) {
#pragma unroll
  for (int b = 0; b < kTopkBatch; ++b) j[b] = k0 + b < K ? S[t * K + k0 + b] : -1;
}

// One wave per row.  stats on entry: (lse, -, log p(y), -) from the
// log-probability forward; on exit (lse, c, sp, bound) with bound = |c| + |sp|
// + max_{j in S} p_j |f_j + 1| >= max_j |dz_j| / |g| (for the backward's fp16
// scale).  Rows with row_mask 0: loss 0, stats 0.
__global__ __launch_bounds__(256) void topk_terms(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                  int N, int V, int H, int K, const int32_t* __restrict__ y,
                                                  const int32_t* __restrict__ S, const float* __restrict__ lpt_S,
                                                  const float* __restrict__ lpt_y,
                                                  const uint8_t* __restrict__ row_mask, float* __restrict__ loss,
                                                  float* __restrict__ stats, float* __restrict__ lps) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;
  float* st = stats + 4 * (int64_t)t;
  if (row_mask && row_mask[t] == 0) {
    if (lane == 0) {
      loss[t] = 0.f;
      st[0] = 0.f; st[1] = 0.f; st[2] = 0.f; st[3] = 0.f;
    }
    if (lps)
      for (int k = lane; k < K; k += 64) lps[(int64_t)t * K + k] = 0.f;
    return;
  }
  const float lse = st[0], lpy = st[2];
  const int yt = y[t];
  float L = 0.f, c = 0.f, bnd = 0.f;
  bool in = false;
  for (int k0 = 0; k0 < K; k0 += kTopkBatch) {
    int j[kTopkBatch];
    float z[kTopkBatch];
    topk_batch_ids(S, t, K, k0, j);
    wave_dots_bf16(h + (int64_t)t * H, W, j, V, H, lane, z);
    // the student's log-probabilities on the support, for the backward
    // (0 for ids outside [0, V)); lane b writes entry k0 + b
    if (lps) {
      float mine = 0.f;
#pragma unroll
      for (int b = 0; b < kTopkBatch; ++b)
        if (lane == b && j[b] >= 0 && j[b] < V) mine = z[b] - lse;
      if (lane < kTopkBatch && k0 + lane < K) lps[(int64_t)t * K + k0 + lane] = mine;
    }
#pragma unroll
    for (int b = 0; b < kTopkBatch; ++b) {
      if (j[b] < 0 || j[b] >= V) continue;
      const float lp = z[b] - lse;
      const float f = lp - lpt_S[(int64_t)t * K + k0 + b];
      const float pr = expf(lp);
      L = fmaf(pr, f, L);
      c = fmaf(pr, f + 1.f, c);
      bnd = fmaxf(bnd, pr * fabsf(f + 1.f));
      in = in || j[b] == yt;
    }
  }
  float sp = 0.f;
  if (!in) {
    const float fy = lpy - lpt_y[t];
    L += fy;
    sp = fy + 1.f;
    c += sp;
  }
  if (lane == 0) {
    loss[t] = L;
    st[1] = c;
    st[2] = sp;
    st[3] = fabsf(c) + fabsf(sp) + bnd;
  }
}

// One wave per row: for each support id j in the chunk [c0, c0 + width), add
// s g p_j (f_j + 1) to the row's fp16 dz entry (lane 0, in support order, so
// repeated ids add up), saturating at fp16's largest finite value.
__global__ __launch_bounds__(256) void topk_dz_add(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                   int N, int V, int H, int K, const int32_t* __restrict__ S,
                                                   const float* __restrict__ lpt_S, const float* __restrict__ lps,
                                                   const uint8_t* __restrict__ row_mask,
                                                   const float* __restrict__ grad, const float* __restrict__ stats,
                                                   const uint32_t* __restrict__ scales, uint16_t* __restrict__ dz,
                                                   int ldz, int c0, int width) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N || (row_mask && row_mask[t] == 0)) return;
  const float gs = (grad ? grad[t] : 1.0f) * __builtin_bit_cast(float, scales[kScaleS]);
  const float lse = stats[4 * (int64_t)t];
  for (int k0 = 0; k0 < K; k0 += kTopkBatch) {
    int j[kTopkBatch];
    float z[kTopkBatch];
    topk_batch_ids(S, t, K, k0, j);
    bool any = false;   // an id of the batch in this chunk (wave-uniform)
#pragma unroll
    for (int b = 0; b < kTopkBatch; ++b) {
      if (j[b] < c0 || j[b] >= c0 + width || j[b] >= V) j[b] = -1;
      any = any || j[b] >= 0;
    }
    if (!any) continue;
    // the forward's log-probabilities when given (the same fp32 values),
    // else the dot products again
    if (!lps) wave_dots_bf16(h + (int64_t)t * H, W, j, V, H, lane, z);
#pragma unroll
    for (int b = 0; b < kTopkBatch; ++b) {
      if (j[b] < 0) continue;
      const float lp = lps ? lps[(int64_t)t * K + k0 + b] : z[b] - lse;
      const float f = lp - lpt_S[(int64_t)t * K + k0 + b];
      if (lane == 0) {
        uint16_t* e = dz + (int64_t)t * ldz + (j[b] - c0);
        const float v = (float)__builtin_bit_cast(_Float16, *e) + gs * expf(lp) * (f + 1.f);
        *e = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_fmed3f(v, -65504.f, 65504.f));
      }
    }
  }
}

// ===========================================================================
// Compaction, gather, scatter, fill.
// ===========================================================================
__global__ __launch_bounds__(1024) void compact_kernel(const uint8_t* __restrict__ mask, int T,
                                                       int32_t* __restrict__ row_idx, int32_t* __restrict__ n_out) {
  __shared__ int wave_cnt[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int base = 0;
  for (int start = 0; start < T; start += 1024) {
    const int t = start + tid;
    const bool f = t < T && mask[t] != 0;
    const unsigned long long bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[w] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < w) off += wave_cnt[i];
      total += wave_cnt[i];
    }
    if (f) row_idx[base + off + before] = t;
    base += total;
    __syncthreads();
  }
  if (tid == 0) *n_out = base;
}

// Stable counting sort of rows by teacher id (one workgroup): bucket k holds
// the rows with id k in [0, K), bucket K those with any other id, each in
// ascending row order.  perm[j] is the row placed at j; teacher_p[j] and
// mask_p[j] (when mask is given) are that row's id and mask byte.
__global__ __launch_bounds__(1024) void group_by_teacher_kernel(const int32_t* __restrict__ teacher,
                                                                const uint8_t* __restrict__ mask, int N, int K,
                                                                int32_t* __restrict__ perm,
                                                                int32_t* __restrict__ teacher_p,
                                                                uint8_t* __restrict__ mask_p) {
  __shared__ int start[32];
  __shared__ int wave_cnt[16][32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  if (tid < 32) start[tid] = 0;
  __syncthreads();
  for (int i = tid; i < N; i += 1024) {
    const int k = teacher[i];
    atomicAdd(&start[(k >= 0 && k < K) ? k : K], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b <= K; ++b) {
      const int c = start[b];
      start[b] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int i = base + tid;
    const int id = i < N ? teacher[i] : 0;
    const int b = i < N ? ((id >= 0 && id < K) ? id : K) : -1;
    int rank = 0;
    for (int k = 0; k <= K; ++k) {
      const unsigned long long bal = __ballot(b == k);
      if (b == k) rank = __popcll(bal & below);
      if (lane == 0) wave_cnt[w][k] = __popcll(bal);
    }
    __syncthreads();
    if (b >= 0) {
      int j = start[b] + rank;
      for (int u = 0; u < w; ++u) j += wave_cnt[u][b];
      perm[j] = i;
      teacher_p[j] = id;
      if (mask) mask_p[j] = mask[i];
    }
    __syncthreads();
    if (tid <= K) {
      int c = 0;
      for (int u = 0; u < 16; ++u) c += wave_cnt[u][tid];
      start[tid] += c;
    }
    __syncthreads();
  }
}

template <typename U>
__global__ __launch_bounds__(256) void gather_kernel(const U* __restrict__ src, int64_t row_units,
                                                     const int32_t* __restrict__ row_idx, U* __restrict__ dst) {
  const int64_t i = blockIdx.x;
  const U* s = src + (int64_t)row_idx[i] * row_units;
  U* d = dst + i * row_units;
  for (int64_t u = (int64_t)blockIdx.y * 256 + threadIdx.x; u < row_units; u += (int64_t)gridDim.y * 256) d[u] = s[u];
}

template <typename U>
__global__ __launch_bounds__(256) void scatter_kernel(const U* __restrict__ src, int64_t row_units,
                                                      const int32_t* __restrict__ row_idx, U* __restrict__ dst) {
  const int64_t i = blockIdx.x;
  const U* s = src + i * row_units;
  U* d = dst + (int64_t)row_idx[i] * row_units;
  for (int64_t u = (int64_t)blockIdx.y * 256 + threadIdx.x; u < row_units; u += (int64_t)gridDim.y * 256) d[u] = s[u];
}

__global__ __launch_bounds__(256) void fill_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// ===========================================================================
// Launchers
// ===========================================================================
namespace {
thread_local hipEvent_t g_launch_ev[2] = {nullptr, nullptr};
}

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
  g_launch_ev[0] = start;
  g_launch_ev[1] = stop;
}

bool launch_events_pending() { return g_launch_ev[0] != nullptr || g_launch_ev[1] != nullptr; }

// kernel<<<grid, block, 0, s>>>(args...), carrying the pending timing events
// (if any): the arguments are converted to the kernel's parameter types and
// passed by address, as the launch API wants them.
template <class... P, class... A>
static hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<std::remove_cv_t<std::remove_reference_t<P>>...> vals(std::forward<A>(a)...);
  void* args[sizeof...(P)];
  std::apply([&args](auto&... v) {
    int i = 0;
    ((args[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  const hipEvent_t e0 = g_launch_ev[0], e1 = g_launch_ev[1];
  g_launch_ev[0] = g_launch_ev[1] = nullptr;
  // untimed: the plain launch (what kernel<<<>>> does, stream capture included)
  if (!e0 && !e1) return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s, e0, e1, 0);
}

static inline unsigned grid1(int64_t n, int64_t per, int64_t cap) {
  int64_t g = (n + per - 1) / per;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

hipError_t launch_fwd_tiles(const FwdParams& p, int mode, hipStream_t s) {
  const unsigned nb = (unsigned)((p.nsplit + p.splits_per_wg - 1) / p.splits_per_wg * p.ntok);
  constexpr int NW = kFusedWaves;
  constexpr unsigned nt = Fused<NW>::kThreads;
  if (mode == kModeHidden)
    return launch(fwd_tiles<kModeHidden, true, NW>, nb, nt, s, p);
  else if (mode == kModeHiddenTeachers)
    return launch(fwd_tiles<kModeHiddenTeachers, true, NW>, nb, nt, s, p);
  else if (mode == kModeLogprobEntropy)
    return launch(fwd_tiles<kModeLogprobEntropy, true, kFusedWavesOne>, nb, Fused<kFusedWavesOne>::kThreads, s, p);
  else if (p.V % 4 == 0)
    return launch(fwd_tiles<kModeTeacherLogits, true, NW>, nb, nt, s, p);
  else
    return launch(fwd_tiles<kModeTeacherLogits, false, NW>, nb, nt, s, p);
}

hipError_t launch_fwd_combine(const float* partial, int nsplit, int N, const uint8_t* row_mask, bool logprob_entropy,
                              float* out0, float* out1, float* stats, hipStream_t s) {
  const unsigned nb = (unsigned)((N + kCombRows - 1) / kCombRows);
  if (logprob_entropy)
    return launch(fwd_combine<kCombineLPE>, nb, 256, s, partial, nsplit, N, row_mask, out0, out1, stats);
  else
    return launch(fwd_combine<kCombineKL>, nb, 256, s, partial, nsplit, N, row_mask, out0, out1, stats);
}

hipError_t launch_fwd_merge(const float* partial, int nsplit, int N, float* merged, hipStream_t s) {
  const unsigned nb = (unsigned)((N + kCombRows - 1) / kCombRows);
  return launch(fwd_combine<kCombineMerged>, nb, 256, s, partial, nsplit, N, nullptr, merged, nullptr, nullptr);
}

hipError_t launch_bwd_dz(const BwdParams& p, int mode, hipStream_t s) {
  const unsigned nb = (unsigned)(p.ngroups * p.ntok);
  constexpr int NW = kFusedWaves;
  constexpr unsigned nt = Fused<NW>::kThreads;
  if (mode == kModeHidden && p.late_w16)
    return launch(bwd_dz_tiles<kModeHidden, true, NW, true>, nb, nt, s, p);
  else if (mode == kModeHidden)
    return launch(bwd_dz_tiles<kModeHidden, true, NW>, nb, nt, s, p);
  else if (mode == kModeHiddenTeachers && p.late_w16)
    return launch(bwd_dz_tiles<kModeHiddenTeachers, true, NW, true>, nb, nt, s, p);
  else if (mode == kModeHiddenTeachers)
    return launch(bwd_dz_tiles<kModeHiddenTeachers, true, NW>, nb, nt, s, p);
  else if (mode == kModeLogprobEntropy)
    return launch(bwd_dz_tiles<kModeLogprobEntropy, true, NW>, nb, nt, s, p);
  else if (mode == kModeTopK)
    return launch(bwd_dz_tiles<kModeTopK, true, kFusedWavesOne>, nb, Fused<kFusedWavesOne>::kThreads, s, p);
  else if (p.V % 4 == 0)
    return launch(bwd_dz_tiles<kModeTeacherLogits, true, NW>, nb, nt, s, p);
  else
    return launch(bwd_dz_tiles<kModeTeacherLogits, false, NW>, nb, nt, s, p);
}

hipError_t launch_grad_scale(const float* grad, const float* grad_h, const uint8_t* row_mask, const float* stats,
                             int N, int mode, int nchunks, uint32_t* scales, hipStream_t s) {
  if (mode == kModeLogprobEntropy)
    return launch(grad_scale<kModeLogprobEntropy>, 1, 1024, s, grad, grad_h, row_mask, stats, N, nchunks, scales);
  else if (mode == kModeTopK)
    return launch(grad_scale<kModeTopK>, 1, 1024, s, grad, grad_h, row_mask, stats, N, nchunks, scales);
  else
    return launch(grad_scale<kModeHidden>, 1, 1024, s, grad, grad_h, row_mask, stats, N, nchunks, scales);
}

hipError_t launch_topk_terms(const uint16_t* h, const uint16_t* W, int N, int V, int H, int K, const int32_t* y,
                             const int32_t* S, const float* lpt_S, const float* lpt_y, const uint8_t* row_mask,
                             float* loss, float* stats, float* lps, hipStream_t s) {
  return launch(topk_terms, (unsigned)((N + 3) / 4), 256, s, h, W, N, V, H, K, y, S, lpt_S, lpt_y, row_mask, loss, stats, lps);
}

hipError_t launch_topk_dz_add(const uint16_t* h, const uint16_t* W, int N, int V, int H, int K, const int32_t* S,
                              const float* lpt_S, const float* lps, const uint8_t* row_mask, const float* grad,
                              const float* stats, const uint32_t* scales, uint16_t* dz, int ldz, int c0, int width,
                              hipStream_t s) {
  return launch(topk_dz_add, (unsigned)((N + 3) / 4), 256, s, h, W, N, V, H, K, S, lpt_S, lps, row_mask, grad, stats, scales,
                                                      dz, ldz, c0, width);
}

hipError_t launch_absmax_bf16(const uint16_t* h, int64_t n, uint32_t* scales, hipStream_t s) {
  return launch(absmax_bf16, grid1(n / 8 + 1, 256 * 4, 256), 256, s, h, n, scales);
}

hipError_t launch_convert_h(const uint16_t* h, int N, int H, const uint32_t* scales, uint16_t* h16, int hrows,
                              hipStream_t s) {
  return launch(convert_h, grid1((int64_t)hrows * H / 8, 256, 4096), 256, s, h, N, H, scales, h16, hrows);
}

hipError_t launch_w_rescale(const uint16_t* W_chunk, int rows, int ntv, int H, const uint32_t* wmag, uint16_t* w16,
                            hipStream_t s) {
  const int64_t n8 = (int64_t)ntv * kFwdTileV * H / 8;
  return launch(w_rescale, grid1(n8, 256 * 4, 2048), 256, s, W_chunk, rows, ntv * kFwdTileV, H, wmag, w16);
}

hipError_t launch_dw(const DwParams& p, hipStream_t s) {
  return launch(dw_gemm<kDwWaves>, (unsigned)(p.ntm * p.ntn), 64 * kDwWaves, s, p);
}

hipError_t launch_dh(const DhParams& p, hipStream_t s) {
  return launch(dh_gemm<kDhWaves>, (unsigned)(p.ntm * p.ntn * (p.partial ? p.nseg : 1)), 64 * kDhWaves, s, p);
}

hipError_t launch_dh_reduce(const DhParams& p, hipStream_t s) {
  return launch(dh_reduce, grid1((int64_t)p.N * p.H / 4, 256, 2048), 256, s, p);
}

hipError_t launch_fwd_rows_logits(const float* z_s, const float* z_t, const int32_t* z_rows, int z_nrows, int N, int V,
                                  const uint8_t* row_mask, float* loss, float* stats, float* merged, hipStream_t s) {
  return launch(fwd_rows_logits, (unsigned)N, 256, s, z_s, z_t, z_rows, z_nrows, N, V, row_mask, loss, stats, merged);
}

hipError_t launch_bwd_rows_logits(const float* z_s, const float* z_t, const int32_t* z_rows, int z_nrows, int N, int V,
                                  const uint8_t* row_mask, const float* grad, const float* stats, float* dz,
                                  hipStream_t s) {
  dim3 g((unsigned)N, (unsigned)((V + 255) / 256));
  return launch(bwd_rows_logits, g, 256, s, z_s, z_t, z_rows, z_nrows, N, V, row_mask, grad, stats, dz);
}

hipError_t launch_compact(const uint8_t* mask, int T, int32_t* row_idx, int32_t* n_out, hipStream_t s) {
  return launch(compact_kernel, 1, 1024, s, mask, T, row_idx, n_out);
}

hipError_t launch_group_by_teacher(const int32_t* teacher, const uint8_t* mask, int N, int K, int32_t* perm,
                                   int32_t* teacher_p, uint8_t* mask_p, hipStream_t s) {
  if (K < 1 || K > 31) return hipErrorInvalidValue;
  return launch(group_by_teacher_kernel, 1, 1024, s, teacher, mask, N, K, perm, teacher_p, mask_p);
}

hipError_t launch_gather(const void* src, int64_t row_bytes, const int32_t* row_idx, int64_t N, void* dst,
                         hipStream_t s) {
  const bool v16 = (row_bytes % 16) == 0;
  const int64_t units = v16 ? row_bytes / 16 : row_bytes / 4;
  dim3 g((unsigned)N, grid1(units, 256, 64));
  if (v16)
    return launch(gather_kernel<u32x4>, g, 256, s, (const u32x4*)src, units, row_idx, (u32x4*)dst);
  else
    return launch(gather_kernel<uint32_t>, g, 256, s, (const uint32_t*)src, units, row_idx, (uint32_t*)dst);
}

hipError_t launch_scatter(const void* src, int64_t row_bytes, const int32_t* row_idx, int64_t N, void* dst,
                          hipStream_t s) {
  const bool v16 = (row_bytes % 16) == 0;
  const int64_t units = v16 ? row_bytes / 16 : row_bytes / 4;
  dim3 g((unsigned)N, grid1(units, 256, 64));
  if (v16)
    return launch(scatter_kernel<u32x4>, g, 256, s, (const u32x4*)src, units, row_idx, (u32x4*)dst);
  else
    return launch(scatter_kernel<uint32_t>, g, 256, s, (const uint32_t*)src, units, row_idx, (uint32_t*)dst);
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  return launch(fill_zero_u32, grid1(n, 256, 8192), 256, s, (uint32_t*)p, n);
}

}  // namespace rkl
