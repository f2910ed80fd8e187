// rkl_internal.h -- kernel parameter blocks and launchers shared by the C ABI
// (rkl_api.hip) and the kernels (rkl_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkl {

struct FwdParams {
  int N, V, Hs, Ht;
  const uint16_t* h_s;
  const uint16_t* W_s;
  const uint16_t* h_t;
  const uint16_t* W_t;
  const float* z_t;        // teacher logits, rows of V (teacher-logits payload)
  const int32_t* z_rows;   // row of z_t for token n (NULL: row n)
  int z_nrows;             // rows z_t holds (z_rows values are clamped to [0, z_nrows))
  const int32_t* y;        // sampled token per row (log-probability / entropy)
  const int32_t* teacher;  // teacher per row (NULL: one teacher)
  int K;                   // teachers: W_t holds K weights, wt_stride elements apart
  int64_t wt_stride;
  float* partial;          // [nsplit][5][N]
  int tiles_per_split;     // 256-row vocabulary tiles per split
  int nsplit;
  int splits_per_wg;       // consecutive splits one workgroup streams through
  int ntok;                // 128-token tiles
  int order_gs, order_tg;  // workgroup order (panel_order)
};

struct BwdParams {
  int N, V, Hs, Ht;
  const uint16_t* h_s;
  const uint16_t* W_s;
  const uint16_t* h_t;
  const uint16_t* W_t;
  const float* z_t;
  const int32_t* z_rows;   // row of z_t for token n (NULL: row n)
  int z_nrows;             // rows z_t holds (z_rows values are clamped to [0, z_nrows))
  const uint8_t* row_mask;
  const float* grad;       // g of L (reverse KL) or of log p(y) (log-probability / entropy)
  const float* grad_h;     // g of the entropy (log-probability / entropy)
  const int32_t* y;        // sampled token per row (log-probability / entropy)
  const int32_t* teacher;  // teacher per row (NULL: one teacher)
  int K;
  int64_t wt_stride;
  const float* stats;
  const uint32_t* scales;  // the backward's scale block (kScaleS: dz is stored as fp16(s * dz))
  uint32_t* wmag;          // this chunk's slot of kScaleWmag: largest |W_s| converted (atomic max)
  uint16_t* dz;            // [ntok * 128, ldz] fp16 chunk workspace (rows past N written as zero)
  uint16_t* w16;           // [ntv * 256, Hs] fp16 copy of the W_s chunk (for dh)
  int ldz;
  int c0;                  // first vocabulary row of the chunk
  int kpad;                // chunk width rounded up to 64 (columns written)
  int ntv;                 // 256-row vocabulary tiles in the chunk
  int tiles_per_group;     // vocabulary tiles one workgroup sweeps
  int ngroups;             // ceil(ntv / tiles_per_group)
  int ntok;
  int order_gs, order_tg;  // workgroup order (panel_order)
  int late_w16;            // convert the fp16 W_s copy after the stream (one job, at most one k-tile per workgroup)
};

struct DwParams {
  const uint32_t* scales;  // kScaleKs, kScaleHmag: dW = 2^-(ks + kh) * sum of the fp16 products
  const uint16_t* dz;
  int ldz, N, kpad, width;
  const uint16_t* h16;     // [hrows, H] fp16(2^kh h_s), rows past N zero
  int hrows, H;
  float* dW;               // dW_s + c0 * H
  int accumulate;
  int ntm, ntn;
};

struct DhParams {
  const uint32_t* scales;  // kScaleKs: dh = 2^-(ks + kw) * sum of the fp16 products
  const uint32_t* wmag;    // this chunk's largest |W_s| (fixes kw)
  const uint16_t* dz;
  int ldz, N, npad, kpad, width;   // npad: dz workspace rows
  int c0;                          // first vocabulary column of the chunk
  const uint16_t* w16;     // fp16 copy of the W_s chunk [>= kpad rows, H]
  int H;
  float* dh;
  int accumulate;
  int ntm, ntn;
  int panel;               // column tiles per panel of the workgroup order
  // Split by segment (grids of fewer tiles than CUs): workgroup (tile, s)
  // writes segment s's raw fp32 sum to partial [nseg][N][H], and dh_reduce
  // adds them in segment order.  partial NULL: one workgroup per tile sums
  // every segment itself.
  float* partial;
  int nseg;
};

// Waves per workgroup: the fused kernels (two waves per SIMD, 64 x 64 of both
// projections per wave), the log-probability / entropy forward and the top-k
// estimator's dz kernel (one projection: one wave per SIMD, 128 x 64 per wave,
// six fragments feed eight MFMAs instead of four feeding four), the dW GEMM
// (two per SIMD) and the dh GEMM (one per SIMD) -- the layouts measured
// fastest; no other count is built.  (The teacher-logits kernels and the
// log-probability / entropy dz kernel keep eight: with four they spill.)
constexpr int kFusedWaves = 8;
constexpr int kFusedWavesOne = 4;
constexpr int kDwWaves = 8;
constexpr int kDhWaves = 4;

// The backward's scale block (32-bit words at the front of its workspace).
// The dz, dW and dh GEMM operands are fp16 copies scaled by powers of two, so
// every copy is exact wherever fp16 represents the scaled value and the GEMM
// epilogues undo the scales exactly:
//   dz   = fp16(2^ks dz),   2^ks puts the largest |g| p_max in [16, 32);
//   h16  = fp16(2^kh h_s),  2^kh puts the largest |h_s| in [2^14, 2^15);
//   W16  = fp16(2^kw W_s) per chunk, kw = 0 while the chunk's largest |W_s|
//          lies in [2^-10, 2^15), else the power of two that puts it in
//          [2^14, 2^15) (the dz kernel converts with kw = 0 and records the
//          largest magnitude; w_rescale converts the chunk again when needed).
constexpr int kScaleS = 0;      // float 2^ks
constexpr int kScaleKs = 1;     // int ks
constexpr int kScaleHmag = 2;   // largest |h_s| as bf16 magnitude bits (atomic max)
constexpr int kScaleWmag = 4;   // first of one slot per chunk: largest |W_s| of the chunk's rows
constexpr int kMaxExpShift = 100;   // |kh|, |kw| are clamped to this

// Tile sizes the host needs for grids and workspace.
constexpr int kFwdTileV = 256;
constexpr int kFwdTileN = 128;
constexpr int kDwTileM = 256, kDwTileN = 256;
constexpr int kDhTileM = 256, kDhTileN = 128;
// dh's fp32 sum over the vocabulary is split at multiples of this column
// index (absolute), whatever the backward's chunk width or the dh GEMM's
// grid: each segment is summed from zero and the segment sums are added in
// order.
constexpr int kDhSegment = 16384;
// The backward's vocabulary chunks are whole multiples of this many columns
// (a multiple of kDhSegment).
constexpr int kChunkUnit = 65536;

// What the fused kernels compute.
enum Mode : int {
  kModeHidden = 0,          // reverse KL, teacher projected from hidden states
  kModeTeacherLogits = 1,   // reverse KL, teacher logits streamed
  kModeLogprobEntropy = 2,  // log p(sampled token) and entropy of one projection
  kModeHiddenTeachers = 3,  // reverse KL, teacher hidden states, teacher chosen per row
  kModeTopK = 4,            // top-k estimator's backward: dense part -p c + spike at the sampled token
};

// Sets the calling thread's rkl_last_error message; returns code.
int set_last_error(int code, const char* msg);

// Per-kernel timing: events that the calling thread's next kernel launch
// takes as its own start and stop (hipExtLaunchKernel stamps them with the
// kernel's begin and end, with no marker packets of their own in the queue;
// without events a launch is the plain one).
// Each launch_* function below launches at most one kernel, and that launch
// clears them; launch_events_pending() is then false.  A launch_* call that
// launched nothing leaves them pending.
void set_launch_events(hipEvent_t start, hipEvent_t stop);
bool launch_events_pending();

hipError_t launch_fwd_tiles(const FwdParams& p, int mode, hipStream_t s);
// out0: loss (reverse KL) or log p(y); out1: entropy (log-probability / entropy only)
hipError_t launch_fwd_combine(const float* partial, int nsplit, int N, const uint8_t* row_mask, bool logprob_entropy,
                              float* out0, float* out1, float* stats, hipStream_t s);
// The splits' merged (m_s, S_s, A, m_t, S_t), not finalised: five planes of N.
hipError_t launch_fwd_merge(const float* partial, int nsplit, int N, float* merged, hipStream_t s);
hipError_t launch_bwd_dz(const BwdParams& p, int mode, hipStream_t s);
// Writes kScaleS / kScaleKs and clears kScaleHmag and the nchunks kScaleWmag slots.
// mode: kModeLogprobEntropy, kModeTopK or a reverse-KL mode (the bound on |dz| / |g| differs).
hipError_t launch_grad_scale(const float* grad, const float* grad_h, const uint8_t* row_mask, const float* stats,
                             int N, int mode, int nchunks, uint32_t* scales, hipStream_t s);
// Top-k estimator, forward: per row, from stats = (lse, -, log p(y), -) of the
// log-probability forward, the support terms over the K ids of S and the
// tail at y; writes loss and stats = (lse, c, sp, bound) (see the kernel).
hipError_t launch_topk_terms(const uint16_t* h, const uint16_t* W, int N, int V, int H, int K, const int32_t* y,
                             const int32_t* S, const float* lpt_S, const float* lpt_y, const uint8_t* row_mask,
                             float* loss, float* stats, float* lps, hipStream_t s);
// Top-k estimator, backward: adds s g p_j (f_j + 1) for the support ids j of
// chunk [c0, c0 + width) into the fp16 dz chunk.
hipError_t launch_topk_dz_add(const uint16_t* h, const uint16_t* W, int N, int V, int H, int K, const int32_t* S,
                              const float* lpt_S, const float* lps, const uint8_t* row_mask, const float* grad,
                              const float* stats, const uint32_t* scales, uint16_t* dz, int ldz, int c0, int width,
                              hipStream_t s);
// scales[kScaleHmag] = max over h [n] of the bf16 magnitude bits (after launch_grad_scale cleared it)
hipError_t launch_absmax_bf16(const uint16_t* h, int64_t n, uint32_t* scales, hipStream_t s);
hipError_t launch_convert_h(const uint16_t* h, int N, int H, const uint32_t* scales, uint16_t* h16, int hrows,
                              hipStream_t s);
// The chunk's W16 again with 2^kw when its recorded largest |W_s| (wmag) is out of band; else nothing.
// W_chunk: the chunk's first row of W_s; rows valid rows, ntv * 256 rows written (zeros past rows).
hipError_t launch_w_rescale(const uint16_t* W_chunk, int rows, int ntv, int H, const uint32_t* wmag, uint16_t* w16,
                            hipStream_t s);
hipError_t launch_dw(const DwParams& p, hipStream_t s);
hipError_t launch_dh(const DhParams& p, hipStream_t s);
hipError_t launch_dh_reduce(const DhParams& p, hipStream_t s);
// merged != NULL: the unfinalised (m_s, S_s, A, m_t, S_t) planes instead of loss / stats
hipError_t launch_fwd_rows_logits(const float* z_s, const float* z_t, const int32_t* z_rows, int z_nrows, int N, int V,
                                  const uint8_t* row_mask, float* loss, float* stats, float* merged, hipStream_t s);
hipError_t launch_bwd_rows_logits(const float* z_s, const float* z_t, const int32_t* z_rows, int z_nrows, int N, int V,
                                  const uint8_t* row_mask, const float* grad, const float* stats, float* dz,
                                  hipStream_t s);
hipError_t launch_compact(const uint8_t* mask, int T, int32_t* row_idx, int32_t* n_out, hipStream_t s);
// Rows grouped by teacher id (stable; ids outside [0, K) last); K in [1, 31].
hipError_t launch_group_by_teacher(const int32_t* teacher, const uint8_t* mask, int N, int K, int32_t* perm,
                                   int32_t* teacher_p, uint8_t* mask_p, hipStream_t s);
hipError_t launch_gather(const void* src, int64_t row_bytes, const int32_t* row_idx, int64_t N, void* dst,
                         hipStream_t s);
hipError_t launch_scatter(const void* src, int64_t row_bytes, const int32_t* row_idx, int64_t N, void* dst,
                          hipStream_t s);
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s);

}  // namespace rkl
