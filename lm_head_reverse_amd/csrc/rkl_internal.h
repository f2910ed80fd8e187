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
  const float* z_t;        // teacher logits [N, V] (teacher-logits payload)
  const int32_t* y;        // sampled token per row (log-probability / entropy)
  const int32_t* teacher;  // teacher per row (NULL: one teacher)
  int K;                   // teachers: W_t holds K weights, wt_stride elements apart
  int64_t wt_stride;
  float* partial;          // [nsplit][5][N]
  int tiles_per_split;     // 256-row vocabulary tiles per split
  int nsplit;
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
  const uint8_t* row_mask;
  const float* grad;       // g of L (reverse KL) or of log p(y) (log-probability / entropy)
  const float* grad_h;     // g of the entropy (log-probability / entropy)
  const int32_t* y;        // sampled token per row (log-probability / entropy)
  const int32_t* teacher;  // teacher per row (NULL: one teacher)
  int K;
  int64_t wt_stride;
  const float* stats;
  const float* gscale;     // [2]: s, 1/s (powers of two); dz is stored as fp16(s * dz)
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
};

struct DwParams {
  const float* gscale;
  const uint16_t* dz;
  int ldz, N, kpad, width;
  const uint16_t* hT;      // [H, ldT] fp16
  int ldT, H;
  float* dW;               // dW_s + c0 * H
  int accumulate;
  int ntm, ntn;
};

struct DhParams {
  const float* gscale;
  const uint16_t* dz;
  int ldz, N, npad, kpad, width;   // npad: dz workspace rows
  int c0;                          // first vocabulary column of the chunk
  const uint16_t* w16;     // fp16 copy of the W_s chunk [>= kpad rows, H]
  int H;
  float* dh;
  int accumulate;
  int ntm, ntn;
  int panel;               // column tiles per panel of the workgroup order
};

// Tile sizes the host needs for grids and workspace.
constexpr int kFwdTileV = 256;
constexpr int kFwdTileN = 128;
constexpr int kDwTileM = 256, kDwTileN = 256;
constexpr int kDhTileM = 256, kDhTileN = 128;
// dh's fp32 sum over the vocabulary is split at multiples of this column
// index (absolute), whatever the backward's chunk width.
constexpr int kDhSegment = 65536;

// What the fused kernels compute.
enum Mode : int {
  kModeHidden = 0,          // reverse KL, teacher projected from hidden states
  kModeTeacherLogits = 1,   // reverse KL, teacher logits streamed
  kModeLogprobEntropy = 2,  // log p(sampled token) and entropy of one projection
  kModeHiddenTeachers = 3,  // reverse KL, teacher hidden states, teacher chosen per row
};

hipError_t launch_fwd_tiles(const FwdParams& p, int mode, int waves, hipStream_t s);
// out0: loss (reverse KL) or log p(y); out1: entropy (log-probability / entropy only)
hipError_t launch_fwd_combine(const float* partial, int nsplit, int N, const uint8_t* row_mask, bool logprob_entropy,
                              float* out0, float* out1, float* stats, hipStream_t s);
// The splits' merged (m_s, S_s, A, m_t, S_t), not finalised: five planes of N.
hipError_t launch_fwd_merge(const float* partial, int nsplit, int N, float* merged, hipStream_t s);
hipError_t launch_bwd_dz(const BwdParams& p, int mode, int waves, hipStream_t s);
hipError_t launch_grad_scale(const float* grad, const float* grad_h, const uint8_t* row_mask, const float* stats,
                             int N, bool logprob_entropy, float* out, hipStream_t s);
hipError_t launch_transpose_h(const uint16_t* h, int N, int H, uint16_t* hT, int ldT, hipStream_t s);
hipError_t launch_dw(const DwParams& p, int waves, hipStream_t s);
hipError_t launch_dh(const DhParams& p, int waves, hipStream_t s);
// merged != NULL: the unfinalised (m_s, S_s, A, m_t, S_t) planes instead of loss / stats
hipError_t launch_fwd_rows_logits(const float* z_s, const float* z_t, int N, int V, const uint8_t* row_mask,
                                  float* loss, float* stats, float* merged, hipStream_t s);
hipError_t launch_bwd_rows_logits(const float* z_s, const float* z_t, int N, int V, const uint8_t* row_mask,
                                  const float* grad, const float* stats, float* dz, hipStream_t s);
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
