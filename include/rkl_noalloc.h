/*
 * rkl_noalloc.h -- an entry point of librkl.so that needs no workspace.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * hidden-state forward of rkl.h with its scratch -- the per-row partial
 * statistics of every vocabulary split -- held in a device array of the
 * library instead of a caller workspace.
 */
#ifndef RKL_NOALLOC_H
#define RKL_NOALLOC_H

#include "rkl.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device scratch the library holds per GPU (from its first use on
 * that GPU until the process ends). */
#define RKL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * rkl_forward_hidden without the workspace arguments: same inputs, outputs,
 * results (bit for bit) and errors.  It calls no hipMalloc or other
 * allocating routine; the first call on a device looks up that device's
 * scratch array.  Limit: 20 N nsplit bytes must fit in
 * RKL_NOALLOC_SCRATCH_BYTES, nsplit being the forward's vocabulary splits
 * (at most 200; 198 at V = 151936, so N <= 8473 there, and N <= 8388 fits
 * any V); larger calls return RKL_UNSUPPORTED with a message and launch
 * nothing.  Every call on a
 * GPU uses that GPU's one scratch array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race.
 * Nothing in the scratch needs clearing: each call writes every partial it
 * reads.
 */
int rkl_forward_hidden_noalloc(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s,
                               const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t, const uint8_t* row_mask,
                               float* loss, float* stats, rkl_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RKL_NOALLOC_H */
