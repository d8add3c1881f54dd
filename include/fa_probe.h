/*
 * fa_probe.h -- measurement probes for the attention kernels of libfa.so,
 * built as a library of their own (libfa_probe.so): they measure, on the
 * device the kernels run on, the two rates those kernels are bounded by, for
 * the benchmark's secondary ceilings.  They are not attention and are not
 * part of libfa.so.  Status codes are the fa_status values of fa.h.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The two rates, measured on the current device.  kind 0 = dense fp16 MFMA:
 * every thread's wave issues `iters` x 4 independent
 * v_mfma_f32_32x32x16_f16 (32,768 flops each) on register operands;
 * kind 1 = v_exp_f32: every thread runs `iters` x 8 independent base-2
 * exponentials (the softmax's exp2 on prescaled scores, "Triton
 * FlashAttention").  One launch of fa_probe_threads() threads (two waves per
 * SIMD on every compute unit) on `stream`; each thread writes one float to
 * sink[thread], a caller-owned device array of at least fa_probe_threads()
 * floats (the library allocates nothing).  Time the launch with events on
 * the same stream to get flops or exponentials per second.  Returns FA_OK,
 * FA_ERR_NULL (sink), FA_ERR_SHAPE (kind not 0 or 1, or iters < 1) or
 * FA_ERR_HIP.
 */
int fa_probe(int kind, int iters, float* sink, void* stream);
int64_t fa_probe_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
