/*
 * fa_ceilings.h -- measurement aids exported by libfa.so beside the attention
 * entry points of fa.h.  They measure what the GPU sustains for the two
 * resources the attention kernels are bound by, so that a kernel's throughput
 * can be read against a measured ceiling as well as against the published
 * peak.  Neither is part of the attention path.
 *
 * Both enqueue one kernel on `stream` (a hipStream_t, NULL = null stream) and
 * return 0, -1 for invalid arguments (checked before any HIP call) or -4 if
 * the launch failed.  Time them with events on the same stream.
 */
#ifndef FA_CEILINGS_H_
#define FA_CEILINGS_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_ceiling_mfma -- `blocks` work-groups of 256 threads (4 waves; two waves
 * share a SIMD) each issue `iters` x 32 dense bf16 matrix-core products
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on register operands, in four
 * independent accumulator chains, cycling through eight A and eight B
 * fragments per lane.  FLOP per launch = blocks * 4 * iters * 32 * 32768.
 * src: DEVICE bf16 operands, blocks * 16 * 256 * 8 values (16-byte aligned),
 * read once at the start -- random values draw the power real operands
 * draw, and the sustained clock (so the rate) depends on it -- or NULL for
 * small constant operands.  out: DEVICE float[blocks * 256], written.
 */
int fa_ceiling_mfma(const void* src, float* out, int blocks, int iters, void* stream);

/*
 * fa_ceiling_read -- `blocks` work-groups of 256 threads read `bytes` bytes at
 * `src` (DEVICE, 16-byte aligned, bytes a multiple of 16) once with 16-byte
 * nontemporal loads: each work-group streams its own contiguous run, eight
 * loads in flight per lane (units past the last whole run are read
 * grid-stride).  out: DEVICE unsigned[blocks * 256], written (an xor of what
 * each thread read).
 */
int fa_ceiling_read(const void* src, size_t bytes, unsigned* out, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_CEILINGS_H_ */
