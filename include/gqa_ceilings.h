/*
 * gqa_ceilings.h - measurement kernels (not attention): measured ceilings
 * that the benchmark reports beside the published MI355X peaks.
 *
 * Conventions of gqa_attn.h: device pointers owned by the caller, work
 * enqueued on `hip_stream` (NULL = default stream), nothing allocated or
 * synchronised.  Return 0 on success, 1 for an invalid argument (nothing
 * launched), 4 when the HIP runtime reports a launch error.
 */
#ifndef GQA_CEILINGS_H
#define GQA_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * MFMA-only loop: n_workgroups workgroups of 8 wave64s (two waves per SIMD,
 * one workgroup per compute unit, the occupancy of the ping-pong prefill
 * kernel); each wave issues iters x 16 v_mfma_f32_32x32x16_bf16 on four
 * independent register accumulators, with no memory access inside the loop.
 *   out  [n_workgroups * 512] float32, written (the accumulators' sums, so
 *        that no work is optimised away; the values carry no meaning).
 * gqa_ceiling_mfma_flops() is the algorithmic flop count of one launch
 * (2 * 32 * 32 * 16 per MFMA); 0 for non-positive arguments.
 */
long long gqa_ceiling_mfma_flops(int n_workgroups, int iters);
int gqa_ceiling_mfma(int n_workgroups, int iters, float* out, void* hip_stream);

/*
 * Streaming read: every 16-byte word of src [bytes] read once (grid-stride
 * over n_workgroups workgroups of 256 threads, non-temporal loads), folded
 * into out [n_workgroups] uint32 (written).  bytes must be a positive
 * multiple of 16 and src 16-byte aligned.
 */
int gqa_ceiling_stream_read(const void* src, size_t bytes, int n_workgroups, uint32_t* out, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_CEILINGS_H */
