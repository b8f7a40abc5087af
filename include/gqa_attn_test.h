/*
 * gqa_attn_test.h - kernel selection for tests of the bf16 / fp16 prefill.
 *
 * The library has two bf16 / fp16 prefill kernels that compute the same
 * result (the forward of include/gqa_attn.h, attn_fwd and attn_prefill_paged)
 * and picks one by shape: a ping-pong kernel of 8 waves and 256 (query, head)
 * rows per workgroup for grids that give every compute unit a workgroup, and
 * a four-wave kernel of 128 rows per workgroup otherwise.  These two entry
 * points take the choice as an argument so that tests can run every shape on
 * both kernels.  Everything else (arguments, layouts, ownership, errors) is
 * that of the call they extend.
 *
 *   kernel  0 = the library's choice by shape (the plain call),
 *           1 = the ping-pong kernel,
 *           2 = the four-wave kernel;
 *           any other value returns GQA_ERR_INVALID_ARG.
 * dtype F32 always runs the fp32 kernel; `kernel` is then checked but unused.
 */
#ifndef GQA_ATTN_TEST_H
#define GQA_ATTN_TEST_H

#include "gqa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

gqa_status_t attn_fwd_with_kernel(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                                  float scale, int causal, gqa_dtype_t dtype, int kernel, void* hip_stream);

gqa_status_t attn_prefill_paged_with_kernel(const void* q, const void* k_cache, const void* v_cache, void* o,
                                            float* lse, const int* qo_indptr, const int* kv_indptr,
                                            const int* kv_indices, const int* kv_last_page_len, int B, int Hq,
                                            int Hkv, int D, int page_size, int max_q_len, float scale, int causal,
                                            gqa_dtype_t dtype, int kernel, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_TEST_H */
