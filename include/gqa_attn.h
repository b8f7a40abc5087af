/*
 * gqa_attn.h - C ABI of the MI355X (gfx950) GQA attention forward library.
 *
 * The forward pass of softmax attention with grouped query heads, prefill and
 * split-K decode, and the backward of the split-K merge:
 *
 *   attn_fwd            prefill / general forward, FlashAttention style
 *                       (causal_forward_kernel.py, `_flash_attention_forward_gqa_kernel`
 *                       and its wrapper `flash_attention_forward`).
 *   attn_fwd_split      the same with the keys split into ranges and merged (small grids).
 *   attn_prefill_paged  the same forward for a batch of ragged requests whose
 *                       keys live in a paged KV cache (the FlashInfer-style
 *                       prefill page gpt-o3 / triton6fd1ef, `run` and
 *                       `_gqa_prefill_kernel`).
 *   attn_decode_splitk  one query per sequence against a (paged) KV cache,
 *                       split along the keys and merged through the
 *                       per-chunk log-sum-exp (splitk_kernels.py,
 *                       `_fwd_kernel_splitK` and `_splitK_reduce`).
 *   attn_decode_splitk_fp8
 *                       the same over an 8-bit float (E4M3) KV cache with a
 *                       binary16 scale and shift per token row and K/V head
 *                       (the FP8_QUANTIZED case of `_fwd_kernel_splitK`).
 *   attn_decode_splitk_multi
 *                       the same with q_len queries per sequence at its last
 *                       positions, causal among themselves (the IS_CAUSAL /
 *                       NUM_QUERIES_CAUSAL case of `_fwd_kernel_splitK`).
 *   attn_fwd_bias, attn_decode_splitk_bias
 *                       prefill / decode with an additive attention bias (the
 *                       HAS_ADDITIVE_BIAS case of `_fwd_kernel_splitK`).
 *   attn_splitk_merge_backward
 *                       gradients of the split-K merge with respect to the
 *                       partial results (`_splitK_reduce_varargs_backward`).
 *   attn_decode_splitk_noalloc
 *                       attn_decode_splitk with the library's own fixed scratch
 *                       instead of a workspace, for callers that cannot allocate.
 *
 * What is computed, for batch b, query head h, query row i:
 *   g      = h / (Hq / Hkv)                       (query head -> K/V head)
 *   s_j    = scale * <q[b,h,i,:], k[b,g,j,:]>
 *   vis(i) = { j < kv_len : !causal || j <= i + (kv_len - q_len) }
 *            (bottom-right aligned causal mask, as in the FlashInfer-style
 *             prefill page gpt-o3 / triton6fd1ef, `_gqa_prefill_kernel`)
 *   lse    = log( sum_{j in vis(i)} exp(s_j) )    (natural log, scale included)
 *   o      = sum_{j in vis(i)} exp(s_j - lse) * v[b,g,j,:]
 * A row with no visible key gets o = 0 and lse = -inf (the zero-fill rule of
 * `_fwd_kernel_splitK`).  Accumulation is in fp32; o is rounded to nearest
 * even into the input dtype; lse is fp32.  For fp16/bf16 inputs the softmax
 * weights are rounded to the input dtype before the P.V product, as in both
 * the causal_forward_kernel.py and splitk_kernels.py kernels.
 *
 * Conventions shared by every call:
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates, frees and synchronises nothing; it only enqueues kernels.
 *   - Work is ordered on `hip_stream` (a hipStream_t; NULL = default stream)
 *     and is asynchronous: outputs are valid once the stream reaches it.
 *   - Arguments are validated before any launch; on error nothing is
 *     launched and outputs are untouched.  No exception crosses the ABI.
 *   - Outputs must not alias inputs.
 *   - Tensors are contiguous, row-major, in the layouts given per call.
 *   - The library holds no mutable global state apart from the per-device
 *     address of the fixed scratch of attn_decode_splitk_noalloc; calls from
 *     several host threads on different streams are safe, except
 *     overlapping attn_decode_splitk_noalloc calls on one GPU.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_F32 = 0,   /* IEEE binary32 */
    GQA_F16 = 1,   /* IEEE binary16 */
    GQA_BF16 = 2   /* bfloat16 */
} gqa_dtype_t;

typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1,  /* null pointer, bad size or geometry */
    GQA_ERR_UNSUPPORTED = 2,  /* valid request with no instantiated kernel (e.g. D not in {64,128}) */
    GQA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than attn_decode_workspace_bytes() */
    GQA_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} gqa_status_t;

/*
 * attn_fwd - attention forward (prefill, or any q_len).
 *
 *   q   [B, Hq,  q_len,  D]  dtype        (read)
 *   k   [B, Hkv, kv_len, D]  dtype        (read)
 *   v   [B, Hkv, kv_len, D]  dtype        (read)
 *   o   [B, Hq,  q_len,  D]  dtype        (written)
 *   lse [B, Hq,  q_len]      float32      (written; natural-log LSE)
 *
 * Requirements: B, q_len, kv_len >= 0; Hq, Hkv > 0; Hq % Hkv == 0 (the group
 * divisibility check of `flash_attention_forward`); D in {64, 128}; scale
 * finite (the usual value is 1/sqrt(D)).  dtype F32 runs an fp32 path with
 * fp32 softmax weights; F16/BF16 run the matrix-core path.
 * causal != 0 applies the bottom-right mask above; with q_len == kv_len it is
 * the usual lower-triangular mask.
 * B == 0 or q_len == 0: nothing to do, returns GQA_OK.
 * kv_len == 0 (or causal rows before the offset): o = 0, lse = -inf.
 * Returns GQA_ERR_INVALID_ARG / GQA_ERR_UNSUPPORTED / GQA_ERR_HIP or GQA_OK.
 *
 * Small grids: attn_fwd runs one pass over the keys per block of 256 (query,
 * head) rows.  When B * Hq * q_len / 256 is below the number of compute units
 * (e.g. one sequence of 1024 queries with 32 heads: 128 blocks on 256 CUs),
 * part of the chip idles.  For such shapes call attn_fwd_kv_splits(); if it
 * returns n > 1, attn_fwd_split() with n key ranges and a workspace of
 * attn_fwd_split_workspace_bytes() bytes computes the same result faster
 * (about 1.3x on that example).
 */
gqa_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                      float scale, int causal, gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_fwd_bias - attn_fwd with an additive attention bias: the
 * HAS_ADDITIVE_BIAS case of splitk_kernels.py (`_fwd_kernel_splitK` loads a
 * block of a strided bias tensor per tile and adds it to the scaled scores).
 *
 *   s_j    = scale * <q[b,h,i,:], k[b,g,j,:]> + bias(b, h, i, j)
 *   bias(b, h, i, j) = bias[b * bias_stride_b + h * bias_stride_h + i * bias_stride_q + j]
 *
 * then the softmax, output and LSE of attn_fwd over the visible keys (the
 * causal flag still applies).  The bias is in the softmax's natural units (a
 * bias of log w multiplies a key's weight by w), stored in `dtype` (F16 or
 * BF16), keys contiguous; strides are in elements, >= 0, and a stride of 0
 * broadcasts over that dimension (e.g. one [q_len, kv_len] bias for every
 * batch entry and head).  A bias of -inf masks a key; a row whose visible keys
 * are all masked gets o = 0, lse = -inf.  +inf or NaN biases are undefined.
 *
 *   bias  device memory, read only at (b, h, i, j) with j < kv_len; 2-byte
 *         aligned.  With D = 128, kv_len a multiple of 64, bias 16-byte
 *         aligned and all strides multiples of 8, the ping-pong kernel runs
 *         (the bias of a 64-key tile reaches LDS by direct loads beside the
 *         K/V tile); otherwise the four-wave kernel (rows that start 8-byte
 *         aligned, i.e. all strides multiples of 4 and bias 8-byte aligned,
 *         are read four keys at a time).
 *
 * Other arguments, layouts and results as attn_fwd; dtype F32 returns
 * GQA_ERR_UNSUPPORTED.
 */
gqa_status_t attn_fwd_bias(const void* q, const void* k, const void* v, const void* bias, long long bias_stride_b,
                           long long bias_stride_h, long long bias_stride_q, void* o, float* lse, int B, int Hq,
                           int Hkv, int q_len, int kv_len, int D, float scale, int causal, gqa_dtype_t dtype,
                           void* hip_stream);

/*
 * attn_fwd_split - the same forward with the keys of every block of query rows
 * cut into kv_splits contiguous ranges processed in parallel, then merged: the
 * split-K partition and LSE merge of splitk_kernels.py (`_fwd_kernel_splitK`
 * writes a partial output and its LSE per key range, `_splitK_reduce` merges
 * them: M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s,
 * LSE = M + log sum w_s), applied to prefill so that shapes with fewer blocks
 * of query rows than compute units still fill the chip.
 *
 * Arguments and results as attn_fwd (results equal up to rounding order),
 * plus:
 *   kv_splits  >= 1 key ranges per block of rows (1: exactly attn_fwd;
 *              at most 64).  Ranges hold whole 64-key tiles; a range can be
 *              empty, and a row that sees no key of a range gives it
 *              (O_s, LSE_s) = (0, -inf).
 *   workspace  device memory owned by the caller, 16-byte aligned, at least
 *              attn_fwd_split_workspace_bytes(B, Hq, q_len, D, kv_splits) bytes
 *              (fp32 partial outputs [B, Hq, q_len, kv_splits, D], then fp32
 *              partial LSEs [B, Hq, q_len, kv_splits]); its contents on entry
 *              do not matter and are undefined afterwards.  Unused when
 *              kv_splits == 1 (may be NULL).
 * dtype F16 or BF16 when kv_splits > 1 (F32: GQA_ERR_UNSUPPORTED).
 * Returns GQA_ERR_WORKSPACE when the workspace is missing, misaligned or too
 * small, otherwise as attn_fwd.  Two launches on hip_stream (ranges, merge).
 */
size_t attn_fwd_split_workspace_bytes(int B, int Hq, int q_len, int D, int kv_splits);
gqa_status_t attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int q_len, int kv_len, int D, float scale, int causal,
                            int kv_splits, void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                            void* hip_stream);

/*
 * attn_fwd_kv_splits - the key-range count the library recommends for
 * attn_fwd_split on this shape on the current device: for F16/BF16 with
 * kv_len >= 2048, as many ranges as fit one workgroup of 256 (query, head) rows
 * per compute unit (CU count / blocks of rows, rounded down, and twice that
 * for causal shapes with kv_len - q_len < q_len when it is at least 2; at most
 * kv_len / 512 so that each range keeps >= 8 key tiles, at most 8); 1 when
 * that is 1 or the shape does not qualify (call attn_fwd).  Host-only; reads
 * the device's CU count.
 */
int attn_fwd_kv_splits(int B, int Hq, int Hkv, int q_len, int kv_len, int D, int causal, gqa_dtype_t dtype);

/*
 * attn_prefill_paged - attention forward for a batch of B ragged requests over
 * a paged KV cache (the FlashInfer-style prefill page, `run`: query tokens
 * located by qo_indptr, key pages by kv_indptr / kv_indices).
 *
 *   q         [total_q, Hq, D]  dtype  (read; token-major, total_q = qo_indptr[B])
 *   o         [total_q, Hq, D]  dtype  (written)
 *   lse       [total_q, Hq]     float32 (written; natural log)
 *   k_cache, v_cache [num_pages, page_size, Hkv, D] dtype (read)
 *   qo_indptr [B + 1] int32: request b owns query tokens [qo_indptr[b], qo_indptr[b+1])
 *   kv_indptr [B + 1] int32: request b owns the page ids
 *             kv_indices[kv_indptr[b] .. kv_indptr[b+1]) (n_b pages, in key order)
 *   kv_indices [kv_indptr[B]] int32: page ids into the pool
 *   kv_last_page_len [B] int32 or NULL: keys in request b's last page
 *             (1..page_size); NULL means every page is full.  Request b has
 *             kv_len_b = (n_b - 1) * page_size + kv_last_page_len[b] keys
 *             (0 when n_b = 0); its key t is row t % page_size of page
 *             kv_indices[kv_indptr[b] + t / page_size].
 *   max_q_len  an upper bound of every request's query count (host value; it
 *             sizes the launch; rows of a longer request would not be computed).
 *
 * Query i of request b sees key t iff !causal or t <= i + kv_len_b - q_len_b
 * (bottom-right per request, as the page's mask kv_allowed = q_idx + 1 + delta);
 * a query with no visible key, and every query of a request without keys, gets
 * o = 0, lse = -inf.  Requests with no queries produce nothing.
 *
 * The contents of the three pointer arrays and of kv_last_page_len are trusted
 * (not bounds-checked on the device); an inconsistent table is undefined
 * behaviour.
 *
 * Requirements: B >= 0, Hq, Hkv > 0, Hq % Hkv == 0, D in {64, 128}, dtype F16
 * or BF16, page_size a power of two, max_q_len >= 0, scale finite and > 0.
 * B == 0 or max_q_len == 0 returns GQA_OK without launching.
 * Returns GQA_ERR_INVALID_ARG / GQA_ERR_UNSUPPORTED / GQA_ERR_HIP or GQA_OK.
 */
gqa_status_t attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                const int* qo_indptr, const int* kv_indptr, const int* kv_indices,
                                const int* kv_last_page_len, int B, int Hq, int Hkv, int D, int page_size,
                                int max_q_len, float scale, int causal, gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_decode_workspace_bytes - device workspace attn_decode_splitk needs:
 * B * Hq * n_splits * (D + 1) * 4 bytes (per-chunk fp32 outputs and LSEs).
 * Returns 0 for non-positive arguments.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int n_splits);

/*
 * attn_decode_splitk - single-query attention per sequence, split-K.
 *
 *   q           [B, Hq, D]         dtype    (read; one query per sequence and head)
 *   o           [B, Hq, D]         dtype    (written)
 *   lse         [B, Hq]            float32  (written; natural log)
 *   seq_lens    [B]                int32    (read; 0 <= seq_lens[b] <= max_kv_len)
 *   block_table != NULL: paged KV cache
 *       k, v        [num_pages, page_size, Hkv, D] dtype
 *       block_table [B, max_pages_per_seq] int32; token t of sequence b lives in
 *                   page block_table[b * max_pages_per_seq + t / page_size],
 *                   row t % page_size (the paged branch of `_fwd_kernel_splitK`).
 *       page_size must be a power of two; max_pages_per_seq * page_size >= max_kv_len.
 *   block_table == NULL: dense cache
 *       k, v        [B, Hkv, max_kv_len, D] dtype; rows >= seq_lens[b] are ignored.
 *       page_size and max_pages_per_seq are ignored.
 *   workspace   >= attn_decode_workspace_bytes(B, Hq, D, n_splits) bytes of device
 *               memory, 16-byte aligned, used as scratch for the per-chunk
 *               results; its contents before and after the call are unspecified.
 *
 * Sequence b is cut into n_splits chunks of ceil(ceil(seq_lens[b]/n_splits)/64)*64
 * tokens (trailing chunks may be empty); each chunk yields a partial output and
 * its LSE, and a second kernel merges the chunks with weights exp(lse_s - max)
 * (`_splitK_reduce`).  The result does not depend on n_splits beyond rounding.
 * seq_lens[b] == 0 gives o = 0, lse = -inf.
 *
 * The contents of seq_lens and block_table are trusted: they are not
 * bounds-checked on the device, and an out-of-range page id or length is
 * undefined behaviour (the split-K page loads its block table unchecked too).
 *
 * Requirements: B >= 0, Hq, Hkv > 0, Hq % Hkv == 0,
 * D in {64, 128}, dtype F16 or BF16, 1 <= n_splits <= 256, max_kv_len >= 0.
 * B == 0 returns GQA_OK without launching.
 */
gqa_status_t attn_decode_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* seq_lens, const int* block_table,
                                int max_pages_per_seq, int page_size,
                                int B, int Hq, int Hkv, int D, int max_kv_len,
                                float scale, int n_splits,
                                void* workspace, size_t workspace_bytes,
                                gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_decode_splitk_fp8 - single-query split-K decode over an 8-bit float KV
 * cache.  splitk_kernels.py, `_fwd_kernel_splitK` with FP8_QUANTIZED: every
 * element of K and V is one OCP E4M3 byte (sign, 4-bit exponent with bias 7,
 * 3-bit fraction, no infinities, S.1111.111 = NaN: the 8-bit float format of
 * gfx950), and every (token row, K/V head) has a uint32 scale-shift word with a
 * binary16 scale in bits 0-15 and a binary16 shift in bits 16-31
 * (`cast_uint32_to_half2`).  The key / value used is byte * scale + shift
 * (`dequantize`); the rest is attn_decode_splitk.
 *
 *   q, o        [B, Hq, D]   dtype (F16 or BF16)
 *   lse         [B, Hq]      float32 (natural log)
 *   k_cache, v_cache  uint8 E4M3, paged [num_pages, page_size, Hkv, D] with
 *               block_table, or dense [B, Hkv, max_kv_len, D] without
 *   k_scale_shift, v_scale_shift  uint32, [num_pages, page_size, Hkv] (paged)
 *               or [B, Hkv, max_kv_len] (dense); 4-byte aligned
 *   seq_lens, block_table, max_pages_per_seq, n_splits, workspace: as for
 *               attn_decode_splitk (workspace >= attn_decode_workspace_bytes()).
 *
 * Requirements: those of attn_decode_splitk; a paged cache needs page_size >= 16
 * (GQA_ERR_UNSUPPORTED otherwise).  The contents of the cache, the scale-shift
 * words, seq_lens and block_table are trusted, as for attn_decode_splitk.
 */
gqa_status_t attn_decode_splitk_fp8(const void* q, const void* k_cache, const void* v_cache,
                                    const uint32_t* k_scale_shift, const uint32_t* v_scale_shift,
                                    void* o, float* lse, const int* seq_lens, const int* block_table,
                                    int max_pages_per_seq, int page_size, int B, int Hq, int Hkv, int D,
                                    int max_kv_len, float scale, int n_splits, void* workspace,
                                    size_t workspace_bytes, gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_decode_workspace_bytes_multi - device workspace attn_decode_splitk_multi
 * needs: B * Hq * q_len * n_splits * (D + 1) * 4 bytes.  Returns 0 for
 * non-positive arguments.  attn_decode_workspace_bytes(B, Hq, D, n) equals
 * attn_decode_workspace_bytes_multi(B, Hq, 1, D, n).
 */
size_t attn_decode_workspace_bytes_multi(int B, int Hq, int q_len, int D, int n_splits);

/*
 * attn_decode_splitk_multi - several queries per sequence (speculative or
 * chunked decode), split-K.  splitk_kernels.py, `_fwd_kernel_splitK` with
 * IS_CAUSAL and NUM_QUERIES_CAUSAL: the q_len queries of sequence b are its
 * last q_len positions, so query i (0 <= i < q_len) sees the keys
 *     t <= seq_lens[b] - q_len + i
 * (query q_len - 1 sees all seq_lens[b] keys; a query placed before the first
 * key sees none and gets o = 0, lse = -inf).
 *
 *   q           [B, Hq, q_len, D]   dtype    (read)
 *   o           [B, Hq, q_len, D]   dtype    (written)
 *   lse         [B, Hq, q_len]      float32  (written; natural log)
 *   seq_lens, block_table, k, v, page_size, max_pages_per_seq, max_kv_len:
 *               as for attn_decode_splitk (seq_lens[b] counts the keys of
 *               sequence b, including those of its q_len query positions).
 *   workspace   >= attn_decode_workspace_bytes_multi(B, Hq, q_len, D, n_splits)
 *               bytes of device memory, 16-byte aligned, contents unspecified
 *               before and after the call.
 *
 * The chunking is that of attn_decode_splitk (it depends on seq_lens[b] only);
 * a chunk that holds no key visible to a query contributes weight 0 to it.
 * With q_len == 1 the call is attn_decode_splitk.
 *
 * Requirements: those of attn_decode_splitk, and 1 <= q_len <= 256,
 * B * Hq * q_len < 2^31.  Errors as for attn_decode_splitk.
 */
gqa_status_t attn_decode_splitk_multi(const void* q, const void* k, const void* v, void* o, float* lse,
                                      const int* seq_lens, const int* block_table,
                                      int max_pages_per_seq, int page_size,
                                      int B, int Hq, int Hkv, int q_len, int D, int max_kv_len,
                                      float scale, int n_splits,
                                      void* workspace, size_t workspace_bytes,
                                      gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_decode_splitk_bias - attn_decode_splitk_multi with an additive
 * attention bias: the HAS_ADDITIVE_BIAS case of splitk_kernels.py
 * (`_fwd_kernel_splitK` adds a strided bias block to the scaled scores).
 * Query i of sequence b and head h scores key t as
 *
 *   s = scale * <q[b,h,i,:], k_t> + bias[b * bias_stride_b + h * bias_stride_h + i * bias_stride_q + t]
 *
 * with the visibility, merge and results of attn_decode_splitk_multi (q_len
 * = 1 is plain decode).  The bias is in the softmax's natural units, stored
 * in `dtype` (F16 / BF16), keys contiguous; -inf masks a key (a query whose
 * visible keys are all masked gets o = 0, lse = -inf).
 *
 *   bias  device memory, 4-byte aligned; strides in elements, >= 0 and even
 *         (0 broadcasts).  Keys are read in pairs: every bias row used must be
 *         readable up to key seq_lens[b] rounded up to an even count (a row
 *         of an odd length needs one more element, e.g. a padded row stride).
 *
 * Other arguments, layouts, errors and the workspace
 * (attn_decode_workspace_bytes_multi) as for attn_decode_splitk_multi.
 */
gqa_status_t attn_decode_splitk_bias(const void* q, const void* k, const void* v, const void* bias,
                                     long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                                     void* o, float* lse, const int* seq_lens, const int* block_table,
                                     int max_pages_per_seq, int page_size, int B, int Hq, int Hkv, int q_len, int D,
                                     int max_kv_len, float scale, int n_splits, void* workspace,
                                     size_t workspace_bytes, gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_decode_splitk_noalloc - attn_decode_splitk without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * The per-chunk partial outputs and LSEs go to a fixed array of 32 MiB in the
 * library's device code object instead of a caller workspace: each GPU the
 * library runs on holds its own copy until the process ends; its address is
 * looked up once per device (with that device current) on the first call.
 * The call itself allocates nothing.  Every other argument, layout and result
 * is that of attn_decode_splitk; the result is bitwise the same.
 *
 * Limit: attn_decode_workspace_bytes(B, Hq, D, n_splits) must not exceed
 * 32 MiB (33554432 bytes: at D = 128 with 32 heads and 16 chunks, up to 127
 * sequences);
 * larger requests return GQA_ERR_WORKSPACE before any HIP call.
 * The array is shared by every call on one GPU and keeps the last call's
 * contents (nothing in it has to start at zero: each chunk's partial is
 * written before the merge reads it).  Calls that overlap in time on one GPU
 * (several streams, or several host threads) race on it and give undefined
 * results: order them on one stream, or use attn_decode_splitk with a
 * workspace per stream.  hip_stream must belong to the current device.
 * Returns GQA_ERR_HIP if the array's address cannot be obtained.
 */
gqa_status_t attn_decode_splitk_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int* seq_lens, const int* block_table,
                                        int max_pages_per_seq, int page_size,
                                        int B, int Hq, int Hkv, int D, int max_kv_len,
                                        float scale, int n_splits, gqa_dtype_t dtype, void* hip_stream);

/*
 * attn_splitk_merge_backward - gradients of the split-K merge with respect to
 * the partial results (splitk_kernels.py, `_splitK_reduce_varargs_backward`,
 * the backward of `_splitK_reduce`).  Per row, the forward merge of n_splits
 * partials (O_s, L_s) is O = sum_s w_s O_s, L = log sum_s exp(L_s), with
 * w_s = exp(L_s - L); given (O, L) and the gradients (dO, dL) of some scalar
 * with respect to them:
 *
 *   dO_s = w_s * dO
 *   dL_s = w_s * (dL + sum_d (O_s[d] - O[d]) * dO[d])
 *
 * A partial with L_s = -inf (an empty chunk), and every partial of a row with
 * L = -inf, gets dO_s = 0, dL_s = 0.
 *
 *   o_parts     [rows, n_splits, D] float32   (read; the layout of the decode
 *   lse_parts   [rows, n_splits]    float32    workspace's partials)
 *   o, d_o      [rows, D]           float32   (read; merged output and its gradient)
 *   lse, d_lse  [rows]              float32   (read; natural-log LSE and its gradient)
 *   d_o_parts   [rows, n_splits, D] float32   (written)
 *   d_lse_parts [rows, n_splits]    float32   (written)
 *
 * All device pointers, 4-byte aligned, owned by the caller; outputs must not
 * alias inputs.  1 <= n_splits <= 65536, 1 <= D <= 512, 0 <= rows < 2^36.
 * With D a multiple of 4 and o_parts, o, d_o, d_o_parts 16-byte aligned the
 * rows move in 16-byte pieces (faster); any other case one float per lane.
 * rows == 0 returns GQA_OK without launching.  Arithmetic in fp32.
 * Returns GQA_ERR_INVALID_ARG / GQA_ERR_HIP or GQA_OK.
 */
gqa_status_t attn_splitk_merge_backward(const float* o_parts, const float* lse_parts, const float* o,
                                        const float* lse, const float* d_o, const float* d_lse, float* d_o_parts,
                                        float* d_lse_parts, long long rows, int n_splits, int D, void* hip_stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* attn_status_str(gqa_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
