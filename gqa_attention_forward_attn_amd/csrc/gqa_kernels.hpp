// gqa_kernels.hpp - host-visible launch interface of the HIP kernels (internal
// to the library; the public ABI is include/gqa_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeF16 = 1;
constexpr int kDtypeBF16 = 2;

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, q_len, kv_len;
    int group;        // Hq / Hkv
    int delta;        // kv_len - q_len (bottom-right causal offset)
    int n_pos_tiles;  // filled by the launcher
    int n_rest;       // filled by the launcher
    int xcd_order;    // ping-pong kernel, dense: XCD-aware work order (filled by the launcher)
    float c;          // scale * log2(e)
    // Split-KV prefill (ping-pong kernel): the key tiles of every row block are
    // cut into kv_splits ranges; range s writes O_s (fp32) and its natural-base
    // LSE_s to part_o [B, Hq, q_len, kv_splits, D] / part_lse [B, Hq, q_len,
    // kv_splits], merged afterwards.  kv_splits = 1: the plain forward.
    int kv_splits;
    float* part_o;
    float* part_lse;
    // Ragged batch over a paged cache (paged prefill only): q, o token-major
    // [total_q, Hq, D], lse [total_q, Hq]; k, v [num_pages, page_size, Hkv, D].
    // q_len holds the largest per-request query count (sizes the grid).
    const int* qo_indptr;         // [B + 1]
    const int* kv_indptr;         // [B + 1] offsets into kv_indices
    const int* kv_indices;        // page ids
    const int* kv_last_page_len;  // [B] tokens in each last page, or nullptr (full pages)
    int page_shift;               // log2(page_size)
    // Additive bias (dense only): bias(b, h, i, j) =
    // bias[b * bias_sb + h * bias_sh + i * bias_sq + j] in the input dtype,
    // added to the scores in the softmax's natural units; bias_k = 1 / scale.
    const uint16_t* bias;
    long long bias_sb, bias_sh, bias_sq;
    float bias_k;
};

// bf16 / fp16 prefill kernel: chosen by shape, or forced (tests).
enum class PrefillKernel { kAuto, kPingPong, kFourWave };

// Validated arguments only.  D in {64, 128}; dtype one of kDtype*.
hipError_t launch_prefill(PrefillArgs a, int D, bool causal, int dtype, PrefillKernel kernel, hipStream_t stream);
// The same with the additive bias of a.bias (bf16 / fp16, four-wave kernel).
hipError_t launch_prefill_bias(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream);
// The same on the ping-pong kernel: D = 128, kv_len a multiple of 64, bias
// base and row strides 16-byte aligned (callers check).
hipError_t launch_prefill_pp_bias(PrefillArgs a, bool causal, int dtype, hipStream_t stream);
// Ragged batch of requests over a paged K/V cache (bf16 / fp16): the ping-pong
// kernel for batches that give every CU a workgroup, else the four-wave kernel
// (or the one `kernel` forces).
hipError_t launch_prefill_paged(PrefillArgs a, int D, bool causal, int dtype, PrefillKernel kernel, hipStream_t stream);
// The ping-pong kernel's paged mode.
hipError_t launch_prefill_pp_paged(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream);
// Ping-pong schedule, 8 waves x 32 rows (bf16 / fp16 only).
hipError_t launch_prefill_pp(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream);
// Split-KV prefill on the ping-pong kernel (a.kv_splits > 1 with part_o / part_lse
// set), then the merge into o / lse.
hipError_t launch_prefill_split(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream);
// Workgroups of the ping-pong kernel for this shape (one per 256 (query, head) rows).
long long prefill_pp_items(int B, int Hq, int Hkv, int q_len);

struct DecodeArgs {
    const void* q;            // [B, Hq, q_len, D]
    const void* k;            // paged [pages, page_size, Hkv, D] or dense [B, Hkv, max_kv_len, D]
    const void* v;
    void* o;                  // [B, Hq, q_len, D]
    float* lse;               // [B, Hq, q_len]
    const int* seq_lens;      // [B] keys per sequence (the q_len queries are its last positions)
    const int* block_table;   // [B, max_pages] or nullptr (dense)
    float* part_o;            // workspace [B, Hq, q_len, n_splits, D]
    float* part_lse;          // workspace [B, Hq, q_len, n_splits]
    int B, Hq, Hkv, D, group;
    int q_len;                // queries per sequence (1: plain decode)
    const uint32_t* k_ss;     // E4M3 cache only: per (token row, K/V head) binary16 scale (bits 0-15)
    const uint32_t* v_ss;     //   and shift (bits 16-31), laid out like the cache without D
    int max_pages;
    int page_shift;           // log2(page_size) (paged)
    int max_kv_len;           // dense row stride in tokens
    int n_splits;
    float c;                  // scale * log2(e)
    // Additive bias (16-bit cache only) or nullptr: query i of sequence b, head
    // h, key t gets bias[b * bias_sb + h * bias_sh + i * bias_sq + t] (input
    // dtype; even strides, 4-byte aligned); bias_k = 1 / scale.
    const uint16_t* bias;
    long long bias_sb, bias_sh, bias_sq;
    float bias_k;
};

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);

// The library's fixed device scratch (csrc/scratch.hip): its size, and the
// address of the current device's copy (looked up once per device).
size_t scratch_capacity_bytes();
hipError_t scratch_device_ptr(void** out);
// K/V as E4M3 bytes with scale-shift words (q_len = 1; pages of >= 16 tokens or dense).
hipError_t launch_decode_fp8(const DecodeArgs& a, int dtype, hipStream_t stream);

// Backward of the split-K merge (fp32): partials [rows, n_splits, D] and
// [rows, n_splits], merged results and their gradients [rows, D] and [rows].
struct MergeBwdArgs {
    const float* o_parts;
    const float* lse_parts;
    const float* o;
    const float* lse;
    const float* d_o;
    const float* d_lse;
    float* d_o_parts;
    float* d_lse_parts;
    long long rows;
    int n_splits, D;
};

int merge_backward_max_dims();
hipError_t launch_merge_backward(const MergeBwdArgs& a, hipStream_t stream);

}  // namespace gqa
