// api.cpp - the extern "C" boundary declared in include/gqa_attn.h: argument
// validation (before any HIP call), instantiation choice and launch on the
// caller's stream.  No allocation, no synchronisation; the only global state
// is the per-device address of the fixed scratch array that
// attn_decode_splitk_noalloc uses (csrc/scratch.hip).
#include "gqa_attn.h"
#include "gqa_attn_test.h"

#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "gqa_kernels.hpp"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool supported_head_dim(int D) { return D == 64 || D == 128; }

bool valid_dtype(gqa_dtype_t t) { return t == GQA_F32 || t == GQA_F16 || t == GQA_BF16; }

int to_kernel_dtype(gqa_dtype_t t) {
    switch (t) {
    case GQA_F16: return gqa::kDtypeF16;
    case GQA_BF16: return gqa::kDtypeBF16;
    default: return gqa::kDtypeF32;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Kernel choice of the two bf16 / fp16 prefill kernels: 0 = by shape, 1 =
// ping-pong, 2 = four-wave (the *_with_kernel entry points of gqa_attn_test.h).
bool to_prefill_kernel(int kernel, gqa::PrefillKernel* out) {
    switch (kernel) {
    case 0: *out = gqa::PrefillKernel::kAuto; return true;
    case 1: *out = gqa::PrefillKernel::kPingPong; return true;
    case 2: *out = gqa::PrefillKernel::kFourWave; return true;
    default: return false;
    }
}

}  // namespace

extern "C" {

gqa_status_t attn_fwd_with_kernel(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                                  float scale, int causal, gqa_dtype_t dtype, int kernel, void* hip_stream) {
    gqa::PrefillKernel choice;
    if (!to_prefill_kernel(kernel, &choice)) return GQA_ERR_INVALID_ARG;
    if (B < 0 || q_len < 0 || kv_len < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_ERR_INVALID_ARG;
    if (!supported_head_dim(D)) return GQA_ERR_UNSUPPORTED;
    if (B == 0 || q_len == 0) return GQA_OK;
    if (!q || !o || !lse) return GQA_ERR_INVALID_ARG;
    if (kv_len > 0 && (!k || !v)) return GQA_ERR_INVALID_ARG;
    // 16-byte vector loads/stores need 16-byte aligned tensors
    if (!aligned16(q) || !aligned16(o) || (kv_len > 0 && (!aligned16(k) || !aligned16(v))))
        return GQA_ERR_INVALID_ARG;
    // rows and elements must fit the kernels' index arithmetic
    const long long rows_q = (long long)B * Hq * q_len;
    const long long rows_kv = (long long)B * Hkv * kv_len;
    if (rows_q > (1LL << 40) || rows_kv > (1LL << 40)) return GQA_ERR_INVALID_ARG;

    gqa::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.q_len = q_len; a.kv_len = kv_len;
    a.group = Hq / Hkv;
    a.delta = kv_len - q_len;
    a.c = scale * kLog2e;
    hipError_t e = gqa::launch_prefill(a, D, causal != 0, to_kernel_dtype(dtype), choice,
                                       static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int q_len, int kv_len, int D,
                      float scale, int causal, gqa_dtype_t dtype, void* hip_stream) {
    return attn_fwd_with_kernel(q, k, v, o, lse, B, Hq, Hkv, q_len, kv_len, D, scale, causal, dtype, 0,
                                hip_stream);
}

gqa_status_t attn_fwd_bias(const void* q, const void* k, const void* v, const void* bias, long long bias_stride_b,
                           long long bias_stride_h, long long bias_stride_q, void* o, float* lse, int B, int Hq,
                           int Hkv, int q_len, int kv_len, int D, float scale, int causal, gqa_dtype_t dtype,
                           void* hip_stream) {
    if (B < 0 || q_len < 0 || kv_len < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_ERR_INVALID_ARG;
    if (bias_stride_b < 0 || bias_stride_h < 0 || bias_stride_q < 0) return GQA_ERR_INVALID_ARG;
    if (!supported_head_dim(D) || dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;
    if (B == 0 || q_len == 0) return GQA_OK;
    if (kv_len == 0)  // no key: every row is (0, -inf), the bias is not read
        return attn_fwd_with_kernel(q, k, v, o, lse, B, Hq, Hkv, q_len, 0, D, scale, causal, dtype, 2, hip_stream);
    if (!q || !k || !v || !o || !lse || !bias) return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v)) return GQA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(bias) & 1u) return GQA_ERR_INVALID_ARG;
    const long long rows_q = (long long)B * Hq * q_len;
    const long long rows_kv = (long long)B * Hkv * kv_len;
    if (rows_q > (1LL << 40) || rows_kv > (1LL << 40)) return GQA_ERR_INVALID_ARG;

    gqa::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.q_len = q_len; a.kv_len = kv_len;
    a.group = Hq / Hkv;
    a.delta = kv_len - q_len;
    a.c = scale * kLog2e;
    a.bias = static_cast<const uint16_t*>(bias);
    a.bias_sb = bias_stride_b;
    a.bias_sh = bias_stride_h;
    a.bias_sq = bias_stride_q;
    a.bias_k = 1.f / scale;
    hipError_t e = gqa::launch_prefill_bias(a, D, causal != 0, to_kernel_dtype(dtype),
                                            static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_fwd_kv_splits(int B, int Hq, int Hkv, int q_len, int kv_len, int D, int causal, gqa_dtype_t dtype) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || q_len <= 0 || kv_len <= 0 || Hq % Hkv != 0) return 1;
    if (!supported_head_dim(D) || (dtype != GQA_BF16 && dtype != GQA_F16)) return 1;
    // Only where the ping-pong kernel would leave at least half of the CUs idle,
    // and only with enough keys that each range keeps a deep tile loop.
    if (kv_len < 2048) return 1;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
        return 1;
    // as many ranges as fit one workgroup per CU (rounded down: for blocks of
    // similar length a second round costs more than the idle CUs it would fill)
    const long long items = gqa::prefill_pp_items(B, Hq, Hkv, q_len);
    long long splits = n_cu / items;
    // causal with an offset below q_len: the blocks' key counts run from a few
    // tiles to all of them, and twice the ranges (a second, shorter round that
    // the longest-first order packs behind the long pieces) balances better
    if (causal && kv_len - q_len < q_len && splits >= 2) splits *= 2;
    const long long max_by_keys = kv_len / 512;  // at least 8 key tiles per range
    if (splits > max_by_keys) splits = max_by_keys;
    if (splits > 8) splits = 8;
    return splits < 2 ? 1 : (int)splits;
}

size_t attn_fwd_split_workspace_bytes(int B, int Hq, int q_len, int D, int kv_splits) {
    if (B <= 0 || Hq <= 0 || q_len <= 0 || D <= 0 || kv_splits <= 1) return 0;
    return (size_t)B * Hq * q_len * kv_splits * (size_t)(D + 1) * sizeof(float);
}

gqa_status_t attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int q_len, int kv_len, int D, float scale, int causal,
                            int kv_splits, void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                            void* hip_stream) {
    if (kv_splits < 1) return GQA_ERR_INVALID_ARG;
    if (kv_splits == 1 || kv_len == 0)
        return attn_fwd(q, k, v, o, lse, B, Hq, Hkv, q_len, kv_len, D, scale, causal, dtype, hip_stream);
    if (B < 0 || q_len < 0 || kv_len < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_ERR_INVALID_ARG;
    if (!supported_head_dim(D) || dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;
    if (B == 0 || q_len == 0) return GQA_OK;
    if (!q || !k || !v || !o || !lse) return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v)) return GQA_ERR_INVALID_ARG;
    const long long rows_q = (long long)B * Hq * q_len;
    const long long rows_kv = (long long)B * Hkv * kv_len;
    if (rows_q > (1LL << 40) || rows_kv > (1LL << 40) || kv_splits > 64) return GQA_ERR_INVALID_ARG;
    const size_t need = attn_fwd_split_workspace_bytes(B, Hq, q_len, D, kv_splits);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return GQA_ERR_WORKSPACE;

    gqa::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.q_len = q_len; a.kv_len = kv_len;
    a.group = Hq / Hkv;
    a.delta = kv_len - q_len;
    a.c = scale * kLog2e;
    a.kv_splits = kv_splits;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = a.part_o + (size_t)rows_q * kv_splits * D;
    hipError_t e = gqa::launch_prefill_split(a, D, causal != 0, to_kernel_dtype(dtype),
                                             static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status_t attn_prefill_paged_with_kernel(const void* q, const void* k_cache, const void* v_cache, void* o,
                                            float* lse, const int* qo_indptr, const int* kv_indptr,
                                            const int* kv_indices, const int* kv_last_page_len, int B, int Hq,
                                            int Hkv, int D, int page_size, int max_q_len, float scale, int causal,
                                            gqa_dtype_t dtype, int kernel, void* hip_stream) {
    gqa::PrefillKernel choice;
    if (!to_prefill_kernel(kernel, &choice)) return GQA_ERR_INVALID_ARG;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_q_len < 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (page_size <= 0 || (page_size & (page_size - 1)) != 0) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_ERR_INVALID_ARG;
    if (!supported_head_dim(D) || dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;
    if (B == 0 || max_q_len == 0) return GQA_OK;
    if (!q || !k_cache || !v_cache || !o || !lse || !qo_indptr || !kv_indptr || !kv_indices)
        return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(o) || !aligned16(k_cache) || !aligned16(v_cache)) return GQA_ERR_INVALID_ARG;
    int page_shift = 0;
    while ((1 << page_shift) < page_size) ++page_shift;

    gqa::PrefillArgs a{};
    a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv;
    a.q_len = max_q_len;  // sizes the grid; each request's own lengths come from the pointers
    a.kv_len = 0;
    a.group = Hq / Hkv;
    a.delta = 0;
    a.c = scale * kLog2e;
    a.qo_indptr = qo_indptr;
    a.kv_indptr = kv_indptr;
    a.kv_indices = kv_indices;
    a.kv_last_page_len = kv_last_page_len;
    a.page_shift = page_shift;
    hipError_t e = gqa::launch_prefill_paged(a, D, causal != 0, to_kernel_dtype(dtype), choice,
                                             static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status_t attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                const int* qo_indptr, const int* kv_indptr, const int* kv_indices,
                                const int* kv_last_page_len, int B, int Hq, int Hkv, int D, int page_size,
                                int max_q_len, float scale, int causal, gqa_dtype_t dtype, void* hip_stream) {
    return attn_prefill_paged_with_kernel(q, k_cache, v_cache, o, lse, qo_indptr, kv_indptr, kv_indices,
                                          kv_last_page_len, B, Hq, Hkv, D, page_size, max_q_len, scale, causal,
                                          dtype, 0, hip_stream);
}

size_t attn_decode_workspace_bytes_multi(int B, int Hq, int q_len, int D, int n_splits) {
    if (B <= 0 || Hq <= 0 || q_len <= 0 || D <= 0 || n_splits <= 0) return 0;
    return (size_t)B * (size_t)Hq * (size_t)q_len * (size_t)n_splits * ((size_t)D + 1) * sizeof(float);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int D, int n_splits) {
    return attn_decode_workspace_bytes_multi(B, Hq, 1, D, n_splits);
}

}  // extern "C"

namespace {

// The 16-bit split-K decode with or without an additive bias (bias == nullptr).
gqa_status_t decode_16bit(const void* q, const void* k, const void* v, const void* bias, long long bias_sb,
                          long long bias_sh, long long bias_sq, void* o, float* lse, const int* seq_lens,
                          const int* block_table, int max_pages_per_seq, int page_size, int B, int Hq, int Hkv,
                          int q_len, int D, int max_kv_len, float scale, int n_splits, void* workspace,
                          size_t workspace_bytes, gqa_dtype_t dtype, void* hip_stream, bool with_bias) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_kv_len < 0) return GQA_ERR_INVALID_ARG;
    if (q_len < 1 || q_len > 256) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (n_splits < 1 || n_splits > 256) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_ERR_INVALID_ARG;
    if (with_bias && (bias_sb < 0 || bias_sh < 0 || bias_sq < 0 || (bias_sb | bias_sh | bias_sq) & 1))
        return GQA_ERR_INVALID_ARG;
    int page_shift = 0;
    if (block_table) {
        if (page_size <= 0 || (page_size & (page_size - 1)) != 0 || max_pages_per_seq <= 0)
            return GQA_ERR_INVALID_ARG;
        if ((long long)max_pages_per_seq * page_size < (long long)max_kv_len) return GQA_ERR_INVALID_ARG;
        while ((1 << page_shift) < page_size) ++page_shift;
    }
    if (!supported_head_dim(D) || dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;
    if (B == 0) return GQA_OK;
    if (!q || !k || !v || !o || !lse || !seq_lens) return GQA_ERR_INVALID_ARG;
    if (with_bias && (!bias || (reinterpret_cast<uintptr_t>(bias) & 3u))) return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return GQA_ERR_INVALID_ARG;
    if ((long long)B * Hq * q_len > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
    const size_t need = attn_decode_workspace_bytes_multi(B, Hq, q_len, D, n_splits);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return GQA_ERR_WORKSPACE;

    gqa::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = a.part_o + (size_t)B * Hq * q_len * n_splits * D;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.group = Hq / Hkv;
    a.q_len = q_len;
    a.max_pages = max_pages_per_seq;
    a.page_shift = page_shift;
    a.max_kv_len = max_kv_len;
    a.n_splits = n_splits;
    a.c = scale * kLog2e;
    if (with_bias) {
        a.bias = static_cast<const uint16_t*>(bias);
        a.bias_sb = bias_sb;
        a.bias_sh = bias_sh;
        a.bias_sq = bias_sq;
        a.bias_k = 1.f / scale;
    }
    hipError_t e = gqa::launch_decode(a, to_kernel_dtype(dtype), static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // namespace

extern "C" {

gqa_status_t attn_decode_splitk_multi(const void* q, const void* k, const void* v, void* o, float* lse,
                                      const int* seq_lens, const int* block_table,
                                      int max_pages_per_seq, int page_size,
                                      int B, int Hq, int Hkv, int q_len, int D, int max_kv_len,
                                      float scale, int n_splits,
                                      void* workspace, size_t workspace_bytes,
                                      gqa_dtype_t dtype, void* hip_stream) {
    return decode_16bit(q, k, v, nullptr, 0, 0, 0, o, lse, seq_lens, block_table, max_pages_per_seq, page_size, B,
                        Hq, Hkv, q_len, D, max_kv_len, scale, n_splits, workspace, workspace_bytes, dtype,
                        hip_stream, false);
}

gqa_status_t attn_decode_splitk_bias(const void* q, const void* k, const void* v, const void* bias,
                                     long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                                     void* o, float* lse, const int* seq_lens, const int* block_table,
                                     int max_pages_per_seq, int page_size, int B, int Hq, int Hkv, int q_len, int D,
                                     int max_kv_len, float scale, int n_splits, void* workspace,
                                     size_t workspace_bytes, gqa_dtype_t dtype, void* hip_stream) {
    return decode_16bit(q, k, v, bias, bias_stride_b, bias_stride_h, bias_stride_q, o, lse, seq_lens, block_table,
                        max_pages_per_seq, page_size, B, Hq, Hkv, q_len, D, max_kv_len, scale, n_splits, workspace,
                        workspace_bytes, dtype, hip_stream, true);
}

gqa_status_t attn_decode_splitk_fp8(const void* q, const void* k_cache, const void* v_cache,
                                    const uint32_t* k_scale_shift, const uint32_t* v_scale_shift,
                                    void* o, float* lse, const int* seq_lens, const int* block_table,
                                    int max_pages_per_seq, int page_size, int B, int Hq, int Hkv, int D,
                                    int max_kv_len, float scale, int n_splits, void* workspace,
                                    size_t workspace_bytes, gqa_dtype_t dtype, void* hip_stream) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_kv_len < 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (n_splits < 1 || n_splits > 256) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return GQA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return GQA_ERR_INVALID_ARG;
    int page_shift = 0;
    if (block_table) {
        if (page_size <= 0 || (page_size & (page_size - 1)) != 0 || max_pages_per_seq <= 0)
            return GQA_ERR_INVALID_ARG;
        if ((long long)max_pages_per_seq * page_size < (long long)max_kv_len) return GQA_ERR_INVALID_ARG;
        while ((1 << page_shift) < page_size) ++page_shift;
    }
    if (!supported_head_dim(D) || dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;
    if (block_table && page_size < 16) return GQA_ERR_UNSUPPORTED;  // a 16-token slice must fit in a page
    if (B == 0) return GQA_OK;
    if (!q || !k_cache || !v_cache || !k_scale_shift || !v_scale_shift || !o || !lse || !seq_lens)
        return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return GQA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(k_scale_shift) & 3u) || (reinterpret_cast<uintptr_t>(v_scale_shift) & 3u))
        return GQA_ERR_INVALID_ARG;
    const size_t need = attn_decode_workspace_bytes(B, Hq, D, n_splits);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return GQA_ERR_WORKSPACE;

    gqa::DecodeArgs a{};
    a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
    a.k_ss = k_scale_shift;
    a.v_ss = v_scale_shift;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = a.part_o + (size_t)B * Hq * n_splits * D;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.group = Hq / Hkv;
    a.q_len = 1;
    a.max_pages = max_pages_per_seq;
    a.page_shift = page_shift;
    a.max_kv_len = max_kv_len;
    a.n_splits = n_splits;
    a.c = scale * kLog2e;
    hipError_t e = gqa::launch_decode_fp8(a, to_kernel_dtype(dtype), static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status_t attn_decode_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* seq_lens, const int* block_table,
                                int max_pages_per_seq, int page_size,
                                int B, int Hq, int Hkv, int D, int max_kv_len,
                                float scale, int n_splits,
                                void* workspace, size_t workspace_bytes,
                                gqa_dtype_t dtype, void* hip_stream) {
    return attn_decode_splitk_multi(q, k, v, o, lse, seq_lens, block_table, max_pages_per_seq, page_size,
                                    B, Hq, Hkv, 1, D, max_kv_len, scale, n_splits, workspace,
                                    workspace_bytes, dtype, hip_stream);
}

gqa_status_t attn_decode_splitk_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int* seq_lens, const int* block_table,
                                        int max_pages_per_seq, int page_size,
                                        int B, int Hq, int Hkv, int D, int max_kv_len,
                                        float scale, int n_splits, gqa_dtype_t dtype, void* hip_stream) {
    // the sizes first: a request beyond the fixed scratch is refused before
    // any HIP call; invalid arguments are left to attn_decode_splitk's checks
    const size_t need = attn_decode_workspace_bytes(B, Hq, D, n_splits);
    if (need > gqa::scratch_capacity_bytes()) return GQA_ERR_WORKSPACE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        if (gqa::scratch_device_ptr(&ws) != hipSuccess) return GQA_ERR_HIP;
        ws_bytes = gqa::scratch_capacity_bytes();
    }
    return attn_decode_splitk(q, k, v, o, lse, seq_lens, block_table, max_pages_per_seq, page_size, B, Hq, Hkv,
                              D, max_kv_len, scale, n_splits, ws, ws_bytes, dtype, hip_stream);
}

gqa_status_t attn_splitk_merge_backward(const float* o_parts, const float* lse_parts, const float* o,
                                        const float* lse, const float* d_o, const float* d_lse, float* d_o_parts,
                                        float* d_lse_parts, long long rows, int n_splits, int D, void* hip_stream) {
    if (rows < 0 || n_splits < 1 || n_splits > 65536 || D < 1 || D > gqa::merge_backward_max_dims())
        return GQA_ERR_INVALID_ARG;
    if (rows == 0) return GQA_OK;
    if (rows > (1LL << 36)) return GQA_ERR_INVALID_ARG;
    const void* ptrs[8] = {o_parts, lse_parts, o, lse, d_o, d_lse, d_o_parts, d_lse_parts};
    for (const void* p : ptrs)
        if (!p || (reinterpret_cast<uintptr_t>(p) & 3u)) return GQA_ERR_INVALID_ARG;
    gqa::MergeBwdArgs a{o_parts, lse_parts, o, lse, d_o, d_lse, d_o_parts, d_lse_parts, rows, n_splits, D};
    hipError_t e = gqa::launch_merge_backward(a, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

const char* attn_status_str(gqa_status_t s) {
    switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG: invalid argument";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: no kernel for this head dim / dtype / group";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: HIP launch error";
    default: return "unknown gqa_status_t";
    }
}

}  // extern "C"
