// gqa_device.hpp - device-side building blocks for the gfx950 attention kernels:
// vector types, MFMA wrappers, cross-lane moves and conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage tags: the element type in memory and the matching MFMA operand type.
struct bf16_tag {
    typedef bf16x8 vec8;
    typedef bf16x2 vec2;
};
struct f16_tag {
    typedef f16x8 vec8;
    typedef f16x2 vec2;
};

// D[32x32] += A[32x16] * B[16x32], fp32 accumulate.  Operand layout: lane l
// holds row/column (l % 32) and 8 consecutive k-slots starting at 8 * (l / 32).
// Result layout: lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// fp32: D[32x32] += A[32x2] * B[2x32]; lane l holds k-slot l / 32.
__device__ __forceinline__ f32x16 mfma_32x32x2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of x held by lane (l ^ 32), for every lane l.  The result must be
// selected per lane: the compiler treats the two results of a swap of one
// value with itself as equal and folds expressions that use both.
__device__ __forceinline__ float xor32(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // r[0]: lanes 0-31 keep their value, lanes 32-63 receive lanes 0-31;
    // r[1]: lanes 0-31 receive lanes 32-63, lanes 32-63 keep theirs.
    uint32_t lane = __lane_id();
    return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// Lane (l ^ mask) via the LDS crossbar (any mask).
__device__ __forceinline__ float shfl_xor(float x, int mask) {
    int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2,
                                                                  __builtin_bit_cast(int, x)));
}

// Two fp32 values -> packed pair in the storage type (round to nearest even).
__device__ __forceinline__ uint32_t pack2(bf16_tag, float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(f16_tag, float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// One output row from the 32x32 MFMA accumulator with the queries as columns:
// lane (q, half) holds dims 32 dt + 8 j + 4 half + 0..3 (j = 0..3) of row q.
// A lane swap between the two 32-lane halves leaves each lane 16 consecutive
// dims of every 32-dim block (half 0 the first 16), scaled by inv and packed:
// chunk 2 dt + e (e = 0, 1) holds dims 32 dt + 16 half + 8 e .. + 7, i.e. the
// 16-byte chunk 4 dt + 2 half + e of the row.  Every lane of the wave must
// execute it (the swap reads the other half).
template <class TAG, int DT>
__device__ __forceinline__ void acc_row_chunks(TAG, const f32x16 (&acc)[DT], float inv, u32x4 (&chunk)[2 * DT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        uint32_t x[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j][0] = pack2(TAG(), acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv);
            x[j][1] = pack2(TAG(), acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv);
        }
        // v_permlane32_swap: lanes 32-63 of the first operand trade places with
        // lanes 0-31 of the second, so half 0 gets half 1's dims 4-7 (and
        // 12-15) and half 1 gets half 0's dims 16-19 (and 24-27)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const auto r02 = __builtin_amdgcn_permlane32_swap(x[0][e], x[2][e], false, false);
            const auto r13 = __builtin_amdgcn_permlane32_swap(x[1][e], x[3][e], false, false);
            x[0][e] = r02[0];
            x[2][e] = r02[1];
            x[1][e] = r13[0];
            x[3][e] = r13[1];
        }
        chunk[2 * dt] = u32x4{x[0][0], x[0][1], x[2][0], x[2][1]};
        chunk[2 * dt + 1] = u32x4{x[1][0], x[1][1], x[3][0], x[3][1]};
    }
}

// The same row written straight to global memory: two 16-byte stores per
// 32-dim block (32 contiguous bytes of the row per lane pair).
template <class TAG, int DT>
__device__ __forceinline__ void store_acc_row(TAG, const f32x16 (&acc)[DT], float inv, uint16_t* row, int half,
                                              bool valid) {
    u32x4 chunk[2 * DT];
    acc_row_chunks(TAG(), acc, inv, chunk);
    if (valid) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            uint16_t* dst = row + dt * 32 + half * 16;
            *reinterpret_cast<u32x4*>(dst) = chunk[2 * dt];
            *reinterpret_cast<u32x4*>(dst + 8) = chunk[2 * dt + 1];
        }
    }
}

// Select 16-bit halves of two dwords: lo16(a) | lo16(b) << 16, and hi16(a) | hi16(b) << 16.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// s_waitcnt vmcnt(0): every outstanding vector-memory load has returned.
// (gfx9 encoding: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].)
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ u32x4 ld_global_16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Sum over the wave of per-lane values in [0, 2^nbits): one ballot per bit.
__device__ __forceinline__ int wave_sum_bits(int v, int nbits) {
    int s = 0;
    for (int j = 0; j < nbits; ++j)
        s += __builtin_popcountll(__builtin_amdgcn_ballot_w64(((v >> j) & 1) != 0)) << j;
    return s;
}

// Work order of a ragged prefill batch over a paged cache (at most 512
// requests: one lane per request in each of 8 chunks of 64).  Item (b, i) is
// request b's i-th block of POS query rows counted from its last query, so its
// rows see at most kv_b - i * POS keys.  Items go in the order of their level
// s_b + i, s_b = (kref - kv_b) / POS with kref = the pages of the whole batch
// times the page size (>= every kv_b), ties in request order: the longest
// blocks of the whole batch come first, and the in-order dispatch of
// workgroups ends on short ones.  Returns the request of item `item` and sets
// `i`, or returns -1 past the last item.  The answer is wave-uniform and the
// same in every wave of a workgroup.
template <int POS>
__device__ int ragged_item(const int* qo_indptr, const int* kv_indptr, const int* kv_last_page_len,
                           int page_shift, int B, int n_pos_tiles, int item, int& i) {
    const int lane = __lane_id();
    const int n_chunks = (B + 63) / 64;
    const long long kref = (long long)(kv_indptr[B] - kv_indptr[0]) << page_shift;
    int npt[8], lvl[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int r = c * 64 + lane;
        int nq = 0;
        long long kv = 0;
        if (r < B) {
            nq = qo_indptr[r + 1] - qo_indptr[r];
            const int np = kv_indptr[r + 1] - kv_indptr[r];
            if (np > 0)
                kv = ((long long)(np - 1) << page_shift) +
                     (kv_last_page_len ? kv_last_page_len[r] : (1 << page_shift));
        }
        npt[c] = (nq + POS - 1) / POS;
        lvl[c] = (int)((kref - kv) / POS);
    }
    // a lane's count is at most 8 * n_pos_tiles
    const int nbits = 35 - __builtin_clz((unsigned)(n_pos_tiles > 0 ? n_pos_tiles : 1));
    auto upto = [&](int L) {  // items at levels <= L
        int v = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (c < n_chunks) v += min(max(L + 1 - lvl[c], 0), npt[c]);
        return wave_sum_bits(v, nbits);
    };
    const int lend = (int)(kref / POS) + n_pos_tiles;  // every level is below lend
    if (item >= upto(lend - 1)) return -1;
    int lo = 0, hi = lend - 1;  // the level of the item: the first L with upto(L) > item
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (upto(mid) > item) hi = mid;
        else lo = mid + 1;
    }
    int k = item - (lo > 0 ? upto(lo - 1) : 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        if (c >= n_chunks) break;
        const bool has = lvl[c] <= lo && lo < lvl[c] + npt[c];
        const uint64_t m = __builtin_amdgcn_ballot_w64(has);
        const int cnt = __builtin_popcountll(m);
        if (k < cnt) {
            // the k-th request (in index order) of this chunk with a block at level lo
            const int rank = __builtin_popcountll(m & ((1ull << lane) - 1ull));
            const int sel = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(has && rank == k));
            i = lo - __builtin_amdgcn_readlane(lvl[c], sel);
            return c * 64 + sel;
        }
        k -= cnt;
    }
    return -1;
}

}  // namespace gqa
