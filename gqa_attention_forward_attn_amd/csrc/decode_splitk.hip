// decode_splitk.hip - split-K single-query attention over a (paged) KV cache.
//
// Method: splitk_kernels.py (xformers), `_fwd_kernel_splitK` and
// `_splitK_reduce`.  Each sequence's keys are cut into n_splits chunks; every
// non-empty chunk runs the online softmax over its keys and writes a partial
// output O_s = acc / l and its natural-base LSE.  The combine kernel merges the
// chunks per (b, h): M = max_s LSE_s, w_s = exp(LSE_s - M),
// O = sum w_s O_s / sum w_s, LSE = M + log(sum w_s); a sequence with no keys
// gives (0, -inf).  Keys of a paged cache are found through the per-sequence
// block table, page block_table[b, t / page_size], row t % page_size (the
// PAGE_SIZE branch of `_fwd_kernel_splitK`).
//
// Several queries per sequence (speculative / chunked decode, the Mq > 1 case
// of `_fwd_kernel_splitK`): a sequence of len keys carries q_len queries at its
// last positions, so query i sees keys t <= len - q_len + i (bottom-right
// causal).  q_len = 1 is plain decode.
//
// gfx950 mapping.  Decode reads every K/V byte once, so it is bound by HBM;
// the arithmetic still goes to the matrix cores so that the vector ALUs stay
// nearly idle.  The query rows of one K/V head group, (head hh, query i) ->
// column hh * q_len + i, are contiguous in q; a workgroup owns one (sequence,
// K/V head, chunk) and 16 of those columns, the 16 columns of the MFMA tiles
// (columns beyond the group are zero).  Each wave streams its own 16-token
// slices of the chunk (wave w takes slices w, w + NW, ...):
//
//   K, V slice (16 rows)  --global_load_lds_dwordx4-->  per-wave LDS ring of NST stages
//   S^T[16 tok x 16 heads] = K q^T        4 x v_mfma_f32_16x16x32 (D = 128)
//   online softmax on S^T (4 values per lane, no cross-lane work unless the
//                          running max grows by more than 2^8)
//   O[16 heads x D] += P V                8 x v_mfma_f32_16x16x16 with V read
//                                         transposed (ds_read_b64_tr_b16)
//
// The S^T result layout (lane: head l%16, tokens 4(l/16)..+3) is exactly the
// A-operand layout of the P.V MFMA, so P never leaves its registers.  Each wave
// keeps one slice in flight: slice k + 1 leaves once slice k has landed and
// loads while slice k is computed (more loads in flight per CU measured slower,
// the memory system queueing them rather than streaming faster).  No barrier is
// taken in the loop: every wave waits only for its own loads.  The NW per-wave
// partial results are merged through LDS at the end of the chunk.
#include "gqa_device.hpp"
#include "gqa_kernels.hpp"

namespace gqa {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(4))) int const_int;

constexpr int kSlice = 16;         // tokens per slice (MFMA rows)
constexpr float kRescaleLog2 = 8.f;

// K/V addressing of the split kernel
enum { kDense = 0, kPaged = 1, kPagedSmall = 2 };

// waves and ring stages of the 16-bit split kernel.  A wave has one slice in
// flight and one being read, so two stages would do; four make the workgroup's
// LDS (q rows + 4 rings, 132 KB at D = 128) hold it to one workgroup per CU,
// i.e. four slices in flight per CU: two workgroups per CU (two stages, eight
// waves) measured 7-9 % slower on the decode workloads.
#ifndef DEC_NW
#define DEC_NW 4
#endif
#ifndef DEC_NST
#define DEC_NST 4
#endif
// waves and ring stages of the E4M3 split kernel
#ifndef DEC8_NW
#define DEC8_NW 4
#endif
#ifndef DEC8_NST
#define DEC8_NST 2
#endif

// Chunk length of the split-K partition (a multiple of 64 tokens); both kernels
// derive the chunk bounds from it.
__device__ __forceinline__ int chunk_tokens(int len, int n_splits) {
    const int per = (len + n_splits - 1) / n_splits;
    return (per + 63) / 64 * 64;
}

// 16 bytes per lane from global memory into LDS (lane i -> lds + 16 i).  The
// compiler does not see the load, so completion is awaited with explicit
// vmcnt waits; the memory clobber keeps LDS reads of the stage it overwrites
// on their side of it.  Every K/V byte of a decode step is read once, so the
// loads are non-temporal (`nt`): they do not displace lines L2 still serves
// (+11 % streaming rate on the paged decode workload).
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
    __asm__ __volatile__("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                         :
                         : "v"(gptr), "s"(lds)
                         : "m0", "memory");
}
// Same, from a wave-uniform base address plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
    __asm__ __volatile__("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                         :
                         : "v"(voff), "s"(sbase), "s"(lds)
                         : "m0", "memory");
}

// 4 bytes per lane from global memory into LDS (lane i -> lds + 4 i).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds) {
    __asm__ __volatile__("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                         :
                         : "v"(gptr), "s"(lds)
                         : "m0", "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __asm__ __volatile__("" ::: "memory");
}

// Wait until at most n * PER direct loads are outstanding (n < 8).
template <int PER>
__device__ __forceinline__ void wait_slices(int n) {
    switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1 * PER>(); break;
    case 2: wait_vm<2 * PER>(); break;
    case 3: wait_vm<3 * PER>(); break;
    case 4: wait_vm<(4 * PER < 64 ? 4 * PER : 63)>(); break;
    case 5: wait_vm<(5 * PER < 64 ? 5 * PER : 63)>(); break;
    case 6: wait_vm<(6 * PER < 64 ? 6 * PER : 63)>(); break;
    default: wait_vm<(7 * PER < 64 ? 7 * PER : 63)>(); break;
    }
}

__device__ __forceinline__ u32x4 lds16(const lds_char* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
__device__ __forceinline__ u32x2 lds_tr(const lds_char* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    return __builtin_bit_cast(u32x2, v);
}

// D[16x16] += A[16x32] B[32x16]; lane l holds row/column l % 16 and k-slots
// 8(l/16)..+7; result lane l: column l % 16, rows 4(l/16)..+3.
__device__ __forceinline__ f32x4 mfma16x32(bf16_tag, u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x32(f16_tag, u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                   c, 0, 0, 0);
}
// D[16x16] += A[16x16] B[16x16]; k-slots 4(l/16)..+3, same result layout.
__device__ __forceinline__ f32x4 mfma16x16(bf16_tag, u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                      c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16(f16_tag, u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b),
                                                  c, 0, 0, 0);
}

// A stored 16-bit value of the input dtype as fp32.
__device__ __forceinline__ float bias_to_f32(bf16_tag, uint32_t u16) { return __builtin_bit_cast(float, u16 << 16); }
__device__ __forceinline__ float bias_to_f32(f16_tag, uint32_t u16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
}

__device__ __forceinline__ float lane_value(float x, int src_lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, x)));
}

// LDS slice layout: 16 rows of 2D bytes; 16-byte chunk c of row r is stored at
// chunk position c ^ swz<D>(r).  LDS has 64 banks of 4 bytes; a 16-byte read is
// served 16 lanes at a time, an 8-byte read 32 lanes at a time, and a read is
// conflict-free when those lanes hit distinct 16-byte bank groups.  K / q
// operand reads: 16 lanes = rows 0..15 at one chunk.  Transposed V reads: 32
// lanes = 8 consecutive rows x chunks (2n, 2n+1).  D = 128 (a row spans all 64
// banks): swz is a bijection on r % 16 that is even on rows 0-7 and odd on rows
// 8-15.  D = 64 (two rows per bank row, group = 8 (r % 2) + position): swz is a
// bijection on (r >> 1) % 8, even on rows 0-7 and odd on rows 8-15.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
    return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// BIAS: the additive bias of `_fwd_kernel_splitK` (HAS_ADDITIVE_BIAS).  Each
// slice also brings the bias of its 16 tokens for the block's 16 columns
// (pairs of keys per 4-byte direct load, 512 bytes after the V slice), added
// to the scores before the softmax.
template <class TAG, int D, int NW, int NST, int PG, bool BIAS = false>
__global__ __launch_bounds__(NW * 64, 1) void decode_split_kernel(DecodeArgs a) {
    constexpr int ROWB = 2 * D;             // bytes per K/V/q row
    constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;           // rows per direct-load instruction
    constexpr int NI = kSlice / RPI;        // direct loads per slice, each of K and V
    constexpr int SLB = kSlice * ROWB;      // bytes of a K (or V) slice
    constexpr int BSB = BIAS ? 16 * kSlice * 2 : 0;  // bias of a slice: 16 columns x 16 keys
    constexpr int STB = 2 * SLB + BSB;      // stage: K slice, V slice[, bias]
    constexpr int QB = 16 * ROWB;           // q rows of the head block, shared by the waves
    constexpr int RINGB = NST * STB;        // LDS ring of a wave
    constexpr int KS = D / 32;              // k-steps of S^T = K q^T
    constexpr int NB = D / 16;              // 16-column blocks of O
    constexpr int PER_SLICE = 2 * NI + (BIAS ? 2 : 0);
    static_assert((NST - 1) * PER_SLICE < 64, "vmcnt range");
    static_assert((NST & (NST - 1)) == 0, "NST must be a power of two");
    static_assert(NST >= 2, "the slice being read and the slice in flight");
    static_assert((NW * 16 * (D + 4) + 3 * NW * 16) * 4 <= QB + NW * RINGB, "merge buffers must fit in LDS");

    __shared__ __attribute__((aligned(1024))) char smem_raw[QB + NW * RINGB];
    lds_char* smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- work item: (b, split, column block, kv head), kv head fastest ------
    const int ncol = a.group * a.q_len;     // query rows of the group
    const int n_hb = (ncol + 15) >> 4;
    int id = blockIdx.x;
    const int g = id % a.Hkv;
    id /= a.Hkv;
    const int hb = id % n_hb;
    id /= n_hb;
    const int s = id % a.n_splits;
    const int b = id / a.n_splits;
    const int nh = min(16, ncol - hb * 16);  // columns of this block
    const size_t qrow0 = ((size_t)b * a.Hq + (size_t)g * a.group) * a.q_len + hb * 16;  // its first query row

    const int len = a.seq_lens[b];
    if (len <= 0) return;
    const int chunk = chunk_tokens(len, a.n_splits);
    const int lo = s * chunk;
    if (lo >= len) return;  // empty chunk: the combine kernel skips it
    const int hi = min(len, lo + chunk);

    const int stride = kSlice * NW;
    const int span = hi - lo;
    const int n_sl = span > kSlice * wave ? (span - kSlice * wave + stride - 1) / stride : 0;
    const int T0 = lo + kSlice * wave;

    const lds_char* wlds = smem + QB + wave * RINGB;  // this wave's ring
    const uint32_t wlds_u = (uint32_t)(uintptr_t)wlds;
    const uint32_t q_u = (uint32_t)(uintptr_t)smem;

    // per-lane constants of the direct loads: lane -> (row in instruction, physical chunk)
    const int drow = lane / CPR;
    const int dchk = lane % CPR;
    int urow[NI], lcol[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        urow[i] = RPI * i + drow;
        lcol[i] = (dchk ^ swz<D>(urow[i])) * 8;  // element offset of the logical chunk
    }

    const int* bt = a.block_table + (size_t)b * a.max_pages;
    const int page_mask = (1 << a.page_shift) - 1;
    const size_t tok_stride = PG == kDense ? (size_t)D : (size_t)a.Hkv * D;
    const size_t head_off = PG == kDense ? ((size_t)b * a.Hkv + g) * (size_t)a.max_kv_len * D : (size_t)g * D;

    // page ids of this wave's first 64 slices, one per lane (paged, page >= 16)
    int pgv = 0;
    if (PG == kPaged && lane < n_sl) pgv = bt[(T0 + stride * lane) >> a.page_shift];

    // direct loads of slice k: wave-uniform base (row T of the slice) plus a
    // per-lane byte offset; rows past the chunk repeat its last row
    const char* kbytes = static_cast<const char*>(a.k);
    const char* vbytes = static_cast<const char*>(a.v);
    // BIAS: lane i of bias load j brings keys (2 (i % 8), +1) of column 8 j + i / 8
    // (columns past the block repeat its last one); its row of the bias
    [[maybe_unused]] const uint16_t* brow[2];
    if constexpr (BIAS) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int qr = hb * 16 + min(8 * j + lane / 8, nh - 1);  // query row in the group
            const int h = g * a.group + qr / a.q_len, qi = qr % a.q_len;
            brow[j] = a.bias + (long long)b * a.bias_sb + (long long)h * a.bias_sh + (long long)qi * a.bias_sq;
        }
    }
    // drain: wait for every load in flight first (after the addresses are
    // computed, so that the slice's loads leave as soon as the previous ones
    // have landed)
    auto issue = [&](int k, bool drain) {
        const int T = T0 + stride * k;
        const uint32_t st = __builtin_amdgcn_readfirstlane(wlds_u + (k & (NST - 1)) * STB);
        const int last = hi - 1 - T;  // rows of the slice at or past `last` repeat row `last`
        if (PG == kPagedSmall) {
            if (drain) wait_vm<0>();
            if constexpr (BIAS) {
                const int t = T + min(2 * (lane & 7), last & ~1);
#pragma unroll
                for (int j = 0; j < 2; ++j) dma4(brow[j] + t, st + 2 * SLB + j * 256);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int t = T + min(urow[i], last);
                const int page = bt[t >> a.page_shift];
                const size_t off = ((((size_t)page << a.page_shift) + (size_t)(t & page_mask)) * tok_stride +
                                    head_off + lcol[i]) * 2;
                dma16(kbytes + off, st + i * 1024);
                dma16(vbytes + off, st + SLB + i * 1024);
            }
            return;
        }
        size_t row0;  // element offset of row T
        if (PG == kPaged) {
            const int page = k < 64 ? __builtin_amdgcn_readlane(pgv, k)
                                    : ((const_int*)bt)[__builtin_amdgcn_readfirstlane(T >> a.page_shift)];
            row0 = (((size_t)page << a.page_shift) + (size_t)(T & page_mask)) * tok_stride + head_off;
        } else {
            row0 = head_off + (size_t)T * D;
        }
        const char* kb = kbytes + row0 * 2;
        const char* vb = vbytes + row0 * 2;
        uint32_t voff_b[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) voff_b[i] = (uint32_t)(min(urow[i], last) * (int)tok_stride + lcol[i]) * 2u;
        if (drain) wait_vm<0>();
        if constexpr (BIAS) {
            // key pairs past the chunk read the pair of its last key; that pair
            // may hold one key past the sequence (rows are readable up to an
            // even key count)
            const int t = T + min(2 * (lane & 7), last & ~1);
#pragma unroll
            for (int j = 0; j < 2; ++j) dma4(brow[j] + t, st + 2 * SLB + j * 256);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            dma16(kb, voff_b[i], st + i * 1024);
            dma16(vb, voff_b[i], st + SLB + i * 1024);
        }
    };

    float m = -INFINITY, l = 0.f;
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
        // q rows of the head block, one buffer for the workgroup: wave w loads
        // rows RPI i .. RPI i + RPI - 1 for i = w, w + NW, ... (rows >= nh repeat
        // the last head; their operand lanes are zeroed below)
        const int nqi = (nh + RPI - 1) / RPI;
        for (int i = wave; i < nqi; i += NW) {
            const int r = min(RPI * i + drow, nh - 1);
            const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow0 + r) * D +
                                 (dchk ^ swz<D>(RPI * i + drow)) * 8;
            dma16(qp, __builtin_amdgcn_readfirstlane(q_u + i * 1024));
        }
    }
    // the page ids are awaited here, before any slice is issued (the compiler
    // does not see the direct loads: a wait for them inside the loop would
    // also wait for every slice in flight)
    __asm__ __volatile__("" ::"v"(pgv));
    if (n_sl > 0) {
        issue(0, false);
        wait_vm<PER_SLICE>();  // this wave's q rows (loaded before its first slice)
    } else {
        wait_vm<0>();
    }
    __syncthreads();  // ... and every other wave's

    if (n_sl > 0) {

        // q^T as the B operand: lane l holds head l % 16, dims 32 ks + 8 (l / 16)..+7
        const int hrow = lane & 15;
        const int kq = lane >> 4;
        u32x4 qop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 x = lds16(smem + hrow * ROWB + (((4 * ks + kq) ^ swz<D>(hrow)) << 4));
            qop[ks] = hrow < nh ? x : u32x4{0u, 0u, 0u, 0u};
        }
        // LDS offsets of the K operand (row l % 16) and of the transposed V reads
        int koff[KS], voff[NB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[ks] = hrow * ROWB + (((4 * ks + kq) ^ swz<D>(hrow)) << 4);
        {
            const int j = lane & 15;
            const int r = 4 * kq + (j >> 2);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int c = 2 * nb + ((j & 3) >> 1);
                voff[nb] = SLB + r * ROWB + ((c ^ swz<D>(r)) << 4) + 8 * (j & 1);
            }
        }

        // causal limit of this lane's column: keys < lim are visible
        const int qi = (hb * 16 + hrow) % a.q_len;
        const int lim = min(hi, len - (a.q_len - 1 - qi));
        const int lim_lo = min(hi, len - (a.q_len - 1));  // smallest limit of the block

        for (int k = 0; k < n_sl; ++k) {
            // one slice in flight per wave: slice k + 1 leaves once slice k,
            // the only load in flight, has landed, and loads while slice k is
            // computed
            if (k + 1 < n_sl) issue(k + 1, true);
            else wait_vm<0>();

            const lds_char* st = wlds + (k & (NST - 1)) * STB;
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc = mfma16x32(TAG(), lds16(st + koff[ks]), qop[ks], sc);

            if constexpr (BIAS) {
                // this lane's column and keys 4 kq .. 4 kq + 3: s * c gains log2(e) * bias
                const u32x2 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
                    st + 2 * SLB + hrow * 32 + kq * 8);
                sc[0] = fmaf(bias_to_f32(TAG(), w[0] & 0xffffu), a.bias_k, sc[0]);
                sc[1] = fmaf(bias_to_f32(TAG(), w[0] >> 16), a.bias_k, sc[1]);
                sc[2] = fmaf(bias_to_f32(TAG(), w[1] & 0xffffu), a.bias_k, sc[2]);
                sc[3] = fmaf(bias_to_f32(TAG(), w[1] >> 16), a.bias_k, sc[3]);
            }
            const int T = T0 + stride * k;
            if (T + kSlice > lim_lo) {  // ragged last slice of the chunk, or keys past a query
                const int tok = T + 4 * kq;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (tok + r >= lim) sc[r] = -INFINITY;
            }
            const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.c;
            if (__builtin_amdgcn_ballot_w64(lm > m + kRescaleLog2)) {
                // new reference max for every head: max over the slice's 16 tokens
                float mt = fmaxf(lm, shfl_xor(lm, 16));
                mt = fmaxf(mt, xor32(mt));
                const float mn = fmaxf(m, mt);
                const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
                m = mn;
                l *= alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = lane_value(alpha, 4 * kq + r);  // acc row 4 (l/16) + r is head 4 (l/16) + r
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[nb][r] *= ar;
                }
            }
            const float mu = m == -INFINITY ? 0.f : m;
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = fast_exp2(fmaf(sc[r], a.c, -mu));
            l += (p[0] + p[1]) + (p[2] + p[3]);
            const u32x2 pop = {pack2(TAG(), p[0], p[1]), pack2(TAG(), p[2], p[3])};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16(TAG(), pop, lds_tr(st + voff[nb]), acc[nb]);
        }
    }

    // ---- merge the NW waves' partial results -------------------------------
    // Every wave's acc goes to LDS (rows padded by 16 bytes, so that the four
    // rows of one store instruction fall into distinct banks); the merged rows
    // are written as 16-byte pieces.  The partial rows are what a workgroup
    // writes last, and with one workgroup per CU the next one starts only when
    // they are out, so their cost grows with the columns of the block (16
    // query rows cost 8 KB per workgroup against 2 KB for one query of four
    // heads).
    l += shfl_xor(l, 16);
    l += xor32(l);
    __syncthreads();  // every wave is done with its ring (and its loads have landed)
    constexpr int SROW = D + 4;                        // floats per padded row
    float* sacc = reinterpret_cast<float*>(smem_raw);  // [NW][16][SROW]
    float* sm = sacc + NW * 16 * SROW;                 // [NW][16]
    float* sl = sm + NW * 16;                          // [NW][16]
    {
        const int kq = lane >> 4, c = lane & 15;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[(wave * 16 + 4 * kq + r) * SROW + 16 * nb + c] = acc[nb][r];
        if (lane < 16) {
            sm[wave * 16 + lane] = m;
            sl[wave * 16 + lane] = l;
        }
    }
    __syncthreads();
    const size_t prow = qrow0 * a.n_splits + s;  // partial row of the block's first column
    // per column: the waves' weights relative to the largest running max,
    // divided by the column's sum, and its LSE; a column with no visible key
    // in this chunk (a query before the chunk's keys) gives (0, -inf)
    float* se = sl + NW * 16;  // [NW][16]
    if (tid < nh) {
        const int h = tid;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * 16 + h]);
        float e[NW], L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = sm[w * 16 + h];
            e[w] = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
            L += e[w] * sl[w * 16 + h];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) se[w * 16 + h] = e[w] * inv;
        a.part_lse[prow + (size_t)h * a.n_splits] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    constexpr int V4 = D / 4;  // 16-byte pieces per row
    for (int i = tid; i < nh * V4; i += NW * 64) {
        const int h = i / V4, d = 4 * (i % V4);
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float e = se[w * 16 + h];
            const f32x4 x = *reinterpret_cast<const f32x4*>(sacc + (w * 16 + h) * SROW + d);
#pragma unroll
            for (int k = 0; k < 4; ++k) O[k] = fmaf(e, x[k], O[k]);
        }
        // streamed past L2: the combine kernel reads them once, after every chunk
        __builtin_nontemporal_store(O, reinterpret_cast<f32x4*>(a.part_o + (prow + (size_t)h * a.n_splits) * D + d));
    }
}

// ---- split kernel over an 8-bit E4M3 K/V cache ---------------------------------
//
// splitk_kernels.py, `_fwd_kernel_splitK` with FP8_QUANTIZED: K and V hold one
// E4M3 byte per element and every (token, K/V head) row carries a binary16
// scale and shift packed in a uint32 (`cast_uint32_to_half2`); the value used
// is byte * scale + shift (`dequantize`).  The affine map is folded out of the
// two contractions, so the matrix cores see the E4M3 values themselves (bf16
// and fp16 hold them exactly):
//   s_t = scale_t * (q . x_t) + shift_t * sum_d q_d
//   O   = (sum_t (p_t scale_t) x_t + sum_t p_t shift_t) / l
// Per 16-token slice, the K and V bytes (16 x D each) and the slice's 32 scale /
// shift words come by direct loads into the wave's LDS ring; the K operand is
// converted to 16-bit floats in registers (v_cvt_scalef32_pk_*_fp8 with scale
// 1), and the V slice is converted once into a 16-bit slice buffer that the
// transposed reads of the P.V product use as in decode_split_kernel.


// Four E4M3 bytes (one dword, element order = byte order) -> four 16-bit floats.
__device__ __forceinline__ u32x2 e4m3x4_to16(bf16_tag, uint32_t w) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}
__device__ __forceinline__ u32x2 e4m3x4_to16(f16_tag, uint32_t w) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
}
// Sum of the two 16-bit floats of a dword.
__device__ __forceinline__ float pair_sum(bf16_tag, uint32_t w) {
    return __builtin_bit_cast(float, w << 16) + __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ float pair_sum(f16_tag, uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffff)) +
           (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// binary16 in bits 0-15 / 16-31 of a scale-shift word
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffff)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// E4M3 K/V slices: rows of D bytes; 16-byte chunk c of row r at position
// c ^ swz8<D>(r).  D = 128 (two rows per 64-bank row): a bijection on
// (r >> 1) % 8 as swz<64>; D = 64 (four rows per bank row): (r >> 2) % 4.  The
// 8-byte K operand reads (16 lanes = 16 rows at one column) then hit 16
// distinct bank groups.
template <int D>
__device__ __forceinline__ int swz8(int r) {
    if (D == 128) return swz<64>(r);
    return (r >> 2) & 3;
}

template <class TAG, int D, int NW, int NST, int PG>
__global__ __launch_bounds__(NW * 64, 1) void decode_split_kernel_fp8(DecodeArgs a) {
    constexpr int QROWB = 2 * D;            // bytes per q row (16-bit floats)
    constexpr int KROWB = D;                // bytes per E4M3 K / V row
    constexpr int CPR = KROWB / 16;         // 16-byte chunks per K / V row
    constexpr int RPI = 64 / CPR;           // rows per direct-load instruction
    constexpr int NI = kSlice / RPI;        // direct loads per slice, each of K and V
    constexpr int SLB = kSlice * KROWB;     // bytes of a K (or V) slice
    constexpr int SSB = 256;                // scale-shift words: K at 0, V at 64 (rest repeats)
    constexpr int STB = 2 * SLB + SSB;      // stage
    constexpr int QB = 16 * QROWB;          // q rows of the head block
    constexpr int VCB = kSlice * QROWB;     // the current V slice in 16-bit floats
    constexpr int WAVEB = QB + NST * STB + VCB;
    constexpr int KS = D / 32;
    constexpr int NB = D / 16;
    constexpr int PER_SLICE = 2 * NI + 1;
    constexpr int SCH = D / 64;             // E4M3 V chunks each lane converts per slice
    constexpr int QCPR = QROWB / 16;        // q: chunks per row, rows per load
    constexpr int QRPI = 64 / QCPR;
    static_assert(PG != kPagedSmall, "E4M3 pages hold at least one 16-token slice");
    static_assert((NST - 1) * PER_SLICE < 64, "vmcnt range");
    static_assert((NST & (NST - 1)) == 0, "NST must be a power of two");
    static_assert((NW * 16 * (D + 4) + 4 * NW * 16) * 4 <= NW * WAVEB, "merge buffers must fit in the ring");

    __shared__ __attribute__((aligned(1024))) char smem_raw[NW * WAVEB];
    lds_char* smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- work item: (b, split, head block, kv head), kv head fastest ----------
    const int ncol = a.group;               // one query per sequence: a column per head
    const int n_hb = (ncol + 15) >> 4;
    int id = blockIdx.x;
    const int g = id % a.Hkv;
    id /= a.Hkv;
    const int hb = id % n_hb;
    id /= n_hb;
    const int s = id % a.n_splits;
    const int b = id / a.n_splits;
    const int nh = min(16, ncol - hb * 16);
    const size_t qrow0 = (size_t)b * a.Hq + (size_t)g * a.group + hb * 16;

    const int len = a.seq_lens[b];
    if (len <= 0) return;
    const int chunk = chunk_tokens(len, a.n_splits);
    const int lo = s * chunk;
    if (lo >= len) return;  // empty chunk: the combine kernel skips it
    const int hi = min(len, lo + chunk);

    const int stride = kSlice * NW;
    const int span = hi - lo;
    const int n_sl = span > kSlice * wave ? (span - kSlice * wave + stride - 1) / stride : 0;
    const int T0 = lo + kSlice * wave;

    const lds_char* wlds = smem + wave * WAVEB;
    const uint32_t wlds_u = (uint32_t)(uintptr_t)wlds;
    lds_char* vcs = smem + wave * WAVEB + QB + NST * STB;  // 16-bit V slice

    // direct loads: lane -> (row in instruction, physical chunk)
    const int drow = lane / CPR;
    const int dchk = lane % CPR;
    int urow[NI], lcol[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        urow[i] = RPI * i + drow;
        lcol[i] = (dchk ^ swz8<D>(urow[i])) * 16;  // byte offset of the logical chunk
    }

    const int* bt = a.block_table + (size_t)b * a.max_pages;
    const int page_mask = (1 << a.page_shift) - 1;
    const size_t tok_stride = PG == kDense ? (size_t)D : (size_t)a.Hkv * D;  // bytes between token rows
    const size_t head_off = PG == kDense ? ((size_t)b * a.Hkv + g) * (size_t)a.max_kv_len * D : (size_t)g * D;

    int pgv = 0;
    if (PG == kPaged && lane < n_sl) pgv = bt[(T0 + stride * lane) >> a.page_shift];

    const char* kbytes = static_cast<const char*>(a.k);
    const char* vbytes = static_cast<const char*>(a.v);
    const uint32_t* ssp = (lane & 16) ? a.v_ss : a.k_ss;  // lanes 0-15 K words, 16-31 V words
    const int ss_tok = lane & 15;
    auto issue = [&](int k) {
        const int T = T0 + stride * k;
        const uint32_t st = __builtin_amdgcn_readfirstlane(wlds_u + QB + (k & (NST - 1)) * STB);
        const int last = hi - 1 - T;  // rows of the slice past `last` repeat row `last`
        size_t row0;                  // byte offset of row T (head g)
        if (PG == kPaged) {
            const int page = k < 64 ? __builtin_amdgcn_readlane(pgv, k)
                                    : ((const_int*)bt)[__builtin_amdgcn_readfirstlane(T >> a.page_shift)];
            row0 = (((size_t)page << a.page_shift) + (size_t)(T & page_mask)) * tok_stride + head_off;
        } else {
            row0 = head_off + (size_t)T * D;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t voff = (uint32_t)(min(urow[i], last) * (int)tok_stride + lcol[i]);
            dma16(kbytes + row0, voff, st + i * 1024);
            dma16(vbytes + row0, voff, st + SLB + i * 1024);
        }
        // the scale-shift word of a (token row, head) sits at its byte offset / D
        dma4(ssp + row0 / D + (size_t)min(ss_tok, last) * (tok_stride / D), st + 2 * SLB);
    };

    float m = -INFINITY, l = 0.f;
    float pb = 0.f;  // sum over this lane's tokens of p_t * shift_t (V)
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (n_sl > 0) {
        // q rows of the head block (rows >= nh repeat the last head; zeroed below)
        const int nqi = (nh + QRPI - 1) / QRPI;
        for (int i = 0; i < nqi; ++i) {
            const int qr = QRPI * i + lane / QCPR;
            const int r = min(qr, nh - 1);
            const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow0 + r) * D +
                                 (((lane % QCPR) ^ swz<D>(qr)) * 8);
            dma16(qp, __builtin_amdgcn_readfirstlane(wlds_u + i * 1024));
        }
        const int pro = min(NST - 1, n_sl);
        for (int k = 0; k < pro; ++k) issue(k);
        wait_slices<PER_SLICE>(pro);

        // q^T as the B operand (lane: head l % 16, dims 32 ks + 8 (l / 16)..+7) and sum_d q_d
        const int hrow = lane & 15;
        const int kq = lane >> 4;
        u32x4 qop[KS];
        float qsum = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 x = lds16(wlds + hrow * QROWB + (((4 * ks + kq) ^ swz<D>(hrow)) << 4));
            qop[ks] = hrow < nh ? x : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) qsum += pair_sum(TAG(), qop[ks][e]);
        }
        qsum += shfl_xor(qsum, 16);
        qsum += xor32(qsum);
        // LDS offsets: K operand (row l % 16, bytes 32 ks + 8 (l / 16)..+7), V
        // conversion (row l / 4, quarter l % 4), transposed V reads
        int koff[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            koff[ks] = hrow * KROWB + (((2 * ks + (kq >> 1)) ^ swz8<D>(hrow)) << 4) + 8 * (kq & 1);
        const int vr = lane >> 2, vq = lane & 3;
        int vsrc[SCH], vdst[2 * SCH];
#pragma unroll
        for (int j = 0; j < SCH; ++j) vsrc[j] = SLB + vr * KROWB + (((vq * SCH + j) ^ swz8<D>(vr)) << 4);
#pragma unroll
        for (int j = 0; j < 2 * SCH; ++j) vdst[j] = vr * QROWB + (((vq * 2 * SCH + j) ^ swz<D>(vr)) << 4);
        int voff[NB];
        {
            const int j = lane & 15;
            const int r = 4 * kq + (j >> 2);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int c = 2 * nb + ((j & 3) >> 1);
                voff[nb] = r * QROWB + ((c ^ swz<D>(r)) << 4) + 8 * (j & 1);
            }
        }

        for (int k = 0; k < n_sl; ++k) {
            if (k + NST - 1 < n_sl) issue(k + NST - 1);
            wait_slices<PER_SLICE>(min(NST - 1, n_sl - 1 - k));

            const lds_char* st = wlds + QB + (k & (NST - 1)) * STB;
            const u32x4 kw = lds16(st + 2 * SLB + 16 * kq);       // tokens 4 kq .. +3: K scale-shift
            const u32x4 vw = lds16(st + 2 * SLB + 64 + 16 * kq);  // and V
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x2 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(st + koff[ks]);
                const u32x2 lo8 = e4m3x4_to16(TAG(), x[0]), hi8 = e4m3x4_to16(TAG(), x[1]);
                sc = mfma16x32(TAG(), u32x4{lo8[0], lo8[1], hi8[0], hi8[1]}, qop[ks], sc);
            }
            // this slice's V as 16-bit floats for the P.V product
#pragma unroll
            for (int j = 0; j < SCH; ++j) {
                const u32x4 x = lds16(st + vsrc[j]);
                const u32x2 a0 = e4m3x4_to16(TAG(), x[0]), a1 = e4m3x4_to16(TAG(), x[1]);
                const u32x2 a2 = e4m3x4_to16(TAG(), x[2]), a3 = e4m3x4_to16(TAG(), x[3]);
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(vcs + vdst[2 * j]) =
                    u32x4{a0[0], a0[1], a1[0], a1[1]};
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(vcs + vdst[2 * j + 1]) =
                    u32x4{a2[0], a2[1], a3[0], a3[1]};
            }
            // dequantized scores: scale * (q . x) + shift * sum(q)
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = fmaf(sc[r], half_lo(kw[r]), half_hi(kw[r]) * qsum);

            const int T = T0 + stride * k;
            if (T + kSlice > hi) {  // ragged last slice of the chunk
                const int tok = T + 4 * kq;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (tok + r >= hi) sc[r] = -INFINITY;
            }
            const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.c;
            if (__builtin_amdgcn_ballot_w64(lm > m + kRescaleLog2)) {
                float mt = fmaxf(lm, shfl_xor(lm, 16));
                mt = fmaxf(mt, xor32(mt));
                const float mn = fmaxf(m, mt);
                const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
                m = mn;
                l *= alpha;
                pb *= alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = lane_value(alpha, 4 * kq + r);  // acc row 4 (l/16) + r is head 4 (l/16) + r
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[nb][r] *= ar;
                }
            }
            const float mu = m == -INFINITY ? 0.f : m;
            float p[4], pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = fast_exp2(fmaf(sc[r], a.c, -mu));
                pv[r] = p[r] * half_lo(vw[r]);            // weight times the V row's scale
                pb = fmaf(p[r], half_hi(vw[r]), pb);      // and the V row's shift
            }
            l += (p[0] + p[1]) + (p[2] + p[3]);
            const u32x2 pop = {pack2(TAG(), pv[0], pv[1]), pack2(TAG(), pv[2], pv[3])};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16(TAG(), pop, lds_tr(vcs + voff[nb]), acc[nb]);
        }
    }

    // ---- merge the NW waves' partial results -------------------------------
    l += shfl_xor(l, 16);
    l += xor32(l);
    pb += shfl_xor(pb, 16);
    pb += xor32(pb);
    __syncthreads();  // every wave is done with its ring (and its loads have landed)
    constexpr int SROW = D + 4;                        // floats per padded row
    float* sacc = reinterpret_cast<float*>(smem_raw);  // [NW][16][SROW]
    float* sm = sacc + NW * 16 * SROW;                 // [NW][16]
    float* sl = sm + NW * 16;                          // [NW][16]
    float* sp = sl + NW * 16;                          // [NW][16]
    {
        const int kq = lane >> 4, c = lane & 15;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[(wave * 16 + 4 * kq + r) * SROW + 16 * nb + c] = acc[nb][r];
        if (lane < 16) {
            sm[wave * 16 + lane] = m;
            sl[wave * 16 + lane] = l;
            sp[wave * 16 + lane] = pb;
        }
    }
    __syncthreads();
    const size_t prow = qrow0 * a.n_splits + s;  // partial row of the block's first head
    // per head: the waves' weights relative to the largest running max,
    // divided by the head's sum, and its LSE
    float* se = sp + NW * 16;  // [NW][16]
    if (tid < nh) {
        const int h = tid;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * 16 + h]);
        float e[NW], L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = sm[w * 16 + h];
            e[w] = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
            L += e[w] * sl[w * 16 + h];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) se[w * 16 + h] = e[w] * inv;
        a.part_lse[prow + (size_t)h * a.n_splits] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    constexpr int V4 = D / 4;  // 16-byte pieces per row
    for (int i = tid; i < nh * V4; i += NW * 64) {
        const int h = i / V4, d = 4 * (i % V4);
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float e = se[w * 16 + h];
            const float shift = sp[w * 16 + h];
            const f32x4 x = *reinterpret_cast<const f32x4*>(sacc + (w * 16 + h) * SROW + d);
#pragma unroll
            for (int k = 0; k < 4; ++k) O[k] = fmaf(e, x[k] + shift, O[k]);
        }
        __builtin_nontemporal_store(O, reinterpret_cast<f32x4*>(a.part_o + (prow + (size_t)h * a.n_splits) * D + d));
    }
}

// Merge of the non-empty chunks' partial results of each query row (b, h, i),
// one wave per row (four rows per workgroup).  The LSEs and partial outputs of
// up to 16 chunks are loaded together, so a row costs one memory round trip
// per 16 chunks; the merge keeps a running maximum across those steps.  Chunks
// with LSE = -inf (no visible key) weigh 0.
template <class TAG, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;  // output dims per lane
    constexpr int CH = 16;       // chunks per step
    const int lane = threadIdx.x & 63;
    const long long rows = (long long)a.B * a.Hq * a.q_len;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * Hq + h) * q_len + i
    if (row >= rows) return;
    const int len = a.seq_lens[row / ((long long)a.Hq * a.q_len)];
    const int nv = len > 0 ? (len + chunk_tokens(len, a.n_splits) - 1) / chunk_tokens(len, a.n_splits) : 0;
    const float* pl = a.part_lse + row * a.n_splits;
    const float* po = a.part_o + row * a.n_splits * D + lane * PER;

    float M = -INFINITY, W = 0.f, O[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] = 0.f;
    for (int s0 = 0; s0 < nv; s0 += CH) {
        const int n = min(CH, nv - s0);
        const float lv = lane < n ? pl[s0 + lane] : -INFINITY;
        float x[CH][PER];
#pragma unroll
        for (int u = 0; u < CH; ++u)  // chunks past n repeat the last one (their weight is 0)
#pragma unroll
            for (int i = 0; i < PER; ++i) x[u][i] = po[(size_t)min(s0 + u, nv - 1) * D + i];
        float mb = lv;
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) mb = fmaxf(mb, shfl_xor(mb, k));
        const float mn = fmaxf(M, mb);
        if (mn == -INFINITY) continue;  // no non-empty chunk so far
        const float sc = M == -INFINITY ? 0.f : fast_exp2((M - mn) * kLog2e);
        M = mn;
        W *= sc;
#pragma unroll
        for (int i = 0; i < PER; ++i) O[i] *= sc;
        const float w = lv == -INFINITY ? 0.f : fast_exp2((lv - M) * kLog2e);
        W += w;  // this lane's chunk (summed over the wave below)
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
            for (int i = 0; i < PER; ++i) O[i] = fmaf(wu, x[u][i], O[i]);
        }
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) W += shfl_xor(W, k);
    const float inv = W > 0.f ? 1.f / W : 0.f;
    uint16_t* op = static_cast<uint16_t*>(a.o) + (size_t)row * D + lane * PER;
    if (PER == 2) {
        *reinterpret_cast<uint32_t*>(op) = pack2(TAG(), O[0] * inv, O[PER - 1] * inv);
    } else {
        const uint32_t w = pack2(TAG(), O[0] * inv, 0.f);
        *op = (uint16_t)(w & 0xffff);
    }
    if (lane == 0) a.lse[row] = W > 0.f ? M + fast_log2(W) * kLn2 : -INFINITY;
}

template <class TAG, int D, int PG, bool BIAS = false>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
    const long long n_hb = ((long long)a.group * a.q_len + 15) / 16;
    const long long blocks = (long long)a.B * a.Hkv * n_hb * a.n_splits;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_split_kernel<TAG, D, DEC_NW, DEC_NST, PG, BIAS>), dim3((unsigned)blocks),
                       dim3(DEC_NW * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.Hq * a.q_len;
    if ((rows + 3) / 4 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_combine_kernel<TAG, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <class TAG, int D, int PG>
hipError_t launch_split_fp8(const DecodeArgs& a, hipStream_t stream) {
    const long long n_hb = (a.group + 15) / 16;
    const long long blocks = (long long)a.B * a.Hkv * n_hb * a.n_splits;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_split_kernel_fp8<TAG, D, DEC8_NW, DEC8_NST, PG>), dim3((unsigned)blocks),
                       dim3(DEC8_NW * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<TAG, D>), dim3((unsigned)(((long long)a.B * a.Hq + 3) / 4)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

template <class TAG>
hipError_t dispatch_fp8(const DecodeArgs& a, hipStream_t stream) {
    const bool paged = a.block_table != nullptr;
    if (a.D == 64)
        return paged ? launch_split_fp8<TAG, 64, kPaged>(a, stream) : launch_split_fp8<TAG, 64, kDense>(a, stream);
    return paged ? launch_split_fp8<TAG, 128, kPaged>(a, stream) : launch_split_fp8<TAG, 128, kDense>(a, stream);
}

template <class TAG, int D, bool BIAS>
hipError_t dispatch_layout(const DecodeArgs& a, hipStream_t stream) {
    if (a.block_table == nullptr) return launch_split<TAG, D, kDense, BIAS>(a, stream);
    if (a.page_shift >= 4) return launch_split<TAG, D, kPaged, BIAS>(a, stream);
    return launch_split<TAG, D, kPagedSmall, BIAS>(a, stream);
}

template <class TAG>
hipError_t dispatch_d(const DecodeArgs& a, hipStream_t stream) {
    if (a.bias) {
        if (a.D == 64) return dispatch_layout<TAG, 64, true>(a, stream);
        return dispatch_layout<TAG, 128, true>(a, stream);
    }
    if (a.D == 64) return dispatch_layout<TAG, 64, false>(a, stream);
    return dispatch_layout<TAG, 128, false>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    if (dtype == kDtypeBF16) return dispatch_d<bf16_tag>(a, stream);
    return dispatch_d<f16_tag>(a, stream);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int dtype, hipStream_t stream) {
    if (dtype == kDtypeBF16) return dispatch_fp8<bf16_tag>(a, stream);
    return dispatch_fp8<f16_tag>(a, stream);
}

}  // namespace gqa
