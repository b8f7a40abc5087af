// prefill_pp.hip - attention forward (prefill), ping-pong schedule.
//
// Method as in prefill_fwd.hip: FlashAttention forward with an online softmax
// (causal_forward_kernel.py, `_flash_attention_forward_gqa_kernel`), the
// bottom-right causal mask of the FlashInfer-style prefill page
// (gpt-o3 / triton6fd1ef, `_gqa_prefill_kernel`) and the zero-fill of empty
// rows of splitk_kernels.py (`_fwd_kernel_splitK`).
//
// Schedule.  On gfx950 the softmax of a 64-key x 32-query tile costs about as
// many VALU cycles as the tile's 32 MFMAs, so matrix and vector work must
// overlap.  A workgroup is 8 wave64s (two per SIMD), each owning 32 query
// rows; the waves form two groups (waves 0-3 and 4-7, one of each per SIMD)
// that run the same phase sequence one phase apart:
//
//     MFMA phase of tile t:  S(t) = K(t) Q^T, then acc += V(t-1) P(t-1)
//     VALU phase of tile t:  mask, row max, lazy rescale, P(t) = exp2(...)
//
// separated by workgroup barriers, so while one wave of a SIMD issues MFMAs
// the other runs its softmax.  K and V tiles (64 keys) are loaded straight
// from global memory into four LDS stages (global_load_lds_dwordx4), two
// tiles ahead; V stays row-major and is read with ds_read_b64_tr_b16 into
// the P.V MFMA's A operand.
#include "gqa_device.hpp"
#include "gqa_kernels.hpp"

namespace gqa {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kRescaleLog2p = 8.f;

#ifndef PP_AHEAD
#define PP_AHEAD 8
#endif

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x8;
constexpr int kSchedDsRead = 0x100;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence (outstanding direct-to-LDS loads
// of later tiles stay in flight); the empty asm statements keep the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);  // no instruction moves across a phase boundary
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __asm__ __volatile__("" ::: "memory");
}

// 16 bytes per lane from global memory into LDS (lane i -> lds_base + 16 i).
// Inline asm so the compiler's wait-count pass does not make every later LDS
// read wait for it; completion is awaited explicitly (vmcnt + barrier).
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
    __asm__ __volatile__("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(gptr), "s"(lds_base)
                         : "m0");
}

// Marks a register value as consumed here.  The softmax arithmetic is pure
// and feeds only the next phase's MFMAs, so without this the compiler sinks it
// across the phase barrier into the MFMA phase.
__device__ __forceinline__ void pin(uint32_t& x) { __asm__ __volatile__("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { __asm__ __volatile__("" : "+v"(x)); }

__device__ __forceinline__ u32x2 lds_read_tr(const lds_char* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
    return __builtin_bit_cast(u32x2, v);
}

// LDS tile layout: rows of D*2 bytes, 16-byte chunk c of row r stored at chunk
// position c ^ swz<D>(r).  LDS has 64 banks of 4 bytes: a 16-byte read is
// served 16 lanes at a time and an 8-byte read 32 lanes at a time, so a read
// is conflict-free when those lanes cover 16 distinct 16-byte bank groups.
// K operand reads: 16 lanes = 16 consecutive rows at one chunk; transposed V
// reads: 32 lanes = 4 consecutive rows x 4 adjacent chunks.  D = 128: one row
// spans all 64 banks, group = position, and swz is a bijection on r % 16 whose
// value >> 2 differs across any 4 aligned rows.  D = 64: two rows per bank
// row, group = 8 (r % 2) + position, and swz is a bijection on (r >> 1) % 8
// differing in bit 2 between rows r and r + 2.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// 16 bytes per lane into LDS from a wave-uniform base address (SGPRs) plus a
// 32-bit per-lane byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    __asm__ __volatile__("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                         :
                         : "v"(voff), "s"(sbase), "s"(lds_base)
                         : "m0");
}

// 4 bytes per lane from global memory into LDS (lane i -> lds_base + 4 i).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
    __asm__ __volatile__("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                         :
                         : "v"(gptr), "s"(lds_base)
                         : "m0");
}

// PAGED: a batch of ragged requests over a paged K/V cache (the FlashInfer-style
// prefill page's `run`: query tokens of request b at qo_indptr[b] .., its key
// pages kv_indices[kv_indptr[b] ..]), q / o token-major [total_q, Hq, D], lse
// [total_q, Hq].  The page id of every key row of a tile is brought into a
// per-wave LDS ring by a direct load two tiles before the tile itself, so the
// tile loads read their page ids from LDS.
// 16-bit additive bias element -> fp32
__device__ __forceinline__ float bias_f32(bf16_tag, uint32_t u16) { return __builtin_bit_cast(float, u16 << 16); }
__device__ __forceinline__ float bias_f32(f16_tag, uint32_t u16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
}

// BIAS (dense keys, D = 128, whole 64-key tiles, 16-byte aligned bias rows):
// the additive bias of splitk_kernels.py (`_fwd_kernel_splitK`,
// HAS_ADDITIVE_BIAS).  Each wave brings the bias of its 32 rows for the next
// tile into its own 4 KB LDS buffer by direct loads at the end of its softmax
// phase, next to its part of the K/V tiles, and adds it to the scores at the
// start of the following softmax phase.
template <class TAG, int D, bool CAUSAL, int NH, bool PAGED, bool BIAS = false>
__global__ __launch_bounds__(512, 1) void prefill_fwd_pp(PrefillArgs a) {
    constexpr int NW = 8;                  // waves per workgroup
    constexpr int BN = 64;                 // keys per tile
    constexpr int WPH = NW / NH;           // waves per head
    constexpr int POS = 32 * WPH;          // query positions per workgroup
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int ROWB = D * 2;
    constexpr int TILEB = BN * ROWB;
    constexpr int STAGEB = 2 * TILEB;
    constexpr int NST = 4;
    constexpr int DS = D / 16;
    constexpr int DT = D / 32;
    constexpr int LPW = CPR / NW;          // direct-load instructions per wave per tile, each of K and V
    static_assert(LPW >= 1, "tile too small for the workgroup");
    typedef typename TAG::vec8 vec8;

    __shared__ __attribute__((aligned(1024))) char smem_raw[NST * STAGEB];
    lds_char* smem = (lds_char*)smem_raw;
    // PAGED: page ids of the rows of tiles t .. t + 3, ring slot t % NST, per wave
    // BIAS: one 4 KB buffer per wave (32 rows x 64 keys); PAGED and BIAS never
    // meet, so the page ring and the bias buffers share one array (the bias
    // kernel's LDS is then 160 KB in all)
    constexpr int BWB = 32 * BN * 2;       // BIAS: bytes of one wave's bias buffer
    constexpr int BW = BWB / 1024;         // BIAS: direct loads per wave per tile
    static_assert(!BIAS || (!PAGED && D == 128), "bias: dense keys, D = 128");
    __shared__ __attribute__((aligned(16))) char aux_raw[PAGED ? NW * NST * BN * 4 : (BIAS ? NW * BWB : 16)];
    int* pg_ring = reinterpret_cast<int*>(aux_raw);
    [[maybe_unused]] char* bias_raw = aux_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;             // ping-pong group: 0 leads, 1 trails by one phase
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // ---- work item ----------------------------------------------------------
    // (position tile, head block, kv head, batch[, key range]), key range fastest
    int id = blockIdx.x;
    int split = 0;
    if (a.kv_splits > 1) {
        split = id % a.kv_splits;
        id /= a.kv_splits;
    }
    const int hgroups = a.group / NH;
    int pt, hg, g, b;
    bool from_end = false;  // PAGED: position tile counted from the request's last query
    if (PAGED && a.B <= 512) {
        // Ragged batch: only real items (request, position tile counted from the
        // request's end), longest first across the whole batch (ragged_item),
        // the heads fastest.  Workgroups past the last item (the grid is sized
        // by the longest request) come last and exit, so that they do not hold
        // up the dispatch of real work.
        const int n_hk = a.Hkv * hgroups;
        int item = id / n_hk;
        int hk = id - item * n_hk;
        hg = hk % hgroups;
        g = hk / hgroups;
        b = ragged_item<POS>(a.qo_indptr, a.kv_indptr, a.kv_last_page_len, a.page_shift, a.B, a.n_pos_tiles,
                             item, pt);
        if (b < 0) return;  // workgroup-uniform, before any barrier: no item left
        from_end = true;
    } else {
        int rest;
        if (!PAGED && a.xcd_order) {
            // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs
            // (blockIdx % 8) and XCD x takes the x-th eighth of the items in
            // (head block, position tile) order, so the workgroups one XCD runs
            // at a time share a few heads' K/V in its L2 instead of streaming
            // every head it hosts once per round of position tiles
            int item = id;
            const int q8 = a.n_pos_tiles * a.n_rest / 8;
            if (item < 8 * q8) item = (item % 8) * q8 + item / 8;
            pt = item % a.n_pos_tiles;
            rest = item / a.n_pos_tiles;
        } else {
            pt = id / a.n_rest;
            rest = id - pt * a.n_rest;
        }
        if (CAUSAL) pt = a.n_pos_tiles - 1 - pt;  // longest rows first
        hg = rest % hgroups;
        rest /= hgroups;
        g = rest % a.Hkv;
        b = rest / a.Hkv;
    }
    const int h = g * a.group + hg * NH + wave / WPH;

    // ---- the request: query rows, keys, causal offset ------------------------
    int q_len = a.q_len, kv_len = a.kv_len, delta = a.delta;
    size_t q_tok0 = 0;  // PAGED: first query token of the request
    int kv_page0 = 0;   // PAGED: first entry of its page list
    if constexpr (PAGED) {
        q_tok0 = (size_t)a.qo_indptr[b];
        q_len = a.qo_indptr[b + 1] - (int)q_tok0;
        kv_page0 = a.kv_indptr[b];
        const int n_pages = a.kv_indptr[b + 1] - kv_page0;
        kv_len = n_pages > 0 ? ((n_pages - 1) << a.page_shift) +
                                   (a.kv_last_page_len ? a.kv_last_page_len[b] : (1 << a.page_shift))
                             : 0;
        delta = kv_len - q_len;
    }
    // first query position of the workgroup (bottom-aligned tiles may start
    // before the request's first query: those rows are not computed or stored)
    const int wg_pos0 = from_end ? q_len - (pt + 1) * POS : pt * POS;
    if (PAGED && wg_pos0 >= q_len) return;  // workgroup-uniform, before any barrier: past the request's queries
    const int pos0 = wg_pos0 + (wave % WPH) * 32;
    const int my_q = pos0 + l32;
    const bool row_ok = my_q >= 0 && my_q < q_len;

    int wg_kv_end = kv_len, wave_full_end = kv_len;
    if (CAUSAL) {
        const int wg_last = min(wg_pos0 + POS, q_len) - 1;
        wg_kv_end = max(0, min(kv_len, wg_last + delta + 1));
        wave_full_end = max(0, min(kv_len, pos0 + delta + 1));
    }
    // this workgroup's key tiles t_lo .. t_lo + n_tiles - 1 (all of them unless
    // the keys are split); loop indices below are relative to t_lo
    const int n_all = (wg_kv_end + BN - 1) / BN;
    const int n_split = a.kv_splits > 1 ? a.kv_splits : 1;
    const int per_split = (n_all + n_split - 1) / n_split;
    const int t_lo = min(n_all, split * per_split);
    const int n_tiles = min(n_all, t_lo + per_split) - t_lo;
    const int n_full = min(wave_full_end / BN, n_all) - t_lo;  // relative tiles below it need no mask
    const int lim = CAUSAL ? min(my_q + delta + 1, kv_len) : kv_len;  // keys < lim are visible

    // element offset of query row `row` of head h in q / o, and its LSE index
    const size_t q_head = ((size_t)b * a.Hq + h) * (size_t)q_len;
    auto row_elt = [&](int row) -> size_t {
        if constexpr (PAGED) return ((q_tok0 + row) * a.Hq + h) * (size_t)D;
        return (q_head + row) * (size_t)D;
    };
    auto lse_idx = [&](int row) -> size_t {
        if constexpr (PAGED) return (q_tok0 + row) * a.Hq + h;
        return q_head + row;
    };
    const size_t o_row_bytes = PAGED ? (size_t)a.Hq * ROWB : (size_t)ROWB;

    // ---- Q (B operand of S^T = K Q^T) ---------------------------------------
    // Each wave's 32 rows reach LDS by direct loads, whole rows per
    // instruction, in the layout of a K tile (chunk c of row r at position
    // c ^ swz(r)) inside ring stages 2 and 3, which no tile occupies before the
    // first barrier; the operands are read back from there before it.  (Loading
    // the operands straight into registers touches each 128-byte line of Q
    // from four instructions, 32 lines per instruction.)
    vec8 qf[DS];
    const int q_stage_off = 2 * STAGEB + wave * (32 * ROWB);
    auto issue_q = [&]() {
        const uint16_t* qb = static_cast<const uint16_t*>(a.q);
        const uint32_t dst = (uint32_t)(uintptr_t)(smem + q_stage_off);
#pragma unroll
        for (int j = 0; j < CPR / 2; ++j) {
            const int p = j * 64 + lane;
            const int r = p / CPR;
            const int c = (p % CPR) ^ swz<D>(r);
            const int row = min(max(pos0 + r, 0), q_len - 1);
            dma16(qb + row_elt(row) + c * 8, __builtin_amdgcn_readfirstlane(dst + j * 1024));
        }
    };

    // ---- direct global -> LDS tile loads --------------------------------------
    // dense: the (b, g) plane; PAGED: head g inside the pool's token rows
    const size_t kv_head = PAGED ? (size_t)g : ((size_t)b * a.Hkv + g) * (size_t)kv_len;
    const char* kg = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k) + kv_head * D);
    const char* vg = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v) + kv_head * D);
    const int last_key = kv_len - 1;
    const int page_mask = PAGED ? (1 << a.page_shift) - 1 : 0;
    const size_t tok_bytes = PAGED ? (size_t)a.Hkv * ROWB : (size_t)ROWB;  // bytes between key rows
    int ld_row[LPW], ld_col[LPW];
    [[maybe_unused]] uint32_t ld_voff[LPW];  // byte offset of the lane's chunk in a dense tile
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int p = (wave * LPW + j) * 64 + lane;  // chunk position in the tile
        const int row = p / CPR, pc = p % CPR;
        ld_row[j] = row;
        ld_col[j] = (pc ^ swz<D>(row)) * 16;
        ld_voff[j] = (uint32_t)(row * ROWB + ld_col[j]);
    }
    // PAGED: this wave's page-id ring; lane i of the load for tile t fetches the
    // page of key row i
    const int* pg_wave = pg_ring + (PAGED ? wave * NST * BN : 0);
    auto issue_pages = [&](int t) {
        if constexpr (PAGED) {
            const int key = min((t_lo + t) * BN + lane, last_key);
            const int* src = a.kv_indices + kv_page0 + (key >> a.page_shift);
            dma4(src, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(pg_wave + (t % NST) * BN)));
        }
    };
    auto issue_tile = [&](int t) {
        const int t0 = (t_lo + t) * BN;
        lds_char* st = smem + (t % NST) * STAGEB;
        if (!PAGED && t0 + BN <= kv_len) {
            // a whole dense tile: one uniform base per tile, constant lane offsets
            const char* kb = kg + (size_t)t0 * ROWB;
            const char* vb = vg + (size_t)t0 * ROWB;
#pragma unroll
            for (int j = 0; j < LPW; ++j) {
                const uint32_t dst = (uint32_t)(uintptr_t)(st + (wave * LPW + j) * 1024);
                dma16(kb, ld_voff[j], dst);
                dma16(vb, ld_voff[j], dst + TILEB);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int key = min(t0 + ld_row[j], last_key);
            size_t off;
            if constexpr (PAGED) {
                const int page = pg_wave[(t % NST) * BN + ld_row[j]];
                off = (((size_t)page << a.page_shift) + (size_t)(key & page_mask)) * tok_bytes + ld_col[j];
            } else {
                off = (size_t)key * ROWB + ld_col[j];
            }
            const uint32_t dst = (uint32_t)(uintptr_t)(st + (wave * LPW + j) * 1024);
            dma16(kg + off, __builtin_amdgcn_readfirstlane(dst));
            dma16(vg + off, __builtin_amdgcn_readfirstlane(dst + TILEB));
        }
    };

    // BIAS: rows pos0 .. pos0 + 31 of the bias for the keys of tile t; 16-byte
    // chunk c of row r at chunk position c ^ (r & 7) of a 128-byte LDS row
    [[maybe_unused]] auto issue_bias = [&](int t) {
        if constexpr (BIAS) {
            const int k0 = (t_lo + t) * BN;
            const uint16_t* bh = a.bias + (long long)b * a.bias_sb + (long long)h * a.bias_sh + k0;
            const uint32_t dst = (uint32_t)(uintptr_t)((lds_char*)bias_raw + wave * BWB);
#pragma unroll
            for (int j = 0; j < BW; ++j) {
                const int p = j * 64 + lane;
                const int r = p >> 3, c = (p & 7) ^ (r & 7);
                const int row = min(max(pos0 + r, 0), q_len - 1);
                dma16(bh + (long long)row * a.bias_sq + c * 8, __builtin_amdgcn_readfirstlane(dst + j * 1024));
            }
        }
    };

    // ---- per-lane LDS read offsets ---------------------------------------------
    int k_off[DS];  // K operand: row l32 (+32 kh), chunk 2 ds + half
    {
        const int sw = swz<D>(l32);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) k_off[ds] = l32 * ROWB + (((2 * ds + half) ^ sw) * 16);
    }
    // V operand through transposed reads: in each 16-lane group, source lane s
    // reads row kbase + s/4, dims d0 + 4 (s%4) .. +3 with d0 = 32 dt + 16 ((lane/16)&1)
    // and kbase = 16 k16 + 8 rd + 4 half; it returns 4 consecutive keys of one dim.
    int v_off[2][DT];  // [rd][dt]: the two 4-key halves of each 16-key step
    {
        const int s = lane & 15;
        const int g1 = (lane >> 4) & 1;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int rsub = 8 * rd + 4 * half + (s >> 2);  // row inside the 16-row block
            const int sw = swz<D>(rsub);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int c = 4 * dt + 2 * g1 + ((s & 3) >> 1);
                v_off[rd][dt] = rsub * ROWB + ((c ^ sw) * 16) + (s & 1) * 8;
            }
        }
    }

    // ---- state -------------------------------------------------------------------
    float m = -INFINITY;
    float l = 0.f;            // this lane's share of the row sum (its half of the keys)
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    f32x16 s[2];               // S^T of the current tile, two 32-key halves
    uint32_t pk[16];           // packed P of the previous tile (pairs of keys)

    // MFMA phase pieces: the scores of tile t, and the P.V of tile t-1
    auto scores = [&](int t) {
        const lds_char* sk = smem + (t % NST) * STAGEB;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kh][r] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const vec8 ka = *reinterpret_cast<const __attribute__((address_space(3))) vec8*>(
                    sk + kh * 32 * ROWB + k_off[ds]);
                s[kh] = mfma_32x32x16(ka, qf[ds], s[kh]);
            }
    };
    auto pv = [&](int t) {  // P.V of tile t - 1
        const lds_char* sv = smem + ((t - 1) % NST) * STAGEB + TILEB;
#pragma unroll
        for (int k16 = 0; k16 < 4; ++k16) {
            const u32x4 pw = {pk[4 * k16], pk[4 * k16 + 1], pk[4 * k16 + 2], pk[4 * k16 + 3]};
            const vec8 pb = __builtin_bit_cast(vec8, pw);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x2 lo = lds_read_tr(sv + 16 * k16 * ROWB + v_off[0][dt]);
                const u32x2 hi = lds_read_tr(sv + 16 * k16 * ROWB + v_off[1][dt]);
                const u32x4 vw = {lo[0], lo[1], hi[0], hi[1]};
                acc[dt] = mfma_32x32x16(__builtin_bit_cast(vec8, vw), pb, acc[dt]);
            }
        }
    };
    // Interior MFMA phase (0 < t < n_tiles): one basic block, operand reads
    // kept about eight MFMAs ahead of their use (LDS latency is several
    // MFMA issue slots).
    auto mfma_phase = [&](int t) {
        scores(t);
        pv(t);
        constexpr int NS = 2 * DS;   // score MFMAs (one K read each)
        constexpr int NP = 4 * DT;   // P.V MFMAs (two transposed reads each)
        constexpr int AHEAD = PP_AHEAD;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD, 0);
#pragma unroll
        for (int i = 0; i < NS - AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
#pragma unroll
        for (int i = 0; i < NP - AHEAD / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i < NP - AHEAD) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
    };
    auto scores_only = [&](int t) {
        scores(t);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
        for (int i = 0; i < 2 * DS; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i + 8 < 2 * DS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
    };
    auto pv_only = [&](int t) {
        pv(t);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
        for (int i = 0; i < 4 * DT; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (i + 4 < 4 * DT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
    };

    // VALU phase of tile t: mask, row max, lazy rescale, weights
    auto valu_phase = [&](int t) {
        if constexpr (BIAS) {
            // this wave's bias of tile t: its loads were followed only by its
            // part of tile t + 1 + grp (tile 0's bias is waited for with Q)
            if (t > 0) {
                if (t + 1 + grp < n_tiles) wait_vmcnt<2 * LPW>();
                else wait_vmcnt<0>();
                __asm__ __volatile__("" ::: "memory");
            }
            const lds_char* bb = (const lds_char*)bias_raw + wave * BWB + l32 * (BN * 2) + half * 8;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const u32x2 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
                        bb + (((kh * 4 + r4) ^ (l32 & 7)) * 16));
                    // keys 32 kh + 8 r4 + 4 half + 0..3: s * c gains log2(e) * bias (bias_k = 1 / scale)
                    s[kh][4 * r4] = fmaf(bias_f32(TAG(), w[0] & 0xffffu), a.bias_k, s[kh][4 * r4]);
                    s[kh][4 * r4 + 1] = fmaf(bias_f32(TAG(), w[0] >> 16), a.bias_k, s[kh][4 * r4 + 1]);
                    s[kh][4 * r4 + 2] = fmaf(bias_f32(TAG(), w[1] & 0xffffu), a.bias_k, s[kh][4 * r4 + 2]);
                    s[kh][4 * r4 + 3] = fmaf(bias_f32(TAG(), w[1] >> 16), a.bias_k, s[kh][4 * r4 + 3]);
                }
        }
        if (t >= n_full) {  // diagonal / tail tile
            const int k0 = (t_lo + t) * BN;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    s[kh][r] = key < lim ? s[kh][r] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
        mx = fmaxf(mx, xor32(mx));
        const float mt = mx * a.c;
        // lazy rescale: the reference max moves only when a row max grew by more
        // than 2^kRescaleLog2p; acc and l share it, so O and the LSE are unchanged
        if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleLog2p)) {
            const float m_new = fmaxf(m, mt);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }
        const float mu = m == -INFINITY ? 0.f : m;
        float ls = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(s[kh][r], a.c, -mu));
                const float p1 = fast_exp2(fmaf(s[kh][r + 1], a.c, -mu));
                pk[kh * 8 + (r >> 1)] = pack2(TAG(), p0, p1);
                ls += p0 + p1;  // row sum of the unrounded weights
            }
        l += ls;
        // the weights are computed here, in the VALU phase, not next to the MFMAs that use them
#pragma unroll
        for (int i = 0; i < 16; ++i) pin(pk[i]);
        pin(l);
    };

    // ---- phase sequence ------------------------------------------------------------
    // Global phase p: group 0 runs step q = p of its sequence, group 1 step
    // q = p - 1; every wave passes one barrier per phase (2 n_tiles + 2 in all).
    // A wave's own steps: scores of tile 0, then (softmax of tile t, MFMAs of
    // tile t+1: scores of t+1 and P.V of t) for each t, the last P.V alone.
    // Tile t must be in LDS (this wave's loads done, then the barrier) from
    // phase 2t on.  Issuing a tile's loads slows the issuing wave for a few
    // hundred cycles, so dense tiles are issued where a wave has slack before
    // a barrier: at the end of its own softmax phase.  Group 0 issues its part
    // of tile t+2 after its softmax of tile t (between barriers 2t+1 and
    // 2t+2), group 1 its part of tile t+3 after its softmax of tile t
    // (between barriers 2t+2 and 2t+3; tile 2 in its idle first phase).  Stage
    // j % NST then held tile j-4, whose last reader (group 1's P.V, in the
    // phase after barrier 2j-5) is done.  At barrier 2t each wave's only loads
    // younger than tile t's are tile t+1's.
    // (D = 64 tiles take half the loads and measure better issued right after
    // the barrier.)  PAGED and D = 64: tile t+2 is issued by every wave right
    // after the barrier of phase 2t, and the page ids of tile t + 4 right after
    // it, so at phase 2t the loads younger than those of tile t + 2's pages are
    // tile t+1's and the pages of t + 3.
    constexpr bool kLateIssue = !PAGED && D == 128;
    if (n_tiles > 0) {
        issue_q();
        issue_bias(0);
        if constexpr (PAGED) {
            issue_pages(0);
            if (n_tiles > 1) issue_pages(1);
            wait_vmcnt<0>();
            __asm__ __volatile__("" ::: "memory");  // the page ids are read below
        }
        issue_tile(0);
        if (n_tiles > 2) issue_pages(2);
        if (n_tiles > 1) issue_tile(1);
        if (n_tiles > 3) issue_pages(3);
        // Q (and tile 0) in LDS: read the operands, and finish reading them
        // before the first barrier, after which tile 2 goes to stage 2
        if constexpr (!PAGED) {
            if (n_tiles > 1) wait_vmcnt<2 * LPW>();
            else wait_vmcnt<0>();
        }
        __asm__ __volatile__("" ::: "memory");  // the direct loads wrote LDS
        {
            const lds_char* sq = smem + q_stage_off;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
                qf[ds] = *reinterpret_cast<const __attribute__((address_space(3))) vec8*>(sq + k_off[ds]);
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
        int p = 0;
        auto sync = [&]() {
            if ((p & 1) == 0) {
                const int t = p >> 1;
                if (t < n_tiles) {
                    if (PAGED && t + 3 < n_tiles) wait_vmcnt<2 * LPW + 1>();   // tile t, pages of t + 2
                    else if (BIAS) {
                        // after tile t this wave issued the bias of tile t (group 0 from
                        // t = 1 on, group 1 from t = 2 on) and its part of tile t + 1
                        const bool b_after = t > 1 || (t == 1 && grp == 0);
                        if (b_after && t + 1 < n_tiles) wait_vmcnt<BW + 2 * LPW>();
                        else if (b_after) wait_vmcnt<BW>();
                        else if (t + 1 < n_tiles) wait_vmcnt<2 * LPW>();
                        else wait_vmcnt<0>();
                    } else if (t + 1 < n_tiles) wait_vmcnt<2 * LPW>();          // tile t (pages of t + 2 if any)
                    else wait_vmcnt<0>();
                }
            }
            barrier_no_fence();
            if constexpr (!kLateIssue) {
                if ((p & 1) == 0 && (p >> 1) + 2 < n_tiles) {
                    issue_tile((p >> 1) + 2);
                    if ((p >> 1) + 4 < n_tiles) issue_pages((p >> 1) + 4);
                }
            }
            ++p;
        };
        if (grp) {  // group 1 starts one phase later
            sync();
            if (kLateIssue && n_tiles > 2) issue_tile(2);
        }
        sync();
        scores_only(0);
        for (int t = 0; t + 1 < n_tiles; ++t) {
            sync();
            valu_phase(t);
            if (BIAS) issue_bias(t + 1);  // before the tile: the next softmax phase waits for it alone
            if (kLateIssue && t + 2 + grp < n_tiles) issue_tile(t + 2 + grp);
            sync();
            mfma_phase(t + 1);
        }
        sync();
        valu_phase(n_tiles - 1);
        sync();
        pv_only(n_tiles);
        if (!grp) sync();  // group 0 waits out the last phase of group 1
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------------
    // The wave's 32 rows are consecutive in o (PAGED: one row of head h every
    // Hq rows).  They are staged in LDS and
    // written as whole rows (a store instruction covers 64 / CPR full rows).
    // Staging area: wave w uses 32 rows of stage (n_tiles + w / 4) % NST, which
    // no wave reads any more (the last tile, still read by group 1's final
    // P.V, sits in stage (n_tiles - 1) % NST) and no load writes (tiles past
    // the last are never issued).  Each wave reads back only what it wrote.
    const float l_tot = l + xor32(l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (!PAGED && a.kv_splits > 1) {
        // partial result of this key range: O_s = acc / l (0 when none of its
        // keys is visible to the row) and LSE_s (-inf then), both fp32
        if (my_q < q_len) {
            const size_t prow = (q_head + my_q) * a.kv_splits + split;
            float* po = a.part_o + prow * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<f32x4*>(po + dt * 32 + 8 * r4 + 4 * half) =
                        f32x4{acc[dt][4 * r4] * inv, acc[dt][4 * r4 + 1] * inv, acc[dt][4 * r4 + 2] * inv,
                              acc[dt][4 * r4 + 3] * inv};
            if (half == 0) a.part_lse[prow] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
        }
        return;
    }
    {
        u32x4 chunk[2 * DT];
        acc_row_chunks(TAG(), acc, inv, chunk);
        lds_char* ob = smem + ((n_tiles + wave / 4) % NST) * STAGEB + (wave % 4) * (32 * ROWB);
        // 16-byte chunk c of row r sits at chunk position c ^ oswz(r): conflict-free
        // for both the row-per-lane writes and the chunk-per-lane reads
        auto oswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
#pragma unroll
        for (int j = 0; j < 2 * DT; ++j) {
            const int c = 4 * (j >> 1) + 2 * half + (j & 1);
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(ob + l32 * ROWB + ((c ^ oswz(l32)) << 4)) =
                chunk[j];
        }
        constexpr int RPI = 64 / CPR;  // rows per store instruction
        char* og0 = reinterpret_cast<char*>(static_cast<uint16_t*>(a.o) + row_elt(0));  // the head's row 0
        const int cc = lane % CPR;
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int rr = RPI * k + lane / CPR;
            const u32x4 v =
                *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(ob + rr * ROWB + ((cc ^ oswz(rr)) << 4));
            const int row = pos0 + rr;
            if (row >= 0 && row < q_len)
                // whole 128-byte lines: streamed past L2 (non-temporal), so the
                // output does not evict K/V tiles other workgroups still read
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(og0 + (size_t)row * o_row_bytes + cc * 16));
        }
    }
    if (row_ok && half == 0) a.lse[lse_idx(my_q)] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

// Merge of the key ranges of a split-KV prefill, the LSE merge of the split-K
// decode (splitk_kernels.py, `_splitK_reduce`): per query row, M = max_s LSE_s,
// w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s, LSE = M + log(sum w_s); a row
// with no visible key in any range gives (0, -inf).  One thread per 8 output
// dims of a row.
template <class TAG, int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a, long long rows) {
    constexpr int G = D / 8;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * G) return;
    const long long row = i / G;
    const int d0 = (int)(i - row * G) * 8;
    const int S = a.kv_splits;
    const float* pl = a.part_lse + row * S;
    // ranges in groups of 8: every LSE and partial output of a group is loaded
    // before any is used (an empty range holds (0, -inf): weight 0 on a zero
    // row), with a running maximum across groups
    float M = -INFINITY, W = 0.f, O[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float lv[8];
        f32x4 x0[8], x1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 + k < S) {
                const float* po = a.part_o + (row * S + s0 + k) * D + d0;
                lv[k] = pl[s0 + k];
                x0[k] = *reinterpret_cast<const f32x4*>(po);
                x1[k] = *reinterpret_cast<const f32x4*>(po + 4);
            }
        }
        float mg = -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (s0 + k < S) mg = fmaxf(mg, lv[k]);
        const float Mn = fmaxf(M, mg);
        if (Mn > M && M != -INFINITY) {  // a later group raised the maximum
            const float r = fast_exp2((M - Mn) * kLog2e);
            W *= r;
#pragma unroll
            for (int e = 0; e < 8; ++e) O[e] *= r;
        }
        M = Mn;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 + k < S) {
                const float w = lv[k] == -INFINITY ? 0.f : fast_exp2((lv[k] - M) * kLog2e);
                W += w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    O[e] += w * x0[k][e];
                    O[4 + e] += w * x1[k][e];
                }
            }
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    const u32x4 packed = {pack2(TAG(), O[0] * inv, O[1] * inv), pack2(TAG(), O[2] * inv, O[3] * inv),
                          pack2(TAG(), O[4] * inv, O[5] * inv), pack2(TAG(), O[6] * inv, O[7] * inv)};
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + row * D + d0) = packed;
    if (d0 == 0) a.lse[row] = W > 0.f ? M + fast_log2(W) * kLn2 : -INFINITY;
}

template <class TAG, int D, bool CAUSAL, int NH, bool PAGED, bool BIAS = false>
hipError_t launch_pp(PrefillArgs a, hipStream_t stream) {
    constexpr int POS = 256 / NH;
    a.n_pos_tiles = (a.q_len + POS - 1) / POS;
    a.n_rest = a.B * a.Hkv * (a.group / NH);
    const long long blocks = (long long)a.n_pos_tiles * a.n_rest * (a.kv_splits > 1 ? a.kv_splits : 1);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // The plain order runs every position tile of a round next to the other
    // heads an XCD hosts, ceil(n_rest / 8) of them: when their K and V outgrow
    // about half of an XCD's 4 MB L2, each round of position tiles reads them
    // from HBM again, and the XCD-aware order keeps them resident instead.
    const long long kv_bytes_head = (long long)a.kv_len * D * 4;  // 16-bit K and V of one (b, kv head)
    a.xcd_order = !PAGED && a.kv_splits <= 1 && a.n_rest >= 8 && (a.n_rest + 7) / 8 * kv_bytes_head > (2LL << 20);
    hipLaunchKernelGGL((prefill_fwd_pp<TAG, D, CAUSAL, NH, PAGED, BIAS>), dim3((unsigned)blocks), dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.kv_splits <= 1) return e;
    const long long rows = (long long)a.B * a.Hq * a.q_len;
    const long long merge_blocks = (rows * (D / 8) + 255) / 256;
    if (merge_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_merge_kernel<TAG, D>), dim3((unsigned)merge_blocks), dim3(256), 0, stream, a, rows);
    return hipGetLastError();
}

template <class TAG, int D, bool CAUSAL, bool PAGED>
hipError_t dispatch_nh(PrefillArgs a, hipStream_t stream) {
    if (a.group % 8 == 0) return launch_pp<TAG, D, CAUSAL, 8, PAGED>(a, stream);
    if (a.group % 4 == 0) return launch_pp<TAG, D, CAUSAL, 4, PAGED>(a, stream);
    if (a.group % 2 == 0) return launch_pp<TAG, D, CAUSAL, 2, PAGED>(a, stream);
    return launch_pp<TAG, D, CAUSAL, 1, PAGED>(a, stream);
}

template <class TAG, bool PAGED>
hipError_t dispatch_d(PrefillArgs a, int D, bool causal, hipStream_t stream) {
    if (D == 64)
        return causal ? dispatch_nh<TAG, 64, true, PAGED>(a, stream) : dispatch_nh<TAG, 64, false, PAGED>(a, stream);
    return causal ? dispatch_nh<TAG, 128, true, PAGED>(a, stream) : dispatch_nh<TAG, 128, false, PAGED>(a, stream);
}

}  // namespace

long long prefill_pp_items(int B, int Hq, int Hkv, int q_len) {
    const int group = Hq / Hkv;
    const int nh = group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    const int pos = 256 / nh;
    return (long long)B * Hkv * (group / nh) * ((q_len + pos - 1) / pos);
}

hipError_t launch_prefill_split(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream) {
    return launch_prefill_pp(a, D, causal, dtype, stream);
}

hipError_t launch_prefill_pp(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream) {
    if (dtype == kDtypeBF16) return dispatch_d<bf16_tag, false>(a, D, causal, stream);
    return dispatch_d<f16_tag, false>(a, D, causal, stream);
}

template <class TAG, bool CAUSAL>
hipError_t dispatch_nh_bias(PrefillArgs a, hipStream_t stream) {
    if (a.group % 8 == 0) return launch_pp<TAG, 128, CAUSAL, 8, false, true>(a, stream);
    if (a.group % 4 == 0) return launch_pp<TAG, 128, CAUSAL, 4, false, true>(a, stream);
    if (a.group % 2 == 0) return launch_pp<TAG, 128, CAUSAL, 2, false, true>(a, stream);
    return launch_pp<TAG, 128, CAUSAL, 1, false, true>(a, stream);
}

hipError_t launch_prefill_pp_bias(PrefillArgs a, bool causal, int dtype, hipStream_t stream) {
    a.kv_splits = 1;
    if (dtype == kDtypeBF16) return causal ? dispatch_nh_bias<bf16_tag, true>(a, stream) : dispatch_nh_bias<bf16_tag, false>(a, stream);
    return causal ? dispatch_nh_bias<f16_tag, true>(a, stream) : dispatch_nh_bias<f16_tag, false>(a, stream);
}

hipError_t launch_prefill_pp_paged(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream) {
    a.kv_splits = 1;
    if (dtype == kDtypeBF16) return dispatch_d<bf16_tag, true>(a, D, causal, stream);
    return dispatch_d<f16_tag, true>(a, D, causal, stream);
}

}  // namespace gqa
