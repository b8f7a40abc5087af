// prefill_fwd.hip - attention forward (prefill) on gfx950 matrix cores.
//
// Method: FlashAttention forward with an online softmax, as in
// causal_forward_kernel.py (`_flash_attention_forward_gqa_kernel`): for each
// block of queries, stream K/V tiles, compute S = scale * Q K^T, keep a running
// row max m and row sum l, rescale the fp32 accumulator by exp2(m_old - m_new),
// add P V, and finish with O = acc / l and the row log-sum-exp.  Scale is folded
// with log2(e) so every exponential is a single v_exp_f32 (2^x).  Masking is the
// bottom-right causal rule of the FlashInfer-style prefill page
// (gpt-o3 / triton6fd1ef, `_gqa_prefill_kernel`: query i sees keys
// j <= i + kv_len - q_len); tiles right of the diagonal are never visited and
// only tiles that cross it (or the end of the keys) pay for the mask, the
// two-phase split of causal_forward_kernel.py.  Empty rows give O = 0 and
// LSE = -inf (the zero-fill rule of splitk_kernels.py, `_fwd_kernel_splitK`).
//
// gfx950 mapping (bf16/fp16):
//   * a workgroup is 4 wave64s; each wave owns 32 query rows of one head, and
//     the workgroup's waves cover NH heads of one K/V group (GQA: the K/V tile
//     staged in LDS once serves every head of the group in the workgroup);
//   * the score tile is computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16 (keys on M, queries on N), so each lane holds one
//     query's scores and the row max / row sum are in-lane plus one
//     lane^32 exchange (v_permlane32_swap);
//   * the P^T accumulator layout feeds the P.V product directly as the MFMA B
//     operand; V is stored transposed in LDS with the key order permuted so
//     that the A operand of each 16-key step is one 16-byte LDS read;
//   * K/V tiles are double buffered in LDS: the global loads of tile t+1 are in
//     flight while tile t is multiplied, one barrier per tile.
//
// PAGED: a batch of ragged requests over a paged K/V cache, the FlashInfer-style
// prefill page's `run` (gpt-o3 / triton6fd1ef): request b owns the query tokens
// [qo_indptr[b], qo_indptr[b+1]) of a token-major q [total_q, Hq, D] and the
// pages kv_indices[kv_indptr[b] ..) of a pool [num_pages, page_size, Hkv, D];
// its key t is row t % page_size of page kv_indices[kv_indptr[b] + t / page_size]
// and the bottom-right offset is per request.  The page ids of a tile's rows are
// loaded one tile ahead of its K/V loads, so the lookup adds no latency.
#include "gqa_device.hpp"
#include "gqa_kernels.hpp"

namespace gqa {

namespace {

// Growth of a row max (log2 units) that triggers a rescale of acc and l.
constexpr float kRescaleLog2 = 8.f;

// A stored 16-bit value of the input dtype as fp32.
__device__ __forceinline__ float to_f32(bf16_tag, uint32_t u16) { return __builtin_bit_cast(float, u16 << 16); }
__device__ __forceinline__ float to_f32(f16_tag, uint32_t u16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
}

// BIAS: 0 = none; otherwise the additive bias of splitk_kernels.py
// (`_fwd_kernel_splitK`, HAS_ADDITIVE_BIAS) is loaded for every score tile and
// added before the softmax.  BIAS = 4: rows 8-byte aligned, four keys per load
// (whole tiles; the tail tile reads key by key); BIAS = 1: key by key.
template <class TAG, int D, bool CAUSAL, int NH, bool PAGED, int BIAS = 0>
__global__ __launch_bounds__(256, 2) void prefill_fwd_mfma(PrefillArgs a) {
    constexpr int BN = 64;                 // keys per tile
    constexpr int WPH = 4 / NH;            // waves per head
    constexpr int POS = 32 * WPH;          // query positions per workgroup
    constexpr int KS = D + 8;              // K tile row stride (elements)
    constexpr int VS = BN + 8;             // V^T tile row stride (elements)
    constexpr int KT = BN * KS;            // elements of one K tile
    constexpr int VT = D * VS;             // elements of one V^T tile
    constexpr int DS = D / 16;             // MFMA k-steps over the head dim
    constexpr int DT = D / 32;             // 32-wide output tiles over the head dim
    constexpr int KCH = BN * D / 8 / 256;  // 16-byte K chunks per thread per tile
    constexpr int VTHREADS = 16 * (D / 8); // threads that stage V (4 keys x 8 dims each)
    typedef typename TAG::vec8 vec8;

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT + VT)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // ---- work item: (position tile, batch, K/V head, head group) ----------
    const int hgroups = a.group / NH;
    int pt, hg, g, b;
    bool from_end = false;  // PAGED: position tile counted from the request's last query
    if (PAGED && a.B <= 512) {
        // Ragged batch: only real items, longest first across the whole batch
        // (ragged_item), heads fastest; the grid's surplus workgroups come last
        // (as in prefill_pp.hip).
        const int n_hk = a.Hkv * hgroups;
        int item = blockIdx.x / n_hk;
        const int hk = blockIdx.x - item * n_hk;
        hg = hk % hgroups;
        g = hk / hgroups;
        b = ragged_item<POS>(a.qo_indptr, a.kv_indptr, a.kv_last_page_len, a.page_shift, a.B, a.n_pos_tiles,
                             item, pt);
        if (b < 0) return;  // workgroup-uniform, before any barrier: no item left
        from_end = true;
    } else {
        pt = blockIdx.x / a.n_rest;
        int rest = blockIdx.x - pt * a.n_rest;
        if (CAUSAL) pt = a.n_pos_tiles - 1 - pt;  // longest rows first
        hg = rest % hgroups;
        rest /= hgroups;
        g = rest % a.Hkv;
        b = rest / a.Hkv;
    }
    const int h = g * a.group + hg * NH + wave / WPH;

    // ---- the request: query rows, keys, causal offset ------------------------
    int q_len = a.q_len, kv_len = a.kv_len, delta = a.delta;
    size_t q_tok0 = 0;   // PAGED: first query token of the request
    int kv_page0 = 0;    // PAGED: first entry of its page list
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
    if (PAGED && wg_pos0 >= q_len) return;  // workgroup-uniform: past this request's queries
    const int pos0 = wg_pos0 + (wave % WPH) * 32;
    const int my_q = pos0 + l32;
    // element offset of query row `row` of head h (q and o), and its LSE index
    auto q_off = [&](int row) -> size_t {
        if constexpr (PAGED) return ((q_tok0 + row) * a.Hq + h) * (size_t)D;
        return (((size_t)b * a.Hq + h) * (size_t)q_len + row) * D;
    };
    auto lse_off = [&](int row) -> size_t {
        if constexpr (PAGED) return (q_tok0 + row) * a.Hq + h;
        return ((size_t)b * a.Hq + h) * (size_t)q_len + row;
    };

    // ---- key ranges -------------------------------------------------------
    // wg_kv_end: keys any row of the workgroup sees; wave_kv_end: keys any row
    // of this wave sees; wave_full_end: keys every row of this wave sees.
    int wg_kv_end = kv_len, wave_kv_end = kv_len, wave_full_end = kv_len;
    if (CAUSAL) {
        const int wg_last = min(wg_pos0 + POS, q_len) - 1;
        wg_kv_end = max(0, min(kv_len, wg_last + delta + 1));
        const int w_last = min(pos0 + 32, q_len) - 1;
        wave_kv_end = pos0 < q_len && pos0 + 32 > 0 ? max(0, min(kv_len, w_last + delta + 1)) : 0;
        wave_full_end = max(0, min(kv_len, pos0 + delta + 1));
    } else if (pos0 >= q_len || pos0 + 32 <= 0) {
        wave_kv_end = 0;
    }
    const int n_tiles = (wg_kv_end + BN - 1) / BN;

    // ---- Q: B operand of S^T = K Q^T, resident in registers ---------------
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const int q_row = min(max(my_q, 0), q_len - 1);
    vec8 qf[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
        qf[ds] = __builtin_bit_cast(vec8, ld_global_16(qp + q_off(q_row) + ds * 16 + half * 8));
    // Q must be resident before the loop: otherwise the wait-count pass makes
    // every use of Q inside the loop wait for the next tile's prefetch loads.
    wait_vmcnt0();

    // dense: the (b, g) plane; PAGED: head g inside the pool's token rows
    const size_t kv_head = PAGED ? (size_t)g : ((size_t)b * a.Hkv + g) * (size_t)kv_len;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + kv_head * D;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + kv_head * D;
    const int last_key = kv_len - 1;

    // ---- tile staging ------------------------------------------------------
    u32x4 kreg[KCH];
    u32x4 vreg[4];
    const int v_kg = tid & 15;  // V: keys 4*v_kg .. +3 of the tile
    const int v_dg = tid >> 4;  // V: dims 8*v_dg .. +7
    // Position of key 4*c+e (c = v_kg & 3) inside its 16-key block of V^T:
    // key 8*a + 4*h + e is stored at 8*h + 4*a + e, so that the 8 keys one
    // lane half feeds to a 16-key MFMA step are contiguous.
    const int v_pos = (v_kg >> 2) * 16 + 8 * (v_kg & 1) + 4 * ((v_kg >> 1) & 1);

    // Element offset of key `key` (clamped to the last key) in its K/V plane;
    // PAGED: the key's pool row from the page id fetched for it beforehand.
    const int page_mask = PAGED ? (1 << a.page_shift) - 1 : 0;
    const size_t tok_stride = PAGED ? (size_t)a.Hkv * D : (size_t)D;
    auto key_row = [&](int key, int page) -> size_t {
        if constexpr (PAGED) return (((size_t)page << a.page_shift) + (size_t)(key & page_mask)) * tok_stride;
        return (size_t)key * D;
    };
    int pg_k[KCH], pg_v[4];  // PAGED: page ids of the rows of the next tile to load
    auto fetch_pages = [&](int t0) {
        if constexpr (PAGED) {
            const int* ix = a.kv_indices + kv_page0;
#pragma unroll
            for (int j = 0; j < KCH; ++j) {
                const int row = (tid + 256 * j) / (D / 8);
                pg_k[j] = ix[min(t0 + row, last_key) >> a.page_shift];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pg_v[r] = tid < VTHREADS ? ix[min(t0 + 4 * v_kg + r, last_key) >> a.page_shift] : 0;
        }
    };
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            const int c = tid + 256 * j;
            const int row = c / (D / 8), col = c % (D / 8);
            const int key = min(t0 + row, last_key);
            kreg[j] = ld_global_16(kp + key_row(key, pg_k[j]) + col * 8);
        }
        if (tid < VTHREADS) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = min(t0 + 4 * v_kg + r, last_key);
                vreg[r] = ld_global_16(vp + key_row(key, pg_v[r]) + v_dg * 8);
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* ks = smem + buf * (KT + VT);
        uint16_t* vs = ks + KT;
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            const int c = tid + 256 * j;
            const int row = c / (D / 8), col = c % (D / 8);
            *reinterpret_cast<u32x4*>(ks + row * KS + col * 8) = kreg[j];
        }
        if (tid < VTHREADS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // dword e holds dims 8*v_dg + 2e, +1
                u32x2 w0 = {pack_lo(vreg[0][e], vreg[1][e]), pack_lo(vreg[2][e], vreg[3][e])};
                u32x2 w1 = {pack_hi(vreg[0][e], vreg[1][e]), pack_hi(vreg[2][e], vreg[3][e])};
                *reinterpret_cast<u32x2*>(vs + (v_dg * 8 + 2 * e) * VS + v_pos) = w0;
                *reinterpret_cast<u32x2*>(vs + (v_dg * 8 + 2 * e + 1) * VS + v_pos) = w1;
            }
        }
    };

    // ---- online softmax state (log2 domain: m is a max of s * c) ------------
    float m = -INFINITY;
    float l = 0.f;  // this lane's share of the row sum (its half of the keys)
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    if (n_tiles > 0) {
        fetch_pages(0);
        load_tile(0);
        if (n_tiles > 1) fetch_pages(BN);
        store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int t0 = it * BN;
        const int buf = it & 1;
        if (it + 1 < n_tiles) load_tile(t0 + BN);
        if (it + 2 < n_tiles) fetch_pages(t0 + 2 * BN);

        if (t0 < wave_kv_end) {  // wave-uniform: skip tiles this wave cannot see
            const uint16_t* ks = smem + buf * (KT + VT);
            const uint16_t* vs = ks + KT;

            // additive bias of this lane's scores (row q_row, keys as in s below);
            // keys past the last one read the last one (they are masked)
            [[maybe_unused]] float bv[2][16];
            if constexpr (BIAS != 0) {
                const uint16_t* brow = a.bias + (long long)b * a.bias_sb + (long long)h * a.bias_sh +
                                       (long long)q_row * a.bias_sq;
                if (BIAS == 4 && t0 + BN <= kv_len) {
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const u32x2 w = *reinterpret_cast<const u32x2*>(brow + t0 + kh * 32 + 8 * j + 4 * half);
                            bv[kh][4 * j] = to_f32(TAG(), w[0] & 0xffffu);
                            bv[kh][4 * j + 1] = to_f32(TAG(), w[0] >> 16);
                            bv[kh][4 * j + 2] = to_f32(TAG(), w[1] & 0xffffu);
                            bv[kh][4 * j + 3] = to_f32(TAG(), w[1] >> 16);
                        }
                } else {
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = min(t0 + kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3), last_key);
                            bv[kh][r] = to_f32(TAG(), brow[key]);
                        }
                }
            }

            // S^T[key][query] for 64 keys (two 32-key halves)
            f32x16 s[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kh][r] = 0.f;
            // the two 32-key halves are independent accumulation chains: interleave them
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    vec8 ka = *reinterpret_cast<const vec8*>(ks + (kh * 32 + l32) * KS + ds * 16 + half * 8);
                    s[kh] = mfma_32x32x16(ka, qf[ds], s[kh]);
                }
            }

            if constexpr (BIAS != 0) {
                // s * c = scale * log2(e) * q.k + log2(e) * bias with bias_k = 1 / scale
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kh][r] = fmaf(bv[kh][r], a.bias_k, s[kh][r]);
            }

            if (t0 + BN > wave_full_end) {  // diagonal or tail tile: apply the mask
                const int lim = CAUSAL ? min(my_q + delta + 1, kv_len) : kv_len;
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = t0 + kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                        if (key >= lim) s[kh][r] = -INFINITY;
                    }
            }

            float mx = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
            mx = fmaxf(mx, xor32(mx));
            // Lazy rescale: the reference max m only moves when some row's max
            // grew by more than kRescaleLog2 (log2 units).  acc and l always use
            // the same m, so O = acc / l and LSE = m + log2 l are unchanged;
            // weights stay below 2^kRescaleLog2.
            const float m_tile = mx * a.c;
            if (__builtin_amdgcn_ballot_w64(m_tile > m + kRescaleLog2)) {
                const float m_new = fmaxf(m, m_tile);
                // 0 when m = -inf; a row that has still seen no key keeps alpha = 1
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            }
            const float m_use = (m == -INFINITY) ? 0.f : m;

            uint32_t pk[2][8];
            float psum = 0.f;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(fmaf(s[kh][r], a.c, -m_use));
                    const float p1 = fast_exp2(fmaf(s[kh][r + 1], a.c, -m_use));
                    psum += p0 + p1;
                    pk[kh][r >> 1] = pack2(TAG(), p0, p1);
                }
            l += psum;

            // O^T[d][query] += V^T[d][key] P^T[key][query], 16 keys per step
#pragma unroll
            for (int k16 = 0; k16 < 4; ++k16) {
                const int kh = k16 >> 1, base = (k16 & 1) * 4;
                const u32x4 pw = {pk[kh][base], pk[kh][base + 1], pk[kh][base + 2], pk[kh][base + 3]};
                const vec8 pb = __builtin_bit_cast(vec8, pw);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    vec8 va = *reinterpret_cast<const vec8*>(vs + (dt * 32 + l32) * VS + k16 * 16 + half * 8);
                    acc[dt] = mfma_32x32x16(va, pb, acc[dt]);
                }
            }
        }

        if (it + 1 < n_tiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2 -------------------
    const float l_tot = l + xor32(l);
    const bool valid = my_q >= 0 && my_q < q_len;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    store_acc_row(TAG(), acc, inv, static_cast<uint16_t*>(a.o) + q_off(min(max(my_q, 0), q_len - 1)), half, valid);
    if (valid && half == 0) a.lse[lse_off(my_q)] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

// fp32 inputs: the same schedule on v_mfma_f32_32x32x2f32 with fp32 softmax
// weights (no rounding of P), one head per workgroup, 32-key tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_fwd_f32(PrefillArgs a) {
    constexpr int BN = 32;
    constexpr int POS = 128;
    constexpr int KS = D + 4;
    constexpr int VS = D + 4;
    constexpr int KT = BN * KS;
    constexpr int VT = BN * VS;
    constexpr int HD = D / 2;          // dims per lane half
    constexpr int DT = D / 32;
    constexpr int CH = BN * D / 4 / 256;  // 16-byte chunks per thread per tile (each of K, V)

    __shared__ __attribute__((aligned(16))) float smem[2 * (KT + VT)];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    int pt = blockIdx.x / a.n_rest;
    int rest = blockIdx.x - pt * a.n_rest;
    if (CAUSAL) pt = a.n_pos_tiles - 1 - pt;
    const int h = rest % a.Hq;
    const int b = rest / a.Hq;
    const int g = h / a.group;
    const int wg_pos0 = pt * POS;
    const int pos0 = wg_pos0 + wave * 32;
    const int my_q = pos0 + l32;

    int wg_kv_end = a.kv_len, wave_kv_end = a.kv_len, wave_full_end = a.kv_len;
    if (CAUSAL) {
        const int wg_last = min(wg_pos0 + POS, a.q_len) - 1;
        wg_kv_end = max(0, min(a.kv_len, wg_last + a.delta + 1));
        const int w_last = min(pos0 + 32, a.q_len) - 1;
        wave_kv_end = pos0 < a.q_len ? max(0, min(a.kv_len, w_last + a.delta + 1)) : 0;
        wave_full_end = max(0, min(a.kv_len, pos0 + a.delta + 1));
    } else if (pos0 >= a.q_len) {
        wave_kv_end = 0;
    }
    const int n_tiles = (wg_kv_end + BN - 1) / BN;

    // Lane half `half` covers dims [half*HD, half*HD + HD); MFMA step j uses dim half*HD + j.
    const size_t q_head = ((size_t)b * a.Hq + h) * (size_t)a.q_len;
    const float* qp = static_cast<const float*>(a.q) + q_head * D;
    const int q_row = min(my_q, a.q_len - 1);
    float qf[HD];
#pragma unroll
    for (int j = 0; j < HD; j += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(qp + (size_t)q_row * D + half * HD + j);
        qf[j] = t[0]; qf[j + 1] = t[1]; qf[j + 2] = t[2]; qf[j + 3] = t[3];
    }
    wait_vmcnt0();

    const size_t kv_head = ((size_t)b * a.Hkv + g) * (size_t)a.kv_len;
    const float* kp = static_cast<const float*>(a.k) + kv_head * D;
    const float* vp = static_cast<const float*>(a.v) + kv_head * D;
    const int last_key = a.kv_len - 1;

    f32x4 kreg[CH], vreg[CH];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = tid + 256 * j;
            const int row = c / (D / 4), col = c % (D / 4);
            const int key = min(t0 + row, last_key);
            kreg[j] = *reinterpret_cast<const f32x4*>(kp + (size_t)key * D + col * 4);
            vreg[j] = *reinterpret_cast<const f32x4*>(vp + (size_t)key * D + col * 4);
        }
    };
    auto store_tile = [&](int buf) {
        float* ks = smem + buf * (KT + VT);
        float* vs = ks + KT;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = tid + 256 * j;
            const int row = c / (D / 4), col = c % (D / 4);
            *reinterpret_cast<f32x4*>(ks + row * KS + col * 4) = kreg[j];
            *reinterpret_cast<f32x4*>(vs + row * VS + col * 4) = vreg[j];
        }
    };

    float m = -INFINITY, l = 0.f;
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int t0 = it * BN;
        const int buf = it & 1;
        if (it + 1 < n_tiles) load_tile(t0 + BN);
        if (t0 < wave_kv_end) {
            const float* ks = smem + buf * (KT + VT);
            const float* vs = ks + KT;
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
            const float* krow = ks + l32 * KS + half * HD;
#pragma unroll
            for (int j = 0; j < HD; j += 4) {
                const f32x4 kv4 = *reinterpret_cast<const f32x4*>(krow + j);
                s = mfma_32x32x2(kv4[0], qf[j], s);
                s = mfma_32x32x2(kv4[1], qf[j + 1], s);
                s = mfma_32x32x2(kv4[2], qf[j + 2], s);
                s = mfma_32x32x2(kv4[3], qf[j + 3], s);
            }
            if (t0 + BN > wave_full_end) {
                const int lim = CAUSAL ? min(my_q + a.delta + 1, a.kv_len) : a.kv_len;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= lim) s[r] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = fmaxf(mx, xor32(mx));
            const float m_tile = mx * a.c;
            if (__builtin_amdgcn_ballot_w64(m_tile > m + kRescaleLog2)) {
                const float m_new = fmaxf(m, m_tile);
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            }
            const float m_use = (m == -INFINITY) ? 0.f : m;
            float p[16];
            float psum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = fast_exp2(fmaf(s[r], a.c, -m_use));
                psum += p[r];
            }
            l += psum;
            // step r pairs key 8*(r/4) + 4*half + r%4 of lane half `half`
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    acc[dt] = mfma_32x32x2(vs[key * VS + dt * 32 + l32], p[r], acc[dt]);
            }
        }
        if (it + 1 < n_tiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l + xor32(l);
    if (my_q < a.q_len) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* op = static_cast<float*>(a.o) + (q_head + my_q) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = dt * 32 + 8 * r4 + 4 * half;
                const f32x4 w = {acc[dt][4 * r4] * inv, acc[dt][4 * r4 + 1] * inv,
                                 acc[dt][4 * r4 + 2] * inv, acc[dt][4 * r4 + 3] * inv};
                *reinterpret_cast<f32x4*>(op + d0) = w;
            }
        if (half == 0)
            a.lse[q_head + my_q] = l_tot > 0.f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
}

template <class TAG, int D, bool CAUSAL, int NH, bool PAGED, int BIAS = 0>
hipError_t launch_mfma(PrefillArgs a, hipStream_t stream) {
    constexpr int POS = 32 * (4 / NH);
    a.n_pos_tiles = (a.q_len + POS - 1) / POS;
    a.n_rest = a.B * a.Hkv * (a.group / NH);
    const long long blocks = (long long)a.n_pos_tiles * a.n_rest;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_fwd_mfma<TAG, D, CAUSAL, NH, PAGED, BIAS>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

template <class TAG, int D, bool CAUSAL, bool PAGED = false, int BIAS = 0>
hipError_t dispatch_nh(PrefillArgs a, hipStream_t stream) {
    if (a.group % 4 == 0) return launch_mfma<TAG, D, CAUSAL, 4, PAGED, BIAS>(a, stream);
    if (a.group % 2 == 0) return launch_mfma<TAG, D, CAUSAL, 2, PAGED, BIAS>(a, stream);
    return launch_mfma<TAG, D, CAUSAL, 1, PAGED, BIAS>(a, stream);
}

template <class TAG, int BIAS>
hipError_t dispatch_d_bias(PrefillArgs a, int D, bool causal, hipStream_t stream) {
    if (D == 64)
        return causal ? dispatch_nh<TAG, 64, true, false, BIAS>(a, stream)
                      : dispatch_nh<TAG, 64, false, false, BIAS>(a, stream);
    return causal ? dispatch_nh<TAG, 128, true, false, BIAS>(a, stream)
                  : dispatch_nh<TAG, 128, false, false, BIAS>(a, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_f32(PrefillArgs a, hipStream_t stream) {
    a.n_pos_tiles = (a.q_len + 127) / 128;
    a.n_rest = a.B * a.Hq;
    const long long blocks = (long long)a.n_pos_tiles * a.n_rest;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_fwd_f32<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <class TAG>
hipError_t dispatch_d(PrefillArgs a, int D, bool causal, hipStream_t stream) {
    if (D == 64) return causal ? dispatch_nh<TAG, 64, true>(a, stream) : dispatch_nh<TAG, 64, false>(a, stream);
    return causal ? dispatch_nh<TAG, 128, true>(a, stream) : dispatch_nh<TAG, 128, false>(a, stream);
}

template <class TAG>
hipError_t dispatch_d_paged(PrefillArgs a, int D, bool causal, hipStream_t stream) {
    if (D == 64)
        return causal ? dispatch_nh<TAG, 64, true, true>(a, stream) : dispatch_nh<TAG, 64, false, true>(a, stream);
    return causal ? dispatch_nh<TAG, 128, true, true>(a, stream) : dispatch_nh<TAG, 128, false, true>(a, stream);
}

}  // namespace

hipError_t launch_prefill_paged(PrefillArgs a, int D, bool causal, int dtype, PrefillKernel kernel,
                                hipStream_t stream) {
    if (kernel == PrefillKernel::kAuto) {
        // the grid is sized by the longest request: B * Hq * max_q_len (query,
        // head) slots, 256 per ping-pong workgroup
        int dev = 0, n_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        // (D = 128 only: at D = 64 the paged ping-pong instantiations lose the
        // MFMA phase's operand read-ahead to the compiler's scheduling)
        const long long rows = (long long)a.B * a.Hq * a.q_len;
        kernel = D == 128 && rows >= 256LL * n_cu ? PrefillKernel::kPingPong : PrefillKernel::kFourWave;
    }
    if (kernel == PrefillKernel::kPingPong) return launch_prefill_pp_paged(a, D, causal, dtype, stream);
    if (dtype == kDtypeBF16) return dispatch_d_paged<bf16_tag>(a, D, causal, stream);
    return dispatch_d_paged<f16_tag>(a, D, causal, stream);
}

hipError_t launch_prefill(PrefillArgs a, int D, bool causal, int dtype, PrefillKernel kernel, hipStream_t stream) {
    if (dtype != kDtypeF32 && kernel == PrefillKernel::kAuto) {
        // the ping-pong kernel owns 256 (query, head) rows per workgroup and runs
        // one workgroup per CU; below one workgroup per CU the four-wave kernel
        // (128 rows, two workgroups per CU) keeps more of the chip busy
        int dev = 0, n_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        const long long rows = (long long)a.B * a.Hq * a.q_len;
        kernel = rows >= 256LL * n_cu ? PrefillKernel::kPingPong : PrefillKernel::kFourWave;
    }
    if (dtype != kDtypeF32 && kernel == PrefillKernel::kPingPong) return launch_prefill_pp(a, D, causal, dtype, stream);
    switch (dtype) {
    case kDtypeBF16: return dispatch_d<bf16_tag>(a, D, causal, stream);
    case kDtypeF16: return dispatch_d<f16_tag>(a, D, causal, stream);
    default:
        if (D == 64) return causal ? launch_f32<64, true>(a, stream) : launch_f32<64, false>(a, stream);
        return causal ? launch_f32<128, true>(a, stream) : launch_f32<128, false>(a, stream);
    }
}

hipError_t launch_prefill_bias(PrefillArgs a, int D, bool causal, int dtype, hipStream_t stream) {
    // the ping-pong kernel takes whole 64-key tiles of 16-byte aligned bias rows
    if (D == 128 && a.kv_len % 64 == 0 && (reinterpret_cast<uintptr_t>(a.bias) & 15) == 0 && a.bias_sb % 8 == 0 &&
        a.bias_sh % 8 == 0 && a.bias_sq % 8 == 0)
        return launch_prefill_pp_bias(a, causal, dtype, stream);
    // four keys per load when every bias row starts 8-byte aligned
    const bool vec = (reinterpret_cast<uintptr_t>(a.bias) & 7) == 0 && a.bias_sb % 4 == 0 && a.bias_sh % 4 == 0 &&
                     a.bias_sq % 4 == 0;
    if (dtype == kDtypeBF16)
        return vec ? dispatch_d_bias<bf16_tag, 4>(a, D, causal, stream) : dispatch_d_bias<bf16_tag, 1>(a, D, causal, stream);
    return vec ? dispatch_d_bias<f16_tag, 4>(a, D, causal, stream) : dispatch_d_bias<f16_tag, 1>(a, D, causal, stream);
}

}  // namespace gqa
