// decode_splitk.hip - split-K single-query attention over a (paged) KV cache.
//
// Method: splitk_kernels.py (xformers), `_fwd_kernel_splitK` and
// `_splitK_reduce`.  Each sequence's keys are cut into n_splits chunks; every
// chunk runs the online softmax over its keys and writes a partial output
// O_s = acc / l (0 when the chunk is empty) and its natural-base LSE
// (-inf when empty).  The combine kernel merges the chunks per (b, h):
// M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s,
// LSE = M + log(sum w_s); all chunks empty gives (0, -inf).  Keys of a paged
// cache are found through the per-sequence block table, page
// block_table[b, t / page_size], row t % page_size (the PAGE_SIZE branch of
// `_fwd_kernel_splitK`).
//
// gfx950 mapping.  Decode reads every K/V byte once and does ~4 flop per
// byte, so it is bound by HBM and runs on the vector ALUs: no MFMA padding of
// the 4-row query block.  A workgroup (4 wave64s) owns one (sequence, K/V head,
// chunk) and every query head of the group (up to 4 per workgroup).  Each wave
// takes 16 tokens of every 64-token tile; a token row is read by 4 lanes with
// 16-byte loads, so a wave's load instruction covers 16 rows x 64 contiguous
// bytes.  q.k uses packed 2-wide dot products (v_dot2_f32_bf16 / _f16) and a
// quad reduction (DPP), the softmax state is per wave, and the waves are merged
// through LDS at the end of the chunk.  The next tile's loads are issued
// before the current tile is consumed.
#include "gqa_device.hpp"
#include "gqa_kernels.hpp"

namespace gqa {

namespace {

constexpr int kTile = 64;  // tokens per workgroup iteration (16 per wave)

// Max over the 16 token lanes-quads of a wave (values are equal inside a quad).
__device__ __forceinline__ float wave_max_over_quads(float x) {
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    x = fmaxf(x, shfl_xor(x, 16));
    x = fmaxf(x, xor32(x));
    return x;
}

// Sum over the 16 lanes of a wave that share (lane & 3).
__device__ __forceinline__ float wave_sum_same_quad_slot(float x) {
    x += dpp<0x128>(x);  // row_ror:8
    x += dpp<0x124>(x);  // row_ror:4
    x += shfl_xor(x, 16);
    x += xor32(x);
    return x;
}

template <class TAG, int D, int GH, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    constexpr int DQ = D / 4;      // dims per lane
    constexpr int NCH = DQ / 8;    // 16-byte chunks per lane per row
    constexpr int NW = DQ / 2;     // packed pairs per lane per row

    __shared__ float sm_acc[4][GH][D];
    __shared__ float sm_m[4][GH];
    __shared__ float sm_l[4][GH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_hb = a.group / GH;
    int id = blockIdx.x;
    const int s = id % a.n_splits;
    id /= a.n_splits;
    const int hb = id % n_hb;
    id /= n_hb;
    const int g = id % a.Hkv;
    const int b = id / a.Hkv;
    const int h0 = g * a.group + hb * GH;

    const int len = a.seq_lens[b];
    const int per = (len + a.n_splits - 1) / a.n_splits;
    const int chunk = (per + kTile - 1) / kTile * kTile;
    const int lo = s * chunk;
    const int hi = min(len, lo + chunk);

    const size_t part_row0 = ((size_t)b * a.Hq + h0) * a.n_splits + s;  // head h0, split s
    if (lo >= hi) {  // empty chunk: (0, -inf)
        for (int i = tid; i < GH * D; i += 256) {
            const int j = i / D, d = i % D;
            a.part_o[(part_row0 + (size_t)j * a.n_splits) * D + d] = 0.f;
        }
        if (tid < GH) a.part_lse[part_row0 + (size_t)tid * a.n_splits] = -INFINITY;
        return;
    }

    const int dq = lane & 3;
    const int tok_in_tile = 16 * wave + (lane >> 2);

    // q for the GH heads, this lane's dims, as packed pairs
    uint32_t qw[GH][NW];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + h0 + j) * D + dq * DQ;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const u32x4 t = ld_global_16(qp + c * 8);
            qw[j][4 * c] = t[0]; qw[j][4 * c + 1] = t[1]; qw[j][4 * c + 2] = t[2]; qw[j][4 * c + 3] = t[3];
        }
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k);
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v);
    const int* bt = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
    const int page_mask = (1 << a.page_shift) - 1;
    auto row_offset = [&](int t) -> size_t {  // element offset of token t's row for head g
        if (PAGED) {
            const size_t page = (size_t)bt[t >> a.page_shift];
            return ((page << a.page_shift) + (size_t)(t & page_mask)) * a.Hkv * D + (size_t)g * D;
        }
        return (((size_t)b * a.Hkv + g) * a.max_kv_len + t) * D;
    };

    u32x4 kr[NCH], vr[NCH];
    auto load = [&](int t0) {
        const int t = min(t0 + tok_in_tile, hi - 1);
        const size_t off = row_offset(t) + dq * DQ;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            kr[c] = ld_global_16(kbase + off + c * 8);
            vr[c] = ld_global_16(vbase + off + c * 8);
        }
    };

    float m[GH], l[GH], acc[GH][DQ];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int d = 0; d < DQ; ++d) acc[j][d] = 0.f;
    }

    load(lo);
    for (int t0 = lo; t0 < hi; t0 += kTile) {
        u32x4 kc[NCH], vc[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) { kc[c] = kr[c]; vc[c] = vr[c]; }
        if (t0 + kTile < hi) load(t0 + kTile);

        const bool valid = t0 + tok_in_tile < hi;
        // scores of this lane's token for each head
        float sc[GH];
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            float x = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) x = dot2(TAG(), kc[c][e], qw[j][4 * c + e], x);
            x += dpp<kQuadXor1>(x);
            x += dpp<kQuadXor2>(x);
            sc[j] = valid ? x : -INFINITY;
        }
        float vf[DQ];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[8 * c + 2 * e] = lo_to_f32(TAG(), vc[c][e]);
                vf[8 * c + 2 * e + 1] = hi_to_f32(TAG(), vc[c][e]);
            }
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            const float mx = wave_max_over_quads(sc[j]);
            const float m_new = fmaxf(m[j], mx * a.c);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m[j] - m_use);
            m[j] = m_new;
            const float p = fast_exp2(fmaf(sc[j], a.c, -m_use));
            l[j] = l[j] * alpha + p;
#pragma unroll
            for (int d = 0; d < DQ; ++d) acc[j][d] = fmaf(p, vf[d], acc[j][d] * alpha);
        }
    }

    // ---- merge the 16 token slots of each wave, then the 4 waves -------------
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        // every lane of a quad holds the same l (same token); count one per quad
        const float lq = (dq == 0) ? l[j] : 0.f;
        float lw = lq;
        lw += dpp<0x128>(lw);
        lw += dpp<0x124>(lw);
        lw += dpp<kQuadXor1>(lw);
        lw += dpp<kQuadXor2>(lw);
        lw += shfl_xor(lw, 16);
        lw += xor32(lw);
#pragma unroll
        for (int d = 0; d < DQ; ++d) acc[j][d] = wave_sum_same_quad_slot(acc[j][d]);
        if (lane < 4) {
#pragma unroll
            for (int d = 0; d < DQ; ++d) sm_acc[wave][j][dq * DQ + d] = acc[j][d];
        }
        if (lane == 0) {
            sm_m[wave][j] = m[j];
            sm_l[wave][j] = lw;
        }
    }
    __syncthreads();
    for (int i = tid; i < GH * D; i += 256) {
        const int j = i / D, d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][j]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sc = fast_exp2(sm_m[w][j] - M);
                L += sc * sm_l[w][j];
                O += sc * sm_acc[w][j][d];
            }
        }
        const size_t row = part_row0 + (size_t)j * a.n_splits;
        a.part_o[row * D + d] = L > 0.f ? O / L : 0.f;
        if (d == 0) a.part_lse[row] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
}

// One wave per (b, h): merge the n_splits partial results.
template <class TAG, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + h
    if (row >= a.B * a.Hq) return;
    const float* pl = a.part_lse + (size_t)row * a.n_splits;
    const float* po = a.part_o + (size_t)row * a.n_splits * D;

    float M = -INFINITY;
    for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, pl[s]);
    float W = 0.f, O[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < a.n_splits; ++s) {
            const float w = fast_exp2((pl[s] - M) * kLog2e);
            W += w;
#pragma unroll
            for (int i = 0; i < PER; ++i) O[i] = fmaf(w, po[(size_t)s * D + lane * PER + i], O[i]);
        }
    }
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

template <class TAG, int D, int GH, bool PAGED>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
    const long long blocks = (long long)a.B * a.Hkv * (a.group / GH) * a.n_splits;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_split_kernel<TAG, D, GH, PAGED>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<TAG, D>), dim3((unsigned)((a.B * a.Hq + 3) / 4)), dim3(256),
                       0, stream, a);
    return hipGetLastError();
}

template <class TAG, int D, bool PAGED>
hipError_t dispatch_group(const DecodeArgs& a, hipStream_t stream) {
    if (a.group % 4 == 0) return launch_split<TAG, D, 4, PAGED>(a, stream);
    if (a.group % 2 == 0) return launch_split<TAG, D, 2, PAGED>(a, stream);
    return launch_split<TAG, D, 1, PAGED>(a, stream);
}

template <class TAG>
hipError_t dispatch_d(const DecodeArgs& a, hipStream_t stream) {
    const bool paged = a.block_table != nullptr;
    if (a.D == 64) return paged ? dispatch_group<TAG, 64, true>(a, stream) : dispatch_group<TAG, 64, false>(a, stream);
    return paged ? dispatch_group<TAG, 128, true>(a, stream) : dispatch_group<TAG, 128, false>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    if (dtype == kDtypeBF16) return dispatch_d<bf16_tag>(a, stream);
    return dispatch_d<f16_tag>(a, stream);
}

}  // namespace gqa
