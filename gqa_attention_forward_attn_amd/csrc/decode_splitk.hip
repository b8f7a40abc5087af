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

// Growth of a running max (log2 units) that triggers a rescale of acc and l;
// acc and l always share the reference max, so the result is unchanged.
constexpr float kRescaleLog2 = 8.f;

template <class TAG, int D, int GH, bool PAGED>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
    constexpr int DL = D / 16;        // dims per lane (16 lanes cover a token row)
    constexpr int NWD = DL / 2;       // packed pairs per lane per row
    constexpr int TPL = 4;            // tokens per lane per tile (stream r: t0 + 16w + r + 4j)
    typedef uint32_t row_t __attribute__((ext_vector_type(NWD)));

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

    const int c = lane & 15;   // dims [c*DL, c*DL + DL)
    const int r = lane >> 4;   // token stream inside the wave

    // q of the GH heads for this lane's dims, as packed pairs
    row_t qw[GH];
#pragma unroll
    for (int j = 0; j < GH; ++j)
        qw[j] = *reinterpret_cast<const row_t*>(static_cast<const uint16_t*>(a.q) +
                                                ((size_t)b * a.Hq + h0 + j) * D + c * DL);

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k);
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v);
    const int* bt = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
    const int page_mask = (1 << a.page_shift) - 1;
    const size_t head_off = PAGED ? (size_t)g * D : ((size_t)b * a.Hkv + g) * (size_t)a.max_kv_len * D;
    const size_t tok_stride = PAGED ? (size_t)a.Hkv * D : (size_t)D;

    auto tok_of = [&](int t0, int j) { return min(t0 + 16 * wave + r + 4 * j, hi - 1); };
    // page ids of this lane's tokens in the tile at t0 (paged only)
    auto fetch_pages = [&](int t0, int (&pg)[TPL]) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) pg[j] = PAGED ? bt[tok_of(t0, j) >> a.page_shift] : 0;
    };
    auto row_index = [&](int t, int page) -> size_t {
        if (PAGED) return (((size_t)page << a.page_shift) + (size_t)(t & page_mask)) * tok_stride + head_off;
        return (size_t)t * tok_stride + head_off;
    };
    auto load = [&](int t0, const int (&pg)[TPL], row_t (&kr)[TPL], row_t (&vr)[TPL]) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const size_t off = row_index(tok_of(t0, j), pg[j]) + c * DL;
            kr[j] = *reinterpret_cast<const row_t*>(kbase + off);
            vr[j] = *reinterpret_cast<const row_t*>(vbase + off);
        }
    };

    float m[GH], l[GH], acc[GH][DL];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int d = 0; d < DL; ++d) acc[h][d] = 0.f;
    }

    // pipeline: page ids run one tile ahead of the K/V loads, which run one
    // tile ahead of the arithmetic
    int pg_next[TPL], pg_far[TPL];
    row_t kc[TPL], vc[TPL], kn[TPL], vn[TPL];
    fetch_pages(lo, pg_next);
    load(lo, pg_next, kn, vn);
    if (lo + kTile < hi) fetch_pages(lo + kTile, pg_far);

    for (int t0 = lo; t0 < hi; t0 += kTile) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) { kc[j] = kn[j]; vc[j] = vn[j]; pg_next[j] = pg_far[j]; }
        if (t0 + kTile < hi) load(t0 + kTile, pg_next, kn, vn);
        if (t0 + 2 * kTile < hi) fetch_pages(t0 + 2 * kTile, pg_far);

        // scores: this lane's 4 tokens x GH heads (reduced over the 16 lanes of the row)
        float sc[TPL][GH];
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const bool valid = t0 + 16 * wave + r + 4 * j < hi;
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                float x = 0.f;
#pragma unroll
                for (int e = 0; e < NWD; ++e) x = dot2(TAG(), kc[j][e], qw[h][e], x);
                x += dpp<kQuadXor1>(x);
                x += dpp<kQuadXor2>(x);
                x += dpp<kRowHalfMirror>(x);
                x += dpp<kRowMirror>(x);
                sc[j][h] = valid ? x : -INFINITY;
            }
        }
        // wave-uniform running max per head; lazy rescale (see prefill)
        float mt[GH];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            float x = fmaxf(fmaxf(sc[0][h], sc[1][h]), fmaxf(sc[2][h], sc[3][h]));
            x = fmaxf(x, shfl_xor(x, 16));
            x = fmaxf(x, xor32(x));
            mt[h] = x * a.c;
            grow |= mt[h] > m[h] + kRescaleLog2;
        }
        if (grow) {  // wave-uniform: mt and m are equal in every lane
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                const float m_new = fmaxf(m[h], mt[h]);
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m[h] - m_new);
                m[h] = m_new;
                l[h] *= alpha;
#pragma unroll
                for (int d = 0; d < DL; ++d) acc[h][d] *= alpha;
            }
        }
        // P.V on token pairs (j, j+1): dot2 of (p_j, p_j+1) with (v_j, v_j+1)
#pragma unroll
        for (int jp = 0; jp < TPL; jp += 2) {
            uint32_t pp[GH];
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                const float mu = (m[h] == -INFINITY) ? 0.f : m[h];
                const float p0 = fast_exp2(fmaf(sc[jp][h], a.c, -mu));
                const float p1 = fast_exp2(fmaf(sc[jp + 1][h], a.c, -mu));
                l[h] += p0 + p1;
                pp[h] = pack2(TAG(), p0, p1);
            }
#pragma unroll
            for (int e = 0; e < NWD; ++e) {
                const uint32_t vlo = pack_lo(vc[jp][e], vc[jp + 1][e]);
                const uint32_t vhi = pack_hi(vc[jp][e], vc[jp + 1][e]);
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    acc[h][2 * e] = dot2(TAG(), pp[h], vlo, acc[h][2 * e]);
                    acc[h][2 * e + 1] = dot2(TAG(), pp[h], vhi, acc[h][2 * e + 1]);
                }
            }
        }
    }

    // ---- merge the 4 token streams of each wave (same m), then the 4 waves ----
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        float lw = l[h];  // identical in the 16 lanes of a stream
        lw += shfl_xor(lw, 16);
        lw += xor32(lw);
#pragma unroll
        for (int d = 0; d < DL; ++d) {
            float x = acc[h][d];
            x += shfl_xor(x, 16);
            x += xor32(x);
            acc[h][d] = x;
        }
        if (r == 0) {
#pragma unroll
            for (int d = 0; d < DL; ++d) sm_acc[wave][h][c * DL + d] = acc[h][d];
        }
        if (lane == 0) {
            sm_m[wave][h] = m[h];
            sm_l[wave][h] = lw;
        }
    }
    __syncthreads();
    for (int i = tid; i < GH * D; i += 256) {
        const int h = i / D, d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sc = fast_exp2(sm_m[w][h] - M);
                L += sc * sm_l[w][h];
                O += sc * sm_acc[w][h][d];
            }
        }
        const size_t row = part_row0 + (size_t)h * a.n_splits;
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
