// merge_bwd.hip - backward of the split-K merge (splitk_kernels.py,
// `_splitK_reduce_varargs_backward`).
//
// The forward merge of n_splits partial results (O_s, L_s) of a row is
// O = sum_s w_s O_s and L = log sum_s exp(L_s) with w_s = exp(L_s - L).  Given
// the merged (O, L) and the gradients (dO, dL) of some scalar with respect to
// them, the gradients with respect to the partials are
//   dO_s = w_s dO,
//   dL_s = w_s (dL + sum_d (O_s - O)_d dO_d),
// zero for an empty partial (L_s = -inf) and for every partial of a row whose
// L is -inf.  One wave per row.  With D a multiple of 4 and 16-byte aligned
// rows, lane groups take several partials of the row at once through 16-byte
// accesses, every load of a step issued before any is used; otherwise lanes
// stride over the D dims one float at a time and the dot product is a wave sum
// per partial.  Memory-bound; everything in fp32.
#include "gqa_device.hpp"
#include "gqa_kernels.hpp"

namespace gqa {

namespace {

constexpr int kMaxDims = 512;  // dims per lane: D / 64 <= 8

template <int PER>
__global__ __launch_bounds__(256) void merge_backward_kernel(MergeBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;  // wave-uniform
    const int D = a.D, S = a.n_splits;
    const float L = a.lse[row];
    const float dL = a.d_lse[row];
    float o[PER], dout[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int d = lane + 64 * j;
        o[j] = d < D ? a.o[row * D + d] : 0.f;
        dout[j] = d < D ? a.d_o[row * D + d] : 0.f;
    }
    for (int s = 0; s < S; ++s) {
        const long long ps = row * S + s;
        const float Ls = a.lse_parts[ps];
        const float w = (Ls == -INFINITY || L == -INFINITY) ? 0.f : expf(Ls - L);
        const float* os = a.o_parts + ps * D;
        float* dos = a.d_o_parts + ps * D;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int d = lane + 64 * j;
            if (d < D) {
                dot = fmaf(os[d] - o[j], dout[j], dot);
                dos[d] = w * dout[j];
            }
        }
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) dot += shfl_xor(dot, k);
        if (lane == 0) a.d_lse_parts[ps] = w == 0.f ? 0.f : w * (dL + dot);
    }
}

// The same with 16-byte accesses, for D a multiple of 4 and 16-byte aligned
// rows: VL lanes (a power of two, VL >= D / 4 / VEC) hold VEC float4 pieces of a
// row each, and the 64 / VL lane groups of a wave take different partials of
// the row at the same time, all of the row's partials issued before any is
// used.
template <int VL, int VEC, int MAXS>
__global__ __launch_bounds__(256) void merge_backward_vec_kernel(MergeBwdArgs a) {
    constexpr int SPW = 64 / VL;  // partials in flight per wave and step
    const int lane = threadIdx.x & 63;
    const int sub = lane / VL, vl = lane % VL;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;  // wave-uniform
    const int D = a.D, S = a.n_splits, D4 = D / 4;
    const float L = a.lse[row];
    const float dL = a.d_lse[row];
    f32x4 o[VEC], dout[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
        const int q = vl + VL * c;  // float4 index in the row
        o[c] = q < D4 ? reinterpret_cast<const f32x4*>(a.o + row * D)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
        dout[c] = q < D4 ? reinterpret_cast<const f32x4*>(a.d_o + row * D)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < S; s0 += SPW * MAXS) {
        f32x4 os[MAXS][VEC];
        float Ls[MAXS];
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            const int s = s0 + SPW * k + sub;
            const long long ps = row * S + min(s, S - 1);
            Ls[k] = a.lse_parts[ps];
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                const int q = vl + VL * c;
                os[k][c] = q < D4 ? reinterpret_cast<const f32x4*>(a.o_parts + ps * D)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            const int s = s0 + SPW * k + sub;
            const long long ps = row * S + s;
            const float w = (Ls[k] == -INFINITY || L == -INFINITY) ? 0.f : expf(Ls[k] - L);
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                const int q = vl + VL * c;
#pragma unroll
                for (int e = 0; e < 4; ++e) dot = fmaf(os[k][c][e] - o[c][e], dout[c][e], dot);
                if (s < S && q < D4)
                    reinterpret_cast<f32x4*>(a.d_o_parts + ps * D)[q] =
                        f32x4{w * dout[c][0], w * dout[c][1], w * dout[c][2], w * dout[c][3]};
            }
#pragma unroll
            for (int m = VL / 2; m >= 1; m >>= 1) dot += shfl_xor(dot, m);  // within the lane group
            if (s < S && vl == 0) a.d_lse_parts[ps] = w == 0.f ? 0.f : w * (dL + dot);
        }
    }
}

template <int VL, int VEC>
hipError_t launch_vec(const MergeBwdArgs& a, hipStream_t stream) {
    const long long blocks = (a.rows + 3) / 4;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    constexpr int SPW = 64 / VL;
    if (a.n_splits >= 2 * SPW)
        hipLaunchKernelGGL((merge_backward_vec_kernel<VL, VEC, 2>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((merge_backward_vec_kernel<VL, VEC, 1>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int PER>
hipError_t launch_per(const MergeBwdArgs& a, hipStream_t stream) {
    const long long blocks = (a.rows + 3) / 4;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((merge_backward_kernel<PER>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int merge_backward_max_dims() { return kMaxDims; }

hipError_t launch_merge_backward(const MergeBwdArgs& a, hipStream_t stream) {
    const void* rows_base[4] = {a.o_parts, a.o, a.d_o, a.d_o_parts};
    bool vec = a.D % 4 == 0;
    for (const void* p : rows_base) vec = vec && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
    if (vec) {
        if (a.D <= 64) return launch_vec<16, 1>(a, stream);
        if (a.D <= 128) return launch_vec<32, 1>(a, stream);
        if (a.D <= 256) return launch_vec<64, 1>(a, stream);
        return launch_vec<64, 2>(a, stream);
    }
    if (a.D <= 64) return launch_per<1>(a, stream);
    if (a.D <= 128) return launch_per<2>(a, stream);
    if (a.D <= 256) return launch_per<4>(a, stream);
    return launch_per<8>(a, stream);
}

}  // namespace gqa
