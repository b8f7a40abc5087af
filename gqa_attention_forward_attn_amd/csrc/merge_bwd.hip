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
// L is -inf.  One wave per row: lanes stride over the D dims, the dot product
// is a wave sum per partial.  Memory-bound; everything in fp32.
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
    if (a.D <= 64) return launch_per<1>(a, stream);
    if (a.D <= 128) return launch_per<2>(a, stream);
    if (a.D <= 256) return launch_per<4>(a, stream);
    return launch_per<8>(a, stream);
}

}  // namespace gqa
