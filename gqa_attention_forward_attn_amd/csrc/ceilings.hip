// ceilings.hip - two measurement kernels that give the rooflines of the
// attention kernels a measured ceiling beside the published peaks:
//
//   * an MFMA-only loop: every wave issues back-to-back
//     v_mfma_f32_32x32x16_bf16 (the instruction of the prefill contractions)
//     on four independent accumulators held in registers, with no memory
//     traffic and no other work, at the occupancy of the ping-pong prefill
//     kernel (8 waves per workgroup, one workgroup per compute unit, two waves
//     per SIMD).  Its rate is what the matrix cores sustain at the clock the
//     chip holds under a full MFMA load.
//   * a streaming read: every byte of a buffer read once with 16-byte loads,
//     grid-stride, summed into one word per workgroup.  Its rate is what HBM
//     delivers to a pure read stream (the access the decode kernels make).
#include "gqa_ceilings.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512, 1) void mfma_loop_kernel(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
        b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    // one word per thread: the accumulators must be live at the end
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, size_t n16, uint32_t* out) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    // four independent loads in flight per thread
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc += v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // wave sum, then one word per workgroup (LDS)
    __shared__ uint32_t part[4];
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

extern "C" {

long long gqa_ceiling_mfma_flops(int n_workgroups, int iters) {
    if (n_workgroups <= 0 || iters <= 0) return 0;
    // 8 waves x iters x 16 MFMAs of 32 x 32 x 16 (2 flop per multiply-add)
    return (long long)n_workgroups * 8 * iters * 16 * (2LL * 32 * 32 * 16);
}

int gqa_ceiling_mfma(int n_workgroups, int iters, float* out, void* hip_stream) {
    if (n_workgroups <= 0 || iters <= 0 || !out) return 1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)n_workgroups), dim3(512), 0,
                       static_cast<hipStream_t>(hip_stream), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int gqa_ceiling_stream_read(const void* src, size_t bytes, int n_workgroups, uint32_t* out, void* hip_stream) {
    if (!src || !out || n_workgroups <= 0 || bytes == 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)n_workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const u32x4*>(src), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
