// state_init.hip -- per-sequence initial table: M[b] = M0 for every sequence b
// (the learned initial state of "Sparse Delta Memory：中文精读笔记" §2.6 is a
// parameter copied into each sequence's state; a bfloat16 table gets M0
// rounded to nearest even), and its adjoint: the gradient of the shared M0 is
// the sum over the sequences of their state gradients.
#include "sdm_internal.h"

namespace sdm {
namespace {

// nearest-even bfloat16 of a finite fp32 value, as its 16 bits
__device__ __forceinline__ uint32_t rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void state_init_kernel(const float4* __restrict__ M0, float4* __restrict__ M,
                                                         int64_t per_seq4, int64_t B) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per_seq4; i += stride) {
        const float4 x = M0[i];
        for (int64_t b = 0; b < B; ++b) M[b * per_seq4 + i] = x;
    }
}

// The same copy into bfloat16 tables: each element rounded to nearest even.
__global__ __launch_bounds__(256) void state_init_bf16_kernel(const float4* __restrict__ M0, uint2* __restrict__ M,
                                                              int64_t per_seq4, int64_t B) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per_seq4; i += stride) {
        const float4 x = M0[i];
        const uint2 h = make_uint2(rne(x.x) | (rne(x.y) << 16), rne(x.z) | (rne(x.w) << 16));
        for (int64_t b = 0; b < B; ++b) M[b * per_seq4 + i] = h;
    }
}

// dM0 = sum over b of dM[b], added in sequence order.
__global__ __launch_bounds__(256) void state_init_backward_kernel(const float4* __restrict__ dM,
                                                                  float4* __restrict__ dM0, int64_t per_seq4,
                                                                  int64_t B) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per_seq4; i += stride) {
        float4 acc = dM[i];
        for (int64_t b = 1; b < B; ++b) {
            const float4 x = dM[b * per_seq4 + i];
            acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
        }
        dM0[i] = acc;
    }
}

}  // namespace

hipError_t launch_state_init_backward(const float* dM, float* dM0, int64_t B, int64_t per_seq, hipStream_t st) {
    const int64_t per4 = per_seq / 4;
    int64_t blocks = (per4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(state_init_backward_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(dM), reinterpret_cast<float4*>(dM0), per4, B);
    return hipGetLastError();
}

hipError_t launch_state_init(const float* M0, void* M, bool m_bf16, int64_t B, int64_t per_seq, hipStream_t st) {
    const int64_t per4 = per_seq / 4;
    int64_t blocks = (per4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (m_bf16)
        hipLaunchKernelGGL(state_init_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                           reinterpret_cast<const float4*>(M0), static_cast<uint2*>(M), per4, B);
    else
        hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                           reinterpret_cast<const float4*>(M0), static_cast<float4*>(M), per4, B);
    return hipGetLastError();
}

}  // namespace sdm
