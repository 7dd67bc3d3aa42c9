// state_init.hip -- per-sequence initial table: M[b] = M0 for every sequence b
// (the learned initial state of "Sparse Delta Memory：中文精读笔记" §2.6 is a
// parameter copied into each sequence's state), and its adjoint: the gradient
// of the shared M0 is the sum over the sequences of their state gradients.
#include "sdm_internal.h"

namespace sdm {
namespace {

__global__ __launch_bounds__(256) void state_init_kernel(const float4* __restrict__ M0, float4* __restrict__ M,
                                                         int64_t per_seq4, int64_t B) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per_seq4; i += stride) {
        const float4 x = M0[i];
        for (int64_t b = 0; b < B; ++b) M[b * per_seq4 + i] = x;
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

hipError_t launch_state_init(const float* M0, float* M, int64_t B, int64_t per_seq, hipStream_t st) {
    const int64_t per4 = per_seq / 4;
    int64_t blocks = (per4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(M0), reinterpret_cast<float4*>(M), per4, B);
    return hipGetLastError();
}

}  // namespace sdm
