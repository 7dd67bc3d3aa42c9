// state_init.hip -- per-sequence initial table: M[b] = M0 for every sequence b
// (the learned initial state of "Sparse Delta Memory：中文精读笔记" §2.6 is a
// parameter copied into each sequence's state).
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

}  // namespace

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
