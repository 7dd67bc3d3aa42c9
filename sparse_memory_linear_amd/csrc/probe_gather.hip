// probe_gather.hip -- a measurement aid, not part of the SDM path: the rate at
// which one MI355X moves random row pieces in place, the access pattern of the
// scan's table traffic (a read of a piece of a random row, and for half of the
// pieces a write back to the same place). It gives the practical ceiling that
// the scan's HBM fraction is set against; the published 8 TB/s stays the peak.
//
// The table is rows x 512 bytes (one d_v = 128 fp32 row each); an access
// reads piece_bytes (64 .. 512) at a random piece of a random row, picked by
// an integer hash of the access number, so every offset is inside the table.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm_probe.h"

namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <int B>
__global__ __launch_bounds__(256) void gather_rmw_kernel(float4* tab, uint32_t rows, int64_t naccess, float* sink) {
    constexpr int LPA = B / 16;  // lanes per access (16 bytes each)
    constexpr int PIECES = 512 / B;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
    const int l = (int)(tid % LPA);
    float acc = 0.f;
    for (int64_t k = tid / LPA; k < naccess; k += nthr / LPA) {
        const uint32_t h = mix32((uint32_t)k * 2654435761u + 12345u);
        const uint32_t row = h % rows, piece = mix32(h) % PIECES;
        const int64_t i = (int64_t)row * 32 + (int64_t)piece * LPA + l;  // < rows * 32 float4
        float4 v = tab[i];
        acc += v.x;
        if (k & 1) {
            v.x += 1.f;
            tab[i] = v;
        }
    }
    sink[tid] = acc;
}

}  // namespace

extern "C" int sdm_probe_gather(float* tab, int64_t rows, int piece_bytes, int64_t naccess, int grid, float* sink,
                                void* stream) {
    if (!tab || !sink || rows < 1 || rows > 0x7FFFFFFF || naccess < 0 || grid < 1 || grid > 65536) return 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float4* t = reinterpret_cast<float4*>(tab);
    const uint32_t r = (uint32_t)rows;
    switch (piece_bytes) {
        case 64: hipLaunchKernelGGL(gather_rmw_kernel<64>, dim3(grid), dim3(256), 0, st, t, r, naccess, sink); break;
        case 128: hipLaunchKernelGGL(gather_rmw_kernel<128>, dim3(grid), dim3(256), 0, st, t, r, naccess, sink); break;
        case 256: hipLaunchKernelGGL(gather_rmw_kernel<256>, dim3(grid), dim3(256), 0, st, t, r, naccess, sink); break;
        case 512: hipLaunchKernelGGL(gather_rmw_kernel<512>, dim3(grid), dim3(256), 0, st, t, r, naccess, sink); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
