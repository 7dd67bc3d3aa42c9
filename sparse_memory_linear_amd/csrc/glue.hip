// glue.hip -- the steps either side of the SDM scan on gfx950.
//
// What they compute ("Sparse Delta Memory：中文精读笔记" §2.4):
//   gates, per token and head, from the layer input x_t:
//     alpha_t = exp(-A softplus(W_a x_t + b_dt)),   beta_t = sigmoid(W_b x_t)
//   output, per head after the read: RMS-Norm of y_t, then an elementwise
//   output gate, read as o = y / sqrt(mean(y^2) + eps) * gamma * sigmoid(g)
//   (the sigmoid is the gate activation "Fast-weight Product Key Memory：中文
//   精读笔记" §2.3 uses; the SDM notes name the gate only).
//
// gates_kernel: the two projections of all heads form one skinny GEMM
// [tokens x d] x [d x 2H]; a wavefront computes a 16-token x 16-column tile on
// MFMA (bf16 16x16x32, or fp32 16x16x4), fp32 accumulation over all of d, and
// applies softplus / exp / sigmoid in the epilogue, writing alpha and beta in
// the [B, H, T] layout the scan reads. x is read once; the weights (2H x d)
// stay in L2. HBM-bound on x.
//
// output_gate_kernel: a group of LG lanes (a power of two up to 64) owns one
// row of d_v values in 16-byte pieces; the sum of squares is a butterfly over
// the group, then each lane scales, multiplies by gamma and the gate, and
// stores. HBM-bound: y and g in, o out.
//
// ypart_gate_kernel: the same step fused into the scan's last pass where the
// scan splits the table rows into P partitions: a lane adds its pieces' P
// partial sums (in partition order, as the plain partial-sum pass does), keeps
// them in registers for the norm and the gate, and stores y only on request.
// Against partial sums + output gate it saves storing y and reading it back:
// per row P * d_v * 4 + g in, o (+ y) out.
#include "sdm_buffer.h"
#include "sdm_internal.h"

namespace sdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int GW = 4;  // wavefronts (16-token tiles) per workgroup

__device__ __forceinline__ float softplusf(float z) {  // log(1 + e^z) without overflow
    return z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z));
}

template <bool BF16>
__global__ __launch_bounds__(GW * 64) void gates_kernel(GatesArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int64_t UT = a.B * a.T;
    const int64_t u0 = ((int64_t)blockIdx.x * GW + wave) * 16;
    if (u0 >= UT) return;  // uniform per wavefront; no barrier in this kernel
    const int H = a.H, d = a.d, ncol = 2 * H;
    const int64_t ux = u0 + m16;                 // this lane's token as an A-operand row
    const bool tok_ok = ux < UT;
    for (int c0 = 0; c0 < ncol; c0 += 16) {
        const int jc = c0 + m16;                 // this lane's gate column as a B-operand column
        const bool col_ok = jc < ncol;
        const int hrow = jc < H ? jc : jc - H;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
            const uint16_t* xp = static_cast<const uint16_t*>(a.x) + (tok_ok ? ux : 0) * d;
            const uint16_t* wp = static_cast<const uint16_t*>(jc < H ? a.Wa : a.Wb) + (col_ok ? hrow : 0) * (int64_t)d;
#pragma unroll 8
            for (int k = 0; k < d; k += 32) {
                const uint4 xa = tok_ok ? *reinterpret_cast<const uint4*>(xp + k + g4 * 8) : make_uint4(0u, 0u, 0u, 0u);
                const uint4 wb = col_ok ? *reinterpret_cast<const uint4*>(wp + k + g4 * 8) : make_uint4(0u, 0u, 0u, 0u);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa),
                                                              __builtin_bit_cast(bf16x8_t, wb), acc, 0, 0, 0);
            }
        } else {
            const float* xp = static_cast<const float*>(a.x) + (tok_ok ? ux : 0) * d;
            const float* wp = static_cast<const float*>(jc < H ? a.Wa : a.Wb) + (col_ok ? hrow : 0) * (int64_t)d;
#pragma unroll 8
            for (int k = 0; k < d; k += 8) {
                const float2 xa = tok_ok ? *reinterpret_cast<const float2*>(xp + k + g4 * 2) : make_float2(0.f, 0.f);
                const float2 wb = col_ok ? *reinterpret_cast<const float2*>(wp + k + g4 * 2) : make_float2(0.f, 0.f);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa.x, wb.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa.y, wb.y, acc, 0, 0, 0);
            }
        }
        // D layout: lane holds tokens u0 + 4*g4 + i of gate column c0 + m16
        if (!col_ok) continue;
        const bool is_a = jc < H;
        const float bias = is_a ? a.bdt[hrow] : 0.f, Ah = is_a ? a.A[hrow] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t u = u0 + 4 * g4 + i;
            if (u >= UT) break;
            const uint32_t uu = (uint32_t)u, b = uu / (uint32_t)a.T, t = uu - b * (uint32_t)a.T;  // u < 2^32
            const int64_t o = ((int64_t)b * H + hrow) * a.T + t;  // B * H may pass 2^32
            if (is_a) a.alpha[o] = expf(-Ah * softplusf(acc[i] + bias));
            else a.beta[o] = 1.f / (1.f + expf(-acc[i]));
        }
    }
}

template <bool GBF16>
__global__ __launch_bounds__(256) void output_gate_kernel(OutGateArgs a) {
    const int LG = a.lg;  // lanes per row (power of two, <= 64)
    const int lane = threadIdx.x & 63;
    const int sub = lane & (LG - 1);
    const int rows_per_wave = 64 / LG;
    const int64_t wave_g = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * 256) >> 6;
    const int nq = a.dv / 4;  // 16-byte pieces (4 values) per row
    for (int64_t r0 = wave_g * rows_per_wave; r0 < a.rows; r0 += nwaves * rows_per_wave) {
        const int64_t row = r0 + lane / LG;
        const bool ok = row < a.rows;
        const int64_t h = ok ? ((uint32_t)row / (uint32_t)a.T) % (uint32_t)a.H : 0;  // rows < 2^32
        const float4* y4 = reinterpret_cast<const float4*>(a.y) + (ok ? row : 0) * nq;
        float ss = 0.f;
        for (int q = sub; q < nq; q += LG) {
            if (!ok) break;
            const float4 v = y4[q];
            ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
        }
        for (int m = 1; m < LG; m <<= 1) ss += __shfl_xor(ss, m);  // the same sum on every lane of the group
        const float r = 1.f / sqrtf(ss / (float)a.dv + a.eps);
        if (!ok) continue;
        const float4* gm4 = reinterpret_cast<const float4*>(a.gamma) + h * nq;
        float4* o4 = reinterpret_cast<float4*>(a.o) + row * nq;
        for (int q = sub; q < nq; q += LG) {
            const float4 v = y4[q], gm = gm4[q];
            float4 gt;
            if constexpr (GBF16) {
                const uint2 p = reinterpret_cast<const uint2*>(a.g)[row * nq + q];
                gt = make_float4(__uint_as_float(p.x << 16), __uint_as_float(p.x & 0xFFFF0000u),
                                 __uint_as_float(p.y << 16), __uint_as_float(p.y & 0xFFFF0000u));
            } else {
                gt = reinterpret_cast<const float4*>(a.g)[row * nq + q];
            }
            auto sg = [](float z) { return 1.f / (1.f + expf(-z)); };
            o4[q] = make_float4(v.x * r * gm.x * sg(gt.x), v.y * r * gm.y * sg(gt.y), v.z * r * gm.z * sg(gt.z),
                                v.w * r * gm.w * sg(gt.w));
        }
    }
}

// o for one row held by a group of LG lanes: pieces v[j] (q = sub + j * LG < nq)
template <bool GBF16, int NJ>
__device__ __forceinline__ void gate_row(const float4 (&v)[NJ], int sub, int LG, int nq, int dv, float eps,
                                         const float4* gm4, const void* g, int64_t row, float4* o4, bool ok) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int q = sub + j * LG;
        if (ok && q < nq) ss = fmaf(v[j].x, v[j].x, fmaf(v[j].y, v[j].y, fmaf(v[j].z, v[j].z, fmaf(v[j].w, v[j].w, ss))));
    }
    for (int m = 1; m < LG; m <<= 1) ss += __shfl_xor(ss, m);  // the same sum on every lane of the group
    const float r = 1.f / sqrtf(ss / (float)dv + eps);
    if (!ok) return;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int q = sub + j * LG;
        if (q >= nq) break;
        const float4 gm = gm4[q];
        float4 gt;
        if constexpr (GBF16) {
            const uint2 p = reinterpret_cast<const uint2*>(g)[row * nq + q];
            gt = make_float4(__uint_as_float(p.x << 16), __uint_as_float(p.x & 0xFFFF0000u),
                             __uint_as_float(p.y << 16), __uint_as_float(p.y & 0xFFFF0000u));
        } else {
            gt = reinterpret_cast<const float4*>(g)[row * nq + q];
        }
        auto sg = [](float z) { return 1.f / (1.f + expf(-z)); };
        o4[q] = make_float4(v[j].x * r * gm.x * sg(gt.x), v[j].y * r * gm.y * sg(gt.y), v[j].z * r * gm.z * sg(gt.z),
                            v[j].w * r * gm.w * sg(gt.w));
    }
}

template <bool GBF16>
__global__ __launch_bounds__(256) void ypart_gate_kernel(YGateArgs a) {
    constexpr int NJ = GATE_FUSED_PIECES;
    const int LG = output_gate_lanes(a.dv);
    const int lane = threadIdx.x & 63;
    const int sub = lane & (LG - 1);
    const int rows_per_wave = 64 / LG;
    const int64_t wave_g = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * 256) >> 6;
    const int nq = a.dv / 4;
    const int64_t rows = a.NS * a.Tc, n = rows * nq;  // float4 per partition
    const float4* yp = reinterpret_cast<const float4*>(a.yp);
    for (int64_t r0 = wave_g * rows_per_wave; r0 < rows; r0 += nwaves * rows_per_wave) {
        const int64_t rl = r0 + lane / LG;  // row of the chunk: stream s, token t0 + t
        const bool ok = rl < rows;
        const int64_t s = ok ? rl / a.Tc : 0, grow = s * a.TS + a.t0 + (ok ? rl - s * a.Tc : 0);
        float4 v[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int q = sub + j * LG;
            v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (!ok || q >= nq) continue;
            float4 acc = yp[rl * nq + q];
            for (int p = 1; p < a.P; ++p) acc = f4_add(acc, yp[p * n + rl * nq + q]);
            v[j] = acc;
            if (a.y) reinterpret_cast<float4*>(a.y)[grow * nq + q] = acc;
        }
        const float4* gm4 = reinterpret_cast<const float4*>(a.gate.gamma) + (s % a.gate.H) * nq;
        gate_row<GBF16, NJ>(v, sub, LG, nq, a.dv, a.gate.eps, gm4, a.gate.g, grow,
                            reinterpret_cast<float4*>(a.gate.o) + grow * nq, ok);
    }
}

}  // namespace

hipError_t launch_ypart_gate(const YGateArgs& a, hipStream_t st) {
    const int lg = output_gate_lanes(a.dv);
    const int64_t waves = (a.NS * a.Tc + (64 / lg) - 1) / (64 / lg);
    int64_t blocks = (waves + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    if (a.gate.g_bf16)
        hipLaunchKernelGGL(ypart_gate_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(ypart_gate_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gates(const GatesArgs& a, hipStream_t st) {
    const int64_t tiles = (a.B * a.T + 15) / 16;
    const int64_t blocks = (tiles + GW - 1) / GW;
    if (a.bf16)
        hipLaunchKernelGGL(gates_kernel<true>, dim3((unsigned)blocks), dim3(GW * 64), 0, st, a);
    else
        hipLaunchKernelGGL(gates_kernel<false>, dim3((unsigned)blocks), dim3(GW * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_output_gate(OutGateArgs a, hipStream_t st) {
    const int lg = output_gate_lanes(a.dv);
    a.lg = lg;
    const int64_t waves = (a.rows + (64 / lg) - 1) / (64 / lg);
    int64_t blocks = (waves + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    if (a.g_bf16)
        hipLaunchKernelGGL(output_gate_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(output_gate_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace sdm
