// scan.hip -- the sparse gated delta scan of the SDM layer on gfx950.
//
// What it computes ("Sparse Delta Memory：中文精读笔记" §2.4 Eq. (3)-(5) and the
// Fig. 2 reading of §2.5): per (sequence, head) and token t, in order:
//   for each selected write row i:  Mt_i = alpha_t M[i]
//       EQ4:  M[i] = Mt_i + beta_t w_i (v_t - Mt_i)
//       FIG2: M[i] = Mt_i + beta_t w_i (v_t - sum_j w_j Mt_j)
//   y_t = sum over the read rows of wr_i M[i]  (after this token's writes).
// Rows that are not selected for writing are never loaded for writing nor
// stored, so they stay bit-identical.
//
// Design. The columns of the table never interact (both forms are per column),
// so one wavefront owns one (stream, column slab of S floats) and runs the whole
// token loop on the device. All indices are known before the scan (they are the
// addressing output), so a planner kernel first resolves every read-after-write
// hazard from the indices alone:
//   * the scan issues the row loads of token t+D while it processes token t
//     (a register ring, D tokens deep), so a row written by a token in
//     [t+D-D, t+D) is stale in HBM at load time; the planner marks such an
//     access "forward from token t+D-d, write position p" and the scan takes the
//     value from an LDS ring of recently written rows instead;
//   * a read of a row written by the same token forwards with d = 0.
// Everything else is ordered by the single wavefront: its loads and stores of
// one address are performed in program order, so a load issued after a store
// (any lane) returns the stored value. No barriers are needed.
//
// Placement: workgroups are dealt to the 8 XCDs round-robin, so blockIdx is
// remapped to put every slab of a stream on the same XCD; the slabs of a row
// then share that XCD's L2 lines, and HBM sees whole 128-byte lines.
#include "sdm_internal.h"

namespace sdm {
namespace {

// Plan entry, one per (token, access): .x = packed, .y = weight bits.
constexpr uint32_t ENT_INVALID = 1u << 31;  // padding or out-of-range index: no access
constexpr uint32_t ENT_FWD = 1u << 30;      // value comes from the LDS ring
constexpr uint32_t ROW_MASK = (1u << 18) - 1u;
constexpr int POS_SHIFT = 18;               // write position of the source (8 bits)
constexpr int DIST_SHIFT = 26;              // token distance of the source (4 bits)

// Lane layout of a slab of S fp32 columns: L = S/4 lanes per row segment
// (16 B each), G = 64/L rows per wavefront-wide load, NGX groups of G rows per
// branch; per token the plan record is a 16-byte header (alpha, beta) followed
// by entries [r][g] for r < G, g < 2*NGX (g < NGX: write p = g*G + r, else read
// p = (g-NGX)*G + r).
constexpr int rec_bytes(int S, int NGX) { return 16 + (64 / (S / 4)) * 2 * NGX * 8; }

struct Inst {
    int S, NGX, D, DM;
};
// Instances: the prefetch depth D and the plan lead DM are set by the VGPR
// budget of each geometry.
constexpr Inst kInst[] = {
    {32, 1, 6, 3},  // W, R <= 8
    {16, 1, 6, 3},  // W, R <= 16
    {8, 2, 3, 2},   // W, R <= 64
    {4, 1, 6, 3},   // W, R <= 64, 16-byte segments (more wavefronts per stream)
    {4, 4, 2, 1},   // W, R <= 256
};

// ------------------------------------------------------------------ planner
constexpr int HT_CAP = 8192;  // LDS hash table entries (64-bit)
constexpr unsigned long long HT_EMPTY = ~0ull;

__device__ __forceinline__ uint32_t ht_hash(uint32_t row) { return (row * 2654435761u) >> (32 - 13); }

__global__ __launch_bounds__(256) void plan_kernel(
    const int32_t* __restrict__ idx_w, const float* __restrict__ wt_w, int W,
    const int32_t* __restrict__ idx_r, const float* __restrict__ wt_r, int R,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    uint8_t* __restrict__ plan, int64_t T, int64_t N, int D, int G, int NGX, int TT,
    int64_t ntile) {
    __shared__ unsigned long long ht[HT_CAP];
    const int tid = threadIdx.x;
    const int64_t s = blockIdx.x / ntile;
    const int64_t t0 = (blockIdx.x % ntile) * TT;
    const int64_t t1 = t0 + TT < T ? t0 + TT : T;
    const int64_t h0 = t0 - D > 0 ? t0 - D : 0;
    const int NG = 2 * NGX;
    const int64_t REC = 16 + (int64_t)G * NG * 8;
    const int32_t* iw = idx_w + s * T * W;
    const float* ww = wt_w + s * T * W;
    const int32_t* ir = idx_r + s * T * R;
    const float* wr = wt_r + s * T * R;
    uint8_t* P = plan + s * T * REC;

    for (int i = tid; i < HT_CAP; i += 256) ht[i] = HT_EMPTY;
    __syncthreads();
    // every write of tokens [h0, t1): key = row, value = (token - h0, position)
    const int64_t nins = (t1 - h0) * W;
    for (int64_t e = tid; e < nins; e += 256) {
        const int64_t tt = h0 + e / W;
        const int p = (int)(e % W);
        const int32_t row = iw[tt * W + p];
        if (row < 0 || row >= N) continue;
        const unsigned long long ent = ((unsigned long long)(uint32_t)row << 32) |
                                       ((unsigned long long)(tt - h0) << 16) | (unsigned)p;
        uint32_t hsh = ht_hash((uint32_t)row);
        while (atomicCAS(&ht[hsh], HT_EMPTY, ent) != HT_EMPTY) hsh = (hsh + 1) & (HT_CAP - 1);
    }
    __syncthreads();

    const int per_tok = G * NG;
    const int64_t nent = (t1 - t0) * per_tok;
    for (int64_t e = tid; e < nent; e += 256) {
        const int64_t tt = t0 + e / per_tok;
        const int rem = (int)(e % per_tok);
        const int rr = rem / NG, g = rem % NG;
        const bool isw = g < NGX;
        const int p = (isw ? g : g - NGX) * G + rr;
        uint32_t packed = ENT_INVALID;
        float w = 0.f;
        if (p < (isw ? W : R)) {
            const int32_t row = isw ? iw[tt * W + p] : ir[tt * R + p];
            if (row >= 0 && row < N) {
                w = isw ? ww[tt * W + p] : wr[tt * R + p];
                packed = (uint32_t)row;
                // latest writer of this row in [tt-D, tt-1] (writes) or [tt-D, tt] (reads)
                const int64_t lo = tt - D, hi = isw ? tt - 1 : tt;
                int64_t best = -1;
                uint32_t bp = 0;
                uint32_t hsh = ht_hash((uint32_t)row);
                unsigned long long ent;
                while ((ent = ht[hsh]) != HT_EMPTY) {
                    if ((uint32_t)(ent >> 32) == (uint32_t)row) {
                        const int64_t tw = h0 + (int64_t)((ent >> 16) & 0xFFFFu);
                        if (tw >= lo && tw <= hi && tw > best) {
                            best = tw;
                            bp = (uint32_t)(ent & 0xFFFFu);
                        }
                    }
                    hsh = (hsh + 1) & (HT_CAP - 1);
                }
                if (best >= 0)
                    packed |= ENT_FWD | ((uint32_t)(tt - best) << DIST_SHIFT) | (bp << POS_SHIFT);
            }
        }
        *reinterpret_cast<int2*>(P + tt * REC + 16 + (int64_t)(rr * NG + g) * 8) =
            make_int2((int)packed, __float_as_int(w));
    }
    for (int64_t tt = t0 + tid; tt < t1; tt += 256)
        *reinterpret_cast<float4*>(P + tt * REC) = make_float4(alpha[s * T + tt], beta[s * T + tt], 0.f, 0.f);
}

// ------------------------------------------------------------------ scan
template <bool BF16>
struct VLoad;
template <>
struct VLoad<false> {
    using T4 = float4;
    __device__ static T4 load(const void* base, int64_t off) {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    }
    __device__ static float4 f(const T4& x) { return x; }
};
template <>
struct VLoad<true> {
    using T4 = uint2;
    __device__ static T4 load(const void* base, int64_t off) {
        return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    }
    __device__ static float4 f(const T4& x) {
        return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u));
    }
};

__device__ __forceinline__ float4 f4_scale(float s, float4 a) {
    return make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
}
__device__ __forceinline__ float4 f4_fma(float s, float4 a, float4 c) {  // s*a + c
    return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}
__device__ __forceinline__ float4 f4_sub(float4 a, float4 b) {
    return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 f4_xor(float4 a, int m) {
    return make_float4(__shfl_xor(a.x, m), __shfl_xor(a.y, m), __shfl_xor(a.z, m), __shfl_xor(a.w, m));
}
__device__ __forceinline__ float4 f4_add(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

template <int S, int NGX, int D, int DM, int FORM, bool VBF16>
__global__ __launch_bounds__(64) void scan_kernel(const uint8_t* __restrict__ plan, const void* __restrict__ v,
                                                  float* M, float* __restrict__ y, float* sink_base, int64_t T,
                                                  int64_t N, int dv, int nslab, int64_t NS) {
    constexpr int L = S / 4, G = 64 / L, NG = 2 * NGX, U = D + DM + 1;
    constexpr int REC = rec_bytes(S, NGX);
    using VL = VLoad<VBF16>;
    using V4 = typename VL::T4;
    __shared__ float4 ring[U][NGX * G][L];

    const int lane = threadIdx.x, r = lane / L, cc = lane % L;
    const int b = blockIdx.x, xcd = b & 7, kq = b >> 3;
    const int64_t s = (int64_t)(kq / nslab) * 8 + xcd;
    const int slab = kq % nslab;
    if (s >= NS) return;
    const int col = slab * S + cc * 4;
    float* Ms = M + s * N * dv + col;
    const uint8_t* Ps = plan + s * T * REC + 16 + r * NG * 8;
    const float2* Hs = reinterpret_cast<const float2*>(plan + s * T * REC);
    const int64_t voff = s * T * dv + col;
    float* ys = y + s * T * dv + col;
    float* sink = sink_base + ((int64_t)blockIdx.x * 64 + lane) * 4;

    struct Meta {
        float2 ab;
        int2 e[NG];
    };
    auto load_meta = [&](int64_t t, Meta& m) {
        m.ab = Hs[t * (REC / 8)];
        const int4* ep = reinterpret_cast<const int4*>(Ps + t * REC);
#pragma unroll
        for (int q = 0; q < NG / 2; ++q) {
            const int4 w4 = ep[q];
            m.e[2 * q] = make_int2(w4.x, w4.y);
            m.e[2 * q + 1] = make_int2(w4.z, w4.w);
        }
    };
    auto load_rows = [&](int64_t t, const Meta& m, float4 (&rw)[NG], V4& vt) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint32_t row = (uint32_t)m.e[g].x & ROW_MASK;
            rw[g] = *reinterpret_cast<const float4*>(Ms + (int64_t)row * dv);
        }
        vt = VL::load(v, voff + t * dv);
    };
    auto fwd_src = [&](int64_t t, uint32_t pk) -> float4 {
        const int d = (int)((pk >> DIST_SHIFT) & 15u);
        const int pos = (int)((pk >> POS_SHIFT) & 255u);
        return ring[(int)((t - d) % U)][pos][cc];
    };
    auto process = [&](int64_t t, int slot, const Meta& m, const float4 (&rw)[NG], const V4& vt) {
        const float alpha = m.ab.x, beta = m.ab.y;
        const float4 vf = VL::f(vt);
        // ---- write rows: decay (Eq. 3), delta correction (Eq. 4 or Fig. 2)
        float4 src[NGX];
        bool fw = false;
#pragma unroll
        for (int g = 0; g < NGX; ++g) {
            src[g] = rw[g];
            fw |= ((uint32_t)m.e[g].x & (ENT_FWD | ENT_INVALID)) == ENT_FWD;
        }
        if (__ballot(fw) != 0ull) {
#pragma unroll
            for (int g = 0; g < NGX; ++g) {
                const uint32_t pk = (uint32_t)m.e[g].x;
                if ((pk & (ENT_FWD | ENT_INVALID)) == ENT_FWD) src[g] = fwd_src(t, pk);
            }
        }
        float4 mt[NGX];
#pragma unroll
        for (int g = 0; g < NGX; ++g) mt[g] = f4_scale(alpha, src[g]);
        float4 vhat = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (FORM == 1) {
#pragma unroll
            for (int g = 0; g < NGX; ++g) {
                const bool ok = ((uint32_t)m.e[g].x & ENT_INVALID) == 0u;
                vhat = f4_fma(ok ? __int_as_float(m.e[g].y) : 0.f, mt[g], vhat);
            }
#pragma unroll
            for (int msk = L; msk < 64; msk <<= 1) vhat = f4_add(vhat, f4_xor(vhat, msk));
        }
#pragma unroll
        for (int g = 0; g < NGX; ++g) {
            const uint32_t pk = (uint32_t)m.e[g].x;
            const float bw = beta * __int_as_float(m.e[g].y);
            const float4 res = f4_sub(vf, FORM == 1 ? vhat : mt[g]);
            const float4 nv = f4_fma(bw, res, mt[g]);
            // masked lanes store into this wavefront's sink instead of branching, so
            // every iteration issues the same memory operations (exact vmcnt waits)
            float* dst = (pk & ENT_INVALID) == 0u ? Ms + (int64_t)(pk & ROW_MASK) * dv : sink;
            *reinterpret_cast<float4*>(dst) = nv;
            ring[slot][g * G + r][cc] = nv;
        }
        // ---- read rows (Eq. 5), after this token's writes
        float4 rs[NGX];
        bool fr = false;
#pragma unroll
        for (int g = 0; g < NGX; ++g) {
            rs[g] = rw[NGX + g];
            fr |= ((uint32_t)m.e[NGX + g].x & (ENT_FWD | ENT_INVALID)) == ENT_FWD;
        }
        if (__ballot(fr) != 0ull) {
#pragma unroll
            for (int g = 0; g < NGX; ++g) {
                const uint32_t pk = (uint32_t)m.e[NGX + g].x;
                if ((pk & (ENT_FWD | ENT_INVALID)) == ENT_FWD) rs[g] = fwd_src(t, pk);
            }
        }
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int g = 0; g < NGX; ++g) {
            const bool ok = ((uint32_t)m.e[NGX + g].x & ENT_INVALID) == 0u;
            acc = f4_fma(ok ? __int_as_float(m.e[NGX + g].y) : 0.f, rs[g], acc);
        }
#pragma unroll
        for (int msk = L; msk < 64; msk <<= 1) acc = f4_add(acc, f4_xor(acc, msk));
        // the butterfly leaves the same sum on every lane of a column chunk: all store it
        *reinterpret_cast<float4*>(ys + t * dv) = acc;
    };

    int64_t t_done = 0;
    if (T >= U) {
        Meta meta[U];
        float4 rows[U][NG];
        V4 vv[U];
#pragma unroll
        for (int q = 0; q < D + DM; ++q) load_meta(q < T ? q : T - 1, meta[q]);
        // keep the plan loads ahead of the row loads: the first loop iteration then
        // waits only for its own data, as every later one does
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < D; ++q) load_rows(q, meta[q], rows[q], vv[q]);
        __builtin_amdgcn_sched_barrier(0);
        for (int64_t t0 = 0; t0 + U <= T; t0 += U) {
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int64_t t = t0 + j;
                const int64_t tm = t + D + DM < T ? t + D + DM : T - 1;
                load_meta(tm, meta[(j + D + DM) % U]);
                const int64_t tr = t + D < T ? t + D : T - 1;
                load_rows(tr, meta[(j + D) % U], rows[(j + D) % U], vv[(j + D) % U]);
                process(t, j, meta[j], rows[j], vv[j]);
            }
            t_done = t0 + U;
        }
    }
    // tail (and short sequences): loads right before use; forwarding stays valid
    for (int64_t t = t_done; t < T; ++t) {
        Meta m;
        float4 rw[NG];
        V4 vt;
        load_meta(t, m);
        load_rows(t, m, rw, vt);
        process(t, (int)(t % U), m, rw, vt);
    }
}

template <int S, int NGX, int D, int DM>
hipError_t launch_scan_inst(const ScanArgs& a, hipStream_t st) {
    const int G = 64 / (S / 4);
    // planner: tiles of TT tokens; the hash table holds the writes of TT + D tokens at load <= 1/2
    int TT = HT_CAP / (2 * a.W) - D;
    if (TT < 1) TT = 1;
    const int64_t ntile = (a.T + TT - 1) / TT;
    uint8_t* plan = static_cast<uint8_t*>(a.workspace);
    hipLaunchKernelGGL(plan_kernel, dim3((unsigned)(ntile * a.NS)), dim3(256), 0, st, a.idx_w, a.wt_w, a.W,
                       a.idx_r, a.wt_r, a.R, a.alpha, a.beta, plan, a.T, a.N, D, G, NGX, TT, ntile);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslab = a.dv / S;
    const int64_t nblk = ((a.NS + 7) / 8) * 8 * nslab;
    float* sink = reinterpret_cast<float*>(plan + a.NS * a.T * rec_bytes(S, NGX));
    dim3 grid((unsigned)nblk);
#define SDM_LAUNCH(FORM, VB)                                                                            \
    hipLaunchKernelGGL((scan_kernel<S, NGX, D, DM, FORM, VB>), grid, dim3(64), 0, st, plan, a.v, a.M, \
                       a.y, sink, a.T, a.N, a.dv, nslab, a.NS)
    if (a.form == 0) {
        if (a.v_bf16) SDM_LAUNCH(0, true); else SDM_LAUNCH(0, false);
    } else {
        if (a.v_bf16) SDM_LAUNCH(1, true); else SDM_LAUNCH(1, false);
    }
#undef SDM_LAUNCH
    return hipGetLastError();
}

int pick_instance(int W, int R, int dv) {
    const int K = W > R ? W : R;
    int forced = 0;
    if (const char* e = getenv("SDM_SCAN_SLAB")) forced = atoi(e);
    for (int i = 0; i < (int)(sizeof(kInst) / sizeof(kInst[0])); ++i) {
        const Inst& in = kInst[i];
        const int G = 64 / (in.S / 4);
        if (K > in.NGX * G || dv % in.S != 0) continue;
        if (forced && forced != in.S) continue;
        return i;
    }
    return -1;
}

}  // namespace

bool scan_geometry(int W, int R, int dv, int* slab, int* rec) {
    const int i = pick_instance(W, R, dv);
    if (i < 0) return false;
    if (slab) *slab = kInst[i].S;
    if (rec) *rec = rec_bytes(kInst[i].S, kInst[i].NGX);
    return true;
}

int64_t scan_workspace_bytes(int64_t NS, int64_t T, int W, int R, int dv) {
    int rec = 0, S = 0;
    if (!scan_geometry(W, R, dv, &S, &rec)) return -1;
    const int64_t nblk = ((NS + 7) / 8) * 8 * (dv / S);
    return NS * T * rec + nblk * 64 * 16;  // plan records + one 16-byte sink per lane
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    switch (pick_instance(a.W, a.R, a.dv)) {
        case 0: return launch_scan_inst<32, 1, 6, 3>(a, st);
        case 1: return launch_scan_inst<16, 1, 6, 3>(a, st);
        case 2: return launch_scan_inst<8, 2, 3, 2>(a, st);
        case 3: return launch_scan_inst<4, 1, 6, 3>(a, st);
        case 4: return launch_scan_inst<4, 4, 2, 1>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdm
