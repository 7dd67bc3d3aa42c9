// scan.hip -- the sparse gated delta scan of the SDM layer on gfx950.
//
// What it computes ("Sparse Delta Memory：中文精读笔记" §2.4 Eq. (3)-(5) and the
// Fig. 2 reading of §2.5): per (sequence, head) and token t, in order:
//   for each selected write row i:  Mt_i = alpha_t M[i]
//       EQ4:  M[i] = Mt_i + beta_t w_i (v_t - Mt_i)
//       FIG2: M[i] = Mt_i + beta_t w_i (v_t - sum_j w_j Mt_j)
//   y_t = sum over the read rows of wr_i M[i]  (after this token's writes).
// Rows that are not selected for writing are never stored, so they stay
// bit-identical.
//
// Design. The columns of the table never interact (both forms are per column),
// so one workgroup owns one (stream, column slab of S floats) and runs the
// whole token loop on the device. Inside it, "writer" wavefronts own the W
// write accesses of every token (G rows each) and "reader" wavefronts the R
// read accesses. One workgroup barrier per token orders them (two for FIG2,
// whose shared prediction sums over all writers); on gfx950 a workgroup-scope
// barrier does not drain the memory counters, so each wavefront keeps D tokens
// of row loads in flight across it.
//
// All indices are known before the scan (they are the addressing output), so
// a planner kernel first resolves every read-after-write hazard from the
// indices alone. A wavefront issues the loads of token t+D while it is at
// token t, after the barrier that closed token t-1; stores of tokens < t are
// visible to those loads, rows written by tokens in [t, t+D) are not. The
// planner marks such accesses "forward from token t+D-d, write position p" and
// the scan takes them from an LDS ring of recently written rows; a read of a
// row written by the same token forwards with d = 0 (after the token's barrier).
//
// Placement: workgroups are dealt to the 8 XCDs round-robin, so blockIdx is
// remapped to put every slab of a stream on the same XCD; the slabs of a row
// then share that XCD's L2 lines.
#include "sdm_internal.h"

namespace sdm {
namespace {

// Plan entry, one per (token, access): .x = packed, .y = weight bits.
constexpr uint32_t ENT_INVALID = 1u << 31;  // padding or out-of-range index: no access
constexpr uint32_t ENT_FWD = 1u << 30;      // value comes from the LDS ring
constexpr uint32_t ROW_MASK = (1u << 18) - 1u;
constexpr int POS_SHIFT = 18;               // write position of the source (8 bits)
constexpr int DIST_SHIFT = 26;              // token distance of the source (4 bits)

// Per slab width: D = tokens of row loads in flight per wavefront; the plan
// entries lead by another D + 1 tokens (memory counters complete in order, so
// waiting on an entry also waits on every older row load: a lead >= D keeps D
// tokens of rows in flight); NWMAX = wavefronts per workgroup (sets the VGPR
// budget: 8 -> 256, 16 -> 128). 32-column slabs move whole 128-byte lines per
// row: on MI355X random 128-byte accesses sustain ~1.4x the bandwidth of 64-byte
// ones.
template <int S>
struct SlabCfg {
    static constexpr int D = 10, NWMAX = 8;
};
template <>
struct SlabCfg<32> {
    static constexpr int D = 6, NWMAX = 16;
};
constexpr int MAX_WAVES = 16;   // largest NWMAX

// Geometry of a slab of S fp32 columns: L = S/4 lanes per row segment (16 B
// each), G = 64/L rows per wavefront; NWW = ceil(W/G) writer and NWR = ceil(R/G)
// reader wavefronts. Plan record per token: a 16-byte header (alpha, beta)
// then entries [wave][G] (int2 each): writer wave w, lane row r -> write
// access w*G + r; reader wave NWW+w -> read access w*G + r.
struct Geom {
    int S, G, NWW, NWR;
    int nw() const { return NWW + NWR; }
    int64_t rec() const { return 16 + (int64_t)nw() * G * 8; }
};

Geom make_geom(int S, int W, int R) {
    Geom g;
    g.S = S;
    g.G = 64 / (S / 4);
    g.NWW = (W + g.G - 1) / g.G;
    g.NWR = (R + g.G - 1) / g.G;
    return g;
}

// ------------------------------------------------------------------ planner
constexpr int HT_CAP = 8192;  // LDS hash table entries (64-bit)
constexpr unsigned long long HT_EMPTY = ~0ull;

__device__ __forceinline__ uint32_t ht_hash(uint32_t row) { return (row * 2654435761u) >> (32 - 13); }

__global__ __launch_bounds__(256) void plan_kernel(
    const int32_t* __restrict__ idx_w, const float* __restrict__ wt_w, int W,
    const int32_t* __restrict__ idx_r, const float* __restrict__ wt_r, int R,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    uint8_t* __restrict__ plan, int64_t T, int64_t N, int D, int G, int NWW, int NWR, int TT,
    int64_t ntile) {
    __shared__ unsigned long long ht[HT_CAP];
    const int tid = threadIdx.x;
    const int64_t s = blockIdx.x / ntile;
    const int64_t t0 = (blockIdx.x % ntile) * TT;
    const int64_t t1 = t0 + TT < T ? t0 + TT : T;
    const int64_t h0 = t0 - D > 0 ? t0 - D : 0;
    const int NW = NWW + NWR;
    const int64_t REC = 16 + (int64_t)NW * G * 8;
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

    const int per_tok = NW * G;
    const int64_t nent = (t1 - t0) * per_tok;
    for (int64_t e = tid; e < nent; e += 256) {
        const int64_t tt = t0 + e / per_tok;
        const int rem = (int)(e % per_tok);
        const int wv = rem / G, rr = rem % G;
        const bool isw = wv < NWW;
        const int p = (isw ? wv : wv - NWW) * G + rr;
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
        *reinterpret_cast<int2*>(P + tt * REC + 16 + (int64_t)rem * 8) = make_int2((int)packed, __float_as_int(w));
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
__device__ __forceinline__ float4 f4_add(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// x + (x rotated by N lanes within each row of 16): DPP row_ror
template <int N>
__device__ __forceinline__ float ror_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
// x + its partner 16 (resp. 32) lanes away: the two halves returned by the
// gfx950 permlane swaps of (x, x) are {x, partner} in some order on every lane.
__device__ __forceinline__ float xor16_add(float x) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_add(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum over the G row-lanes that share a column chunk (lanes with equal lane % L);
// every lane ends with its chunk's sum, bit-identical across those lanes.
template <int L>
__device__ __forceinline__ float row_sum(float x) {
    if constexpr (L <= 8) x = ror_add<8>(x);
    if constexpr (L <= 4) x = ror_add<4>(x);
    if constexpr (L <= 2) x = ror_add<2>(x);
    if constexpr (L <= 1) x = ror_add<1>(x);
    x = xor16_add(x);
    return xor32_add(x);
}
template <int L>
__device__ __forceinline__ float4 row_sum4(float4 a) {
    return make_float4(row_sum<L>(a.x), row_sum<L>(a.y), row_sum<L>(a.z), row_sum<L>(a.w));
}

template <int S, int FORM, bool VBF16>
__global__ __launch_bounds__(SlabCfg<S>::NWMAX * 64) void scan_kernel(
    const uint8_t* __restrict__ plan, const void* __restrict__ v, float* M, float* __restrict__ y,
    float* sink_base, int T, int64_t N, int dv, int nslab, int64_t NS, int NWW, int NWR) {
    constexpr int L = S / 4, G = 64 / L;
    constexpr int D = SlabCfg<S>::D, NWMAX = SlabCfg<S>::NWMAX;
    constexpr int DM = D + 1;       // plan-entry lead beyond D
    constexpr int UP = D + 1;       // row / value register rings: D in flight + the one in use
    constexpr int U = D + DM + 1;   // plan-entry ring = unroll factor (a multiple of UP, so
                                    // every ring index is static in the unrolled loop)
    static_assert(U % UP == 0, "ring sizes");
    constexpr int UR = D + 2;       // LDS ring of written rows (see the ring-reuse note below)
    using VL = VLoad<VBF16>;
    using V4 = typename VL::T4;
    extern __shared__ float4 lds[];
    const int NW = NWW + NWR;
    float4* ring = lds;                                  // [UR][NWW*G][L]
    float4* ybuf = lds + UR * NWW * G * L;               // [2][NWR][L]
    float4* vbuf = ybuf + 2 * NWR * L;                   // [NWW][L]

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane / L, cc = lane % L;
    const int b = blockIdx.x, xcd = b & 7, kq = b >> 3;
    const int64_t s = (int64_t)(kq / nslab) * 8 + xcd;
    const int slab = kq % nslab;
    if (s >= NS) return;  // uniform over the workgroup
    const int col = slab * S + cc * 4;
    const float* Mr = M + s * N * dv;                    // this stream's table (row base)
    float* Mw = M + s * N * dv;
    const int64_t REC = 16 + (int64_t)NW * G * 8;
    const uint8_t* Pe = plan + s * (int64_t)T * REC + 16 + (int64_t)(wave * G + r) * 8;
    const uint8_t* Ph = plan + s * (int64_t)T * REC;
    const int64_t voff = s * (int64_t)T * dv + col;
    float* ys = y + s * (int64_t)T * dv + col;
    float* sink = sink_base + ((int64_t)blockIdx.x * (MAX_WAVES * 64) + threadIdx.x) * 4;
    const bool writer = wave < NWW;
    const int pos = wave * G + r;                        // write position of a writer lane
    const int rw = wave - NWW;                           // reader index

    auto ring_at = [&](int slot, int p) -> float4& { return ring[((int64_t)slot * NWW * G + p) * L + cc]; };
    auto load_entry = [&](int t) -> int2 { return *reinterpret_cast<const int2*>(Pe + (int64_t)t * REC); };
    auto load_ab = [&](int t) -> float2 { return *reinterpret_cast<const float2*>(Ph + (int64_t)t * REC); };
    auto load_row = [&](int2 e) -> float4 {
        const uint32_t off = (((uint32_t)e.x & ROW_MASK) * (uint32_t)dv + (uint32_t)col);
        return *reinterpret_cast<const float4*>(Mr + off);
    };
    auto source = [&](int t, int2 e, float4 pre) -> float4 {
        // forwarded rows come from the LDS ring; the ballot keeps the common
        // no-forward case free of LDS traffic
        const uint32_t pk = (uint32_t)e.x;
        const bool f = (pk & (ENT_FWD | ENT_INVALID)) == ENT_FWD;
        if (__ballot(f) != 0ull && f) {
            const int d = (int)((pk >> DIST_SHIFT) & 15u);
            const int p = (int)((pk >> POS_SHIFT) & 255u);
            pre = ring_at((t - d) % UR, p);
        }
        return pre;
    };

    // one token of a writer wavefront (barriers: [B'_t], B_t)
    auto write_token = [&](int t, int2 e, float2 ab, float4 pre, V4 vt) {
        const uint32_t pk = (uint32_t)e.x;
        const bool ok = (pk & ENT_INVALID) == 0u;
        const float w = __int_as_float(e.y);
        const float4 mt = f4_scale(ab.x, source(t, e, pre));
        float4 pred = mt;
        if constexpr (FORM == 1) {
            const float4 part = row_sum4<L>(f4_scale(ok ? w : 0.f, mt));
            if (r == 0) vbuf[wave * L + cc] = part;
            __syncthreads();
            pred = vbuf[cc];
#pragma unroll
            for (int q = 1; q < NWMAX; ++q)
                if (q < NWW) pred = f4_add(pred, vbuf[q * L + cc]);
        }
        const float4 nv = f4_fma(ab.y * w, f4_sub(VL::f(vt), pred), mt);
        float* dst = ok ? Mw + (((pk & ROW_MASK) * (uint32_t)dv + (uint32_t)col)) : sink;
        *reinterpret_cast<float4*>(dst) = nv;
        ring_at(t % UR, pos) = nv;
        __syncthreads();
    };
    // one token of a reader wavefront (barriers: [B'_t], B_t); the partial sums
    // of token t are combined by reader 0 after the next barrier
    auto read_token = [&](int t, int2 e, float4 pre) {
        if constexpr (FORM == 1) __syncthreads();
        __syncthreads();
        const uint32_t pk = (uint32_t)e.x;
        const float w = (pk & ENT_INVALID) == 0u ? __int_as_float(e.y) : 0.f;
        const float4 part = row_sum4<L>(f4_scale(w, source(t, e, pre)));
        if (r == 0) ybuf[((t & 1) * NWR + rw) * L + cc] = part;
        // every reader sums the previous token's partials; reader 0 stores the
        // result, the others (and token 0, which has no predecessor) hit the sink
        const int pb = (t - 1) & 1;
        float4 acc = ybuf[(pb * NWR) * L + cc];
#pragma unroll
        for (int q = 1; q < NWMAX; ++q)
            if (q < NWR) acc = f4_add(acc, ybuf[(pb * NWR + q) * L + cc]);
        float* dst = (rw == 0 && t > 0) ? ys + (int64_t)(t - 1) * dv : sink;
        *reinterpret_cast<float4*>(dst) = acc;
    };

    // Main loop: U tokens per trip, fully unrolled so that the register rings
    // are statically indexed. Each role gets its own prologue that issues the
    // steady-state sequence of loads (with a sink store standing in for each
    // token's store), so that the loop header merges like states and the
    // compiler's memory waits stay D tokens deep.
    int t_done = 0;
    if (T >= U) {
        int2 ent[U];
        float4 pre[UP];
        if (writer) {
            float2 ab[U];
            V4 vv[UP];
#pragma unroll
            for (int q = 0; q < D + DM; ++q) {
                ent[q] = load_entry(q);
                ab[q] = load_ab(q);
                if (q >= DM) {
                    pre[q - DM] = load_row(ent[q - DM]);
                    vv[q - DM] = VL::load(v, voff + (int64_t)(q - DM) * dv);
                }
                *reinterpret_cast<float4*>(sink) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            for (int t0 = 0; t0 + U <= T; t0 += U) {
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const int t = t0 + j;
                    const int tm = t + D + DM < T ? t + D + DM : T - 1;
                    ent[(j + D + DM) % U] = load_entry(tm);
                    ab[(j + D + DM) % U] = load_ab(tm);
                    const int tr = t + D < T ? t + D : T - 1;
                    pre[(j + D) % UP] = load_row(ent[(j + D) % U]);
                    vv[(j + D) % UP] = VL::load(v, voff + (int64_t)tr * dv);
                    write_token(t, ent[j], ab[j], pre[j % UP], vv[j % UP]);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < D + DM; ++q) {
                ent[q] = load_entry(q);
                if (q >= DM) pre[q - DM] = load_row(ent[q - DM]);
                *reinterpret_cast<float4*>(sink) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            for (int t0 = 0; t0 + U <= T; t0 += U) {
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const int t = t0 + j;
                    const int tm = t + D + DM < T ? t + D + DM : T - 1;
                    ent[(j + D + DM) % U] = load_entry(tm);
                    pre[(j + D) % UP] = load_row(ent[(j + D) % U]);
                    read_token(t, ent[j], pre[j % UP]);
                }
            }
        }
        t_done = (T / U) * U;
    }
    // tail (and short sequences): loads right before use; forwarding stays valid
    for (int t = t_done; t < T; ++t) {
        const int2 e = load_entry(t);
        const float4 pre = load_row(e);
        if (writer) write_token(t, e, load_ab(t), pre, VL::load(v, voff + (int64_t)t * dv));
        else read_token(t, e, pre);
    }
    // the last token's partial sums
    __syncthreads();
    if (!writer && rw == 0 && T > 0) {
        const int pb = (T - 1) & 1;
        float4 acc = ybuf[(pb * NWR) * L + cc];
        for (int q = 1; q < NWR; ++q) acc = f4_add(acc, ybuf[(pb * NWR + q) * L + cc]);
        *reinterpret_cast<float4*>(ys + (int64_t)(T - 1) * dv) = acc;
    }
}
// Ring reuse: the writer of token t overwrites slot t % UR, last used by token
// t - UR; its readers (tokens up to t - UR + D) have finished once every
// wavefront passed barrier B_{t-1}, which needs t - UR + D <= t - 2, so UR = D + 2.

template <int S>
size_t scan_lds_bytes(const Geom& g) {
    const int L = S / 4;
    return ((size_t)(SlabCfg<S>::D + 2) * g.NWW * g.G * L + 2 * g.NWR * L + g.NWW * L) * 16;
}

template <int S>
hipError_t launch_scan_slab(const ScanArgs& a, const Geom& g, hipStream_t st) {
    constexpr int D = SlabCfg<S>::D;
    static_assert(D <= 15, "the plan stores forward distances in 4 bits");
    // planner: tiles of TT tokens; the hash table holds the writes of TT + D tokens at load <= 1/2
    int TT = HT_CAP / (2 * a.W) - D;
    if (TT < 1) TT = 1;
    const int64_t ntile = (a.T + TT - 1) / TT;
    uint8_t* plan = static_cast<uint8_t*>(a.workspace);
    hipLaunchKernelGGL(plan_kernel, dim3((unsigned)(ntile * a.NS)), dim3(256), 0, st, a.idx_w, a.wt_w, a.W,
                       a.idx_r, a.wt_r, a.R, a.alpha, a.beta, plan, a.T, a.N, D, g.G, g.NWW, g.NWR, TT,
                       ntile);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nslab = a.dv / S;
    const int64_t nblk = ((a.NS + 7) / 8) * 8 * nslab;
    float* sink = reinterpret_cast<float*>(plan + a.NS * a.T * g.rec());
    const size_t lds = scan_lds_bytes<S>(g);
    dim3 grid((unsigned)nblk), block((unsigned)(g.nw() * 64));
#define SDM_LAUNCH(FORM, VB)                                                                          \
    hipLaunchKernelGGL((scan_kernel<S, FORM, VB>), grid, block, lds, st, plan, a.v, a.M, a.y, sink, \
                       (int)a.T, a.N, a.dv, nslab, a.NS, g.NWW, g.NWR)
    if (a.form == 0) {
        if (a.v_bf16) SDM_LAUNCH(0, true); else SDM_LAUNCH(0, false);
    } else {
        if (a.v_bf16) SDM_LAUNCH(1, true); else SDM_LAUNCH(1, false);
    }
#undef SDM_LAUNCH
    return hipGetLastError();
}

int slab_nwmax(int S) { return S == 32 ? SlabCfg<32>::NWMAX : SlabCfg<16>::NWMAX; }

// Slab width: SDM_SCAN_SLAB forces one. Otherwise, among the widths whose groups
// of G rows tile W and R without padding and that need at most 8 wavefronts
// (the 16-wavefront form has a shallower pipeline), the widest one that still
// gives at least 128 workgroups (half the CUs): wider slabs move longer row
// segments, narrower ones give more independent workgroups. Failing that, the
// width with the most workgroups, then the one with the least padding.
// (Measured on the N=65536, W=R=64, d_v=128 shapes: 32 streams -> 16 columns,
// 8 streams -> 8 columns.)
int pick_slab(int64_t NS, int W, int R, int dv) {
    int forced = 0;
    if (const char* e = getenv("SDM_SCAN_SLAB")) forced = atoi(e);
    struct Cand {
        int S;
        long waste, units;
        int nw;
    };
    auto better = [](const Cand& a, const Cand& b) {
        if ((a.waste == 0) != (b.waste == 0)) return a.waste == 0;
        if ((a.nw <= 8) != (b.nw <= 8)) return a.nw <= 8;
        const bool ea = a.units >= 128, eb = b.units >= 128;
        if (ea != eb) return ea;
        if (ea) return a.S > b.S;
        if (a.units != b.units) return a.units > b.units;
        return a.waste < b.waste;
    };
    Cand best{0, 0, 0, 0};
    for (int S : {32, 16, 8, 4}) {
        if (dv % S != 0 || (forced && forced != S)) continue;
        const Geom g = make_geom(S, W, R);
        if (g.nw() > slab_nwmax(S)) continue;
        const Cand c{S, (long)g.NWW * g.G - W + (long)g.NWR * g.G - R, (long)NS * (dv / S), g.nw()};
        if (best.S == 0 || better(c, best)) best = c;
    }
    return best.S;
}

}  // namespace

bool scan_geometry(int64_t NS, int W, int R, int dv, int* slab, int* rec) {
    const int S = pick_slab(NS, W, R, dv);
    if (S == 0) return false;
    if (slab) *slab = S;
    if (rec) *rec = (int)make_geom(S, W, R).rec();
    return true;
}

int64_t scan_workspace_bytes(int64_t NS, int64_t T, int W, int R, int dv) {
    int rec = 0, S = 0;
    if (!scan_geometry(NS, W, R, dv, &S, &rec)) return -1;
    const int64_t nblk = ((NS + 7) / 8) * 8 * (dv / S);
    return NS * T * rec + nblk * MAX_WAVES * 64 * 16;  // plan records + one 16-byte sink per thread
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    const int S = pick_slab(a.NS, a.W, a.R, a.dv);
    if (S == 0) return hipErrorInvalidValue;
    const Geom g = make_geom(S, a.W, a.R);
    switch (S) {
        case 32: return launch_scan_slab<32>(a, g, st);
        case 16: return launch_scan_slab<16>(a, g, st);
        case 8: return launch_scan_slab<8>(a, g, st);
        default: return launch_scan_slab<4>(a, g, st);
    }
}

}  // namespace sdm
