// scan_bwd.hip -- backward of the sparse gated delta scan on gfx950, undoing
// the forward's writes in place.
//
// What it computes ("Sparse Delta Memory：中文精读笔记" §2.9 Appendix A, backward
// memory: the forward writes the table in place, the backward recovers the
// earlier states by undoing the sparse updates; the recurrence differentiated is
// §2.4 Eq. (3)-(5) and the Fig. 2 reading of §2.5). Per (sequence, head), tokens
// t = T-1 .. 0, with M the table and G the adjoint table dL/dM (both given as
// they are after the call), write rows i_p with weights w_p and pre-images
// m_p = M_{t-1}[i_p] (stored by the training forward), read rows j_q with
// weights r_q, a = alpha_t, b = beta_t:
//   reads:   dr_q = <dy_t, M[j_q]>;  G[j_q] += r_q dy_t
//   writes, with g_p = G[i_p] after the reads:
//     EQ4:  u_p = v_t - a m_p;  dv_t = sum_p b w_p g_p;
//           dalpha_t = sum_p (1 - b w_p) <g_p, m_p>;  dbeta_t = sum_p w_p <g_p, u_p>;
//           dw_p = b <g_p, u_p>;  G[i_p] = a (1 - b w_p) g_p
//     FIG2: s = sum_p w_p m_p, u = v_t - a s, gh = sum_p w_p g_p;  dv_t = b gh;
//           dalpha_t = sum_p <g_p, m_p> - b <gh, s>;  dbeta_t = <gh, u>;
//           dw_p = b <g_p, u> - a b <gh, m_p>;  G[i_p] = a g_p - a b w_p gh
//   and M[i_p] = m_p (the undo).
// After token 0, M is the state before the call (bit for bit) and G = dL/dM there.
//
// Design. As in the forward, one workgroup owns one (stream, column slab of S
// floats): writer wavefronts hold the W write rows of a token (G rows each, one
// 16-byte segment per lane), reader wavefronts the R read rows. What no write
// changes (indices, weights, gates, v, dy, pre-images) is loaded one token
// ahead. The table rows (M and G of the reads, G of the writes) are loaded
// after the barrier that closes the previous token, so they see every earlier
// store of the workgroup (same CU) and nothing is forwarded across tokens.
// Within a token, readers and writers load at the same time; a write row that
// the token also reads takes the readers' new G value from LDS (the readers
// publish row -> read position in a small LDS hash table), so a token costs
// one memory round trip. The gradients of the weights and gates are column
// sums: each workgroup writes its slab's partial sums and a second kernel adds
// them over the slabs in slab order (deterministic).
//
// Row partitions (per-slot form). The per-slot write never couples two rows,
// so, as in the forward, the rows of a stream's table are split into P
// partitions by a hash of the row index and each partition is walked by its
// own workgroups: a token costs each of them the same round trip, and P times
// as many workgroups keep P times as many rows in flight. A workgroup takes the
// accesses of its partition and leaves the others' lanes idle (a wavefront
// with no access of its partition in a token skips it). dv_t and the gate
// gradients are then partial sums per partition, added in partition order.
#include "sdm_buffer.h"
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int BWD_NWMAX = 16;   // wavefronts per workgroup (1024 threads, 128 VGPRs)
#ifndef SDM_BWD_DEPTH
#define SDM_BWD_DEPTH 6
#endif
// tokens of streamed inputs in flight per wavefront (fp32 v takes two more
// registers per token, so its ring is shorter)
template <bool VBF16>
constexpr int ring_depth() { return VBF16 ? SDM_BWD_DEPTH : SDM_BWD_DEPTH - 2; }
constexpr int HS = 512;         // LDS hash slots per token parity: R <= 256 keeps the load <= 1/2
constexpr int HS_BITS = 9;

__device__ __forceinline__ int hslot(uint32_t row) { return (int)((row * 2654435761u) >> (32 - HS_BITS)); }

struct BwdKArgs {
    const int32_t* idx_w; const float* wt_w;
    const int32_t* idx_r; const float* wt_r;
    const float* alpha; const float* beta;
    const void* v; const float* snap; const float* dy;
    float* M; float* G; float* dvo;
    float* pw; float* pr;               // partial sums of this launch: [nslab][NS][T][W], [nslab][NS][T][R]
    float* pab;                         // [nslab * P][NS][T][2]
    float* pdv;                         // P > 1: [P][NS][T][dv]
    int64_t TS, t0;                     // tokens per stream; first token of this launch
    int T, W, R;
    int64_t N;
    int dv, nslab, P, pshift;
    int64_t NS;
    int NWW, NWR;
};

__device__ __forceinline__ int row_part(uint32_t row, int pshift) {
    return pshift == 0 ? 0 : (int)((row * 0x9E3779B1u) >> (32 - pshift));
}

template <int S, int FORM, bool VBF16>
__global__ __launch_bounds__(BWD_NWMAX * 64) void scan_backward_kernel(BwdKArgs a) {
    constexpr int L = S / 4, G = 64 / L;
    using VL = VLoad<VBF16>;
    using V4 = typename VL::T4;
    constexpr int DP = ring_depth<VBF16>();
    __shared__ int hkey[2][HS];                 // read rows of the token (parity t & 1), -1 = empty
    __shared__ int hpos[2][HS];                 // their read positions
    __shared__ float4 rg[BWD_NWMAX * 64];       // readers' new G segments [read position][L]
    __shared__ float4 xb[2][BWD_NWMAX][L];      // per writer wavefront: dv (EQ4) or gh and s (FIG2) partials
    __shared__ float ab[BWD_NWMAX][2];          // per writer wavefront: dalpha, dbeta partials

    const int NWW = a.NWW, T = a.T, dv = a.dv, W = a.W, R = a.R;
    // the wavefront index through readfirstlane: the compiler then knows it is
    // uniform, so role branches stay scalar (no per-lane descriptor loops)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, r = lane / L,
              cc = lane % L;
    // workgroups are dealt to the 8 XCDs round-robin: all slabs and partitions
    // of a stream go to the same XCD (they share its L2)
    const int b = blockIdx.x, xcd = b & 7, kq = b >> 3, units = a.nslab * a.P;
    const int64_t s = (int64_t)(kq / units) * 8 + xcd;
    const int slab = kq % a.nslab, part = (kq % units) / a.nslab;
    if (s >= a.NS) return;  // uniform over the workgroup
    const int col = slab * S + cc * 4;
    const bool writer = wave < NWW;
    const int rw = wave - NWW;
    const int pos = writer ? wave * G + r : rw * G + r;  // access position of this lane's row
    const int K = writer ? W : R;
    const bool has = pos < K;
    const int64_t tok0 = s * a.TS + a.t0;               // stream s's first token of this launch
    const int32_t* ix = (writer ? a.idx_w : a.idx_r) + tok0 * K;
    const float* wx = (writer ? a.wt_w : a.wt_r) + tok0 * K;
    const float* alp = a.alpha + tok0;
    const float* bep = a.beta + tok0;
    const rsrc_t Rm = make_rsrc(a.M + s * a.N * dv, a.N * dv * 4);
    const rsrc_t Rg = make_rsrc(a.G + s * a.N * dv, a.N * dv * 4);
    const rsrc_t Rv = make_rsrc(static_cast<const char*>(a.v) + tok0 * dv * VL::ESZ, (int64_t)T * dv * VL::ESZ);
    const rsrc_t Rd = make_rsrc(a.dy + tok0 * dv, (int64_t)T * dv * 4);
    const rsrc_t Rs = make_rsrc(a.snap + tok0 * W * dv, (int64_t)T * W * dv * 4);
    const rsrc_t Ro = a.P > 1 ? make_rsrc(a.pdv + ((int64_t)part * a.NS + s) * T * dv, (int64_t)T * dv * 4)
                              : make_rsrc(a.dvo + tok0 * dv, (int64_t)T * dv * 4);
    const uint32_t dv4 = (uint32_t)dv * 4u, col4 = (uint32_t)col * 4u;
    const uint32_t vstride = (uint32_t)dv * VL::ESZ, v_off = (uint32_t)col * VL::ESZ;
    const uint32_t sstride = (uint32_t)W * dv4;                  // pre-image bytes per token
    const uint32_t s_lane = has ? (uint32_t)pos * dv4 + col4 : OOB;
    const int64_t ps = (int64_t)slab * a.NS + s;
    float* pw = a.pw + ps * T * W;
    float* pr = a.pr + ps * T * R;
    float* pab = a.pab + ((int64_t)(slab * a.P + part) * a.NS + s) * T * 2;

    for (int i = threadIdx.x; i < 2 * HS; i += blockDim.x) (&hkey[0][0])[i] = -1;
    for (int i = threadIdx.x; i < 2 * BWD_NWMAX * L; i += blockDim.x)
        (&xb[0][0][0])[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    // the lane's access, if its row is valid and in this workgroup's partition
    auto off_of = [&](int32_t row) -> uint32_t {
        return (row >= 0 && row < a.N && row_part((uint32_t)row, a.pshift) == part)
                   ? __umul24((uint32_t)row, dv4) + col4 : OOB;
    };
    // partition 0 writes the (zero) weight gradients of positions whose row is out of range
    auto owns_pos = [&](int32_t row, uint32_t off) -> bool {
        return off != OOB || (part == 0 && has && !(row >= 0 && row < a.N));
    };
    // The inputs no write changes (index, weight, gates; v and the pre-image for
    // writers, dy for readers) come DP tokens ahead, from a register ring that
    // the unrolled loop indexes statically. A token first issues its table-row
    // loads, then the ring refill: the memory counters complete in order, so
    // waiting for the rows does not wait for the refill.
    struct In {
        int32_t row;
        float w, al, be;
        V4 v;
        float4 x;
    };
    auto fetch = [&](int tk) -> In {
        In d;
        const int64_t o = (int64_t)tk * K + pos;
        d.row = has ? ix[o] : -1;
        d.w = has ? wx[o] : 0.f;
        d.al = alp[tk];
        d.be = bep[tk];
        if (writer) {
            d.v = VL::load(Rv, v_off, (uint32_t)tk * vstride);
            d.x = ld_f4(Rs, s_lane, (uint32_t)tk * sstride);
        } else {
            d.v = V4{};
            d.x = ld_f4(Rd, col4, (uint32_t)tk * dv4);
        }
        return d;
    };
    In ring[DP];
#pragma unroll
    for (int j = 0; j < DP; ++j)
        if (T - 1 - j >= 0) ring[j] = fetch(T - 1 - j);
    int ins = -1;  // readers: the hash slot of this lane's row in the previous token's table

    // wavefront 0: token tk's dv (per-slot form: the writers' partial sums) and
    // gate partial sums. Called once the next token's row loads are issued, so
    // its LDS reads overlap them; the writers overwrite xb and ab only after
    // the next token's first barrier.
    auto finish = [&](int tk) {
        if constexpr (FORM == 0) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < BWD_NWMAX; ++q)  // xb of absent wavefronts holds zeros
                acc += reinterpret_cast<const float*>(xb[0][q])[lane < S ? lane : 0];
            st_f1(acc, Ro, lane < S ? (uint32_t)(slab * S + lane) * 4u : OOB, (uint32_t)tk * dv4);
        }
        const float sa = wave_sum(lane < NWW ? ab[lane][0] : 0.f), sb = wave_sum(lane < NWW ? ab[lane][1] : 0.f);
        if (lane == 0) {
            pab[2 * (int64_t)tk] = sa;
            pab[2 * (int64_t)tk + 1] = sb;
        }
    };

    for (int t0 = T - 1; t0 >= 0; t0 -= DP) {
#pragma unroll
    for (int j = 0; j < DP; ++j) {
        const int tl = t0 - j;
        if (tl < 0) break;  // uniform
        const In cur = ring[j];
        auto refill = [&]() {
            if (tl - DP >= 0) ring[j] = fetch(tl - DP);  // uniform
        };
        const int32_t row = cur.row;
        const uint32_t off = off_of(row);
        const float w = off == OOB ? 0.f : cur.w, al = cur.al, be = cur.be;
        const V4 vt = cur.v;
        const float4 xt = cur.x;
        const int tb = tl & 1;
        const bool run = __ballot(off != OOB) != 0ull;  // wavefront has an access of this partition
        if (writer) {
            float4 g = ld_f4(Rg, run ? off : OOB, 0u);  // after the barrier that closed token tl + 1
            refill();
            const float4 m = xt;                         // the pre-image M_{t-1}[i]
            if (wave == 0 && tl + 1 < T) finish(tl + 1);
            __syncthreads();                             // B1: the readers' new G values are in LDS
            if (off != OOB) {               // a row this token also reads: its G after the reads
                int h = hslot((uint32_t)row), k;
                while ((k = hkey[tb][h]) != -1) {
                    if (k == row) {
                        g = rg[hpos[tb][h] * L + cc];
                        break;
                    }
                    h = (h + 1) & (HS - 1);
                }
            }
            if constexpr (FORM == 0) {
                const float bw = be * w, c1 = 1.f - bw;
                const float4 u = f4_sub(VL::f(vt), f4_scale(al, m));
                const float part = rows_reduce<L>(f4_scale(bw, g));
                if ((lane & 15) < L) reinterpret_cast<float*>(xb[0][wave])[4 * (lane & 15) + (lane >> 4)] = part;
                float da = 0.f, db = 0.f;
                if (run) {  // uniform per wavefront
                    const float gm = dot4(g, m), gu = dot4(g, u);
                    const float gur = group_sum<L>(gu);
                    if (owns_pos(row, off) && cc == 0) pw[(int64_t)tl * W + pos] = off == OOB ? 0.f : be * gur;
                    da = wave_sum(c1 * gm);
                    db = wave_sum(w * gu);
                    st_f4(f4_scale(al * c1, g), Rg, off, 0u);
                } else if (owns_pos(row, off) && cc == 0) {
                    pw[(int64_t)tl * W + pos] = 0.f;
                }
                if (lane == 0) {
                    ab[wave][0] = da;
                    ab[wave][1] = db;
                }
            } else {
                const float pg = rows_reduce<L>(f4_scale(w, g)), pm = rows_reduce<L>(f4_scale(w, m));
                if ((lane & 15) < L) {
                    reinterpret_cast<float*>(xb[0][wave])[4 * (lane & 15) + (lane >> 4)] = pg;
                    reinterpret_cast<float*>(xb[1][wave])[4 * (lane & 15) + (lane >> 4)] = pm;
                }
                __syncthreads();  // BX: every writer's partial sums are in
                float4 gh = xb[0][0][cc], sm = xb[1][0][cc];
                for (int q = 1; q < NWW; ++q) {
                    gh = f4_add(gh, xb[0][q][cc]);
                    sm = f4_add(sm, xb[1][q][cc]);
                }
                const float4 u = f4_sub(VL::f(vt), f4_scale(al, sm));
                const float gm = dot4(g, m), gu = dot4(g, u), hm = dot4(gh, m);
                const float gur = group_sum<L>(gu), hmr = group_sum<L>(hm);
                if (owns_pos(row, off) && cc == 0)
                    pw[(int64_t)tl * W + pos] = off == OOB ? 0.f : be * gur - al * be * hmr;
                float xa = gm, xc = 0.f;
                if (wave == 0 && r == 0) {  // the per-slab terms, once
                    xa -= be * dot4(gh, sm);
                    xc = dot4(gh, u);
                    st_f4(f4_scale(be, gh), Ro, col4, (uint32_t)tl * dv4);  // dv_t = b gh
                }
                const float da = wave_sum(xa), db = wave_sum(xc);
                if (lane == 0) {
                    ab[wave][0] = da;
                    ab[wave][1] = db;
                }
                st_f4(f4_sub(f4_scale(al, g), f4_scale(al * be * w, gh)), Rg, off, 0u);
            }
            if (run) st_f4(m, Rm, off, 0u);  // the undo
            __syncthreads();                 // B2
        } else {
            if (ins >= 0) hkey[tb ^ 1][ins] = -1;  // the previous token's writers are done with it
            ins = -1;
            float4 m = make_float4(0.f, 0.f, 0.f, 0.f), g = m;
            if (run) {  // uniform per wavefront
                m = ld_f4(Rm, off, 0u);  // M_t: rows of later tokens are already undone
                g = ld_f4(Rg, off, 0u);
            }
            refill();
            if (run) {
                if (off != OOB && cc == 0) {  // publish the row while the loads are in flight
                    int h = hslot((uint32_t)row);
                    while (atomicCAS(&hkey[tb][h], -1, row) != -1) h = (h + 1) & (HS - 1);
                    hpos[tb][h] = pos;
                    ins = h;
                }
                const float dr = group_sum<L>(dot4(xt, m));
                const float4 gn = f4_fma(w, xt, g);
                st_f4(gn, Rg, off, 0u);
                rg[pos * L + cc] = gn;
                if (owns_pos(row, off) && cc == 0) pr[(int64_t)tl * R + pos] = off == OOB ? 0.f : dr;
            } else if (owns_pos(row, off) && cc == 0) {
                pr[(int64_t)tl * R + pos] = 0.f;
            }
            __syncthreads();                           // B1
            if constexpr (FORM == 1) __syncthreads();  // BX
            __syncthreads();                           // B2
        }
    }
    }
    if (wave == 0) finish(0);  // writers' last partial sums are complete since the last B2
}

// dwt_w, dwt_r, dalpha, dbeta of one launch: the slabs' partial sums added in
// slab order.
// With P > 1 row partitions, the gate gradients also add the partitions'
// partial sums (slab-major, then partition) and dv_t those of the partitions.
__global__ __launch_bounds__(256) void bwd_partials_reduce(const float* __restrict__ pw, const float* __restrict__ pr,
                                                           const float* __restrict__ pab,
                                                           const float* __restrict__ pdv, int nslab, int P,
                                                           int64_t NS, int64_t T, int W, int R, int dv, int64_t TS,
                                                           int64_t t0, float* dwt_w, float* dwt_r, float* dalpha,
                                                           float* dbeta, float* dv_out) {
    const int64_t nw = NS * T * W, nr = NS * T * R, na = NS * T * 2, nd = P > 1 ? NS * T * dv : 0;
    const int64_t n = nw + nr + na + nd;
    const int nab = nslab * P;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        if (i < nw) {
            float acc = pw[i];
            for (int k = 1; k < nslab; ++k) acc += pw[k * nw + i];
            const int64_t st = i / (T * W), rem = i - st * T * W;
            dwt_w[(st * TS + t0) * W + rem] = acc;
        } else if (i < nw + nr) {
            const int64_t j = i - nw;
            float acc = pr[j];
            for (int k = 1; k < nslab; ++k) acc += pr[k * nr + j];
            const int64_t st = j / (T * R), rem = j - st * T * R;
            dwt_r[(st * TS + t0) * R + rem] = acc;
        } else if (i < nw + nr + na) {
            const int64_t j = i - nw - nr;
            float acc = pab[j];
            for (int k = 1; k < nab; ++k) acc += pab[k * na + j];
            const int64_t st = j / (T * 2), rem = j - st * T * 2;
            (rem & 1 ? dbeta : dalpha)[st * TS + t0 + rem / 2] = acc;
        } else {
            const int64_t j = i - nw - nr - na;
            float acc = pdv[j];
            for (int q = 1; q < P; ++q) acc += pdv[q * nd + j];
            const int64_t st = j / (T * dv), rem = j - st * T * dv;
            dv_out[(st * TS + t0) * dv + rem] = acc;
        }
    }
}

struct BGeom {
    int S = 0, G = 0, NWW = 0, NWR = 0;
};
BGeom bwd_geom(int S, int W, int R) {
    BGeom g;
    g.S = S;
    g.G = 64 / (S / 4);
    g.NWW = (W + g.G - 1) / g.G;
    g.NWR = (R + g.G - 1) / g.G;
    return g;
}
bool bwd_fits(int S, int W, int R, int dv) {
    if (dv % S != 0) return false;
    const BGeom g = bwd_geom(S, W, R);
    return g.NWW + g.NWR <= BWD_NWMAX;
}

int env_int(const char* name) {
    const char* e = getenv(name);
    return e ? atoi(e) : 0;
}

constexpr int BWD_MAX_PARTS = 16;

// Slab width and row partitions. The per-slot form takes whole 128-byte lines
// (32-column slabs) and the smallest power-of-two P (<= 16) that gives 256
// workgroups (one per CU: a second workgroup on a CU stretches every token of
// both, measured); the shared-residual form, which cannot split rows,
// takes the widest slab that still gives 256 workgroups, else the one with the
// most. SDM_BWD_SLAB and SDM_BWD_PARTS force a choice.
struct BCfg {
    int S = 0, P = 1;
};
BCfg bwd_cfg(int64_t NS, int W, int R, int dv, int form) {
    BCfg c;
    const int fs = env_int("SDM_BWD_SLAB"), fp = env_int("SDM_BWD_PARTS");
    if (form == 0 && (fs == 0 || fs == 32) && fp != 1 && bwd_fits(32, W, R, dv)) {
        c.S = 32;
    } else {
        int64_t best_units = 0;
        for (int S : {32, 16, 8, 4}) {
            if ((fs && fs != S) || !bwd_fits(S, W, R, dv)) continue;
            const int64_t units = NS * (dv / S);
            if (c.S == 0 || (best_units < 256 && units > best_units)) {
                c.S = S;
                best_units = units;
            }
        }
        if (c.S == 0) return c;
    }
    if (form == 0) {
        if (fp == 1 || fp == 2 || fp == 4 || fp == 8 || fp == 16) {
            c.P = fp;
        } else {
            const int64_t units = (NS > 0 ? NS : 1) * (dv / c.S);
            while (c.P < BWD_MAX_PARTS && units * c.P < 256) c.P *= 2;
        }
    }
    return c;
}

int64_t bwd_chunk_tokens(int64_t T, int W, int dv) {
    const int64_t per_tok = (int64_t)(W > 1 ? W : 1) * dv * 4;
    const int64_t cap = (int64_t)0x7FFFFFFF / per_tok;
    return T < cap ? T : cap;
}

// Workspace of one launch of Tn tokens: pw, pr, pab, then (P > 1) pdv.
int64_t bwd_ws_floats(const BCfg& c, int64_t NS, int64_t Tn, int W, int R, int dv) {
    const int nslab = dv / c.S;
    return (int64_t)nslab * NS * Tn * (W + R) + (int64_t)nslab * c.P * NS * Tn * 2 +
           (c.P > 1 ? (int64_t)c.P * NS * Tn * dv : 0);
}

template <int S>
hipError_t launch_bwd_slab(const BwdArgs& a, const BCfg& c, hipStream_t st) {
    const BGeom g = bwd_geom(S, a.W, a.R);
    const int nslab = a.dv / S;
    const int64_t Tc = bwd_chunk_tokens(a.T, a.W, a.dv);
    float* pw = static_cast<float*>(a.workspace);
    int psh = 0;
    while ((1 << psh) < c.P) ++psh;
    const int64_t nblk = ((a.NS + 7) / 8) * 8 * nslab * c.P;
    const int esz = a.v_bf16 ? 2 : 4;
    const int64_t nchunk = (a.T + Tc - 1) / Tc;
    for (int64_t ci = nchunk - 1; ci >= 0; --ci) {  // the chunks in reverse
        const int64_t c0 = ci * Tc, Tn = a.T - c0 < Tc ? a.T - c0 : Tc;
        BwdKArgs k{};
        k.idx_w = a.idx_w; k.wt_w = a.wt_w; k.idx_r = a.idx_r; k.wt_r = a.wt_r;
        k.alpha = a.alpha; k.beta = a.beta;
        k.v = a.v; k.snap = a.snap; k.dy = a.dy;
        k.M = a.M; k.G = a.dM; k.dvo = a.dv_out;
        k.pw = pw;
        k.pr = pw + nslab * a.NS * Tn * a.W;
        k.pab = k.pr + nslab * a.NS * Tn * a.R;
        k.pdv = k.pab + (int64_t)nslab * c.P * a.NS * Tn * 2;
        k.TS = a.T; k.t0 = c0; k.T = (int)Tn; k.W = a.W; k.R = a.R;
        k.N = a.N; k.dv = a.dv; k.nslab = nslab; k.P = c.P; k.pshift = psh;
        k.NS = a.NS; k.NWW = g.NWW; k.NWR = g.NWR;
        (void)esz;
        dim3 grid((unsigned)nblk), block((unsigned)((g.NWW + g.NWR) * 64));
        const int sel = (a.form ? 2 : 0) | (a.v_bf16 ? 1 : 0);
        switch (sel) {
            case 0: hipLaunchKernelGGL((scan_backward_kernel<S, 0, false>), grid, block, 0, st, k); break;
            case 1: hipLaunchKernelGGL((scan_backward_kernel<S, 0, true>), grid, block, 0, st, k); break;
            case 2: hipLaunchKernelGGL((scan_backward_kernel<S, 1, false>), grid, block, 0, st, k); break;
            default: hipLaunchKernelGGL((scan_backward_kernel<S, 1, true>), grid, block, 0, st, k); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n = a.NS * Tn * (a.W + a.R + 2 + (c.P > 1 ? a.dv : 0));
        const int64_t nb = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
        hipLaunchKernelGGL(bwd_partials_reduce, dim3((unsigned)nb), dim3(256), 0, st, k.pw, k.pr, k.pab, k.pdv,
                           nslab, c.P, a.NS, Tn, a.W, a.R, a.dv, a.T, c0, a.dwt_w, a.dwt_r, a.dalpha, a.dbeta,
                           a.dv_out);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

bool scan_backward_geometry(int64_t NS, int W, int R, int dv) {
    return bwd_cfg(NS, W, R, dv, 0).S != 0 && bwd_cfg(NS, W, R, dv, 1).S != 0;
}

int64_t scan_backward_workspace_bytes(int64_t NS, int64_t T, int W, int R, int dv) {
    int64_t need = 0;
    for (int form = 0; form < 2; ++form) {
        const BCfg c = bwd_cfg(NS, W, R, dv, form);
        if (c.S == 0) return -1;
        const int64_t b = bwd_ws_floats(c, NS, bwd_chunk_tokens(T, W, dv), W, R, dv) * 4;
        if (b > need) need = b;
    }
    return need;
}

hipError_t launch_scan_backward(const BwdArgs& a, hipStream_t st) {
    const BCfg c = bwd_cfg(a.NS, a.W, a.R, a.dv, a.form);
    switch (c.S) {
        case 32: return launch_bwd_slab<32>(a, c, st);
        case 16: return launch_bwd_slab<16>(a, c, st);
        case 8: return launch_bwd_slab<8>(a, c, st);
        case 4: return launch_bwd_slab<4>(a, c, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdm
