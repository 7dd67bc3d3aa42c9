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
// 16-byte segment per lane), reader wavefronts the R read rows. Each token's
// loads (index words, weights, gates, v or dy, pre-images and the table rows)
// are issued D tokens before the token is processed, so the walk is not one
// memory round trip per token. A write whose row the same token reads adds
// that read's term itself, so the reads and writes of one token run side by
// side and one workgroup barrier per token (two for the shared-residual form)
// orders the walk. Rows that a token of that window will still
// change are not taken from memory: a planner kernel resolves, from the
// indices alone, where each access finds its row instead (the adjoint row from
// an LDS ring of the rows the nearest later toucher produced; a read's table
// row from the pre-image of the nearest later write). Every load and store in
// the token loop is a buffer access that every lane issues (out-of-range
// offsets where a lane has none), so the number of memory operations in flight
// is the same on every path and the compiler's counter waits drain only the
// token being consumed. The gradients of the weights and gates are column
// sums: each workgroup writes its slab's partial sums and a second kernel adds
// them over the slabs in slab order (deterministic).
//
// Row partitions (per-slot form). The per-slot write never couples
// two rows, so the rows of a stream's table can be split into P partitions by a
// hash of the row index, each walked by its own workgroups, which take the
// accesses of their partition and leave the other lanes idle. dv_t and the
// gate gradients are then partial sums per partition, added in partition order.
#include "sdm_buffer.h"
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int BWD_NWMAX = 16;   // wavefronts per workgroup (1024 threads, 128 VGPRs)

struct BwdKArgs {
    const int32_t* idx_w; const float* wt_w;
    const int32_t* idx_r; const float* wt_r;
    const float* alpha; const float* beta;
    const void* v; const float* snap; const float* dy;
    float* M; float* G; float* dvo;
    float* pw; float* pr;               // partial sums of this launch: [nslab][NS][T][W], [nslab][NS][T][R]
    float* pab;                         // [nslab * P][NS][T][2]
    float* pdv;                         // P > 1: [P][NS][T][dv]
    const uint32_t* plan;               // [NS][T][W + 2R] source words of this launch (bwd_plan_kernel)
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

// ------------------------------------------------------------------ planner
// The reverse walk issues a token's table-row loads D tokens before the
// token is processed (processing runs t = T-1 .. 0), so a load of token u does
// not see what tokens u+1 .. u+D will store. All indices are known, so for
// every access of token u a planner finds, from the indices alone:
//   G source: the token of (u, u+D] nearest to u that touches the row; the
//     row's adjoint after that token (its writer's new G if it writes the row,
//     else its reader's) comes from an LDS ring.
//   Same-token pairs: a write whose row the same token also reads adds that
//     read's r_q dy_u itself (the read position q is in its word), and that
//     read's new G is marked superseded (the write's replaces it), so the
//     reads and writes of one token need no ordering between them.
//   M source (reads): the token of (u, u+D+1] nearest to u that writes the
//     row; the row's state after token u is that write's pre-image, read from
//     the forward's stored pre-images (which nothing modifies) instead of the
//     table. (The walk stores a token's undo one token late, so that a read of
//     the same token has taken the row before it changes; the window is one
//     token longer for that.)
// Without a source in the window, the table in memory is already right.
// Word layout: bit 31 = from the ring / from the pre-images, bits 9-11 =
// distance d, bits 0-8 = source position (writer p < W, reader W + q); G words
// also: bit 30 = a write the same token reads (read position in bits 12-19),
// bit 29 = a read the same token writes.
constexpr uint32_t BSRC_ON = 1u << 31;
constexpr uint32_t BSRC_OWN = 1u << 30;
constexpr uint32_t BSRC_DEAD = 1u << 29;
constexpr int BSRC_DSHIFT = 9;
constexpr int BSRC_QSHIFT = 12;
constexpr uint32_t BSRC_POS = 511u;
constexpr int BHT_BITS = 13;
constexpr int BHT_CAP = 1 << BHT_BITS;     // 64-bit LDS hash entries (64 KiB)
constexpr uint64_t BHT_EMPTY = ~0ull;
constexpr int BPLAN_THREADS = 512;

struct BPlanArgs {
    const int32_t* idx_w; const int32_t* idx_r;   // the launch's first token of stream 0; stream stride TS
    uint32_t* plan;                               // [NS][Tn][W + 2R]
    int64_t Tn, TS, N;
    int W, R, D, TT;
    int64_t ntile;
};

__device__ __forceinline__ uint32_t bht_hash(uint32_t row) { return (row * 2654435761u) >> (32 - BHT_BITS); }

// One workgroup per (stream, tile of TT tokens [u0, u1)): an LDS hash holds every
// access of tokens [u0, u1 + D + 1) as (row << 32 | token - u0 << 10 | is_write << 9 |
// position), at most a quarter full; each access of the tile then walks its row's
// entries and keeps the nearest later touch and write.
__global__ __launch_bounds__(BPLAN_THREADS) void bwd_plan_kernel(BPlanArgs a) {
    __shared__ uint64_t ht[BHT_CAP];
    const int tid = threadIdx.x;
    const int W = a.W, R = a.R, D = a.D, K = W + R, RW = W + 2 * R;
    const int64_t s = blockIdx.x / a.ntile;
    const int64_t u0 = (blockIdx.x % a.ntile) * a.TT;
    const int64_t u1 = u0 + a.TT < a.Tn ? u0 + a.TT : a.Tn;
    const int64_t h1 = u1 + D + 1 < a.Tn ? u1 + D + 1 : a.Tn;
    const int32_t* iw = a.idx_w + s * a.TS * W;
    const int32_t* ir = a.idx_r + s * a.TS * R;
    uint32_t* Ps = a.plan + s * a.Tn * RW;
    for (int i = tid; i < BHT_CAP; i += BPLAN_THREADS) ht[i] = BHT_EMPTY;
    __syncthreads();
    const int n1 = (int)(h1 - u0) * K;
    for (int e = tid; e < n1; e += BPLAN_THREADS) {
        const int tk = e / K, pos = e - tk * K;
        const bool isw = pos < W;
        const int q = isw ? pos : pos - W;
        const int32_t row = isw ? iw[(u0 + tk) * W + q] : ir[(u0 + tk) * R + q];
        if (row < 0 || row >= a.N) continue;
        const uint64_t ent = ((uint64_t)(uint32_t)row << 32) | ((uint64_t)tk << 10) | ((uint64_t)isw << 9) |
                             (uint64_t)q;
        uint32_t h = bht_hash((uint32_t)row);
        while (atomicCAS((unsigned long long*)&ht[h], (unsigned long long)BHT_EMPTY, (unsigned long long)ent) !=
               (unsigned long long)BHT_EMPTY)
            h = (h + 1) & (BHT_CAP - 1);
    }
    __syncthreads();
    const int n2 = (int)(u1 - u0) * K;
    for (int e = tid; e < n2; e += BPLAN_THREADS) {
        const int tk = e / K, pos = e - tk * K;
        const bool isw = pos < W;
        const int q = isw ? pos : pos - W;
        const int32_t row = isw ? iw[(u0 + tk) * W + q] : ir[(u0 + tk) * R + q];
        uint32_t gs = 0u, ms = 0u;
        if (row >= 0 && row < a.N) {
            int gd = D + 1, md = D + 2;
            bool gw = false, own = false, dead = false;
            uint32_t gp = 0u, mp = 0u, op = 0u;
            uint32_t h = bht_hash((uint32_t)row);
            uint64_t ent;
            while ((ent = ht[h]) != BHT_EMPTY) {
                if ((uint32_t)(ent >> 32) == (uint32_t)row) {
                    const int d = (int)((ent >> 10) & 1023u) - tk;
                    const bool ew = (ent >> 9) & 1u;
                    const uint32_t ep = (uint32_t)(ent & 511u);
                    if (d == 0 && isw && !ew) {
                        own = true;
                        op = ep;
                    }
                    if (d == 0 && !isw && ew) dead = true;
                    if (d >= 1 && d <= D && (d < gd || (d == gd && ew && !gw))) {
                        gd = d;
                        gw = ew;
                        gp = ew ? ep : (uint32_t)W + ep;
                    }
                    if (d >= 1 && d <= D + 1 && ew && d < md) {
                        md = d;
                        mp = ep;
                    }
                }
                h = (h + 1) & (BHT_CAP - 1);
            }
            if (gd <= D) gs = BSRC_ON | ((uint32_t)gd << BSRC_DSHIFT) | gp;
            if (own) gs |= BSRC_OWN | (op << BSRC_QSHIFT);
            if (dead) gs |= BSRC_DEAD;
            if (!isw && md <= D + 1) ms = BSRC_ON | ((uint32_t)md << BSRC_DSHIFT) | mp;
        }
        uint32_t* rec = Ps + (u0 + tk) * RW;
        if (isw) {
            rec[q] = gs;
        } else {
            rec[W + q] = gs;
            rec[W + R + q] = ms;
        }
    }
}

// ------------------------------------------------------------------ reverse walk
// The backward of the header with each token's rows loaded D tokens early.
// Per token, in the reverse walk: address words (index and the planner's source words)
// come D + DM tokens early; values (weight, gates, v or dy, pre-image) and
// table rows (G of every access, M of the reads, or the pre-image a read's M
// comes from) D tokens early, issued right after the barrier that closed the
// previous token. Every token leaves the adjoint rows it produced (writers' and
// readers' new G) in an LDS ring of D + 1 token slots [slot][W + R][L], where
// later-processed tokens of the window find them after the token's barrier.
// Two instantiations: up to 16 wavefronts per workgroup (128 VGPRs) with
// D = 1, which the layouts of more than 8 wavefronts take (32 streams of 8192
// tokens, W = R = 64, d_v = 128: 32-column slabs), and up to 8 wavefronts (256
// VGPRs) with D = 4, which every layout of at most 8 wavefronts takes. With 16
// wavefronts D = 2 fits 128 VGPRs but runs slower (that shape: 16.2 against
// 15.1 ms; D = 3 spills). With 8 wavefronts, D = 4 against D = 2 took one
// stream of 65536 tokens (W = R = 8, d_v = 512) from 75 to 65 ms and 16
// streams of 4096 tokens from 4.8 to 4.2 ms; D = 6 is slower on the first (58.9
// against 30.6 ms) and no faster on the others.
constexpr int BWD_D = 1;
constexpr int BWD_D_DEEP = 4;
constexpr int BWD_NW_DEEP = 8;
static_assert(BWD_D_DEEP + 1 <= 7, "plan words keep the distance in 3 bits");

template <bool B>
struct BRole {
    static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t ld_u1(rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, (int)so, 0);
}

template <int S, int FORM, bool VBF16, int D, int NWM>
__global__ __launch_bounds__(NWM * 64) void scan_backward_kernel(BwdKArgs a) {
    constexpr int L = S / 4, G = 64 / L;
    using VL = VLoad<VBF16>;
    using V4 = typename VL::T4;
    constexpr int DM = D + 1;
    constexpr int UP = D + 1;          // value/row ring
    constexpr int U = D + DM + 1;      // address ring = unroll factor (a multiple of UP)
    static_assert(U % UP == 0, "ring sizes");
    constexpr int UR = D + 1;          // LDS ring slots
    extern __shared__ float4 lring[];  // [UR][W + R][L]
    // per-slot form: each writer's dv partial, by token parity; shared-residual
    // form: the writers' partials of gh (0) and s (1) within a token
    __shared__ float4 xb[2][NWM][L];
    __shared__ float ab[2][NWM][2][64];  // each writer lane's gate-gradient terms, by token parity

    const int NWW = a.NWW, T = a.T, dv = a.dv, W = a.W, R = a.R, KR = W + R, RW = W + 2 * R;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, r = lane / L,
              cc = lane % L;
    int64_t s;
    int kq;
    block_unit(blockIdx.x, a.NS, a.nslab * a.P, s, kq);
    const int slab = kq % a.nslab, part = kq / a.nslab;
    if (s >= a.NS) return;  // uniform over the workgroup
    const int col = slab * S + cc * 4;
    const bool writer = wave < NWW;
    const int rw = wave - NWW;
    const int pos = writer ? wave * G + r : rw * G + r;
    const int K = writer ? W : R;
    const bool has = pos < K;
    const int64_t tok0 = s * a.TS + a.t0;
    const int32_t* ix = (writer ? a.idx_w : a.idx_r) + tok0 * K;
    const float* wx = (writer ? a.wt_w : a.wt_r) + tok0 * K;
    const float* alp = a.alpha + tok0;
    const float* bep = a.beta + tok0;
    const uint32_t* pl = a.plan + s * (int64_t)T * RW;
    const int pg_off = writer ? pos : W + pos;    // this lane's G-source word in a token record
    const uint32_t dv4 = (uint32_t)dv * 4u, col4 = (uint32_t)col * 4u;
    const uint32_t vstride = (uint32_t)dv * VL::ESZ, v_off = (uint32_t)col * VL::ESZ;
    const uint32_t sstride = (uint32_t)W * dv4;
    const uint32_t s_lane = has ? (uint32_t)pos * dv4 + col4 : OOB;
    const int64_t ps = (int64_t)slab * a.NS + s;
    float* pw = a.pw + ps * T * W;
    float* pr = a.pr + ps * T * R;
    float* pab = a.pab + ((int64_t)(slab * a.P + part) * a.NS + s) * T * 2;

    for (int i = threadIdx.x; i < 2 * NWM * L; i += blockDim.x)
        (&xb[0][0][0])[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    const uint32_t N32 = (uint32_t)(a.N < 0x7FFFFFFF ? a.N : 0x7FFFFFFF);
    auto off_of = [&](int32_t row) -> uint32_t {
        return ((uint32_t)row < N32 && row_part((uint32_t)row, a.pshift) == part) ? __umul24((uint32_t)row, dv4) + col4
                                                                                   : OOB;
    };
    auto owns_pos = [&](int32_t row, uint32_t off) -> bool {
        return off != OOB || (part == 0 && has && !((uint32_t)row < N32));
    };
    auto ring_at = [&](int slot, int p) -> float4& { return lring[(slot * KR + p) * L + cc]; };

    // Buffer descriptors are made in each role's own path (and the finishing
    // sums' in theirs), so that scalar registers hold only one role's set.
    auto make_ro = [&]() {
        return a.P > 1 ? make_rsrc(a.pdv + ((int64_t)part * a.NS + s) * T * dv, (int64_t)T * dv * 4)
                       : make_rsrc(a.dvo + tok0 * dv, (int64_t)T * dv * 4);
    };
    struct BD {
        rsrc_t ix, wx, pl, g, m, s, d, v, al, be, wr, pw, pr, o;
    };
    auto make_desc = [&](auto wr_c) -> BD {
        constexpr bool WR = decltype(wr_c)::value;
        BD d;
        d.ix = make_rsrc(ix, (int64_t)T * K * 4);
        d.wx = make_rsrc(wx, (int64_t)T * K * 4);
        d.pl = make_rsrc(pl, (int64_t)T * RW * 4);
        d.g = make_rsrc(a.G + s * a.N * dv, a.N * dv * 4);
        d.m = make_rsrc(a.M + s * a.N * dv, a.N * dv * 4);
        d.s = make_rsrc(a.snap + tok0 * W * dv, (int64_t)T * W * dv * 4);
        d.d = make_rsrc(a.dy + tok0 * dv, (int64_t)T * dv * 4);
        if constexpr (WR) {
            d.v = make_rsrc(static_cast<const char*>(a.v) + tok0 * dv * VL::ESZ, (int64_t)T * dv * VL::ESZ);
            d.al = make_rsrc(alp, (int64_t)T * 4);
            d.be = make_rsrc(bep, (int64_t)T * 4);
            d.wr = make_rsrc(a.wt_r + tok0 * R, (int64_t)T * R * 4);  // same-token read weights
            d.pw = make_rsrc(pw, (int64_t)T * W * 4);
            if constexpr (FORM == 1) d.o = make_ro();
        } else {
            d.pr = make_rsrc(pr, (int64_t)T * R * 4);
        }
        return d;
    };
    const uint32_t lane_k = has ? (uint32_t)pos * 4u : OOB;
    const uint32_t lane_pg = has ? (uint32_t)pg_off * 4u : OOB;
    const uint32_t lane_pm = (has && !writer) ? (uint32_t)(W + R + pos) * 4u : OOB;

    struct Ad {
        int32_t row;
        uint32_t gs, ms;
    };
    struct Va {
        float w, al, be;
        float4 x;   // writers: the pre-image of the write; readers: dy
        float4 g;   // the adjoint row (unless it comes from the ring)
        float4 y;   // writers: v_t (its raw bits); readers: M_t of the row (table or pre-image)
        float4 dy;  // writers: dy_t
        float wr;   // writers: the weight of this token's read of the row (0 if none)
        uint32_t off;  // the row's byte offset in the tables (OOB if none here)
    };
    auto v_of = [&](const float4& y) -> V4 {
        if constexpr (VBF16) return make_int2(__float_as_int(y.x), __float_as_int(y.y));
        else return y;
    };
    // Each role (WR: writer wavefronts) issues only the loads it uses, the same
    // ones for every token, so the loads in flight per token are the same on
    // every path of that role's loop (a lane without the access gets an
    // out-of-range offset).
    auto fetch_ad = [&](auto wr_c, const BD& D_, int tk) -> Ad {
        constexpr bool WR = decltype(wr_c)::value;
        Ad d;
        const int32_t row = (int32_t)ld_u1(D_.ix, lane_k, (uint32_t)tk * (uint32_t)K * 4u);
        d.row = has ? row : -1;
        d.gs = ld_u1(D_.pl, lane_pg, (uint32_t)tk * (uint32_t)RW * 4u);
        if constexpr (WR) d.ms = 0u;
        else d.ms = ld_u1(D_.pl, lane_pm, (uint32_t)tk * (uint32_t)RW * 4u);
        return d;
    };
    auto fetch_va = [&](auto wr_c, const BD& D_, int tk, const Ad& d) -> Va {
        constexpr bool WR = decltype(wr_c)::value;
        Va x;
        const uint32_t off = off_of(d.row);
        x.off = off;
        x.w = __uint_as_float(ld_u1(D_.wx, lane_k, (uint32_t)tk * (uint32_t)K * 4u));
        x.g = ld_f4(D_.g, (d.gs & BSRC_ON) ? OOB : off, 0u);
        if constexpr (WR) {
            x.al = __uint_as_float(ld_u1(D_.al, 0u, (uint32_t)tk * 4u));
            x.be = __uint_as_float(ld_u1(D_.be, 0u, (uint32_t)tk * 4u));
            const uint32_t oq = (d.gs >> BSRC_QSHIFT) & 255u;
            x.wr = __uint_as_float(ld_u1(D_.wr, (d.gs & BSRC_OWN) && off != OOB ? oq * 4u : OOB,
                                         (uint32_t)tk * (uint32_t)R * 4u));
            x.dy = ld_f4(D_.d, col4, (uint32_t)tk * dv4);
            const V4 vv = VL::load(D_.v, v_off, (uint32_t)tk * vstride);
            x.x = ld_f4(D_.s, s_lane, (uint32_t)tk * sstride);
            if constexpr (VBF16) x.y = make_float4(__int_as_float(vv.x), __int_as_float(vv.y), 0.f, 0.f);
            else x.y = vv;
        } else {
            x.al = 0.f;
            x.be = 0.f;
            x.wr = 0.f;
            x.dy = make_float4(0.f, 0.f, 0.f, 0.f);
            x.x = ld_f4(D_.d, col4, (uint32_t)tk * dv4);
            // a read's M_t: from the table, or from a later write's pre-image (the
            // other load's offset is out of range: it is dropped)
            const bool from_pre = (d.ms & BSRC_ON) && off != OOB;
            const uint32_t dd = (d.ms >> BSRC_DSHIFT) & 7u, sp = d.ms & BSRC_POS;
            const float4 mt = ld_f4(D_.m, from_pre ? OOB : off, 0u);
            const float4 mp = ld_f4(D_.s, from_pre ? __umul24(dd, sstride) + __umul24(sp, dv4) + col4 : OOB,
                                    (uint32_t)tk * sstride);
            x.y = from_pre ? mp : mt;
        }
        return x;
    };

    // the first reader wavefront, while the writers work on the next token: token
    // tk's dv (per-slot form) and gate-gradient sums over the writers' partials
    // (kept by token parity, so the next token's writers do not overwrite them)
    auto finish = [&](int tk) {
        const int par = tk & 1;
        const rsrc_t Ro = make_ro(), Rpab = make_rsrc(pab, (int64_t)T * 8);
        if constexpr (FORM == 0) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < NWM; ++q)
                acc += reinterpret_cast<const float*>(xb[par][q])[lane < S ? lane : 0];
            st_f1(acc, Ro, lane < S ? (uint32_t)(slab * S + lane) * 4u : OOB, (uint32_t)tk * dv4);
        }
        float pa = 0.f, pb = 0.f;
        for (int q = 0; q < NWW; ++q) {
            pa += ab[par][q][0][lane];
            pb += ab[par][q][1][lane];
        }
        const float sa = wave_sum(pa), sb = wave_sum(pb);
        st_f1(lane == 0 ? sa : sb, Rpab, lane < 2 ? (uint32_t)lane * 4u : OOB, (uint32_t)tk * 8u);
    };

    // a wavefront the launch adds beyond the writers and readers (when the
    // layout leaves room) does nothing but the finishing sums, off the readers'
    // path; it keeps the barrier count of the others
    const bool xf = (int)(blockDim.x >> 6) > NWW + a.NWR;
    if (wave == NWW + a.NWR) {
        for (int tl = T - 1; tl >= 0; --tl) {
            if constexpr (FORM == 1) __syncthreads();  // BX
            if (tl + 1 < T) finish(tl + 1);
            __syncthreads();                           // B
        }
        finish(0);
        return;
    }

    int slot = (T - 1) % UR;  // LDS ring slot of the token being processed
    // a writer's undo, stored one token late: this token's reads of the row
    // (other wavefronts, loads issued tokens ago) have taken it by then
    float4 undo_m = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t undo_off = OOB;
    auto process = [&](auto wr_c, const BD& D_, int tl, const Ad& d, const Va& x) {
        constexpr bool WR = decltype(wr_c)::value;
        const int32_t row = d.row;
        const uint32_t off = x.off;
        const float w = off == OOB ? 0.f : x.w, al = x.al, be = x.be;
        const bool run = __ballot(off != OOB) != 0ull;  // else every lane's offset is out of range
        const bool fwd = (d.gs & BSRC_ON) && off != OOB;
        int fslot = slot + (int)((d.gs >> BSRC_DSHIFT) & 7u);
        if (fslot >= UR) fslot -= UR;
        const int fpos = (int)(d.gs & BSRC_POS);
        const bool own = owns_pos(row, off) && cc == 0;
        if constexpr (WR) {
            const float4 m = x.x;  // the pre-image M_{t-1}[i]
            const int par = tl & 1;
            st_f4(undo_m, D_.m, undo_off, 0u);  // the previous token's undo
            undo_m = m;
            undo_off = off;
            float4 g = x.g;
            if (fwd) g = ring_at(fslot, fpos);
            g = f4_fma(x.wr, x.dy, g);  // G after this token's reads
            float4 gn = make_float4(0.f, 0.f, 0.f, 0.f);
            float pwv = 0.f;
            if constexpr (FORM == 0) {
                const float bw = be * w, c1 = 1.f - bw;
                const float4 u = f4_sub(VL::f(v_of(x.y)), f4_scale(al, m));
                const float part = rows_reduce<L>(f4_scale(bw, g));
                if ((lane & 15) < L) reinterpret_cast<float*>(xb[par][wave])[4 * (lane & 15) + (lane >> 4)] = part;
                float da = 0.f, db = 0.f;  // this lane's terms; the finishing wavefront sums them
                if (run) {
                    const float gm = dot4(g, m), gu = dot4(g, u);
                    const float gur = group_sum<L>(gu);
                    pwv = off == OOB ? 0.f : be * gur;
                    da = c1 * gm;
                    db = w * gu;
                    gn = f4_scale(al * c1, g);
                    if (off != OOB) ring_at(slot, pos) = gn;
                }
                ab[par][wave][0][lane] = da;
                ab[par][wave][1][lane] = db;
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
                const float4 u = f4_sub(VL::f(v_of(x.y)), f4_scale(al, sm));
                const float gm = dot4(g, m), gu = dot4(g, u), hm = dot4(gh, m);
                const float gur = group_sum<L>(gu), hmr = group_sum<L>(hm);
                pwv = off == OOB ? 0.f : be * gur - al * be * hmr;
                const bool lead = wave == 0 && r == 0;
                const float xa = lead ? gm - be * dot4(gh, sm) : gm, xc = lead ? dot4(gh, u) : 0.f;
                st_f4(f4_scale(be, gh), D_.o, lead ? col4 : OOB, (uint32_t)tl * dv4);
                ab[par][wave][0][lane] = xa;  // summed by the finishing wavefront
                ab[par][wave][1][lane] = xc;
                gn = f4_sub(f4_scale(al, g), f4_scale(al * be * w, gh));
                if (off != OOB) ring_at(slot, pos) = gn;
            }
            st_f1(pwv, D_.pw, own ? (uint32_t)pos * 4u : OOB, (uint32_t)tl * (uint32_t)W * 4u);
            st_f4(gn, D_.g, off, 0u);
            __syncthreads();  // B: this token's new G rows are in the ring
        } else {
            float4 gn = make_float4(0.f, 0.f, 0.f, 0.f);
            float dr = 0.f;
            if (run) {
                float4 g = x.g;
                if (fwd) g = ring_at(fslot, fpos);
                dr = group_sum<L>(dot4(x.x, x.y));
                gn = f4_fma(w, x.x, g);
                if (off != OOB) ring_at(slot, W + pos) = gn;
            }
            st_f4(gn, D_.g, (d.gs & BSRC_DEAD) ? OOB : off, 0u);  // a same-token write replaces it
            st_f1(off == OOB ? 0.f : dr, D_.pr, own ? (uint32_t)pos * 4u : OOB, (uint32_t)tl * (uint32_t)R * 4u);
            if constexpr (FORM == 1) __syncthreads();  // BX
            if (rw == 0 && !xf && tl + 1 < T) finish(tl + 1);
            __syncthreads();                           // B
        }
        slot = slot == 0 ? UR - 1 : slot - 1;
    };

    // Main loop: U tokens per trip, fully unrolled so the register rings are
    // statically indexed; the token being processed is tl = T - 1 - k. Each role
    // runs its own copy.
    auto run = [&](auto wr_c) {
        constexpr bool WR = decltype(wr_c)::value;
        const BD R_ = make_desc(wr_c);
        int k_done = 0;
        if (T >= U) {
            Ad ad[U];
            Va va[UP];
#pragma unroll
            for (int q = 0; q < D + DM; ++q) ad[q] = fetch_ad(wr_c, R_, T - 1 - q);
#pragma unroll
            for (int q = 0; q < D; ++q) va[q] = fetch_va(wr_c, R_, T - 1 - q, ad[q]);
            for (int k0 = 0; k0 + U <= T; k0 += U) {
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const int tl = T - 1 - (k0 + j);
                    // early loads of tokens before 0 fetch token 0 again, unused
                    ad[(j + D + DM) % U] = fetch_ad(wr_c, R_, tl - D - DM >= 0 ? tl - D - DM : 0);
                    va[(j + D) % UP] = fetch_va(wr_c, R_, tl - D >= 0 ? tl - D : 0, ad[(j + D) % U]);
                    process(wr_c, R_, tl, ad[j], va[j % UP]);
                }
            }
            k_done = (T / U) * U;
        }
        for (int k = k_done; k < T; ++k) {  // the rest: loads right before use
            const int tl = T - 1 - k;
            const Ad d = fetch_ad(wr_c, R_, tl);
            process(wr_c, R_, tl, d, fetch_va(wr_c, R_, tl, d));
        }
        if constexpr (WR) st_f4(undo_m, R_.m, undo_off, 0u);  // token 0's undo
    };
    if (writer) run(BRole<true>{});
    else run(BRole<false>{});
    if (wave == NWW && !xf) finish(0);
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
// LDS of the reverse walk: the ring of D + 1 token slots of W + R rows.
size_t bwd_ring_bytes(int S, int W, int R, int D) {
    return (size_t)(D + 1) * (W + R) * (S / 4) * 16;
}

bool bwd_fits(int S, int W, int R, int dv) {
    // (a token's pre-images span W * dv * 4 bytes, multiplied in 24 bits)
    if (dv % S != 0 || (int64_t)W * dv * 4 >= (1 << 24)) return false;
    const BGeom g = bwd_geom(S, W, R);
    return g.NWW + g.NWR <= BWD_NWMAX && bwd_ring_bytes(S, W, R, BWD_D) <= 128 * 1024;
}

// The deeper instantiation: at most 8 wavefronts and its ring within 128 KiB.
bool bwd_deep(int S, int W, int R) {
    const BGeom g = bwd_geom(S, W, R);
    return g.NWW + g.NWR <= BWD_NW_DEEP && bwd_ring_bytes(S, W, R, BWD_D_DEEP) <= 128 * 1024;
}

int env_int(const char* name) {
    const char* e = getenv(name);
    return e ? atoi(e) : 0;
}

// Slab width and row partitions. The per-slot form takes the widest slab that
// fills the CUs (256 workgroups) in one row partition, or in two where the
// layout has two or more writer wavefronts. Every workgroup of a partition
// steps through every token, so more partitions cost more than they bring (8
// streams of 131072 tokens, 8-column slabs in 2 / 4 partitions: 112.8 / 162
// ms), while wider slabs pay off because a random row piece costs the DRAM a
// whole 128-byte line (32 streams of 8192 tokens: 32-column slabs in 2
// partitions 15.1 ms against 16.5 for 16-column slabs in one; 16 streams of
// 4096 tokens, W = R = 16, d_v = 64: 4-column slabs 2.01 ms against 2.13 for
// 8-column ones on half the CUs). Where no layout fills the CUs that way, and
// for the shared-residual form (no partitions): the widest slab whose layout
// has at most 8 wavefronts (the deeper window) and gives at least 128
// workgroups, else the widest that still gives 256, else the one with the
// most; the per-slot form then takes 2 partitions where half the CUs would
// idle and the layout has two or more writer wavefronts. SDM_BWD_SLAB and
// SDM_BWD_PARTS (per-slot form only) force a choice.
struct BCfg {
    int S = 0, P = 1;
};
BCfg bwd_cfg(int64_t NS, int W, int R, int dv, int form) {
    BCfg c;
    const int fs = env_int("SDM_BWD_SLAB"), fp = env_int("SDM_BWD_PARTS");
    if (form == 0 && !fs && !fp) {  // 256 workgroups with the widest slab
        for (int S : {32, 16, 8, 4}) {
            if (!bwd_fits(S, W, R, dv)) continue;
            const int64_t units = NS * (dv / S);
            const int P = units >= 256 ? 1 : (bwd_geom(S, W, R).NWW >= 2 && units * 2 >= 256) ? 2 : 0;
            if (P) {
                c.S = S;
                c.P = P;
                return c;
            }
        }
    }
    // first choice: the widest slab whose layout takes the deeper-window
    // instantiation (at most 8 wavefronts) with at least 128 workgroups
    for (int S : {32, 16, 8, 4}) {
        if (fs || !bwd_fits(S, W, R, dv) || !bwd_deep(S, W, R) || NS * (dv / S) < 128) continue;
        c.S = S;
        break;
    }
    int64_t best_units = c.S ? 1 << 30 : 0;
    for (int S : {32, 16, 8, 4}) {
        if ((fs && fs != S) || !bwd_fits(S, W, R, dv)) continue;
        const int64_t units = NS * (dv / S);
        if (c.S == 0 || (best_units < 256 && units > best_units)) {
            c.S = S;
            best_units = units;
        }
    }
    if (c.S == 0) return c;
    if (form == 0 && (fp == 2 || fp == 4 || fp == 8 || fp == 16)) {
        c.P = fp;
    } else if (form == 0 && fp == 0 && !fs) {
        // few streams, where no layout fills the CUs: 2 row partitions where
        // half of them would idle and there are two or more writer wavefronts;
        // with one, the walk is bound by its fixed per-token steps (one stream
        // of 65536 tokens, W = R = 8, d_v = 512, 4-column slabs: 30.6 ms in one
        // partition, 30.4 in two)
        const BGeom g = bwd_geom(c.S, W, R);
        const int64_t units = NS * (dv / c.S);
        if (g.NWW >= 2 && units * 2 <= 256) c.P = 2;
    }
    return c;
}

// Tokens per launch: every buffer one stream spans in a launch stays below
// 2 GiB, so its 32-bit offsets and the dropped-access offset work. Per token a
// stream holds W pre-image rows, one row of v, dy and dv, W + R index and
// weight words, W + 2R planner words and W + R partial sums per slab.
int64_t bwd_chunk_tokens(int64_t T, int W, int R, int dv) {
    int64_t per_tok = (int64_t)(W > 1 ? W : 1) * dv * 4;
    if ((int64_t)(W + 2 * R) * 4 > per_tok) per_tok = (int64_t)(W + 2 * R) * 4;
    if ((int64_t)dv * 4 > per_tok) per_tok = (int64_t)dv * 4;
    const int64_t cap = (int64_t)0x7FFFFFFF / per_tok;
    return T < cap ? T : cap;
}

// Workspace of one launch of Tn tokens: pw, pr, pab, (P > 1) pdv, then the plan.
int64_t bwd_ws_floats(const BCfg& c, int64_t NS, int64_t Tn, int W, int R, int dv) {
    const int nslab = dv / c.S;
    return (int64_t)nslab * NS * Tn * (W + R) + (int64_t)nslab * c.P * NS * Tn * 2 +
           (c.P > 1 ? (int64_t)c.P * NS * Tn * dv : 0) + NS * Tn * (W + 2 * R);
}

template <int S>
hipError_t launch_bwd_slab(const BwdArgs& a, const BCfg& c, hipStream_t st) {
    const BGeom g = bwd_geom(S, a.W, a.R);
    const int nslab = a.dv / S;
    const int64_t Tc = bwd_chunk_tokens(a.T, a.W, a.R, a.dv);
    float* pw = static_cast<float*>(a.workspace);
    int psh = 0;
    while ((1 << psh) < c.P) ++psh;
    const int64_t nblk = unit_grid(a.NS, (int64_t)nslab * c.P);
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
        const bool deep = bwd_deep(S, a.W, a.R);
        // one more wavefront for the finishing sums where the instantiation has room
        const int xw = g.NWW + g.NWR < (deep ? BWD_NW_DEEP : BWD_NWMAX) ? 1 : 0;
        dim3 grid((unsigned)nblk), block((unsigned)((g.NWW + g.NWR + xw) * 64));
        const int sel = (a.form ? 2 : 0) | (a.v_bf16 ? 1 : 0);
        // the planner, then the reverse walk
        uint32_t* plan = reinterpret_cast<uint32_t*>(k.pdv + (c.P > 1 ? (int64_t)c.P * a.NS * Tn * a.dv : 0));
        BPlanArgs pa{};
        pa.idx_w = a.idx_w + c0 * a.W; pa.idx_r = a.idx_r + c0 * a.R; pa.plan = plan;
        const int D = deep ? BWD_D_DEEP : BWD_D;
        pa.Tn = Tn; pa.TS = a.T; pa.N = a.N; pa.W = a.W; pa.R = a.R; pa.D = D;
        // the hash holds (TT + D + 1) * (W + R) entries at load <= 1/4, which
        // keeps the probe chains a wavefront walks short; with TT clamped to 1
        // (W + R > 256 at D = 6) it holds at most 8 * 512 of its 8192 entries;
        // token fields have 10 bits
        pa.TT = (BHT_CAP / 4) / (a.W + a.R) - D - 1;
        if (pa.TT > 1000) pa.TT = 1000;
        if (pa.TT < 1) pa.TT = 1;
        pa.ntile = (Tn + pa.TT - 1) / pa.TT;
        hipLaunchKernelGGL(bwd_plan_kernel, dim3((unsigned)(pa.ntile * a.NS)), dim3(BPLAN_THREADS), 0, st, pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        k.plan = plan;
        const size_t lds = bwd_ring_bytes(S, a.W, a.R, D);
        constexpr int DD = BWD_D_DEEP, D2 = BWD_D, N8 = BWD_NW_DEEP, N16 = BWD_NWMAX;
        switch (sel | (deep ? 4 : 0)) {
            case 0: hipLaunchKernelGGL((scan_backward_kernel<S, 0, false, D2, N16>), grid, block, lds, st, k); break;
            case 1: hipLaunchKernelGGL((scan_backward_kernel<S, 0, true, D2, N16>), grid, block, lds, st, k); break;
            case 2: hipLaunchKernelGGL((scan_backward_kernel<S, 1, false, D2, N16>), grid, block, lds, st, k); break;
            case 3: hipLaunchKernelGGL((scan_backward_kernel<S, 1, true, D2, N16>), grid, block, lds, st, k); break;
            case 4: hipLaunchKernelGGL((scan_backward_kernel<S, 0, false, DD, N8>), grid, block, lds, st, k); break;
            case 5: hipLaunchKernelGGL((scan_backward_kernel<S, 0, true, DD, N8>), grid, block, lds, st, k); break;
            case 6: hipLaunchKernelGGL((scan_backward_kernel<S, 1, false, DD, N8>), grid, block, lds, st, k); break;
            default: hipLaunchKernelGGL((scan_backward_kernel<S, 1, true, DD, N8>), grid, block, lds, st, k); break;
        }
        e = hipGetLastError();
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
        const int64_t b = bwd_ws_floats(c, NS, bwd_chunk_tokens(T, W, R, dv), W, R, dv) * 4;
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
