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
// The token loop is bound by instruction issue as much as by memory, so every
// memory access is a buffer instruction with a 32-bit lane offset and the
// token's offset in a scalar register; an access that must not happen (padding
// lanes, the y store of all but one wavefront) gets an offset past the end of
// its buffer, which the hardware drops (loads return 0). A writer entry carries
// the token's gate values with the row (per-slot form: the update's two
// coefficients c = alpha (1 - beta w) and b = beta w, so M[i] = c M[i] + b v is
// one multiply-add per element), so a writer issues one plan load per token.
//
// Placement: workgroups are dealt to the 8 XCDs round-robin, so with at least
// 8 streams blockIdx is remapped to put every slab of a stream on the same XCD
// (the slabs of a row then share that XCD's L2 lines and the plan records);
// with fewer streams a stream's slabs are spread over all XCDs.
#include "sdm_buffer.h"
#include "sdm_internal.h"

namespace sdm {
namespace {

// Plan entry word: row, flags and the forward source.
constexpr uint32_t ENT_INVALID = 1u << 31;  // padding or out-of-range index: no access
constexpr uint32_t ENT_FWD = 1u << 30;      // value comes from the LDS ring
constexpr uint32_t ROW_MASK = (1u << 18) - 1u;
constexpr uint32_t OFF_MASK = (1u << 30) - 1u;
// The forward source of a shared-residual writer entry: token distance and
// write position in the entry word. Reader entries and per-slot writer entries
// carry the LDS byte offset of the source row in the ring instead (reader: in
// the entry word, which then needs no row; writer: in the last word), so the
// scan adds its lane's offset and reads.
constexpr int POS_SHIFT = 18;               // write position of the source (8 bits)
constexpr int DIST_SHIFT = 26;              // token distance of the source (4 bits)

// Per slab width: D = tokens of row loads in flight per wavefront; the plan
// entries lead by another D + 1 tokens (memory counters complete in order, so
// waiting on an entry also waits on every older row load: a lead >= D keeps D
// tokens of rows in flight); NWMAX = wavefronts per workgroup (sets the VGPR
// budget: 8 -> 256, 16 -> 128). The token loop is unrolled U times so that
// every register ring index is static: U is a multiple of D + 1 (row and
// entry rings), of UR (the LDS ring of written rows, token t in slot t % UR,
// reuse needs UR >= D + 2) and of NBT (the ring of loaded entry blocks; a
// lane loads the entries of BT <= 4 consecutive tokens at once, and a block
// stays until the row loads of its tokens are issued).
template <int S>
struct SlabCfg {
    static constexpr int D = 7, NWMAX = 8, U = 24, UR = 12, NBT = 12, BT = 4;
};
// 16-column slabs: one entry per load. This layout serves the few-stream
// shapes, whose per-token chain of dependent steps sets the pace; there the
// broadcasts cost more than the saved loads (8 streams x 131072 tokens:
// 30.4 ms with one entry per load, 31.3 with four, 31.5 with two).
template <>
struct SlabCfg<16> {
    static constexpr int D = 7, NWMAX = 8, U = 24, UR = 12, NBT = 12, BT = 1;
};
template <>
struct SlabCfg<32> {
    static constexpr int D = 5, NWMAX = 16, U = 12, UR = 12, NBT = 12, BT = 4;
};
// tokens whose plan entries one lane load fetches: the lanes of a row segment
// (in groups of at most 4, a DPP quad) take consecutive tokens
template <int S>
constexpr int entry_batch() {
    constexpr int l = S / 4 >= 4 ? 4 : S / 4;
    return SlabCfg<S>::BT < l ? SlabCfg<S>::BT : l;
}
template <int S>
constexpr bool slab_cfg_ok() {
    constexpr int D = SlabCfg<S>::D, U = SlabCfg<S>::U, UR = SlabCfg<S>::UR, NBT = SlabCfg<S>::NBT;
    constexpr int BT = entry_batch<S>();
    return U % (D + 1) == 0 && U % UR == 0 && U % NBT == 0 && NBT % BT == 0 && UR >= D + 2 &&
           NBT / BT >= 1 + (BT + D) / BT && D <= 15 && (BT & (BT - 1)) == 0 && UR <= 31;
}
static_assert(slab_cfg_ok<4>() && slab_cfg_ok<8>() && slab_cfg_ok<16>() && slab_cfg_ok<32>(), "ring sizes");

// Geometry of a slab of S fp32 columns: L = S/4 lanes per row segment (16 B
// each), G = 64/L rows per wavefront; NWW = ceil(W/G) writer and NWR = ceil(R/G)
// reader wavefronts. Plan record per token: writer entries [NWW][G] of 16 bytes
// (per-slot form: packed word, c, b, write position | ring offset << 8;
// shared-residual form: packed word, weight, alpha, beta), then reader entries
// [NWR][G] of 8 bytes (packed word, weight): writer wave w, lane row r -> write
// access w*G + r, reader wave w -> read access w*G + r. Records come in blocks
// of BT tokens, entry-major within a block, so that one lane load fetches an
// entry of BT consecutive tokens.
struct Geom {
    int S, G, NWW, NWR;
    __host__ __device__ int nw() const { return NWW + NWR; }
    __host__ __device__ int64_t wbytes() const { return (int64_t)NWW * G * 16; }
    __host__ __device__ int64_t rec() const { return wbytes() + (int64_t)NWR * G * 8; }
};

Geom make_geom(int S, int W, int R) {
    Geom g;
    g.S = S;
    g.G = 64 / (S / 4);
    g.NWW = (W + g.G - 1) / g.G;
    g.NWR = (R + g.G - 1) / g.G;
    return g;
}

// Readers whose partial sums are added per token: the largest reader count a slab width
// can have (R <= 256, at most NWMAX wavefronts in all); partial-sum slots of
// absent readers stay zero.
template <int S>
constexpr int nrmax() {
    constexpr int g = 64 / (S / 4), byr = 256 / g, nwm = SlabCfg<S>::NWMAX;
    return byr < nwm ? byr : nwm;
}

// ------------------------------------------------------------------ planner
// The rows of a stream's table may be split into P partitions (a hash of the
// row index), each scanned by its own workgroups: every partition gets its own
// plan records, in which the accesses of a token that fall into it are packed
// to the front in access order (their "rank"); the rest is padding.
//
// One workgroup per (stream, tile of TT tokens). An LDS hash table holds every
// write of tokens [t0 - D, t0 + TT) as a 32-bit entry (row << 14 | tok << pb |
// rank) with tok the token relative to t0 - D; the table is kept at most a
// quarter full. A bitmap over all N rows marks the rows written anywhere in the tile,
// so the common access (no writer nearby) is settled by one LDS read; the
// others look up the latest writer of their row inside their window. Each
// wavefront handles whole tokens (lanes = access positions, ranks by ballot)
// and issues the index loads of PNB tokens together.
constexpr int HT_CAP = 16384;              // LDS hash table entries (32-bit): 64 KiB
constexpr int HT_BITS = 14;
constexpr int HT_WRITES = HT_CAP / 4;      // writes held per tile: at load <= 1/4 the probe chains,
                                           // which a wavefront walks as long as its longest lane's,
                                           // stay short (planner 550 -> 422 us against load 1/2 on
                                           // 32 streams x 8192 tokens; load 1/8: 447 us)
constexpr uint32_t HT_EMPTY = ~0u;         // never a valid entry (see the launch)
constexpr int PLAN_WAVES = 8;
constexpr int PLAN_THREADS = PLAN_WAVES * 64;
constexpr int PNB = 2;                     // tokens whose loads a wavefront issues together (keeps the
                                           // planner under 128 VGPRs: two workgroups per CU)
constexpr int MAX_PARTS = 8;

__device__ __forceinline__ uint32_t ht_hash(uint32_t row) { return (row * 2654435761u) >> (32 - HT_BITS); }
__device__ __forceinline__ int row_part(uint32_t row, int pshift) {
    return pshift == 0 ? 0 : (int)((row * 0x9E3779B1u) >> (32 - pshift));
}

// One launch over a chunk of Tc tokens taken from streams of TS tokens.
struct PlanArgs {
    const int32_t* idx_w; const float* wt_w; int W;
    const int32_t* idx_r; const float* wt_r; int R;
    const float* alpha; const float* beta;
    uint8_t* plan;                         // [NS][P][Tc][rec]
    uint32_t* maxc;                        // [NS][P][2]: most writes / reads of one token (zeroed)
    int64_t Tc, TS, N;
    int D, G, NWW, NWR, TT, pb, P, pshift;
    int64_t ntile;
    int wpos;   // per-slot training forward: writer entries carry the write position
    int form;   // 0: per-slot writer entries (packed, c, b, position | ring offset << 8), c = alpha (1 - beta w),
                // b = beta w; 1: shared-residual writer entries (packed, w, alpha, beta)
    int ur;     // LDS ring of the scan: slots (token t uses slot t % ur), write positions per slot,
    int rpos;   // bytes per position (16 per lane of a row segment)
    int rlane;
    int bt;     // records in blocks of bt tokens: [writer positions][bt] entries, then [reader positions][bt]
    int bts;    // log2(bt): bt is a power of two
    uint32_t urm;  // ceil(2^32 / ur): x % ur = x - ur * umulhi(x, urm) for x < 2^32 / ur
    int64_t tp; // tokens of a (stream, partition) record region (Tc rounded up to bt)
};

// Rank of this lane's access among the valid accesses of its partition at
// lower positions, given the counts cnt[q] of the chunks before; updates cnt.
__device__ __forceinline__ int part_rank(bool ok, int part, int P, uint64_t below, int (&cnt)[MAX_PARTS]) {
    int rank = 0;
#pragma unroll
    for (int q = 0; q < MAX_PARTS; ++q) {
        if (q < P) {
            const uint64_t m = __ballot(ok && part == q);
            if (ok && part == q) rank = cnt[q] + __popcll(m & below);
            cnt[q] += __popcll(m);
        }
    }
    return rank;
}

// The latest write of `row` at a token in [lo, hi] (relative to the window
// start): returns its token (or -1) and its rank in its partition.
__device__ __forceinline__ int fwd_src(const uint32_t* ht, const uint32_t* bm, uint32_t row, int lo, int hi,
                                       int pb, uint32_t& bp) {
    bp = 0;
    if (!((bm[row >> 5] >> (row & 31)) & 1u)) return -1;
    int best = -1;
    uint32_t h = ht_hash(row), ent;
    while ((ent = ht[h]) != HT_EMPTY) {
        if ((ent >> HT_BITS) == row) {
            const int tw = (int)((ent & ((1u << HT_BITS) - 1u)) >> pb);
            if (tw >= lo && tw <= hi && tw > best) {
                best = tw;
                bp = ent & ((1u << pb) - 1u);
            }
        }
        h = (h + 1) & (HT_CAP - 1);
    }
    return best;
}

__global__ __launch_bounds__(PLAN_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void plan_kernel(PlanArgs a) {
    __shared__ uint32_t ht[HT_CAP];
    __shared__ uint32_t smax[2][MAX_PARTS];   // this tile's largest per-partition counts
    extern __shared__ uint32_t bm[];          // ceil(N / 32) words
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    const int W = a.W, R = a.R, D = a.D, G = a.G, NWW = a.NWW, NWR = a.NWR, pb = a.pb, P = a.P, psh = a.pshift;
    const int64_t T = a.Tc, N = a.N;
    const int64_t s = blockIdx.x / a.ntile;
    const int64_t t0 = (blockIdx.x % a.ntile) * a.TT;
    const int64_t t1 = t0 + a.TT < T ? t0 + a.TT : T;
    const int64_t h0 = t0 - D > 0 ? t0 - D : 0;
    const int64_t WB = (int64_t)NWW * G * 16;
    const int64_t REC = WB + (int64_t)NWR * G * 8;
    const int32_t* iw = a.idx_w + s * a.TS * W;
    const float* ww = a.wt_w + s * a.TS * W;
    const int32_t* ir = a.idx_r + s * a.TS * R;
    const float* wr = a.wt_r + s * a.TS * R;
    const float* al = a.alpha + s * a.TS;
    const float* be = a.beta + s * a.TS;
    uint8_t* Ps = a.plan + s * P * a.tp * REC;   // this stream's records [P][tp][rec]
    const int BT = a.bt, BTS = a.bts;
    // byte offset of the entry of token tt at writer / reader position k in a partition's records
    // (blocks of BT tokens, a power of two: shifts, not divisions)
    // (32-bit: the launch's chunking keeps a partition's records below 2 GiB)
    const uint32_t REC32 = (uint32_t)REC, WB32 = (uint32_t)WB;
    auto w_at = [&](int64_t tt, int k) -> uint32_t {
        const uint32_t t = (uint32_t)tt;
        return ((t >> BTS) << BTS) * REC32 + (((uint32_t)k << BTS) + (t & (uint32_t)(BT - 1))) * 16u;
    };
    auto r_at = [&](int64_t tt, int k) -> uint32_t {
        const uint32_t t = (uint32_t)tt;
        return ((t >> BTS) << BTS) * REC32 + (WB32 << BTS) + (((uint32_t)k << BTS) + (t & (uint32_t)(BT - 1))) * 8u;
    };
    // ring slot of a token: x % ur by a multiply-high with ceil(2^32 / ur), exact for x < 2^32 / ur
    // (x = a token of the launch: below 2^27, since the chunking keeps 16+ bytes per token of a
    // stream's region below 2 GiB, and ur <= 31)
    const uint32_t UR = (uint32_t)a.ur, URM = a.urm;
    auto slot_of = [&](uint32_t x) -> uint32_t { return x - UR * __umulhi(x, URM); };

    for (int i = tid; i < HT_CAP / 4; i += PLAN_THREADS)
        reinterpret_cast<uint4*>(ht)[i] = make_uint4(HT_EMPTY, HT_EMPTY, HT_EMPTY, HT_EMPTY);
    const int nbm = (int)((N + 31) >> 5);
    for (int i = tid; i < nbm; i += PLAN_THREADS) bm[i] = 0u;
    if (tid < 2 * MAX_PARTS) smax[tid / MAX_PARTS][tid % MAX_PARTS] = 0u;
    __syncthreads();

    // phase 1: the writes of tokens [h0, t1), with their rank inside their partition
    const int n1 = (int)(t1 - h0);
    for (int k0 = wave; k0 < n1; k0 += PLAN_WAVES * PNB) {
        int cnt[PNB][MAX_PARTS] = {};
        for (int c = 0; c < W; c += 64) {
            int32_t row[PNB];
#pragma unroll
            for (int u = 0; u < PNB; ++u) {
                const int tk = k0 + u * PLAN_WAVES, p = c + lane;
                row[u] = (tk < n1 && p < W) ? iw[(h0 + tk) * W + p] : -1;
            }
#pragma unroll
            for (int u = 0; u < PNB; ++u) {
                const int tk = k0 + u * PLAN_WAVES;
                if (tk >= n1) break;  // uniform
                const bool ok = row[u] >= 0 && row[u] < N;
                const int part = ok ? row_part((uint32_t)row[u], psh) : 0;
                const int rank = part_rank(ok, part, P, below, cnt[u]);
                if (ok) {
                    atomicOr(&bm[row[u] >> 5], 1u << (row[u] & 31));
                    const uint32_t ent = ((uint32_t)row[u] << HT_BITS) | ((uint32_t)tk << pb) | (uint32_t)rank;
                    uint32_t h = ht_hash((uint32_t)row[u]);
                    while (atomicCAS(&ht[h], HT_EMPTY, ent) != HT_EMPTY) h = (h + 1) & (HT_CAP - 1);
                }
            }
        }
    }
    __syncthreads();

    // phase 2: the records of tokens [t0, t1): writes, then reads, then padding;
    // the largest per-partition counts are collected in LDS
    const int n2 = (int)(t1 - t0);
    for (int k0 = wave; k0 < n2; k0 += PLAN_WAVES * PNB) {
        for (int br = 0; br < 2; ++br) {
            const bool isw = br == 0;
            const int K = isw ? W : R;
            const int32_t* ix = isw ? iw : ir;
            const float* wx = isw ? ww : wr;
            int cnt[PNB][MAX_PARTS] = {};
            for (int c = 0; c < K; c += 64) {
                int32_t row[PNB];
                float w[PNB];
#pragma unroll
                for (int u = 0; u < PNB; ++u) {
                    const int tk = k0 + u * PLAN_WAVES, p = c + lane;
                    const bool in = tk < n2 && p < K;
                    row[u] = in ? ix[(t0 + tk) * K + p] : -1;
                    w[u] = in ? wx[(t0 + tk) * K + p] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < PNB; ++u) {
                    const int tk = k0 + u * PLAN_WAVES;
                    if (tk >= n2) break;  // uniform
                    const int64_t tt = t0 + tk;
                    const bool ok = row[u] >= 0 && row[u] < N;
                    const int part = ok ? row_part((uint32_t)row[u], psh) : 0;
                    const int rank = part_rank(ok, part, P, below, cnt[u]);
                    if (!ok) continue;
                    // latest writer of this row in [tt-D, tt-1] (writes) or [tt-D, tt] (reads)
                    const int cur = (int)(tt - h0);
                    uint32_t bp;
                    const int src = fwd_src(ht, bm, (uint32_t)row[u], cur - D, cur - (isw ? 1 : 0), pb, bp);
                    // LDS byte offset of the source row in the scan's ring (slot of its token, its rank)
                    const uint32_t roff =
                        src < 0 ? 0u : (slot_of((uint32_t)(h0 + src)) * (uint32_t)a.rpos + bp) * (uint32_t)a.rlane;
                    uint8_t* rec = Ps + (int64_t)part * a.tp * REC;
                    if (isw && a.form == 0) {
                        const float b = be[tt] * w[u], cw = al[tt] * (1.f - b);
                        const uint32_t w4 = (a.wpos ? (uint32_t)(c + lane) : 0u) | (roff << 8);
                        *reinterpret_cast<int4*>(rec + w_at(tt, rank)) =
                            make_int4((int)((uint32_t)row[u] | (src < 0 ? 0u : ENT_FWD)), __float_as_int(cw),
                                      __float_as_int(b), (int)w4);
                    } else if (isw) {
                        const uint32_t fb =
                            src < 0 ? 0u : ENT_FWD | ((uint32_t)(cur - src) << DIST_SHIFT) | (bp << POS_SHIFT);
                        *reinterpret_cast<int4*>(rec + w_at(tt, rank)) = make_int4(
                            (int)((uint32_t)row[u] | fb), __float_as_int(w[u]), __float_as_int(al[tt]),
                            __float_as_int(be[tt]));
                    } else {
                        *reinterpret_cast<int2*>(rec + r_at(tt, rank)) =
                            make_int2((int)(src < 0 ? (uint32_t)row[u] : ENT_FWD | roff), __float_as_int(w[u]));
                    }
                }
            }
            // padding: slots past each partition's count
            const int cap = (isw ? NWW : NWR) * G;
#pragma unroll
            for (int u = 0; u < PNB; ++u) {
                const int tk = k0 + u * PLAN_WAVES;
                if (tk >= n2) break;
                const int64_t tt = t0 + tk;
#pragma unroll
                for (int q = 0; q < MAX_PARTS; ++q) {
                    if (q >= P) break;
                    if (lane == 0) atomicMax(&smax[br][q], (uint32_t)cnt[u][q]);
                    uint8_t* rec = Ps + (int64_t)q * a.tp * REC;
                    for (int k = cnt[u][q] + lane; k < cap; k += 64) {
                        if (isw)
                            *reinterpret_cast<int4*>(rec + w_at(tt, k)) = make_int4((int)ENT_INVALID, 0, 0, 0);
                        else
                            *reinterpret_cast<int2*>(rec + r_at(tt, k)) = make_int2((int)ENT_INVALID, 0);
                    }
                }
            }
        }
    }
    __syncthreads();
    if (tid < 2 * P) atomicMax(&a.maxc[(s * P + tid / 2) * 2 + tid % 2], smax[tid % 2][tid / 2]);
}

__global__ void zero_u32(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------ scan
template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// Entry of token i (0 <= i < BT) of a block: the lanes of a row segment hold
// consecutive tokens' entries (lane l holds token l % BT), a DPP quad
// permutation hands token i's to every lane of the segment.
template <int BT, int I>
__device__ __forceinline__ int ent_bcast_c(int x) {
    if constexpr (BT == 2) return __builtin_amdgcn_mov_dpp(x, I | (I << 2) | ((2 + I) << 4) | ((2 + I) << 6), 0xF, 0xF, false);
    else return __builtin_amdgcn_mov_dpp(x, I | (I << 2) | (I << 4) | (I << 6), 0xF, 0xF, false);
}
template <int BT>
__device__ __forceinline__ int ent_bcast(int x, int i) {
    if constexpr (BT == 1) return x;
    else if constexpr (BT == 2) return i == 0 ? ent_bcast_c<2, 0>(x) : ent_bcast_c<2, 1>(x);
    else {
        switch (i) {
            case 0: return ent_bcast_c<4, 0>(x);
            case 1: return ent_bcast_c<4, 1>(x);
            case 2: return ent_bcast_c<4, 2>(x);
            default: return ent_bcast_c<4, 3>(x);
        }
    }
}

// Sum of the first Q partial-sum slots (stride S) as a balanced tree. Slots of
// readers that do not run hold zero, so any power of two Q >= the number of
// running readers gives the same sum: the tree over 2Q adds a zero subtree.
template <int Q, int S>
__device__ __forceinline__ float tree_sum(const float* p) {
    if constexpr (Q == 1) return p[0];
    else return tree_sum<Q / 2, S>(p) + tree_sum<Q / 2, S>(p + (Q / 2) * S);
}
template <int NRMAX, int S>
__device__ __forceinline__ float readers_sum(const float* p, int nra) {
    if (nra <= 1) return tree_sum<1, S>(p);
    if (nra <= 2) return tree_sum<2, S>(p);
    if constexpr (NRMAX >= 4) if (nra <= 4) return tree_sum<4, S>(p);
    if constexpr (NRMAX >= 8) if (nra <= 8) return tree_sum<8, S>(p);
    if constexpr (NRMAX >= 16) return tree_sum<16, S>(p);
    return tree_sum<NRMAX, S>(p);
}

struct ScanKArgs {
    const uint8_t* plan;  // [NS][P][T][rec]
    const uint32_t* maxc; // [NS][P][2]: most writes / reads of one token in a partition
    const void* v;
    void* M;              // fp32 or bfloat16 elements
    float* y;       // y of (stream s, partition p) at y + s * ys + p * yp
    int64_t ys, yp;
    int T;          // tokens in this launch
    int64_t TS;     // tokens per stream in v (stream stride)
    int64_t N;
    int dv, nslab, P;
    int64_t NS;
    int NWW, NWR;
    float* snap;    // SAVE: pre-images of stream s at snap + s * snap_s, [T][W][dv]
    int64_t snap_s;
    int W;
};

// SAVE (training forward): every write also stores its row as it was before
// this token's decay (the pre-image M_{t-1}[i]) at [t][write position][col],
// which the backward uses to undo the write. The per-slot form's writer
// entries carry the write position for it; the shared-residual form runs with
// one row partition, where a writer's rank in its token is the write position.
// MBF16: the table is stored in bfloat16. A lane's 16 bytes of a row then hold
// 8 columns instead of 4, so the same lane layout covers twice the columns
// (slab width S = 2 * SL) and every row access moves half the bytes; rows are
// unpacked to fp32 for the update and rounded to nearest-even bfloat16 on the
// store (and in the LDS ring, which holds the stored bytes).
// SL = 4 * (lanes per row segment): the slab width in columns of an fp32 table.
template <int SL, int FORM, bool VBF16, bool SAVE, bool MBF16>
__global__ __launch_bounds__(SlabCfg<SL>::NWMAX * 64) void scan_kernel(ScanKArgs a) {
    static_assert(!(SAVE && MBF16), "pre-images are taken of fp32 tables only");
    using RF = RowFmt<MBF16>;
    constexpr int L = SL / 4, G = 64 / L, NQ = RF::NQ, CPL = RF::CPL, S = L * CPL;
    constexpr int D = SlabCfg<SL>::D, NWMAX = SlabCfg<SL>::NWMAX, NRMAX = nrmax<SL>();
    constexpr int DM = D + 1;                   // plan-entry lead beyond D
    constexpr int UP = D + 1;                   // row / value / entry rings: D in flight + the one in use
    constexpr int U = SlabCfg<SL>::U;           // unroll factor: every ring index is static
    constexpr int UR = SlabCfg<SL>::UR;         // LDS ring of written rows: token t in slot t % UR
    constexpr int BT = entry_batch<SL>();       // tokens whose entries one lane load fetches
    constexpr int NB = SlabCfg<SL>::NBT / BT;   // ring of loaded entry blocks
    using VL = VLoadN<VBF16, NQ>;
    using V4 = typename VL::T;
    const int NWW = a.NWW, NWR = a.NWR, T = a.T, dv = a.dv;
    extern __shared__ float4 lds[];
    float4* ring = lds;                                              // [UR][NWW*G][L]
    float* ybuf = reinterpret_cast<float*>(lds + UR * NWW * G * L);  // [2][NRMAX][S]
    float4* vbuf = reinterpret_cast<float4*>(ybuf + 2 * NRMAX * S);  // [NWW][S/4] (FIG2)

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane / L, cc = lane % L;
    int64_t s;
    int kq;
    block_unit(blockIdx.x, a.NS, a.nslab * a.P, s, kq);
    const int slab = kq % a.nslab, part = kq / a.nslab;
    if (s >= a.NS) return;  // uniform over the workgroup
    const int col = slab * S + cc * CPL;
    const Geom geo{SL, G, NWW, NWR};
    const uint32_t REC = (uint32_t)geo.rec();
    // plan records of this (stream, partition): blocks of BT tokens, each block
    // [writer positions][BT tokens] entries then [reader positions][BT tokens]
    const int64_t TP = ((int64_t)T + BT - 1) / BT * BT;
    const rsrc_t Rp = make_rsrc(a.plan + (s * a.P + part) * TP * REC, TP * REC);
    const rsrc_t Rm = make_rsrc(static_cast<char*>(a.M) + s * a.N * dv * RF::ESZ, a.N * dv * RF::ESZ);
    const rsrc_t Rv = make_rsrc(static_cast<const char*>(a.v) + s * a.TS * dv * VL::ESZ, (int64_t)T * dv * VL::ESZ);
    const rsrc_t Ry = make_rsrc(a.y + s * a.ys + part * a.yp, (int64_t)T * dv * 4);
    const rsrc_t Rs = make_rsrc(SAVE ? a.snap + s * a.snap_s : a.M, SAVE ? (int64_t)T * a.W * dv * 4 : 0);
    const bool writer = wave < NWW;
    const int pos = wave * G + r;                        // write position of a writer lane
    const int rw = wave - NWW;                           // reader index
    const uint32_t e_off = writer ? ((uint32_t)pos * BT + (uint32_t)(cc % BT)) * 16u
                                  : (uint32_t)geo.wbytes() * BT + ((uint32_t)(rw * G + r) * BT + (uint32_t)(cc % BT)) * 8u;
    const uint32_t BREC = (uint32_t)BT * REC;  // bytes of one block of entries
    const uint32_t dv4 = (uint32_t)dv * 4u, col4 = (uint32_t)col * 4u;          // fp32 rows (y, snapshots)
    const uint32_t mrow = (uint32_t)dv * RF::ESZ, colb = (uint32_t)col * RF::ESZ;  // table rows
    const uint32_t v_off = (uint32_t)col * VL::ESZ;
    const uint32_t vstride = (uint32_t)dv * VL::ESZ;
    const uint32_t sstride = (uint32_t)a.W * dv4;                    // snapshot bytes per token
    const uint32_t s_lane = (uint32_t)pos * dv4 + col4;
    const int ylane = lane < S ? lane : 0;

    // partial sums of absent readers stay zero (made visible by the first barrier)
    for (int i = threadIdx.x; i < 2 * NRMAX * S; i += blockDim.x) ybuf[i] = 0.f;

    // The planner packs a partition's accesses to the front of its records, so
    // wavefronts whose slots no token of this launch reaches have nothing to do:
    // they only keep the barrier count (one barrier per token, one at the end).
    // Reader 0 always runs. The readers' partial sums of a token are added, and
    // y stored, by the last reader wavefront when it is such an idle one (then
    // the running readers only scan rows), else by reader 0. The shared-residual
    // form uses all writers' partial sums and runs every wavefront.
    // nra: reader wavefronts whose partial sums are added (a power of two)
    int nra = NWR;
    bool sum0 = true;  // reader 0 adds the partial sums
    int sw = 0;        // else this reader wavefront does
    if constexpr (FORM == 0) {
        const uint32_t* mc = a.maxc + (s * a.P + part) * 2;
        nra = ((int)mc[1] + G - 1) / G;
        // summing candidate: the extra wavefront the launch adds to a layout
        // with one reader wavefront, else the last reader wavefront
        sw = (int)(blockDim.x >> 6) > NWW + NWR ? NWR : NWR - 1;
        sum0 = !(sw >= 1 && nra <= sw);
        const bool idle = writer ? (uint32_t)(wave * G) >= mc[0] : (rw > 0 && (uint32_t)(rw * G) >= mc[1]);
        if (idle && (sum0 || rw != sw)) {
            for (int t = 0; t <= T; ++t) __syncthreads();
            return;
        }
    }
    {
        int q = 1;
        while (q < nra) q *= 2;
        nra = q;
    }
    // the summing wavefront's first S lanes store y[t-1] (one column each); every
    // other y store is dropped
    const bool ysum = !writer && rw == (sum0 ? 0 : sw);
    const uint32_t y_off = (ysum && lane < S) ? (uint32_t)(slab * S + lane) * 4u : OOB;
    if (FORM == 0 && ysum && !sum0) {
        // an idle reader wavefront: token t - 1's partial sums are complete at
        // token t's barrier and are not overwritten before token t + 1's
        for (int t = 0; t < T; ++t) {
            __syncthreads();
            if (t > 0) st_f1(readers_sum<NRMAX, S>(ybuf + ((t - 1) & 1) * NRMAX * S + ylane, nra), Ry, y_off, (uint32_t)(t - 1) * dv4);
        }
        __syncthreads();
        if (T > 0) st_f1(readers_sum<NRMAX, S>(ybuf + ((T - 1) & 1) * NRMAX * S + ylane, nra), Ry, y_off, (uint32_t)(T - 1) * dv4);
        return;
    }

    // A forwarded access loads nothing (its value comes from the ring); the
    // store of a written row goes to its table offset. Token offsets sit in the
    // per-lane offset, which the hardware range-checks, so a prefetch past the
    // last token is dropped and needs no clamp.
    auto row_off = [&](uint32_t pk) -> uint32_t {
        return (pk & ENT_INVALID) ? OOB : __umul24(pk & ROW_MASK, mrow) + colb;
    };
    auto load_row = [&](uint32_t pk) -> float4 { return ld_f4(Rm, (pk & ENT_FWD) ? OOB : row_off(pk), 0u); };
    auto ring_at = [&](int slot, int p) -> float4& { return ring[((int64_t)slot * NWW * G + p) * L + cc]; };
    // forwarded rows come from the LDS ring; the ballot keeps the common
    // no-forward case free of LDS traffic
    auto source = [&](int slot, uint32_t pk, float4 pre) -> float4 {  // shared-residual writers
        const bool f = (pk & (ENT_FWD | ENT_INVALID)) == ENT_FWD;
        if (__ballot(f) != 0ull && f) {
            int sl = slot - (int)((pk >> DIST_SHIFT) & 15u);
            if (sl < 0) sl += UR;
            pre = ring_at(sl, (int)((pk >> POS_SHIFT) & 255u));
        }
        return pre;
    };
    auto source_at = [&](uint32_t pk, uint32_t off, float4 pre) -> float4 {  // readers, per-slot writers
        // a uniform branch around one 16-byte read of every lane (off is a
        // multiple of 16; lanes that do not forward read slot 0 and keep pre)
        const bool f = (pk & (ENT_FWD | ENT_INVALID)) == ENT_FWD;
        if (__ballot(f) != 0ull) {
            const float4 x = ring[(f ? off >> 4 : 0u) + cc];
            pre.x = f ? x.x : pre.x;  // per component (a float4 select goes through memory)
            pre.y = f ? x.y : pre.y;
            pre.z = f ? x.z : pre.z;
            pre.w = f ? x.w : pre.w;
        }
        return pre;
    };

    // one token of a writer wavefront (barriers: [B'_t], B_t)
    auto write_token = [&](int t, int slot, int4 e, float4 pre, V4 vt, uint32_t soff) {
        const uint32_t pk = (uint32_t)e.x;
        float4 old;
        if constexpr (FORM == 0) old = source_at(pk, (uint32_t)e.w >> 8, pre);
        else old = source(slot, pk, pre);
        if constexpr (SAVE) {
            // per-slot entries carry the write position (partitions reorder them)
            const uint32_t so = FORM == 0 ? __umul24((uint32_t)e.w & 255u, dv4) + col4 : s_lane;
            st_f4(old, Rs, (pk & ENT_INVALID) ? OOB : so, (uint32_t)t * sstride);
        }
        float4 mt[NQ], vf[NQ], nv[NQ];
        RF::unpack(old, mt);
        VL::f(vt, vf);
        if constexpr (FORM == 0) {
            // entry = (packed, c, b, ...): M[i] = c M[i] + b v, c = alpha (1 - beta w), b = beta w
            const float cw = __int_as_float(e.y), b = __int_as_float(e.z);
#pragma unroll
            for (int i = 0; i < NQ; ++i) nv[i] = f4_fma(cw, mt[i], f4_scale(b, vf[i]));
        } else {
            // entry = (packed, w, alpha, beta): M[i] = alpha M[i] + beta w (v - sum_j w_j alpha M[j])
            const float w = __int_as_float(e.y), al = __int_as_float(e.z), be = __int_as_float(e.w);
            float4 pred[NQ];
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                mt[i] = f4_scale(al, mt[i]);
                const float part = rows_reduce<L>(f4_scale(w, mt[i]));
                if ((lane & 15) < L)
                    reinterpret_cast<float*>(vbuf)[wave * S + CPL * (lane & 15) + 4 * i + (lane >> 4)] = part;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                pred[i] = vbuf[NQ * cc + i];
#pragma unroll
                for (int q = 1; q < NWMAX; ++q)
                    if (q < NWW) pred[i] = f4_add(pred[i], vbuf[q * (S / 4) + NQ * cc + i]);
            }
#pragma unroll
            for (int i = 0; i < NQ; ++i) nv[i] = f4_fma(be * w, f4_sub(vf[i], pred[i]), mt[i]);
        }
        const float4 st = RF::pack(nv);
        st_f4(st, Rm, soff, 0u);
        ring_at(slot, pos) = st;
        __syncthreads();
    };
    // one token of a reader wavefront (barriers: [B'_t], B_t); the partial sums
    // of token t are added by the summing wavefront after the next barrier
    auto read_barrier = [&]() {
        if constexpr (FORM == 1) __syncthreads();
        __syncthreads();
    };
    // YS: this wavefront adds the readers' partial sums and stores y (a
    // separate copy of the loop, so the other readers issue no y store)
    auto read_token = [&](auto ys_c, int t, int2 e, float4 pre, uint32_t yv, uint32_t ys) {
        constexpr bool YS = decltype(ys_c)::value;
        // when it sums, reader 0 first adds the previous token's partials
        // (complete since this token's barrier), so their LDS reads overlap
        // the row sum below
        float acc = 0.f;
        if constexpr (YS) acc = readers_sum<NRMAX, S>(ybuf + ((t - 1) & 1) * NRMAX * S + ylane, nra);
        const uint32_t pk = (uint32_t)e.x;
        float4 cur[NQ];
        RF::unpack(source_at(pk, pk & OFF_MASK, pre), cur);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const float part = rows_reduce<L>(f4_scale(__int_as_float(e.y), cur[i]));
            if ((lane & 15) < L) ybuf[((t & 1) * NRMAX + rw) * S + CPL * (lane & 15) + 4 * i + (lane >> 4)] = part;
        }
        if constexpr (YS) st_f1(acc, Ry, yv, ys);  // y of token t - 1: dropped at t = 0 and beyond S lanes
    };

    // Main loop: U tokens per trip, fully unrolled so that the register rings
    // are statically indexed. Each role gets its own prologue that issues the
    // steady-state sequence of memory operations (with a dropped store standing
    // in for each token's store), so that the loop header merges like states and
    // the compiler's memory waits stay D tokens deep.
    // the table offset of each prefetched write is kept for its store where
    // the VGPR budget allows (layouts of at most 8 wavefronts)
    constexpr bool KEEP_OFF = NWMAX <= 8;
    int t_done = 0;
    if (T >= U) {
        float4 pre[UP];
        uint32_t ve = e_off;  // per-lane offset of the next block of entries
        if (writer) {
            int4 blk[NB], ent[UP];
            V4 vv[UP];
            uint32_t so[KEEP_OFF ? UP : 1];
            uint32_t vo = v_off;  // per-lane offset of the next v to load
            auto load_block = [&](int q) {  // entries of tokens q .. q + BT - 1
                blk[(q / BT) % NB] = ld_i4(Rp, ve, 0u);
                ve += BREC;
            };
            auto prefetch = [&](int q) {  // token q: its entry, row and v
                const int4 b = blk[(q / BT) % NB];
                const int4 e = make_int4(ent_bcast<BT>(b.x, q % BT), ent_bcast<BT>(b.y, q % BT),
                                         ent_bcast<BT>(b.z, q % BT), ent_bcast<BT>(b.w, q % BT));
                ent[q % UP] = e;
                const uint32_t pk = (uint32_t)e.x;
                const uint32_t ro = row_off(pk);
                if constexpr (KEEP_OFF) so[q % UP] = ro;
                pre[q % UP] = ld_f4(Rm, (pk & ENT_FWD) ? OOB : ro, 0u);
                vv[q % UP] = VL::load(Rv, vo, 0u);
                vo += vstride;
            };
#pragma unroll
            for (int p = 0; p < D + DM; ++p) {
                if (p % BT == 0) load_block(p);
                if (p >= DM) prefetch(p - DM);
                // the dropped stores get distinct offsets (identical ones would be
                // merged away) and the scheduling barrier keeps this order, so
                // the counter state entering the loop is the steady-state one
                st_f4(make_float4(0.f, 0.f, 0.f, 0.f), Rm, OOB, (uint32_t)p * 16u);
                if constexpr (SAVE) st_f4(make_float4(0.f, 0.f, 0.f, 0.f), Rs, OOB, (uint32_t)p * 16u);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int t0 = 0; t0 + U <= T; t0 += U) {
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    if ((j + D + DM) % BT == 0) load_block(j + D + DM);
                    prefetch(j + D);
                    write_token(t0 + j, j % UR, ent[j % UP], pre[j % UP], vv[j % UP],
                                KEEP_OFF ? so[j % UP] : row_off((uint32_t)ent[j % UP].x));
                }
            }
        } else {
            auto reader_loop = [&](auto ys_c) {
                constexpr bool YS = decltype(ys_c)::value;
                int2 blk[NB], ent[UP];
                uint32_t ys = 0u - dv4;  // y of token t - 1
                auto load_block = [&](int q) {
                    blk[(q / BT) % NB] = ld_i2(Rp, ve, 0u);
                    ve += BREC;
                };
                auto prefetch = [&](int q) {
                    const int2 b = blk[(q / BT) % NB];
                    const int2 e = make_int2(ent_bcast<BT>(b.x, q % BT), ent_bcast<BT>(b.y, q % BT));
                    ent[q % UP] = e;
                    pre[q % UP] = load_row((uint32_t)e.x);
                };
#pragma unroll
                for (int p = 0; p < D + DM; ++p) {
                    if (p % BT == 0) load_block(p);
                    if (p >= DM) prefetch(p - DM);
                    if constexpr (YS) st_f1(0.f, Ry, OOB, (uint32_t)p * 4u);
                    __builtin_amdgcn_sched_barrier(0);
                }
                for (int t0 = 0; t0 + U <= T; t0 += U) {
#pragma unroll
                    for (int j = 0; j < U; ++j) {
                        if ((j + D + DM) % BT == 0) load_block(j + D + DM);
                        prefetch(j + D);
                        read_barrier();
                        read_token(ys_c, t0 + j, ent[j % UP], pre[j % UP], (j > 0 || t0 > 0) ? y_off : OOB, ys);
                        ys += dv4;
                    }
                }
            };
            if (ysum) reader_loop(BoolC<true>{});
            else reader_loop(BoolC<false>{});
        }
        t_done = (T / U) * U;
    }
    // tail (and short sequences): loads right before use; forwarding stays valid
    for (int t = t_done; t < T; ++t) {
        const uint32_t bo = e_off + (uint32_t)(t / BT) * BREC;
        const int i = t % BT;
        if (writer) {
            const int4 b = ld_i4(Rp, bo, 0u);
            const int4 e = make_int4(ent_bcast<BT>(b.x, i), ent_bcast<BT>(b.y, i), ent_bcast<BT>(b.z, i),
                                     ent_bcast<BT>(b.w, i));
            write_token(t, t % UR, e, load_row((uint32_t)e.x), VL::load(Rv, v_off + (uint32_t)t * vstride, 0u),
                        row_off((uint32_t)e.x));
        } else {
            const int2 b = ld_i2(Rp, bo, 0u);
            const int2 e = make_int2(ent_bcast<BT>(b.x, i), ent_bcast<BT>(b.y, i));
            const float4 pr = load_row((uint32_t)e.x);
            read_barrier();
            if (ysum) read_token(BoolC<true>{}, t, e, pr, t > 0 ? y_off : OOB, (uint32_t)(t - 1) * dv4);
            else read_token(BoolC<false>{}, t, e, pr, OOB, 0u);
        }
    }
    // the last token's partial sums
    __syncthreads();
    if (ysum && T > 0) {
        const float acc = readers_sum<NRMAX, S>(ybuf + ((T - 1) & 1) * NRMAX * S + ylane, nra);
        st_f1(acc, Ry, y_off, (uint32_t)(T - 1) * dv4);
    }
}
// ------------------------------------------------------------------ short scans
// For a few tokens per call (decoding: one token per sequence and call, the
// table kept between calls) the prefetch pipeline and its planner cost more
// than they hide. The direct form reads the indices itself and issues a
// token's row loads only after the barrier that closes the previous token, so
// every load sees every earlier store (same workgroup, same CU) and nothing is
// forwarded. Per token: writers load, update and store their rows; barrier;
// readers load theirs (after this token's writes) and reduce; barrier; reader
// 0 sums the readers' partials and stores y. The indices, weights, gates and v
// of the next token are loaded while the current one runs.
struct DirectArgs {
    const int32_t* idx_w; const float* wt_w; int W;
    const int32_t* idx_r; const float* wt_r; int R;
    const float* alpha; const float* beta;
    const void* v;
    void* M;        // fp32 or bfloat16 elements
    float* y;
    int T;
    int64_t N;
    int dv, nslab;
    int64_t NS;
    int NWW, NWR;
    float* snap;    // SAVE: [NS][T][W][dv] pre-images
};

template <int SL, int FORM, bool VBF16, bool SAVE, bool MBF16>
__global__ __launch_bounds__(SlabCfg<SL>::NWMAX * 64) void scan_direct_kernel(DirectArgs a) {
    static_assert(!(SAVE && MBF16), "pre-images are taken of fp32 tables only");
    using RF = RowFmt<MBF16>;
    constexpr int L = SL / 4, G = 64 / L, NQ = RF::NQ, CPL = RF::CPL, S = L * CPL;
    constexpr int NWMAX = SlabCfg<SL>::NWMAX, NRMAX = nrmax<SL>();
    using VL = VLoadN<VBF16, NQ>;
    using V4 = typename VL::T;
    const int NWW = a.NWW, NWR = a.NWR, T = a.T, dv = a.dv, W = a.W, R = a.R;
    __shared__ float ybuf[NRMAX * S];
    __shared__ float4 vbuf[NWMAX * S / 4];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane / L, cc = lane % L;
    int64_t s;
    int slab;
    block_unit(blockIdx.x, a.NS, a.nslab, s, slab);
    if (s >= a.NS) return;  // uniform over the workgroup
    const int col = slab * S + cc * CPL;
    const bool writer = wave < NWW;
    const int rw = wave - NWW;
    const int pos = writer ? wave * G + r : rw * G + r;  // access position of this lane's row
    const int K = writer ? W : R;
    const bool has = pos < K;
    const int32_t* ix = (writer ? a.idx_w : a.idx_r) + s * (int64_t)T * K;
    const float* wx = (writer ? a.wt_w : a.wt_r) + s * (int64_t)T * K;
    const rsrc_t Rm = make_rsrc(static_cast<char*>(a.M) + s * a.N * dv * RF::ESZ, a.N * dv * RF::ESZ);
    const rsrc_t Rv = make_rsrc(static_cast<const char*>(a.v) + s * (int64_t)T * dv * VL::ESZ,
                                (int64_t)T * dv * VL::ESZ);
    const rsrc_t Ry = make_rsrc(a.y + s * (int64_t)T * dv, (int64_t)T * dv * 4);
    const rsrc_t Rs = make_rsrc(SAVE ? a.snap + s * (int64_t)T * W * dv : a.M, SAVE ? (int64_t)T * W * dv * 4 : 0);
    const uint32_t dv4 = (uint32_t)dv * 4u, col4 = (uint32_t)col * 4u;          // fp32 rows (y, snapshots)
    const uint32_t mrow = (uint32_t)dv * RF::ESZ, colb = (uint32_t)col * RF::ESZ;  // table rows
    const uint32_t y_off = (!writer && rw == 0 && lane < S) ? (uint32_t)(slab * S + lane) * 4u : OOB;
    const int ylane = lane < S ? lane : 0;
    int nra = 1;
    while (nra < NWR) nra *= 2;
    for (int i = threadIdx.x; i < NRMAX * S; i += blockDim.x) ybuf[i] = 0.f;
    __syncthreads();

    auto off_of = [&](int32_t row) -> uint32_t {
        return (row >= 0 && row < a.N) ? __umul24((uint32_t)row, mrow) + colb : OOB;
    };
    // this lane's access of token t: row offset and weight (0 when absent)
    int32_t row_n = has ? ix[pos] : -1;
    float w_n = has ? wx[pos] : 0.f;
    float al_n = a.alpha[s * (int64_t)T], be_n = a.beta[s * (int64_t)T];
    V4 v_n = VL::load(Rv, (uint32_t)col * VL::ESZ, 0u);
    for (int t = 0; t < T; ++t) {
        const uint32_t off = off_of(row_n);
        const float w = off == OOB ? 0.f : w_n, al = al_n, be = be_n;
        const V4 vt = v_n;
        if (t + 1 < T) {  // uniform: the next token's indices, weights, gates and v
            const int64_t o = (int64_t)(t + 1) * K + pos;
            row_n = has ? ix[o] : -1;
            w_n = has ? wx[o] : 0.f;
            al_n = a.alpha[s * (int64_t)T + t + 1];
            be_n = a.beta[s * (int64_t)T + t + 1];
            v_n = VL::load(Rv, (uint32_t)col * VL::ESZ, (uint32_t)(t + 1) * (uint32_t)dv * VL::ESZ);
        }
        if (writer) {
            const float4 pre = ld_f4(Rm, off, 0u);  // after the barrier that closed token t-1
            if constexpr (SAVE)
                st_f4(pre, Rs, off == OOB ? OOB : (uint32_t)pos * dv4 + col4, (uint32_t)t * (uint32_t)W * dv4);
            float4 mt[NQ], pred[NQ], vf[NQ], nv[NQ];
            RF::unpack(pre, mt);
            VL::f(vt, vf);
            if constexpr (FORM == 0) {
                // M[i] = c M[i] + b v with c = alpha (1 - beta w), b = beta w: the
                // pipelined form's arithmetic, so a sequence split over both forms
                // gives the same bits
                const float b = be * w, cw = al * (1.f - b);
#pragma unroll
                for (int i = 0; i < NQ; ++i) nv[i] = f4_fma(cw, mt[i], f4_scale(b, vf[i]));
            } else {
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    mt[i] = f4_scale(al, mt[i]);
                    pred[i] = mt[i];
                }
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const float part = rows_reduce<L>(f4_scale(w, mt[i]));
                    if ((lane & 15) < L)
                        reinterpret_cast<float*>(vbuf)[wave * S + CPL * (lane & 15) + 4 * i + (lane >> 4)] = part;
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    pred[i] = vbuf[NQ * cc + i];
                    for (int q = 1; q < NWW; ++q) pred[i] = f4_add(pred[i], vbuf[q * (S / 4) + NQ * cc + i]);
                }
#pragma unroll
                for (int i = 0; i < NQ; ++i) nv[i] = f4_fma(be * w, f4_sub(vf[i], pred[i]), mt[i]);
            }
            st_f4(RF::pack(nv), Rm, off, 0u);
            __syncthreads();  // B1: this token's rows are written
            __syncthreads();  // B2
        } else {
            if constexpr (FORM == 1) __syncthreads();
            __syncthreads();  // B1
            float4 cur[NQ];
            RF::unpack(ld_f4(Rm, off, 0u), cur);  // the rows after this token's writes
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const float part = rows_reduce<L>(f4_scale(w, cur[i]));
                if ((lane & 15) < L) ybuf[rw * S + CPL * (lane & 15) + 4 * i + (lane >> 4)] = part;
            }
            __syncthreads();  // B2: all partial sums are in
            float acc = 0.f;
            if (rw == 0) acc = readers_sum<NRMAX, S>(ybuf + ylane, nra);
            st_f1(acc, Ry, y_off, (uint32_t)t * dv4);
        }
    }
}

// Ring reuse: the writer of token t overwrites slot t % UR, last used by token
// t - UR; its readers (tokens up to t - UR + D) have finished once every
// wavefront passed barrier B_{t-1}, which needs t - UR + D <= t - 2, i.e.
// UR >= D + 2 (checked for every slab configuration).

template <int SL>
size_t scan_lds_bytes(const Geom& g, int cpl) {
    constexpr int UR = SlabCfg<SL>::UR, L = SL / 4;
    const int S = L * cpl;
    return (size_t)UR * g.NWW * g.G * L * 16 + (size_t)2 * nrmax<SL>() * S * 4 + (size_t)g.NWW * S * 4;
}

// Partial y of P row partitions summed in partition order: y[s, t] = sum_p yp[p, s, t].
__global__ __launch_bounds__(256) void ypart_reduce(const float4* __restrict__ yp, float4* __restrict__ y, int P,
                                                    int64_t NS, int64_t Tc, int64_t TS, int64_t dq) {
    const int64_t per_s = Tc * dq, n = NS * per_s;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t st = i / per_s, rem = i - st * per_s;
        float4 acc = yp[i];
        for (int q = 1; q < P; ++q) acc = f4_add(acc, yp[q * n + i]);
        y[st * TS * dq + rem] = acc;
    }
}

// Tokens per launch: every buffer one stream spans in a launch (plan records, v,
// y) stays below 2 GiB, so 32-bit offsets and the dropped-access offset work.
int64_t chunk_tokens(int64_t T, const Geom& g, int dv, int save_w = 0) {
    int64_t per_tok = g.rec() > (int64_t)dv * 4 ? g.rec() : (int64_t)dv * 4;
    if ((int64_t)save_w * dv * 4 > per_tok) per_tok = (int64_t)save_w * dv * 4;
    const int64_t cap = (int64_t)0x7FFFFFFF / per_tok - 4;  // room for the records' block padding
    return T < cap ? T : cap;
}

// Tokens of a launch's plan record region: rounded up to a whole block of
// entries (at most 4 tokens a block)
inline int64_t plan_tokens(int64_t Tc) { return (Tc + 3) / 4 * 4; }

// A scan configuration: slab width S, row partitions P and the wavefront layout.
struct Cfg {
    int S = 0, P = 1;
    Geom g{};
};

// Bytes of workspace one launch needs: plan records, then (P > 1) partial y.
struct WsLayout {
    int64_t plan_bytes, ypart_off, maxc_off, total;
};
WsLayout ws_layout(const Cfg& c, int64_t NS, int64_t Tc, int dv) {
    WsLayout w;
    w.plan_bytes = NS * c.P * plan_tokens(Tc) * c.g.rec();
    w.ypart_off = (w.plan_bytes + 255) / 256 * 256;
    const int64_t yend = c.P > 1 ? w.ypart_off + (int64_t)c.P * NS * Tc * dv * 4 : w.plan_bytes;
    w.maxc_off = (yend + 255) / 256 * 256;
    w.total = w.maxc_off + NS * c.P * 2 * 4;
    return w;
}

// One instance of the token-loop kernel per (slab, form, v dtype, pre-image
// stores, table dtype); pre-images are taken only of fp32 tables, and a bf16
// table never takes SL = 32 slabs in the loop (slab_fits), so neither has an
// instance.
template <int SL>
hipError_t launch_scan_inst(int form, bool vb, bool save, bool mb, dim3 grid, dim3 block, size_t lds,
                            hipStream_t st, const ScanKArgs& k) {
    const int sel = (form ? 8 : 0) | (vb ? 4 : 0) | (save ? 2 : 0) | (mb ? 1 : 0);
    if constexpr (SL == 32) {
        if (mb) return hipErrorInvalidValue;
    }
    switch (sel) {
        case 0: hipLaunchKernelGGL((scan_kernel<SL, 0, false, false, false>), grid, block, lds, st, k); break;
        case 2: hipLaunchKernelGGL((scan_kernel<SL, 0, false, true, false>), grid, block, lds, st, k); break;
        case 4: hipLaunchKernelGGL((scan_kernel<SL, 0, true, false, false>), grid, block, lds, st, k); break;
        case 6: hipLaunchKernelGGL((scan_kernel<SL, 0, true, true, false>), grid, block, lds, st, k); break;
        case 8: hipLaunchKernelGGL((scan_kernel<SL, 1, false, false, false>), grid, block, lds, st, k); break;
        case 10: hipLaunchKernelGGL((scan_kernel<SL, 1, false, true, false>), grid, block, lds, st, k); break;
        case 12: hipLaunchKernelGGL((scan_kernel<SL, 1, true, false, false>), grid, block, lds, st, k); break;
        case 14: hipLaunchKernelGGL((scan_kernel<SL, 1, true, true, false>), grid, block, lds, st, k); break;
        default:
            if constexpr (SL != 32) {
                switch (sel) {
                    case 1: hipLaunchKernelGGL((scan_kernel<SL, 0, false, false, true>), grid, block, lds, st, k); break;
                    case 5: hipLaunchKernelGGL((scan_kernel<SL, 0, true, false, true>), grid, block, lds, st, k); break;
                    case 9: hipLaunchKernelGGL((scan_kernel<SL, 1, false, false, true>), grid, block, lds, st, k); break;
                    case 13: hipLaunchKernelGGL((scan_kernel<SL, 1, true, false, true>), grid, block, lds, st, k); break;
                    default: return hipErrorInvalidValue;  // pre-images of a bf16 table: rejected by the C ABI
                }
            } else {
                return hipErrorInvalidValue;
            }
    }
    return hipSuccess;
}

// the fused output step keeps a lane's pieces of a row in registers
bool gate_fusable(int dv) { return dv / 4 <= GATE_FUSED_PIECES * output_gate_lanes(dv); }

template <int SL>
hipError_t launch_scan_slab(const ScanArgs& a, const Cfg& c, hipStream_t st) {
    constexpr int D = SlabCfg<SL>::D;
    static_assert(D <= 15, "the plan stores forward distances in 4 bits");
    const Geom& g = c.g;
    // planner: tiles of TT tokens; the hash table holds the writes of TT + D tokens
    // at load <= 1/4. With pb = ceil(log2 W) (so 2^pb < 2W), the entry ids
    // tok << pb | rank stay below (TT + D) << pb < 2 * HT_WRITES = 2^13 < 2^14, so
    // no entry equals HT_EMPTY.
    int pb = 0;
    while ((1 << pb) < a.W) ++pb;
    int psh = 0;
    while ((1 << psh) < c.P) ++psh;
    int TT = HT_WRITES / a.W - D;
    if (TT < 1) TT = 1;
    const bool save = a.snap != nullptr;
    int64_t Tc = chunk_tokens(a.T, g, a.dv, save ? a.W : 0);
    if (a.max_tokens > 0 && Tc > a.max_tokens) Tc = a.max_tokens;
    const WsLayout wl = ws_layout(c, a.NS, Tc, a.dv);
    const int cpl = a.m_bf16 ? 8 : 4;
    const int nslab = a.dv / (SL / 4 * cpl);
    const int64_t nblk = unit_grid(a.NS, (int64_t)nslab * c.P);
    const size_t lds = scan_lds_bytes<SL>(g, cpl);
    const size_t bm_bytes = (size_t)((a.N + 31) / 32) * 4;
    const int esz = a.v_bf16 ? 2 : 4;
    uint8_t* plan = static_cast<uint8_t*>(a.workspace);
    float* ypart = reinterpret_cast<float*>(plan + wl.ypart_off);
    uint32_t* maxc = reinterpret_cast<uint32_t*>(plan + wl.maxc_off);
    const int nmax = (int)(a.NS * c.P * 2);
    for (int64_t c0 = 0; c0 < a.T; c0 += Tc) {
        const int64_t Tn = a.T - c0 < Tc ? a.T - c0 : Tc;
        hipLaunchKernelGGL(zero_u32, dim3((unsigned)((nmax + 255) / 256)), dim3(256), 0, st, maxc, nmax);
        PlanArgs p{};
        p.idx_w = a.idx_w + c0 * a.W; p.wt_w = a.wt_w + c0 * a.W; p.W = a.W;
        p.idx_r = a.idx_r + c0 * a.R; p.wt_r = a.wt_r + c0 * a.R; p.R = a.R;
        p.alpha = a.alpha + c0; p.beta = a.beta + c0;
        p.plan = plan;
        p.maxc = maxc;
        p.Tc = Tn; p.TS = a.T; p.N = a.N;
        p.D = D; p.G = g.G; p.NWW = g.NWW; p.NWR = g.NWR; p.TT = TT; p.pb = pb; p.P = c.P; p.pshift = psh;
        p.ntile = (Tn + TT - 1) / TT;
        p.wpos = save && a.form == 0;
        p.form = a.form;
        p.ur = SlabCfg<SL>::UR;      // the scan kernel's ring of written rows: token slots
        p.bt = entry_batch<SL>();    // tokens per block of entries
        p.bts = p.bt == 4 ? 2 : p.bt == 2 ? 1 : 0;
        p.urm = (uint32_t)((((uint64_t)1 << 32) + (uint64_t)p.ur - 1) / (uint64_t)p.ur);
        p.tp = (Tn + p.bt - 1) / p.bt * p.bt;
        p.rpos = g.NWW * g.G;        // write positions per slot
        p.rlane = (SL / 4) * 16;     // bytes per position: 16 per lane of a row segment
        hipLaunchKernelGGL(plan_kernel, dim3((unsigned)(p.ntile * a.NS)), dim3(PLAN_THREADS), bm_bytes, st, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ScanKArgs k{};
        k.plan = plan;
        k.maxc = maxc;
        k.v = static_cast<const char*>(a.v) + c0 * a.dv * esz;
        k.M = a.M;
        if (c.P > 1) {
            k.y = ypart; k.ys = Tn * a.dv; k.yp = a.NS * Tn * a.dv;
        } else {
            k.y = a.y + c0 * a.dv; k.ys = a.T * a.dv; k.yp = 0;
        }
        k.T = (int)Tn; k.TS = a.T; k.N = a.N; k.dv = a.dv; k.nslab = nslab; k.P = c.P; k.NS = a.NS;
        k.NWW = g.NWW; k.NWR = g.NWR;
        k.W = a.W;
        k.snap = save ? a.snap + c0 * a.W * a.dv : nullptr;
        k.snap_s = a.T * a.W * a.dv;
        // per-slot form with one reader wavefront: one more wavefront adds the
        // readers' partial sums and stores y
        const int xw = (a.form == 0 && g.NWR == 1 && g.nw() < SlabCfg<SL>::NWMAX && g.NWR < nrmax<SL>()) ? 1 : 0;
        dim3 grid((unsigned)nblk), block((unsigned)((g.nw() + xw) * 64));
        e = launch_scan_inst<SL>(a.form, a.v_bf16, save, a.m_bf16, grid, block, lds, st, k);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (c.P > 1 && a.gate && gate_fusable(a.dv)) {
            YGateArgs ga{};
            ga.yp = ypart; ga.y = a.y; ga.gate = *a.gate; ga.P = c.P;
            ga.NS = a.NS; ga.Tc = Tn; ga.TS = a.T; ga.t0 = c0; ga.dv = a.dv;
            e = launch_ypart_gate(ga, st);
            if (e != hipSuccess) return e;
        } else if (c.P > 1) {
            const int64_t n4 = a.NS * Tn * (a.dv / 4);
            const int64_t nb = (n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096;
            hipLaunchKernelGGL(ypart_reduce, dim3((unsigned)nb), dim3(256), 0, st,
                               reinterpret_cast<const float4*>(ypart), reinterpret_cast<float4*>(a.y + c0 * a.dv),
                               c.P, a.NS, Tn, a.T, (int64_t)(a.dv / 4));
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <int SL>
hipError_t launch_scan_direct(const ScanArgs& a, hipStream_t st) {
    const Geom g = make_geom(SL, a.W, a.R);
    DirectArgs d{};
    d.idx_w = a.idx_w; d.wt_w = a.wt_w; d.W = a.W;
    d.idx_r = a.idx_r; d.wt_r = a.wt_r; d.R = a.R;
    d.alpha = a.alpha; d.beta = a.beta; d.v = a.v; d.M = a.M; d.y = a.y;
    d.T = (int)a.T; d.N = a.N; d.dv = a.dv; d.nslab = a.dv / (SL / 4 * (a.m_bf16 ? 8 : 4)); d.NS = a.NS;
    d.NWW = g.NWW; d.NWR = g.NWR;
    d.snap = a.snap;
    const int64_t nblk = unit_grid(a.NS, d.nslab);
    dim3 grid((unsigned)nblk), block((unsigned)(g.nw() * 64));
    const int sel = (a.form ? 8 : 0) | (a.v_bf16 ? 4 : 0) | (a.snap ? 2 : 0) | (a.m_bf16 ? 1 : 0);
    switch (sel) {
        case 0: hipLaunchKernelGGL((scan_direct_kernel<SL, 0, false, false, false>), grid, block, 0, st, d); break;
        case 1: hipLaunchKernelGGL((scan_direct_kernel<SL, 0, false, false, true>), grid, block, 0, st, d); break;
        case 2: hipLaunchKernelGGL((scan_direct_kernel<SL, 0, false, true, false>), grid, block, 0, st, d); break;
        case 4: hipLaunchKernelGGL((scan_direct_kernel<SL, 0, true, false, false>), grid, block, 0, st, d); break;
        case 5: hipLaunchKernelGGL((scan_direct_kernel<SL, 0, true, false, true>), grid, block, 0, st, d); break;
        case 6: hipLaunchKernelGGL((scan_direct_kernel<SL, 0, true, true, false>), grid, block, 0, st, d); break;
        case 8: hipLaunchKernelGGL((scan_direct_kernel<SL, 1, false, false, false>), grid, block, 0, st, d); break;
        case 9: hipLaunchKernelGGL((scan_direct_kernel<SL, 1, false, false, true>), grid, block, 0, st, d); break;
        case 10: hipLaunchKernelGGL((scan_direct_kernel<SL, 1, false, true, false>), grid, block, 0, st, d); break;
        case 12: hipLaunchKernelGGL((scan_direct_kernel<SL, 1, true, false, false>), grid, block, 0, st, d); break;
        case 13: hipLaunchKernelGGL((scan_direct_kernel<SL, 1, true, false, true>), grid, block, 0, st, d); break;
        case 14: hipLaunchKernelGGL((scan_direct_kernel<SL, 1, true, true, false>), grid, block, 0, st, d); break;
        default: return hipErrorInvalidValue;  // pre-images of a bf16 table: rejected by the C ABI
    }
    return hipGetLastError();
}

// Slab widths are named by SL = 4 * (lanes per row segment), which fixes the
// wavefront layout (G = 64 / (SL / 4) rows per wavefront) and the plan
// records; a slab holds SL columns of an fp32 table and 2 * SL of a bf16 one
// (cpl = 4 or 8 columns per 16-byte lane).
int slab_nwmax(int S) {
    return S == 32 ? SlabCfg<32>::NWMAX : S == 16 ? SlabCfg<16>::NWMAX : S == 8 ? SlabCfg<8>::NWMAX : SlabCfg<4>::NWMAX;
}
int slab_nrmax(int S) {
    return S == 32 ? nrmax<32>() : S == 16 ? nrmax<16>() : S == 8 ? nrmax<8>() : nrmax<4>();
}
// LDS of one workgroup of the prefetching loop (its ring grows with W)
size_t slab_lds(int S, const Geom& g, int cpl) {
    return S == 32 ? scan_lds_bytes<32>(g, cpl) : S == 16 ? scan_lds_bytes<16>(g, cpl)
         : S == 8 ? scan_lds_bytes<8>(g, cpl) : scan_lds_bytes<4>(g, cpl);
}
constexpr size_t LDS_MAX = 160 * 1024;  // per workgroup on gfx950

// The token loop does not take a bf16 table in SL = 32 slabs (64 columns): with
// its two float4 of widened values per row it needs more than the 128 VGPRs of
// a 16-wavefront workgroup and spills; such tables take narrower slabs there.
// The direct form (loop = false) keeps them.
bool slab_fits(int S, int W, int R, int dv, int cpl, bool loop = true) {
    if (dv % (S / 4 * cpl) != 0) return false;
    if (loop && S == 32 && cpl == 8) return false;
    const Geom g = make_geom(S, W, R);
    return g.nw() <= slab_nwmax(S) && g.NWR <= slab_nrmax(S) && slab_lds(S, g, cpl) <= LDS_MAX;
}

int env_int(const char* name) {
    const char* e = getenv(name);
    return e ? atoi(e) : 0;
}

// Slab width without row partitions: among the widths whose groups of G rows
// tile W and R without padding and that need at most 8 wavefronts (the
// 16-wavefront form has a shallower pipeline), the widest one that still gives
// at least 128 workgroups (half the CUs; 256 for a bf16 table): wider slabs
// move longer row segments, narrower ones give more independent workgroups.
// Failing that, the width with the most workgroups, then the one with the least
// padding. (Measured on the N=65536, W=R=64, d_v=128 shapes: fp32, 32 streams
// -> 16 columns, 8 streams -> 8; bf16, 32 streams -> 16 columns (SL = 8).)
int pick_slab(int64_t NS, int W, int R, int dv, int cpl, int forced, bool loop = true) {
    const long enough = cpl == 8 ? 256 : 128;
    // fp32 table, few streams: the 8-wavefront 16-column layout and its deeper
    // prefetch (one stream, W = R = 8, d_v = 512, shared-residual form: 19.8 ms
    // against 35.3 for 32-column slabs)
    if (!forced && cpl == 4 && (long)NS * (dv / 32) < enough && slab_fits(16, W, R, dv, cpl, loop)) return 16;
    struct Cand {
        int S;
        long waste, units;
        int nw;
    };
    auto better = [enough](const Cand& a, const Cand& b) {
        if ((a.waste == 0) != (b.waste == 0)) return a.waste == 0;
        if ((a.nw <= 8) != (b.nw <= 8)) return a.nw <= 8;
        const bool ea = a.units >= enough, eb = b.units >= enough;
        if (ea != eb) return ea;
        if (ea) return a.S > b.S;
        if (a.units != b.units) return a.units > b.units;
        return a.waste < b.waste;
    };
    Cand best{0, 0, 0, 0};
    for (int S : {32, 16, 8, 4}) {
        if ((forced && forced != S) || !slab_fits(S, W, R, dv, cpl, loop)) continue;
        const Geom g = make_geom(S, W, R);
        const Cand c{S, (long)g.NWW * g.G - W + (long)g.NWR * g.G - R, (long)NS * (dv / (S / 4 * cpl)), g.nw()};
        if (best.S == 0 || better(c, best)) best = c;
    }
    return best.S;
}

// The per-slot form (EQ4) never couples two rows, so it may split the rows into
// partitions, each walked by its own workgroups. With an fp32 table it takes
// whole 128-byte lines (32-column slabs) when at most 2 partitions give 256
// workgroups (many streams: the per-CU line misses in flight bound the scan,
// and a line that carries 128 useful bytes is worth more than the padding
// lanes of a partitioned record), else 16-column slabs (the 8-wavefront layout
// with its deeper prefetch) and the smallest power-of-two P <= 4 towards 256
// workgroups: with few streams the per-token chain of a workgroup bounds the
// loop. Measured on MI355X, scan call in ms (32-col/P against 16-col/P):
// 32 streams, W=R=64, d_v=128: 5.56 (32/2) against 6.70 (16/1); 8 streams x
// 131072 tokens: 39.5 (32/8) against 38.2 (16/4); one stream, W=R=8, d_v=512:
// 29.1 (32/8) against 11.3 (16/4); 16 streams, W=R=16, d_v=64: 2.11 (32/8)
// against 0.94 (16/4). The shared-residual form (FIG2) couples all rows of a
// token and keeps P = 1.
// A bf16 table halves the bytes of every access, so its loop is bound by the
// per-token work of a workgroup rather than by line misses: there the 8-wavefront
// layouts with their deeper prefetch win. Measured (N=65536, W=R=64, d_v=128):
// 32 streams -> 32-column slabs (SL = 16), P = 2 (3.9 ms against 4.4 for whole
// lines at P = 4); 8 streams -> 16-column slabs (SL = 8), P = 8 (512 workgroups:
// 41 ms against 51 at 256).
// SDM_SCAN_SLAB (an SL value) and SDM_SCAN_PARTS force a width and a partition count.
Cfg choose_cfg(int64_t NS, int W, int R, int dv, int form, int cpl) {
    Cfg c;
    const int fs = env_int("SDM_SCAN_SLAB"), fp = env_int("SDM_SCAN_PARTS");
    const int64_t ns = NS > 0 ? NS : 1;
    int want = 256;  // workgroups the partitions should reach
    int pcap = MAX_PARTS;
    if (form == 0 && cpl == 4 && fs == 0 && slab_fits(32, W, R, dv, cpl) && ns * (dv / 32) * 2 >= 256) {
        c.S = 32;
    } else if (form == 0 && cpl == 4 && fs == 0 && slab_fits(16, W, R, dv, cpl)) {
        c.S = 16;
        pcap = 4;
    } else if (form == 0 && cpl == 8 && fs == 0 && slab_fits(16, W, R, dv, cpl) && slab_fits(8, W, R, dv, cpl)) {
        const bool many = ns * (dv / 32) >= 128;
        c.S = many ? 16 : 8;
        want = many ? 256 : 512;
    } else {
        c.S = pick_slab(NS, W, R, dv, cpl, fs);
        if (c.S == 0) return c;
    }
    if (form == 0) {
        if (fp == 1 || fp == 2 || fp == 4 || fp == 8) {
            c.P = fp;
        } else {
            const int64_t units = ns * (dv / (c.S / 4 * cpl));
            while (c.P < pcap && units * c.P < want) c.P *= 2;
        }
    }
    c.g = make_geom(c.S, W, R);
    return c;
}

}  // namespace

bool scan_geometry(int64_t NS, int W, int R, int dv, bool m_bf16, int* slab, int* rec) {
    const int cpl = m_bf16 ? 8 : 4;
    for (int form = 0; form < 2; ++form)
        if (choose_cfg(NS, W, R, dv, form, cpl).S == 0) return false;
    const Cfg c = choose_cfg(NS, W, R, dv, 0, cpl);
    if (slab) *slab = c.S;
    if (rec) *rec = (int)c.g.rec();
    return true;
}

// The workspace covers both forms and both table dtypes (where a dtype's
// slabs fit dv), so one size serves every call with these sizes.
int64_t scan_workspace_bytes(int64_t NS, int64_t T, int W, int R, int dv) {
    int64_t need = 0;
    for (int cpl : {4, 8}) {
        if (cpl == 8 && dv % 8 != 0) continue;
        for (int form = 0; form < 2; ++form) {
            const Cfg c = choose_cfg(NS, W, R, dv, form, cpl);
            if (c.S == 0) {
                if (cpl == 4) return -1;
                continue;
            }
            const int64_t b = ws_layout(c, NS, chunk_tokens(T, c.g, dv), dv).total;
            if (b > need) need = b;
        }
    }
    return need;
}

// Calls of at most this many tokens take the direct form (SDM_SCAN_DIRECT_T
// overrides; 0 turns it off).
int64_t direct_max_tokens() {
    const char* e = getenv("SDM_SCAN_DIRECT_T");
    return e ? atoll(e) : 8;
}

int64_t scan_tokens_within(int64_t NS, int64_t T, int W, int R, int dv, bool m_bf16, int form, int64_t bytes) {
    if (T <= direct_max_tokens()) return T;  // the short-call form needs no workspace
    const Cfg c = choose_cfg(NS, W, R, dv, form, m_bf16 ? 8 : 4);
    if (c.S == 0) return 0;
    const int64_t cap = chunk_tokens(T, c.g, dv);
    auto fits = [&](int64_t tc) { return ws_layout(c, NS, tc, dv).total <= bytes; };
    if (!fits(1)) return 0;
    int64_t lo = 1, hi = cap;  // fits(lo); the answer lies in [lo, hi]
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (fits(mid)) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

bool scan_fuses_gate(int64_t NS, int64_t T, int W, int R, int dv, bool m_bf16, int form) {
    const int cpl = m_bf16 ? 8 : 4;
    if (T <= direct_max_tokens() && T * (int64_t)dv * 4 < 0x7FFFFFFF &&
        pick_slab(NS, W, R, dv, cpl, env_int("SDM_SCAN_SLAB"), false) != 0)
        return false;  // the short-call form: no partial sums
    return choose_cfg(NS, W, R, dv, form, cpl).P > 1 && gate_fusable(dv);
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    const int cpl = a.m_bf16 ? 8 : 4;
    const int64_t per_tok = (int64_t)a.dv * 4 * (a.snap ? (a.W > 1 ? a.W : 1) : 1);
    if (a.T <= direct_max_tokens() && a.T * per_tok < 0x7FFFFFFF) {
        switch (pick_slab(a.NS, a.W, a.R, a.dv, cpl, env_int("SDM_SCAN_SLAB"), false)) {
            case 32: return launch_scan_direct<32>(a, st);
            case 16: return launch_scan_direct<16>(a, st);
            case 8: return launch_scan_direct<8>(a, st);
            case 4: return launch_scan_direct<4>(a, st);
            default: break;
        }
    }
    const Cfg c = choose_cfg(a.NS, a.W, a.R, a.dv, a.form, cpl);
    switch (c.S) {
        case 32: return launch_scan_slab<32>(a, c, st);
        case 16: return launch_scan_slab<16>(a, c, st);
        case 8: return launch_scan_slab<8>(a, c, st);
        case 4: return launch_scan_slab<4>(a, c, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdm
