// address.hip -- product-key addressing of the SDM layer on gfx950.
//
// What it computes ("Sparse Delta Memory：中文精读笔记" §2.3; "Fast-weight
// Product Key Memory：中文精读笔记" §2.2): per token and branch, the two
// half-queries are scored against the sqrt(N) subkeys of their half, each half
// keeps its best k_h = min(k, n) sub-scores, the outer sums of the kept pairs
// are the candidate slot scores (slot (a, b) = row a*n + b), the k best
// candidates are selected and weighted by a softmax over their scores.
// Ties go to the lower index (sub-index per half, slot index at the end).
//
// Design (one workgroup of NWA = 8 wavefronts per 16 tokens of one (b, h, branch)):
//   a1  half-scores: a [16 tokens x d_h] x [d_h x 16 subkeys] MFMA tile per
//       step (v_mfma_f32_16x16x32_bf16 for bf16 inputs, 16x16x4 f32 for fp32),
//       fp32 accumulation, staged in LDS as [token][half][subkey].
//   a2  per-half top-k_h: the scores become order-preserving 32-bit keys; a
//       wave-wide radix select (one ballot per bit and element) finds the k_h-th
//       key, ties at the threshold are cut by a second radix pass over the
//       (inverted) index; winners are compacted with mbcnt and sorted by a
//       64-lane bitonic network on (key, ~index).
//   a3  combine: only pairs of sorted ranks (i, j) with (i+1)(j+1) <= k can be
//       among the k best (each such pair is dominated by the (i+1)(j+1)-1 pairs
//       of better ranks, since fp32 rounding is monotone), so at most 280
//       candidates for k = 64 instead of k^2. The same select + sort picks the k
//       winners. Exactness certificate: the best pruned pair of each rank row
//       is its first pruned one; if any of those scores is >= the k-th winner's
//       score (a tie that the slot order could decide differently), the token
//       is redone over the full k_h x k_h grid.
//   a4  softmax in fp32 (max-subtracted, expf), butterfly sum.
// Inverse-distance scores ("Fast-weight Product Key Memory：中文精读笔记" §2.2,
// FwPKM's default): s = -log(1e-3 + ||q - K_a||^2). The squared distance is
// ||q||^2 + ||K_a||^2 - 2 <q, K_a>, so the contraction stays on MFMA; each lane
// also sums the squares of the q and subkey elements it loads for the MFMA, a
// 4-lane butterfly completes the norms, and the epilogue of a1 turns the dot
// products into scores. Everything after a1 is the same for both scorings.
// The wavefronts share the MFMA tiles of a1; then each selects TG = 2 tokens.
// The selection is a chain of dependent wave-wide steps, so the 2 tokens are
// carried through it together (independent chains interleave), and every
// cross-lane exchange uses DPP or the gfx950 permlane swaps instead of LDS.
// A wavefront reuses the LDS block of its own scores for its sorted lists, so a
// workgroup needs ~33 KB (n = 256) and four fit a CU: eight wavefronts per
// SIMD, whose scalar (ballot/popcount) and vector work overlap. (Measured at
// n = 256, k = 64: 2 tokens per wavefront beat 1, 4 and 8.)
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int TOK = 16;       // tokens per workgroup = one MFMA M tile
constexpr int TG = 2;         // tokens selected together by one wavefront
constexpr int NWA = TOK / TG; // wavefronts per workgroup
constexpr int EC = 5;         // candidate chunks per lane: sum_{i<=64} floor(64/i) = 280 <= 320

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ uint32_t ord_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Value of lane (lane ^ M), without LDS: DPP quad permutes (1, 2), DPP
// half-row mirror + quad permute (4), DPP row rotate (8), gfx950 permlane
// swaps (16, 32).
template <int M>
__device__ __forceinline__ uint32_t xlane(uint32_t x, int lane) {
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    } else if constexpr (M == 4) {
        // lane ^ 4 = (lane ^ 7) ^ 3: row_half_mirror, then quad_perm 3,2,1,0
        const int m = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);
    } else if constexpr (M == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (M == 16) {
        auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? p[0] : p[1];
    } else {
        auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? p[0] : p[1];
    }
}

template <int M>
__device__ __forceinline__ uint64_t xlane64(uint64_t x, int lane) {
    return ((uint64_t)xlane<M>((uint32_t)(x >> 32), lane) << 32) | xlane<M>((uint32_t)x, lane);
}

template <int M>
__device__ __forceinline__ float xlanef(float x, int lane) {
    return __uint_as_float(xlane<M>(__float_as_uint(x), lane));
}

__device__ __forceinline__ float wave_sum(float v, int lane) {
    v += xlanef<32>(v, lane);
    v += xlanef<16>(v, lane);
    v += xlanef<8>(v, lane);
    v += xlanef<4>(v, lane);
    v += xlanef<2>(v, lane);
    v += xlanef<1>(v, lane);
    return v;  // the butterfly adds the same pairs on every lane: identical on all lanes
}

// Select output rows: OSTR words per token-chain; a winner goes to one of the
// first k words, every other lane stores to word OSTR / 2 + lane (unused), so
// the compaction stores need no lane mask.
constexpr int OSTR = 128;

// f(e) for e < NCH (compile-time, unrolled) or e < nch (run time).
template <int NCH, typename F>
__device__ __forceinline__ void for_chunks(int nch, F f) {
    if constexpr (NCH > 0) {
#pragma unroll
        for (int e = 0; e < NCH; ++e) f(e);
    } else {
        for (int e = 0; e < nch; ++e) f(e);
    }
}

// Select, for each of the NT token-chains g, the k best candidates (larger key
// first, then smaller id) among candidates c = e*64 + lane, e < nch, read
// through get(g, e, key, id). Key 0 marks an absent candidate; ids are below
// 2^18. Exactly k winners (k <= number of present candidates) are written in
// candidate order to okey/oid[g*OSTR + 0..k).
// tau0 / b0 (optional): bits of the k-th key known before the search — for
// each token, its bits above some position equal tau0[g]'s (and tau0[g]'s lower
// bits are 0); b0 is one bit at or above every token's first unknown bit. The
// walk then starts at b0. (Walking a token's known bits again changes nothing:
// a known 1 is taken at once, a known 0 would leave fewer than k keys.)
template <int NT, int NCH, typename Get>
__device__ __forceinline__ void wave_select(Get get, int nch_rt, int k, uint32_t* okey, uint32_t* oid,
                                            int lane, const uint32_t* tau0 = nullptr,
                                            uint32_t b0 = 0x80000000u) {
    // Radix select of the k-th largest key, most significant bit first: tau
    // keeps the bits fixed so far, cur = count(key >= tau) >= k. A bit is taken
    // when the count at tau with the bit set still reaches k. Once cur == k the
    // winners are the keys at or above tau, and taking further bits keeps
    // exactly those k keys at or above it (a bit is only taken while the count
    // stays >= k, and it cannot exceed cur), so a finished token needs no
    // branch of its own; the loop ends when every token has cur == k (with
    // distinct keys, once the prefix separates the k-th from the (k+1)-th key).
    uint32_t tau[NT];
    int cur[NT];
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        tau[g] = tau0 ? tau0[g] : 0u;
        cur[g] = -1;  // unknown, >= k
    }
    for (uint32_t b = b0; b != 0u; b >>= 1) {
        int cnt[NT];
        uint32_t t[NT];
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            cnt[g] = 0;
            t[g] = tau[g] | b;
        }
        for_chunks<NCH>(nch_rt, [&](int e) {
#pragma unroll
            for (int g = 0; g < NT; ++g) {
                uint32_t kk, ii;
                get(g, e, kk, ii);
                cnt[g] += popc(__ballot(kk >= t[g]));
            }
        });
        uint32_t left = 0u;
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            const bool take = cnt[g] >= k;
            tau[g] = take ? t[g] : tau[g];
            cur[g] = take ? cnt[g] : cur[g];
            left |= (uint32_t)(cur[g] ^ k);
        }
        if (left == 0u) break;
    }
    uint32_t open = 0u;
#pragma unroll
    for (int g = 0; g < NT; ++g) open |= (cur[g] != k ? 1u : 0u) << g;
    // compaction: the winners are the keys at or above tau (with cut: of the
    // keys equal to tau, those whose inverted id reaches sig)
    auto compact = [&](const uint32_t (&th)[NT], uint32_t cutm, const uint32_t (&sig)[NT]) {
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            const bool cut = (cutm >> g) & 1u;
            int base = 0;
            for_chunks<NCH>(nch_rt, [&](int e) {
                uint32_t kk, ii;
                get(g, e, kk, ii);
                const bool sel = kk > th[g] || (kk == th[g] && (!cut || (0x3FFFFu - ii) >= sig[g]));
                const uint64_t m = __ballot(sel);
                const int pos = sel ? base + lanes_below(m) : OSTR / 2 + lane;
                okey[g * OSTR + pos] = kk;
                oid[g * OSTR + pos] = ii;
                base += popc(m);
            });
        }
    };
    if (open != 0u) {
        // Rare: a token went through bit 0, so its tau is the k-th key itself,
        // and more keys may equal it than places are left (exact ties): those
        // keep the lowest ids, by a second radix pass over the inverted id.
        // The thresholds pass through readfirstlane (a no-op on a uniform
        // value) so that none of this path's compares is hoisted into the
        // common one.
        uint32_t th[NT], sig[NT], cutm = 0u;
        int need[NT];
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            th[g] = (uint32_t)__builtin_amdgcn_readfirstlane((int)tau[g]);
            sig[g] = 0u;
            int gt = 0, eq = 0;
            for_chunks<NCH>(nch_rt, [&](int e) {
                uint32_t kk, ii;
                get(g, e, kk, ii);
                gt += popc(__ballot(kk > th[g]));
                eq += popc(__ballot(kk == th[g]));
            });
            need[g] = k - gt;
            if (((open >> g) & 1u) && eq > need[g]) cutm |= 1u << g;
        }
        if (cutm != 0u) {
            for (int bit = 17; bit >= 0; --bit) {
                int cnt[NT];
#pragma unroll
                for (int g = 0; g < NT; ++g) cnt[g] = 0;
                for_chunks<NCH>(nch_rt, [&](int e) {
#pragma unroll
                    for (int g = 0; g < NT; ++g) {
                        uint32_t kk, ii;
                        get(g, e, kk, ii);
                        cnt[g] += popc(__ballot(kk == th[g] && (0x3FFFFu - ii) >= (sig[g] | (1u << bit))));
                    }
                });
#pragma unroll
                for (int g = 0; g < NT; ++g)
                    if (cnt[g] >= need[g]) sig[g] |= 1u << bit;
            }
        }
        compact(th, cutm, sig);
        return;
    }
    const uint32_t nosig[NT] = {};
    compact(tau, 0u, nosig);
}

// Lanes of a bitonic stage (partner distance J, merge size K) that keep the
// smaller of the pair: bit l of the mask. A compile-time constant, so each
// stage applies it to the compare mask with two scalar XORs on literals.
template <int J, int K>
constexpr uint64_t keep_min_lanes() {
    uint64_t m = 0;
    for (int l = 0; l < 64; ++l)
        if (((l & J) == 0) != ((l & K) == 0)) m |= 1ull << l;
    return m;
}

template <int J, int K, int NT>
__device__ __forceinline__ void sort_stage(uint64_t (&x)[NT], int lane) {
    constexpr uint64_t KMIN = keep_min_lanes<J, K>();
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        // keep the larger of (x, partner) where the lane keeps the maximum, the
        // smaller elsewhere: one compare, one scalar mask operation, one select
        if constexpr (J >= 16) {
            // a permlane swap of (v, v) returns {v, partner's v} in an order that
            // depends only on the lane half, the same order for both words; max
            // and min of the pair are then the same on both lanes
            const uint32_t lo = (uint32_t)x[g], hi = (uint32_t)(x[g] >> 32);
            uint32_t l0, l1, h0, h1;
            if constexpr (J == 16) {
                const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
                const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
                l0 = pl[0]; l1 = pl[1]; h0 = ph[0]; h1 = ph[1];
            } else {
                const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
                const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
                l0 = pl[0]; l1 = pl[1]; h0 = ph[0]; h1 = ph[1];
            }
            const uint64_t a0 = ((uint64_t)h0 << 32) | l0, a1 = ((uint64_t)h1 << 32) | l1;
            const bool take0 = __builtin_amdgcn_inverse_ballot_w64(__ballot(a0 > a1) ^ KMIN);
            x[g] = take0 ? a0 : a1;
        } else {
            const uint64_t o = xlane64<J>(x[g], lane);
            const bool keep = __builtin_amdgcn_inverse_ballot_w64(__ballot(x[g] > o) ^ KMIN);
            x[g] = keep ? x[g] : o;
        }
    }
}

// Bitonic sort across the 64 lanes, one 64-bit key per lane, descending, for
// NT independent sequences at once.
template <int NT>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&x)[NT], int lane) {
    sort_stage<1, 2>(x, lane);
    sort_stage<2, 4>(x, lane); sort_stage<1, 4>(x, lane);
    sort_stage<4, 8>(x, lane); sort_stage<2, 8>(x, lane); sort_stage<1, 8>(x, lane);
    sort_stage<8, 16>(x, lane); sort_stage<4, 16>(x, lane); sort_stage<2, 16>(x, lane);
    sort_stage<1, 16>(x, lane);
    sort_stage<16, 32>(x, lane); sort_stage<8, 32>(x, lane); sort_stage<4, 32>(x, lane);
    sort_stage<2, 32>(x, lane); sort_stage<1, 32>(x, lane);
    sort_stage<32, 64>(x, lane); sort_stage<16, 64>(x, lane); sort_stage<8, 64>(x, lane);
    sort_stage<4, 64>(x, lane); sort_stage<2, 64>(x, lane); sort_stage<1, 64>(x, lane);
}

// The same network on one 32-bit word per lane.
template <int J, int K, int NT>
__device__ __forceinline__ void sort_stage32(uint32_t (&x)[NT], int lane) {
    constexpr uint64_t KMIN = keep_min_lanes<J, K>();
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        if constexpr (J >= 16) {
            uint32_t a0, a1;
            if constexpr (J == 16) {
                const auto p = __builtin_amdgcn_permlane16_swap(x[g], x[g], false, false);
                a0 = p[0]; a1 = p[1];
            } else {
                const auto p = __builtin_amdgcn_permlane32_swap(x[g], x[g], false, false);
                a0 = p[0]; a1 = p[1];
            }
            const bool take0 = __builtin_amdgcn_inverse_ballot_w64(__ballot(a0 > a1) ^ KMIN);
            x[g] = take0 ? a0 : a1;
        } else {
            const uint32_t o = xlane<J>(x[g], lane);
            const bool keep = __builtin_amdgcn_inverse_ballot_w64(__ballot(x[g] > o) ^ KMIN);
            x[g] = keep ? x[g] : o;
        }
    }
}

template <int NT>
__device__ __forceinline__ void wave_sort_desc32(uint32_t (&x)[NT], int lane) {
    sort_stage32<1, 2>(x, lane);
    sort_stage32<2, 4>(x, lane); sort_stage32<1, 4>(x, lane);
    sort_stage32<4, 8>(x, lane); sort_stage32<2, 8>(x, lane); sort_stage32<1, 8>(x, lane);
    sort_stage32<8, 16>(x, lane); sort_stage32<4, 16>(x, lane); sort_stage32<2, 16>(x, lane);
    sort_stage32<1, 16>(x, lane);
    sort_stage32<16, 32>(x, lane); sort_stage32<8, 32>(x, lane); sort_stage32<4, 32>(x, lane);
    sort_stage32<2, 32>(x, lane); sort_stage32<1, 32>(x, lane);
    sort_stage32<32, 64>(x, lane); sort_stage32<16, 64>(x, lane); sort_stage32<8, 64>(x, lane);
    sort_stage32<4, 64>(x, lane); sort_stage32<2, 64>(x, lane); sort_stage32<1, 64>(x, lane);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t id) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

// The k winners of a select (okey/oid rows, in candidate order) sorted by (key
// desc, id asc) into x[g] (composite words, lanes >= k zero). A 32-bit network
// sorts the keys with their low 6 bits replaced by 63 - (candidate position):
// that orders every pair whose keys differ above those bits, and equal
// truncated keys by position. The full (key, id) words, gathered by position,
// are then checked to be strictly descending over the lanes; a token where some
// neighbours are not (keys equal in their top 26 bits but not below, or equal
// keys whose ids run against the candidate order) is sorted again with the
// 64-bit network.
template <int NT>
__device__ __forceinline__ void sort_winners(uint64_t (&x)[NT], const uint32_t* okey, const uint32_t* oid, int k,
                                             int lane) {
    uint32_t v[NT];
#pragma unroll
    for (int g = 0; g < NT; ++g) v[g] = lane < k ? (okey[g * OSTR + lane] & ~63u) | (63u - (uint32_t)lane) : 0u;
    wave_sort_desc32<NT>(v, lane);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        const uint32_t p = 63u - (v[g] & 63u);
        x[g] = lane < k ? composite(okey[g * OSTR + p], oid[g * OSTR + p]) : 0ull;
        // lane - 1's word (DPP wave shift right by one; lane 0 keeps its own)
        const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)x[g], (int)(uint32_t)x[g], 0x138,
                                                                   0xF, 0xF, false);
        const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(x[g] >> 32),
                                                                   (int)(uint32_t)(x[g] >> 32), 0x138, 0xF, 0xF,
                                                                   false);
        const uint64_t prev = ((uint64_t)phi << 32) | plo;
        if (__ballot(lane >= 1 && lane < k && !(prev > x[g])) != 0ull) {
            uint64_t y1[1] = {lane < k ? composite(okey[g * OSTR + lane], oid[g * OSTR + lane]) : 0ull};
            wave_sort_desc<1>(y1, lane);
            x[g] = y1[0];
        }
    }
}

// Floats per wavefront block of LDS: the half-scores of TG tokens or the sorted
// lists + select buffers, whichever is larger.
__host__ __device__ inline int block_floats(int n) {
    const int scores = TG * 2 * n, lists = TG * (128 * 2 + OSTR * 2);
    return scores > lists ? scores : lists;
}


// Sum of squares of the 8 bf16 (packed in a uint4) or 2 fp32 elements a lane loads.
__device__ __forceinline__ float sumsq(const uint4& x) {
    float s = 0.f;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}
__device__ __forceinline__ float sumsq(const float2& x) { return fmaf(x.y, x.y, x.x * x.x); }

constexpr float IDW_EPS = 1e-3f;  // the constant FwPKM adds to the squared distance

// Up to n = 256: 8 wavefronts per SIMD (four workgroups per CU). The selection
// is bound by instruction issue, and more wavefronts keep both issue ports
// busier (gdn_matched 1.18 -> 1.11 ms against the register budget of 6 per
// SIMD). At n = 512 the contraction (d_h up to 256, 8 tiles a wavefront) takes
// most of the time and keeps all its tiles in flight instead (large_table:
// 2.24 ms, against 3.57 ms with tiles in groups of 2 for 8 per SIMD).
template <bool BF16, int EH, bool IDW>
__global__ __launch_bounds__(NWA * 64) __attribute__((amdgpu_waves_per_eu(EH <= 4 ? 8 : 1))) void address_kernel(AddressArgs a) {
    extern __shared__ __align__(16) uint32_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = a.n, dh = a.dh;
    // A tile is TOK consecutive tokens of one head in (sequence, position)
    // order, u = b * T + t: within a sequence for long calls, across sequences
    // when a call carries few tokens per sequence (decoding). Every token of a
    // tile uses the same subkeys.
    // token numbers u = b * T + t stay below 2^32 (checked by the C ABI), so
    // the tile and row arithmetic is 32-bit (64-bit division is a long
    // software sequence on the GPU)
    const int64_t UT = a.B * a.T;
    const uint32_t ntile = (uint32_t)((UT + TOK - 1) / TOK), T32 = (uint32_t)a.T;
    const int h = (int)(blockIdx.x / ntile);
    const int64_t u0 = (int64_t)(blockIdx.x - (uint32_t)h * ntile) * TOK;
    const int br = blockIdx.y;
    auto row_of = [&](int64_t u) -> int64_t {  // row of token u in the [B, H, T] layout
        const uint32_t uu = (uint32_t)u, b = uu / T32;
        return ((int64_t)b * a.H + h) * a.T + (uu - b * T32);
    };

    // LDS: one block of pw floats per wavefront, then the pruned rank pairs. A
    // block first holds the half-scores [TG][2][n] of the wavefront's tokens;
    // once the wavefront has them in registers it reuses the block for its
    // sorted half lists and select buffers, so a workgroup needs little more
    // than its score tile and four workgroups fit a CU.
    const int pw = block_floats(n);
    float* smf = reinterpret_cast<float*>(smem);
    auto sc_tok = [&](int m) -> float* {  // [2][n]
        return smf + __umul24((uint32_t)(m / TG), (uint32_t)pw) + __umul24((uint32_t)(m % TG), (uint32_t)(2 * n));
    };
    uint32_t* pairs = reinterpret_cast<uint32_t*>(smf + NWA * pw);  // [EC*64] pruned rank pairs
    float* ls = smf + wave * pw;                      // [TG][2][64] sorted half scores
    uint32_t* lid = reinterpret_cast<uint32_t*>(ls + TG * 128);  // [TG][2][64] their sub-indices
    uint32_t* bkey = lid + TG * 128;                  // [TG][OSTR] select output
    uint32_t* bid = bkey + TG * OSTR;                 // [TG][OSTR]

    // ---------------- a1: half-scores on MFMA ----------------
    // The 2 * n/16 subkey tiles are dealt round-robin to the wavefronts. A
    // wavefront takes its tiles in groups of TPG: for each k-step it loads its
    // tokens' half-queries and the subkeys of the group's tiles together, so the
    // loads of a step are in flight at once; up to n = 256, groups of 2 keep the
    // accumulators and subkey registers of only 2 tiles live, which keeps the
    // kernel within the 64 VGPRs of 8 wavefronts per SIMD.
    constexpr int TPW = (2 * (64 * EH / 16) + NWA - 1) / NWA;  // most tiles per wavefront
    constexpr int TPG = EH > 4 || TPW < 2 ? TPW : 2;           // tiles per group
    const int nt16 = n / 16, ntiles = 2 * nt16;
    const int m16 = lane & 15, g4 = lane >> 4;
    const int64_t tq = u0 + m16;
    const bool tok_ok = tq < UT;
    const int64_t qrow = row_of(tok_ok ? tq : 0) * 2 * dh;  // half 0; half 1 follows
#pragma unroll
    for (int grp = 0; grp < TPW; grp += TPG) {  // tiles past ntiles are skipped inside
        f32x4_t acc[TPG];
        float qsq[2] = {0.f, 0.f}, ksq[TPG];  // IDW: partial squared norms of what this lane loads
        uint32_t krow[TPG];  // element offset of this lane's subkey row of each tile within the head's table
#pragma unroll
        for (int i = 0; i < TPG; ++i) {
            acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ksq[i] = 0.f;
            const int tile = wave + (grp + i) * NWA, j = tile / nt16, a0 = (tile % nt16) * 16;
            krow[i] = (uint32_t)((j * n + a0 + m16) * dh);  // < 2 * 512 * 256
        }
        if constexpr (BF16) {
            const uint16_t* q = static_cast<const uint16_t*>(a.q[br]) + qrow;
            const uint16_t* kp = static_cast<const uint16_t*>(a.K[br]) + (int64_t)h * 2 * n * dh;  // this head's
            for (int c0 = 0; c0 < dh; c0 += 32) {
                uint4 qa[2], kb[TPG];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    qa[jj] = tok_ok ? *reinterpret_cast<const uint4*>(q + jj * dh + c0 + g4 * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int i = 0; i < TPG; ++i)
                    if (wave + (grp + i) * NWA < ntiles)
                        kb[i] = *reinterpret_cast<const uint4*>(kp + krow[i] + c0 + g4 * 8);
                if constexpr (IDW) {
                    qsq[0] += sumsq(qa[0]);
                    qsq[1] += sumsq(qa[1]);
#pragma unroll
                    for (int i = 0; i < TPG; ++i)
                        if (wave + (grp + i) * NWA < ntiles) ksq[i] += sumsq(kb[i]);
                }
#pragma unroll
                for (int i = 0; i < TPG; ++i) {
                    const int tile = wave + (grp + i) * NWA;
                    if (tile < ntiles)
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, tile < nt16 ? qa[0] : qa[1]),
                            __builtin_bit_cast(bf16x8_t, kb[i]), acc[i], 0, 0, 0);
                }
            }
        } else {
            const float* q = static_cast<const float*>(a.q[br]) + qrow;
            const float* kp = static_cast<const float*>(a.K[br]) + (int64_t)h * 2 * n * dh;  // this head's table
            for (int c0 = 0; c0 < dh; c0 += 8) {
                float2 qa[2], kb[TPG];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    qa[jj] = tok_ok ? *reinterpret_cast<const float2*>(q + jj * dh + c0 + g4 * 2)
                                    : make_float2(0.f, 0.f);
#pragma unroll
                for (int i = 0; i < TPG; ++i)
                    if (wave + (grp + i) * NWA < ntiles)
                        kb[i] = *reinterpret_cast<const float2*>(kp + krow[i] + c0 + g4 * 2);
                if constexpr (IDW) {
                    qsq[0] += sumsq(qa[0]);
                    qsq[1] += sumsq(qa[1]);
#pragma unroll
                    for (int i = 0; i < TPG; ++i)
                        if (wave + (grp + i) * NWA < ntiles) ksq[i] += sumsq(kb[i]);
                }
#pragma unroll
                for (int i = 0; i < TPG; ++i) {
                    const int tile = wave + (grp + i) * NWA;
                    if (tile < ntiles) {
                        const float2 qv = tile < nt16 ? qa[0] : qa[1];
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(qv.x, kb[i].x, acc[i], 0, 0, 0);
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(qv.y, kb[i].y, acc[i], 0, 0, 0);
                    }
                }
            }
        }
        // D layout: lane holds tokens 4*(lane/16)+i of subkey column lane%16
        float qn[2][4];  // IDW: ||q||^2 of the 4 tokens of this lane's D rows, per half
        if constexpr (IDW) {
            // lanes m16 + 16 g4 (g4 = 0..3) loaded disjoint chunks of token m16 / subkey row m16
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float t = qsq[jj];
                t += xlanef<16>(t, lane);
                t += xlanef<32>(t, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) qn[jj][r] = __shfl(t, g4 * 4 + r);
            }
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                ksq[i] += xlanef<16>(ksq[i], lane);
                ksq[i] += xlanef<32>(ksq[i], lane);
            }
        }
#pragma unroll
        for (int i = 0; i < TPG; ++i) {
            const int tile = wave + (grp + i) * NWA;
            if (tile < ntiles) {
                const int j = tile / nt16, a0 = (tile % nt16) * 16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float sc = acc[i][r];
                    if constexpr (IDW) {
                        const float d2 = fmaf(-2.f, sc, (j ? qn[1][r] : qn[0][r]) + ksq[i]);
                        sc = -logf(IDW_EPS + fmaxf(d2, 0.f));
                    }
                    sc_tok(g4 * 4 + r)[j * n + a0 + m16] = sc;
                }
            }
        }
    }
    __syncthreads();

    if (a.half_out) {  // test hook: the contraction only
        for (int e = threadIdx.x; e < TOK * 2 * n; e += NWA * 64) {
            const int m = e / (2 * n);
            if (u0 + m < UT) a.half_out[row_of(u0 + m) * 2 * n + (e - m * 2 * n)] = sc_tok(m)[e - m * 2 * n];
        }
        return;
    }

    // ---------------- pruned rank pairs for this branch's k ----------------
    const int k = a.k[br];
    const int kh = k < n ? k : n;
    int len = 0;
    if (lane < kh) {
        len = k / (lane + 1);
        if (len > kh) len = kh;
    }
    int incl = len;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    const int C = __builtin_amdgcn_readlane(incl, 63);
    if (wave == 0)
        for (int jj = 0, off = incl - len; jj < len; ++jj) pairs[off + jj] = ((uint32_t)lane << 8) | (uint32_t)jj;
    __syncthreads();

    int32_t* idx_out = a.idx[br];
    float* wt_out = a.wt[br];
    float* sc_out = a.score[br];

    {
        const int m0 = wave * TG;
        if (u0 + m0 >= UT) return;
        // tokens past T run on the zero scores of their masked rows; nothing is stored

        // ---------------- a2: per-half top-k_h, sorted ----------------
        // both halves' scores into registers first: the block is reused below
        uint32_t keys[2][TG][EH];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                const float* s = sc_tok(m0 + g) + j * n;
#pragma unroll
                for (int e = 0; e < EH; ++e) {
                    const int aa = e * 64 + lane;
                    keys[j][g][e] = aa < n ? ord_key(s[aa]) : 0u;
                }
            }
        uint32_t kth0[TG];  // half 0's k_h-th key, per token
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // Half 1's scores come from the same subkey distribution and a
            // half-query of similar norm, so its k_h-th key is usually near half
            // 0's: two counts test the bracket [0.75 x, 1.35 x) around it (x the
            // half-0 value) and, when it holds, the select starts below the
            // bracket's common leading bits (else, for that token, at bit 31).
            uint32_t tau0[TG], b0 = 0x80000000u;
            if (j == 1) {
                uint32_t bx = 0u;
#pragma unroll
                for (int g = 0; g < TG; ++g) {
                    const float f = key_float(kth0[g]), m = fabsf(f);
                    const uint32_t klo = ord_key(f - 0.25f * m), khi = ord_key(f + 0.35f * m);
                    int clo = 0, chi = 0;
#pragma unroll
                    for (int e = 0; e < EH; ++e) {
                        clo += popc(__ballot(keys[1][g][e] >= klo));
                        chi += popc(__ballot(keys[1][g][e] >= khi));
                    }
                    tau0[g] = 0u;
                    uint32_t top = 0x80000000u;
                    if (clo >= kh && chi < kh && khi > klo) {  // klo <= S_k <= khi - 1
                        const uint32_t d = klo ^ (khi - 1u);
                        top = d ? 0x80000000u >> __clz(d) : 1u;
                        tau0[g] = klo & (d ? ~((top << 1) - 1u) : ~0u);
                    }
                    bx |= top;
                }
                b0 = 0x80000000u >> __clz(bx);
            }
            wave_select<TG, EH>(
                [&](int g, int e, uint32_t& kk, uint32_t& ii) {
                    kk = keys[j][g][e];
                    ii = (uint32_t)(e * 64 + lane);
                },
                EH, kh, bkey, bid, lane, j == 1 ? tau0 : nullptr, b0);
            uint64_t x[TG];
            sort_winners<TG>(x, bkey, bid, kh, lane);
            if (j == 0) {
#pragma unroll
                for (int g = 0; g < TG; ++g)
                    kth0[g] = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x[g] >> 32), kh - 1);
            }
#pragma unroll
            for (int g = 0; g < TG; ++g)
                if (lane < kh) {
                    ls[(g * 2 + j) * 64 + lane] = key_float((uint32_t)(x[g] >> 32));
                    lid[(g * 2 + j) * 64 + lane] = 0xFFFFFFFFu - (uint32_t)x[g];
                }
        }

        // ---------------- a3: combine over the pruned pairs ----------------
        uint32_t ck[TG][EC], ci[TG][EC];
#pragma unroll
        for (int e = 0; e < EC; ++e) {
            const int c = e * 64 + lane;
            const uint32_t p = c < C ? pairs[c] : 0u;
            const int i = (int)(p >> 8), jj = (int)(p & 255u);
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                ck[g][e] = c < C ? ord_key(ls[(g * 2) * 64 + i] + ls[(g * 2 + 1) * 64 + jj]) : 0u;
                ci[g][e] = __umul24(lid[(g * 2) * 64 + i], (uint32_t)n) + lid[(g * 2 + 1) * 64 + jj];
            }
        }
        // Known leading bits of each token's k-th candidate key S_k: the pairs
        // (i, 0), i < k, are all candidates, so S_k >= s_0[k-1] + s_1[0]
        // (likewise s_0[0] + s_1[k-1]), and S_k <= s_0[0] + s_1[0]; the bits
        // above the highest one where these two bounds differ are S_k's. (Only
        // when k <= n: else fewer than k pairs have rank 0 in a half.)
        uint32_t tau0[TG], bx = 0u;
#pragma unroll
        for (int g = 0; g < TG; ++g) {
            tau0[g] = 0u;
            if (k <= n) {
                const float* l0 = ls + (g * 2) * 64;
                const float* l1 = ls + (g * 2 + 1) * 64;
                const uint32_t lo_a = ord_key(l0[k - 1] + l1[0]), lo_b = ord_key(l0[0] + l1[k - 1]);
                const uint32_t lo = lo_a > lo_b ? lo_a : lo_b, hi = ord_key(l0[0] + l1[0]);
                const uint32_t d = lo ^ hi;                             // lo <= hi
                const uint32_t top = d ? 0x80000000u >> __clz(d) : 0u;  // highest differing bit
                tau0[g] = lo & (top ? ~((top << 1) - 1u) : ~0u);         // the bits above it (all if none)
                bx |= top ? top : 1u;
                tau0[g] = (uint32_t)__builtin_amdgcn_readfirstlane((int)tau0[g]);
            } else {
                bx |= 0x80000000u;
            }
        }
        bx = (uint32_t)__builtin_amdgcn_readfirstlane((int)bx);
        const uint32_t b0 = 0x80000000u >> __clz(bx);  // the highest start bit of the tokens
        wave_select<TG, EC>(
            [&](int g, int e, uint32_t& kk, uint32_t& ii) {
                kk = ck[g][e];
                ii = ci[g][e];
            },
            EC, k, bkey, bid, lane, tau0, b0);
        uint64_t x[TG];
        sort_winners<TG>(x, bkey, bid, k, lane);

        // certificate: every pruned pair must score strictly below the k-th winner
#pragma unroll
        for (int g = 0; g < TG; ++g) {
            const uint32_t kth = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x[g] >> 32), k - 1);
            uint32_t bnd = 0u;
            if (lane < kh) {
                const int jb = k / (lane + 1);
                if (jb < kh) bnd = ord_key(ls[(g * 2) * 64 + lane] + ls[(g * 2 + 1) * 64 + jb]);
            }
            if (u0 + m0 + g < UT && __ballot(bnd != 0u && bnd >= kth) != 0ull) {
                const int full = kh * kh;
                const float* l0 = ls + (g * 2) * 64;
                const float* l1 = ls + (g * 2 + 1) * 64;
                const uint32_t* i0 = lid + (g * 2) * 64;
                const uint32_t* i1 = lid + (g * 2 + 1) * 64;
                wave_select<1, 0>(
                    [&](int, int e, uint32_t& kk, uint32_t& ii) {
                        const int c = e * 64 + lane;
                        kk = 0u;
                        ii = 0u;
                        if (c < full) {
                            const int i = c / kh, jj = c - (c / kh) * kh;
                            kk = ord_key(l0[i] + l1[jj]);
                            ii = i0[i] * (uint32_t)n + i1[jj];
                        }
                    },
                    (full + 63) / 64, k, bkey + g * OSTR, bid + g * OSTR, lane);
                uint64_t y1[1] = {lane < k ? composite(bkey[g * OSTR + lane], bid[g * OSTR + lane]) : 0ull};
                wave_sort_desc<1>(y1, lane);
                x[g] = y1[0];
            }
        }

        // ---------------- a4: softmax over the k winners ----------------
#pragma unroll
        for (int g = 0; g < TG; ++g) {
            const int64_t u = u0 + m0 + g;
            const float S = key_float((uint32_t)(x[g] >> 32));
            const uint32_t slot = 0xFFFFFFFFu - (uint32_t)x[g];
            const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), 0));
            const float ex = lane < k ? expf(S - mx) : 0.f;
            const float sum = wave_sum(ex, lane);
            if (lane < k && u < UT) {
                const int64_t o = row_of(u) * k + lane;
                idx_out[o] = (int32_t)slot;
                wt_out[o] = ex / sum;
                if (sc_out) sc_out[o] = S;
            }
        }
    }
}

template <bool BF16, int EH>
hipError_t launch_inst(const AddressArgs& a, hipStream_t st) {
    const int64_t ntile = (a.B * a.T + TOK - 1) / TOK;
    const size_t lds = (size_t)NWA * block_floats(a.n) * 4 + EC * 64 * 4;
    dim3 grid((unsigned)(ntile * a.H), (unsigned)a.nbranch);
    if (a.idw)
        hipLaunchKernelGGL((address_kernel<BF16, EH, true>), grid, dim3(NWA * 64), lds, st, a);
    else
        hipLaunchKernelGGL((address_kernel<BF16, EH, false>), grid, dim3(NWA * 64), lds, st, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const AddressArgs& a, hipStream_t st) {
    if (a.n <= 64) return launch_inst<BF16, 1>(a, st);
    if (a.n <= 128) return launch_inst<BF16, 2>(a, st);
    if (a.n <= 256) return launch_inst<BF16, 4>(a, st);
    return launch_inst<BF16, 8>(a, st);
}

}  // namespace

hipError_t launch_address(const AddressArgs& a, hipStream_t st) {
    return a.bf16 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

}  // namespace sdm
