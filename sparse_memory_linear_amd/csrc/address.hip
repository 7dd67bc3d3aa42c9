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
// Design (one wavefront per workgroup, 16 tokens of one (b, h, branch)):
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
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int TOK = 16;       // tokens per wavefront = one MFMA M tile
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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;  // the butterfly adds the same pairs on every lane: identical on all lanes
}

// Select the k best candidates (larger key first, then smaller id) among
// candidates c = e*64 + lane, e < nch, read through get(e, key, id). Key 0
// marks an absent candidate; ids are below 2^18. Exactly k winners (k <= number
// of present candidates) are written in candidate order to okey/oid[0..k).
template <int NCH, typename Get>
__device__ void wave_select(Get get, int nch_rt, int k, uint32_t* okey, uint32_t* oid, int lane) {
    const int nch = NCH > 0 ? NCH : nch_rt;
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < nch; ++e) {
            uint32_t kk, ii;
            get(e, kk, ii);
            cnt += popc(__ballot(kk >= cand));
        }
        if (cnt >= k) tau = cand;
    }
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < nch; ++e) {
        uint32_t kk, ii;
        get(e, kk, ii);
        gt += popc(__ballot(kk > tau));
        eq += popc(__ballot(kk == tau));
    }
    const int need = k - gt;
    const bool cut = eq > need;  // more ties at the threshold than places left
    uint32_t sig = 0u;
    if (cut) {
        for (int bit = 17; bit >= 0; --bit) {
            const uint32_t cand = sig | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < nch; ++e) {
                uint32_t kk, ii;
                get(e, kk, ii);
                cnt += popc(__ballot(kk == tau && (0x3FFFFu - ii) >= cand));
            }
            if (cnt >= need) sig = cand;
        }
    }
    int base = 0;
#pragma unroll
    for (int e = 0; e < nch; ++e) {
        uint32_t kk, ii;
        get(e, kk, ii);
        const bool sel = kk > tau || (kk == tau && (!cut || (0x3FFFFu - ii) >= sig));
        const uint64_t m = __ballot(sel);
        if (sel) {
            const int pos = base + lanes_below(m);
            okey[pos] = kk;
            oid[pos] = ii;
        }
        base += popc(m);
    }
}

// Bitonic sort across the 64 lanes, one 64-bit key per lane, descending.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t o = shfl_xor_u64(x, j);
            const bool keep_max = (((lane & j) == 0) == ((lane & k) == 0));
            const uint64_t mx = x > o ? x : o;
            const uint64_t mn = x > o ? o : x;
            x = keep_max ? mx : mn;
        }
    }
    return x;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t id) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

template <bool BF16, int EH>
__global__ __launch_bounds__(64) void address_kernel(AddressArgs a) {
    extern __shared__ __align__(16) uint32_t smem[];
    const int lane = threadIdx.x;
    const int n = a.n, dh = a.dh;
    const int64_t ntile = (a.T + TOK - 1) / TOK;
    const int64_t bh = blockIdx.x / ntile;
    const int64_t t0 = (blockIdx.x % ntile) * TOK;
    const int br = blockIdx.y;
    const int h = (int)(bh % a.H);

    float* sc = reinterpret_cast<float*>(smem);      // [TOK][2][n]
    float* ls = sc + TOK * 2 * n;                     // [2][64] sorted half scores
    uint32_t* lid = reinterpret_cast<uint32_t*>(ls + 128);  // [2][64] their sub-indices
    uint32_t* bkey = lid + 128;                       // [64] select output
    uint32_t* bid = bkey + 64;                        // [64]
    uint32_t* pairs = bid + 64;                       // [EC*64] pruned rank pairs

    // ---------------- a1: half-scores on MFMA ----------------
    const int m16 = lane & 15, g4 = lane >> 4;
    const int64_t tq = t0 + m16;
    const bool tok_ok = tq < a.T;
    for (int j = 0; j < 2; ++j) {
        for (int a0 = 0; a0 < n; a0 += 16) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BF16) {
                const uint16_t* q = static_cast<const uint16_t*>(a.q[br]) +
                                    ((bh * a.T + (tok_ok ? tq : 0)) * 2 + j) * dh;
                const uint16_t* kp = static_cast<const uint16_t*>(a.K[br]) +
                                     (((int64_t)h * 2 + j) * n + a0 + m16) * dh;
                for (int c0 = 0; c0 < dh; c0 += 32) {
                    uint4 qa = tok_ok ? *reinterpret_cast<const uint4*>(q + c0 + g4 * 8)
                                      : make_uint4(0u, 0u, 0u, 0u);
                    uint4 kb = *reinterpret_cast<const uint4*>(kp + c0 + g4 * 8);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, qa), __builtin_bit_cast(bf16x8_t, kb), acc, 0, 0, 0);
                }
            } else {
                const float* q = static_cast<const float*>(a.q[br]) +
                                 ((bh * a.T + (tok_ok ? tq : 0)) * 2 + j) * dh;
                const float* kp = static_cast<const float*>(a.K[br]) +
                                  (((int64_t)h * 2 + j) * n + a0 + m16) * dh;
                for (int c0 = 0; c0 < dh; c0 += 8) {
                    float2 qa = tok_ok ? *reinterpret_cast<const float2*>(q + c0 + g4 * 2)
                                       : make_float2(0.f, 0.f);
                    float2 kb = *reinterpret_cast<const float2*>(kp + c0 + g4 * 2);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa.x, kb.x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa.y, kb.y, acc, 0, 0, 0);
                }
            }
            // D layout: lane holds tokens 4*(lane/16)+i of subkey column lane%16
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[((g4 * 4 + i) * 2 + j) * n + a0 + m16] = acc[i];
        }
    }
    __syncthreads();

    if (a.half_out) {  // test hook: the contraction only
        for (int e = lane; e < TOK * 2 * n; e += 64) {
            const int m = e / (2 * n);
            if (t0 + m < a.T) a.half_out[(bh * a.T + t0) * 2 * n + e] = sc[e];
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
    const int C = __shfl(incl, 63);
    for (int jj = 0, off = incl - len; jj < len; ++jj) pairs[off + jj] = ((uint32_t)lane << 8) | (uint32_t)jj;
    __syncthreads();

    int32_t* idx_out = a.idx[br];
    float* wt_out = a.wt[br];
    float* sc_out = a.score[br];

    for (int m = 0; m < TOK; ++m) {
        const int64_t t = t0 + m;
        if (t >= a.T) break;

        // ---------------- a2: per-half top-k_h, sorted ----------------
        for (int j = 0; j < 2; ++j) {
            const float* s = sc + (m * 2 + j) * n;
            uint32_t key[EH], id[EH];
#pragma unroll
            for (int e = 0; e < EH; ++e) {
                const int aa = e * 64 + lane;
                key[e] = aa < n ? ord_key(s[aa]) : 0u;
                id[e] = (uint32_t)aa;
            }
            wave_select<EH>([&](int e, uint32_t& kk, uint32_t& ii) { kk = key[e]; ii = id[e]; },
                            EH, kh, bkey, bid, lane);
            uint64_t x = lane < kh ? composite(bkey[lane], bid[lane]) : 0ull;
            x = wave_sort_desc(x, lane);
            if (lane < kh) {
                ls[j * 64 + lane] = key_float((uint32_t)(x >> 32));
                lid[j * 64 + lane] = 0xFFFFFFFFu - (uint32_t)x;
            }
        }

        // ---------------- a3: combine over the pruned pairs ----------------
        uint32_t ck[EC], ci[EC];
#pragma unroll
        for (int e = 0; e < EC; ++e) {
            const int c = e * 64 + lane;
            ck[e] = 0u;
            ci[e] = 0u;
            if (c < C) {
                const uint32_t p = pairs[c];
                const int i = (int)(p >> 8), jj = (int)(p & 255u);
                ck[e] = ord_key(ls[i] + ls[64 + jj]);
                ci[e] = lid[i] * (uint32_t)n + lid[64 + jj];
            }
        }
        wave_select<EC>([&](int e, uint32_t& kk, uint32_t& ii) { kk = ck[e]; ii = ci[e]; },
                        EC, k, bkey, bid, lane);
        uint64_t x = lane < k ? composite(bkey[lane], bid[lane]) : 0ull;
        x = wave_sort_desc(x, lane);

        // certificate: every pruned pair must score strictly below the k-th winner
        const uint32_t kth = (uint32_t)(__shfl((int)(uint32_t)(x >> 32), k - 1));
        uint32_t bnd = 0u;
        if (lane < kh) {
            const int jb = k / (lane + 1);
            if (jb < kh) bnd = ord_key(ls[lane] + ls[64 + jb]);
        }
        if (__ballot(bnd != 0u && bnd >= kth) != 0ull) {
            const int full = kh * kh;
            wave_select<0>(
                [&](int e, uint32_t& kk, uint32_t& ii) {
                    const int c = e * 64 + lane;
                    kk = 0u;
                    ii = 0u;
                    if (c < full) {
                        const int i = c / kh, jj = c - (c / kh) * kh;
                        kk = ord_key(ls[i] + ls[64 + jj]);
                        ii = lid[i] * (uint32_t)n + lid[64 + jj];
                    }
                },
                (full + 63) / 64, k, bkey, bid, lane);
            x = lane < k ? composite(bkey[lane], bid[lane]) : 0ull;
            x = wave_sort_desc(x, lane);
        }

        // ---------------- a4: softmax over the k winners ----------------
        const float S = key_float((uint32_t)(x >> 32));
        const uint32_t slot = 0xFFFFFFFFu - (uint32_t)x;
        const float mx = __shfl(S, 0);
        const float ex = lane < k ? expf(S - mx) : 0.f;
        const float sum = wave_sum(ex);
        if (lane < k) {
            const int64_t o = (bh * a.T + t) * k + lane;
            idx_out[o] = (int32_t)slot;
            wt_out[o] = ex / sum;
            if (sc_out) sc_out[o] = S;
        }
    }
}

template <bool BF16, int EH>
hipError_t launch_inst(const AddressArgs& a, hipStream_t st) {
    const int64_t ntile = (a.T + TOK - 1) / TOK;
    const size_t lds = (size_t)TOK * 2 * a.n * 4 + (128 + 128 + 64 + 64 + EC * 64) * 4;
    dim3 grid((unsigned)(ntile * a.B * a.H), (unsigned)a.nbranch);
    hipLaunchKernelGGL((address_kernel<BF16, EH>), grid, dim3(64), lds, st, a);
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
