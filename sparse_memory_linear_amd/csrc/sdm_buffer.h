// sdm_buffer.h -- device helpers shared by the scan kernels: raw buffer
// loads and stores (32-bit lane offset + scalar offset, out-of-range accesses
// dropped by the hardware), float4 arithmetic and wavefront row reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
using rsrc_t = __amdgpu_buffer_rsrc_t;
// A buffer offset beyond every buffer the scan addresses (each is < 2 GiB): the
// hardware's range check drops the access and a load returns zeros.
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
    // raw buffer: stride 0, num_records = size in bytes, 32-bit data format (gfx9 word 3)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ int4 ld_i4(rsrc_t r, uint32_t vo, uint32_t so) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)so, 0);
    return make_int4((int)x.x, (int)x.y, (int)x.z, (int)x.w);
}
__device__ __forceinline__ int2 ld_i2(rsrc_t r, uint32_t vo, uint32_t so) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)vo, (int)so, 0);
    return make_int2((int)x.x, (int)x.y);
}
__device__ __forceinline__ float4 ld_f4(rsrc_t r, uint32_t vo, uint32_t so) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)so, 0);
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
}
__device__ __forceinline__ void st_f4(float4 v, rsrc_t r, uint32_t vo, uint32_t so) {
    u32x4 x;
    x.x = __float_as_uint(v.x); x.y = __float_as_uint(v.y); x.z = __float_as_uint(v.z); x.w = __float_as_uint(v.w);
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ void st_f1(float v, rsrc_t r, uint32_t vo, uint32_t so) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)vo, (int)so, 0);
}

// Workgroup -> (stream, unit of that stream: a column slab, or a slab and row
// partition). The hardware deals workgroups to the 8 XCDs round-robin
// (blockIdx mod 8). With at least 8 streams, all units of a stream go to one
// XCD, so its slabs share that XCD's L2 for the rows' lines and for the plan
// records they all read; with fewer, a stream's units are dealt over all 8
// XCDs, since one XCD's 32 CUs would otherwise carry every workgroup.
__device__ __forceinline__ void block_unit(int b, int64_t NS, int units, int64_t& s, int& u) {
    if (NS >= 8) {
        s = (int64_t)((b >> 3) / units) * 8 + (b & 7);
        u = (b >> 3) % units;
    } else {
        s = b / units;
        u = b % units;
    }
}
// Workgroups to launch for NS streams of `units` units each (with at least 8
// streams, rounded up to whole XCD rounds; the extra ones return at once).
inline int64_t unit_grid(int64_t NS, int64_t units) { return NS >= 8 ? ((NS + 7) / 8) * 8 * units : NS * units; }

// v_t of this lane's 4 columns.
template <bool BF16>
struct VLoad;
template <>
struct VLoad<false> {
    using T4 = float4;
    static constexpr int ESZ = 4;
    __device__ static T4 load(rsrc_t r, uint32_t vo, uint32_t so) { return ld_f4(r, vo, so); }
    __device__ static float4 f(const T4& x) { return x; }
};
template <>
struct VLoad<true> {
    using T4 = int2;
    static constexpr int ESZ = 2;
    __device__ static T4 load(rsrc_t r, uint32_t vo, uint32_t so) { return ld_i2(r, vo, so); }
    __device__ static float4 f(const T4& x) {
        const uint32_t a = (uint32_t)x.x, b = (uint32_t)x.y;
        return make_float4(__uint_as_float(a << 16), __uint_as_float(a & 0xFFFF0000u),
                           __uint_as_float(b << 16), __uint_as_float(b & 0xFFFF0000u));
    }
};

// v_t of this lane's 8 columns (a lane of a bf16-table row holds 8 columns).
template <bool BF16>
struct VLoad8;
template <>
struct VLoad8<false> {
    struct T4 { float4 a, b; };
    static constexpr int ESZ = 4;
    __device__ static T4 load(rsrc_t r, uint32_t vo, uint32_t so) { return {ld_f4(r, vo, so), ld_f4(r, vo + 16u, so)}; }
    __device__ static void f(const T4& x, float4 (&o)[2]) { o[0] = x.a; o[1] = x.b; }
};
template <>
struct VLoad8<true> {
    using T4 = int4;
    static constexpr int ESZ = 2;
    __device__ static T4 load(rsrc_t r, uint32_t vo, uint32_t so) { return ld_i4(r, vo, so); }
    __device__ static void f(const T4& x, float4 (&o)[2]) {
        o[0] = VLoad<true>::f(make_int2(x.x, x.y));
        o[1] = VLoad<true>::f(make_int2(x.z, x.w));
    }
};
// v of a lane's CPL columns as NQ = CPL / 4 float4
template <bool VBF16, int NQ>
struct VLoadN;
template <bool VBF16>
struct VLoadN<VBF16, 1> {
    using VL = VLoad<VBF16>;
    using T = typename VL::T4;
    static constexpr int ESZ = VL::ESZ;
    __device__ static T load(rsrc_t r, uint32_t vo, uint32_t so) { return VL::load(r, vo, so); }
    __device__ static void f(const T& x, float4 (&o)[1]) { o[0] = VL::f(x); }
};
template <bool VBF16>
struct VLoadN<VBF16, 2> {
    using VL = VLoad8<VBF16>;
    using T = typename VL::T4;
    static constexpr int ESZ = VL::ESZ;
    __device__ static T load(rsrc_t r, uint32_t vo, uint32_t so) { return VL::load(r, vo, so); }
    __device__ static void f(const T& x, float4 (&o)[2]) { VL::f(x, o); }
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));


// A lane's 16-byte piece of a table row: 4 fp32 columns (NQ = 1) or 8
// bfloat16 columns (NQ = 2), unpacked to NQ float4 for the arithmetic and
// packed back (bfloat16: rounded to nearest even) for the store. The packed
// 16 bytes are exactly what the table holds, so they are also what an LDS
// copy of a written row keeps.
template <bool MBF16>
struct RowFmt;
template <>
struct RowFmt<false> {
    static constexpr int NQ = 1, CPL = 4, ESZ = 4;
    __device__ static void unpack(float4 m, float4 (&x)[1]) { x[0] = m; }
    __device__ static float4 pack(const float4 (&x)[1]) { return x[0]; }
};
template <>
struct RowFmt<true> {
    static constexpr int NQ = 2, CPL = 8, ESZ = 2;
    __device__ static void unpack(float4 m, float4 (&x)[2]) {
        const uint32_t a = __float_as_uint(m.x), b = __float_as_uint(m.y);
        const uint32_t c = __float_as_uint(m.z), d = __float_as_uint(m.w);
        x[0] = make_float4(__uint_as_float(a << 16), __uint_as_float(a & 0xFFFF0000u),
                           __uint_as_float(b << 16), __uint_as_float(b & 0xFFFF0000u));
        x[1] = make_float4(__uint_as_float(c << 16), __uint_as_float(c & 0xFFFF0000u),
                           __uint_as_float(d << 16), __uint_as_float(d & 0xFFFF0000u));
    }
    // two values per v_cvt_pk_bf16_f32, gfx950's round-to-nearest-even
    // conversion: for finite values bit for bit (u + 0x7FFF + lsb) >> 16 of the
    // fp32 bits u (checked on MI355X over every exponent with tie and near-tie
    // low bits, both signs, denormals, and 2^26 random values)
    __device__ static uint32_t pk(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
    }
    __device__ static float4 pack(const float4 (&x)[2]) {
        return make_float4(__uint_as_float(pk(x[0].x, x[0].y)), __uint_as_float(pk(x[0].z, x[0].w)),
                           __uint_as_float(pk(x[1].x, x[1].y)), __uint_as_float(pk(x[1].z, x[1].w)));
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
// Sum over the G rows of a wavefront (lane = row * L + chunk), as a
// reduce-scatter: the gfx950 permlane swaps exchange one register between lane
// halves (32) and quarter pairs (16), so each swap + add halves the number of
// components a lane carries. Lane l ends with component l / 16 of column chunk
// l % L summed over all rows; lanes that share (l / 16, l % L) hold equal bits.
//   swap32(A, B): lanes < 32 get {A[l], A[l+32]}, lanes >= 32 get {B[l-32], B[l]}
//   swap16(A, B): the same between even and odd rows of 16 lanes
template <int L>
__device__ __forceinline__ float rows_reduce(float4 x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.x), __float_as_uint(x.z), false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x.y), __float_as_uint(x.w), false, false);
    const float a = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // comp 0 (lanes < 32) or 2
    const float b = __uint_as_float(q[0]) + __uint_as_float(q[1]);  // comp 1 (lanes < 32) or 3
    const auto u = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    float c = __uint_as_float(u[0]) + __uint_as_float(u[1]);        // comp lane / 16
    if constexpr (L <= 8) c = ror_add<8>(c);
    if constexpr (L <= 4) c = ror_add<4>(c);
    if constexpr (L <= 2) c = ror_add<2>(c);
    if constexpr (L <= 1) c = ror_add<1>(c);
    return c;
}

// Sum over the L consecutive lanes that hold one row segment (L = 1, 2, 4, 8);
// every lane of the group gets the sum. DPP quad permutations add the lane
// pairs (xor 1) and the pairs of pairs (xor 2); the half-row mirror pairs the
// two quads of a group of 8.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (L >= 2) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    if constexpr (L >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    if constexpr (L >= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}
// Sum over all 64 lanes (every lane gets it): rotations within each row of
// 16 lanes, then the 16- and 32-lane swaps.
__device__ __forceinline__ float wave_sum(float x) {
    x = ror_add<8>(x);
    x = ror_add<4>(x);
    x = ror_add<2>(x);
    x = ror_add<1>(x);
    const auto u = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(u[0]) + __uint_as_float(u[1]);
    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

}  // namespace
}  // namespace sdm
