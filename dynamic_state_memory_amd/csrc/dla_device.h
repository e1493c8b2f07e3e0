// dla_device.h -- device helpers shared by the libdla kernels: MFMA operand
// fragments, wave reductions, fixed-point and fp16 scaling helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dla {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return static_cast<__bf16>(x); }

// k >> s for s in [0, 64]; a shift by 64 gives 0.
__device__ __forceinline__ uint64_t shr64(uint64_t x, int s) { return s >= 64 ? 0ull : (x >> s); }
__device__ __forceinline__ uint64_t low_bits(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }

// The 2^-32 fixed-point value of a float information score (round half even).
__device__ __forceinline__ int64_t fixed_point(float s) {
    return __double2ll_rn(static_cast<double>(s) * 4294967296.0);
}

// 1 - cos from double-precision dot and squared norms, rounded once to float.
__device__ __forceinline__ float cosine_distance(double d, double a, double b) {
    const double ab = a * b;
    if (ab == 0.0) return 1.0f;
    return static_cast<float>(1.0 - d / sqrt(ab));
}

// Eight consecutive elements, the per-lane operand of one 16x16x32 MFMA step.
template <typename T> struct Frag;
template <> struct Frag<__bf16> { bf16x8 v; };
template <> struct Frag<_Float16> { f16x8 v; };
template <> struct Frag<float> { float v[8]; };

// Operand type of the inter-chunk read: bf16 inputs are read against an fp16
// copy of the states (11-bit significands, normalised per state by a power of
// two), fp32 inputs against the fp32 states themselves.
template <typename TIO> struct ReadT;
template <> struct ReadT<__bf16> { typedef _Float16 type; };
template <> struct ReadT<float> { typedef float type; };

__device__ __forceinline__ void load_frag(Frag<__bf16> &f, const __bf16 *p) {
    f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_frag(Frag<_Float16> &f, const _Float16 *p) {
    f.v = *reinterpret_cast<const f16x8 *>(p);
}
__device__ __forceinline__ void load_frag(Frag<float> &f, const float *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void zero_frag(Frag<__bf16> &f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = static_cast<__bf16>(0.0f);
}
__device__ __forceinline__ void zero_frag(Frag<_Float16> &f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = static_cast<_Float16>(0.0f);
}
__device__ __forceinline__ void zero_frag(Frag<float> &f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = 0.0f;
}
// Zero the elements whose index (base + e) lies outside [lo, hi).
__device__ __forceinline__ void mask_frag(Frag<__bf16> &f, int base, int lo, int hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (base + e < lo || base + e >= hi) f.v[e] = static_cast<__bf16>(0.0f);
}
__device__ __forceinline__ void mask_frag(Frag<float> &f, int base, int lo, int hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (base + e < lo || base + e >= hi) f.v[e] = 0.0f;
}

// acc(16x16) += A(16x32) * B(32x16).  Lane l holds A row (l % 16) and B
// column (l % 16) at reduction indices 8*(l/16) + e, e = 0..7; A and B use the
// same index map, so the product sums every reduction index exactly once.
// The accumulator holds D[4*(l/16) + r][l % 16], r = 0..3.
__device__ __forceinline__ void mma32(floatx4 &acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(floatx4 &acc, const Frag<_Float16> &a, const Frag<_Float16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(floatx4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// not for its global loads and stores, so prefetches stay in flight across it.
// Use __syncthreads() where waves exchange data through global memory.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Cross-lane moves within a row of 16 lanes (DPP): lane l reads lane l ^ 1,
// l ^ 2, (l & ~7) + 7 - (l & 7) and (l & ~15) + 15 - (l & 15).  Every source
// lane lies in the same row, so no lane reads outside its row.
template <int CTRL> __device__ __forceinline__ uint32_t dpp32(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

// Lane l reads lane l + 1 across the whole wave (DPP wave_shl:1, registers
// only); lane 63 reads 0.  Callers use the value only where lane l + 1 holds
// data.
constexpr int kDppWaveShl1 = 0x130;
template <typename T> __device__ __forceinline__ T lane_down1(T x) {
    if constexpr (sizeof(T) == 8) {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = dpp32<kDppWaveShl1>(static_cast<uint32_t>(u));
        const uint32_t hi = dpp32<kDppWaveShl1>(static_cast<uint32_t>(u >> 32));
        return __builtin_bit_cast(T, (static_cast<uint64_t>(hi) << 32) | lo);
    } else {
        return __builtin_bit_cast(T, dpp32<kDppWaveShl1>(__builtin_bit_cast(uint32_t, x)));
    }
}

template <int CTRL> __device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, dpp32<CTRL>(__builtin_bit_cast(uint32_t, x)));
}
template <int CTRL> __device__ __forceinline__ int32_t dpp_move(int32_t x) {
    return static_cast<int32_t>(dpp32<CTRL>(static_cast<uint32_t>(x)));
}
template <int CTRL> __device__ __forceinline__ uint64_t dpp_move64(uint64_t x) {
    const uint32_t lo = dpp32<CTRL>(static_cast<uint32_t>(x));
    const uint32_t hi = dpp32<CTRL>(static_cast<uint32_t>(x >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <int CTRL> __device__ __forceinline__ double dpp_move(double x) {
    return __builtin_bit_cast(double, dpp_move64<CTRL>(__builtin_bit_cast(uint64_t, x)));
}
template <int CTRL> __device__ __forceinline__ int64_t dpp_move(int64_t x) {
    return static_cast<int64_t>(dpp_move64<CTRL>(static_cast<uint64_t>(x)));
}

// DPP move that reads 0 in every lane outside the rows set in ROWS (bit r:
// lanes 16 r .. 16 r + 15) and in every lane whose source lies outside the wave
// or its row: row_shr:n (0x110 + n), row_bcast:15 (0x142), row_bcast:31
// (0x143) and wave_shr:1 (0x138).
template <int CTRL, int ROWS> __device__ __forceinline__ uint32_t dpp32_rows(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS, typename T> __device__ __forceinline__ T dpp_rows(T x) {
    static_assert(sizeof(T) == 8, "64-bit values");
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = dpp32_rows<CTRL, ROWS>(static_cast<uint32_t>(u));
    const uint32_t hi = dpp32_rows<CTRL, ROWS>(static_cast<uint32_t>(u >> 32));
    return __builtin_bit_cast(T, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP: shifts by 1, 2, 4
// and 8 lanes within each row of 16, then the last lane of row 0 (2) added
// into row 1 (3), then the last lane of row 1 into rows 2 and 3.  The whole
// wave must be active.
template <typename T> __device__ __forceinline__ T wave_incl_scan_dpp(T x) {
    x += dpp_rows<0x111, 0xF>(x);
    x += dpp_rows<0x112, 0xF>(x);
    x += dpp_rows<0x114, 0xF>(x);
    x += dpp_rows<0x118, 0xF>(x);
    x += dpp_rows<0x142, 0xA>(x);
    x += dpp_rows<0x143, 0xC>(x);
    return x;
}
// The value of the lane below (lane 0 reads 0).
template <typename T> __device__ __forceinline__ T lane_up1(T x) { return dpp_rows<0x138, 0xF>(x); }

template <typename T> __device__ __forceinline__ T readlane_any(T x, int l) {
    if constexpr (sizeof(T) == 8) {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), l);
        const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), l);
        return __builtin_bit_cast(T, (static_cast<uint64_t>(hi) << 32) | lo);
    } else {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    }
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32), in every lane of the
// group: DPP steps within a row of 16, then (G = 32) one exchange between
// the two rows of the group.
template <int G, typename T> __device__ __forceinline__ T group_sum_dpp(T x) {
    static_assert(G == 8 || G == 16 || G == 32, "groups of 8, 16 or 32 lanes");
    x += dpp_move<kDppXor1>(x);
    x += dpp_move<kDppXor2>(x);
    x += dpp_move<kDppHalfMirror>(x);
    if constexpr (G >= 16) x += dpp_move<kDppMirror>(x);
    if constexpr (G == 32) x += __shfl_xor(x, 16);
    return x;
}

// Sum / maximum over the 64 lanes of a wave, returned in every lane: four
// DPP steps reduce each row of 16 lanes, then the four row results are
// combined from lanes 0, 16, 32, 48.  The whole wave must be active.
// (Summation order: pairs, quads, halves, rows, then rows 0 + 1 + 2 + 3;
// sums of exactly representable terms, as in the score, are order-free.)
template <typename T> __device__ __forceinline__ T wave_sum(T x) {
    x += dpp_move<kDppXor1>(x);
    x += dpp_move<kDppXor2>(x);
    x += dpp_move<kDppHalfMirror>(x);
    x += dpp_move<kDppMirror>(x);
    return (readlane_any(x, 0) + readlane_any(x, 16)) + (readlane_any(x, 32) + readlane_any(x, 48));
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_move<kDppXor1>(x));
    x = fmaxf(x, dpp_move<kDppXor2>(x));
    x = fmaxf(x, dpp_move<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_move<kDppMirror>(x));
    return fmaxf(fmaxf(readlane_any(x, 0), readlane_any(x, 16)), fmaxf(readlane_any(x, 32), readlane_any(x, 48)));
}

// Exponent e with max * 2^-e in [2^14, 2^15): the largest magnitude then uses
// the top of fp16's range; 0 for an all-zero block.
__device__ __forceinline__ int f16_exponent(float maxabs) {
    return maxabs > 0.0f ? ilogbf(maxabs) - 14 : 0;
}

// The query chunk's A fragment of the inter-chunk read: fp16, scaled by 2^-e.
__device__ __forceinline__ void read_frag_from(Frag<_Float16> &f, const __bf16 *p, int e) {
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = static_cast<_Float16>(ldexpf(static_cast<float>(x[j]), -e));
}
__device__ __forceinline__ void read_frag_from(Frag<float> &f, const float *p, int) { load_frag(f, p); }

__device__ __forceinline__ int64_t min_i64(int64_t a, int64_t b) { return b < a ? b : a; }

// Four floats rounded to bf16 (nearest even), packed little-end first, and back.
__device__ __forceinline__ uint2 pack_bf16x4(float4 v)
{
    const __bf16 a = static_cast<__bf16>(v.x), b = static_cast<__bf16>(v.y);
    const __bf16 c = static_cast<__bf16>(v.z), d = static_cast<__bf16>(v.w);
    return make_uint2(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16),
                      static_cast<uint32_t>(__builtin_bit_cast(uint16_t, c)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, d)) << 16));
}
__device__ __forceinline__ float4 unpack_bf16x4(uint2 u)
{
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Lane holding the smallest of the fractions num / den (num >= 0, den >= 1)
// over the lanes with ok set, the lowest such lane on ties; the same in every
// lane (64 if no lane is ok).  a / b < c / d is decided as a d < c b in
// 128-bit integers, so the comparison is exact.  A butterfly over the 64
// lanes; the whole wave must be active.
__device__ __forceinline__ int wave_argmin_frac(int64_t num, int64_t den, bool ok)
{
    int idx = ok ? static_cast<int>(__lane_id()) : 64;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t n2 = __shfl_xor(num, off);
        const int64_t d2 = __shfl_xor(den, off);
        const int i2 = __shfl_xor(idx, off);
        const __int128 lhs = static_cast<__int128>(n2) * den;   // n2 / d2 < num / den  <=>  lhs < rhs
        const __int128 rhs = static_cast<__int128>(num) * d2;
        const bool take = i2 < 64 && (idx == 64 || lhs < rhs || (lhs == rhs && i2 < idx));
        if (take) {
            num = n2;
            den = d2;
            idx = i2;
        }
    }
    return __builtin_amdgcn_readfirstlane(idx);
}

// Minimum over the 64 lanes of a wave, in every lane (DPP row steps, then the
// four row results; the whole wave must be active).
__device__ __forceinline__ int64_t wave_min_i64(int64_t x) {
    x = min_i64(x, dpp_move<kDppXor1>(x));
    x = min_i64(x, dpp_move<kDppXor2>(x));
    x = min_i64(x, dpp_move<kDppHalfMirror>(x));
    x = min_i64(x, dpp_move<kDppMirror>(x));
    return min_i64(min_i64(readlane_any(x, 0), readlane_any(x, 16)), min_i64(readlane_any(x, 32), readlane_any(x, 48)));
}

// Inclusive scan over a 64-lane wave.
template <typename T> __device__ __forceinline__ T wave_incl_scan(T x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

}  // namespace dla
