// dtype_cvt.h -- element loads, stores and conversions between the storage
// formats of the C ABI (fp32, fp16, bf16, and fp8 e4m3 for the state) and
// fp32 registers, shared by the HIP kernels.  Narrowing rounds to nearest,
// ties to even (gfx950 converts a pair of floats in one instruction);
// widening is exact.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../../include/gdn_spec.h"

namespace gdn_dev {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw bits of two consecutive elements: one dword for 16-bit types, two for
// fp32.  Loads keep raw bits so that conversion waits can be deferred.
template <int DT>
struct Pair {
    using raw = typename std::conditional<DT == GDN_F32, uint2, uint32_t>::type;
};

template <int DT>
__device__ __forceinline__ float2 unpack_pair(typename Pair<DT>::raw w)
{
    if constexpr (DT == GDN_F32) {
        return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
    } else if constexpr (DT == GDN_BF16) {
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    } else {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        return make_float2(static_cast<float>(h.x), static_cast<float>(h.y));
    }
}

template <int DT>
__device__ __forceinline__ float unpack_one(uint32_t w)
{
    if constexpr (DT == GDN_F32)
        return __uint_as_float(w);
    else if constexpr (DT == GDN_BF16)
        return __uint_as_float(w << 16);
    else
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}

// Two values rounded to nearest even into one dword (low element first);
// gfx950 converts the pair in one instruction.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    const f32x2 x = {lo, hi};
    if constexpr (DT == GDN_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

template <int DT>
__device__ __forceinline__ typename Pair<DT>::raw load_pair_raw(const void* base, int64_t idx)
{
    if constexpr (DT == GDN_F32)
        return *reinterpret_cast<const uint2*>(static_cast<const float*>(base) + idx);
    else
        return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + idx);
}

template <int DT>
__device__ __forceinline__ uint32_t load_one_raw(const void* base, int64_t idx)
{
    if constexpr (DT == GDN_F32)
        return static_cast<const uint32_t*>(base)[idx];
    else
        return static_cast<const uint16_t*>(base)[idx];
}

template <int DT>
__device__ __forceinline__ void store_pair(void* base, int64_t idx, float2 x)
{
    if constexpr (DT == GDN_F32)
        *reinterpret_cast<float2*>(static_cast<float*>(base) + idx) = x;
    else
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + idx) = pack2<DT>(x.x, x.y);
}

// ---- FP8 E4M3 (OCP, no infinities; S.1111.111 is NaN; largest finite 448) --
// The hardware conversion rounds to nearest even but turns every value that
// rounds past 448 into NaN, so finite values beyond the range are first
// saturated to +-448.  A NaN fails the comparison and reaches the conversion
// unchanged, which keeps it NaN (a med3 clamp would turn it into -448).
// Decoding converts a pair per instruction, exactly.
__device__ __forceinline__ float sat_f8(float x)
{
    return fabsf(x) > 448.0f ? copysignf(448.0f, x) : x;
}

__device__ __forceinline__ uint32_t pack4_f8(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_f8(a), sat_f8(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_f8(c), sat_f8(d), w, true);
    return static_cast<uint32_t>(w);
}

__device__ __forceinline__ void unpack4_f8(uint32_t w, float& a, float& b, float& c, float& d)
{
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    a = lo.x; b = lo.y; c = hi.x; d = hi.y;
}

// ---- 16-byte chunks of state elements (4 fp32, 8 fp16/bf16, 16 fp8) -------
template <int ST>
struct StateChunk {
    static constexpr int N = ST == GDN_F32 ? 4 : (ST == GDN_F8E4M3 ? 16 : 8);
};

template <int ST>
__device__ __forceinline__ void chunk_to_f32(const uint4& w, float* f)
{
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (ST == GDN_F32) {
            f[m] = __uint_as_float(u[m]);
        } else if constexpr (ST == GDN_F8E4M3) {
            unpack4_f8(u[m], f[4 * m], f[4 * m + 1], f[4 * m + 2], f[4 * m + 3]);
        } else {
            const float2 v = unpack_pair<ST>(u[m]);
            f[2 * m] = v.x;
            f[2 * m + 1] = v.y;
        }
    }
}

template <int ST>
__device__ __forceinline__ u32x4 f32_to_chunk(const float* f)
{
    u32x4 w;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (ST == GDN_F32)
            w[m] = __float_as_uint(f[m]);
        else if constexpr (ST == GDN_F8E4M3)
            w[m] = pack4_f8(f[4 * m], f[4 * m + 1], f[4 * m + 2], f[4 * m + 3]);
        else
            w[m] = pack2<ST>(f[2 * m], f[2 * m + 1]);
    }
    return w;
}

// n rows of 16 values to E4M3 chunks, as f32_to_chunk<GDN_F8E4M3> does, at
// a fraction of its cost when nothing saturates.  The bare conversion is
// already exact for |x| <= 464 (448 < |x| <= 464 rounds to 448); larger
// magnitudes and NaN come out as a NaN code, S.1111.111.  Adding 1 to the low
// seven bits of each byte carries into bit 7 exactly for those codes, so one
// OR over the chunks tells whether any byte needs the saturating conversion;
// only then (rarely) are the lane's rows converted again with it.  w's
// prior contents are overwritten; passing the previous call's words lets
// the conversions write in place instead of clearing a register first.
template <int NR>
__device__ __forceinline__ void encode_f8_rows(const float (&f)[NR][16], u32x4 (&w)[NR])
{
    uint32_t probe = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float* x = &f[r][4 * m];
            // Each conversion writes one half of the dword in place; both
            // halves are rewritten, so w's prior contents do not matter.
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], static_cast<int>(w[r][m]), false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
            w[r][m] = static_cast<uint32_t>(v);
            probe |= (w[r][m] & 0x7f7f7f7fu) + 0x01010101u;
        }
    }
    if (probe & 0x80808080u) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
            w[r] = f32_to_chunk<GDN_F8E4M3>(f[r]);
    }
}

// A pair of state values after a round trip through the storage format.
template <int ST>
__device__ __forceinline__ void round_pair(float& x, float& y)
{
    if constexpr (ST == GDN_F8E4M3) {
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_f8(x), sat_f8(y), 0, false);
        const f32x2 r = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        x = r.x;
        y = r.y;
    } else if constexpr (ST != GDN_F32) {
        const float2 r = unpack_pair<ST>(pack2<ST>(x, y));
        x = r.x;
        y = r.y;
    }
}

}  // namespace gdn_dev
