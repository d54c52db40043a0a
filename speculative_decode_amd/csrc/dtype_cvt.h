// dtype_cvt.h -- element loads, stores and conversions between the storage
// formats of the C ABI (fp32, fp16, bf16) and fp32 registers, shared by the
// HIP kernels.  Narrowing rounds to nearest, ties to even (gfx950 converts a
// pair of floats in one instruction); widening is exact.
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

}  // namespace gdn_dev
