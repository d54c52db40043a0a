// lane_ops.h -- cross-lane sums over 8-lane row groups and over a wave64,
// built from DPP row operations, and the scalar math of the per-token gates,
// norms and gated RMSNorm, shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn_dev {

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the
// same bits: quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror.
__device__ __forceinline__ float sum8(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x;
}

// Sum over the wave; wave-uniform result.
__device__ __forceinline__ float sum64(float x)
{
    x = sum8(x);
    x += dpp<0x140>(x);  // row_mirror: 16-lane sums
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// Four wave sums at once, each wave-uniform: (x0, x1, x2, x3) are replaced by
// their sums over the 64 lanes.  Two exchange steps inside each quad leave
// lane l with the quad's partial sum of x_{l % 4}; two rotations finish the
// sums of the lanes of a 16-lane row with the same l % 4; the gfx950 row
// swaps (v_permlane16_swap: rows 0/1 and 2/3; v_permlane32_swap: the two
// halves), which stay in the vector ALU, add the rows; lanes 0..3 hand out
// the four results.  Both operands of every add are the same two values in
// every lane, so all lanes hold the same bits.  About a third of the
// instructions of four separate sum64 calls.
__device__ __forceinline__ void sum64x4(float& x0, float& x1, float& x2, float& x3)
{
    const int lane = static_cast<int>(__lane_id());
    const bool odd = lane & 1, hi = lane & 2;
    float a = odd ? x1 : x0, c = odd ? x3 : x2;
    a += dpp<0xB1>(odd ? x0 : x1);   // quad_perm(1,0,3,2): the neighbour's copy
    c += dpp<0xB1>(odd ? x2 : x3);
    float e = hi ? c : a;
    e += dpp<0x4E>(hi ? a : c);       // quad_perm(2,3,0,1)
    e += dpp<0x124>(e);               // row_ror:4
    e += dpp<0x128>(e);               // row_ror:8
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_int(e), __float_as_int(e),
                                                      false, false);
    e = __int_as_float(r16[0]) + __int_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_int(e), __float_as_int(e),
                                                      false, false);
    e = __int_as_float(r32[0]) + __int_as_float(r32[1]);
    x0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), 0));
    x1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), 1));
    x2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), 2));
    x3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), 3));
}

// Per-token scalar math on the hardware transcendental units: v_exp_f32 and
// v_log_f32 (base 2), v_rcp_f32 and v_rsq_f32, each within about one ulp.
// They replace the correctly rounded library sequences, which cost tens of
// instructions each, in the prologue and epilogue of every unit; the
// resulting differences (order 1e-7 relative) are far inside the parity
// bars.  Limits: fexp(-inf) = 0, fexp(+inf) = +inf, frcp(+inf) = 0.
__device__ __forceinline__ float fexp(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float flog(float x)
{
    return __builtin_amdgcn_logf(x) * 0.6931471805599453f;
}

__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float frsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// softplus(x) = log(1 + e^x), linear above 20; for very negative x the sum
// 1 + e^x rounds, an absolute error below 2^-24.
__device__ __forceinline__ float softplus_fast(float x)
{
    return x > 20.0f ? x : flog(1.0f + fexp(x));
}

__device__ __forceinline__ float sigmoid_fast(float x) { return frcp(1.0f + fexp(-x)); }

}  // namespace gdn_dev
