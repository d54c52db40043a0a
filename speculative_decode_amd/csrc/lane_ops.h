// lane_ops.h -- cross-lane sums over 8-lane row groups and over a wave64,
// built from DPP row operations, shared by the HIP kernels.
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

}  // namespace gdn_dev
