// probe_kernels.hip -- the issue probe of include/gdn_bench.h: FP32 matrix
// and FP32 vector instruction streams in two waves of each SIMD, alone and
// together.  A measurement helper, not part of the method.
//
// Compile: hipcc --offload-arch=gfx950 (gfx950 only).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Waves 0-3: two interleaved chains of n_mfma 32 x 32 x 2 FP32 matrix
// products each (mode bit 0), so that the matrix unit never waits for a
// result.  Waves 4-7, which the block places on the same four SIMDs: eight
// independent chains of n_valu FP32 FMAs (mode bit 1), enough to issue one
// FMA every cycle the SIMD allows.  Each thread stores one float.
__global__ void __launch_bounds__(512) gdn_issue_probe_kernel(float* out, int mode, int n_mfma,
                                                              int n_valu)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    float r = 0.0f;
    if (wave < 4) {
        if (mode & 1) {
            f32x16 c0 = {}, c1 = {};
            const float a = static_cast<float>(lane) * 0.001f, b = 0.5f;
            for (int i = 0; i < n_mfma; ++i) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e)
                r += c0[e] + c1[e];
        }
    } else if (mode & 2) {
        float x[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            x[c] = static_cast<float>(lane + c);
        const float y0 = 1.0001f, y1 = 0.9999f;
        for (int i = 0; i < n_valu; ++i) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                x[c] = fmaf(x[c], y0, y1);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
            r += x[c];
    }
    out[static_cast<size_t>(blockIdx.x) * 512 + threadIdx.x] = r;
}

}  // namespace

extern "C" gdn_status gdn_issue_probe(float* out, int32_t blocks, int32_t mode, int32_t n_mfma,
                                      int32_t n_valu, hipStream_t stream)
{
    gdn::clear_error();
    if (!out)
        return gdn::fail(GDN_ERR_INVALID, "out is NULL");
    if (mode < 1 || mode > 3)
        return gdn::fail(GDN_ERR_INVALID, "mode %d outside 1..3", mode);
    if (blocks < 1 || blocks > 65536)
        return gdn::fail(GDN_ERR_INVALID, "blocks %d outside 1..65536", blocks);
    if (n_mfma < 0 || n_mfma > 1000000 || n_valu < 0 || n_valu > 1000000)
        return gdn::fail(GDN_ERR_INVALID, "chain lengths %d, %d outside 0..1000000", n_mfma,
                         n_valu);
    int m = mode, nm = n_mfma, nv = n_valu;
    void* argv[] = {&out, &m, &nm, &nv};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&gdn_issue_probe_kernel),
                        dim3(static_cast<uint32_t>(blocks)), dim3(512), argv, 0, stream);
    if (e != hipSuccess)
        return gdn::fail(GDN_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}
