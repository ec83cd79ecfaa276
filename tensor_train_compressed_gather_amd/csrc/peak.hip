// peak.hip -- measured peak of the FP32 matrix cores on this device, the
// figure the contraction kernels' achieved rates are also compared against
// (besides the datasheet's 157.3 TFLOP/s).  Each wave runs eight independent
// chains of v_mfma_f32_16x16x4_f32 (no loads, no LDS), so nothing but the
// matrix-core issue rate bounds it.
#include "../../include/tt_emb.h"
#include "internal.h"

namespace ttemb {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_mfma_peak(float *out, int iters)
{
    const int lane = threadIdx.x & 63;
    float a = 1.0f + 1e-7f * lane, b = 1.0f - 1e-7f * lane;
    floatx4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    // one store per block keeps the chains live
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

} // namespace ttemb

extern "C" int tt_emb_peak_mfma(int32_t blocks, int32_t iters, float *out, void *stream)
{
    if (blocks <= 0 || iters <= 0 || !out) return TT_EMB_ERR_ARG;
    hipLaunchKernelGGL(ttemb::k_mfma_peak, dim3(blocks), dim3(ttemb::kThreads), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? TT_EMB_OK : TT_EMB_ERR_HIP;
}
