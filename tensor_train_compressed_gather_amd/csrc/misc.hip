// misc.hip -- SGD update and fills (gfx950).
#include "internal.h"

namespace ttemb {

// G <- G - lr * dG over one core (plain SGD step of the training workload).
__global__ __launch_bounds__(kThreads) void k_sgd(float *g, const float *dg, int64_t n, float lr)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool vec = ((reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(dg)) & 15u) == 0;
    if (vec) {
        const int64_t n4 = n >> 2;
        float4 *g4 = reinterpret_cast<float4 *>(g);
        const float4 *d4 = reinterpret_cast<const float4 *>(dg);
        for (int64_t i = tid; i < n4; i += stride) {
            float4 a = g4[i];
            const float4 d = d4[i];
            a.x = fmaf(-lr, d.x, a.x);
            a.y = fmaf(-lr, d.y, a.y);
            a.z = fmaf(-lr, d.z, a.z);
            a.w = fmaf(-lr, d.w, a.w);
            g4[i] = a;
        }
        for (int64_t i = (n4 << 2) + tid; i < n; i += stride) g[i] = fmaf(-lr, dg[i], g[i]);
    } else {
        for (int64_t i = tid; i < n; i += stride) g[i] = fmaf(-lr, dg[i], g[i]);
    }
}

__global__ __launch_bounds__(kThreads) void k_fill_i32(int32_t *p, int32_t v, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ __launch_bounds__(kThreads) void k_fill_f32(float *p, float v, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

static int grid_for(int64_t n, int per_thread)
{
    int64_t g = (n + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
    if (g < 1) g = 1;
    if (g > 8192) g = 8192;
    return (int)g;
}

hipError_t launch_sgd(float *g, const float *dg, int64_t count, float lr, hipStream_t s)
{
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sgd, dim3(grid_for(count, 16)), dim3(kThreads), 0, s, g, dg, count, lr);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int32_t v, int64_t count, hipStream_t s)
{
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3(grid_for(count, 4)), dim3(kThreads), 0, s, p, v, count);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, float v, int64_t count, hipStream_t s)
{
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(count, 4)), dim3(kThreads), 0, s, p, v, count);
    return hipGetLastError();
}

} // namespace ttemb
