// misc.hip -- SGD update and fills (gfx950).
#include "internal.h"

namespace ttemb {

// G <- G - lr * dG over a batch of cores (plain SGD step of the training
// workload).  Core k owns blocks [blk[k], blk[k+1]) of the grid, each block a
// contiguous span of kSgdSpan elements; every pointer is 16-byte aligned.
constexpr int kSgdSpan = kThreads * 4 * 4;

__global__ __launch_bounds__(kThreads) void k_sgd(SgdBatch b, float lr)
{
    int k = 0;
    while (k + 1 < b.n && b.blk[k + 1] <= (int)blockIdx.x) ++k;
    const int64_t n = b.cnt[k];
    const int64_t lo = (int64_t)(blockIdx.x - b.blk[k]) * kSgdSpan;
    const int64_t hi = lo + kSgdSpan < n ? lo + kSgdSpan : n;
    float *g = b.g[k];
    const float *dg = b.dg[k];
    const int64_t hi4 = lo + ((hi - lo) & ~int64_t(3));
#pragma unroll 4
    for (int64_t i = lo + 4 * threadIdx.x; i < hi4; i += 4 * kThreads) {
        float4 a = *reinterpret_cast<float4 *>(g + i);
        const float4 d = *reinterpret_cast<const float4 *>(dg + i);
        a.x = fmaf(-lr, d.x, a.x);
        a.y = fmaf(-lr, d.y, a.y);
        a.z = fmaf(-lr, d.z, a.z);
        a.w = fmaf(-lr, d.w, a.w);
        *reinterpret_cast<float4 *>(g + i) = a;
    }
    for (int64_t i = hi4 + threadIdx.x; i < hi; i += kThreads) g[i] = fmaf(-lr, dg[i], g[i]);
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

hipError_t launch_sgd(float *const *g, const float *const *dg, const int64_t *count, int ncores, float lr,
                      hipStream_t s)
{
    SgdBatch b{};
    auto flush = [&]() -> hipError_t {
        if (b.n == 0) return hipSuccess;
        hipLaunchKernelGGL(k_sgd, dim3(b.blk[b.n]), dim3(kThreads), 0, s, b, lr);
        b = SgdBatch{};
        return hipGetLastError();
    };
    for (int k = 0; k < ncores; ++k) {
        if (count[k] <= 0) continue;
        const int64_t nb = (count[k] + kSgdSpan - 1) / kSgdSpan;
        if (b.n == kSgdMaxCores || (int64_t)b.blk[b.n] + nb > 0x7fffffff) {
            hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        b.g[b.n] = g[k];
        b.dg[b.n] = dg[k];
        b.cnt[b.n] = count[k];
        b.blk[b.n + 1] = b.blk[b.n] + (int)nb;
        ++b.n;
    }
    return flush();
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
