// kcores.hip -- tables of K >= 4 TT cores: prefix reuse at every prefix length.
//
// The FlowTT page states the lookup as a chain of TT-core contractions whose
// early row digits select the leading cores (section 2.4), and reuses the
// intermediate of rows that share those digits (section 3.3).  With K cores a
// row i = (i_0 .. i_{K-1}) is
//     V_1 = G_0[i_0]                      [d_0][R_1]
//     V_m = V_{m-1} . G_{m-1}[i_{m-1}]    [d_0 .. d_{m-1}][R_m],  m = 2 .. K
// and the row is V_K (R_K = 1).  Rows sorted by index share V_m for every m
// up to their common prefix length, so each distinct prefix of length m
// (2 <= m <= K-1) is contracted once: a level of groups over the unique rows,
// each group's intermediate built from its parent group's one level up.
//
// gfx950 mapping: plain fp32 FMAs (shapes vary per level and table), one
// block per group with the parent intermediate and the core slice staged in
// LDS; the rows of the last level are formed per group of length K-1 and
// pooled by the bag-major pooling kernel.
#include "primitives.h"

namespace ttemb {

struct KArgs {
    const TableDesc *tab;
    int T;
    Ws ws;
    KPlan kp;
    KCorePtrs cores;
};

// Groups of unique rows that share their first m digits (scan over the unique
// rows, which are sorted by (table, row)).
struct KLevOp {
    KArgs a;
    int m;
    __device__ int64_t count() const { return a.ws.ctrl[CTRL_U]; }
    __device__ void info(int64_t u, int *t, int64_t *q) const
    {
        *t = segment_of(a.ws.tab_uniq_start, a.T, u);
        *q = (int64_t)a.ws.uniq_row[u] / a.kp.dkt[*t].div[m - 1];
    }
    __device__ uint64_t value(int64_t u) const
    {
        if (u == 0) return 1;
        int t0, t1;
        int64_t q0, q1;
        info(u - 1, &t0, &q0);
        info(u, &t1, &q1);
        return (t0 != t1 || q0 != q1) ? 1 : 0;
    }
    __device__ void emit(int64_t u, uint64_t excl, uint64_t v) const
    {
        const int32_t g = (int32_t)(excl + v) - 1;
        a.kp.ugrp[m][u] = g;
        if (v) a.kp.gfirst[m][g] = (int32_t)u;
    }
    __device__ void total(uint64_t tot, int64_t n) const
    {
        a.ws.ctrl[CTRL_KLEV + m] = (int32_t)tot;
        a.kp.gfirst[m][tot] = (int32_t)n;
    }
};

// Level m (2 <= m <= K-1): V_m[g] = V_{m-1}[parent] . G_{m-1}[i_{m-1}], one
// block per group; V_1 is the core slice G_0[i_0] itself.
__global__ __launch_bounds__(kThreads) void k_klevel(KArgs a, int m)
{
    __shared__ float Vp[kKLds];
    __shared__ float Gs[kKLds];
    const Ws &ws = a.ws;
    const int K = a.kp.K;
    const int64_t ng = ws.ctrl[CTRL_KLEV + m];
    for (int64_t g = blockIdx.x; g < ng; g += gridDim.x) {
        const int u0 = a.kp.gfirst[m][g];
        const int t = segment_of(ws.tab_uniq_start, a.T, u0);
        const KTab &kt = a.kp.dkt[t];
        const int64_t row = ws.uniq_row[u0];
        const int c = m - 1; // core applied at this level
        const int P = kt.P[m - 1], Rin = kt.R[m - 1], dk = kt.d[c], Rout = kt.R[m];
        const int64_t ic = row / kt.div[c] % kt.n[c];
        // parent intermediate [P][Rin]
        const float *par;
        if (m == 2) {
            const int64_t i0 = row / kt.div[0] % kt.n[0];
            par = a.cores.g[t * K] + i0 * (int64_t)kt.d[0] * kt.R[1];
        } else {
            par = a.kp.V[m - 1] + (int64_t)a.kp.ugrp[m - 1][u0] * a.kp.smax[m - 1];
        }
        for (int e = threadIdx.x; e < P * Rin; e += kThreads) Vp[e] = par[e];
        const float *gsl = a.cores.g[t * K + c] + ic * (int64_t)Rin * dk * Rout;
        for (int e = threadIdx.x; e < Rin * dk * Rout; e += kThreads) Gs[e] = gsl[e];
        __syncthreads();
        float *out = a.kp.V[m] + g * a.kp.smax[m];
        const int cols = dk * Rout;
        for (int e = threadIdx.x; e < P * cols; e += kThreads) {
            const int p = e / cols, jr = e - p * cols; // jr = j * Rout + r
            float acc = 0.f;
            for (int q = 0; q < Rin; ++q) acc = fmaf(Vp[p * Rin + q], Gs[q * cols + jr], acc);
            out[e] = acc; // row p * dk + j, column r
        }
        __syncthreads();
    }
}

// Rows: E[u] = V_{K-1}[group of u] . G_{K-1}[i_{K-1}(u)] for the unique rows
// of each group of length K-1 (contiguous in the unique-row order).
__global__ __launch_bounds__(kThreads) void k_krows(KArgs a)
{
    __shared__ float Vp[kKLds];
    const Ws &ws = a.ws;
    const int K = a.kp.K, m = K - 1;
    const int64_t ng = ws.ctrl[CTRL_KLEV + m];
    for (int64_t g = blockIdx.x; g < ng; g += gridDim.x) {
        const int u0 = a.kp.gfirst[m][g], u1 = a.kp.gfirst[m][g + 1];
        const int t = segment_of(ws.tab_uniq_start, a.T, u0);
        const KTab &kt = a.kp.dkt[t];
        const TableDesc &tb = a.tab[t];
        const int P = kt.P[m], Rin = kt.R[m], dk = kt.d[K - 1];
        const float *par = a.kp.V[m] + g * a.kp.smax[m];
        for (int e = threadIdx.x; e < P * Rin; e += kThreads) Vp[e] = par[e];
        __syncthreads();
        const float *GK = a.cores.g[t * K + K - 1];
        float *Et = ws.E + ws.ebase[t];
        const int D = P * dk;
        for (int64_t e = threadIdx.x; e < (int64_t)(u1 - u0) * D; e += kThreads) {
            const int r = (int)(e / D), col = (int)(e - (int64_t)r * D);
            const int u = u0 + r;
            const int64_t ik = ws.uniq_row[u] % kt.n[K - 1];
            const int p = col / dk, j = col - p * dk;
            const float *gk = GK + ik * (int64_t)Rin * dk + j; // [Rin][dk][1]
            float acc = 0.f;
            for (int q = 0; q < Rin; ++q) acc = fmaf(Vp[p * Rin + q], gk[q * dk], acc);
            Et[(int64_t)u * tb.Dp + col] = acc;
        }
        __syncthreads();
    }
}

hipError_t launch_forward_k(const Plan &p, const KCorePtrs &cores, const int64_t *offsets, float *out,
                            hipStream_t s)
{
    KArgs a{p.dtab, p.T, p.ws, p.kp, cores};
    const int K = p.kp.K;
    timer_begin(p.timing, TM_CONTRACT, s);
    if (p.nnz > 0) {
        for (int m = 2; m <= K - 1; ++m) {
            KLevOp op{a, m};
            hipError_t e = run_scan(op, p.ws.part, scan_blocks(p.nnz), s);
            if (e != hipSuccess) return e;
        }
        const int g = p.num_blocks * 8;
        for (int m = 2; m <= K - 1; ++m) hipLaunchKernelGGL(k_klevel, dim3(g), dim3(kThreads), 0, s, a, m);
        hipLaunchKernelGGL(k_krows, dim3(g), dim3(kThreads), 0, s, a);
    }
    timer_end(p.timing, TM_CONTRACT, s);
    timer_begin(p.timing, TM_POOL, s);
    hipError_t e = launch_pool(p, offsets, out, s);
    timer_end(p.timing, TM_POOL, s);
    return e != hipSuccess ? e : hipGetLastError();
}

} // namespace ttemb
