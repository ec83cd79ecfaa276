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
// wave per group of a level and one wave per unique row of the last step,
// operands read from L2 with no LDS staging; the rows are pooled by the
// bag-major pooling kernel.
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
        *q = (uint32_t)a.ws.uniq_row[u] / (uint32_t)a.kp.dkt[*t].div[m - 1];
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
// wave per group; V_1 is the core slice G_0[i_0] itself.  The lanes take 64
// output columns (j, r) at a time and up to 8 rows p: the core slice is read
// coalesced straight from L2 (a core is small and shared by many groups), the
// parent's entries are wave-uniform and come through scalar loads.  No LDS,
// so many waves per SIMD hide the load latency.
constexpr int kKRowBlk = 8;
__global__ __launch_bounds__(kThreads) void k_klevel(KArgs a, int m)
{
    const Ws &ws = a.ws;
    const int K = a.kp.K, lane = threadIdx.x & 63;
    const int64_t ng = ws.ctrl[CTRL_KLEV + m];
    const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + uni(threadIdx.x >> 6); g < ng; g += nw) {
        const int u0 = uni(a.kp.gfirst[m][g]);
        const int t = uni(segment_of(ws.tab_uniq_start, a.T, u0));
        const auto &kt = kconst(a.kp.dkt)[t];
        const int64_t row = uni((int)ws.uniq_row[u0]);
        const int c = m - 1; // core applied at this level
        const int P = kt.P[m - 1], Rin = kt.R[m - 1], dk = kt.d[c], Rout = kt.R[m];
        // rows and digit strides are below 2^31 (checked at create): 32-bit division
        const uint32_t urow = (uint32_t)row;
        const int64_t ic = urow / (uint32_t)kt.div[c] % (uint32_t)kt.n[c];
        const float *par;
        if (m == 2) {
            const int64_t i0 = urow / (uint32_t)kt.div[0] % (uint32_t)kt.n[0];
            par = a.cores.g[t * K] + i0 * (int64_t)kt.d[0] * kt.R[1];
        } else {
            par = a.kp.V[m - 1] + (int64_t)uni(a.kp.ugrp[m - 1][u0]) * a.kp.smax[m - 1];
        }
        const auto *pc = kconst(par); // [P][Rin], wave-uniform reads
        const float *gsl = a.cores.g[t * K + c] + ic * (int64_t)Rin * dk * Rout; // [Rin][dk * Rout]
        float *out = a.kp.V[m] + g * a.kp.smax[m];                            // [P][dk * Rout]
        const int cols = dk * Rout;
        for (int c0 = 0; c0 < cols; c0 += 64) {
            const int jr = c0 + lane;
            const bool ok = jr < cols;
            const int jrc = ok ? jr : cols - 1; // clamped: loads stay inside the slice
            for (int p0 = 0; p0 < P; p0 += kKRowBlk) {
                const int np = P - p0 < kKRowBlk ? P - p0 : kKRowBlk;
                float acc[kKRowBlk];
#pragma unroll
                for (int i = 0; i < kKRowBlk; ++i) acc[i] = 0.f;
#pragma unroll 8
                for (int q = 0; q < Rin; ++q) {
                    const float gv = gsl[(int64_t)q * cols + jrc];
#pragma unroll
                    for (int i = 0; i < kKRowBlk; ++i)
                        if (i < np) acc[i] = fmaf(pc[(p0 + i) * Rin + q], gv, acc[i]);
                }
                if (ok) {
#pragma unroll
                    for (int i = 0; i < kKRowBlk; ++i)
                        if (i < np) out[(int64_t)(p0 + i) * cols + jr] = acc[i]; // row (p, j), column r
                }
            }
        }
    }
}

// Rows: E[u] = V_{K-1}[group of u] . G_{K-1}[i_{K-1}(u)], one wave per unique
// row, lanes over the D = P * d_{K-1} columns (p, j); the group's intermediate
// and the last core slice are read from L2 / L1 (both shared by many lanes).
__global__ __launch_bounds__(kThreads) void k_krows(KArgs a)
{
    const Ws &ws = a.ws;
    const int K = a.kp.K, m = K - 1, lane = threadIdx.x & 63;
    const int64_t U = ws.ctrl[CTRL_U];
    const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t u = (int64_t)blockIdx.x * (kThreads / 64) + uni(threadIdx.x >> 6); u < U; u += nw) {
        const int t = uni(segment_of(ws.tab_uniq_start, a.T, u));
        const auto &kt = kconst(a.kp.dkt)[t];
        const int P = kt.P[m], Rin = kt.R[m], dk = kt.d[K - 1], D = P * dk;
        const int g = uni(a.kp.ugrp[m][u]);
        const int64_t ik = (uint32_t)uni((int)ws.uniq_row[u]) % (uint32_t)kt.n[K - 1];
        const float *V = a.kp.V[m] + (int64_t)g * a.kp.smax[m];          // [P][Rin]
        const float *gk = a.cores.g[t * K + K - 1] + ik * (int64_t)Rin * dk; // [Rin][dk]
        float *Er = ws.E + kconst(ws.ebase)[t] + u * (int64_t)kconst(a.tab)[t].Dp;
        for (int c0 = 0; c0 < D; c0 += 64) {
            const int col = c0 + lane;
            const bool ok = col < D;
            const int cc = ok ? col : D - 1;
            const int p = cc / dk, j = cc - p * dk;
            const float *vr = V + (int64_t)p * Rin;
            float acc = 0.f;
#pragma unroll 8
            for (int q = 0; q < Rin; ++q) acc = fmaf(vr[q], gk[q * dk + j], acc);
            if (ok) Er[col] = acc;
        }
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
        const int g = p.num_blocks * 16; // 64 waves per compute unit, grid-stride
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
