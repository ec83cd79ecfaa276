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
// bag-major pooling kernel.  The backward (second half of this file) walks
// the same levels in reverse, again one wave per group, and sums every core
// slice's gradient from per-row / per-group partials in a fixed order.
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
// wave per group; V_1 is the core slice G_0[i_0] itself.  When the output's
// columns (j, r) come in whole 16s the product runs on the matrix cores as
// O^T = G^T . V^T: v_mfma_f32_16x16x4_f32 with A = 16 columns of the core
// slice (read coalesced straight from L2: a core is small and shared by many
// groups), B = the parent's rows p (up to 16 per pass; fewer rows leave part
// of the tile empty), K = the shared rank Rin four at a time, so each lane
// ends with four consecutive output columns of one row p.  Other shapes take
// the FMA form: the lanes over 64 output columns at a time and up to 8 rows p,
// the parent's entries wave-uniform through scalar loads.  No LDS, so many
// waves per SIMD hide the load latency.
constexpr int kKRowBlk = 8;
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int kKLastP = 32, kKLastD = 8; // register fast path of the last level's dV
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
        if (cols % 16 == 0) {
            // Tile c of a 64-column block takes the columns cb + 4i + c (i = the
            // tile row), so lane li loads one float4 G[q][cb + 4li .. +3] for four
            // tiles, and after the products holds, over the tiles c and its
            // outputs v, the 16 consecutive columns cb + 16kq + 4v + c of row p.
            const int li = lane & 15, kq = lane >> 4;
            for (int pb = 0; pb < P; pb += 16) {
                const int p = pb + li;
                const bool okp = p < P;
                const float *vrow = par + (int64_t)(okp ? p : 0) * Rin; // B: V[p][q]
                for (int cb = 0; cb < cols; cb += 64) {
                    const bool full = cols - cb >= 64; // else a 16-, 32- or 48-column rest
                    const int nt = full ? 4 : (cols - cb) / 16;
                    floatx4 acc[4];
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) acc[c4] = floatx4{0.f, 0.f, 0.f, 0.f};
                    for (int q0 = 0; q0 < Rin; q0 += 4) {
                        const int q = q0 + kq;
                        const bool okq = q < Rin;
                        const float vb = vrow[okq ? q : 0];
                        const float bv = (okp && okq) ? vb : 0.f;
                        const float *grow = gsl + (int64_t)(okq ? q : 0) * cols + cb;
                        float ga[4];
                        if (full) {
                            const float4 g4 = *reinterpret_cast<const float4 *>(grow + 4 * li);
                            ga[0] = g4.x;
                            ga[1] = g4.y;
                            ga[2] = g4.z;
                            ga[3] = g4.w;
                        } else {
                            // the rest block: tile c takes the columns cb + 16c + i
#pragma unroll
                            for (int c4 = 0; c4 < 4; ++c4) ga[c4] = grow[16 * (c4 < nt ? c4 : 0) + li];
                        }
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4)
                            if (c4 < nt) acc[c4] = __builtin_amdgcn_mfma_f32_16x16x4f32(okq ? ga[c4] : 0.f, bv, acc[c4], 0, 0, 0);
                    }
                    if (okp) {
                        float *orow = out + (int64_t)p * cols + cb;
                        if (full) {
                            // columns 16kq + 4v + c
#pragma unroll
                            for (int v = 0; v < 4; ++v)
#pragma unroll
                                for (int c4 = 0; c4 < 4; ++c4) orow[16 * kq + 4 * v + c4] = acc[c4][v];
                        } else {
                            // columns 16c + 4kq + v
#pragma unroll
                            for (int c4 = 0; c4 < 4; ++c4)
                                if (c4 < nt)
#pragma unroll
                                    for (int v = 0; v < 4; ++v) orow[16 * c4 + 4 * kq + v] = acc[c4][v];
                        }
                    }
                }
            }
            continue;
        }
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

// ------------------------------------------------------------------ backward
//
// The backward reverses the chain (FlowTT section 3.2) with the same prefix
// sharing as the forward: a group's intermediate gradient dV_m is formed once
// from its children and passed up, and each core slice's gradient is the sum of
// per-item partials (one per unique row for the last core, one per prefix
// group for the middle cores, one per first-digit group for core 0) taken in
// a fixed order -- the items sorted stably by (table, digit) -- with no atomics.

// Last core (k = K-1), one wave per group g of prefix length K-1, its unique
// rows u in order, g_u the output-gradient row of u ([P][d] with P = P_{K-1}):
//   dV_{K-1}[g][p][q] = sum_u sum_j g_u[p][j] G_{K-1}[i(u)][q][j]
//   partial of u:  PK[u][q][j] = sum_p V_{K-1}[g][p][q] g_u[p][j]
__global__ __launch_bounds__(kThreads) void k_kb_last(KArgs a)
{
    const Ws &ws = a.ws;
    const int K = a.kp.K, m = K - 1, lane = threadIdx.x & 63;
    const int64_t ng = ws.ctrl[CTRL_KLEV + m];
    const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + uni(threadIdx.x >> 6); g < ng; g += nw) {
        const int u0 = uni(a.kp.gfirst[m][g]), u1 = uni(a.kp.gfirst[m][g + 1]);
        const int t = uni(segment_of(ws.tab_uniq_start, a.T, u0));
        const auto &kt = kconst(a.kp.dkt)[t];
        const int P = kt.P[m], Rin = kt.R[m], dk = kt.d[K - 1], Dp = kconst(a.tab)[t].Dp;
        const float *V = a.kp.V[m] + g * a.kp.smax[m];            // [P][Rin]
        const float *GK = a.cores.g[t * K + K - 1];                // [n][Rin][dk]
        const float *Et = ws.E + kconst(ws.ebase)[t];             // g_u rows, stride Dp
        float *dV = a.kp.dV[m] + g * a.kp.smax[m];
        const uint32_t nk = (uint32_t)kt.n[K - 1];
        if (dk % 4 == 0 && 16 % dk == 0 && P <= 32 && Rin <= 32) {
            // Matrix cores.  dV = sum over the rows u and j of g_u[p][j] G_u[q][j]:
            // output tiles (p block, q block), K = (u, j) four j at a time.
            // PK_u[q][j] = sum_p V[p][q] g_u[p][j]: 16 / dk rows stacked as the
            // tile rows (row slot, j), the columns q, K = p four at a time.
            const int li = lane & 15, kq = lane >> 4;
            const int npt = (P + 15) / 16, nqt = (Rin + 15) / 16;
            floatx4 acc[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int k = 0; k < 2; ++k) acc[i][k] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int u = u0; u < u1; ++u) {
                const float *gu = Et + (int64_t)u * Dp;
                const float *gs = GK + (int64_t)((uint32_t)uni(ws.uniq_row[u]) % nk) * Rin * dk;
                for (int jb = 0; jb < dk; jb += 4) {
                    const int j = jb + kq;
                    float av[2], bv[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int p = i * 16 + li, q = i * 16 + li;
                        const float x = gu[(p < P ? p : 0) * dk + j], y = gs[(q < Rin ? q : 0) * dk + j];
                        av[i] = p < P ? x : 0.f;
                        bv[i] = q < Rin ? y : 0.f;
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int k = 0; k < 2; ++k)
                            if (i < npt && k < nqt) acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[k], acc[i][k], 0, 0, 0);
                }
            }
            // lane (kq, li) holds dV[p = 16i + 4kq + v][q = 16k + li]
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int q = 16 * k + li;
                    if (i < npt && k < nqt && q < Rin) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int p = 16 * i + 4 * kq + v;
                            if (p < P) dV[p * Rin + q] = acc[i][k][v];
                        }
                    }
                }
            const int RT = 16 / dk, slot = li / dk, jl = li - slot * dk;
            for (int r0 = u0; r0 < u1; r0 += RT) {
                const int us = r0 + slot < u1 ? r0 + slot : u1 - 1; // padding slots: the tile's last row
                const float *gu = Et + (int64_t)us * Dp + jl;       // g_u[p][jl] at p * dk
                floatx4 pa[2];
                pa[0] = pa[1] = floatx4{0.f, 0.f, 0.f, 0.f};
                for (int p0 = 0; p0 < P; p0 += 4) {
                    const int p = p0 + kq;
                    const bool okp = p < P;
                    const float x = gu[(okp ? p : 0) * dk];
                    const float ax = okp ? x : 0.f;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int q = 16 * k + li;
                        const float y = V[(okp ? p : 0) * Rin + (q < Rin ? q : 0)];
                        if (k < nqt) pa[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(ax, (okp && q < Rin) ? y : 0.f, pa[k], 0, 0, 0);
                    }
                }
                // lane (kq, li) holds PK of row slot (4kq+v)/dk, j = (4kq+v)%dk, q = 16k + li
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int q = 16 * k + li;
                    if (k < nqt && q < Rin) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int r = 4 * kq + v, sl = r / dk, jj = r - sl * dk;
                            if (r0 + sl < u1) a.kp.PK[(int64_t)(r0 + sl) * a.kp.pkmax + q * dk + jj] = pa[k][v];
                        }
                    }
                }
            }
            continue;
        }
        if (P <= kKLastP && Rin <= 64 && dk <= kKLastD) {
            // lane q keeps the P sums of column q; the rows' g_u entries are
            // wave-uniform (scalar loads), the lane's G slice column in
            // registers; same sums, same order (rows, then j)
            const int q = lane < Rin ? lane : Rin - 1;
            float acc[kKLastP];
#pragma unroll
            for (int p = 0; p < kKLastP; ++p) acc[p] = 0.f;
            for (int u = u0; u < u1; ++u) {
                const auto *gu = kconst(Et + (int64_t)u * Dp);
                const float *gs = GK + (int64_t)((uint32_t)uni(ws.uniq_row[u]) % (uint32_t)kt.n[K - 1]) * Rin * dk + q * dk;
                float gq[kKLastD];
#pragma unroll
                for (int j = 0; j < kKLastD; ++j) gq[j] = j < dk ? gs[j] : 0.f;
#pragma unroll
                for (int p = 0; p < kKLastP; ++p) {
                    if (p >= P) break;
#pragma unroll
                    for (int j = 0; j < kKLastD; ++j)
                        if (j < dk) acc[p] = fmaf(gu[p * dk + j], gq[j], acc[p]);
                }
            }
            if (lane < Rin) {
#pragma unroll
                for (int p = 0; p < kKLastP; ++p)
                    if (p < P) dV[p * Rin + lane] = acc[p];
            }
        } else {
            for (int e0 = 0; e0 < P * Rin; e0 += 64) {
                const int e = e0 + lane;
                const int ec = e < P * Rin ? e : P * Rin - 1;
                const int p = ec / Rin, q = ec - p * Rin;
                float acc = 0.f;
                for (int u = u0; u < u1; ++u) {
                    const float *gu = Et + (int64_t)u * Dp + p * dk;
                    const float *gs = GK + (int64_t)((uint32_t)ws.uniq_row[u] % (uint32_t)kt.n[K - 1]) * Rin * dk + q * dk;
                    for (int j = 0; j < dk; ++j) acc = fmaf(gu[j], gs[j], acc);
                }
                if (e < P * Rin) dV[e] = acc;
            }
        }
        for (int u = u0; u < u1; ++u) {
            const float *gu = Et + (int64_t)u * Dp;
            float *pk = a.kp.PK + (int64_t)u * a.kp.pkmax;
            for (int e0 = 0; e0 < Rin * dk; e0 += 64) {
                const int e = e0 + lane;
                const int ec = e < Rin * dk ? e : Rin * dk - 1;
                const int q = ec / dk, j = ec - q * dk;
                float acc = 0.f;
                for (int p = 0; p < P; ++p) acc = fmaf(V[p * Rin + q], gu[p * dk + j], acc);
                if (e < Rin * dk) pk[e] = acc;
            }
        }
    }
}

// Level m (K-1 down to 2), core c = m-1, per prefix-m group g with parent pg
// (its prefix-(m-1) group) and core slice G = G_c[i_c(g)] ([Rin][dk * Rout]):
//   dV_{m-1}[pg][p][q] = sum_g sum_{(j,r)} dV_m[g][p][(j,r)] G[q][(j,r)]
//   partial of g:  Q_m[g][q][(j,r)] = sum_p V_{m-1}[pg][p][q] dV_m[g][p][(j,r)]
// k_kb_q takes one wave per group g and forms its partial Q_m[g] and its
// contribution Cc_m[g] = dV_m[g] . G^T to the parent; k_kb_level then adds the
// contributions of each parent's children (consecutive groups) in order.
// V_1 of a first-digit group is the core slice G_0[i_0].
__global__ __launch_bounds__(kThreads) void k_kb_q(KArgs a, int m)
{
    const Ws &ws = a.ws;
    const int K = a.kp.K, lane = threadIdx.x & 63, c = m - 1;
    const int64_t ng = ws.ctrl[CTRL_KLEV + m];
    const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + uni(threadIdx.x >> 6); g < ng; g += nw) {
        const int r0 = uni(a.kp.gfirst[m][g]);
        const int t = uni(segment_of(ws.tab_uniq_start, a.T, r0));
        const auto &kt = kconst(a.kp.dkt)[t];
        const int P = kt.P[m - 1], Rin = kt.R[m - 1], dk = kt.d[c], Rout = kt.R[m], cols = dk * Rout;
        const uint32_t urow = (uint32_t)ws.uniq_row[r0];
        const float *Vp;
        if (m == 2) {
            const uint32_t i0 = urow / (uint32_t)kt.div[0] % (uint32_t)kt.n[0];
            Vp = a.cores.g[t * K] + (int64_t)i0 * kt.d[0] * kt.R[1];
        } else {
            Vp = a.kp.V[m - 1] + (int64_t)uni(a.kp.ugrp[m - 1][r0]) * a.kp.smax[m - 1];
        }
        const uint32_t ic = urow / (uint32_t)kt.div[c] % (uint32_t)kt.n[c];
        const float *gsl = a.cores.g[t * K + c] + (int64_t)ic * Rin * cols; // [Rin][cols]
        const float *dv = a.kp.dV[m] + g * a.kp.smax[m];                   // [P][cols]
        float *qo = a.kp.Q[m] + g * a.kp.qmax[m];
        if (cols % 16 == 0 && a.kp.smax[m] % 4 == 0 && a.kp.qmax[m] % 4 == 0) {
            // Matrix cores (float4 rows of dV_m and of the core slice: the
            // workspace strides are multiples of 4 floats and cores 16-byte
            // aligned).  Q^T[col][q] = sum_p dV[p][col] Vp[p][q]: tiles of 16
            // columns (tile c of a 64-column block takes the columns cb + 4i + c,
            // so one float4 feeds four tiles), the parent's columns q as B,
            // K = p four at a time.
            const int li = lane & 15, kq = lane >> 4;
            for (int qb = 0; qb < Rin; qb += 16) {
                const int q = qb + li;
                const bool okq = q < Rin;
                for (int cb = 0; cb < cols; cb += 64) {
                    const bool full = cols - cb >= 64;
                    const int nt = full ? 4 : (cols - cb) / 16;
                    floatx4 acc[4];
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) acc[c4] = floatx4{0.f, 0.f, 0.f, 0.f};
                    for (int p0 = 0; p0 < P; p0 += 4) {
                        const int pp = p0 + kq;
                        const bool okp = pp < P;
                        const float vb = Vp[(okp ? pp : 0) * Rin + (okq ? q : 0)];
                        const float bv = (okp && okq) ? vb : 0.f;
                        const float *drow = dv + (int64_t)(okp ? pp : 0) * cols + cb;
                        float da[4];
                        if (full) {
                            const float4 d4 = *reinterpret_cast<const float4 *>(drow + 4 * li);
                            da[0] = d4.x;
                            da[1] = d4.y;
                            da[2] = d4.z;
                            da[3] = d4.w;
                        } else {
#pragma unroll
                            for (int c4 = 0; c4 < 4; ++c4) da[c4] = drow[16 * (c4 < nt ? c4 : 0) + li];
                        }
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4)
                            if (c4 < nt) acc[c4] = __builtin_amdgcn_mfma_f32_16x16x4f32(okp ? da[c4] : 0.f, bv, acc[c4], 0, 0, 0);
                    }
                    if (okq) {
                        float *orow = qo + (int64_t)q * cols + cb;
                        if (full) {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                *reinterpret_cast<float4 *>(orow + 16 * kq + 4 * v) =
                                    make_float4(acc[0][v], acc[1][v], acc[2][v], acc[3][v]);
                        } else {
#pragma unroll
                            for (int c4 = 0; c4 < 4; ++c4)
                                if (c4 < nt)
                                    *reinterpret_cast<float4 *>(orow + 16 * c4 + 4 * kq) =
                                        make_float4(acc[c4][0], acc[c4][1], acc[c4][2], acc[c4][3]);
                        }
                    }
                }
            }
            // Cc[p][q] = sum_col dV[p][col] G[q][col]: K = the columns, in each
            // block of 16 lane kq takes the columns 4kq .. 4kq+3 over four steps
            // (one float4 of each operand; the sum covers every column once)
            float *cc = a.kp.Cc[m] + g * a.kp.smax[m - 1];
            for (int pb = 0; pb < P; pb += 16) {
                const int pr = pb + li;
                const bool okp = pr < P;
                for (int qb = 0; qb < Rin; qb += 32) {
                    floatx4 acc[2];
                    acc[0] = acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
                    for (int c16 = 0; c16 < cols; c16 += 16) {
                        const float4 a4 = *reinterpret_cast<const float4 *>(dv + (int64_t)(okp ? pr : 0) * cols + c16 + 4 * kq);
                        float4 b4[2];
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2) {
                            const int q = qb + 16 * k2 + li;
                            b4[k2] = *reinterpret_cast<const float4 *>(gsl + (int64_t)(q < Rin ? q : 0) * cols + c16 + 4 * kq);
                        }
                        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2) {
                            const bool okq = qb + 16 * k2 + li < Rin;
                            const float bv[4] = {b4[k2].x, b4[k2].y, b4[k2].z, b4[k2].w};
                            if (qb + 16 * k2 < Rin) {
#pragma unroll
                                for (int s4 = 0; s4 < 4; ++s4)
                                    acc[k2] = __builtin_amdgcn_mfma_f32_16x16x4f32(okp ? av[s4] : 0.f, okq ? bv[s4] : 0.f,
                                                                                  acc[k2], 0, 0, 0);
                            }
                        }
                    }
                    // lane (kq, li) holds Cc[p = pb + 4kq + v][q = qb + 16k2 + li]
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        const int q = qb + 16 * k2 + li;
                        if (q < Rin) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int p = pb + 4 * kq + v;
                                if (p < P) cc[p * Rin + q] = acc[k2][v];
                            }
                        }
                    }
                }
            }
            continue;
        }
        if (P <= kKRowBlk) {
            // lanes over the columns (j, r): the P entries of dV_m in registers,
            // the parent's entries wave-uniform (scalar loads); same sums, same order
            const auto *vpc = kconst(Vp);
            for (int j0 = 0; j0 < cols; j0 += 64) {
                const int jr = j0 + lane;
                const bool ok = jr < cols;
                const int jc = ok ? jr : cols - 1;
                float dvr[kKRowBlk];
#pragma unroll
                for (int i = 0; i < kKRowBlk; ++i) dvr[i] = i < P ? dv[i * cols + jc] : 0.f;
                for (int q = 0; q < Rin; ++q) {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < kKRowBlk; ++i)
                        if (i < P) acc = fmaf(vpc[i * Rin + q], dvr[i], acc);
                    if (ok) qo[q * cols + jr] = acc;
                }
            }
        } else {
            for (int e0 = 0; e0 < Rin * cols; e0 += 64) {
                const int e = e0 + lane;
                const int ec = e < Rin * cols ? e : Rin * cols - 1;
                const int q = ec / cols, jr = ec - q * cols;
                float acc = 0.f;
#pragma unroll 4
                for (int p = 0; p < P; ++p) acc = fmaf(Vp[p * Rin + q], dv[p * cols + jr], acc);
                if (e < Rin * cols) qo[e] = acc;
            }
        }
        float *cc = a.kp.Cc[m] + g * a.kp.smax[m - 1];
        for (int e0 = 0; e0 < P * Rin; e0 += 64) {
            const int e = e0 + lane;
            const int ec = e < P * Rin ? e : P * Rin - 1;
            const int p = ec / Rin, q = ec - p * Rin;
            const float *dvr = dv + p * cols, *gr = gsl + q * cols;
            float acc = 0.f;
#pragma unroll 8
            for (int jr = 0; jr < cols; ++jr) acc = fmaf(dvr[jr], gr[jr], acc);
            if (e < P * Rin) cc[e] = acc;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_kb_level(KArgs a, int m)
{
    const Ws &ws = a.ws;
    const int lane = threadIdx.x & 63;
    const int64_t np = ws.ctrl[CTRL_KLEV + m - 1];
    const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t pg = (int64_t)blockIdx.x * (kThreads / 64) + uni(threadIdx.x >> 6); pg < np; pg += nw) {
        const int r0 = uni(a.kp.gfirst[m - 1][pg]), r1 = uni(a.kp.gfirst[m - 1][pg + 1]);
        const int g0 = uni(a.kp.ugrp[m][r0]), g1 = uni(a.kp.ugrp[m][r1 - 1]) + 1; // children [g0, g1)
        const int t = uni(segment_of(ws.tab_uniq_start, a.T, r0));
        const auto &kt = kconst(a.kp.dkt)[t];
        const int n = kt.P[m - 1] * kt.R[m - 1];
        float *dVp = a.kp.dV[m - 1] + pg * a.kp.smax[m - 1];
        for (int e = lane; e < n; e += 64) {
            float acc = 0.f;
            for (int g = g0; g < g1; ++g) acc += a.kp.Cc[m][g * a.kp.smax[m - 1] + e];
            dVp[e] = acc;
        }
    }
}

// Sort keys of the items whose partials make up core k's slices: item i is a
// unique row (k = K-1) or a group of prefix length m (k = m-1; m = 1 for
// k = 0); key = the slice (table base + digit k of the item's first row).
__global__ __launch_bounds__(kThreads) void k_kb_keys(KArgs a, int k, int m, uint32_t *keys, int32_t *vals)
{
    const Ws &ws = a.ws;
    const int64_t n = m == 0 ? ws.ctrl[CTRL_U] : ws.ctrl[CTRL_KLEV + m];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int u = m == 0 ? (int)i : a.kp.gfirst[m][i];
        const int t = segment_of(ws.tab_uniq_start, a.T, u);
        const KTab &kt = a.kp.dkt[t];
        const uint32_t dig = (uint32_t)ws.uniq_row[u] / (uint32_t)kt.div[k] % (uint32_t)kt.n[k];
        keys[i] = (uint32_t)kt.nbase[k] + dig;
        vals[i] = (int32_t)i;
    }
}

// dG_k of table t from the sorted partials, in two fixed-order passes so that
// a slice with many items is spread over kKbSplit blocks: pass 1, block
// (slice i, part c) sums part c of the slice's items (its stable sorted order,
// cut into kKbSplit near-equal ranges, four interleaved accumulators added in a
// fixed order) into red[i][c]; pass 2 adds the kKbSplit sums of each slice in
// order.  A slice no item touches gets 0 (m < 0: no items at all).
constexpr int kKbSplit = 16;
__global__ __launch_bounds__(kThreads) void k_kb_reduce1(KArgs a, int t, int k, int m, const uint32_t *keys,
                                                         const int32_t *vals, const float *part, int64_t pstride,
                                                         float *red)
{
    const Ws &ws = a.ws;
    const KTab &kt = a.kp.dkt[t];
    const int64_t n = m < 0 ? 0 : (m == 0 ? ws.ctrl[CTRL_U] : ws.ctrl[CTRL_KLEV + m]);
    const int S = kt.R[k] * kt.d[k] * kt.R[k + 1];
    const int c = blockIdx.y;
    for (int i = blockIdx.x; i < kt.n[k]; i += gridDim.x) {
        const uint32_t key = (uint32_t)kt.nbase[k] + (uint32_t)i;
        int64_t lo = 0, hi = n; // first item with key >= key
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (keys[mid] < key) lo = mid + 1;
            else hi = mid;
        }
        int64_t lo2 = lo, hi2 = n; // first item with key > key
        while (lo2 < hi2) {
            const int64_t mid = (lo2 + hi2) >> 1;
            if (keys[mid] <= key) lo2 = mid + 1;
            else hi2 = mid;
        }
        const int64_t len = lo2 - lo;
        const int64_t b = lo + len * c / kKbSplit, e1 = lo + len * (c + 1) / kKbSplit;
        for (int e = threadIdx.x; e < S; e += blockDim.x) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            int64_t j = b;
            for (; j + 4 <= e1; j += 4) {
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[x] += part[(int64_t)vals[j + x] * pstride + e];
            }
            for (; j < e1; ++j) acc[0] += part[(int64_t)vals[j] * pstride + e];
            red[((int64_t)i * kKbSplit + c) * S + e] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_kb_reduce2(KArgs a, int t, int k, const float *red, float *dG)
{
    const KTab &kt = a.kp.dkt[t];
    const int S = kt.R[k] * kt.d[k] * kt.R[k + 1];
    for (int i = blockIdx.x; i < kt.n[k]; i += gridDim.x)
        for (int e = threadIdx.x; e < S; e += blockDim.x) {
            float acc = 0.f;
            for (int c = 0; c < kKbSplit; ++c) acc += red[((int64_t)i * kKbSplit + c) * S + e];
            dG[(int64_t)i * S + e] = acc;
        }
}

hipError_t launch_backward_k(const Plan &p, const float *grad_out, const KCorePtrs &cores, const int64_t *offsets,
                             float *const *core_grads, hipStream_t s)
{
    KArgs a{p.dtab, p.T, p.ws, p.kp, cores};
    const int K = p.kp.K;
    timer_begin(p.timing, TM_BWD_GATHER, s);
    hipError_t e = launch_gu_gather(p, grad_out, offsets, s);
    if (e != hipSuccess) return e;
    timer_end(p.timing, TM_BWD_GATHER, s);
    timer_begin(p.timing, TM_BWD_CONTRACT, s);
    const int g = p.num_blocks * 16;
    if (p.nnz > 0) {
        // groups of every prefix length 1..K-1 and the forward intermediates
        // (lengths 2..K-1 kept from the forward when the caller says so)
        for (int m = 1; m <= (p.reuse_c ? 1 : K - 1); ++m) {
            KLevOp op{a, m};
            if ((e = run_scan(op, p.ws.part, scan_blocks(p.nnz), s)) != hipSuccess) return e;
        }
        if (!p.reuse_c)
            for (int m = 2; m <= K - 1; ++m) hipLaunchKernelGGL(k_klevel, dim3(g), dim3(kThreads), 0, s, a, m);
        hipLaunchKernelGGL(k_kb_last, dim3(g), dim3(kThreads), 0, s, a);
        for (int m = K - 1; m >= 2; --m) {
            hipLaunchKernelGGL(k_kb_q, dim3(g), dim3(kThreads), 0, s, a, m);
            hipLaunchKernelGGL(k_kb_level, dim3(g), dim3(kThreads), 0, s, a, m);
        }
    }
    timer_end(p.timing, TM_BWD_CONTRACT, s);
    timer_begin(p.timing, TM_BWD_REDUCE, s);
    for (int k = 0; k < K; ++k) {
        // items of core k: first-digit groups (k = 0), prefix-(k+1) groups, unique rows (k = K-1)
        const int m = k == K - 1 ? 0 : k + 1;
        const float *part = k == K - 1 ? p.kp.PK : (k == 0 ? p.kp.dV[1] : p.kp.Q[k + 1]);
        const int64_t pstride = k == K - 1 ? p.kp.pkmax : (k == 0 ? p.kp.smax[1] : p.kp.qmax[k + 1]);
        const uint32_t *keys = p.ws.keys0;
        const int32_t *vals = p.ws.u3order;
        if (p.nnz > 0) {
            int gk = ceil_div(p.nnz, kThreads);
            gk = gk > 4096 ? 4096 : gk;
            hipLaunchKernelGGL(k_kb_keys, dim3(gk), dim3(kThreads), 0, s, a, k, m, p.ws.keys0, p.ws.u3order);
            bool in1 = false;
            const int32_t *cnt = m == 0 ? &p.ws.ctrl[CTRL_U] : &p.ws.ctrl[CTRL_KLEV + m];
            if ((e = radix_sort_pairs(p, p.ws.keys0, p.ws.u3order, p.ws.keys1, p.ws.uvals_free, p.nnz, cnt,
                                      p.kp.key_bits[k], &in1, s)) != hipSuccess)
                return e;
            keys = in1 ? p.ws.keys1 : p.ws.keys0;
            vals = in1 ? p.ws.uvals_free : p.ws.u3order;
        }
        // a call with no lookups reads no item and zeroes every slice
        for (int t = 0; t < p.T; ++t) {
            const int ns = p.kp_n[t * K + k], gb = ns < 1024 ? ns : 1024;
            hipLaunchKernelGGL(k_kb_reduce1, dim3(gb, kKbSplit), dim3(kThreads), 0, s, a, t, k, p.nnz > 0 ? m : -1,
                               keys, vals, part, pstride, p.kp.red);
            hipLaunchKernelGGL(k_kb_reduce2, dim3(gb), dim3(kThreads), 0, s, a, t, k, p.kp.red, core_grads[t * K + k]);
        }
    }
    timer_end(p.timing, TM_BWD_REDUCE, s);
    return hipGetLastError();
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
