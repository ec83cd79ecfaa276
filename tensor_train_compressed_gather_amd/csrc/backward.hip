// backward.hip -- prefix-grouped reverse TT contraction on gfx950.
//
// The FlowTT page ("FlowTT: Exploiting Computation Flow Reuse in Irregular
// Tensor-Train Embedding", section 3.2) states that the backward reverses the
// forward C = A.B, E = C.D, pooling; section 4 notes that it dominates the
// training cost.  For the loss sum(grad_out * out), with g_u the sum of the
// output gradients of every lookup of unique row u:
//   dE_u        = g_u                                  (reverse pooling)
//   dC_p       += g_u . G3[i3_u]^T        over the rows u of prefix unit p
//   dG3[i3]    += C_p^T . g_u             over unique rows with that i3
//   dG1[i1]    += dC_p . G2[i2]^T         over units with that i1
//   dG2[i2]    += G1[i1]^T . dC_p         over units with that i2
// Every sum runs in a fixed order and no floating-point atomic touches a
// result, so the gradients are bit-reproducible:
//   * g_u is summed over the sorted lookup run of u; the sorted positions are
//     cut into fixed tasks and the parts of a run cut by task edges are added
//     in task order;
//   * one block owns one run of units sharing (table, i2) and keeps dG2[i2] in
//     registers, writing it once;
//   * dG1 and dG3 contributions go to per-unit / per-row partial buffers and
//     are reduced per slice in canonical order (units sorted by prefix, rows
//     re-sorted stably by i3).
#include "primitives.h"

namespace ttemb {

struct BwdArgs {
    const TableDesc *tab;
    int T;
    int64_t B;
    Ws ws;
    CorePtrs cores;
    GradPtrs grads;
    const float *grad_out;
    const int64_t *offsets;
    int64_t nnz;
    int SD;
    int gstride; // row stride of the gather partial slots (max Dp)
    int force_generic;
    int g1stride; // row stride of the G1 partials (max d1*R1)
    int g2p_slots; // dG2 partial slots in the workspace (pieces of split runs)
};

// Bag within its table of every lookup, in lookup order.  A block takes
// kThreads bags; their lookups are contiguous, so lanes walk them coalesced
// and find their bag by binary search over the block's offsets in LDS.
__global__ __launch_bounds__(kThreads) void k_lookup_meta(BwdArgs a)
{
    __shared__ int64_t so[kThreads + 1];
    const int64_t nbags = (int64_t)a.T * a.B;
    for (int64_t b0 = (int64_t)blockIdx.x * kThreads; b0 < nbags; b0 += (int64_t)gridDim.x * kThreads) {
        const int nb = nbags - b0 < kThreads ? (int)(nbags - b0) : kThreads;
        for (int i = threadIdx.x; i <= nb; i += kThreads) {
            const int64_t o = a.offsets[b0 + i];
            so[i] = o < 0 ? 0 : (o > a.nnz ? a.nnz : o);
        }
        __syncthreads();
        const int64_t lo = so[0], hi = so[nb];
        for (int64_t l = lo + threadIdx.x; l < hi; l += kThreads) {
            int i0 = 0, i1 = nb; // last i < nb with so[i] <= l
            while (i1 - i0 > 1) {
                const int mid = (i0 + i1) >> 1;
                if (so[mid] <= l) i0 = mid;
                else i1 = mid;
            }
            const int64_t b = b0 + i0;
            a.ws.lb[l] = (int)(b - (b / a.B) * a.B);
        }
        __syncthreads();
    }
}

// Gather task numbering.  The sorted positions of table t,
// [tstart[t], tstart[t+1]), are cut into tasks of kGuTask positions; table t
// owns tasks [base[t], base[t+1]) of the global order (partial slots, cut-run
// records).  The gather works on ids over (table, column piece, task): table t
// holds ids [qb[t], qb[t+1]), piece-major.  The prefixes are built in LDS by
// wave 0.  Per-table values a gather task needs are copied to LDS once per
// block so that no global load issued between a worker's stores has to wait
// for them.
struct GuTab {
    int64_t ebase;
    int ts, te, u0, u1, D, Dp, col_off, ntask;
};

__device__ void gu_bases(const BwdArgs &a, int *base, int *qb, GuTab *gt)
{
    if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        int n = 0, q = 0;
        if (t < a.T) {
            const TableDesc &tb = a.tab[t];
            const int len = a.ws.tstart[t + 1] - a.ws.tstart[t];
            n = len > 0 ? (len + kGuTask - 1) / kGuTask : 0;
            q = n * (tb.D > kGuCols ? (tb.D + kGuCols - 1) / kGuCols : 1);
            gt[t] = GuTab{a.ws.ebase[t], a.ws.tstart[t], a.ws.tstart[t + 1], a.ws.tab_uniq_start[t],
                          a.ws.tab_uniq_start[t + 1], tb.D, tb.Dp, tb.col_off, n};
        }
        for (int o = 1; o < 64; o <<= 1) {
            const int yn = __shfl_up(n, o, 64), yq = __shfl_up(q, o, 64);
            if (t >= o) {
                n += yn;
                q += yq;
            }
        }
        if (t == 0) base[0] = qb[0] = 0;
        if (t < a.T) {
            base[t + 1] = n;
            qb[t + 1] = q;
        }
    }
    __syncthreads();
}

// Last table t < T with pre[t] <= id (pre non-decreasing, pre[0] = 0 <= id).
__device__ inline int gu_table(const int *pre, int T, int id)
{
    int lo = 0, hi = T;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= id) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Sorted-order metadata of the gather: Ws::sm[k] = (bag of the lookup at
// sorted position k, its unique row).  Chunks of kSmChunk positions; the
// blocks of virtual XCD x = blockIdx % 8 (launched in multiples of 8) take
// the x-th eighth of the chunks, so the random reads of lb stay inside the
// few tables that one L2 holds.  The unique row comes from the run starts:
// the block loads the starts of the runs from the one holding its first
// position (inv of that lookup) on, and each lane finds the last start at or
// before its position.
constexpr int kSmPer = 4, kSmChunk = kSmPer * kThreads;

__global__ __launch_bounds__(kThreads) void k_sorted_meta(BwdArgs a)
{
    __shared__ int win[kSmChunk + 1];
    const Ws &ws = a.ws;
    const int64_t n = a.nnz, nch = (n + kSmChunk - 1) / kSmChunk;
    const int x = blockIdx.x & 7, nbx = gridDim.x >> 3;
    const int64_t c_hi = nch * (x + 1) / 8;
    const int U = ws.ctrl[CTRL_U];
    for (int64_t c = nch * x / 8 + (blockIdx.x >> 3); c < c_hi; c += nbx) {
        const int64_t p0 = c * kSmChunk;
        int l[kSmPer];
#pragma unroll
        for (int i = 0; i < kSmPer; ++i) {
            const int64_t pos = p0 + threadIdx.x + i * kThreads;
            l[i] = ws.perm[pos < n ? pos : n - 1];
        }
        int u0 = ws.inv[ws.perm[p0]];
        // the bags of the chunk's lookups, all in flight before any store of
        // this chunk (a load behind a store waits for it: one counter for both)
        int bg[kSmPer];
#pragma unroll
        for (int i = 0; i < kSmPer; ++i) bg[i] = ws.lb[l[i]];
        u0 = u0 < 0 ? 0 : (u0 >= U ? U - 1 : u0);
        __syncthreads(); // previous chunk's window read
        // window of run starts: unconditional loads at clamped positions
        // (uniq_start holds U + 1 entries), then the entries past U masked
        constexpr int kWinPer = (kSmChunk + 1 + kThreads - 1) / kThreads;
        int wv[kWinPer];
#pragma unroll
        for (int k = 0; k < kWinPer; ++k) {
            const int j = threadIdx.x + k * kThreads;
            wv[k] = ws.uniq_start[u0 + j <= U ? u0 + j : U];
        }
#pragma unroll
        for (int k = 0; k < kWinPer; ++k) {
            const int j = threadIdx.x + k * kThreads;
            if (j <= kSmChunk) win[j] = u0 + j <= U ? wv[k] : 0x7fffffff;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSmPer; ++i) {
            const int64_t pos = p0 + threadIdx.x + i * kThreads;
            if (pos >= n) break;
            // the chunk holds at most kSmChunk - 1 run starts after u0's, so
            // the last start at or before pos is one of win[0 .. kSmChunk - 1]
            int jl = 0, jh = kSmChunk;
            while (jh - jl > 1) {
                const int mid = (jl + jh) >> 1;
                if (win[mid] <= pos) jl = mid;
                else jh = mid;
            }
            ws.sm[pos] = make_int2(bg[i], u0 + jl);
        }
    }
}

// Gradient gather g_u = sum of grad_out rows over the lookups of unique row u.
// A worker is LPR = kGuCols / 4 lanes, a float4 each: one piece of kGuCols
// columns of a grad_out row (a whole row when D <= kGuCols).  It walks the
// positions of its task in sorted order, kGuBatch rows in flight, summing
// runs of equal u.  A run that lies inside the task goes straight to u's slot
// of the unique-row buffer (E's space); a run cut by the task's left or right
// edge leaves its sum in the task's left or right partial slot (this piece's
// columns), recorded in gu_ml / gu_mr, and k_gu_join adds the parts in task
// order.  The order of every sum is fixed by the task cut alone.  The blocks
// of virtual XCD x = blockIdx % 8 (launched in multiples of 8) take the x-th
// eighth of the ids in order, so one XCD's workers read the rows of about one
// table at a time.  Measured on the 26-table training step: the random row
// reads are bound by the line misses a compute unit keeps in flight, so whole
// lines per request matter and L2 residency hardly does (64-column pieces
// with these ids 0.70 ms; 32-column 0.72; 16-column pieces of a per-table
// copy of grad_out, 2 MB per XCD, 1.1 ms; ids without XCD affinity, same
// time as with).
template <bool VEC>
__device__ __forceinline__ float4 gu_row(const float *gr, int nv)
{
    if (VEC) return *reinterpret_cast<const float4 *>(gr);
    // unaligned or partial: clamped scalar loads (columns past nv are dropped by the caller)
    const int m = nv > 0 ? nv - 1 : 0;
    return make_float4(gr[0 < m ? 0 : m], gr[1 < m ? 1 : m], gr[2 < m ? 2 : m], gr[3 < m ? 3 : m]);
}

template <bool VEC, int LPR, int NS>
__device__ __forceinline__ void gu_walk(const BwdArgs &a, const Ws &ws, int k0, int k1, int u0, int u1, int uleft,
                                        int uright, const float *go, int nv, float *Ej, int Dp, float *slotLj,
                                        float *slotRj, int grp, int gl, int &mL, int &mR)
{
    auto clampu = [&](int u) { return u < u0 ? u0 : (u >= u1 ? u1 - 1 : u); };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int ucur = clampu(ws.sm[k0].y);
    bool first = true;
    auto store = [&](float *dst) {
        if (VEC || nv == 4) {
            *reinterpret_cast<float4 *>(dst) = acc;
        } else {
            if (nv > 0) dst[0] = acc.x;
            if (nv > 1) dst[1] = acc.y;
            if (nv > 2) dst[2] = acc.z;
        }
    };
    // metadata of a batch: position kb + e sits in lane e % LPR, slot e / LPR.
    // Loads are unconditional (positions past the task read its last one, and
    // their rows are never added), so all are in flight together; the next
    // batch's metadata is loaded while this batch's rows are summed
    int2 meta[NS];
    auto load_meta = [&](int kb) {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const int pos = kb + sl * LPR + gl;
            meta[sl] = ws.sm[pos < k1 ? pos : k1 - 1];
        }
    };
    load_meta(k0);
    for (int kb = k0; kb < k1; kb += kGuBatch) {
        int bg[NS], uu[NS];
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            bg[sl] = meta[sl].x < 0 ? 0 : (meta[sl].x >= a.B ? (int)a.B - 1 : meta[sl].x);
            uu[sl] = clampu(meta[sl].y);
        }
        float4 row[kGuBatch];
#pragma unroll
        for (int ii = 0; ii < kGuBatch; ++ii) {
            const int b = __shfl(bg[ii / LPR], grp * LPR + ii % LPR, 64);
            row[ii] = gu_row<VEC>(go + (int64_t)b * a.SD, nv);
        }
        load_meta(kb + kGuBatch < k1 ? kb + kGuBatch : kb);
#pragma unroll
        for (int ii = 0; ii < kGuBatch; ++ii) {
            const int u = __shfl(uu[ii / LPR], grp * LPR + ii % LPR, 64);
            if (kb + ii < k1) {
                if (u != ucur) {
                    // a run ends inside the task: its own row, or the left cut
                    const bool cutl = first && ucur == uleft;
                    if (cutl) mL = ucur;
                    store(cutl ? slotLj : Ej + (int64_t)ucur * Dp);
                    first = false;
                    ucur = u;
                    acc = make_float4(0.f, 0.f, 0.f, 0.f);
                }
                acc.x += row[ii].x;
                acc.y += row[ii].y;
                acc.z += row[ii].z;
                acc.w += row[ii].w;
            }
        }
    }
    const bool cutl = first && ucur == uleft, cutr = ucur == uright;
    if (cutl) mL = ucur;
    if (cutr) mR = ucur;
    store(cutl ? slotLj : (cutr ? slotRj : Ej + (int64_t)ucur * Dp));
}

__global__ __launch_bounds__(kThreads) void k_gu_gather(BwdArgs a)
{
    constexpr int LPR = kGuCols / 4, G = 64 / LPR, NS = kGuBatch / LPR; // NS metadata slots per lane
    static_assert(LPR * NS == kGuBatch && G * LPR == 64, "batch and workers tile the wave");
    __shared__ int base[kMaxTables + 1], qb[kMaxTables + 1];
    __shared__ GuTab gt[kMaxTables];
    gu_bases(a, base, qb, gt);
    const Ws &ws = a.ws;
    const int T = a.T, nid = qb[T];
    const int lane = threadIdx.x & 63, grp = lane / LPR, gl = lane - grp * LPR;
    const int x = blockIdx.x & 7, nbx = gridDim.x >> 3;
    const int id_hi = (int)((int64_t)nid * (x + 1) / 8);
    const int wk = ((blockIdx.x >> 3) * (kThreads / 64) + (threadIdx.x >> 6)) * G + grp;
    const int nwk = nbx * (kThreads / 64) * G;
    // rows move as float4 when every row of every table starts 16-byte aligned
    const bool rows16 = (a.SD & 3) == 0 && (reinterpret_cast<uintptr_t>(a.grad_out) & 15) == 0;
    for (int id = (int)((int64_t)nid * x / 8) + wk; id < id_hi; id += nwk) {
        const int t = gu_table(qb, T, id);
        const GuTab tb = gt[t];
        const int r = id - qb[t], pc = r / tb.ntask, k = r - pc * tb.ntask;
        const int task = base[t] + k;
        const int ts = tb.ts, te = tb.te;
        const int k0 = ts + k * kGuTask;
        const int k1 = k0 + kGuTask < te ? k0 + kGuTask : te;
        const int u0 = tb.u0, u1 = tb.u1;
        int mL = -1, mR = -1;
        if (u1 > u0) {
            auto clampu = [&](int u) { return u < u0 ? u0 : (u >= u1 ? u1 - 1 : u); };
            const int j = pc * kGuCols + 4 * gl; // first column of this lane
            int nv = tb.D - j;                   // columns of this lane's float4 inside the table
            nv = nv < 0 ? 0 : (nv > 4 ? 4 : nv);
            const float *go = a.grad_out + tb.col_off + (nv > 0 ? j : 0);
            float *Ej = ws.E + tb.ebase + j;
            float *slotLj = ws.P3 + (int64_t)(2 * task) * a.gstride + j, *slotRj = slotLj + a.gstride;
            // unique rows of the positions just outside the task (-1: table edge)
            const int uleft = k0 > ts ? clampu(ws.sm[k0 - 1].y) : -1;
            const int uright = k1 < te ? clampu(ws.sm[k1].y) : -1;
            const bool vec = rows16 && (tb.col_off & 3) == 0 && nv == 4;
            if (__all(vec)) // wave-uniform: every lane of the wave reads whole float4
                gu_walk<true, LPR, NS>(a, ws, k0, k1, u0, u1, uleft, uright, go, nv, Ej, tb.Dp, slotLj, slotRj,
                                       grp, gl, mL, mR);
            else
                gu_walk<false, LPR, NS>(a, ws, k0, k1, u0, u1, uleft, uright, go, nv, Ej, tb.Dp, slotLj, slotRj,
                                        grp, gl, mL, mR);
        }
        if (gl == 0 && pc == 0) { // every piece of a task sees the same runs
            ws.gu_ml[task] = mL;
            ws.gu_mr[task] = mR;
        }
    }
}

// Cut runs: the task where a cut run starts (its right edge cuts run u, which
// does not also enter from the left) adds its right partial and the left
// partials of the following tasks up to the one holding u's last position, in
// that order, into u's slot.  One wave per task, lanes over columns.
__global__ __launch_bounds__(kThreads) void k_gu_join(BwdArgs a)
{
    __shared__ int base[kMaxTables + 1], qb[kMaxTables + 1];
    __shared__ GuTab gt[kMaxTables];
    gu_bases(a, base, qb, gt);
    const Ws &ws = a.ws;
    const int T = a.T, ntask = base[T];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int task = blockIdx.x * (kThreads / 64) + w; task < ntask; task += gridDim.x * (kThreads / 64)) {
        const int u = ws.gu_mr[task];
        if (u < 0 || ws.gu_ml[task] == u) continue;
        const int t = gu_table(base, T, task);
        const GuTab tb = gt[t];
        const int e = ws.uniq_start[u + 1] - 1; // u's last sorted position
        int last = base[t] + (e - tb.ts) / kGuTask;
        last = last > base[t + 1] - 1 ? base[t + 1] - 1 : last;
        float *dst = ws.E + tb.ebase + (int64_t)u * tb.Dp;
        const float *part = ws.P3;
        const int64_t gs = a.gstride;
        for (int j = lane; j < tb.D; j += 64) {
            float s = part[(2 * (int64_t)task + 1) * gs + j];
#pragma unroll 8
            for (int k = task + 1; k <= last; ++k) s += part[2 * (int64_t)k * gs + j];
            dst[j] = s;
        }
    }
}

// One block per run of units sharing (table, i2), units in i1 order.
// LDS: the unit's prefix intermediate C and its gradient dC ([d1*d2][R2]).
constexpr int kBwdCMax = 4096;
constexpr int kBwdG2Regs = 64; // dG2 slice elements per thread (R1*d2*R2 <= 16384)

__global__ __launch_bounds__(kThreads) void k_bwd_runs(BwdArgs a)
{
    __shared__ float Cl[kBwdCMax];
    __shared__ float dCl[kBwdCMax];
    const Ws &ws = a.ws;
    const int64_t nruns = ws.ctrl[CTRL_RUNS];
    for (int64_t run = blockIdx.x; run < nruns; run += gridDim.x) {
        const int k0 = ws.run_start[run], k1 = ws.run_start[run + 1];
        const int t = segment_of(ws.tab_unit_start, a.T, ws.uorder[k0]);
        const TableDesc &tb = a.tab[t];
        if (!a.force_generic && tb.cls >= 0) continue; // matrix-core kernel owns this run
        const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, R1 = tb.R1, R2 = tb.R2, D = tb.D;
        const int D12 = d1 * d2, CN = D12 * R2, G2N = R1 * d2 * R2;
        const int i2 = ws.unit_prefix[ws.uorder[k0]] % tb.n2;
        const float *G1 = a.cores.g[t][0];
        const float *G2 = a.cores.g[t][1] + (int64_t)i2 * G2N;
        const float *G3 = a.cores.g[t][2];
        float acc2[kBwdG2Regs];
#pragma unroll
        for (int i = 0; i < kBwdG2Regs; ++i) acc2[i] = 0.f;
        for (int k = k0; k < k1; ++k) {
            const int unit = ws.uorder[k];
            const int i1 = ws.unit_prefix[unit] / tb.n2;
            const float *g1 = G1 + (int64_t)i1 * d1 * R1;
            const int us = ws.unit_start[unit], ue = ws.unit_start[unit + 1];
            // C[m2][r2] = sum_r1 G1[i1][j1][r1] G2[i2][r1][j2][r2]
            for (int e = threadIdx.x; e < CN; e += kThreads) {
                const int m2 = e / R2, r2 = e - m2 * R2, j1 = m2 / d2, j2 = m2 - j1 * d2;
                float c = 0.f;
                for (int r1 = 0; r1 < R1; ++r1) c = fmaf(g1[j1 * R1 + r1], G2[((int64_t)r1 * d2 + j2) * R2 + r2], c);
                Cl[e] = c;
            }
            // dC[m2][r2] = sum_u sum_j3 g_u[m2*d3+j3] G3[i3_u][r2][j3]
            for (int e = threadIdx.x; e < CN; e += kThreads) {
                const int m2 = e / R2, r2 = e - m2 * R2;
                float c = 0.f;
                for (int u = us; u < ue; ++u) {
                    const float *gu = ws.E + ws.ebase[t] + (int64_t)u * tb.Dp + m2 * d3;
                    const float *g3 = G3 + ((int64_t)(ws.uniq_row[u] % tb.n3) * R2 + r2) * d3;
                    for (int j3 = 0; j3 < d3; ++j3) c = fmaf(gu[j3], g3[j3], c);
                }
                dCl[e] = c;
            }
            __syncthreads();
            // G3 partial of every row: P3_u[r2][j3] = sum_m2 C[m2][r2] g_u[m2*d3+j3]
            {
                const int per = R2 * d3;
                for (int64_t e = threadIdx.x; e < (int64_t)(ue - us) * per; e += kThreads) {
                    const int r = (int)(e / per), rem = (int)(e - (int64_t)r * per);
                    const int r2 = rem / d3, j3 = rem - r2 * d3;
                    const int u = us + r;
                    const float *gu = ws.E + ws.ebase[t] + (int64_t)u * tb.Dp + j3;
                    float c = 0.f;
                    for (int m2 = 0; m2 < D12; ++m2) c = fmaf(Cl[m2 * R2 + r2], gu[m2 * d3], c);
                    ws.P3[ws.p3base[t] + (int64_t)u * per + rem] = c;
                }
            }
            // G1 partial of the unit: sum_{j2,r2} dC[j1*d2+j2][r2] G2[i2][r1][j2][r2]
            for (int e = threadIdx.x; e < d1 * R1; e += kThreads) {
                const int j1 = e / R1, r1 = e - j1 * R1;
                float c = 0.f;
                for (int j2 = 0; j2 < d2; ++j2)
                    for (int r2 = 0; r2 < R2; ++r2)
                        c = fmaf(dCl[(j1 * d2 + j2) * R2 + r2], G2[((int64_t)r1 * d2 + j2) * R2 + r2], c);
                ws.G1P[(int64_t)k * a.g1stride + e] = c;
            }
            // dG2 slice: sum_j1 G1[i1][j1][r1] dC[j1*d2+j2][r2]
#pragma unroll
            for (int i = 0; i < kBwdG2Regs; ++i) {
                const int e = threadIdx.x + i * kThreads;
                if (e < G2N) {
                    const int r1 = e / (d2 * R2), rem = e - r1 * d2 * R2;
                    const int j2 = rem / R2, r2 = rem - j2 * R2;
                    float c = acc2[i];
                    for (int j1 = 0; j1 < d1; ++j1) c = fmaf(g1[j1 * R1 + r1], dCl[(j1 * d2 + j2) * R2 + r2], c);
                    acc2[i] = c;
                }
            }
            __syncthreads();
        }
        float *dG2 = a.grads.g[t][1] + (int64_t)i2 * G2N;
#pragma unroll
        for (int i = 0; i < kBwdG2Regs; ++i) {
            const int e = threadIdx.x + i * kThreads;
            if (e < G2N) dG2[e] = acc2[i];
        }
    }
}

// dG1[t][i1] = sum of the unit partials of table t whose prefix has digit i1
// (a contiguous range of the prefix-sorted units); zero when none.
// Table of a reduction slot: the last table whose slot base (i1_base, or
// i3_base when I3) is at most slot.  The bases ascend from 0 and T <= 64, so
// each lane tests one table and the answer is the count of passing lanes: one
// load round trip instead of a dependent walk over the tables.
template <bool I3>
__device__ __forceinline__ int slot_table(const TableDesc *tab, int T, int slot)
{
    const int lane = threadIdx.x & 63;
    const TableDesc &d = tab[lane < T ? lane : 0];
    const uint32_t base = I3 ? d.i3_base : d.i1_base;
    return __popcll(__ballot(lane < T && base <= (uint32_t)slot)) - 1;
}

// First position in [lo, hi) of the ascending array v holding a value >= key
// (hi if none), found by the whole wave: 64 probes per round, so a range of
// 64^r positions takes r load round trips instead of log2 of its size.
__device__ __forceinline__ int wave_lower_bound(const int32_t *v, int lo, int hi, int key)
{
    const int lane = threadIdx.x & 63;
    if (hi <= lo) return lo; // empty range: no load at all
    while (hi - lo > 64) {
        const int step = (hi - lo + 63) / 64;
        const int idx = lo + lane * step;
        const bool ge = idx >= hi || v[idx < hi ? idx : lo] >= key;
        const uint64_t m = __ballot(ge);
        const int f = m ? __ffsll((unsigned long long)m) - 1 : 64; // lane 63 probes below hi, so f < 64 unless none
        if (f == 0) return lo;
        const int nhi = lo + f * step < hi ? lo + f * step : hi;
        lo = lo + (f - 1) * step + 1;
        hi = nhi;
    }
    const int idx = lo + lane;
    const bool ge = idx >= hi || v[idx < hi ? idx : lo] >= key;
    const uint64_t m = __ballot(ge);
    return m ? lo + __ffsll((unsigned long long)m) - 1 : hi;
}

__global__ __launch_bounds__(kThreads) void k_reduce_g1(BwdArgs a, int total_slots)
{
    const Ws &ws = a.ws;
    for (int slot = blockIdx.x; slot < total_slots; slot += gridDim.x) {
        const int t = slot_table<false>(a.tab, a.T, slot);
        const TableDesc &tb = a.tab[t];
        const int i1 = slot - (int)tb.i1_base;
        if (i1 >= tb.n1) continue;
        const int lo0 = ws.tab_unit_start[t], hi0 = ws.tab_unit_start[t + 1];
        const int qlo = i1 * tb.n2, qhi = qlo + tb.n2;
        // the table's units with prefix in [qlo, qhi) (prefixes ascend within a table)
        const int first = wave_lower_bound(ws.unit_prefix, lo0, hi0, qlo);
        const int last = wave_lower_bound(ws.unit_prefix, first, hi0, qhi);
        const int per = tb.d1 * tb.R1;
        float *dst = a.grads.g[t][0] + (int64_t)i1 * per;
        // partial rows of the slot's units (in unit order) staged kThreads at a
        // time in LDS, then summed in that order with 8 loads in flight
        __shared__ int rows[kThreads];
        for (int e0 = 0; e0 < per; e0 += 4 * kThreads) {
            float c[4] = {0.f, 0.f, 0.f, 0.f}; // elements e0 + threadIdx.x + k*kThreads
            for (int u0 = first; u0 < last; u0 += kThreads) {
                const int n = last - u0 < kThreads ? last - u0 : kThreads;
                __syncthreads();
                if ((int)threadIdx.x < n) rows[threadIdx.x] = ws.uinv[u0 + threadIdx.x];
                __syncthreads();
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e = e0 + threadIdx.x + k * kThreads;
                    if (e >= per) break;
                    float s = c[k];
#pragma unroll 8
                    for (int i = 0; i < n; ++i) s += ws.G1P[(int64_t)rows[i] * a.g1stride + e];
                    c[k] = s;
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = e0 + threadIdx.x + k * kThreads;
                if (e < per) dst[e] = c[k];
            }
        }
        __syncthreads();
    }
}

// Sort keys of unique rows by (table, i3).
__global__ __launch_bounds__(kThreads) void k_key3(BwdArgs a, uint32_t *k, int32_t *v)
{
    const Ws &ws = a.ws;
    const int64_t U = ws.ctrl[CTRL_U];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < U; u += stride) {
        const int t = segment_of(ws.tab_uniq_start, a.T, u);
        k[u] = a.tab[t].i3_base + (uint32_t)(ws.uniq_row[u] % a.tab[t].n3);
        v[u] = (int32_t)u;
    }
}

// Row range of every G3 slice in the (table, i3)-sorted unique rows: run
// edges of the sorted keys (slots without rows keep the empty range 0..0).
__global__ __launch_bounds__(kThreads) void k_g3_bounds(BwdArgs a, const uint32_t *k3, int total_slots)
{
    const Ws &ws = a.ws;
    const int64_t U = ws.ctrl[CTRL_U];
    int32_t *first = ws.g3rng, *last = ws.g3rng + total_slots;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < U; q += stride) {
        const uint32_t key = k3[q];
        if (key >= (uint32_t)total_slots) continue;
        if (q == 0 || k3[q - 1] != key) first[key] = (int32_t)q;
        if (q == U - 1 || k3[q + 1] != key) last[key] = (int32_t)(q + 1);
    }
}

// dG3[t][i3] = sum over unique rows of table t with that i3, in unique-id
// order, of their partials; zero when none.  Each (phase, element) thread
// keeps kG3Acc interleaved partial sums over its rows, added in order, and
// the phases are added in order: a fixed order with several loads in flight.
// The slot's row ids are staged in LDS (one coalesced load), so a row's
// partial is one global load; a stage holds a whole number of groups of
// kG3Acc * rp rows, so no group straddles two stages and the order of the
// sums does not depend on the staging.
constexpr int kG3Acc = 8;
constexpr int kG3Stage = kG3Acc * kThreads; // at least one group for any phase count

__global__ __launch_bounds__(kThreads) void k_reduce_g3(BwdArgs a, const int32_t *order, int total_slots)
{
    const Ws &ws = a.ws;
    __shared__ float part[kThreads];
    __shared__ int32_t ord[kG3Stage];
    for (int slot = blockIdx.x; slot < total_slots; slot += gridDim.x) {
        const int t = slot_table<true>(a.tab, a.T, slot);
        const TableDesc &tb = a.tab[t];
        const int i3 = slot - (int)tb.i3_base;
        if (i3 >= tb.n3) continue;
        const int64_t first = ws.g3rng[slot], last = ws.g3rng[total_slots + slot];
        const int per = tb.R2 * tb.d3;
        float *dst = a.grads.g[t][2] + (int64_t)i3 * per;
        const float *src = ws.P3 + ws.p3base[t];
        const int rp = per >= kThreads ? 1 : kThreads / per;
        const int ph = threadIdx.x / per < rp ? threadIdx.x / per : rp; // rp = idle
        const int64_t stg = (int64_t)(kG3Stage / (kG3Acc * rp)) * (kG3Acc * rp); // rows per stage
        for (int e0 = 0; e0 < per; e0 += kThreads) {
            const int e = e0 + (rp == 1 ? threadIdx.x : threadIdx.x - ph * per);
            const bool act = ph < rp && e < per;
            float acc[kG3Acc];
#pragma unroll
            for (int k = 0; k < kG3Acc; ++k) acc[k] = 0.f;
            int64_t q = first + ph;
            for (int64_t b0 = first; b0 < last; b0 += stg) {
                const int64_t b1 = b0 + stg < last ? b0 + stg : last;
                __syncthreads(); // previous stage read
                for (int i = threadIdx.x; i < b1 - b0; i += kThreads) ord[i] = order[b0 + i];
                __syncthreads();
                if (act) {
                    for (; q + (kG3Acc - 1) * rp < b1; q += kG3Acc * rp) {
#pragma unroll
                        for (int k = 0; k < kG3Acc; ++k) acc[k] += src[(int64_t)ord[q - b0 + k * rp] * per + e];
                    }
                    if (b1 == last) {
#pragma unroll
                        for (int k = 0; k < kG3Acc; ++k)
                            if (q + k * rp < last) acc[k] += src[(int64_t)ord[q - b0 + k * rp] * per + e];
                    }
                }
            }
            float c = 0.f;
#pragma unroll
            for (int k = 0; k < kG3Acc; ++k) c += acc[k];
            if (rp == 1) {
                if (e < per) dst[e] = c;
            } else {
                __syncthreads();
                part[threadIdx.x] = c;
                __syncthreads();
                if (threadIdx.x < per) {
                    float sum = 0.f;
                    for (int k = 0; k < rp; ++k) sum += part[k * per + threadIdx.x];
                    dst[threadIdx.x] = sum;
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------ matrix-core reverse contraction
//
// One block per (table, i2) run of a rank class R (R1 = R2 = R, d1, d2 <= 4,
// d3 <= 16), one kernel per class, runs taken from a per-class counter.  The
// run is walked through the forward's chunk records (tiles of <= 4 units,
// chunks of <= 32 rows with their i3 digits), so no dependent index chasing
// happens in the loop.  The G2[i2] slice is staged in LDS once per run with an
// XOR swizzle (column ^ (row & 31)) so it can be read along columns (C and dG2)
// and along rows (dG1 partials) without bank conflicts.  Per chunk the G1
// slices of the tile, the output-gradient rows g_u and the transposed G3
// slices of the rows are staged in LDS with one burst of independent loads.
// Per tile of <= 4 units (g) and column col = j2*R + r2:
//   (1) C[(g,j1)][col]  = sum_r1 G1[i1_g][j1][r1] G2[r1][col]          -> LDS
//   (2) per row u:  dC_g += g_u . G3[i3_u]^T ;  P3_u = C_g^T . g_u     (P3 -> partial buffer)
//   (3) G1P_g[j1][r1]   = sum_col dC[(g,j1)][col] G2[r1][col]           -> partial buffer
//   (4) dG2[r1][col]   += sum_(g,j1) G1[i1_g][j1][r1] dC[(g,j1)][col]  (registers for the run)
// All products are v_mfma_f32_16x16x4_f32 tiles.

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS layout (floats) of the class kernel for rank R.
template <int R>
struct BwdLds {
    static constexpr int CLS = R == 8 ? 0 : R == 16 ? 1 : R == 32 ? 2 : 3;
    static constexpr int NCOL = 4 * R;                 // columns (j2, r2), d2 padded to 4
    static constexpr int CSTR = R + 4;                 // row stride of C / dC
    static constexpr int CUNIT = 16 * CSTR + 16;       // floats per unit
    static constexpr int G2ST = NCOL + 1;              // odd row stride of the G2 slice
    static constexpr int G2S = R * G2ST;
    static constexpr int CS = 4 * CUNIT;
    static constexpr int G1ST = R + 1;                 // odd row stride: (1) reads rows across lanes
    static constexpr int G1S = 16 * G1ST;              // [unit][j1][r1]
    static constexpr int DTST = 17;                    // transposed dC: [col][(g, j1)], stride 17
    static constexpr int STAGE = CLS == 3 ? 14336 : CLS == 2 ? 10240 : 6144;
    static constexpr int TOTAL = G2S + 2 * CS + G1S + STAGE;
    static constexpr int OCC = CLS == 3 ? 1 : CLS == 1 ? 3 : 2; // blocks per CU
    static constexpr int NW = CLS == 3 ? 8 : 4;                  // waves per block
    // float4 registers per thread that carry the next chunk's first rows while
    // this chunk computes (the rows of a 64-column table at chunk_rows 32)
    static constexpr int PF = CLS == 3 ? 2 : CLS == 2 ? 6 : CLS == 1 ? 4 : 2;
};

// REUSE: the prefix tiles C come from the forward (Ws::Cg) instead of step (1).
template <int R, bool REUSE>
__global__ __launch_bounds__(BwdLds<R>::NW * 64, BwdLds<R>::OCC) void k_bwd_class(BwdArgs a)
{
    using L = BwdLds<R>;
    constexpr int NW = L::NW, BT = NW * 64;
    constexpr int NCOL = L::NCOL, NT = NCOL / 16, NTW = (NT + NW - 1) / NW, MT = (R + 15) / 16, KQ = R / 4;
    // (2) rows: at ranks <= 32 wave (mb, rg) takes every RG-th row of every
    // unit for r2 block mb and the wave partials of dC are added at tile end
    // (balanced whatever the unit sizes); at rank 64, where units hold few
    // rows, wave w owns the (unit, r2 block) items w + NW*i whole
    constexpr bool kBal = R <= 32;
    constexpr int RG = NW / MT;                    // row groups (waves per r2 block)
    constexpr int NIT = (4 * MT + NW - 1) / NW;    // items per wave (rank 64)
    constexpr int NACC = kBal ? 4 : NIT;           // dC accumulators per wave
    static_assert(RG * MT == NW && (!kBal || RG * 4 * MT * 256 <= L::STAGE), "(2) wave partials fit in the staging region");
    // (3): waves form NP groups of MTW r1 blocks times KG groups of SPW columns
    constexpr int MTW = MT >= 2 ? 2 : 1, NP = MT / MTW, KG = NW / NP, SPW = R / KG;
    constexpr int CSTR = L::CSTR, CUNIT = L::CUNIT, PF = L::PF;
    // guards that hold for every lane are folded at compile time, and LDS
    // operand loads are unconditional (clamped addresses, then a select):
    // a branch around each load would keep the scheduler from hoisting loads
    // ahead of the MFMAs that consume them
    constexpr bool kAllNT = NT % NW == 0, kAllR = R % 16 == 0;
    static_assert(NP * KG == NW && SPW * KG == R && (R & (R - 1)) == 0, "(3) splits the columns evenly");
    static_assert(KG * MT * 256 <= L::STAGE, "(3) partials fit in the staging region");
    static_assert(4 * R <= BT, "one G1 float4 per thread");
    __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
    __shared__ ChunkRec recs[3]; // records of chunks c, c+1 and (arriving) c+2
    __shared__ int s_run;
    __shared__ long long s_t0;
    if (threadIdx.x == 0) s_t0 = wall_clock64();
    int nwork = 0, nchunks = 0; // scheduling record (thread 0)
    // Cs holds C during a tile and dC at its end (C is dead by then); dT holds
    // dC transposed ([col][(g, j1)]) for the dG1 partials
    float *G2s = lds, *Cs = lds + L::G2S, *dT = Cs + L::CS, *G1s = dT + L::CS, *Sg = G1s + L::G1S;
    static_assert(L::NCOL * L::DTST <= L::CS, "transposed dC fits in its region");
    constexpr int G1ST = L::G1ST, DTST = L::DTST, G2ST = L::G2ST;
    const Ws &ws = a.ws;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, kq = lane >> 4;
    const int mb = w % MT, rg = w / MT; // (2): this wave's r2 block and row group
    const int rbeg = ws.ctrl[CTRL_PIECE_CLS + L::CLS], rend = ws.ctrl[CTRL_PIECE_CLS + L::CLS + 1];
    for (;;) {
        if (tid == 0) {
            // pieces (whole runs, or tile-aligned parts of long ones) are
            // claimed longest first: the class's slice of the sorted order
            const int k = rbeg + atomicAdd(&ws.ctrl[CTRL_BWD_NEXT + L::CLS], 1);
            s_run = k < rend ? ws.rorder[k] : -1;
        }
        __syncthreads();
        const int piece = s_run;
        if (piece < 0) break;
        const int c0 = ws.tile_cstart[ws.piece_tb[piece]], c1 = ws.tile_cstart[ws.piece_te[piece]];
        const int slot = __builtin_amdgcn_readfirstlane(ws.piece_slot[piece]);
        if (tid == 0) {
            ++nwork;
            nchunks += c1 - c0;
        }
        if (w == 0) {
            reinterpret_cast<int *>(&recs[0])[lane] = reinterpret_cast<const int *>(&ws.crec[c0])[lane];
            if (c0 + 1 < c1)
                reinterpret_cast<int *>(&recs[1])[lane] = reinterpret_cast<const int *>(&ws.crec[c0 + 1])[lane];
        }
        __syncthreads();
        // wave-uniform: the table data below become scalar loads
        const int t = __builtin_amdgcn_readfirstlane(recs[0].t), i2 = __builtin_amdgcn_readfirstlane(recs[0].i2);
        const auto &tb = kconst(a.tab)[t];
        const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, D12 = d1 * d2, Dp = tb.Dp, P = small_div(16, d3);
        const float *G1 = a.cores.g[t][0];
        const float *G3t = ws.g3t + tb.g3t_off;
        // per-table bases read once per run: a global load issued after this
        // run's stores would wait for all of them (stores and loads share one counter)
        const float *Et = ws.E + kconst(ws.ebase)[t];
        float *P3t = ws.P3 + kconst(ws.p3base)[t];
        // staged rows: g_u at stride Dp + 4, G3 slices as [j3][R + 16] (bank-spread)
        const int GST = Dp + 4, G3J = R + 16, G3ST = d3 * G3J;
        int rb = L::STAGE / (GST + G3ST);
        rb = rb < kMaxChunkRows ? rb : kMaxChunkRows;
        float *Gs = Sg, *G3s = Sg + rb * GST;
        {   // stage G2[i2] as G2s[r][col] (row stride NCOL + 1), zero-padded to NCOL
            // columns: float4 loads (source rows of d2*R floats, 16-byte aligned),
            // all of a thread's in flight at once -- unconditional, from a clamped
            // address for the padding columns, which are written as zeros (a load
            // under a condition is waited for before the next one is issued)
            const float *src = a.cores.g[t][1] + (int64_t)i2 * R * d2 * R;
            constexpr int N4 = R * NCOL / 4, PER = (N4 + BT - 1) / BT; // float4 per slice, per thread
            constexpr int CH = PER < 4 ? PER : 4;                       // in flight together
            static_assert(PER % CH == 0, "whole batches");
            const int rowlen = d2 * R;
#pragma unroll
            for (int k0 = 0; k0 < PER; k0 += CH) {
                float4 gv[CH];
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    const int f = tid + (k0 + k) * BT, r = f / R, c4 = f - r * R; // NCOL / 4 == R float4 per row
                    const bool ok = f < N4 && 4 * c4 < rowlen;
                    gv[k] = *reinterpret_cast<const float4 *>(src + (ok ? r * rowlen + 4 * c4 : 0));
                }
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    const int f = tid + (k0 + k) * BT, r = f / R, c4 = f - r * R;
                    if (f < N4) {
                        const bool ok = 4 * c4 < rowlen;
                        float *d = G2s + r * G2ST + 4 * c4;
                        d[0] = ok ? gv[k].x : 0.f;
                        d[1] = ok ? gv[k].y : 0.f;
                        d[2] = ok ? gv[k].z : 0.f;
                        d[3] = ok ? gv[k].w : 0.f;
                    }
                }
            }
        }
        // this wave's part of the units' dC; at rank 64 (few rows per wave
        // and unit) a second chain takes every other row
        constexpr int NACC2 = kBal ? 1 : NACC;
        floatx4 g2acc[MT][NTW], dacc[NACC], dacc2[NACC2];
#pragma unroll
        for (int i = 0; i < NACC; ++i) dacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NACC2; ++i) dacc2[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) g2acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        const int c4g = Dp >> 2, c4t = (d3 * R) >> 2, c4r = c4g + c4t; // float4 per staged row
        const int pf_cap = PF * BT / c4r;                                // rows the prefetch carries
        // e / c4r as a multiply-high (exact for e, c4r < 2^16: e < 32 rows x c4r here)
        const uint32_t c4m = (uint32_t)((0x100000000ull + (uint64_t)c4r - 1) / (uint64_t)c4r);
        auto row_of = [&](int e) __attribute__((always_inline)) { return (int)__umulhi((uint32_t)e, c4m); };
        auto first_rows = [&](const ChunkRec &r) __attribute__((always_inline)) {
            const int n = r.rowoff[4] < rb ? r.rowoff[4] : rb;
            return n < pf_cap ? n : pf_cap;
        };
        // Stage rows q0 .. q0+n-1 of chunk r into the batch that starts at row sb.
        auto stage_rows = [&](const ChunkRec &r, int sb, int q0, int n) __attribute__((always_inline)) {
            for (int e = tid; e < n * c4r; e += BT) {
                const int qq = row_of(e), rem = e - qq * c4r, q = q0 + qq;
                const int j = (q >= r.rowoff[1]) + (q >= r.rowoff[2]) + (q >= r.rowoff[3]); // unit of row q
                if (rem < c4g) {
                    const int u = r.ustart[j] + (q - r.rowoff[j]);
                    *reinterpret_cast<float4 *>(Gs + (q - sb) * GST + 4 * rem) =
                        reinterpret_cast<const float4 *>(Et + (int64_t)u * Dp)[rem];
                } else {
                    const int r4 = rem - c4g, j3 = (4 * r4) / R, rr = 4 * r4 - j3 * R;
                    *reinterpret_cast<float4 *>(G3s + (q - sb) * G3ST + j3 * G3J + rr) =
                        reinterpret_cast<const float4 *>(G3t + (int64_t)r.i3[q] * d3 * R)[r4];
                }
            }
        };
        // The next chunk's first rows (and its tile's G1 slices, G1s[(g*4 + j1)*G1ST
        // + r1], zeros outside) travel in registers while this chunk computes.
        // Loads are unconditional (clamped to the chunk's first row when out of
        // range) and validity is applied when committing: zeroing a register that
        // a load may still target makes the compiler wait for every outstanding
        // load and store of the wave.
        floatx4 pfv[PF], pg1; // native vectors (a struct copy here would live in scratch)
        // with REUSE, the next tile's kept C (4 units x 16 rows x R floats,
        // compact in Cg by work position) travels with them
        constexpr int CPB = REUSE ? (16 * R + BT - 1) / BT : 1;
        floatx4 pc[CPB];
        const float *Cgt = ws.Cg + kconst(ws.cbase)[t];
        auto pf_issue = [&](const ChunkRec &r, bool tile_start) __attribute__((always_inline)) {
            const int n = first_rows(r);
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                int e = tid + i * BT;
                e = e < n * c4r ? e : 0;
                const int q = row_of(e), rem = e - q * c4r;
                const int j = (q >= r.rowoff[1]) + (q >= r.rowoff[2]) + (q >= r.rowoff[3]); // unit of row q
                const floatx4 *src = rem < c4g
                    ? reinterpret_cast<const floatx4 *>(Et + (int64_t)(r.ustart[j] + (q - r.rowoff[j])) * Dp) + rem
                    : reinterpret_cast<const floatx4 *>(G3t + (int64_t)r.i3[q] * d3 * R) + (rem - c4g);
                pfv[i] = *src;
            }
            if (tile_start) {
                const int e = tid < 4 * R ? tid : 0;
                const int gj = e / (R / 4), r4 = e - gj * (R / 4), g = gj >> 2, j1 = gj & 3;
                const bool ok = g < r.nu && j1 < d1;
                pg1 = reinterpret_cast<const floatx4 *>(G1 + ((int64_t)(ok ? r.i1[g] : r.i1[0]) * d1 + (ok ? j1 : 0)) * R)[r4];
                if constexpr (REUSE) {
                    const floatx4 *src = reinterpret_cast<const floatx4 *>(Cgt + (int64_t)r.ubeg * 16 * R);
#pragma unroll
                    for (int i = 0; i < CPB; ++i) {
                        // float4 e of the tile = (unit * 16 + row) * R/4 + col4; units
                        // past the tile's read unit 0 (their C rows are never used)
                        const int e = tid + i * BT;
                        const bool in = e < 16 * R && e / (4 * R) < r.nu;
                        pc[i] = src[in ? e : 0];
                    }
                }
            }
        };
        auto pf_commit = [&](const ChunkRec &r, bool tile_start) __attribute__((always_inline)) {
            const int n = first_rows(r);
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int e = tid + i * BT;
                if (e < n * c4r) {
                    const int q = row_of(e), rem = e - q * c4r;
                    if (rem < c4g) {
                        *reinterpret_cast<floatx4 *>(Gs + q * GST + 4 * rem) = pfv[i];
                    } else {
                        const int r4 = rem - c4g, j3 = (4 * r4) / R, rr = 4 * r4 - j3 * R;
                        *reinterpret_cast<floatx4 *>(G3s + q * G3ST + j3 * G3J + rr) = pfv[i];
                    }
                }
            }
            if constexpr (REUSE) {
                if (tile_start) {
#pragma unroll
                    for (int i = 0; i < CPB; ++i) {
                        const int e = tid + i * BT;
                        if (e < 16 * R) {
                            const int j = e / (4 * R), f = e - j * (4 * R), m = f / (R / 4), c4q = f - m * (R / 4);
                            *reinterpret_cast<floatx4 *>(Cs + j * CUNIT + m * CSTR + 4 * c4q) = pc[i];
                        }
                    }
                }
            }
            if (tile_start && tid < 4 * R) {
                const int gj = tid / (R / 4), r4 = tid - gj * (R / 4), g = gj >> 2, j1 = gj & 3;
                const bool ok = g < r.nu && j1 < d1;
                float *d = G1s + gj * G1ST + 4 * r4;
                d[0] = ok ? pg1[0] : 0.f;
                d[1] = ok ? pg1[1] : 0.f;
                d[2] = ok ? pg1[2] : 0.f;
                d[3] = ok ? pg1[3] : 0.f;
            }
        };
        pf_issue(recs[0], true);
        pf_commit(recs[0], true);
        int cur_tile = -1;
        for (int c = c0; c < c1; ++c) {
            const int slot = (c - c0) % 3;
            __syncthreads(); // staged rows, G1 slices and the record of chunk c+1 are visible
            const ChunkRec &rec = recs[slot];
            const ChunkRec &nrec = recs[slot == 2 ? 0 : slot + 1];
            const bool has_next = c + 1 < c1;
            const bool next_new = has_next && nrec.tile != rec.tile;
            const bool tile_end = !has_next || next_new;
            // record c+2 and the rows of chunk c+1 travel while this chunk runs
            const int pre = reinterpret_cast<const int *>(&ws.crec[c + 2 < c1 ? c + 2 : c])[lane];
            if (has_next) pf_issue(nrec, next_new);
            const int nu = rec.nu;
            const bool new_tile = rec.tile != cur_tile;
            const int nrows = rec.rowoff[4];
            {   // rows of the first batch the prefetch could not carry
                const int n0 = nrows < rb ? nrows : rb, npf = first_rows(rec);
                if (npf < n0) {
                    stage_rows(rec, 0, npf, n0 - npf);
                    __syncthreads();
                }
            }
            if (new_tile) {
                // ---- (1) prefix tile C (with REUSE it is already in Cs, committed
                // with the tile's first rows)
                if constexpr (!REUSE) {
                    // two independent chains per output tile (even and odd k steps)
                    const int g = li >> 2, j1 = li & 3;
                    floatx4 acc[NTW], acc2[NTW];
#pragma unroll
                    for (int j = 0; j < NTW; ++j) acc[j] = acc2[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KQ; s += 2) {
                        const int r = kq * KQ + s;
                        const float av = G1s[(g * 4 + j1) * G1ST + r];
                        const float av2 = G1s[(g * 4 + j1) * G1ST + r + 1];
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            const int ntg = w + NW * j;
                            if (kAllNT || ntg < NT) {
                                const int col = ntg * 16 + li;
                                acc[j] = mfma4(av, G2s[r * G2ST + col], acc[j]);
                                acc2[j] = mfma4(av2, G2s[(r + 1) * G2ST + col], acc2[j]);
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[j][v] += acc2[j][v];
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int ntg = w + NW * j;
                        if (kAllNT || ntg < NT) {
                            const int col = ntg * 16 + li, j2 = col / R, r2 = col % R;
                            if (j2 < d2) {
#pragma unroll
                                for (int v = 0; v < 4; ++v)
                                    if (v < d1) Cs[kq * CUNIT + (v * d2 + j2) * CSTR + r2] = acc[j][v];
                            }
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < NACC; ++i) dacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < NACC2; ++i) dacc2[i] = floatx4{0.f, 0.f, 0.f, 0.f};
                cur_tile = rec.tile;
                // with REUSE the tile's C was committed before the loop-top barrier
                if constexpr (!REUSE) __syncthreads(); // C tile written
            }
            // ---- (2) rows of this chunk, in staged batches of rb rows (the first is
            // staged).  Wave (mb, rg) covers r2 block mb for every RG-th row of each
            // unit, so the waves share the rows evenly whatever the unit sizes.
            for (int sb = 0; sb < nrows; sb += rb) {
                const int n = nrows - sb < rb ? nrows - sb : rb;
                if (sb > 0) {
                    __syncthreads(); // previous batch consumed
                    stage_rows(rec, sb, sb, n);
                    __syncthreads();
                }
#pragma unroll
                for (int i = 0; i < (kBal ? 4 : NIT); ++i) {
                    // (unit g, r2 block bm) of accumulator i, and the rows it takes
                    const int item = kBal ? 0 : w + NW * i;
                    const int g = kBal ? i : item / MT, bm = kBal ? mb : item % MT;
                    const int rs = kBal ? RG : 1;
                    if (item >= 4 * MT || g >= nu) continue;
                    const int r2 = bm * 16 + li;
                    const bool okr = r2 < R;
                    const int qa = sb > rec.rowoff[g] ? sb : rec.rowoff[g];
                    const int qe = rec.rowoff[g] + rec.ccnt[g];
                    const int qb = sb + n < qe ? sb + n : qe;
                    // row-group wave rg takes the chunk's rows q = rg (mod RG) and its
                    // output tiles t = rg (mod RG), counted over the whole chunk, so
                    // the waves share the rows evenly across units (counting within
                    // each unit gave the first wave a unit's odd row every time)
                    const int r0 = kBal ? ((rg - qa) % RG + RG) % RG : 0;
                    const int r0p = kBal ? ((rg - rec.pstart[g]) % RG + RG) % RG : 0;
                    // (2a) dC_g[m2][r2] += sum_j3 g_u[m2][j3] G3[i3_u][r2][j3]; with
                    // d3 = 4 (one k step per row) two rows per step into two chains
                    auto row_ops = [&](int q, int j0, float &av, float &bv) {
                        const float *gq = Gs + (q - sb) * GST;
                        const float *g3 = G3s + (q - sb) * G3ST + (okr ? r2 : 0);
                        const int j3 = j0 + kq;
                        const bool okj = j3 < d3;
                        const float ga = gq[(li < D12 ? li : 0) * d3 + (okj ? j3 : 0)];
                        const float gb = g3[(okj ? j3 : 0) * G3J];
                        av = (li < D12 && okj) ? ga : 0.f;
                        bv = (okr && okj) ? gb : 0.f;
                    };
                    int q = qa + r0;
                    if constexpr (!kBal) {
                        if (d3 == 4) {
                            for (; q + rs < qb; q += 2 * rs) {
                                float a0, b0, a1, b1;
                                row_ops(q, 0, a0, b0);
                                row_ops(q + rs, 0, a1, b1);
                                dacc[i] = mfma4(a0, b0, dacc[i]);
                                dacc2[i < NACC2 ? i : 0] = mfma4(a1, b1, dacc2[i < NACC2 ? i : 0]);
                            }
                        }
                    }
                    for (; q < qb; q += rs) {
                        for (int j0 = 0; j0 < d3; j0 += 4) {
                            float a0, b0;
                            row_ops(q, j0, a0, b0);
                            dacc[i] = mfma4(a0, b0, dacc[i]);
                        }
                    }
                    // (2b) P3_u[r2][j3] = sum_m2 C_g[m2][r2] g_u[m2][j3], P rows per output
                    // tile, the row groups dealt round-robin over the row-group waves.
                    // The output tile is (row, j3) x r2, so a lane holds 4 consecutive
                    // j3 of one row (d3 >= 4) and 16 lanes write 16 consecutive r2:
                    // whole 256-byte runs of P3_u
                    if (qa + r0p * P < qb) {
                        float ca[4];
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int m2 = kq * 4 + s;
                            const float cv = Cs[g * CUNIT + m2 * CSTR + (okr ? r2 : 0)];
                            ca[s] = (m2 < D12 && okr) ? cv : 0.f;
                        }
                        const int slot_r = small_div(li, d3), j3 = li - slot_r * d3; // A row of this lane
                        for (int qs = qa + r0p * P; qs < qb; qs += rs * P) {
                            const int cnt = qb - qs < P ? qb - qs : P;
                            const bool okb = slot_r < cnt;
                            floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const int m2 = kq * 4 + s;
                                const float gv = Gs[(qs + (okb ? slot_r : 0) - sb) * GST + (m2 < D12 ? m2 : 0) * d3 + j3];
                                acc = mfma4((okb && m2 < D12) ? gv : 0.f, ca[s], acc);
                            }
                            // lane (li, kq) holds output rows 4kq + v = (row, j3) of column r2
                            if (okr) {
                                const int64_t ub = rec.ustart[g] + (qs - rec.rowoff[g]);
                                if (d3 >= 4) {
                                    const int sr = small_div(4 * kq, d3), j0 = 4 * kq - sr * d3;
                                    if (sr < cnt)
                                        *reinterpret_cast<floatx4 *>(P3t + (ub + sr) * R * d3 + r2 * d3 + j0) = acc;
                                } else {
#pragma unroll 1
                                    for (int v = 0; v < 4; ++v) {
                                        const int sr = small_div(4 * kq + v, d3), jj = 4 * kq + v - sr * d3;
                                        if (sr < cnt) P3t[(ub + sr) * R * d3 + r2 * d3 + jj] = acc[v];
                                    }
                                }
                            }
                        }
                    }
                }
            }
            // rows done: C and the staged rows are free.  At rank 64 a tile's end
            // needs no barrier here: every wave reads C only in the blocks of its
            // own items, which its dC replaces, and the staged rows are next
            // written after the barrier that publishes dC
            if (kBal || !tile_end) __syncthreads();
            if (tile_end) {
                if constexpr (!kBal) {
#pragma unroll
                    for (int i = 0; i < NACC; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v) dacc[i][v] += dacc2[i < NACC2 ? i : 0][v];
                }
                if constexpr (kBal) {
                    // dC of each unit = the RG wave partials added in order; it goes
                    // to Cs (C is dead) and, transposed, to dT
                    float *part = Sg; // [rg][g][mb][v][lane]
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int v = 0; v < 4; ++v) part[(((rg * 4 + g) * MT + mb) * 4 + v) * 64 + lane] = dacc[g][v];
                    __syncthreads();
                    for (int e = tid; e < 4 * MT * 256; e += BT) {
                        float sum = 0.f;
#pragma unroll
                        for (int k = 0; k < RG; ++k) sum += part[k * 4 * MT * 256 + e];
                        const int g = e / (MT * 256), bm = (e >> 8) % MT, v = (e >> 6) & 3, ln = e & 63;
                        const int rr = bm * 16 + (ln & 15), m2 = 4 * (ln >> 4) + v;
                        if (rr < R) {
                            Cs[g * CUNIT + m2 * CSTR + rr] = sum;
                            if (m2 < D12) dT[((m2 % d2) * R + rr) * DTST + g * 4 + m2 / d2] = sum;
                        }
                    }
                } else {
                    // each item's dC block is whole in one wave
#pragma unroll
                    for (int i = 0; i < NIT; ++i) {
                        const int item = w + NW * i, g = item / MT, bm = item % MT;
                        const int rr = bm * 16 + li;
                        if (item < 4 * MT && rr < R) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int m2 = 4 * kq + v;
                                Cs[g * CUNIT + m2 * CSTR + rr] = dacc[i][v];
                                if (m2 < D12) dT[((m2 % d2) * R + rr) * DTST + g * 4 + m2 / d2] = dacc[i][v];
                            }
                        }
                    }
                }
                __syncthreads();
                constexpr int NRED = (MT * 256 + BT - 1) / BT; // (3) outputs per thread
                float rsum[NRED];
                // ---- (3) G1 partial of each unit: sum over the columns (j2, r2) of
                // dC[(g,j1)][col] G2[r1][col].  A wave takes MTW r1 blocks over
                // one of KG column groups (independent accumulator chains of
                // SPW steps); the group partials are added in group order.
                {
                    const int g = li >> 2, j1 = li & 3, kg = w % KG, mt0 = (w / KG) * MTW;
                    const bool oka = kq < d2 && j1 < d1;
                    const float *acol = dT + kq * R * DTST + li; // dT[(kq*R + s)][(g, j1) = li]
                    // the two k-quarters sharing a half-wave walk column blocks 16
                    // apart (bit 4 of the column flipped for odd kq), so their dT
                    // and G2s reads fall in distinct banks; the addresses stay
                    // base + constant along the loop
                    static_assert(SPW <= 16 || R < 32, "the column flip must not touch the step index");
                    const int sbase = (kg * SPW) ^ (R >= 32 ? 16 * (kq & 1) : 0);
                    const float *ab = acol + sbase * DTST;
                    const float *g2r[MTW];
                    bool okr1[MTW];
#pragma unroll
                    for (int m = 0; m < MTW; ++m) {
                        const int r1 = (mt0 + m) * 16 + li;
                        okr1[m] = kAllR || r1 < R;
                        g2r[m] = G2s + (okr1[m] ? r1 : 0) * G2ST + kq * R + sbase;
                    }
                    // two independent chains per output tile (even and odd steps)
                    floatx4 acc[MTW], acc2[MTW];
#pragma unroll
                    for (int m = 0; m < MTW; ++m) acc[m] = acc2[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int sl = 0; sl < SPW; sl += 2) {
                        const float a1 = ab[sl * DTST], a2 = ab[(sl + 1) * DTST];
                        const float av = oka ? a1 : 0.f, av2 = oka ? a2 : 0.f;
#pragma unroll
                        for (int m = 0; m < MTW; ++m) {
                            const float b1 = g2r[m][sl], b2 = g2r[m][sl + 1];
                            acc[m] = mfma4(av, okr1[m] ? b1 : 0.f, acc[m]);
                            acc2[m] = mfma4(av2, okr1[m] ? b2 : 0.f, acc2[m]);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < MTW; ++m)
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[m][v] += acc2[m][v];
                    float *red = Sg; // [kg][mt][v][lane]; the staged rows are no longer needed
#pragma unroll
                    for (int m = 0; m < MTW; ++m)
#pragma unroll
                        for (int v = 0; v < 4; ++v) red[((kg * MT + mt0 + m) * 4 + v) * 64 + lane] = acc[m][v];
                    __syncthreads();
                    // the group sums, in group order
                    if constexpr (kBal) {
                        for (int e = tid; e < MT * 256; e += BT) {
                            float sum = 0.f;
#pragma unroll
                            for (int k = 0; k < KG; ++k) sum += red[k * MT * 256 + e];
                            // e = (mt*4 + v)*64 + lane: row (g = lane/16, j1 = v), r1 = mt*16 + lane%16
                            const int mt = e >> 8, v = (e >> 6) & 3, ln = e & 63;
                            const int r1 = mt * 16 + (ln & 15), gg = ln >> 4;
                            if (r1 < R && gg < nu && v < d1)
                                ws.G1P[(int64_t)(rec.ubeg + gg) * a.g1stride + v * R + r1] = sum;
                        }
                    } else {
                        // rank 64: stored after (4), whose MFMAs cover the LDS
                        // latency (at lower ranks the registers held across (4) spill)
#pragma unroll
                        for (int i = 0; i < NRED; ++i) {
                            const int e = tid + i * BT;
                            float sum = 0.f;
#pragma unroll
                            for (int k = 0; k < KG; ++k) sum += red[k * MT * 256 + (e < MT * 256 ? e : 0)];
                            rsum[i] = sum;
                        }
                    }
                }
                // ---- (4) dG2 += G1^T dC over (g, j1)
                {
                    float ga[MT][4];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int r1 = mt * 16 + li;
                            const float gv = G1s[(kq * 4 + s) * G1ST + ((kAllR || r1 < R) ? r1 : 0)];
                            ga[mt][s] = (kAllR || r1 < R) ? gv : 0.f;
                        }
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int ntg = w + NW * j;
                        if (kAllNT || ntg < NT) {
                            const int col = ntg * 16 + li, j2 = col / R, r2 = col % R;
                            float bv[4];
#pragma unroll
                            for (int s = 0; s < 4; ++s) {
                                const float cv = Cs[kq * CUNIT + (s * d2 + (j2 < d2 ? j2 : 0)) * CSTR + r2];
                                bv[s] = (j2 < d2 && s < d1) ? cv : 0.f;
                            }
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                                for (int s = 0; s < 4; ++s) g2acc[mt][j] = mfma4(ga[mt][s], bv[s], g2acc[mt][j]);
                        }
                    }
                }
                if constexpr (!kBal) {
#pragma unroll
                    for (int i = 0; i < NRED; ++i) {
                        const int e = tid + i * BT;
                        const int mt = e >> 8, v = (e >> 6) & 3, ln = e & 63;
                        const int r1 = mt * 16 + (ln & 15), gg = ln >> 4;
                        if (e < MT * 256 && r1 < R && gg < nu && v < d1)
                            ws.G1P[(int64_t)(rec.ubeg + gg) * a.g1stride + v * R + r1] = rsum[i];
                    }
                }
                __syncthreads(); // (3) partials read, G1s and dC read before they are replaced
            }
            if (has_next) pf_commit(nrec, next_new);
            if (w == 0 && c + 2 < c1) reinterpret_cast<int *>(&recs[slot == 0 ? 2 : slot - 1])[lane] = pre;
        }
        // a whole run writes its dG2 slice; a piece of a split run its partial
        float *dst = slot < 0 ? a.grads.g[t][1] + (int64_t)i2 * R * d2 * R : ws.G2P + (int64_t)slot * kG2PStride;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int ntg = w + NW * j;
            if (ntg >= NT) continue;
            const int col = ntg * 16 + li;
            if (col >= d2 * R) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r1 = mt * 16 + 4 * kq + v;
                    if (r1 < R) dst[(int64_t)r1 * d2 * R + col] = g2acc[mt][j][v];
                }
        }
        __syncthreads();
    }
    if (tid == 0) block_stat_write(ws.bstat + (4 + L::CLS) * kStatBlocks, s_t0, nwork, nchunks);
}

// Run-class boundaries (runs are class-major like the units) and counters.
__global__ void k_bwd_prep(BwdArgs a)
{
    const Ws &ws = a.ws;
    const int nruns = ws.ctrl[CTRL_RUNS];
    const int c = threadIdx.x;
    if (c <= 4) {
        int lo = 0, hi = nruns;
        while (lo < hi) { // first run whose class rank is >= c
            const int mid = (lo + hi) >> 1;
            const int t = segment_of(ws.tab_unit_start, a.T, ws.uorder[ws.run_start[mid]]);
            const int cls = a.tab[t].cls, rank = cls < 0 ? 4 : cls;
            if (rank < c) lo = mid + 1;
            else hi = mid;
        }
        ws.ctrl[CTRL_RUN_CLS + c] = lo;
    }
    if (c == 5) ws.ctrl[CTRL_RUN_CLS + 5] = nruns;
    if (c == 6) { // tiles per piece of a split run: >= kPieceTiles and >= 2 * tiles / slots
        const int64_t tiles = ws.ctrl[CTRL_TILES];
        const int64_t need = (2 * tiles + a.g2p_slots - 1) / a.g2p_slots;
        ws.ctrl[CTRL_PIECE_TILES] = (int)(need > kPieceTiles ? need : kPieceTiles);
    }
    if (c < 4) {
        ws.ctrl[CTRL_BWD_NEXT + c] = 0;
        ws.bstat[(4 + c) * kStatBlocks].nb = 0; // backward class records
    }
}

// Backward pieces.  A (table, i2) run accumulates its dG2 slice in registers
// from its first tile to its last, so one long run (a Zipf-hot i2 digit of a
// large table) is a single block's work; at ranks <= 32 such runs are longer
// than a block's fair share.  A run of those classes with more than PT tiles
// is cut into ceil(tiles / PT) tile-aligned pieces of near-equal size; each
// piece writes its dG2 partial to a slot of its own and k_reduce_g2p adds the
// slots of a run in piece order (fixed order, no atomics).  PT >= 8 and
// PT >= 2 * tiles / slots, so the slots in the workspace always suffice.
struct PieceOp {
    BwdArgs a;
    __device__ int64_t count() const { return a.ws.ctrl[CTRL_RUNS]; }
    __device__ uint64_t value(int64_t r) const
    {
        const Ws &ws = a.ws;
        const int t = segment_of(ws.tab_unit_start, a.T, ws.uorder[ws.run_start[r]]);
        const int cls = a.tab[t].cls;
        const int nt = ws.run_tile_start[r + 1] - ws.run_tile_start[r];
        const int PT = ws.ctrl[CTRL_PIECE_TILES];
        if (cls < 0 || cls > kSplitMaxCls || nt <= PT) return (uint64_t)1 << 32; // one piece, no slot
        const uint64_t np = (uint64_t)((nt + PT - 1) / PT);
        return (np << 32) | np; // pieces (high word) and slots (low word)
    }
    __device__ void emit(int64_t r, uint64_t excl, uint64_t) const
    {
        a.ws.run_pbase[r] = (int32_t)(excl >> 32);
        a.ws.run_sbase[r] = (int32_t)(excl & 0xffffffffu);
    }
    __device__ void total(uint64_t tot, int64_t n) const
    {
        a.ws.ctrl[CTRL_PIECES] = (int32_t)(tot >> 32);
        a.ws.ctrl[CTRL_SLOTS] = (int32_t)(tot & 0xffffffffu);
        a.ws.run_pbase[n] = (int32_t)(tot >> 32);
        a.ws.run_sbase[n] = (int32_t)(tot & 0xffffffffu);
    }
};

// Pieces of every run, and their claim order keys (longest-processing-time
// first, so that long pieces do not start last and leave a tail): key = class
// rank (runs, hence pieces, are class-major, so each class keeps its slice of
// positions) above the piece's chunk count, descending; the stable sort keeps
// equal pieces in piece order.  The order changes only which block computes a
// piece: every piece writes its own results, so the output does not depend on it.
constexpr int kRunKeyBits = 16, kRunCostBits = 13;
__global__ __launch_bounds__(kThreads) void k_piece_fill(BwdArgs a)
{
    const Ws &ws = a.ws;
    const int nruns = ws.ctrl[CTRL_RUNS];
    if (blockIdx.x == 0 && threadIdx.x < 6) // first piece of each class, then the total
        ws.ctrl[CTRL_PIECE_CLS + threadIdx.x] = ws.run_pbase[ws.ctrl[CTRL_RUN_CLS + threadIdx.x]];
    for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < nruns; r += gridDim.x * blockDim.x) {
        const int t = segment_of(ws.tab_unit_start, a.T, ws.uorder[ws.run_start[r]]);
        const int cls = a.tab[t].cls, rank = cls < 0 ? 4 : cls;
        const int pb = ws.run_pbase[r], np = ws.run_pbase[r + 1] - pb, sb = ws.run_sbase[r];
        const int tb0 = ws.run_tile_start[r], nt = ws.run_tile_start[r + 1] - tb0;
        constexpr int cmax = (1 << kRunCostBits) - 1;
        for (int j = 0; j < np; ++j) {
            const int k = pb + j;
            const int tb = tb0 + (int)((int64_t)j * nt / np), te = tb0 + (int)((int64_t)(j + 1) * nt / np);
            ws.piece_tb[k] = tb;
            ws.piece_te[k] = te;
            ws.piece_slot[k] = np > 1 ? sb + j : -1;
            int nch = ws.tile_cstart[te] - ws.tile_cstart[tb];
            nch = nch < cmax ? nch : cmax;
            ws.rkey0[k] = ((uint32_t)rank << kRunCostBits) | (uint32_t)(cmax - nch);
            ws.rval0[k] = k;
        }
    }
}

// dG2[i2] of every split run = its pieces' partials added in piece order.
__global__ __launch_bounds__(kThreads) void k_reduce_g2p(BwdArgs a)
{
    const Ws &ws = a.ws;
    const int nruns = ws.ctrl[CTRL_RUNS];
    for (int r = blockIdx.x; r < nruns; r += gridDim.x) {
        const int pb = ws.run_pbase[r], np = ws.run_pbase[r + 1] - pb;
        if (np <= 1) continue;
        const int sb = ws.run_sbase[r];
        const ChunkRec &rec = ws.crec[ws.tile_cstart[ws.run_tile_start[r]]];
        const int t = rec.t, i2 = rec.i2;
        const TableDesc &tb = a.tab[t];
        const int n = tb.R1 * tb.d2 * tb.R2;
        float *dst = a.grads.g[t][1] + (int64_t)i2 * n;
        for (int e = threadIdx.x; e < n; e += blockDim.x) {
            float acc = ws.G2P[(int64_t)sb * kG2PStride + e];
            for (int j = 1; j < np; ++j) acc += ws.G2P[(int64_t)(sb + j) * kG2PStride + e];
            dst[e] = acc;
        }
    }
}

// Transposed G3 copies of the MFMA-class tables (G3t[i3][j3][r2]).
__global__ __launch_bounds__(kThreads) void k_bwd_g3t(BwdArgs a)
{
    const int t = blockIdx.y;
    const TableDesc &tb = a.tab[t];
    if (tb.cls < 0) return;
    const int R2 = tb.R2, d3 = tb.d3, per = R2 * d3;
    const int64_t n = (int64_t)tb.n3 * per;
    const float *src = a.cores.g[t][2];
    float *dst = a.ws.g3t + tb.g3t_off;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i3 = i / per;
        const int rem = (int)(i - i3 * per), j3 = rem / R2, r2 = rem - j3 * R2;
        dst[i] = src[(i3 * R2 + r2) * d3 + j3];
    }
}

// Zero every dG2 core (runs overwrite the slices they own) and the run counter.
__global__ __launch_bounds__(kThreads) void k_zero_g2(BwdArgs a)
{
    const int t = blockIdx.y;
    const TableDesc &tb = a.tab[t];
    const int64_t n = (int64_t)tb.n2 * tb.R1 * tb.d2 * tb.R2;
    float *g = a.grads.g[t][1];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        g[i] = 0.f;
}

hipError_t launch_lookup_meta(const Plan &p, const int64_t *offsets, hipStream_t s)
{
    BwdArgs a{p.dtab, p.T, p.B, p.ws, CorePtrs{}, GradPtrs{}, nullptr, offsets, p.nnz, p.sumD, p.Dpmax,
              p.force_generic, p.g1stride};
    const int64_t nbags = (int64_t)p.T * p.B;
    if (p.nnz > 0 && nbags > 0) {
        int g = ceil_div(nbags, kThreads);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(k_lookup_meta, dim3(g), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gu_gather(const Plan &p, const float *grad_out, const int64_t *offsets, hipStream_t s)
{
    BwdArgs a{p.dtab, p.T, p.B, p.ws, CorePtrs{}, GradPtrs{}, grad_out, offsets, p.nnz, p.sumD, p.Dpmax,
              p.force_generic, p.g1stride, p.g2p_slots};
    const int T = p.T;
    if (p.nnz > 0) {
        const int64_t nbags = (int64_t)T * p.B;
        int g = ceil_div(nbags, kThreads);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(k_lookup_meta, dim3(g), dim3(kThreads), 0, s, a);
        // virtual-XCD launches: multiples of 8 blocks
        // one chunk per block where the grid allows (the chain of loads per
        // chunk is then overlapped across resident blocks)
        int64_t gm = ceil_div(p.nnz, (int64_t)kSmChunk);
        gm = (gm + 7) & ~int64_t(7);
        gm = gm > 65536 ? 65536 : gm;
        hipLaunchKernelGGL(k_sorted_meta, dim3((int)gm), dim3(kThreads), 0, s, a);
        const int64_t tasks = p.nnz / kGuTask + T + 1;
        int gg = (kGuBlocksPerCu * p.num_blocks) & ~7;
        gg = gg < 8 ? 8 : gg;
        hipLaunchKernelGGL(k_gu_gather, dim3(gg), dim3(kThreads), 0, s, a);
        int gj = ceil_div(tasks, kThreads / 64);
        gj = gj > 4096 ? 4096 : gj;
        hipLaunchKernelGGL(k_gu_join, dim3(gj), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_backward(const Plan &p, const float *grad_out, const CorePtrs &cores,
                           const int64_t *offsets, const GradPtrs &grads, hipStream_t s)
{
    BwdArgs a{p.dtab, p.T, p.B, p.ws, cores, grads, grad_out, offsets, p.nnz, p.sumD, p.Dpmax, p.force_generic,
              p.g1stride, p.g2p_slots};
    const int T = p.T;
    const int sum_n1 = p.sum_n[0], sum_n3 = p.sum_n[2];
    timer_begin(p.timing, TM_BWD_GATHER, s);
    hipLaunchKernelGGL(k_zero_g2, dim3(256, T), dim3(kThreads), 0, s, a);
    {
        hipError_t e = launch_gu_gather(p, grad_out, offsets, s);
        if (e != hipSuccess) return e;
    }
    timer_end(p.timing, TM_BWD_GATHER, s);
    timer_begin(p.timing, TM_BWD_CONTRACT, s);
    if (p.nnz > 0) {
        if (!p.force_generic) {
            hipLaunchKernelGGL(k_bwd_prep, dim3(1), dim3(64), 0, s, a);
            hipLaunchKernelGGL(k_bwd_g3t, dim3(64, T), dim3(kThreads), 0, s, a);
            {   // pieces of the runs and their claim order (bounds as in the workspace plan)
                const int64_t runs_bound = (p.nnz < p.sum_n[1] ? p.nnz : p.sum_n[1]) + 1;
                const int64_t pieces_bound = runs_bound + p.g2p_slots;
                PieceOp op{a};
                hipError_t e = run_scan(op, p.ws.part, scan_blocks(runs_bound), s);
                if (e != hipSuccess) return e;
                int g = ceil_div(runs_bound, kThreads);
                g = g > 1024 ? 1024 : g;
                hipLaunchKernelGGL(k_piece_fill, dim3(g), dim3(kThreads), 0, s, a);
                bool in1 = false;
                e = radix_sort_pairs(p, p.ws.rkey0, p.ws.rval0, p.ws.rkey1, p.ws.rval1, pieces_bound,
                                     &p.ws.ctrl[CTRL_PIECES], kRunKeyBits, &in1, s);
                if (e != hipSuccess) return e;
                a.ws.rorder = in1 ? p.ws.rval1 : p.ws.rval0;
            }
            for (int c = 0; c < 4; ++c) {
                if (!(p.cls_mask & (1 << c))) continue;
                timer_begin(p.timing, TM_BWD_CLS0 + c, s);
                switch (c * 2 + (p.reuse_c && c >= kKeepMinCls ? 1 : 0)) {
#define TT_BWD_CLASS(RR, RU)                                                                                    \
    hipLaunchKernelGGL((k_bwd_class<RR, RU>), dim3(p.num_blocks * BwdLds<RR>::OCC), dim3(BwdLds<RR>::NW * 64), 0, \
                       s, a)
                case 0: TT_BWD_CLASS(8, false); break;
                case 2: TT_BWD_CLASS(16, false); break;
                case 4: TT_BWD_CLASS(32, false); break;
                case 5: TT_BWD_CLASS(32, true); break;
                case 6: TT_BWD_CLASS(64, false); break;
                default: TT_BWD_CLASS(64, true); break;
#undef TT_BWD_CLASS
                }
                timer_end(p.timing, TM_BWD_CLS0 + c, s);
            }
            int g = p.sum_n[1] < 4096 ? p.sum_n[1] : 4096;
            hipLaunchKernelGGL(k_reduce_g2p, dim3(g > 0 ? g : 1), dim3(kThreads), 0, s, a);
        }
        if (p.force_generic || p.any_generic)
            hipLaunchKernelGGL(k_bwd_runs, dim3(p.num_blocks * 2), dim3(kThreads), 0, s, a);
    }
    timer_end(p.timing, TM_BWD_CONTRACT, s);
    timer_begin(p.timing, TM_BWD_REDUCE, s);
    hipLaunchKernelGGL(k_reduce_g1, dim3(sum_n1 > 0 ? (sum_n1 < 65535 ? sum_n1 : 65535) : 1), dim3(kThreads), 0,
                       s, a, sum_n1);
    // dG3: sort unique rows by (table, i3) into buffers the forward no longer needs
    const uint32_t *k3 = nullptr;
    const int32_t *o3 = nullptr;
    if (p.nnz > 0) {
        int g = ceil_div(p.nnz, kThreads * 4);
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(k_key3, dim3(g), dim3(kThreads), 0, s, a, p.ws.keys0, p.ws.u3order);
        bool in1 = false;
        hipError_t e = radix_sort_pairs(p, p.ws.keys0, p.ws.u3order, p.ws.keys1, p.ws.uvals_free,
                                        p.nnz, &p.ws.ctrl[CTRL_U], p.key3_bits, &in1, s);
        if (e != hipSuccess) return e;
        k3 = in1 ? p.ws.keys1 : p.ws.keys0;
        o3 = in1 ? p.ws.uvals_free : p.ws.u3order;
    } else {
        k3 = p.ws.keys0;
        o3 = p.ws.u3order;
    }
    {
        hipError_t e = launch_fill_i32(p.ws.g3rng, 0, 2 * (int64_t)sum_n3, s);
        if (e != hipSuccess) return e;
        int g = ceil_div(p.nnz > 0 ? p.nnz : 1, kThreads);
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(k_g3_bounds, dim3(g), dim3(kThreads), 0, s, a, k3, sum_n3);
    }
    hipLaunchKernelGGL(k_reduce_g3, dim3(sum_n3 > 0 ? (sum_n3 < 65535 ? sum_n3 : 65535) : 1), dim3(kThreads), 0,
                       s, a, o3, sum_n3);
    timer_end(p.timing, TM_BWD_REDUCE, s);
    return hipGetLastError();
}

} // namespace ttemb
