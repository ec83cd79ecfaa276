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
//   * g_u is summed over the sorted lookup run of u; runs longer than one
//     piece are cut into fixed pieces whose partials are added in order;
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
    int Dmax; // row stride of the gather partials
};

// bag_of[l] for every lookup (clamped ranges; used only through clamps).
__global__ __launch_bounds__(kThreads) void k_bag_of(BwdArgs a)
{
    const int64_t nbags = (int64_t)a.T * a.B;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nbags; b += stride) {
        int64_t lo = a.offsets[b], hi = a.offsets[b + 1];
        lo = lo < 0 ? 0 : (lo > a.nnz ? a.nnz : lo);
        hi = hi < lo ? lo : (hi > a.nnz ? a.nnz : hi);
        for (int64_t l = lo; l < hi; ++l) a.ws.bag_of[l] = (int32_t)b;
    }
}

// Pieces of the gradient gather: run u is cut into ceil(len / kGuPiece) pieces.
struct PieceOp {
    Ws ws;
    __device__ int64_t count() const { return ws.ctrl[CTRL_U]; }
    __device__ uint64_t value(int64_t u) const
    {
        const int64_t len = ws.uniq_start[u + 1] - ws.uniq_start[u];
        return (uint64_t)((len + kGuPiece - 1) / kGuPiece);
    }
    __device__ void emit(int64_t u, uint64_t excl, uint64_t v) const
    {
        ws.u_piece_start[u] = (int32_t)excl;
        for (uint64_t j = 0; j < v; ++j) {
            ws.piece_u[excl + j] = (int32_t)u;
            ws.piece_k[excl + j] = ws.uniq_start[u] + (int32_t)j * kGuPiece;
        }
    }
    __device__ void total(uint64_t tot, int64_t U) const
    {
        ws.ctrl[CTRL_PIECES] = (int32_t)tot;
        ws.u_piece_start[U] = (int32_t)tot;
    }
};

// One wave per piece: sum grad_out rows of the piece's lookups (sorted order).
// Single-piece runs write g_u straight into the unique-row buffer (E's space);
// longer runs write a partial, combined in piece order by k_gu_combine.
__global__ __launch_bounds__(kThreads) void k_gu_pieces(BwdArgs a)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const Ws &ws = a.ws;
    const int64_t np = ws.ctrl[CTRL_PIECES];
    const int64_t nbags = (int64_t)a.T * a.B;
    for (int64_t p = (int64_t)blockIdx.x * 4 + w; p < np; p += (int64_t)gridDim.x * 4) {
        const int u = ws.piece_u[p];
        const int k0 = ws.piece_k[p];
        const int kend = ws.uniq_start[u + 1];
        const int k1 = k0 + kGuPiece < kend ? k0 + kGuPiece : kend;
        const int t = segment_of(ws.tab_uniq_start, a.T, u);
        const TableDesc &tb = a.tab[t];
        const int D = tb.D;
        const bool single = (ws.u_piece_start[u + 1] - ws.u_piece_start[u]) == 1;
        float *dst = single ? ws.E + ws.ebase[t] + (int64_t)u * tb.Dp : ws.P3 + p * (int64_t)a.Dmax;
        for (int j0 = 0; j0 < D; j0 += 64) {
            const int j = j0 + lane;
            float acc = 0.f;
            for (int k = k0; k < k1; ++k) {
                int64_t bag = ws.bag_of[ws.perm[k]];
                bag = bag < 0 ? 0 : (bag >= nbags ? nbags - 1 : bag);
                const int64_t b = bag - (int64_t)t * a.B;
                const int64_t bb = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
                if (j < D) acc += a.grad_out[bb * a.SD + tb.col_off + j];
            }
            if (j < D) dst[j] = acc;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_gu_combine(BwdArgs a)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const Ws &ws = a.ws;
    const int64_t U = ws.ctrl[CTRL_U];
    for (int64_t u = (int64_t)blockIdx.x * 4 + w; u < U; u += (int64_t)gridDim.x * 4) {
        const int p0 = ws.u_piece_start[u], p1 = ws.u_piece_start[u + 1];
        if (p1 - p0 <= 1) continue;
        const int t = segment_of(ws.tab_uniq_start, a.T, u);
        const TableDesc &tb = a.tab[t];
        float *dst = ws.E + ws.ebase[t] + u * (int64_t)tb.Dp;
        for (int j = lane; j < tb.D; j += 64) {
            float acc = 0.f;
            for (int p = p0; p < p1; ++p) acc += ws.P3[p * (int64_t)a.Dmax + j];
            dst[j] = acc;
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
                ws.G1P[ws.g1base[t] + (int64_t)unit * d1 * R1 + e] = c;
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
__global__ __launch_bounds__(kThreads) void k_reduce_g1(BwdArgs a, int total_slots)
{
    const Ws &ws = a.ws;
    for (int slot = blockIdx.x; slot < total_slots; slot += gridDim.x) {
        int t = 0;
        while (t + 1 < a.T && a.tab[t + 1].i1_base <= (uint32_t)slot) ++t;
        const TableDesc &tb = a.tab[t];
        const int i1 = slot - (int)tb.i1_base;
        if (i1 >= tb.n1) continue;
        const int lo0 = ws.tab_unit_start[t], hi0 = ws.tab_unit_start[t + 1];
        const int qlo = i1 * tb.n2, qhi = qlo + tb.n2;
        int lo = lo0, hi = hi0;
        while (lo < hi) { // first unit with prefix >= qlo
            const int mid = (lo + hi) >> 1;
            if (ws.unit_prefix[mid] < qlo) lo = mid + 1;
            else hi = mid;
        }
        const int first = lo;
        hi = hi0;
        while (lo < hi) { // first unit with prefix >= qhi
            const int mid = (lo + hi) >> 1;
            if (ws.unit_prefix[mid] < qhi) lo = mid + 1;
            else hi = mid;
        }
        const int last = lo;
        const int per = tb.d1 * tb.R1;
        float *dst = a.grads.g[t][0] + (int64_t)i1 * per;
        for (int e = threadIdx.x; e < per; e += kThreads) {
            float c = 0.f;
            for (int unit = first; unit < last; ++unit) c += ws.G1P[ws.g1base[t] + (int64_t)unit * per + e];
            dst[e] = c;
        }
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

// dG3[t][i3] = sum over unique rows of table t with that i3, in unique-id
// order, of their partials; zero when none.
__global__ __launch_bounds__(kThreads) void k_reduce_g3(BwdArgs a, const uint32_t *k3,
                                                        const int32_t *order, int total_slots)
{
    const Ws &ws = a.ws;
    const int64_t U = ws.ctrl[CTRL_U];
    for (int slot = blockIdx.x; slot < total_slots; slot += gridDim.x) {
        int t = 0;
        while (t + 1 < a.T && a.tab[t + 1].i3_base <= (uint32_t)slot) ++t;
        const TableDesc &tb = a.tab[t];
        const int i3 = slot - (int)tb.i3_base;
        if (i3 >= tb.n3) continue;
        int64_t lo = 0, hi = U;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (k3[mid] < (uint32_t)slot) lo = mid + 1;
            else hi = mid;
        }
        const int64_t first = lo;
        hi = U;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (k3[mid] <= (uint32_t)slot) lo = mid + 1;
            else hi = mid;
        }
        const int64_t last = lo;
        const int per = tb.R2 * tb.d3;
        float *dst = a.grads.g[t][2] + (int64_t)i3 * per;
        for (int e = threadIdx.x; e < per; e += kThreads) {
            float c = 0.f;
            for (int64_t q = first; q < last; ++q) c += ws.P3[ws.p3base[t] + (int64_t)order[q] * per + e];
            dst[e] = c;
        }
    }
}

// Zero every dG2 core (runs overwrite the slices they own).
__global__ __launch_bounds__(kThreads) void k_zero_g2(BwdArgs a)
{
    const int t = blockIdx.y;
    const TableDesc &tb = a.tab[t];
    const int64_t n = (int64_t)tb.n2 * tb.R1 * tb.d2 * tb.R2;
    float *g = a.grads.g[t][1];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        g[i] = 0.f;
}

hipError_t launch_backward(const Plan &p, const float *grad_out, const CorePtrs &cores,
                           const int64_t *offsets, const GradPtrs &grads, hipStream_t s)
{
    BwdArgs a{p.dtab, p.T, p.B, p.ws, cores, grads, grad_out, offsets, p.nnz, p.sumD, p.Dmax};
    const int T = p.T;
    const int sum_n1 = p.sum_n[0], sum_n3 = p.sum_n[2];
    timer_begin(p.timing, TM_BWD_GATHER, s);
    hipLaunchKernelGGL(k_zero_g2, dim3(256, T), dim3(kThreads), 0, s, a);
    if (p.nnz > 0) {
        const int64_t nbags = (int64_t)T * p.B;
        int g = ceil_div(nbags, kThreads);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(k_bag_of, dim3(g), dim3(kThreads), 0, s, a);
        PieceOp pop{p.ws};
        hipError_t e = run_scan(pop, p.ws.part, scan_blocks(p.nnz), s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_gu_pieces, dim3(4096), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(k_gu_combine, dim3(2048), dim3(kThreads), 0, s, a);
    }
    timer_end(p.timing, TM_BWD_GATHER, s);
    timer_begin(p.timing, TM_BWD_CONTRACT, s);
    if (p.nnz > 0) hipLaunchKernelGGL(k_bwd_runs, dim3(p.num_blocks * 2), dim3(kThreads), 0, s, a);
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
    hipLaunchKernelGGL(k_reduce_g3, dim3(sum_n3 > 0 ? (sum_n3 < 65535 ? sum_n3 : 65535) : 1), dim3(kThreads), 0,
                       s, a, k3, o3, sum_n3);
    timer_end(p.timing, TM_BWD_REDUCE, s);
    return hipGetLastError();
}

} // namespace ttemb
