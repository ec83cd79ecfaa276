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
    int force_generic;
    int g1stride; // row stride of the G1 partials (max d1*R1)
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
        const float *go = a.grad_out + tb.col_off;
        // lanes per row: float4 columns rounded up to a power of two; rows in flight
        const int c4n = (D + 3) >> 2;
        int lpr = 1;
        while (lpr < c4n) lpr <<= 1;
        const bool vec = lpr <= 64 && ((a.SD | tb.col_off) & 3) == 0;
        if (vec) {
            const int rf = 64 / lpr, c4 = lane & (lpr - 1), r = lane / lpr;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int kb = k0; kb < k1; kb += 64) {
                const int nk = k1 - kb < 64 ? k1 - kb : 64;
                // the bag (row of grad_out) of lookups kb .. kb+63, one per lane
                int64_t bb = 0;
                if (lane < nk) {
                    int64_t bag = ws.bag_of[ws.perm[kb + lane]];
                    bag = bag < 0 ? 0 : (bag >= nbags ? nbags - 1 : bag);
                    const int64_t b = bag - (int64_t)t * a.B;
                    bb = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
                }
#pragma unroll 4
                for (int i = 0; i < nk; i += rf) {
                    const int64_t row = __shfl(bb, i + r < 64 ? i + r : 0, 64);
                    if (i + r < nk && c4 < c4n) {
                        const float4 v = reinterpret_cast<const float4 *>(go + row * a.SD)[c4];
                        acc.x += v.x;
                        acc.y += v.y;
                        acc.z += v.z;
                        acc.w += v.w;
                    }
                }
            }
            for (int m = lpr; m < 64; m <<= 1) {
                acc.x += __shfl_xor(acc.x, m, 64);
                acc.y += __shfl_xor(acc.y, m, 64);
                acc.z += __shfl_xor(acc.z, m, 64);
                acc.w += __shfl_xor(acc.w, m, 64);
            }
            if (r == 0 && c4 < c4n) {
                const int j = 4 * c4;
                if (j + 0 < D) dst[j + 0] = acc.x;
                if (j + 1 < D) dst[j + 1] = acc.y;
                if (j + 2 < D) dst[j + 2] = acc.z;
                if (j + 3 < D) dst[j + 3] = acc.w;
            }
        } else {
            for (int j0 = 0; j0 < D; j0 += 64) {
                const int j = j0 + lane;
                float acc = 0.f;
                for (int k = k0; k < k1; ++k) {
                    int64_t bag = ws.bag_of[ws.perm[k]];
                    bag = bag < 0 ? 0 : (bag >= nbags ? nbags - 1 : bag);
                    const int64_t b = bag - (int64_t)t * a.B;
                    const int64_t bb = b < 0 ? 0 : (b >= a.B ? a.B - 1 : b);
                    if (j < D) acc += go[bb * a.SD + j];
                }
                if (j < D) dst[j] = acc;
            }
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
            for (int unit = first; unit < last; ++unit) c += ws.G1P[(int64_t)ws.uinv[unit] * a.g1stride + e];
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
        const float *src = ws.P3 + ws.p3base[t];
        // rp row phases of per-element threads; phase ph sums rows first+ph,
        // first+ph+rp, ... in order, then the phases are added in order.
        const int rp = per >= kThreads ? 1 : kThreads / per;
        const int ph = threadIdx.x / per < rp ? threadIdx.x / per : rp; // rp = idle
        __shared__ float part[kThreads];
        for (int e0 = 0; e0 < per; e0 += kThreads) {
            const int e = e0 + (rp == 1 ? threadIdx.x : threadIdx.x - ph * per);
            float c = 0.f;
            if (ph < rp && e < per) {
#pragma unroll 8
                for (int64_t q = first + ph; q < last; q += rp) c += src[(int64_t)order[q] * per + e];
            }
            if (rp == 1) {
                if (e < per) dst[e] = c;
            } else {
                part[threadIdx.x] = c;
                __syncthreads();
                if (threadIdx.x < per) {
                    float s = 0.f;
                    for (int k = 0; k < rp; ++k) s += part[k * per + threadIdx.x];
                    dst[threadIdx.x] = s;
                }
                __syncthreads();
            }
        }
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
    static constexpr int G2S = R * NCOL;
    static constexpr int CS = 4 * CUNIT;
    static constexpr int G1ST = R + 1;                 // odd row stride: (1) reads rows across lanes
    static constexpr int G1S = 16 * G1ST;              // [unit][j1][r1]
    static constexpr int DTST = 17;                    // transposed dC: [col][(g, j1)], stride 17
    static constexpr int STAGE = CLS == 3 ? 14336 : CLS == 2 ? 10240 : 6144;
    static constexpr int TOTAL = G2S + 2 * CS + G1S + STAGE;
    static constexpr int OCC = CLS == 3 ? 1 : CLS == 2 ? 2 : 4; // blocks per CU
    static constexpr int NW = CLS == 3 ? 8 : 4;                  // waves per block
};

template <int R>
__global__ __launch_bounds__(BwdLds<R>::NW * 64, BwdLds<R>::OCC) void k_bwd_class(BwdArgs a)
{
    using L = BwdLds<R>;
    constexpr int NW = L::NW, BT = NW * 64;
    constexpr int NCOL = L::NCOL, NT = NCOL / 16, NTW = (NT + NW - 1) / NW, MT = (R + 15) / 16, KQ = R / 4;
    constexpr int NIT = (4 * MT + NW - 1) / NW;  // (unit, r-block) items per wave
    constexpr int KS = NW / MT, SPL = R / KS, CSTR = L::CSTR, CUNIT = L::CUNIT;
    static_assert((SPL & (SPL - 1)) == 0, "k-split length is a power of two");
    __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
    __shared__ ChunkRec recs[2];
    __shared__ int s_run;
    // Cs holds C during a tile and dC at its end (C is dead by then); dT holds
    // dC transposed ([col][(g, j1)]) for the dG1 partials
    float *G2s = lds, *Cs = lds + L::G2S, *dT = Cs + L::CS, *G1s = dT + L::CS, *Sg = G1s + L::G1S;
    static_assert(L::NCOL * L::DTST <= L::CS, "transposed dC fits in its region");
    constexpr int G1ST = L::G1ST, DTST = L::DTST;
    const Ws &ws = a.ws;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, kq = lane >> 4;
    const int rbeg = ws.ctrl[CTRL_RUN_CLS + L::CLS], rend = ws.ctrl[CTRL_RUN_CLS + L::CLS + 1];
    for (;;) {
        if (tid == 0) s_run = rbeg + atomicAdd(&ws.ctrl[CTRL_BWD_NEXT + L::CLS], 1);
        __syncthreads();
        const int run = s_run;
        if (run >= rend) break;
        const int c0 = ws.tile_cstart[ws.run_tile_start[run]], c1 = ws.tile_cstart[ws.run_tile_start[run + 1]];
        if (w == 0) reinterpret_cast<int *>(&recs[0])[lane] = reinterpret_cast<const int *>(&ws.crec[c0])[lane];
        __syncthreads();
        const int t = recs[0].t, i2 = recs[0].i2;
        const TableDesc &tb = a.tab[t];
        const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, D12 = d1 * d2, Dp = tb.Dp, P = 16 / d3;
        const float *G1 = a.cores.g[t][0];
        const float *G3t = ws.g3t + tb.g3t_off;
        // staged rows: g_u at stride Dp + 4, G3 slices as [j3][R + 16] (bank-spread)
        const int GST = Dp + 4, G3J = R + 16, G3ST = d3 * G3J;
        int rb = L::STAGE / (GST + G3ST);
        rb = rb < kMaxChunkRows ? rb : kMaxChunkRows;
        float *Gs = Sg, *G3s = Sg + rb * GST;
        {   // stage G2[i2] as G2s[r][col ^ (r & 31)], zero-padded to NCOL columns
            const float *src = a.cores.g[t][1] + (int64_t)i2 * R * d2 * R;
            for (int e = tid; e < R * NCOL; e += BT) {
                const int r = e / NCOL, c = e - r * NCOL;
                G2s[r * NCOL + (c ^ (r & 31))] = c < d2 * R ? src[r * d2 * R + c] : 0.f;
            }
        }
        floatx4 g2acc[MT][NTW], dacc[NIT];
#pragma unroll
        for (int ii = 0; ii < NIT; ++ii) dacc[ii] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) g2acc[mt][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        int cur_tile = -1, buf = 0;
        for (int c = c0; c < c1; ++c) {
            const ChunkRec &rec = recs[buf];
            // the next record travels while this chunk runs
            int pre = 0;
            if (w == 0 && c + 1 < c1) pre = reinterpret_cast<const int *>(&ws.crec[c + 1])[lane];
            const int nu = rec.nu;
            const bool new_tile = rec.tile != cur_tile;
            const int nrows = rec.rowoff[4];
            // ---- one burst of independent loads: the tile's G1 slices (new tile
            // only, G1s[(g*4 + j1)*G1ST + r1], zeros outside) and the first batch of rows
            const int c4g = Dp >> 2, c4t = (d3 * R) >> 2;
            auto stage_rows = [&](int sb, int n) {
                for (int e = tid; e < n * (c4g + c4t); e += BT) {
                    const int qq = e / (c4g + c4t), rem = e - qq * (c4g + c4t), q = sb + qq;
                    int j = 0;
                    while (j < 3 && q >= rec.rowoff[j + 1]) ++j;
                    if (rem < c4g) {
                        const int u = rec.ustart[j] + (q - rec.rowoff[j]);
                        *reinterpret_cast<float4 *>(Gs + qq * GST + 4 * rem) =
                            reinterpret_cast<const float4 *>(ws.E + ws.ebase[t] + (int64_t)u * Dp)[rem];
                    } else {
                        const int r4 = rem - c4g, j3 = (4 * r4) / R, r = 4 * r4 - j3 * R;
                        *reinterpret_cast<float4 *>(G3s + qq * G3ST + j3 * G3J + r) =
                            reinterpret_cast<const float4 *>(G3t + (int64_t)rec.i3[q] * d3 * R)[r4];
                    }
                }
            };
            if (new_tile) {
                for (int e = tid; e < 4 * R; e += BT) {
                    const int gj = e / (R / 4), r4 = e - gj * (R / 4), g = gj >> 2, j1 = gj & 3;
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (g < nu && j1 < d1) v = reinterpret_cast<const float4 *>(G1 + ((int64_t)rec.i1[g] * d1 + j1) * R)[r4];
                    float *d = G1s + gj * G1ST + 4 * r4;
                    d[0] = v.x;
                    d[1] = v.y;
                    d[2] = v.z;
                    d[3] = v.w;
                }
            }
            stage_rows(0, nrows < rb ? nrows : rb);
            __syncthreads();
            if (new_tile) {
                // ---- (1) prefix tile C
                {
                    const int g = li >> 2, j1 = li & 3;
                    floatx4 acc[NTW];
#pragma unroll
                    for (int j = 0; j < NTW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KQ; ++s) {
                        const int r = kq * KQ + s;
                        const float av = G1s[(g * 4 + j1) * G1ST + r];
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            const int ntg = w + NW * j;
                            if (ntg < NT) {
                                const int col = ntg * 16 + li;
                                acc[j] = mfma4(av, G2s[r * NCOL + (col ^ (r & 31))], acc[j]);
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int ntg = w + NW * j;
                        if (ntg < NT) {
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
                for (int ii = 0; ii < NIT; ++ii) dacc[ii] = floatx4{0.f, 0.f, 0.f, 0.f};
                cur_tile = rec.tile;
            }
            // ---- (2) rows of this chunk, in staged batches of rb rows (the first is staged)
            for (int sb = 0; sb < nrows; sb += rb) {
                const int n = nrows - sb < rb ? nrows - sb : rb;
                __syncthreads(); // C tile written; previous batch consumed
                if (sb > 0) {
                    stage_rows(sb, n);
                    __syncthreads();
                }
#pragma unroll
                for (int ii = 0; ii < NIT; ++ii) {
                    const int item = w + NW * ii, g = item / MT, mb = item % MT;
                    if (item >= 4 * MT || g >= nu) continue;
                    const int r2 = mb * 16 + li;
                    const bool okr = r2 < R;
                    const int qa = sb > rec.rowoff[g] ? sb : rec.rowoff[g];
                    const int qe = rec.rowoff[g] + rec.ccnt[g];
                    const int qb = sb + n < qe ? sb + n : qe;
                    // (2a) dC_g[m2][r2] += sum_j3 g_u[m2][j3] G3[i3_u][r2][j3]
                    for (int q = qa; q < qb; ++q) {
                        const float *gq = Gs + (q - sb) * GST;
                        const float *g3 = G3s + (q - sb) * G3ST + (okr ? r2 : 0);
                        for (int j0 = 0; j0 < d3; j0 += 4) {
                            const int j3 = j0 + kq;
                            const float av = (li < D12 && j3 < d3) ? gq[li * d3 + j3] : 0.f;
                            const float bv = (okr && j3 < d3) ? g3[j3 * G3J] : 0.f;
                            dacc[ii] = mfma4(av, bv, dacc[ii]);
                        }
                    }
                    // (2b) P3_u[r2][j3] = sum_m2 C_g[m2][r2] g_u[m2][j3], P rows per output tile
                    float ca[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int m2 = kq * 4 + s;
                        ca[s] = (m2 < D12 && okr) ? Cs[g * CUNIT + m2 * CSTR + r2] : 0.f;
                    }
                    const int slot = li / d3, j3 = li - slot * d3;
                    for (int qs = qa; qs < qb; qs += P) {
                        const int cnt = qb - qs < P ? qb - qs : P;
                        const bool okb = slot < cnt;
                        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int m2 = kq * 4 + s;
                            const float bv = (okb && m2 < D12) ? Gs[(qs + slot - sb) * GST + m2 * d3 + j3] : 0.f;
                            acc = mfma4(ca[s], bv, acc);
                        }
                        if (okb) {
                            const int u = rec.ustart[g] + (qs + slot - rec.rowoff[g]);
                            float *dst = ws.P3 + ws.p3base[t] + (int64_t)u * R * d3 + j3;
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int rr = mb * 16 + 4 * kq + v;
                                if (rr < R) dst[rr * d3] = acc[v];
                            }
                        }
                    }
                }
            }
            // ---- the record of the next chunk, and whether this tile ends here
            __syncthreads();
            if (w == 0 && c + 1 < c1) reinterpret_cast<int *>(&recs[buf ^ 1])[lane] = pre;
            __syncthreads();
            const bool tile_end = c + 1 == c1 || recs[buf ^ 1].tile != rec.tile;
            if (tile_end) {
#pragma unroll
                for (int ii = 0; ii < NIT; ++ii) {
                    const int item = w + NW * ii, g = item / MT, mb = item % MT;
                    const int r2 = mb * 16 + li;
                    if (item < 4 * MT && r2 < R) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int m2 = 4 * kq + v;
                            Cs[g * CUNIT + m2 * CSTR + r2] = dacc[ii][v];
                            if (m2 < D12) dT[((m2 % d2) * R + r2) * DTST + g * 4 + m2 / d2] = dacc[ii][v];
                        }
                    }
                }
                __syncthreads();
                // ---- (3) G1 partial of each unit: sum_col dC[(g,j1)][col] G2[r1][col]
                {
                    const int mb = w % MT, ks = w / MT;
                    const int g = li >> 2, j1 = li & 3;
                    const bool oka = kq < d2 && j1 < d1;
                    const float *acol = dT + kq * R * DTST + li; // dT[(kq*R + s)][(g, j1) = li]
                    const int r1 = mb * 16 + li;
                    const bool okr = r1 < R;
                    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
                    // lanes of the two k-quarters sharing a half-wave walk their
                    // columns 16 apart, so dT and G2s reads land in distinct banks
                    const int rot = SPL >= 32 ? 16 * (kq & 1) : 0;
#pragma unroll 8
                    for (int sl = 0; sl < SPL; ++sl) {
                        const int s = ks * SPL + ((sl + rot) & (SPL - 1));
                        const int col = kq * R + s;
                        const float av = oka ? acol[s * DTST] : 0.f;
                        const float bv = okr ? G2s[r1 * NCOL + (col ^ (r1 & 31))] : 0.f;
                        acc = mfma4(av, bv, acc);
                    }
                    if constexpr (KS > 1) {
                        float *red = Sg; // staged rows are no longer needed
#pragma unroll
                        for (int v = 0; v < 4; ++v) red[(w * 64 + lane) * 4 + v] = acc[v];
                        __syncthreads();
                        if (ks == 0) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                float sum = 0.f;
#pragma unroll
                                for (int kk = 0; kk < KS; ++kk) sum += red[((mb + kk * MT) * 64 + lane) * 4 + v];
                                acc[v] = sum;
                            }
                        }
                    }
                    if (ks == 0 && okr && kq < nu) {
                        // partials are indexed by the unit's position in the work order
                        float *dst = ws.G1P + (int64_t)(rec.ubeg + kq) * a.g1stride + r1;
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (v < d1) dst[v * R] = acc[v];
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
                            ga[mt][s] = r1 < R ? G1s[(kq * 4 + s) * G1ST + r1] : 0.f;
                        }
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int ntg = w + NW * j;
                        if (ntg < NT) {
                            const int col = ntg * 16 + li, j2 = col / R, r2 = col % R;
                            float bv[4];
#pragma unroll
                            for (int s = 0; s < 4; ++s)
                                bv[s] = (j2 < d2 && s < d1) ? Cs[kq * CUNIT + (s * d2 + j2) * CSTR + r2] : 0.f;
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                                for (int s = 0; s < 4; ++s) g2acc[mt][j] = mfma4(ga[mt][s], bv[s], g2acc[mt][j]);
                        }
                    }
                }
                __syncthreads(); // before the next tile reuses G1s / Cs / dT
            }
            buf ^= 1;
        }
        float *dst = a.grads.g[t][1] + (int64_t)i2 * R * d2 * R;
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
    if (c < 4) ws.ctrl[CTRL_BWD_NEXT + c] = 0;
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

hipError_t launch_backward(const Plan &p, const float *grad_out, const CorePtrs &cores,
                           const int64_t *offsets, const GradPtrs &grads, hipStream_t s)
{
    BwdArgs a{p.dtab, p.T, p.B, p.ws, cores, grads, grad_out, offsets, p.nnz, p.sumD, p.Dmax, p.force_generic,
              p.g1stride};
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
    if (p.nnz > 0) {
        if (!p.force_generic) {
            hipLaunchKernelGGL(k_bwd_prep, dim3(1), dim3(64), 0, s, a);
            hipLaunchKernelGGL(k_bwd_g3t, dim3(64, T), dim3(kThreads), 0, s, a);
            if (p.cls_mask & 1)
                hipLaunchKernelGGL(k_bwd_class<8>, dim3(p.num_blocks * BwdLds<8>::OCC), dim3(BwdLds<8>::NW * 64), 0, s, a);
            if (p.cls_mask & 2)
                hipLaunchKernelGGL(k_bwd_class<16>, dim3(p.num_blocks * BwdLds<16>::OCC), dim3(BwdLds<16>::NW * 64), 0,
                                   s, a);
            if (p.cls_mask & 4)
                hipLaunchKernelGGL(k_bwd_class<32>, dim3(p.num_blocks * BwdLds<32>::OCC), dim3(BwdLds<32>::NW * 64), 0,
                                   s, a);
            if (p.cls_mask & 8)
                hipLaunchKernelGGL(k_bwd_class<64>, dim3(p.num_blocks * BwdLds<64>::OCC), dim3(BwdLds<64>::NW * 64), 0,
                                   s, a);
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
    hipLaunchKernelGGL(k_reduce_g3, dim3(sum_n3 > 0 ? (sum_n3 < 65535 ? sum_n3 : 65535) : 1), dim3(kThreads), 0,
                       s, a, k3, o3, sum_n3);
    timer_end(p.timing, TM_BWD_REDUCE, s);
    return hipGetLastError();
}

} // namespace ttemb
