// forward.hip -- fused prefix-shared TT contraction and bag pooling on gfx950.
//
// Follows the FlowTT page ("FlowTT: Exploiting Computation Flow Reuse in
// Irregular Tensor-Train Embedding"): section 3.2 (compute C = A.B once per
// prefix group, keep it on chip, reuse it for every E = C.D, then pool),
// section 3.3 (prefix groups are the execution units) and section 3.4
// (persistent blocks run their assigned range first, then steal chunks; a
// prefix tile split over chunks is checkpointed through L2 so other blocks can
// reuse it).
//
// gfx950 mapping (one 256-thread block = 4 waves):
//  * a tile holds up to four prefix units that share (table, i2).  Their four
//    G1[i1] slices are stacked into the 16 rows of a v_mfma_f32_16x16x4_f32 A
//    operand (row = 4*unit + j1), so the skinny d1 x R1 by R1 x d2R2 products
//    run on the matrix cores at full width.  The G2[i2] slice is the B operand
//    and stays in VGPRs while consecutive tiles share i2 ("B-stationary").
//  * the 4 x 16 x R2 prefix tile is written to LDS; each row group of up to
//    16/d3 unique rows of a unit is one 16x16 output tile of E = C.G3[i3],
//    A read from LDS, B from the G3 slices of those rows.
//  * pooling is a separate bag-major pass over the unique-row buffer: one wave
//    per bag, a fixed summation order and no atomics, so the output is
//    bit-reproducible.
#include "primitives.h"

namespace ttemb {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kCStride = 68;                   // LDS row stride of a prefix tile (R2 <= 64)
constexpr int kCUnit = 16 * kCStride + 16;     // floats per unit (extra 16 rotates banks)
constexpr int kCTile = kUnitsPerTile * kCUnit; // floats per prefix tile
constexpr int kEsFloats = 32 * 68;              // E rows staged per chunk (32 rows of D <= 64)
constexpr int kSchedStatic = 1, kSchedSteal = 2, kSchedStealL2 = 3;

struct FwdArgs {
    const TableDesc *tab;
    int T;
    Ws ws;
    CorePtrs cores;
    int sched;
};

// Victim order for stealing: own range, then blocks on the same XCD (blocks
// are dispatched round-robin over the 8 XCDs), then the other XCDs.
__device__ __forceinline__ int victim_of(int me, int vi, int nb)
{
    const int per = nb >> 3;
    const int xo = vi / per, k = vi - xo * per;
    return ((me & 7) + xo) % 8 + 8 * (((me >> 3) + k) % per);
}

__device__ __forceinline__ int range_begin(int v, int64_t C, int nb) { return (int)((int64_t)v * C / nb); }

// Chunks are class-major (rank class 0..3, generic tables last).  Find the
// first chunk of every class and give each class its own static ranges.
// Queue heads sit on their own 128-byte lines (atomics on a shared line
// serialise in L2).
constexpr int kHeadPad = 32;

// Blocks per CU of each rank class's persistent kernel (register-limited).
constexpr int kClsOcc[4] = {4, 4, 3, 2};
struct ClassGrid {
    int nb[4];
};

__global__ __launch_bounds__(kThreads) void k_queue_init(Ws ws, ClassGrid g, int stride)
{
    __shared__ int cstart[6];
    const int64_t C = ws.ctrl[CTRL_CHUNKS];
    int split = ws.ctrl[CTRL_SPLIT];
    if (split > kMaxCkptSlots) split = kMaxCkptSlots;
    if (threadIdx.x <= 5) {
        const int c = threadIdx.x; // first chunk whose class rank is >= c
        int lo = 0, hi = (int)C;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const int cls = ws.crec[mid].cls;
            const int rank = cls < 0 ? 4 : cls;
            if (rank < c) lo = mid + 1;
            else hi = mid;
        }
        cstart[c] = c == 5 ? (int)C : lo;
    }
    __syncthreads();
    for (int c = 0; c < 4; ++c)
        for (int b = threadIdx.x; b < g.nb[c]; b += blockDim.x)
            ws.heads[(c * stride + b) * kHeadPad] = cstart[c] + range_begin(b, cstart[c + 1] - cstart[c], g.nb[c]);
    for (int i = threadIdx.x; i < split; i += blockDim.x) ws.flags[i] = 0;
    if (threadIdx.x < 5) ws.ctrl[CTRL_CLS_START + threadIdx.x] = cstart[threadIdx.x];
    if (threadIdx.x == 0) {
        ws.ctrl[CTRL_STEALS] = 0;
        ws.ctrl[CTRL_CKPT_HIT] = 0;
        ws.ctrl[CTRL_CKPT_MISS] = 0;
    }
}

// Transposed copy G3t[i3][j3][r2] = G3[i3][r2][j3] of every MFMA-class table,
// so a lane's run of r2 values is contiguous (float4 loads).
__global__ __launch_bounds__(kThreads) void k_g3t(FwdArgs a)
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

// Claiming work (wave 0 of a block).  claim_start() issues the atomic on the
// current victim's head; claim_finish() checks it and, when that victim is
// drained, probes the next 64 victims in parallel and retries.  Every chunk is
// handed out exactly once (heads only grow) and the loop ends once every
// victim has been seen drained.
__device__ __forceinline__ int claim_start(int32_t *heads, int me, int vi, int nb, int nvict)
{
    int raw = 0x7fffffff;
    if (vi < nvict && (threadIdx.x & 63) == 0) raw = atomicAdd(&heads[victim_of(me, vi, nb) * kHeadPad], 1);
    return raw;
}

// heads / chunk ids are offset by `base`, the class's first chunk; C = its count
__device__ int claim_finish(int32_t *heads, int base, int me, int &vi, int nb, int nvict, int64_t C, int raw,
                            int &steals)
{
    const int lane = threadIdx.x & 63;
    for (;;) {
        if (vi >= nvict) return -1;
        const int v = victim_of(me, vi, nb);
        int got = -1;
        if (lane == 0 && raw < base + range_begin(v + 1, C, nb)) got = raw;
        got = __shfl(got, 0, 64);
        if (got >= 0) {
            steals += vi != 0;
            return got;
        }
        const int cand = vi + 1 + lane;
        bool avail = false;
        if (cand < nvict) {
            const int vv = victim_of(me, cand, nb);
            avail = __hip_atomic_load(&heads[vv * kHeadPad], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                    base + range_begin(vv + 1, C, nb);
        }
        const uint64_t m = __ballot(avail);
        vi = m ? vi + 1 + (__ffsll((unsigned long long)m) - 1) : vi + 65;
        raw = claim_start(heads, me, vi, nb, nvict);
    }
}

// One chunk of a tile on the matrix cores, R1 = R2 = R.
// A operand of the next chunk's prefix tile (its G1 slices), issued before the
// current chunk's E stores: on gfx9 loads and stores share one in-order
// counter, so a load issued after the stores would also wait for them.
__device__ __forceinline__ void prefetch_a(const FwdArgs &a, const ChunkRec &nr, float (&apf)[16], int &apf_tile)
{
    apf_tile = -1;
    // record fields are wave-uniform: scalar loads of the table data then stay
    // off the vector memory counter
    const int cls = __builtin_amdgcn_readfirstlane(nr.cls), t = __builtin_amdgcn_readfirstlane(nr.t);
    if (cls < 0) return;
    const int R = 8 << cls, KQ = R >> 2;
    const TableDesc &tb = a.tab[t];
    const int d1 = tb.d1;
    const int lane = threadIdx.x & 63, li = lane & 15, kq = lane >> 4;
    const int g = li >> 2, j1 = li & 3;
    // out-of-range lanes read the first unit's slice (always valid) and are
    // zeroed when used: zeroing a register a load may still target would make
    // the wave wait for all of its outstanding stores
    const bool ok = g < nr.nu && j1 < d1;
    const float *src = a.cores.g[t][0] + ((int64_t)(ok ? nr.i1[g] : nr.i1[0]) * d1 + (ok ? j1 : 0)) * R + kq * KQ;
    if (KQ >= 4) {
#pragma unroll
        for (int s = 0; s < 16; s += 4) {
            const floatx4 v = *reinterpret_cast<const floatx4 *>(src + (s < KQ ? s : 0));
            apf[s] = v[0];
            apf[s + 1] = v[1];
            apf[s + 2] = v[2];
            apf[s + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) apf[s] = src[s < KQ ? s : 0];
    }
    apf_tile = nr.tile;
}

template <int R, class Mid>
__device__ __forceinline__ void chunk_mfma(const FwdArgs &a, const ChunkRec &rec, float *Cs, float *Es,
                                           float (&breg)[64], int &bkey, int &lds_tile, int *s_flag,
                                           float (&apf)[16], int &apf_tile, ChunkRec *rnext, bool has_next,
                                           int pre, int &hits, int &misses, int c, int cn, Mid &&mid)
{
    constexpr int KQ = R / 4;           // K values each lane feeds per output tile
    constexpr int NT = R / 4;           // 16-column tiles of the padded d2*R2 (d2 <= 4)
    constexpr int NTW = (NT + 3) / 4;   // per wave
    // wave-uniform table index: the table data below become scalar loads,
    // which do not wait behind this wave's outstanding vector loads and stores
    const int t = __builtin_amdgcn_readfirstlane(rec.t);
    const TableDesc &tb = a.tab[t];
    const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, D12 = d1 * d2, Dp = tb.Dp;
    float *Et = a.ws.E + a.ws.ebase[t];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, kq = lane >> 4;
    const float *G1 = a.cores.g[t][0];
    const float *G2 = a.cores.g[t][1];
    const float *G3t = a.ws.g3t + tb.g3t_off;
    const int P = 16 / d3;
    const int np = rec.pstart[rec.nu];
    const int slot = li / d3, j3 = li - slot * d3;

    // output tile e -> unit j, first row (chunk numbering) and row count
    auto piece = [&](int e, int &j, int &rb, int &cnt) {
        j = 0;
        while (j < 3 && e >= rec.pstart[j + 1]) ++j;
        rb = rec.rowoff[j] + (e - rec.pstart[j]) * P;
        const int rem = rec.rowoff[j] + rec.ccnt[j] - rb;
        cnt = rem < P ? rem : P;
    };
    // B operand of an output tile: G3t[i3][j3][kq*KQ .. kq*KQ+KQ-1] of the lane's row
    auto load_b = [&](int e, float (&b)[KQ]) {
        int j, rb, cnt;
        piece(e, j, rb, cnt);
        // lanes past the tile's rows read the tile's first row; their outputs
        // are never stored (no zeroing: see prefetch_a)
        const bool ok = slot < cnt;
        const float *src = G3t + ((int64_t)rec.i3[rb + (ok ? slot : 0)] * d3 + j3) * R + kq * KQ;
        if constexpr (KQ % 4 == 0) {
#pragma unroll
            for (int s = 0; s < KQ; s += 4) {
                const floatx4 v = *reinterpret_cast<const floatx4 *>(src + s);
                b[s] = v[0];
                b[s + 1] = v[1];
                b[s + 2] = v[2];
                b[s + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int s = 0; s < KQ; ++s) b[s] = src[s];
        }
    };
    float bnext[KQ];
    if (w < np) load_b(w, bnext); // in flight while the prefix tile is computed

    // -------- prefix tile C_u = G1[i1_u] . G2[i2] for the (<= 4) units
    if (lds_tile != rec.tile) {
        bool have = false;
        const bool split = rec.slot >= 0 && a.sched == kSchedStealL2;
        if (split && rec.rbeg > 0) {
            if (threadIdx.x == 0)
                *s_flag = __hip_atomic_load(&a.ws.flags[rec.slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (*s_flag) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const float4 *src = reinterpret_cast<const float4 *>(a.ws.ckpt + (size_t)rec.slot * kCTile);
                float4 *dst = reinterpret_cast<float4 *>(Cs);
                for (int i = threadIdx.x; i < kCTile / 4; i += kThreads) dst[i] = src[i];
                have = true;
            }
            if (have) ++hits;
            else ++misses;
        }
        if (!have) {
            const int g = li >> 2, j1 = li & 3;
            const bool oka = g < rec.nu && j1 < d1;
            const float *srcA = G1 + ((int64_t)(oka ? rec.i1[g] : rec.i1[0]) * d1 + (oka ? j1 : 0)) * R + kq * KQ;
            float areg[KQ];
            if (apf_tile == rec.tile) {
#pragma unroll
                for (int s = 0; s < KQ; ++s) areg[s] = apf[s];
            } else if constexpr (KQ % 4 == 0) {
#pragma unroll
                for (int s = 0; s < KQ; s += 4) {
                    const floatx4 v = *reinterpret_cast<const floatx4 *>(srcA + s);
                    areg[s] = v[0];
                    areg[s + 1] = v[1];
                    areg[s + 2] = v[2];
                    areg[s + 3] = v[3];
                }
            } else {
#pragma unroll
                for (int s = 0; s < KQ; ++s) areg[s] = srcA[s];
            }
            // rows of absent units / j1 contribute zeros to C (their C rows are never read)
#pragma unroll
            for (int s = 0; s < KQ; ++s) areg[s] = oka ? areg[s] : 0.f;
            const int key = (int)(tb.i2_base + (uint32_t)rec.i2);
            if (bkey != key) {
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int ntg = w + 4 * j;
                    const int col = ntg * 16 + li;
                    const int j2 = col / R, r2 = col % R;
                    const bool ok = ntg < NT && j2 < d2;
                    const float *src = G2 + ((int64_t)rec.i2 * R * d2 + (ok ? j2 : 0)) * R + r2;
#pragma unroll
                    for (int s = 0; s < KQ; ++s) {
                        const int k = kq * KQ + s;
                        breg[j * KQ + s] = ok ? src[(int64_t)k * d2 * R] : 0.f;
                    }
                }
                bkey = key;
            }
            floatx4 acc[NTW];
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KQ; ++s) {
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    if (NT % 4 == 0 || w + 4 * j < NT) // folded when every wave has NTW tiles
                        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(areg[s], breg[j * KQ + s], acc[j], 0, 0, 0);
            }
            // lane (kq, li) holds rows 4*kq + v = (unit kq, j1 = v), column ntg*16 + li
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int ntg = w + 4 * j;
                if (NT % 4 == 0 || ntg < NT) {
                    const int col = ntg * 16 + li;
                    const int j2 = col / R, r2 = col % R;
                    if (j2 < d2 && kq < rec.nu) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (v < d1) Cs[kq * kCUnit + (v * d2 + j2) * kCStride + r2] = acc[j][v];
                    }
                }
            }
            __syncthreads();
            // publish only when another block may run a later chunk of this tile:
            // this block already holds the next claimed chunk, so a two-chunk
            // tile whose second chunk is that one never needs the checkpoint
            // (an agent-scope release writes back L2, which is not free)
            if (split && rec.rbeg == 0 && (rec.nch > 2 || cn != c + 1)) {
                float4 *dst = reinterpret_cast<float4 *>(a.ws.ckpt + (size_t)rec.slot * kCTile);
                const float4 *src = reinterpret_cast<const float4 *>(Cs);
                for (int i = threadIdx.x; i < kCTile / 4; i += kThreads) dst[i] = src[i];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __syncthreads();
                if (threadIdx.x == 0)
                    __hip_atomic_store(&a.ws.flags[rec.slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        lds_tile = rec.tile;
    }
    __syncthreads();
    // the next chunk's record (its load was issued when this chunk started)
    if (has_next && w == 0) reinterpret_cast<int *>(rnext)[lane] = pre;
    __syncthreads();
    if (has_next && rnext->tile != rec.tile) prefetch_a(a, *rnext, apf, apf_tile);

    // -------- unique rows E_u = C_unit . G3[i3_u], 16/d3 rows per output tile,
    // staged in LDS (Es, row stride Dp + 4) and stored coalesced once every
    // load of the chunk has been waited for
    mid();
    const int EST = Dp + 4;
    const bool staged = rec.rowoff[4] * EST <= kEsFloats; // else rows go straight to E
    const bool okm = li < D12;
    for (int e = w; e < np; e += 4) {
        float bcur[KQ];
#pragma unroll
        for (int s = 0; s < KQ; ++s) bcur[s] = bnext[s];
        if (e + 4 < np) load_b(e + 4, bnext);
        int j, rb, cnt;
        piece(e, j, rb, cnt);
        const float *ca = Cs + j * kCUnit + (okm ? li : 0) * kCStride + kq * KQ;
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        if constexpr (KQ % 4 == 0) {
#pragma unroll
            for (int s = 0; s < KQ; s += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(ca + s);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(okm ? v.x : 0.f, bcur[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(okm ? v.y : 0.f, bcur[s + 1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(okm ? v.z : 0.f, bcur[s + 2], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(okm ? v.w : 0.f, bcur[s + 3], acc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < KQ; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(okm ? ca[s] : 0.f, bcur[s], acc, 0, 0, 0);
        }
        if (slot < cnt) {
            float *Erow = staged ? Es + (rb + slot) * EST
                                 : Et + (int64_t)(rec.ustart[j] + (rb - rec.rowoff[j]) + slot) * Dp;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m2 = kq * 4 + v;
                if (m2 < D12) Erow[m2 * d3 + j3] = acc[v];
            }
        }
    }
    if (staged) {
        __syncthreads();
        const int nrows = rec.rowoff[4], c4 = Dp >> 2;
        for (int e = threadIdx.x; e < nrows * c4; e += kThreads) {
            const int q = e / c4, r4 = e - q * c4;
            const int j = (q >= rec.rowoff[1]) + (q >= rec.rowoff[2]) + (q >= rec.rowoff[3]);
            const int u = rec.ustart[j] + (q - rec.rowoff[j]);
            reinterpret_cast<floatx4 *>(Et + (int64_t)u * Dp)[r4] = *reinterpret_cast<const floatx4 *>(Es + q * EST + 4 * r4);
        }
    }
}

template <int R>
__global__ __launch_bounds__(kThreads, 2) void k_contract(FwdArgs a, int heads_stride)
{
    constexpr int CLS = R == 8 ? 0 : R == 16 ? 1 : R == 32 ? 2 : 3;
    __shared__ __attribute__((aligned(16))) float Cs[kCTile];
    __shared__ __attribute__((aligned(16))) float Es[kEsFloats];
    __shared__ ChunkRec rbuf[2];
    __shared__ int s_cur, s_next, s_next2, s_flag;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nb = gridDim.x, me = blockIdx.x;
    const Ws &ws = a.ws;
    const int base = ws.ctrl[CTRL_CLS_START + CLS];
    const int64_t C = ws.ctrl[CTRL_CLS_START + CLS + 1] - base;
    int32_t *heads = ws.heads + CLS * heads_stride * kHeadPad;
    const int nvict = a.sched == kSchedStatic ? 1 : nb;
    float breg[64], apf[16];
#pragma unroll
    for (int i = 0; i < 64; ++i) breg[i] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) apf[i] = 0.f;
    int bkey = -1, lds_tile = -1, vi = 0, apf_tile = -1, steals = 0, hits = 0, misses = 0;
    if (w == 0) {
        const int c0 = claim_finish(heads, base, me, vi, nb, nvict, C, claim_start(heads, me, vi, nb, nvict), steals);
        const int c1 = c0 < 0 ? -1
                              : claim_finish(heads, base, me, vi, nb, nvict, C, claim_start(heads, me, vi, nb, nvict), steals);
        if (c0 >= 0) reinterpret_cast<int *>(&rbuf[0])[lane] = reinterpret_cast<const int *>(&ws.crec[c0])[lane];
        if (lane == 0) {
            s_cur = c0;
            s_next = c1;
        }
    }
    __syncthreads();
    int buf = 0;
    for (;;) {
        const int c = s_cur, cn = s_next;
        if (c < 0) break;
        int pre = 0, raw = 0x7fffffff;
        if (w == 0 && cn >= 0) {
            pre = reinterpret_cast<const int *>(&ws.crec[cn])[lane];
            raw = claim_start(heads, me, vi, nb, nvict);
        }
        // the claim of chunk c+2 completes before this chunk's stores are issued
        // (a wait on the atomic issued after them would also wait for them)
        auto mid = [&]() {
            if (w == 0) {
                const int c2 = cn < 0 ? -1 : claim_finish(heads, base, me, vi, nb, nvict, C, raw, steals);
                if (lane == 0) s_next2 = c2;
            }
        };
        chunk_mfma<R>(a, rbuf[buf], Cs, Es, breg, bkey, lds_tile, &s_flag, apf, apf_tile, &rbuf[buf ^ 1], cn >= 0,
                      pre, hits, misses, c, cn, mid);
        __syncthreads(); // everyone is done with rbuf[buf], s_cur and s_next
        if (threadIdx.x == 0) {
            s_cur = cn;
            s_next = s_next2;
        }
        __syncthreads();
        buf ^= 1;
    }
    // scheduling statistics, one atomic per block
    if (threadIdx.x == 0) {
        if (steals) atomicAdd(&ws.ctrl[CTRL_STEALS], steals);
        if (hits) atomicAdd(&ws.ctrl[CTRL_CKPT_HIT], hits);
        if (misses) atomicAdd(&ws.ctrl[CTRL_CKPT_MISS], misses);
    }
}

// Plain fp32 contraction for any shape within the create-time limits: one
// block per unit, the prefix intermediate in LDS, then every unique row.
__global__ __launch_bounds__(kThreads) void k_contract_generic(FwdArgs a, int force)
{
    __shared__ float Cg[4096];
    const Ws &ws = a.ws;
    const int64_t Un = ws.ctrl[CTRL_UNITS];
    for (int64_t unit = blockIdx.x; unit < Un; unit += gridDim.x) {
        const int t = segment_of(ws.tab_unit_start, a.T, unit);
        const TableDesc &tb = a.tab[t];
        if (!force && tb.cls >= 0) continue;
        const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, R1 = tb.R1, R2 = tb.R2, D = tb.D;
        const int q = ws.unit_prefix[unit];
        const int i1 = q / tb.n2, i2 = q % tb.n2;
        const float *G1 = a.cores.g[t][0] + (int64_t)i1 * d1 * R1;
        const float *G2 = a.cores.g[t][1] + (int64_t)i2 * R1 * d2 * R2;
        const float *G3 = a.cores.g[t][2];
        for (int e = threadIdx.x; e < d1 * d2 * R2; e += kThreads) {
            const int m2 = e / R2, r2 = e - m2 * R2, j1 = m2 / d2, j2 = m2 - j1 * d2;
            float acc = 0.f;
            for (int r1 = 0; r1 < R1; ++r1) acc = fmaf(G1[j1 * R1 + r1], G2[((int64_t)r1 * d2 + j2) * R2 + r2], acc);
            Cg[e] = acc;
        }
        __syncthreads();
        const int us = ws.unit_start[unit], ue = ws.unit_start[unit + 1];
        float *Et = ws.E + ws.ebase[t];
        for (int64_t e = threadIdx.x; e < (int64_t)(ue - us) * D; e += kThreads) {
            const int r = (int)(e / D), col = (int)(e - (int64_t)r * D);
            const int u = us + r;
            const int i3 = ws.uniq_row[u] % tb.n3;
            const int m2 = col / d3, j3 = col - m2 * d3;
            const float *g3 = G3 + (int64_t)i3 * R2 * d3 + j3;
            float acc = 0.f;
            for (int r2 = 0; r2 < R2; ++r2) acc = fmaf(Cg[m2 * R2 + r2], g3[r2 * d3], acc);
            Et[(int64_t)u * tb.Dp + col] = acc;
        }
        __syncthreads();
    }
}

// Bag-major sum pooling: one wave per bag; lanes split the columns in float4
// and the lookups in 64/lanes-per-row interleaved streams, combined in a fixed
// xor-tree order.  Empty bags write zeros.
__global__ __launch_bounds__(kThreads) void k_pool(const TableDesc *tab, int T, int64_t B,
                                                   const int64_t *offsets, int64_t nnz, Ws ws,
                                                   float *out, int SD)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t bag = (int64_t)blockIdx.x * (kThreads / 64) + w;
    if (bag >= (int64_t)T * B) return;
    const int t = (int)(bag / B);
    const int64_t b = bag - (int64_t)t * B;
    const TableDesc &tb = tab[t];
    int64_t lo = offsets[bag], hi = offsets[bag + 1];
    lo = lo < 0 ? 0 : (lo > nnz ? nnz : lo);
    hi = hi < lo ? lo : (hi > nnz ? nnz : hi);
    const int u0 = ws.tab_uniq_start[t], u1 = ws.tab_uniq_start[t + 1];
    if (u1 <= u0) hi = lo;
    const float *Et = ws.E + ws.ebase[t];
    float *o = out + b * SD + tb.col_off;
    const int D = tb.D;
    if (D <= 256) {
        // lanes per row: smallest power of two >= D/4 (float4 columns)
        const int c4n = (D + 3) >> 2;
        int lpr = 1;
        while (lpr < c4n) lpr <<= 1;
        const int rf = 64 / lpr;
        const int c4 = lane & (lpr - 1), r = lane / lpr;
        const int cc = c4 < c4n ? c4 : 0;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        // 64 lookups at a time: one coalesced load of their unique rows, then
        // the E rows in flight together (rf rows per instruction, 4 deep)
        for (int64_t l0 = lo; l0 < hi; l0 += 64) {
            const int n = hi - l0 < 64 ? (int)(hi - l0) : 64;
            int uu = ws.inv[l0 + (lane < n ? lane : 0)];
            uu = uu < u0 ? u0 : (uu >= u1 ? u1 - 1 : uu);
            const int nk = (n + rf - 1) / rf; // row steps, uniform over the wave
            for (int k0 = 0; k0 < nk; k0 += 4) {
                float4 v[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int i = r + (k0 + kk) * rf;
                    const int u = __shfl(uu, i < n ? i : 0, 64);
                    v[kk] = *reinterpret_cast<const float4 *>(Et + (int64_t)u * tb.Dp + 4 * cc);
                    if (!(i < n && k0 + kk < nk && c4 < c4n)) v[kk] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    acc.x += v[kk].x;
                    acc.y += v[kk].y;
                    acc.z += v[kk].z;
                    acc.w += v[kk].w;
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
            if (j + 0 < D) o[j + 0] = acc.x;
            if (j + 1 < D) o[j + 1] = acc.y;
            if (j + 2 < D) o[j + 2] = acc.z;
            if (j + 3 < D) o[j + 3] = acc.w;
        }
    } else {
        for (int j = lane; j < D; j += 64) {
            float acc = 0.f;
            for (int64_t l = lo; l < hi; ++l) {
                int u = ws.inv[l];
                u = u < u0 ? u0 : (u >= u1 ? u1 - 1 : u);
                acc += Et[(int64_t)u * tb.Dp + j];
            }
            o[j] = acc;
        }
    }
}

hipError_t launch_forward(const Plan &p, const CorePtrs &cores, const int64_t *offsets, float *out,
                          hipStream_t s)
{
    FwdArgs a{p.dtab, p.T, p.ws, cores, p.sched_mode};
    timer_begin(p.timing, TM_CONTRACT, s);
    if (p.nnz > 0) {
        ClassGrid cg;
        for (int c = 0; c < 4; ++c) cg.nb[c] = p.num_blocks * kClsOcc[c];
        const int hs = p.num_blocks * 4;
        hipLaunchKernelGGL(k_queue_init, dim3(1), dim3(kThreads), 0, s, p.ws, cg, hs);
        if (!p.force_generic) {
            hipLaunchKernelGGL(k_g3t, dim3(64, p.T), dim3(kThreads), 0, s, a);
            for (int c = 0; c < 4; ++c) {
                if (!(p.cls_mask & (1 << c))) continue;
                timer_begin(p.timing, TM_FWD_CLS0 + c, s);
                switch (c) {
                case 0: hipLaunchKernelGGL(k_contract<8>, dim3(cg.nb[0]), dim3(kThreads), 0, s, a, hs); break;
                case 1: hipLaunchKernelGGL(k_contract<16>, dim3(cg.nb[1]), dim3(kThreads), 0, s, a, hs); break;
                case 2: hipLaunchKernelGGL(k_contract<32>, dim3(cg.nb[2]), dim3(kThreads), 0, s, a, hs); break;
                default: hipLaunchKernelGGL(k_contract<64>, dim3(cg.nb[3]), dim3(kThreads), 0, s, a, hs); break;
                }
                timer_end(p.timing, TM_FWD_CLS0 + c, s);
            }
        }
        if (p.force_generic || p.any_generic)
            hipLaunchKernelGGL(k_contract_generic, dim3(p.num_blocks * 4), dim3(kThreads), 0, s, a,
                               p.force_generic ? 1 : 0);
    }
    timer_end(p.timing, TM_CONTRACT, s);
    timer_begin(p.timing, TM_POOL, s);
    const int64_t nbags = (int64_t)p.T * p.B;
    if (nbags > 0) {
        const int64_t g = (nbags + 3) / 4;
        hipLaunchKernelGGL(k_pool, dim3((unsigned)g), dim3(kThreads), 0, s, p.dtab, p.T, p.B, offsets,
                           p.nnz, p.ws, out, p.sumD);
    }
    timer_end(p.timing, TM_POOL, s);
    return hipGetLastError();
}

} // namespace ttemb
