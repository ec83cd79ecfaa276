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
typedef __attribute__((address_space(3))) float lds_float;

constexpr int kCTile = kUnitsPerTile * (16 * 68 + 16); // floats per checkpoint slot (R2 <= 64)

// Per-rank layout of a class kernel: LDS row stride of the prefix tile
// (R + 4), floats per unit (an extra 16 rotates banks between units), E rows
// staged per chunk, and blocks per CU (measured: six rank-16 blocks per CU
// ran slower than four, the chunk loop being bound by instruction issue).
template <int R>
struct FwdCfg {
    static constexpr int CSTR = R + 4;
    static constexpr int CUNIT = 16 * CSTR + 16;
    static constexpr int CTILE = kUnitsPerTile * CUNIT;
    static constexpr int ES = R <= 16 ? 32 * 68 : 32 * 132; // 32 rows of D <= 64, or <= 128
    static constexpr int OCC = R <= 16 ? 5 : R == 32 ? 4 : 2;
    static constexpr int BREG = ((R / 4 + 3) / 4) * (R / 4); // G2 slice registers per lane
};
static_assert(FwdCfg<64>::CTILE == kCTile, "checkpoint slot holds the largest prefix tile");
constexpr int kMaxClsOcc = 8; // queue heads per CU reserved for each class
constexpr int kPoolCap = 64;  // fused pooling: lookups of a row pooled by the contraction itself
constexpr int kSchedStatic = 1, kSchedSteal = 2, kSchedStealL2 = 3;
// Default scheduling per rank class (8, 16, 32, 64), from the scheduling
// ablation on the 26-table batch-32768 forward: static ranges are already
// balanced to within 0.82-0.85 of the span, and a claimed chunk of a rank-16
// or rank-32 tile is short enough that stealing's extra claims and broken
// (table, i2) continuity cost more than the idle tail they remove (rank 16:
// 0.16 ms static, 0.22 ms stealing, 0.42 ms with checkpoints); rank-64 chunks
// are long and stealing pays (1.15 -> 1.04 ms).  Checkpoints were consulted
// by under 1 % of the chunks of split tiles and are left to the explicit mode.
constexpr int kDefaultSched[4] = {kSchedStatic, kSchedStatic, kSchedStatic, kSchedSteal};

struct FwdArgs {
    const TableDesc *tab;
    int T;
    Ws ws;
    CorePtrs cores;
    int sched;
    float *out; // fused pooling only: the pooled output [B][SD]
    int SD;
    int64_t B;
};

__device__ __forceinline__ int range_begin(int v, int64_t C, int nb) { return (int)((int64_t)v * C / nb); }

// Chunks are class-major (rank class 0..3, generic tables last).  Find the
// first chunk of every class and give each class its own static ranges.
// Queue heads sit on their own 128-byte lines (atomics on a shared line
// serialise in L2).
constexpr int kHeadPad = 32;

// Blocks per CU of each rank class's persistent kernel (register-limited).
constexpr int kClsOcc[4] = {FwdCfg<8>::OCC, FwdCfg<16>::OCC, FwdCfg<32>::OCC, FwdCfg<64>::OCC};
struct ClassGrid {
    int nb[4];
};

// Queue heads and counters of the persistent kernels (block (0, 0)), and the
// transposed G3 copies (all blocks, when g3t != 0): one launch for both.
__device__ void g3t_copy(const FwdArgs &a);
__global__ __launch_bounds__(kThreads) void k_queue_init(FwdArgs a, ClassGrid g, int stride, int g3t)
{
    if (g3t) g3t_copy(a);
    if (blockIdx.x != 0 || blockIdx.y != 0) return;
    const Ws &ws = a.ws;
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
    if (threadIdx.x < 4) ws.bstat[threadIdx.x * kStatBlocks].nb = 0; // forward class records
    if (threadIdx.x == 0) {
        ws.ctrl[CTRL_STEALS] = 0;
        ws.ctrl[CTRL_CKPT_HIT] = 0;
        ws.ctrl[CTRL_CKPT_MISS] = 0;
    }
}

// Transposed copy G3t[i3][j3][r2] = G3[i3][r2][j3] of every MFMA-class table
// (table blockIdx.y), so a lane's run of r2 values is contiguous (float4 loads).
__device__ void g3t_copy(const FwdArgs &a)
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
    int res;
    for (;;) {
        const bool live = vi < nvict;
        const int v = victim_of(me, live ? vi : 0, nb);
        int got = -1;
        if ((lane == 0) & live & (raw < base + range_begin(v + 1, C, nb))) got = raw;
        got = uni(got); // lane 0's value (every lane of the wave is active here)
        if (got >= 0) {
            steals += vi != 0;
            res = got;
            break;
        }
        if (!live) {
            res = -1;
            break;
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
        if (vi >= nvict) {
            res = -1;
            break;
        }
        // a retry (a drained victim, rare) waits for its claim right here, so
        // no claim is ever left in flight past this function: a register that
        // a load may still target makes later writes to it wait for every
        // load and store the wave has in flight
        raw = uni(claim_start(heads, me, vi, nb, nvict));
    }
    return res;
}

// Output tile e of a chunk (16/d3 rows of one unit, P rows per tile) -> unit
// j, first row in chunk numbering and row count.
__device__ __forceinline__ void chunk_piece(const ChunkRec &r, int P, int e, int &j, int &rb, int &cnt)
{
    j = 0;
    while (j < 3 && e >= r.pstart[j + 1]) ++j;
    rb = r.rowoff[j] + (e - r.pstart[j]) * P;
    const int rem = r.rowoff[j] + r.ccnt[j] - rb;
    cnt = rem < P ? rem : P;
}

// Pieces of a chunk whose B operands a wave keeps in registers from one chunk
// to the next: they are loaded while the previous chunk finishes.
// (one fewer at rank 64 when the prefix intermediates are kept: its C stores
// need the registers)
template <int R, bool KEEP> constexpr int fwd_nq() { return R <= 32 ? 3 : KEEP ? 1 : 2; }

// B operand of output tile e of chunk r: G3t[i3][j3][kq*KQ .. kq*KQ+KQ-1] of
// the lane's row.  Lanes past the tile's rows read its first row; their
// outputs are never stored (and never zeroed: see load_a).
template <int R>
__device__ __forceinline__ void load_b_piece(const FwdArgs &a, const ChunkRec &r, int e, float (&b)[R / 4])
{
    constexpr int KQ = R / 4;
    const int t = __builtin_amdgcn_readfirstlane(r.t);
    const auto &tb = kconst(a.tab)[t];
    const int d3 = tb.d3;
    const int lane = threadIdx.x & 63, li = lane & 15, kq = lane >> 4;
    const int slot = li / d3, j3 = li - slot * d3;
    int j, rb, cnt;
    chunk_piece(r, 16 / d3, e, j, rb, cnt);
    const bool ok = slot < cnt;
    const float *src = a.ws.g3t + tb.g3t_off + ((int64_t)r.i3[rb + (ok ? slot : 0)] * d3 + j3) * R + kq * KQ;
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
}

// A operand of a chunk's prefix tile: the G1[i1] slices of its units, lane
// (kq, li) holding row 4*unit + j1 = li, K values kq*KQ .. kq*KQ+KQ-1.  Lanes
// outside the tile read the first unit's slice (always valid) and are masked
// where the operand is used: zeroing a register that a load may still target
// would make the wave wait for every load and store it has in flight.
template <int R>
__device__ __forceinline__ void load_a(const FwdArgs &a, const ChunkRec &r, float (&av)[R / 4])
{
    constexpr int KQ = R / 4;
    const int t = __builtin_amdgcn_readfirstlane(r.t);
    const auto &tb = kconst(a.tab)[t];
    const int d1 = tb.d1;
    const int lane = threadIdx.x & 63, li = lane & 15, kq = lane >> 4;
    const int g = li >> 2, j1 = li & 3;
    const bool ok = g < r.nu && j1 < d1;
    const float *src = a.cores.g[t][0] + ((int64_t)(ok ? r.i1[g] : r.i1[0]) * d1 + (ok ? j1 : 0)) * R + kq * KQ;
    if constexpr (KQ % 4 == 0) {
#pragma unroll
        for (int s = 0; s < KQ; s += 4) {
            const floatx4 v = *reinterpret_cast<const floatx4 *>(src + s);
            av[s] = v[0];
            av[s + 1] = v[1];
            av[s + 2] = v[2];
            av[s + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int s = 0; s < KQ; ++s) av[s] = src[s];
    }
}

// Every operand a chunk loads from memory except its G2 slice: the A operand
// and the B operands of the wave's first NQ output tiles.  Issued while the
// previous chunk finishes, before its E stores.
template <int R, bool KEEP>
__device__ __forceinline__ void load_operands(const FwdArgs &a, const ChunkRec &r, float (&av)[R / 4],
                                              float (&bq)[fwd_nq<R, KEEP>()][R / 4])
{
    load_a<R>(a, r, av);
    const int w = uni(threadIdx.x >> 6);
    const int np = r.pstart[r.nu];
#pragma unroll
    for (int k = 0; k < fwd_nq<R, KEEP>(); ++k) load_b_piece<R>(a, r, w + 4 * k < np ? w + 4 * k : (np > 0 ? np - 1 : 0), bq[k]);
}

// E rows of a chunk staged in LDS are written out with this many float4
// stores per thread, always the same number (the last element is written
// again by the threads past the end, with the same value).  A fixed count of
// stores lets the next chunk wait for its operands, loaded before these
// stores, without waiting for the stores.
constexpr int kFlushPerThread = 4; // 32 rows of D <= 128
// With the prefix intermediates kept for the backward, the tile's first chunk
// also writes its C tile (4 units x 16 rows x R, compact), again with a fixed
// number of float4 stores per thread.
template <int R> constexpr int keep_per_thread() { return (16 * R + kThreads - 1) / kThreads; }
static_assert((kFlushPerThread + keep_per_thread<64>()) * kThreads * 4 <= kSinkFloats,
              "scratch line holds one flush");

// One chunk of a tile on the matrix cores, R1 = R2 = R.  On entry the chunk's
// A operand (apf) and first B operands (bq) are loaded or in flight; on exit
// those of the next chunk are.
template <int R, bool KEEP, bool POOL, class Mid, class End>
__device__ __forceinline__ void chunk_mfma(const FwdArgs &a, const ChunkRec &rec, float *Cs, float *Es,
                                           float (&breg)[FwdCfg<R>::BREG], int &bkey, int &lds_tile, int *s_flag,
                                           float (&apf)[R / 4], float (&bq)[fwd_nq<R, KEEP>()][R / 4], ChunkRec *rnext,
                                           bool has_next, int pre, int &hits, int &misses, int c, int cn,
                                           Mid &&mid, End &&endc)
{
    constexpr int KQ = R / 4;           // K values each lane feeds per output tile
    constexpr int NT = R / 4;           // 16-column tiles of the padded d2*R2 (d2 <= 4)
    constexpr int NTW = (NT + 3) / 4;   // per wave
    constexpr int NQ = fwd_nq<R, KEEP>();     // output tiles per wave with B operands loaded ahead
    using L = FwdCfg<R>;
    // wave-uniform table index: the table data below become scalar loads,
    // which do not wait behind this wave's outstanding vector loads and stores
    const int t = __builtin_amdgcn_readfirstlane(rec.t);
    const auto &tb = kconst(a.tab)[t];
    const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, D12 = d1 * d2, Dp = tb.Dp;
    float *Et = a.ws.E + kconst(a.ws.ebase)[t];
    const int w = uni(threadIdx.x >> 6), lane = threadIdx.x & 63, li = lane & 15, kq = lane >> 4;
    const float *G2 = a.cores.g[t][1];
    const int P = 16 / d3;
    // record fields that steer control flow, made wave-uniform: a branch on a
    // value the compiler takes as per-lane runs both sides under exec masks,
    // and the waits of one side then apply to the other
    const int tile = uni(rec.tile), nu = uni(rec.nu), i2 = uni(rec.i2), cslot = uni(rec.slot);
    const int rbeg = uni(rec.rbeg), nch = uni(rec.nch);
    const int np = uni(rec.pstart[nu]);
    const int slot = li / d3, j3 = li - slot * d3;

    // -------- prefix tile C_u = G1[i1_u] . G2[i2] for the (<= 4) units
    if (uni(lds_tile) != tile) {
        bool have = false;
        const bool split = cslot >= 0 && a.sched == kSchedStealL2;
        if (split && rbeg > 0) {
            if (threadIdx.x == 0)
                *s_flag = __hip_atomic_load(&a.ws.flags[cslot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (uni(*s_flag)) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const float4 *src = reinterpret_cast<const float4 *>(a.ws.ckpt + (size_t)cslot * kCTile);
                float4 *dst = reinterpret_cast<float4 *>(Cs);
                for (int i = threadIdx.x; i < L::CTILE / 4; i += kThreads) dst[i] = src[i];
                have = true;
            }
            if (have) ++hits;
            else ++misses;
        }
        if (!have) {
            auto step1 = [&]() {
                floatx4 acc[NTW];
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KQ; ++s) {
                    // rows of absent units / j1 hold the first unit's slice: C
                    // rows are independent and theirs are never stored
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
                        if (NT % 4 == 0 || w + 4 * j < NT) // folded when every wave has NTW tiles
                            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(apf[s], breg[j * KQ + s], acc[j], 0, 0, 0);
                }
                // lane (kq, li) holds rows 4*kq + v = (unit kq, j1 = v), column ntg*16 + li
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int ntg = w + 4 * j;
                    if (NT % 4 == 0 || ntg < NT) {
                        const int col = ntg * 16 + li;
                        const int j2 = col / R, r2 = col % R;
                        if (j2 < d2 && kq < nu) {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (v < d1) Cs[kq * L::CUNIT + (v * d2 + j2) * L::CSTR + r2] = acc[j][v];
                        }
                    }
                }
            };
            const int key = (int)(tb.i2_base + (uint32_t)i2);
            if (uni(bkey) == key) {
                step1(); // every operand was loaded before the previous chunk's stores
            } else {
                // a new G2 slice: this copy of the tile waits for its loads
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int ntg = w + 4 * j;
                    const int col = ntg * 16 + li;
                    const int j2 = col / R, r2 = col % R;
                    const bool ok = ntg < NT && j2 < d2;
                    const float *src = G2 + ((int64_t)i2 * R * d2 + (ok ? j2 : 0)) * R + r2;
#pragma unroll
                    for (int s = 0; s < KQ; ++s) {
                        const int k = kq * KQ + s;
                        breg[j * KQ + s] = ok ? src[(int64_t)k * d2 * R] : 0.f;
                    }
                }
                bkey = key;
                step1();
            }
            __syncthreads();
            // publish only when another block may run a later chunk of this tile:
            // this block already holds the next claimed chunk, so a two-chunk
            // tile whose second chunk is that one never needs the checkpoint
            // (an agent-scope release writes back L2, which is not free)
            if (split && rbeg == 0 && (nch > 2 || cn != c + 1)) {
                float4 *dst = reinterpret_cast<float4 *>(a.ws.ckpt + (size_t)cslot * kCTile);
                const float4 *src = reinterpret_cast<const float4 *>(Cs);
                for (int i = threadIdx.x; i < L::CTILE / 4; i += kThreads) dst[i] = src[i];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __syncthreads();
                if (threadIdx.x == 0)
                    __hip_atomic_store(&a.ws.flags[cslot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        lds_tile = tile;
    }
    __syncthreads();
    // the next chunk's record (loaded while the previous chunk finished)
    if (has_next && w == 0) reinterpret_cast<int *>(rnext)[lane] = pre;
    __syncthreads();
    mid();

    // -------- unique rows E_u = C_unit . G3[i3_u], 16/d3 rows per output tile,
    // staged in LDS (Es, row stride Dp + 4) and written out at the chunk's end
    const int EST = Dp + 4, nrows = uni(rec.rowoff[4]), c4 = Dp >> 2;
    const bool staged = nrows >= 1 && nrows * EST <= L::ES && nrows * c4 <= kFlushPerThread * kThreads;
    const bool okm = li < D12;
    auto piece_mfma = [&](int e, const float (&bcur)[KQ]) {
        int j, rb, cnt;
        chunk_piece(rec, P, e, j, rb, cnt);
        const float *ca = Cs + j * L::CUNIT + (okm ? li : 0) * L::CSTR + kq * KQ;
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
        // two separate stores (LDS or global): a pointer that may be either
        // would be a flat store, counted by both the LDS and the memory counter
        if (slot < cnt && staged) {
            lds_float *Erow = (lds_float *)(Es + (rb + slot) * EST);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m2 = kq * 4 + v;
                if (m2 < D12) Erow[m2 * d3 + j3] = acc[v];
            }
        } else if (slot < cnt) {
            float *Erow = Et + (int64_t)(rec.ustart[j] + (rb - rec.rowoff[j]) + slot) * Dp;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m2 = kq * 4 + v;
                if (m2 < D12) Erow[m2 * d3 + j3] = acc[v];
            }
        }
    };
#pragma unroll
    for (int k = 0; k < NQ; ++k)
        if (w + 4 * k < np) piece_mfma(w + 4 * k, bq[k]);
    // later tiles (chunks of more than 4*NQ output tiles, d3 >= 8): loaded
    // and used in turn, so no load is left in flight past the loop (a
    // register that may still be a load's target makes any later write to it
    // wait for every outstanding load and store)
    for (int e = w + 4 * NQ; e < np; e += 4) {
        float bcur[KQ];
        load_b_piece<R>(a, rec, e, bcur);
        piece_mfma(e, bcur);
    }

    // -------- end of the chunk: the next chunk's record, claim and operands
    // (the last chunk reloads its own, so every chunk issues the same
    // loads), then this chunk's E rows
    endc();
    load_operands<R, KEEP>(a, has_next ? *rnext : rec, apf, bq);
    if constexpr (POOL) {
        // fused pooling (the pages' pooling inside the contraction): every
        // lookup of each unique row of the chunk adds the row into its bag's
        // output with float atomics; the summation order is not fixed, so the
        // output is not bit-reproducible.  A wave takes rows, lanes columns;
        // the bags of 64 lookups are loaded at once and broadcast.
        __syncthreads(); // rows complete in Es (staged) or in E (written directly)
        const int D = tb.D, col_off = tb.col_off;
        const int r1 = rec.rowoff[1], r2 = rec.rowoff[2], r3 = rec.rowoff[3];
        for (int q = w; q < nrows; q += 4) {
            const int j = (q >= r1) + (q >= r2) + (q >= r3);
            const int u = rec.ustart[j] + (q - rec.rowoff[j]);
            const int s0 = a.ws.uniq_start[u], s1 = a.ws.uniq_start[u + 1];
            // a row's first kPoolCap lookups are pooled here; a hot row (skewed
            // indices) leaves its other lookups to k_pool_tail, which spreads
            // them over the whole grid, and so keeps its row in E
            const int se = s1 - s0 > kPoolCap ? s0 + kPoolCap : s1;
            for (int cb = 0; cb < D; cb += 64) {
                const int c = cb + lane;
                float v = 0.f;
                if (c < D) v = staged ? Es[q * EST + c] : Et[(int64_t)u * Dp + c];
                if (staged && se < s1 && c < D) Et[(int64_t)u * Dp + c] = v;
                for (int sb = s0; sb < se; sb += 64) {
                    const int n = se - sb < 64 ? se - sb : 64;
                    const int bag = lane < n ? a.ws.lk[a.ws.perm[sb + lane]].x : 0;
                    for (int k = 0; k < n; ++k) {
                        const int b = __shfl(bag, k, 64);
                        // (a lookup outside every bag, from malformed offsets, is skipped)
                        if (c < D && (uint64_t)b < (uint64_t)a.B) atomicAdd(a.out + (int64_t)b * a.SD + col_off + c, v);
                    }
                }
            }
        }
        return;
    }
    if (staged) __syncthreads();
    {
        const int tot = nrows * c4;
        const int r1 = rec.rowoff[1], r2 = rec.rowoff[2], r3 = rec.rowoff[3];
#pragma unroll
        for (int k = 0; k < kFlushPerThread; ++k) {
            int e = threadIdx.x + k * kThreads;
            e = e < tot ? e : tot - 1;
            e = e > 0 ? e : 0;
            const int q = e / (c4 > 0 ? c4 : 1), r4 = e - q * c4;
            const int j = (q >= r1) + (q >= r2) + (q >= r3);
            const int u = rec.ustart[j] + (q - rec.rowoff[j]);
            // chunks not staged (wide rows) store into a scratch line instead
            floatx4 *dst = staged ? reinterpret_cast<floatx4 *>(Et + (int64_t)u * Dp) + r4
                                  : reinterpret_cast<floatx4 *>(a.ws.sink) + threadIdx.x + k * kThreads;
            *dst = *reinterpret_cast<const floatx4 *>(Es + (staged ? q * EST + 4 * r4 : 0));
        }
    }
    if constexpr (KEEP) {
        // C_u of the tile's units, [unit position in the work order][16][R]:
        // the tile's first chunk writes them (lanes past the tile's units
        // write element 0 again, with the same value), other chunks write the
        // scratch line (a wave-uniform base, 32-bit offsets per lane)
        const bool first = rbeg == 0;
        floatx4 *base = first ? reinterpret_cast<floatx4 *>(a.ws.Cg + kconst(a.ws.cbase)[t] +
                                                              (int64_t)rec.ubeg * 16 * R)
                              : reinterpret_cast<floatx4 *>(a.ws.sink) + kFlushPerThread * kThreads;
#pragma unroll
        for (int k = 0; k < keep_per_thread<R>(); ++k) {
            const int e = threadIdx.x + k * kThreads; // float4 of the tile, = (j * 16 + m) * R/4 + c4q
            const bool in = e < 16 * R && e / (4 * R) < nu;
            const int ec = in ? e : 0;
            const int j = ec / (4 * R), f = ec - j * (4 * R), m = f / (R / 4), c4q = f - m * (R / 4);
            base[first ? ec : e] = *reinterpret_cast<const floatx4 *>(Cs + j * L::CUNIT + m * L::CSTR + 4 * c4q);
        }
    }
}

template <int R, bool KEEP, bool POOL>
__global__ __launch_bounds__(kThreads, FwdCfg<R>::OCC) void k_contract(FwdArgs a, int heads_stride)
{
    constexpr int CLS = R == 8 ? 0 : R == 16 ? 1 : R == 32 ? 2 : 3;
    __shared__ __attribute__((aligned(16))) float Cs[FwdCfg<R>::CTILE];
    __shared__ __attribute__((aligned(16))) float Es[FwdCfg<R>::ES];
    __shared__ ChunkRec rbuf[2];
    __shared__ int s_cur, s_next, s_next2, s_flag;
    __shared__ long long s_t0;
    if (threadIdx.x == 0) s_t0 = wall_clock64();
    const int lane = threadIdx.x & 63, w = uni(threadIdx.x >> 6); // wave index, in a scalar register
    const int nb = gridDim.x, me = blockIdx.x;
    const Ws &ws = a.ws;
    const int base = ws.ctrl[CTRL_CLS_START + CLS];
    const int64_t C = ws.ctrl[CTRL_CLS_START + CLS + 1] - base;
    int32_t *heads = ws.heads + CLS * heads_stride * kHeadPad;
    // stealing stays on the block's own XCD (victims 0 .. nb/8 - 1 of victim_of):
    // the scan a drained block makes before it exits is an eighth as long
    // (the grid is a whole number of rounds over the 8 XCDs: blocks per CU
    // times a multiple of 8 compute units)
    const int nvict = a.sched == kSchedStatic ? 1 : nb >> 3;
    float breg[FwdCfg<R>::BREG], apf[R / 4], bq[fwd_nq<R, KEEP>()][R / 4];
#pragma unroll
    for (int i = 0; i < FwdCfg<R>::BREG; ++i) breg[i] = 0.f;
    int bkey = -1, lds_tile = -1, vi = 0, steals = 0, hits = 0, misses = 0, nwork = 0, nrows = 0;
    // wave 0 runs the claims two chunks ahead: chunk c+2 is claimed while
    // chunk c runs, and the record of chunk c+1 is loaded at the end of chunk c-1
    int pre = 0, raw = 0x7fffffff, c2w = -1;
    if (w == 0) {
        const int c0 = claim_finish(heads, base, me, vi, nb, nvict, C, claim_start(heads, me, vi, nb, nvict), steals);
        const int c1 = c0 < 0 ? -1
                              : claim_finish(heads, base, me, vi, nb, nvict, C, claim_start(heads, me, vi, nb, nvict), steals);
        if (c0 >= 0) reinterpret_cast<int *>(&rbuf[0])[lane] = reinterpret_cast<const int *>(&ws.crec[c0])[lane];
        if (c1 >= 0) {
            pre = reinterpret_cast<const int *>(&ws.crec[c1])[lane];
            raw = claim_start(heads, me, vi, nb, nvict);
        }
        if (lane == 0) {
            s_cur = c0;
            s_next = c1;
        }
    }
    __syncthreads();
    // the first chunk's operands, then as many stores as every chunk's end
    // issues (the loop is entered only from here, so the compiler's count of
    // loads and stores in flight is the same on every path into it)
    if (uni(s_cur) >= 0) {
        load_operands<R, KEEP>(a, rbuf[0], apf, bq);
        constexpr int NST = kFlushPerThread + (KEEP ? keep_per_thread<R>() : 0);
#pragma unroll
        for (int k = 0; k < NST; ++k)
            reinterpret_cast<floatx4 *>(ws.sink)[threadIdx.x + k * kThreads] = floatx4{0.f, 0.f, 0.f, 0.f};
        int buf = 0;
        for (;;) {
            const int c = uni(s_cur), cn = uni(s_next);
            if (c < 0) break;
            // claim of chunk c+2 (started at the end of chunk c-1)
            auto mid = [&]() {
                if (w == 0) {
                    c2w = cn < 0 ? -1 : claim_finish(heads, base, me, vi, nb, nvict, C, raw, steals);
                    if (lane == 0) s_next2 = c2w;
                }
            };
            // record of chunk c+2 and the claim of chunk c+3
            auto endc = [&]() {
                if (w == 0 && c2w >= 0) {
                    pre = reinterpret_cast<const int *>(&ws.crec[c2w])[lane];
                    raw = claim_start(heads, me, vi, nb, nvict);
                }
            };
            chunk_mfma<R, KEEP, POOL>(a, rbuf[buf], Cs, Es, breg, bkey, lds_tile, &s_flag, apf, bq, &rbuf[buf ^ 1], cn >= 0,
                          pre, hits, misses, c, cn, mid, endc);
            __syncthreads(); // everyone is done with rbuf[buf], s_cur and s_next
            if (threadIdx.x == 0) {
                ++nwork;
                nrows += rbuf[buf].rend - rbuf[buf].rbeg;
                s_cur = cn;
                s_next = s_next2;
            }
            __syncthreads();
            buf ^= 1;
        }
    }
    // scheduling statistics, one atomic per block, and the block's record
    if (threadIdx.x == 0) {
        block_stat_write(ws.bstat + CLS * kStatBlocks, s_t0, nwork, nrows);
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
                                                   float *out, int SD, int skip_mfma)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t bag = (int64_t)blockIdx.x * (kThreads / 64) + w;
    if (bag >= (int64_t)T * B) return;
    const int t = (int)(bag / B);
    const int64_t b = bag - (int64_t)t * B;
    const TableDesc &tb = tab[t];
    if (skip_mfma && tb.cls >= 0) return; // pooled inside the contraction
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

// Fused pooling: the remaining lookups of hot rows (those past a row's first
// kPoolCap), one wave per 64 sorted positions over the whole grid; each such
// lookup adds its row (kept in E) into its bag with float atomics.
__global__ __launch_bounds__(kThreads) void k_pool_tail(FwdArgs a, int64_t nnz)
{
    const Ws &ws = a.ws;
    const int lane = threadIdx.x & 63;
    const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t s0 = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 64; s0 < nnz; s0 += nw * 64) {
        const int64_t sp = s0 + lane;
        int u = 0, bag = 0;
        bool tail = false;
        if (sp < nnz) {
            const int l = ws.perm[sp];
            u = ws.inv[l];
            tail = sp - ws.uniq_start[u] >= kPoolCap;
            bag = ws.lk[l].x;
        }
        uint64_t m = __ballot(tail);
        while (m) {
            const int k = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            const int uk = __shfl(u, k, 64), bk = __shfl(bag, k, 64);
            const int t = segment_of(ws.tab_uniq_start, a.T, uk);
            const auto &tb = kconst(a.tab)[t];
            if (tb.cls < 0 || (uint64_t)bk >= (uint64_t)a.B) continue; // generic tables: pooled by k_pool
            const float *Erow = ws.E + kconst(ws.ebase)[t] + (int64_t)uk * tb.Dp;
            for (int c = lane; c < tb.D; c += 64) atomicAdd(a.out + (int64_t)bk * a.SD + tb.col_off + c, Erow[c]);
        }
    }
}

hipError_t launch_pool(const Plan &p, const int64_t *offsets, float *out, hipStream_t s)
{
    const int64_t nbags = (int64_t)p.T * p.B;
    if (nbags > 0) {
        const int64_t g = (nbags + 3) / 4;
        hipLaunchKernelGGL(k_pool, dim3((unsigned)g), dim3(kThreads), 0, s, p.dtab, p.T, p.B, offsets, p.nnz,
                           p.ws, out, p.sumD, 0);
    }
    return hipGetLastError();
}

hipError_t launch_forward(const Plan &p, const CorePtrs &cores, const int64_t *offsets, float *out,
                          hipStream_t s)
{
    FwdArgs a{p.dtab, p.T, p.ws, cores, p.sched_mode, out, p.sumD, p.B};
    const int64_t nbags = (int64_t)p.T * p.B;
    // fused pooling: out accumulates from zero, and every lookup's bag is
    // looked up once before the contraction
    const bool fused = p.pool_atomic && !p.force_generic;
    timer_begin(p.timing, TM_CONTRACT, s);
    if (fused && nbags > 0) {
        hipError_t e = launch_fill_f32(out, 0.f, p.B * (int64_t)p.sumD, s);
        if (e != hipSuccess) return e;
        if ((e = launch_lookup_meta(p, offsets, s)) != hipSuccess) return e;
    }
    if (p.nnz > 0) {
        ClassGrid cg;
        for (int c = 0; c < 4; ++c) cg.nb[c] = p.num_blocks * kClsOcc[c];
        const int hs = p.num_blocks * kMaxClsOcc;
        if (p.force_generic) hipLaunchKernelGGL(k_queue_init, dim3(1), dim3(kThreads), 0, s, a, cg, hs, 0);
        else hipLaunchKernelGGL(k_queue_init, dim3(64, p.T), dim3(kThreads), 0, s, a, cg, hs, 1);
        if (!p.force_generic) {
            for (int c = 0; c < 4; ++c) {
                if (!(p.cls_mask & (1 << c))) continue;
                timer_begin(p.timing, TM_FWD_CLS0 + c, s);
                const dim3 grid(cg.nb[c]), block(kThreads);
                static_assert(kKeepMinCls == 2, "kept-prefix kernels exist for ranks 32 and 64");
                FwdArgs ac = a;
                ac.sched = p.sched_mode != 0 ? p.sched_mode : kDefaultSched[c];
#define TT_FWD_CLASS(RR, KK, PP) hipLaunchKernelGGL((k_contract<RR, KK, PP>), grid, block, 0, s, ac, hs)
                if (fused) {
                    switch (c) {
                    case 0: TT_FWD_CLASS(8, false, true); break;
                    case 1: TT_FWD_CLASS(16, false, true); break;
                    case 2: TT_FWD_CLASS(32, false, true); break;
                    default: TT_FWD_CLASS(64, false, true); break;
                    }
                } else if (p.keep_c && c >= kKeepMinCls) {
                    if (c == 2) TT_FWD_CLASS(32, true, false);
                    else TT_FWD_CLASS(64, true, false);
                } else {
                    switch (c) {
                    case 0: TT_FWD_CLASS(8, false, false); break;
                    case 1: TT_FWD_CLASS(16, false, false); break;
                    case 2: TT_FWD_CLASS(32, false, false); break;
                    default: TT_FWD_CLASS(64, false, false); break;
                    }
                }
#undef TT_FWD_CLASS
                timer_end(p.timing, TM_FWD_CLS0 + c, s);
            }
        }
        if (fused) {
            int g = ceil_div(p.nnz, kThreads);
            g = g > 8192 ? 8192 : g;
            hipLaunchKernelGGL(k_pool_tail, dim3(g), dim3(kThreads), 0, s, a, p.nnz);
        }
        if (p.force_generic || p.any_generic)
            hipLaunchKernelGGL(k_contract_generic, dim3(p.num_blocks * 4), dim3(kThreads), 0, s, a,
                               p.force_generic ? 1 : 0);
    }
    timer_end(p.timing, TM_CONTRACT, s);
    timer_begin(p.timing, TM_POOL, s);
    if (nbags > 0 && (!fused || p.any_generic)) {
        // with fused pooling only the tables of the generic kernels are left
        const int64_t g = (nbags + 3) / 4;
        hipLaunchKernelGGL(k_pool, dim3((unsigned)g), dim3(kThreads), 0, s, p.dtab, p.T, p.B, offsets,
                           p.nnz, p.ws, out, p.sumD, fused ? 1 : 0);
    }
    timer_end(p.timing, TM_POOL, s);
    return hipGetLastError();
}

} // namespace ttemb
