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
constexpr int kMaxClsOcc = kMaxWorkersPerCu; // queue heads per CU reserved for each class
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
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // the table's record for the class kernels
        const int t = blockIdx.y;
        const TableDesc &tb = a.tab[t];
        FwdTab f;
        f.g1 = a.cores.g[t][0];
        f.g2 = a.cores.g[t][1];
        f.g3t = a.ws.g3t + tb.g3t_off;
        f.E = a.ws.E + a.ws.ebase[t];
        f.Cg = a.ws.Cg ? a.ws.Cg + a.ws.cbase[t] : nullptr;
        f.d1 = tb.d1;
        f.d2 = tb.d2;
        f.d3 = tb.d3;
        f.i2_base = (int32_t)tb.i2_base;
        f.Dp = tb.Dp;
        f.pad = 0;
        a.ws.ftab[t] = f;
    }
    if (blockIdx.x != 0 || blockIdx.y != 0) return;
    const Ws &ws = a.ws;
    __shared__ int cstart[6];
    int split = ws.ctrl[CTRL_SPLIT];
    if (split > ws.ckpt_slots) split = ws.ckpt_slots;
    // first chunk of each rank class, from the work list (k_chunk_records)
    if (threadIdx.x <= 5) cstart[threadIdx.x] = ws.ctrl[CTRL_CLS_START + threadIdx.x];
    __syncthreads();
    for (int c = 0; c < 4; ++c)
        for (int b = threadIdx.x; b < g.nb[c]; b += blockDim.x)
            ws.heads[(c * stride + b) * kHeadPad] = cstart[c] + range_begin(b, cstart[c + 1] - cstart[c], g.nb[c]);
    for (int i = threadIdx.x; i < split; i += blockDim.x) ws.flags[i] = 0;
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

// Claiming work (one wave of a block).  claim_start() issues the atomic on the
// current victim's head; claim_finish() checks it and, when that victim is
// drained, probes the next 64 victims in parallel and retries.  Every chunk is
// handed out exactly once (heads only grow) and the loop ends once every
// victim has been seen drained.
//
// The current victim (its order index vi, block v and range end, chunk ids
// offset by the class's first chunk), recomputed only when vi changes: the
// victim order and the range bounds take integer divisions by run-time
// values, some hundred scalar instructions per claim otherwise.
struct Victim {
    int vi = -1, v = 0, end = 0;
    __device__ __forceinline__ void at(int nvi, int me, int nb, int base, int64_t C)
    {
        if (nvi == vi) return;
        vi = nvi;
        v = victim_of(me, nvi, nb);
        end = base + range_begin(v + 1, C, nb);
    }
};

__device__ __forceinline__ int claim_start(int32_t *heads, int me, int vi, int nb, int nvict)
{
    int raw = 0x7fffffff;
    if (vi < nvict && (threadIdx.x & 63) == 0) raw = atomicAdd(&heads[victim_of(me, vi, nb) * kHeadPad], 1);
    return raw;
}

// claim_start() without its wait: lane 0's atomic stays in flight in the
// returned register until claim_finish() reads it at the caller's next claim,
// so a claim costs no round trip of its own.  The atomic is an increment that
// wraps at 2^32 - 1 (heads stay far below): the compiler turns a single-lane
// atomicAdd into a wave-aggregated one whose result it reads back at once,
// which is the very wait this avoids.
// The victim is cv (cv.vi == vi whenever vi < nvict).
__device__ __forceinline__ int claim_issue(int32_t *heads, const Victim &cv, int vi, int nvict)
{
    int raw = 0x7fffffff;
    if (vi < nvict && (threadIdx.x & 63) == 0)
        raw = (int)atomicInc(reinterpret_cast<unsigned *>(&heads[cv.v * kHeadPad]), 0xffffffffu);
    return raw;
}

// heads / chunk ids are offset by `base`, the class's first chunk; C = its count
// (cv caches the current victim; it is left at the victim of the chunk returned)
__device__ int claim_finish(int32_t *heads, int base, int me, int &vi, int nb, int nvict, int64_t C, int raw,
                            int &steals, Victim &cv)
{
    const int lane = threadIdx.x & 63;
    int res;
    for (;;) {
        const bool live = vi < nvict;
        if (live) cv.at(vi, me, nb, base, C);
        int got = -1;
        if ((lane == 0) & live & (raw < cv.end)) got = raw;
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
    const int slot = small_div(li, d3), j3 = li - slot * d3;
    int j, rb, cnt;
    chunk_piece(r, small_div(16, d3), e, j, rb, cnt);
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
    const int P = small_div(16, d3);
    // record fields that steer control flow, made wave-uniform: a branch on a
    // value the compiler takes as per-lane runs both sides under exec masks,
    // and the waits of one side then apply to the other
    const int tile = uni(rec.tile), nu = uni(rec.nu), i2 = uni(rec.i2), cslot = uni(rec.slot);
    const int rbeg = uni(rec.rbeg), nch = uni(rec.nch);
    const int np = uni(rec.pstart[nu]);
    const int slot = small_div(li, d3), j3 = li - slot * d3;

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
                    const int bag = lane < n ? a.ws.lb[a.ws.perm[sb + lane]] : 0;
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
    Victim cv;
    // wave 0 runs the claims two chunks ahead: chunk c+2 is claimed while
    // chunk c runs, and the record of chunk c+1 is loaded at the end of chunk c-1
    int pre = 0, raw = 0x7fffffff, c2w = -1;
    if (w == 0) {
        const int c0 = claim_finish(heads, base, me, vi, nb, nvict, C, claim_start(heads, me, vi, nb, nvict), steals, cv);
        const int c1 = c0 < 0 ? -1
                              : claim_finish(heads, base, me, vi, nb, nvict, C, claim_start(heads, me, vi, nb, nvict), steals, cv);
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
                    c2w = cn < 0 ? -1 : claim_finish(heads, base, me, vi, nb, nvict, C, raw, steals, cv);
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

// Wave-uniform reads of values held one per lane (a record or a table entry).
__device__ __forceinline__ int rl(int v, int k) { return __builtin_amdgcn_readlane(v, k); }
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) floatx4 gfloatx4;
// A global-memory pointer held as two dwords (lanes k, k+1): the address space
// is stated so that accesses through it are global (vector memory counter
// only), not flat ones, which the LDS counter also tracks.
template <class T> __device__ __forceinline__ __attribute__((address_space(1))) T *rl_ptr(int v, int k)
{
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane(v, k), hi = (uint32_t)__builtin_amdgcn_readlane(v, k + 1);
    return reinterpret_cast<__attribute__((address_space(1))) T *>(lo | (hi << 32));
}
// ChunkRec fields as dword indices
enum RecField { RF_TILE = 0, RF_T = 1, RF_NU = 2, RF_RBEG = 3, RF_REND = 4, RF_SLOT = 5, RF_I2 = 6, RF_I1 = 8,
                RF_USTART = 12, RF_CCNT = 16, RF_PSTART = 20, RF_ROWOFF = 25, RF_NCH = 30, RF_UBEG = 31,
                RF_I3 = 32 };
static_assert(offsetof(ChunkRec, i1) == 4 * RF_I1 && offsetof(ChunkRec, ustart) == 4 * RF_USTART &&
                  offsetof(ChunkRec, ccnt) == 4 * RF_CCNT && offsetof(ChunkRec, pstart) == 4 * RF_PSTART &&
                  offsetof(ChunkRec, rowoff) == 4 * RF_ROWOFF && offsetof(ChunkRec, nch) == 4 * RF_NCH &&
                  offsetof(ChunkRec, ubeg) == 4 * RF_UBEG && offsetof(ChunkRec, i3) == 4 * RF_I3,
              "record field indices");
static_assert(offsetof(FwdTab, g2) == 4 * FT_G2 && offsetof(FwdTab, g3t) == 4 * FT_G3T &&
                  offsetof(FwdTab, E) == 4 * FT_E && offsetof(FwdTab, Cg) == 4 * FT_CG &&
                  offsetof(FwdTab, d1) == 4 * FT_D1 && offsetof(FwdTab, i2_base) == 4 * FT_I2BASE &&
                  offsetof(FwdTab, Dp) == 4 * FT_DP,
              "table field indices");

// Output tile e of a chunk (record rv, one dword per lane): unit j, first row
// in chunk numbering rb, rows cnt (P rows per output tile).  Wave-uniform.
__device__ __forceinline__ void rec_piece(int rv, int P, int e, int &j, int &rb, int &cnt)
{
    const int ps1 = rl(rv, RF_PSTART + 1), ps2 = rl(rv, RF_PSTART + 2), ps3 = rl(rv, RF_PSTART + 3);
    j = (e >= ps1) + (e >= ps2) + (e >= ps3);
    const int ps = j == 0 ? 0 : j == 1 ? ps1 : j == 2 ? ps2 : ps3;
    const int ro = __builtin_amdgcn_readlane(rv, RF_ROWOFF + j);
    rb = ro + (e - ps) * P;
    const int rem = ro + __builtin_amdgcn_readlane(rv, RF_CCNT + j) - rb;
    cnt = rem < P ? rem : P;
}

// ---------------------------------------------------------------------------
// Per-wave contraction of the rank classes R <= 16 (R1 = R2 = R, d1, d2 <= 4,
// d3 <= 16).  Every wave of the grid is an independent persistent worker with
// its own static range of chunks (and, in the stealing modes, its own queue
// head): no block barrier anywhere in the chunk loop.  Per chunk (one tile of
// up to four prefix units sharing (table, i2), at most 32 of its unique rows):
//  * C for the tile's units, [16 rows (unit, j1)] x [4R columns (j2, r2)], on
//    v_mfma_f32_16x16x4_f32 with the G1[i1] slices stacked into the A operand
//    and the whole G2[i2] slice as the B operand, held in the wave's registers
//    while consecutive chunks keep (table, i2) (B-stationary: (R/4)^2 VGPRs);
//  * C is written to the wave's own LDS region as [unit][m2 = j1*d2 + j2][r2]
//    and stays there while the wave's next chunks continue the same tile;
//  * rows: per output tile of P = 16/d3 rows of one unit,
//      O[(slot, j3)][m2] = sum_r2 G3t[i3_slot][j3][r2] * C_u[m2][r2],
//    A = the rows' transposed G3 slices (float4 loads), B = C_u read from LDS
//    along r2; each lane then holds four consecutive columns of one E row
//    (column m2*d3 + j3), written with one float4 store when d3 is 4, 8 or 16.
// FlowTT page section 3.2 (C = A.B computed once per prefix group and kept
// on chip, E = C.D for each row), section 3.3 (prefix groups as the unit of
// work) and section 3.4 (persistent workers, stealing, L2 checkpoints of a
// prefix tile split over several workers).
template <int R>
struct FwdW {
    static constexpr int KQ = R / 4;       // K values each lane feeds per 16x16 output tile
    static constexpr int NT = R / 4;       // 16-column tiles of the 4R columns of C
    static constexpr int BREG = NT * KQ;   // G2 slice registers per lane
    static constexpr int CSTR = R + 4;     // LDS row stride of C (floats)
    static constexpr int CU = 16 * CSTR;   // floats per unit
    // blocks of four waves per CU: rank 16 at five (96 VGPRs; on the 26-table
    // training step 0.214 -> 0.200 ms against four, six spills)
    static constexpr int OCC = R == 16 ? 5 : 4;
    static constexpr int NQ = 4;           // row tiles whose operands are loaded together
};
template <int R> constexpr int fwd_workers_per_cu() { return FwdW<R>::OCC * (kThreads / 64); }
static_assert(fwd_workers_per_cu<8>() <= kMaxClsOcc && fwd_workers_per_cu<16>() <= kMaxClsOcc,
              "one queue head per worker");

template <int R, bool STEAL>
__global__ __launch_bounds__(kThreads, FwdW<R>::OCC) void k_contract_w(FwdArgs a, int heads_stride)
{
    static_assert(R == 8 || R == 16, "ranks 32 and 64 run the tile-pipelined kernel");
    using L = FwdW<R>;
    constexpr int CLS = R == 8 ? 0 : 1;
    constexpr int KQ = L::KQ, NT = L::NT, CSTR = L::CSTR, CU = L::CU, NQ = L::NQ;
    __shared__ __attribute__((aligned(16))) float Cs_all[kThreads / 64][4 * CU];
    __shared__ long long s_t0;
    __shared__ int s_work, s_rows, s_steals, s_hits, s_misses;
    const int lane = threadIdx.x & 63, w = uni(threadIdx.x >> 6), li = lane & 15, kq = lane >> 4;
    if (threadIdx.x == 0) {
        s_t0 = wall_clock64();
        s_work = s_rows = s_steals = s_hits = s_misses = 0;
    }
    float *Cw = Cs_all[w];
    const Ws &ws = a.ws;
    // worker numbering with worker % 8 = the XCD of its block (blocks go
    // round-robin over the 8 XCDs and the grid is a multiple of 8 blocks)
    const int nb = gridDim.x * (kThreads / 64), me = w * gridDim.x + blockIdx.x;
    const int base = ws.ctrl[CTRL_CLS_START + CLS];
    const int64_t C = ws.ctrl[CTRL_CLS_START + CLS + 1] - base;
    int32_t *heads = ws.heads + CLS * heads_stride * kHeadPad;
    const int nvict = STEAL ? nb >> 3 : 1;
    int vi = 0, steals = 0, hits = 0, misses = 0, nwork = 0, nrows = 0;
    float breg[L::BREG];
#pragma unroll
    for (int i = 0; i < L::BREG; ++i) breg[i] = 0.f;
    int bkey = -1, ctile = -1;
    Victim cv;
    int cstat = base + range_begin(me, C, nb); // next chunk of the static range
    const int cend = base + range_begin(me + 1, C, nb);
    int raw = 0x7fffffff; // stealing: the claim in flight
    // next chunk of this wave: its static range in order (no atomics), or in
    // the stealing modes a claim from the workers of its XCD, the claim of the
    // chunk after it left in flight
    auto next_id = [&]() -> int {
        if constexpr (!STEAL) {
            return cstat < cend ? cstat++ : -1;
        } else {
            const int got = claim_finish(heads, base, me, vi, nb, nvict, C, raw, steals, cv);
            raw = claim_issue(heads, cv, got >= 0 ? vi : nvict, nvict);
            return got;
        }
    };
    if constexpr (STEAL) {
        cv.at(0, me, nb, base, C);
        raw = claim_issue(heads, cv, 0, nvict);
    }
    // the next chunk is known (and its record loaded) while chunk c runs; the
    // record load is unconditional (past the last chunk chunk 0's, never
    // used): a load in a branch leaves its register to be copied at the join,
    // and the copy waits for the load
    int c = next_id();
    int rec = reinterpret_cast<const int *>(&ws.crec[c >= 0 ? c : 0])[lane];
    while (c >= 0) {
        const int cn = next_id();
        const int recn = reinterpret_cast<const int *>(&ws.crec[cn >= 0 ? cn : 0])[lane];
        // record fields (ChunkRec, one dword per lane), wave-uniform
        auto fld = [&](int i) { return __builtin_amdgcn_readlane(rec, i); };
        const int tile = fld(0), t = fld(1), nu = fld(2), rbeg = fld(3), cslot = fld(5), i2 = fld(6);
        const int nch = fld(30), ubeg = fld(31);
        const int ps1 = fld(21), ps2 = fld(22), ps3 = fld(23), np = fld(20 + nu);
        const auto &tb = kconst(a.tab)[t];
        const int d1 = tb.d1, d2 = tb.d2, d3 = tb.d3, D12 = d1 * d2, Dp = tb.Dp, P = small_div(16, d3);
        if (tile != ctile) {
            // ---- prefix tile C_u = G1[i1_u] . G2[i2] for the tile's units
            bool have = false;
            const bool split = cslot >= 0 && a.sched == kSchedStealL2;
            if (split && rbeg > 0) {
                int f = 0;
                if (lane == 0) f = __hip_atomic_load(&ws.flags[cslot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
                if (uni(f)) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    const float4 *src = reinterpret_cast<const float4 *>(ws.ckpt + (size_t)cslot * kCTile);
                    for (int e = lane; e < 4 * 16 * R / 4; e += 64) {
                        const int j = e / (4 * R), f2 = e - j * (4 * R), m = f2 / (R / 4), c4 = f2 - m * (R / 4);
                        *reinterpret_cast<float4 *>(Cw + j * CU + m * CSTR + 4 * c4) = src[e];
                    }
                    have = true;
                }
                if (have) ++hits;
                else ++misses;
            }
            if (!have) {
                const int key = (int)(tb.i2_base + (uint32_t)i2);
                if (key != bkey) {
                    // a new G2 slice: lane (kq, li) holds G2[i2][kq*KQ + s][col] for
                    // its columns col = 16*n + li (zero past d2*R)
                    const float *G2 = a.cores.g[t][1] + (int64_t)i2 * R * d2 * R;
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        const int col = n * 16 + li, j2 = col / R, r2 = col - j2 * R;
                        const bool ok = j2 < d2;
                        const float *src = G2 + (ok ? j2 : 0) * R + r2;
#pragma unroll
                        for (int s2 = 0; s2 < KQ; ++s2) {
                            const float v = src[(int64_t)(kq * KQ + s2) * d2 * R];
                            breg[n * KQ + s2] = ok ? v : 0.f;
                        }
                    }
                    bkey = key;
                }
                // A operand: lane (kq, li) holds G1[i1_u][j1][kq*KQ ..] of row li = (u, j1)
                float av[KQ];
                {
                    const int g = li >> 2, j1 = li & 3;
                    const int i1 = __shfl(rec, 8 + (g < nu ? g : 0), 64);
                    const float *src = a.cores.g[t][0] + ((int64_t)i1 * d1 + (j1 < d1 ? j1 : 0)) * R + kq * KQ;
                    if constexpr (KQ % 4 == 0) {
#pragma unroll
                        for (int s2 = 0; s2 < KQ; s2 += 4) {
                            const float4 v = *reinterpret_cast<const float4 *>(src + s2);
                            av[s2] = v.x;
                            av[s2 + 1] = v.y;
                            av[s2 + 2] = v.z;
                            av[s2 + 3] = v.w;
                        }
                    } else {
#pragma unroll
                        for (int s2 = 0; s2 < KQ; ++s2) av[s2] = src[s2];
                    }
                }
                floatx4 acc[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < KQ; ++s2)
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s2], breg[n * KQ + s2], acc[n], 0, 0, 0);
                // lane (kq, li) holds rows 4*kq + v = (unit kq, j1 = v) of column 16n + li
                const bool pub = split && rbeg == 0 && (nch > 2 || cn != c + 1);
                float *ck = ws.ckpt + (size_t)(cslot >= 0 ? cslot : 0) * kCTile;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int col = n * 16 + li, j2 = col / R, r2 = col - j2 * R;
                    if (j2 < d2 && kq < nu) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            if (v < d1) {
                                const int m = v * d2 + j2;
                                Cw[kq * CU + m * CSTR + r2] = acc[n][v];
                                if (pub) ck[(kq * 16 + m) * R + r2] = acc[n][v];
                            }
                        }
                    }
                }
                if (pub) {
                    // publish when another worker may run a later chunk of this tile
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                    if (lane == 0) __hip_atomic_store(&ws.flags[cslot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            ctile = tile;
            __builtin_amdgcn_wave_barrier();
        }

        // ---- rows: output tiles e = 0 .. np-1, NQ at a time
        float *Et = ws.E + kconst(ws.ebase)[t];
        const float *G3t = ws.g3t + tb.g3t_off;
        const int slot = small_div(li, d3), j3l = li - slot * d3;
        const int ro0 = fld(25), ro1 = fld(26), ro2 = fld(27), ro3 = fld(28);
        const int cc0 = fld(16), cc1 = fld(17), cc2 = fld(18), cc3 = fld(19);
        const int us0 = fld(12), us1 = fld(13), us2 = fld(14), us3 = fld(15);
        auto sel = [](int j, int x0, int x1, int x2, int x3) { return j == 0 ? x0 : j == 1 ? x1 : j == 2 ? x2 : x3; };
        // output tile e -> unit j, its first row (chunk numbering) and row count
        auto piece = [&](int e, int &j, int &rb, int &cnt) {
            j = (e >= ps1) + (e >= ps2) + (e >= ps3);
            const int ro = sel(j, ro0, ro1, ro2, ro3);
            rb = ro + (e - sel(j, 0, ps1, ps2, ps3)) * P;
            const int rem = ro + sel(j, cc0, cc1, cc2, cc3) - rb;
            cnt = rem < P ? rem : P;
        };
        for (int e0 = 0; e0 < np; e0 += NQ) {
            float ga[NQ][KQ];
            // operands of NQ output tiles: each lane's G3 row run (clamped to a
            // valid row of the tile; results of padding rows are not stored)
#pragma unroll
            for (int k = 0; k < NQ; ++k) {
                const int e = e0 + k < np ? e0 + k : np - 1;
                int j, rb, cnt;
                piece(e, j, rb, cnt);
                const int q = rb + (slot < cnt ? slot : 0);
                const int i3 = __shfl(rec, 32 + q, 64);
                const float *src = G3t + ((int64_t)i3 * d3 + j3l) * R + kq * KQ;
                if constexpr (KQ % 4 == 0) {
#pragma unroll
                    for (int s2 = 0; s2 < KQ; s2 += 4) {
                        const float4 v = *reinterpret_cast<const float4 *>(src + s2);
                        ga[k][s2] = v.x;
                        ga[k][s2 + 1] = v.y;
                        ga[k][s2 + 2] = v.z;
                        ga[k][s2 + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int s2 = 0; s2 < KQ; ++s2) ga[k][s2] = src[s2];
                }
            }
#pragma unroll
            for (int k = 0; k < NQ; ++k) {
                const int e = e0 + k;
                if (e >= np) break;
                int j, rb, cnt;
                piece(e, j, rb, cnt);
                const float *cb = Cw + j * CU + (li < D12 ? li : 0) * CSTR + kq * KQ;
                floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
                if constexpr (KQ % 4 == 0) {
#pragma unroll
                    for (int s2 = 0; s2 < KQ; s2 += 4) {
                        const float4 v = *reinterpret_cast<const float4 *>(cb + s2);
                        o = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[k][s2], v.x, o, 0, 0, 0);
                        o = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[k][s2 + 1], v.y, o, 0, 0, 0);
                        o = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[k][s2 + 2], v.z, o, 0, 0, 0);
                        o = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[k][s2 + 3], v.w, o, 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int s2 = 0; s2 < KQ; ++s2)
                        o = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[k][s2], cb[s2], o, 0, 0, 0);
                }
                // lane (kq, li) holds O[4kq + v][li]: row slot (4kq+v)/d3, column li*d3 + (4kq+v)%d3
                const int us = sel(j, us0, us1, us2, us3) + (rb - sel(j, ro0, ro1, ro2, ro3));
                if (li < D12) {
                    if (d3 == 4 || d3 == 8 || d3 == 16) {
                        const int r4 = 4 * kq, sl = small_div(r4, d3), jj = r4 - sl * d3;
                        if (sl < cnt)
                            *reinterpret_cast<floatx4 *>(Et + (int64_t)(us + sl) * Dp + li * d3 + jj) = o;
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int r = 4 * kq + v, sl = small_div(r, d3), jj = r - sl * d3;
                            if (sl < cnt) Et[(int64_t)(us + sl) * Dp + li * d3 + jj] = o[v];
                        }
                    }
                }
            }
        }
        ++nwork;
        nrows += fld(4) - rbeg;
        rec = recn;
        c = cn;
    }
    // scheduling statistics and the block's record
    if (lane == 0) {
        atomicAdd(&s_work, nwork);
        atomicAdd(&s_rows, nrows);
        atomicAdd(&s_steals, steals);
        atomicAdd(&s_hits, hits);
        atomicAdd(&s_misses, misses);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        block_stat_write(ws.bstat + CLS * kStatBlocks, s_t0, s_work, s_rows);
        if (s_steals) atomicAdd(&ws.ctrl[CTRL_STEALS], s_steals);
        if (s_hits) atomicAdd(&ws.ctrl[CTRL_CKPT_HIT], s_hits);
        if (s_misses) atomicAdd(&ws.ctrl[CTRL_CKPT_MISS], s_misses);
    }
}

// ---------------------------------------------------------------------------
// Tile-pipelined block contraction of the rank classes 32 and 64 (R1 = R2 =
// R, d1, d2 <= 4, d3 <= 16): one persistent block of four waves walks its
// chunks (static range, or claimed in the stealing modes), one block barrier
// per chunk.  In the iteration of chunk c the waves
//  (1) compute C of chunk c+1's prefix tile when it starts a new tile, wave w
//      the columns of j2 = w (its quarter of the G2[i2] slice is held in
//      registers while consecutive tiles keep (table, i2)), into the LDS slot
//      that chunk c is not reading (two slots, double-buffered);
//  (2) compute the rows of chunk c from the other slot, output tile e of the
//      chunk on wave e mod 4, O[(slot, j3)][m2] = sum_r2 G3t[i3][j3][r2] *
//      C_u[m2][r2] (A = transposed G3 slices, B = C read from LDS along r2;
//      one float4 store per lane writes four columns of an E row), the next
//      chunk's operands reloaded into the registers each tile has consumed
//      before its result is stored;
//  (3) prefetch the G1 slices of the tile computed in the next iteration.
// So the matrix cores see C of one tile and the rows of another between two
// barriers, and every operand arrives an iteration before it is used.
// FlowTT page section 3.2 (C = A.B once per prefix group, kept on chip,
// reused by each E = C.D; loads of the next TT slices overlapped with compute,
// the pages' ping-pong buffering), section 3.4 (persistent blocks, stealing,
// L2 checkpoints of split prefix tiles).
template <int R>
struct FwdT {
    static constexpr int KQ = R / 4;           // K values each lane feeds per 16x16 output tile
    static constexpr int NTW = R / 16;         // 16-column tiles of C per wave (one j2 each)
    static constexpr int BREG = NTW * KQ;      // G2 registers per lane
    static constexpr int CSTR = R + 4;         // LDS row stride of C (floats)
    static constexpr int CU = 16 * CSTR + 16;  // floats per unit (+16 rotates banks between units)
    static constexpr int CT = 4 * CU;          // floats per tile slot
    static constexpr int OCC = R == 64 ? 2 : 4; // blocks per CU (register-limited, no spills; rank 32: 116 VGPRs)
    static constexpr int PQ = R == 64 ? 3 : 2;  // output tiles per wave whose operands are prefetched
};
static_assert(FwdT<32>::OCC <= kMaxClsOcc && FwdT<64>::OCC <= kMaxClsOcc, "one queue head per block");

template <int R, bool KEEP, bool STEAL>
__global__ __launch_bounds__(kThreads, FwdT<R>::OCC) void k_contract_t(FwdArgs a, int heads_stride)
{
    using L = FwdT<R>;
    constexpr int CLS = R == 32 ? 2 : 3;
    constexpr int KQ = L::KQ, NTW = L::NTW, CSTR = L::CSTR, CU = L::CU, PQ = L::PQ;
    __shared__ __attribute__((aligned(16))) float Cs[2][L::CT];
    // records of ring entries k .. k+2 (iteration k), entry k+3 being written;
    // entry k+4's record travels in the ring owner's registers for a whole iteration
    constexpr int NR = 5;
    __shared__ ChunkRec rr[NR];
    __shared__ int cid[NR], s_ck[NR];
    __shared__ long long s_t0;
    // the table records, read from LDS in the chunk loop (a table change then
    // waits for an LDS read, not for the wave's memory operations in flight)
    __shared__ int s_tab[kMaxTables * 16];
    const int lane = threadIdx.x & 63, w = uni(threadIdx.x >> 6), li = lane & 15, kq = lane >> 4;
    if (threadIdx.x == 0) s_t0 = wall_clock64();
    const Ws &ws = a.ws;
    for (int e = threadIdx.x; e < a.T * 16; e += kThreads) s_tab[e] = reinterpret_cast<const int *>(ws.ftab)[e];
    const int nb = gridDim.x, me = blockIdx.x;
    const int base = ws.ctrl[CTRL_CLS_START + CLS];
    const int64_t C = ws.ctrl[CTRL_CLS_START + CLS + 1] - base;
    const int cend = base + range_begin(me + 1, C, nb); // end of the static range
    int32_t *heads = ws.heads + CLS * heads_stride * kHeadPad;
    const int nvict = STEAL ? nb >> 3 : 1;
    int vi = 0, steals = 0, hits = 0, misses = 0, nwork = 0, nrows = 0;
    int raw = 0x7fffffff; // ring owner (stealing): the claim in flight
    Victim cv;
    int cstat = base + range_begin(me, C, nb); // next chunk of the static range
    const bool l2 = a.sched == kSchedStealL2;

    // next chunk id of this block (ring owner): its static range in order, then
    // (stealing modes) chunks claimed from the other blocks of its XCD
    auto next_id = [&]() -> int {
        if constexpr (!STEAL) {
            return cstat < cend ? cstat++ : -1;
        } else {
            const int got = claim_finish(heads, base, me, vi, nb, nvict, C, raw, steals, cv);
            raw = claim_issue(heads, cv, got >= 0 ? vi : nvict, nvict);
            return got;
        }
    };
    // checkpoint flag of ring entry i, read (thread 0) an iteration before its C is needed
    auto read_ck = [&](int i, int prev_tile) {
        int ok = 0;
        const ChunkRec &r = rr[i];
        if (l2 && cid[i] >= 0 && r.slot >= 0 && r.rbeg > 0 && r.tile != prev_tile)
            ok = __hip_atomic_load(&ws.flags[r.slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        s_ck[i] = ok;
    };
    // the ring's owner is the last wave: the output tiles w, w+4, ... leave it
    // the fewest rows when a chunk's tile count is not a multiple of 4
    constexpr int kRing = kThreads / 64 - 1;
    int pre = 0, pre_id = -1; // ring owner: the record of the next ring entry to write, and its chunk
    if (w == kRing) {
        if constexpr (STEAL) {
            cv.at(vi, me, nb, base, C);
            raw = claim_issue(heads, cv, vi, nvict);
        }
        int prev = 0;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int id = prev >= 0 ? next_id() : -1;
            prev = id;
            if (id >= 0) reinterpret_cast<int *>(&rr[i])[lane] = reinterpret_cast<const int *>(&ws.crec[id])[lane];
            if (lane == 0) cid[i] = id;
        }
        pre_id = prev >= 0 ? next_id() : -1;
        pre = reinterpret_cast<const int *>(&ws.crec[pre_id >= 0 ? pre_id : 0])[lane];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        read_ck(0, -1);
        read_ck(1, rr[0].tile);
    }
    __syncthreads();

    float breg[L::BREG];
#pragma unroll
    for (int i = 0; i < L::BREG; ++i) breg[i] = 0.f;
    int bkey = -1;
    float anext[KQ], g3p[PQ][KQ];

    // table records, one dword per lane; reloaded only when the table changes
    auto tab_load = [&](int t) { return s_tab[(t >= 0 && t < a.T ? t : 0) * 16 + (lane & 15)]; };
    // G1 slices of record rv's units: lane (kq, li) holds row li = (unit, j1), K run kq*KQ ..
    auto load_a = [&](int rv, int tv, float (&av)[KQ]) __attribute__((always_inline)) {
        const int nu = rl(rv, RF_NU), d1 = rl(tv, FT_D1), g = li >> 2, j1 = li & 3;
        const int i1 = __shfl(rv, RF_I1 + (g < nu ? g : 0), 64);
        const gfloatx4 *src = reinterpret_cast<const gfloatx4 *>(rl_ptr<const float>(tv, FT_G1) +
                                                                 ((int64_t)i1 * d1 + (j1 < d1 ? j1 : 0)) * R + kq * KQ);
#pragma unroll
        for (int s4 = 0; s4 < KQ / 4; ++s4) {
            const floatx4 v = src[s4];
            av[4 * s4] = v[0];
            av[4 * s4 + 1] = v[1];
            av[4 * s4 + 2] = v[2];
            av[4 * s4 + 3] = v[3];
        }
    };
    // A operand of output tile e of record rv: the lane's G3t run of its row
    // (clamped to the tile's first row for padding lanes; their results are not
    // stored), as an offset in floats from the table's G3t
    auto g3_off = [&](int rv, int tv, int e) __attribute__((always_inline)) -> int {
        const int d3 = rl(tv, FT_D3), P = small_div(16, d3);
        int j, rb, cnt;
        rec_piece(rv, P, e, j, rb, cnt);
        const int slot = small_div(li, d3), j3 = li - slot * d3;
        const int i3 = __shfl(rv, RF_I3 + rb + (slot < cnt ? slot : 0), 64);
        return (i3 * d3 + j3) * R + kq * KQ;
    };
    auto load_g3_at = [&](const gfloat *src0, float (&gv)[KQ]) __attribute__((always_inline)) {
        const gfloatx4 *src = reinterpret_cast<const gfloatx4 *>(src0);
#pragma unroll
        for (int s4 = 0; s4 < KQ / 4; ++s4) {
            const floatx4 v = src[s4];
            gv[4 * s4] = v[0];
            gv[4 * s4 + 1] = v[1];
            gv[4 * s4 + 2] = v[2];
            gv[4 * s4 + 3] = v[3];
        }
    };
    auto load_g3 = [&](int rv, int tv, int e, float (&gv)[KQ]) __attribute__((always_inline)) {
        load_g3_at(rl_ptr<const float>(tv, FT_G3T) + g3_off(rv, tv, e), gv);
    };
    // (1): C of record rv's tile into slot Ct, wave w the columns of j2 = w
    auto compute_c = [&](int rv, int tv, const float (&av)[KQ], float *Ct) __attribute__((always_inline)) {
        const int nu = rl(rv, RF_NU), i2 = rl(rv, RF_I2), d1 = rl(tv, FT_D1), d2 = rl(tv, FT_D2);
        if (w >= d2) return; // no columns of this j2
        const int key = rl(tv, FT_I2BASE) + i2;
        if (key != bkey) {
            // lane (kq, li) holds G2[i2][kq*KQ + s][w][16*j + li]
            const gfloat *G2 = rl_ptr<const float>(tv, FT_G2) + ((int64_t)i2 * R * d2 + w) * R + li;
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int s2 = 0; s2 < KQ; ++s2) breg[j * KQ + s2] = G2[(int64_t)(kq * KQ + s2) * d2 * R + 16 * j];
            bkey = key;
            // wait here (rare: a new (table, i2) run), not at every tile's first MFMA
            __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0)
        }
        floatx4 acc[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KQ; ++s2)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s2], breg[j * KQ + s2], acc[j], 0, 0, 0);
        // lane (kq, li) holds C[(unit kq, j1 = v)][j2 = w][r2 = 16j + li]
        if (kq < nu) {
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (v < d1) Ct[kq * CU + (v * d2 + w) * CSTR + 16 * j + li] = acc[j][v];
        }
    };
    // (2): output tile e of record rv from slot Ct with operands gv, when
    // act; then gv always takes the operands at nsrc (a valid tile, also
    // where they go unused), before the E row is stored.  The reload is
    // unconditional: a load in a branch leaves its registers to be copied at
    // the join, and the copy waits for the load to arrive.
    auto rows_tile = [&](int rv, int tv, int e, bool act, float (&gv)[KQ], const float *Ct,
                         const gfloat *nsrc) __attribute__((always_inline)) {
        const int d1 = rl(tv, FT_D1), d2 = rl(tv, FT_D2), d3 = rl(tv, FT_D3), D12 = d1 * d2, Dp = rl(tv, FT_DP);
        const int P = small_div(16, d3);
        int j, rb, cnt;
        rec_piece(rv, P, e, j, rb, cnt);
        floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
        if (act) {
            const float4 *cb = reinterpret_cast<const float4 *>(Ct + j * CU + (li < D12 ? li : 0) * CSTR + kq * KQ);
#pragma unroll
            for (int s4 = 0; s4 < KQ / 4; ++s4) {
                const float4 v = cb[s4];
                o = __builtin_amdgcn_mfma_f32_16x16x4f32(gv[4 * s4], v.x, o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x4f32(gv[4 * s4 + 1], v.y, o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x4f32(gv[4 * s4 + 2], v.z, o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x4f32(gv[4 * s4 + 3], v.w, o, 0, 0, 0);
            }
        }
        // keep the reload after this tile's products and before its store:
        // the products wait only for operands that arrived an iteration ago
        __builtin_amdgcn_sched_barrier(0);
        load_g3_at(nsrc, gv);
        __builtin_amdgcn_sched_barrier(0);
        if (!act) return;
        const int us = __builtin_amdgcn_readlane(rv, RF_USTART + j) + (rb - __builtin_amdgcn_readlane(rv, RF_ROWOFF + j));
        gfloat *Et = rl_ptr<float>(tv, FT_E);
        if (li < D12) {
            if (d3 == 4 || d3 == 8 || d3 == 16) {
                const int r4 = 4 * kq, sl = small_div(r4, d3), jj = r4 - sl * d3;
                if (sl < cnt) *reinterpret_cast<gfloatx4 *>(Et + (int64_t)(us + sl) * Dp + li * d3 + jj) = o;
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int rr4 = 4 * kq + v, sl = small_div(rr4, d3), jj = rr4 - sl * d3;
                    if (sl < cnt) Et[(int64_t)(us + sl) * Dp + li * d3 + jj] = o[v];
                }
            }
        }
    };
    // C of a tile from a published checkpoint ([unit][16][R] compact) into a slot
    auto ck_copy = [&](int cslot, float *Ct) __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const float4 *src = reinterpret_cast<const float4 *>(ws.ckpt + (size_t)cslot * kCTile);
        for (int e = threadIdx.x; e < 16 * R; e += kThreads) {
            const int j = e / (4 * R), f = e - j * (4 * R), m = f / (R / 4), c4 = f - m * (R / 4);
            *reinterpret_cast<float4 *>(Ct + j * CU + m * CSTR + 4 * c4) = src[e];
        }
    };

    int cs = 0;
    // records of the current chunk and the next, one dword per lane, with their
    // tables' records (carried from one iteration to the next)
    int recv = reinterpret_cast<const int *>(&rr[0])[lane], nrecv = reinterpret_cast<const int *>(&rr[1])[lane];
    const int c0 = uni(cid[0]), c1 = uni(cid[1]);
    int tv = 0, tvn = 0;
    if (c0 >= 0) {
        tv = tab_load(rl(recv, RF_T));
        tvn = c1 >= 0 ? tab_load(rl(nrecv, RF_T)) : tv;
        // prologue: C of the first chunk's tile, the next tile's G1 slices and
        // the first chunk's row operands
        if (uni(s_ck[0])) {
            ck_copy(rl(recv, RF_SLOT), Cs[0]);
            ++hits;
        } else {
            if (l2 && rl(recv, RF_SLOT) >= 0 && rl(recv, RF_RBEG) > 0) ++misses;
            float a0[KQ];
            load_a(recv, tv, a0);
            compute_c(recv, tv, a0, Cs[0]);
        }
        if (c1 >= 0 && rl(nrecv, RF_TILE) != rl(recv, RF_TILE)) load_a(nrecv, tvn, anext);
        const int np0 = __builtin_amdgcn_readlane(recv, RF_PSTART + rl(recv, RF_NU));
#pragma unroll
        for (int jq = 0; jq < PQ; ++jq) {
            const int e = w + 4 * jq < np0 ? w + 4 * jq : np0 - 1;
            load_g3(recv, tv, e, g3p[jq]);
        }
    }
    __syncthreads();
    int pub_slot = -1; // checkpoint whose flag this block sets after the next barrier
    int i = 0; // ring slot of entry k
    for (int k = 0;; ++k) {
        const int i1 = i == NR - 1 ? 0 : i + 1, i2r = i1 == NR - 1 ? 0 : i1 + 1, i3r = i2r == NR - 1 ? 0 : i2r + 1;
        const int c = uni(cid[i]);
        if (c < 0) break;
        if (threadIdx.x == 0 && pub_slot >= 0)
            __hip_atomic_store(&ws.flags[pub_slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        pub_slot = -1;
        const int cn = uni(cid[i1]), c2 = uni(cid[i2r]);
        const int r2v = reinterpret_cast<const int *>(&rr[i2r])[lane];
        const int tile = rl(recv, RF_TILE), ntile = rl(nrecv, RF_TILE);
        const bool has_next = cn >= 0, next_new = has_next && ntile != tile;
        const int ck_next = uni(s_ck[i1]);
        // table record of entry k+2 (the same table as entry k+1 nearly always)
        int tv2 = tvn;
        if (c2 >= 0 && rl(r2v, RF_T) != rl(nrecv, RF_T)) tv2 = tab_load(rl(r2v, RF_T));
        // (1) C of the next chunk's tile
        if (next_new) {
            if (ck_next) {
                ck_copy(rl(nrecv, RF_SLOT), Cs[cs ^ 1]);
                ++hits;
            } else {
                if (l2 && rl(nrecv, RF_SLOT) >= 0 && rl(nrecv, RF_RBEG) > 0) ++misses;
                compute_c(nrecv, tvn, anext, Cs[cs ^ 1]);
            }
        }
        // (3) G1 slices of the tile computed in the next iteration
        if (c2 >= 0 && rl(r2v, RF_TILE) != ntile) load_a(r2v, tv2, anext);
        // (2) rows of chunk c: output tiles w, w+4, ... of the chunk
        {
            const int np = __builtin_amdgcn_readlane(recv, RF_PSTART + rl(recv, RF_NU));
            const int npn = has_next ? __builtin_amdgcn_readlane(nrecv, RF_PSTART + rl(nrecv, RF_NU)) : 0;
            const float *Ct = Cs[cs];
            // the operands reloaded for the next chunk's tiles (a chunk has at
            // least one tile; past the last chunk the block's own last tile)
            const int rn = has_next ? nrecv : recv, tn = has_next ? tvn : tv, nlast = has_next ? npn - 1 : np - 1;
            // the reloads' sources first, as independent chains the compiler
            // interleaves (behind each tile's products they ran one by one)
            const gfloat *G3n = rl_ptr<const float>(tn, FT_G3T);
            int noff[PQ];
#pragma unroll
            for (int jq = 0; jq < PQ; ++jq) {
                const int e = w + 4 * jq;
                noff[jq] = g3_off(rn, tn, e < nlast ? e : nlast);
            }
#pragma unroll
            for (int jq = 0; jq < PQ; ++jq) {
                const int e = w + 4 * jq;
                rows_tile(recv, tv, e < np ? e : np - 1, e < np, g3p[jq], Ct, G3n + noff[jq]);
            }
            // tiles past the prefetched ones (chunks of more than 4 * PQ output tiles)
            for (int e = w + 4 * PQ; e < np; e += 4) {
                float gv[KQ];
                load_g3(recv, tv, e, gv);
                const gfloat *src = rl_ptr<const float>(tv, FT_G3T) + g3_off(recv, tv, e);
                rows_tile(recv, tv, e, true, gv, Ct, src);
            }
        }
        const int rbeg = rl(recv, RF_RBEG), nu = rl(recv, RF_NU);
        // the tile's first chunk publishes its C when a later chunk of the tile
        // may run on another block (the next chunk here is not its continuation)
        const int cslot = rl(recv, RF_SLOT);
        if (l2 && cslot >= 0 && rbeg == 0 && (rl(recv, RF_NCH) > 2 || cn != c + 1)) {
            float4 *dst = reinterpret_cast<float4 *>(ws.ckpt + (size_t)cslot * kCTile);
            for (int e = threadIdx.x; e < 16 * R; e += kThreads) {
                const int j = e / (4 * R), f = e - j * (4 * R), m = f / (R / 4), c4 = f - m * (R / 4);
                dst[e] = *reinterpret_cast<const float4 *>(Cs[cs] + j * CU + m * CSTR + 4 * c4);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            pub_slot = cslot;
        }
        if constexpr (KEEP) {
            if (rbeg == 0) {
                gfloatx4 *dst = reinterpret_cast<gfloatx4 *>(rl_ptr<float>(tv, FT_CG) + (int64_t)rl(recv, RF_UBEG) * 16 * R);
                for (int e = threadIdx.x; e < nu * 4 * R; e += kThreads) {
                    const int j = e / (4 * R), f = e - j * (4 * R), m = f / (R / 4), c4 = f - m * (R / 4);
                    dst[e] = *reinterpret_cast<const floatx4 *>(Cs[cs] + j * CU + m * CSTR + 4 * c4);
                }
            }
        }
        // ring owner: entry k+3 (its record loaded an iteration ago) goes to the
        // slot of entry k-2; the next chunk is claimed and the record of entry
        // k+4 loaded.  Both loads are unconditional (past the last chunk, chunk
        // 0's record under id -1, never used): a load in a branch is waited for
        // at the join.  Placed after the rows' operand reloads, so that on
        // every path the record and the claim issued an iteration ago are
        // older than those reloads and no wait here covers them.
        if (w == kRing) {
            reinterpret_cast<int *>(&rr[i3r])[lane] = pre;
            if (lane == 0) cid[i3r] = pre_id;
            pre_id = pre_id >= 0 ? next_id() : -1;
            pre = reinterpret_cast<const int *>(&ws.crec[pre_id >= 0 ? pre_id : 0])[lane];
        }
        if (threadIdx.x == 0) {
            ++nwork;
            nrows += rl(recv, RF_REND) - rbeg;
            // checkpoint flag of entry k+2, whose tile the next iteration computes
            read_ck(i2r, ntile);
        }
        __syncthreads(); // entry k done, entry k+3 written, C of the next tile complete
        if (next_new) cs ^= 1;
        i = i1;
        recv = nrecv;
        nrecv = r2v;
        tv = tvn;
        tvn = tv2;
    }
    if (threadIdx.x == 0 && pub_slot >= 0)
        __hip_atomic_store(&ws.flags[pub_slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) block_stat_write(ws.bstat + CLS * kStatBlocks, s_t0, nwork, nrows);
    if (lane == 0 && w == kRing && steals) atomicAdd(&ws.ctrl[CTRL_STEALS], steals);
    // hits and misses are counted by every wave alike; wave 0 reports them
    if (lane == 0 && w == 0) {
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

// Bag-major sum pooling of the tables of one lane class (LPR lanes per row,
// one float4 column -- or one float when VEC is false -- per lane; the class
// of a table is its TableDesc::gcls).  A wave pools G = 64 / LPR consecutive
// bags of one table at once, lane group g the bag bag0 + g: one load of the
// G + 1 offsets, then per step of LPR lookups one load of their unique-row
// ids and the row loads of every group issued back to back, up to eight per
// lane (UNR) at once, so a bag's rows are in flight together instead of one
// short batch after another.
// Each lane adds its bag's rows in lookup order (a fixed order, no atomics:
// the output is bit-reproducible); empty bags write zeros.
template <int LPR, bool VEC>
__global__ __launch_bounds__(kThreads) void k_pool(const TableDesc *tab, int64_t B, const int64_t *offsets,
                                                   int64_t nnz, Ws ws, float *out, int SD, int gcls,
                                                   int skip_mfma)
{
    constexpr int G = 64 / LPR;
    // row loads in flight per lane: eight keeps the kernel at eight waves per
    // SIMD (measured on the 26-table forward at batch 32768: 0.43 ms with
    // sixteen, 0.36 ms with eight)
    constexpr int UNR = LPR < 8 ? LPR : 8;
    const int t = blockIdx.y;
    const auto &tb = kconst(tab)[t];
    if (tb.gcls != gcls || (skip_mfma && tb.cls >= 0)) return; // pooled inside the contraction
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane / LPR, gl = lane - grp * LPR;
    const int64_t bag0 = ((int64_t)blockIdx.x * (kThreads / 64) + w) * G;
    if (bag0 >= B) return;
    // the lane group's bag and its lookup range (clamped into [0, nnz])
    const bool live = bag0 + grp < B;
    const int64_t bag = (int64_t)t * B + (live ? bag0 + grp : B - 1);
    int64_t olo = offsets[bag], ohi = offsets[bag + 1];
    olo = olo < 0 ? 0 : (olo > nnz ? nnz : olo);
    ohi = ohi < 0 ? 0 : (ohi > nnz ? nnz : ohi);
    const int lo = (int)olo;
    int hi = (int)ohi;
    const int u0 = kconst(ws.tab_uniq_start)[t], u1 = kconst(ws.tab_uniq_start)[t + 1];
    if (!live || hi < lo || u1 <= u0) hi = lo;
    const int len = hi - lo;
    int maxlen = len;
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
        const int y = __shfl_xor(maxlen, m, 64);
        maxlen = y > maxlen ? y : maxlen;
    }
    maxlen = __builtin_amdgcn_readfirstlane(maxlen);
    const float *Et = ws.E + kconst(ws.ebase)[t];
    const int D = tb.D, Dp = tb.Dp, col_off = tb.col_off;
    float *o_row = out + (int64_t)(bag0 + (live ? grp : 0)) * SD + col_off;
    const int cn = VEC ? (D + 3) >> 2 : D;
    for (int cb = 0; cb < cn; cb += LPR) {
        const int c = cb + gl;
        const bool okc = c < cn;
        const int cc = okc ? c : 0;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k0 = 0; k0 < maxlen; k0 += LPR) {
            // unique-row ids of lookups k0 .. k0 + LPR - 1 of this lane's bag
            int uu = k0 + gl < len ? ws.inv[lo + k0 + gl] : u0;
            uu = uu < u0 ? u0 : (uu >= u1 ? u1 - 1 : uu);
            const int nk = maxlen - k0 < LPR ? maxlen - k0 : LPR;
            for (int kb = 0; kb < nk; kb += UNR) {
                float4 v[UNR];
#pragma unroll
                for (int k = 0; k < UNR; ++k) {
                    const int u = __shfl(uu, grp * LPR + ((kb + k) & (LPR - 1)), 64);
                    const float *src = Et + (int64_t)u * Dp;
                    if (VEC) v[k] = *reinterpret_cast<const float4 *>(src + 4 * cc);
                    else v[k] = make_float4(src[cc], 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int k = 0; k < UNR; ++k) {
                    if (k0 + kb + k < len) {
                        acc.x += v[k].x;
                        if (VEC) {
                            acc.y += v[k].y;
                            acc.z += v[k].z;
                            acc.w += v[k].w;
                        }
                    }
                }
            }
        }
        if (live && okc) {
            if (VEC) {
                const int j = 4 * c;
                if (j + 3 < D) {
                    *reinterpret_cast<float4 *>(o_row + j) = acc;
                } else {
                    if (j + 0 < D) o_row[j + 0] = acc.x;
                    if (j + 1 < D) o_row[j + 1] = acc.y;
                    if (j + 2 < D) o_row[j + 2] = acc.z;
                }
            } else {
                o_row[c] = acc.x;
            }
        }
    }
}

// One pooling launch per lane class present among the tables.
static hipError_t launch_pool_classes(const Plan &p, const int64_t *offsets, float *out, int skip_mfma,
                                      hipStream_t s)
{
    if (p.B <= 0) return hipSuccess;
    for (int c = 0; c < 16; ++c) {
        if (!(p.gcls_mask & (1 << c))) continue;
        const int lpr = 1 << (c & 7), G = 64 / lpr;
        const int64_t gx = (p.B + (int64_t)G * (kThreads / 64) - 1) / ((int64_t)G * (kThreads / 64));
        const dim3 grid((unsigned)gx, (unsigned)p.T), block(kThreads);
#define TT_POOL(L, V) hipLaunchKernelGGL((k_pool<L, V>), grid, block, 0, s, p.dtab, p.B, offsets, p.nnz, p.ws, out, \
                                         p.sumD, c, skip_mfma)
        switch (c) {
        case 0: TT_POOL(1, false); break;
        case 1: TT_POOL(2, false); break;
        case 2: TT_POOL(4, false); break;
        case 3: TT_POOL(8, false); break;
        case 4: TT_POOL(16, false); break;
        case 5: TT_POOL(32, false); break;
        case 6: TT_POOL(64, false); break;
        case 8: TT_POOL(1, true); break;
        case 9: TT_POOL(2, true); break;
        case 10: TT_POOL(4, true); break;
        case 11: TT_POOL(8, true); break;
        case 12: TT_POOL(16, true); break;
        case 13: TT_POOL(32, true); break;
        case 14: TT_POOL(64, true); break;
        default: return hipErrorInvalidValue;
        }
#undef TT_POOL
    }
    return hipGetLastError();
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
            bag = ws.lb[l];
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
    return launch_pool_classes(p, offsets, out, 0, s);
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
        // workers of each class's persistent launch: waves of the per-wave
        // kernel (ranks <= 32, deterministic pooling), blocks otherwise
        // (ranks 8, 16 and 32: waves of the per-wave kernel; rank 64: blocks of
        // the tile-pipelined kernel; fused pooling: blocks of k_contract)
        ClassGrid cg;
        const int wpc[4] = {fwd_workers_per_cu<8>(), fwd_workers_per_cu<16>(), FwdT<32>::OCC,
                            FwdT<64>::OCC};
        for (int c = 0; c < 4; ++c) cg.nb[c] = p.num_blocks * (!fused ? wpc[c] : kClsOcc[c]);
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
                } else if (c < 2) {
#define TT_FWD_WAVE(RR, SS) hipLaunchKernelGGL((k_contract_w<RR, SS>), dim3(p.num_blocks * FwdW<RR>::OCC), block, 0, s, ac, hs)
#define TT_FWD_WAVES(RR) if (ac.sched != kSchedStatic) TT_FWD_WAVE(RR, true); else TT_FWD_WAVE(RR, false)
                    if (c == 0) TT_FWD_WAVES(8);
                    else TT_FWD_WAVES(16);
#undef TT_FWD_WAVES
#undef TT_FWD_WAVE
                } else {
                    // ranks 32 and 64: the tile-pipelined block kernel, also when it
                    // keeps C for the backward (measured on the 26-table training
                    // step: rank 64 0.97 ms against 1.10 for the block-cooperative
                    // kernel k_contract; rank 32 0.14 against 0.17 ms, and 0.30
                    // against 0.30 on the 26-table forward, for the per-wave kernel)
                    const bool steal = ac.sched != kSchedStatic;
#define TT_FWD_TILE(RR, KK, SS) hipLaunchKernelGGL((k_contract_t<RR, KK, SS>), dim3(p.num_blocks * FwdT<RR>::OCC), block, 0, s, ac, hs)
#define TT_FWD_TILES(RR) if (p.keep_c) { if (steal) TT_FWD_TILE(RR, true, true); else TT_FWD_TILE(RR, true, false); } \
                         else if (steal) TT_FWD_TILE(RR, false, true); else TT_FWD_TILE(RR, false, false)
                    if (c == 2) { TT_FWD_TILES(32); }
                    else { TT_FWD_TILES(64); }
#undef TT_FWD_TILES
#undef TT_FWD_TILE
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
        hipError_t e = launch_pool_classes(p, offsets, out, fused ? 1 : 0, s);
        if (e != hipSuccess) return e;
    }
    timer_end(p.timing, TM_POOL, s);
    return hipGetLastError();
}

} // namespace ttemb
