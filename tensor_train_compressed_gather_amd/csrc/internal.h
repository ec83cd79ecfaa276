// internal.h -- shared definitions of the gfx950 TT-EmbeddingBag library.
//
// Data layout in device memory (all caller-owned except the table
// descriptors):
//   cores     fp32 [n_k][R_{k-1}][d_k][R_k] per table and core
//   indices   int64 [nnz], offsets int64 [T*B+1] (table-major CSR)
//   out       fp32 [B][sum_t D_t]
//   workspace one caller buffer carved into the regions of WsLayout.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ttemb {

constexpr int kMaxTables = 64;
constexpr int kThreads = 256;       // threads per block for every kernel
constexpr int kScanBlocks = 4096;   // blocks of the 3-phase scans (at most)
constexpr int kSortTile = 4096;     // keys per radix-sort block (256 threads x 16)
constexpr int kSortItems = kSortTile / kThreads;
// Radix-sort blocks (tiles) for n keys, a multiple of 8 so that tiles can be
// laid out XCD by XCD.
inline int64_t sort_blocks(int64_t n) { return ((n > 0 ? (n + kSortTile - 1) / kSortTile : 1) + 7) & ~int64_t(7); }
constexpr int kMaxCkptSlots = 4096; // L2 checkpoint slots for split prefix tiles
constexpr int kUnitsPerTile = 4;    // prefix units sharing (table, i2) per tile
constexpr int kGuTask = 256;        // sorted lookup positions per gradient-gather task
constexpr int kGuBatch = 32;        // positions whose grad_out rows a gather worker has in flight
constexpr int kGuCols = 64;         // columns of one gradient-gather piece (256 bytes: two lines)
constexpr int kGuBlocksPerCu = 2;   // gradient-gather blocks per compute unit
constexpr int kPieceTiles = 8;      // least tiles per piece of a split backward run
constexpr int kSplitMaxCls = 2;     // runs of the rank classes 8, 16, 32 may be split
constexpr int kMaxG2Slots = 32768;  // dG2 partial slots (pieces of split runs)
constexpr int kG2PStride = 32 * 4 * 32; // floats per slot: R1 * d2 * R2 of a splittable table

// Control words at the head of the workspace.
enum CtrlSlot {
    CTRL_ERR = 0,     // error bits (ERRB_*)
    CTRL_U = 1,       // unique rows
    CTRL_G = 2,       // prefix groups
    CTRL_UNITS = 3,   // work units (groups, or unique rows in UNIQUE_ONLY mode)
    CTRL_RUNS = 4,    // runs of units sharing (table, i2)
    CTRL_TILES = 5,   // tiles of <= 4 units
    CTRL_CHUNKS = 6,  // forward work chunks
    CTRL_SPLIT = 7,   // tiles split over several chunks
    CTRL_STEALS = 9,  // chunks taken from another block's range (statistics)
    CTRL_CKPT_HIT = 10,  // split-tile chunks that found a published checkpoint
    CTRL_CKPT_MISS = 11, // split-tile chunks that recomputed the prefix tile
    CTRL_BWD_NEXT = 40,  // 4 words: next run of each class's backward contraction
    CTRL_CLS_START = 16, // 5 words: first chunk of each MFMA rank class (chunks are class-major)
    CTRL_RUN_CLS = 24,   // 6 words: first run of each class, then the run count
    CTRL_KLEV = 48,      // 8 words: groups of each prefix length (tables of K >= 4 cores)
    CTRL_PIECE_CLS = 32, // 6 words: first backward piece of each class, then the piece count
    CTRL_PIECE_TILES = 56, // tiles per piece of a split backward run
    CTRL_PIECES = 57,    // backward pieces
    CTRL_SLOTS = 58,     // dG2 partial slots of split runs
    CTRL_N = 64
};
enum ErrBits { ERRB_INDEX = 1, ERRB_OFFSETS = 2, ERRB_CAPACITY = 4 };

// Per-table descriptor, copied to the device at create time.
struct TableDesc {
    int64_t N;
    int32_t n1, n2, n3;
    int32_t d1, d2, d3;
    int32_t R1, R2;
    int32_t D;
    int32_t col_off;   // first column of this table in out
    uint32_t key_base; // sum of N over earlier tables (sort key = key_base + row)
    uint32_t i1_base;  // sum of n1 over earlier tables
    uint32_t i2_base;  // sum of n2 over earlier tables
    uint32_t i3_base;  // sum of n3 over earlier tables
    int32_t cls;       // MFMA rank class (0: R=8, 1: 16, 2: 32, 3: 64) or -1
    int32_t Dp;        // row stride of the unique-row buffer E (D rounded up to 4)
    int32_t gcls;      // gradient-gather class: log2(lanes per row) + 8 when rows move as float4
    int64_t g3t_off;   // offset of this table's transposed G3 copy ([n3][d3][R2]) in Ws::g3t
};

constexpr int kMaxChunkRows = 32; // rows per forward work chunk (upper limit)
constexpr int kMaxWorkersPerCu = 32; // persistent workers (blocks or waves) per CU of one forward class
constexpr int kSinkFloats = 8 * 4 * 256; // 8 float4 stores per thread of a 256-thread block
// Prefix intermediates are kept from forward to backward for the rank classes
// from this one up (ranks >= 32).  Measured: at rank 16 the forward's extra C
// stores cost what the backward's saved recompute gained.
constexpr int kKeepMinCls = 2;

// Context of one forward work chunk, built once per grouping (one 256-byte
// record so the persistent kernel fetches it with a single wave-wide load).
struct ChunkRec {
    int32_t tile, t, nu, rbeg, rend, slot, i2, cls;
    int32_t i1[4];      // first digit of each unit
    int32_t ustart[4];  // unique id of each unit's first row inside the chunk
    int32_t ccnt[4];    // rows of each unit inside the chunk
    int32_t pstart[5];  // prefix of output tiles (16/d3 rows each) per unit
    int32_t rowoff[5];  // prefix of ccnt
    int32_t nch;        // chunks of this chunk's tile
    int32_t ubeg;       // position of the tile's first unit in the work order
    int32_t i3[kMaxChunkRows]; // third digit of every row of the chunk
};
static_assert(sizeof(ChunkRec) == 256, "chunk record is one 256-byte line");

// What the forward class kernels need of a table, 16 dwords, rebuilt by every
// forward: a wave loads it with one dword per lane and reads fields with
// readlane, so no scalar memory load sits in the chunk loops.
struct FwdTab {
    const float *g1, *g2; // cores 0 and 1
    const float *g3t;     // transposed core 2, [n3][d3][R2]
    float *E;             // unique-row buffer of the table, indexed by unique id (ebase applied)
    float *Cg;            // kept prefix intermediates, indexed by work position (cbase applied)
    int32_t d1, d2, d3, i2_base, Dp, pad;
};
static_assert(sizeof(FwdTab) == 64, "table record is 16 dwords");
enum FwdTabField { FT_G1 = 0, FT_G2 = 2, FT_G3T = 4, FT_E = 6, FT_CG = 8, FT_D1 = 10, FT_D2 = 11, FT_D3 = 12,
                   FT_I2BASE = 13, FT_DP = 14 };

// Per-block record of the persistent matrix-core kernels (scheduling
// evidence: how the work of one launch spread over blocks and compute units).
// Kernel slots 0..3 are the forward rank classes, 4..7 the backward ones.
constexpr int kStatKernels = 8;
constexpr int kStatBlocks = 2048; // blocks past this many leave no record
struct BlockStat {
    int64_t t0, t1;  // wall clock (constant-rate counter) at block start / end
    int32_t work;    // chunks (forward) or (table, i2) runs (backward) processed
    int32_t rows;    // unique rows computed (forward) or chunks (backward)
    int32_t cu;      // compute unit the block ran on (XCC, SE and CU ids)
    int32_t nb;      // grid size of the launch; entry 0 is cleared before each launch
};
static_assert(sizeof(BlockStat) == 32, "block record is 32 bytes");

struct CorePtrs {
    const float *g[kMaxTables][3];
};
struct GradPtrs {
    float *g[kMaxTables][3];
};

// Device views of the workspace regions (filled by the host plan).
struct Ws {
    int32_t *ctrl;
    uint32_t *keys0, *keys1;
    int32_t *vals0, *vals1;
    uint32_t *hist;     // radix histograms [radix][blocks]
    uint64_t *part;     // scan partials [kScanBlocks + 1]
    int32_t *tstart;    // [T+1] first lookup of each table (clamped offsets[t*B])
    // canonical grouping
    uint32_t *skeys;    // sorted keys [nnz]
    int32_t *perm;      // sorted positions [nnz]
    int32_t *inv;       // [nnz]
    uint32_t *ukey;     // key of each unique row [nnz]
    int32_t *uniq_row;  // [nnz]
    int32_t *uniq_start;// [nnz+1]
    int32_t *grp_prefix;// [nnz]
    int32_t *grp_start; // [nnz+1]
    int32_t *tab_uniq_start; // [T+1]
    int32_t *tab_grp_start;  // [T+1]
    int64_t *ebase;     // [T] element offset of table t's unique rows in E, minus tab_uniq_start*D
    int64_t *p3base;    // [T] same for the backward G3 partials
    // work units and the B-stationary work list
    int32_t *unit_prefix;    // [nnz]   (aliases grp_prefix in PREFIX mode)
    int32_t *unit_start;     // [nnz+1] (aliases grp_start in PREFIX mode)
    int32_t *tab_unit_start; // [T+1]
    uint32_t *ukey2;         // sorted (i2_base + i2) of units [nnz]
    int32_t *uorder;         // units in (table, i2, i1) order [nnz]
    int32_t *run_start;      // [nnz+1] into uorder
    int32_t *run_tile_start; // [nnz+1]
    int32_t *tile_ubeg;      // [nnz] into uorder
    int32_t *tile_nu;        // [nnz]
    int32_t *tile_rows;      // [nnz]
    int32_t *tile_slot;      // [nnz] checkpoint slot or -1
    int32_t *tile_cstart;    // [tiles+1] first chunk of each tile
    int32_t *uinv;           // [units] position of each unit in the work order
    int32_t *chunk_tile;     // [2*nnz]
    int32_t *chunk_rbeg;     // [2*nnz]
    int32_t *chunk_rend;     // [2*nnz]
    ChunkRec *crec;          // [chunk_cap]
    int64_t chunk_cap;       // capacity of the chunk arrays
    float *g3t;              // transposed G3 copies of the MFMA-class tables
    int32_t *heads;          // [num_blocks] queue heads
    int32_t *flags;          // [ckpt_slots] checkpoint ready flags
    float *ckpt;             // [ckpt_slots][4][16][max R2 + 4]
    int32_t ckpt_slots;      // min(kMaxCkptSlots, chunk bound of the workspace)
    float *E;                // unique rows, per-table segments
    float *Cg;               // kept prefix intermediates: [work position][16][R2] per table (keep_prefix)
    int64_t *cbase;          // [T] offset of table t's units in Cg, minus tab_unit_start[t]*16*R2
    float *sink;             // [kSinkFloats] scratch target of stores that carry no result
    struct FwdTab *ftab;     // [T] per-table pointers and shapes of the forward class kernels
    BlockStat *bstat;        // [kStatKernels][kStatBlocks] per-block scheduling records
    // backward
    int32_t *lb;             // [nnz] bag within its table of each lookup, in lookup order
    int2 *sm;                // [nnz] (bag within its table, unique row) of each sorted position
    int32_t *gu_ml;          // [gather tasks] unique row of the run cut at the task's left edge, or -1
    int32_t *gu_mr;          // [gather tasks] unique row of the run cut at its right edge, or -1
    // the partial sums of cut runs ([task][left, right][gstride]) live in P3's space
    float *P3;               // per-unique-row G3 partials
    float *G1P;              // per-unit G1 partials
    int32_t *g3rng;          // [2][sum n3] row range of each G3 slice in the (table, i3) order
    uint32_t *key3;          // sorted (i3_base + i3) of unique rows
    int32_t *u3order;        // unique rows in (table, i3, unique id) order
    // backward pieces: a (table, i2) run of the rank classes up to kSplitMaxCls
    // with more than CTRL_PIECE_TILES tiles is cut into tile-aligned pieces
    // whose dG2 partials (G2P slots) are summed in piece order afterwards
    int32_t *run_pbase;      // [runs + 1] first piece of each run
    int32_t *run_sbase;      // [runs + 1] first G2P slot of each run
    int32_t *piece_tb, *piece_te, *piece_slot; // [pieces] tile range, slot or -1
    float *G2P;              // [g2p_slots][kG2PStride] dG2 partials of split runs
    // backward claim order of the pieces: class-major, longest first
    uint32_t *rkey0, *rkey1;
    int32_t *rval0, *rval1;
    const int32_t *rorder;   // the sorted piece ids (one of rval0 / rval1, set at launch)
    // sort buffers of the unit order (kept apart from the canonical perm)
    int32_t *uvals0, *uvals1;
    int32_t *uvals_free; // the unit-sort value buffer that does not hold uorder
};

enum TimerId {
    TM_GROUP_SORT = 0, TM_GROUP_RLE, TM_CONTRACT, TM_POOL, TM_BWD_GATHER, TM_BWD_CONTRACT,
    TM_BWD_REDUCE, TM_SGD, TM_FWD_CLS0, TM_BWD_CLS0 = TM_FWD_CLS0 + 4, TM_STAGE_DECODE = TM_BWD_CLS0 + 4,
    TM_STAGE_SORT, TM_STAGE_UNIQUE, TM_STAGE_PREFIX, TM_STAGE_ORDER, TM_STAGE_WORKLIST, TM_COUNT
};
struct Timing; // host-side event rings (api.hip)
void timer_begin(Timing *tm, int id, hipStream_t s);
void timer_end(Timing *tm, int id, hipStream_t s);

// Tables of K >= 4 TT cores (one K per handle).  Core k of a table is
// [n_k][R_k][d_k][R_{k+1}] (R_0 = R_K = 1); digits are big-endian.
constexpr int kMaxK = 8;
constexpr int kMaxKPtrs = 3 * kMaxTables; // core pointers of a K-core handle, T * K of them
constexpr int kKLds = 8192;               // floats of each staged operand of a prefix level
struct KTab {
    int32_t K;
    int32_t n[kMaxK], d[kMaxK], R[kMaxK + 1];
    int64_t div[kMaxK]; // product of n_j over j > k: digit k = row / div[k] % n[k]
    int32_t P[kMaxK + 1]; // product of d_j over j < m: rows of the prefix-m intermediate
    int32_t nbase[kMaxK]; // sum of n_k over earlier tables (backward sort key of a core-k slice)
};
struct KCorePtrs {
    const float *g[kMaxKPtrs]; // table t, core k at t * K + k
};
struct KPlan {
    int K;
    const KTab *dkt;            // device copy, one per table
    int32_t *ugrp[kMaxK];       // prefix length m: [U] group of each unique row
    int32_t *gfirst[kMaxK];     // [U + 1] first unique row of each group
    float *V[kMaxK];            // [groups][smax[m]] prefix-m intermediates
    int64_t smax[kMaxK];        // floats per group of prefix length m
    // backward (prefix lengths m = 1 .. K-1; m = 1 groups share the first digit)
    float *dV[kMaxK];           // [groups][smax[m]] gradient of each group's intermediate
    float *Q[kMaxK];            // [groups][qmax[m]] core m-1 partial of each prefix-m group
    float *Cc[kMaxK];           // [groups][smax[m-1]] each prefix-m group's share of its parent's dV
    int64_t qmax[kMaxK];        // R_{m-1} * d_{m-1} * R_m, max over tables
    float *PK;                  // [unique rows][pkmax] last-core partial of each unique row
    int64_t pkmax;              // R_{K-1} * d_{K-1}, max over tables
    int key_bits[kMaxK];        // sort key bits of the core-k slices (sum over tables of n_k)
    float *red;                 // [n_k][16][slice] split sums of one (table, core) reduction
};

struct Plan {
    Timing *timing; // nullptr unless phase timing is enabled
    int32_t T;
    int64_t B, nnz;
    int num_blocks;
    int sched_mode, group_mode, chunk_rows, check_indices, force_generic;
    int keep_c, reuse_c; // forward stores C_p in Ws::Cg / backward reads it
    int pool_atomic;     // forward pools inside the contraction with float atomics
    KPlan kp;            // K >= 4 cores (kp.K == 0 for three-core handles)
    const int32_t *kp_n; // host copy of n_k of every table, [T*K] (K >= 4 cores)
    bool any_generic;
    int cls_mask; // bit c set when some table is in MFMA rank class c
    int gcls_mask; // bit c set when some table is in gradient-gather class c
    int key_bits, key2_bits, key3_bits;
    int Dmax, Dpmax, R2max, sumD;
    int sum_n[3]; // sum over tables of n1, n2, n3
    int g1stride; // row stride of the G1 partials (max d1*R1 over tables)
    int g2p_slots; // G2P slots in the workspace
    const TableDesc *dtab; // device copy
    Ws ws;
};

// ----------------------------------------------------------------- kernels
// Grouping (group.hip)
hipError_t launch_grouping(const Plan &p, const int64_t *indices, const int64_t *offsets,
                           hipStream_t s);
// Forward contraction and pooling (forward.hip)
hipError_t launch_forward(const Plan &p, const CorePtrs &cores, const int64_t *offsets, float *out,
                          hipStream_t s);
// Backward (backward.hip)
hipError_t launch_backward(const Plan &p, const float *grad_out, const CorePtrs &cores,
                           const int64_t *offsets, const GradPtrs &grads, hipStream_t s);
// Bag (within its table) of every lookup, Ws::lb.
hipError_t launch_lookup_meta(const Plan &p, const int64_t *offsets, hipStream_t s);
// Bag-major pooling of the unique rows of every table (forward.hip).
hipError_t launch_pool(const Plan &p, const int64_t *offsets, float *out, hipStream_t s);
// Forward of K >= 4 cores: every prefix length's intermediates, rows, pooling (kcores.hip).
hipError_t launch_forward_k(const Plan &p, const KCorePtrs &cores, const int64_t *offsets, float *out,
                            hipStream_t s);
// Backward of K >= 4 cores into core_grads [T*K] (kcores.hip).
hipError_t launch_backward_k(const Plan &p, const float *grad_out, const KCorePtrs &cores, const int64_t *offsets,
                             float *const *core_grads, hipStream_t s);
// Output-gradient rows g_u of every unique row into Ws::E (backward.hip).
hipError_t launch_gu_gather(const Plan &p, const float *grad_out, const int64_t *offsets, hipStream_t s);
// SGD and fills (misc.hip)
constexpr int kSgdMaxCores = 32; // cores per SGD launch (kernel-argument batch)
struct SgdBatch {
    int n;                       // cores in the batch
    int blk[kSgdMaxCores + 1];   // first block of each core
    float *g[kSgdMaxCores];
    const float *dg[kSgdMaxCores];
    int64_t cnt[kSgdMaxCores];
};
hipError_t launch_sgd(float *const *g, const float *const *dg, const int64_t *count, int ncores, float lr,
                      hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int32_t v, int64_t count, hipStream_t s);
hipError_t launch_fill_f32(float *p, float v, int64_t count, hipStream_t s);

// Shared radix sort of (u32 key, i32 value) pairs; n is an upper bound known on
// the host, n_dev (optional) the actual count on the device.
hipError_t radix_sort_pairs(const Plan &p, uint32_t *k0, int32_t *v0, uint32_t *k1, int32_t *v1,
                            int64_t n_max, const int32_t *n_dev, int bits, bool *result_in_1,
                            hipStream_t s);

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Victim order of the persistent kernels' work stealing: for a grid of nb
// blocks (nb a positive multiple of 8: blocks are dispatched round-robin over
// the 8 XCDs, so block b runs on XCD b mod 8), the vi-th victim of block me is
// its own range first, then the other blocks of its own XCD, then those of the
// other XCDs, one XCD after another.  For every such nb, vi -> victim is a
// permutation of the blocks with victim 0 = me, so each static range is
// claimed by its owner first and every range has a thief.
__host__ __device__ inline int victim_of(int me, int vi, int nb)
{
    const int per = nb >> 3;
    const int xo = vi / per, k = vi - xo * per;
    return ((me & 7) + xo) % 8 + 8 * (((me >> 3) + k) % per);
}

} // namespace ttemb
