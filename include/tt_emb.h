/*
 * tt_emb.h -- C ABI of the MI355X (gfx950) TT-EmbeddingBag library, libtt_emb.so.
 *
 * The operator is an EmbeddingBag with sum pooling whose rows are rebuilt from
 * tensor-train cores ("TT-Rec: Tensor Train Compression for Deep Learning
 * Recommendation Models", abstract: TT-EmbeddingBag), evaluated the way the
 * FlowTT page ("FlowTT: Exploiting Computation Flow Reuse in Irregular
 * Tensor-Train Embedding") describes: lookups are grouped by the shared
 * high-order mixed-radix digits of their row (section 3.3), each group's prefix
 * intermediate C = G1[i1].G2[i2] is computed once and kept on chip, every row
 * of the group is E = C.G3[i3], rows are pooled per bag (section 3.2), and the
 * work runs on persistent blocks with chunk stealing and L2 checkpoints of
 * prefix intermediates (section 3.4).  The backward reverses the contraction
 * (section 3.2).
 *
 * Conventions (the pages leave these open; the choices are the plainest ones):
 *  - table t has N_t rows factored as n = (n1, n2, n3), n1*n2*n3 >= N_t, and
 *    D_t = d1*d2*d3 columns; TT ranks R = (1, R1, R2, 1);
 *  - row index digits are big-endian: i = (i1*n2 + i2)*n3 + i3; the prefix of
 *    a row is (i1, i2), i.e. q = i div n3;
 *  - core k of table t is fp32, row-major [n_k][R_{k-1}][d_k][R_k];
 *  - output column j = (j1*d2 + j2)*d3 + j3;
 *  - indices and offsets are int64; offsets are table-major CSR with T*B+1
 *    entries (offsets[0] = 0, non-decreasing, offsets[T*B] = nnz); bag (t, b)
 *    is indices[offsets[t*B+b] .. offsets[t*B+b+1]); an empty bag pools to 0;
 *    lookups need bags: nnz > 0 with B = 0 is TT_EMB_ERR_ARG;
 *  - out is fp32 [B][sum_t D_t], bag-major, tables concatenated in order;
 *  - valid rows are 0 <= i < N_t; anything else is an index error.
 *
 * Ownership and ordering: the caller owns every device buffer (cores, indices,
 * offsets, out, gradients, workspace).  The handle owns host metadata and a
 * small device copy of the table descriptors made at create time.  Forward,
 * backward and the update never allocate memory and never synchronise the
 * host: all work is enqueued on the given stream (a hipStream_t passed as
 * void*, NULL = the default stream).  Concurrent calls on one handle need
 * distinct workspaces.
 *
 * Errors: argument errors the host can see are returned synchronously and
 * nothing is enqueued.  Errors only the device can see (an index out of range,
 * malformed offsets) set a flag in the workspace; tt_emb_poll_error reports
 * it.  After such an error the outputs are unspecified but every kernel stays
 * in bounds.  No C++ exception crosses this interface.
 */
#ifndef TT_EMB_H
#define TT_EMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tt_emb *tt_emb_t;

enum {
    TT_EMB_OK = 0,
    TT_EMB_ERR_ARG = -1,         /* bad argument (null pointer, bad size or shape) */
    TT_EMB_ERR_INDEX = -2,       /* an index outside [0, N_t) (device-detected) */
    TT_EMB_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    TT_EMB_ERR_UNSUPPORTED = -4, /* shape outside what this build supports */
    TT_EMB_ERR_HIP = -5,         /* a HIP runtime call failed */
    TT_EMB_ERR_NOMEM = -6,       /* host or create-time device allocation failed */
    TT_EMB_ERR_OFFSETS = -7,     /* malformed offsets (device-detected) */
    TT_EMB_ERR_TOO_LARGE = -8    /* input needs more than tt_emb_forward_noalloc's fixed scratch */
};

/* Scheduling of the persistent contraction kernel (FlowTT section 3.4 and the
 * scheduling ablation of section 4). */
enum {
    TT_EMB_SCHED_DEFAULT = 0,  /* per rank class: STATIC for ranks 8, 16 and 32, STEAL for
                                  rank 64 (the fastest of each, measured) */
    TT_EMB_SCHED_STATIC = 1,   /* each block runs only its static range of chunks */
    TT_EMB_SCHED_STEAL = 2,    /* static range first, then steal chunks of blocks on the same
                                  XCD (grids a multiple of 8 blocks; otherwise of any block);
                                  no checkpoints */
    TT_EMB_SCHED_STEAL_L2 = 3  /* stealing plus L2 checkpoints of split prefix tiles */
};

/* Reuse granularity (FlowTT section 4, prefix reuse vs. exact deduplication). */
enum {
    TT_EMB_GROUP_DEFAULT = 0,    /* = PREFIX */
    TT_EMB_GROUP_PREFIX = 1,     /* one prefix intermediate per (table, i1, i2) */
    TT_EMB_GROUP_UNIQUE_ONLY = 2 /* one prefix intermediate per unique row */
};

/* Options; a zeroed struct (or NULL) selects the defaults. */
typedef struct {
    int32_t sched_mode;    /* TT_EMB_SCHED_* */
    int32_t group_mode;    /* TT_EMB_GROUP_* */
    int32_t chunk_rows;    /* max rows per forward work chunk, 1..32 (0 = 32) */
    int32_t num_blocks;    /* persistent grid size (0 = one block per compute unit) */
    int32_t check_indices; /* 0 = on (default), 1 = on, -1 = off (caller guarantees) */
    int32_t force_generic; /* 1 = use the plain (non-MFMA) contraction kernels (testing) */
    int32_t keep_prefix;   /* 1 = the workspace also has room for the prefix intermediates
                              C_p of the matrix-core tables (TT_EMB_KEEP_PREFIX and
                              TT_EMB_REUSE_PREFIX below); 0 = no room, flags rejected */
    int32_t reserved;
} tt_emb_options;

/* tt_emb_forward / tt_emb_backward flags. */
#define TT_EMB_REUSE_GROUPING 1u /* ws already holds the grouping of these exact
                                    (indices, offsets, B, nnz); skip rebuilding it */
/* Training mode (FlowTT section 3.2: the backward reverses the forward's
 * contraction flow).  TT_EMB_KEEP_PREFIX (forward): also store every prefix
 * unit's C_p = G1[i1] . G2[i2] of the matrix-core tables of rank >= 32 in ws
 * (smaller ranks recompute it: cheaper than storing and reading it).
 * TT_EMB_REUSE_PREFIX (backward): read C_p from ws instead of recomputing it;
 * valid only with TT_EMB_REUSE_GROUPING, after a forward on the same ws, the
 * same grouping and the same cores with TT_EMB_KEEP_PREFIX (the caller
 * asserts this, as with the grouping).  Both need a handle created with
 * keep_prefix = 1, else TT_EMB_ERR_ARG (checked before any device work).
 * The backward's gradients then use the forward's C_p, which the forward sums
 * over r1 in one chain where the recomputing backward uses two: results
 * agree to rounding, not bit for bit, and each path is itself deterministic. */
#define TT_EMB_KEEP_PREFIX 2u
#define TT_EMB_REUSE_PREFIX 4u
/* Forward: fused pooling with float atomics (FlowTT section 3.2 pools inside
 * the contraction, batching in on-chip memory and adding into the output with
 * atomics).  Each unique row, still on chip, is added into the bag of every
 * lookup of it; out is zeroed first.  The summation order then depends on
 * scheduling, so the output is NOT bit-reproducible (within fp32 rounding of
 * the deterministic path); the default bag-major pooling is.  Not with
 * TT_EMB_KEEP_PREFIX (TT_EMB_ERR_ARG). */
#define TT_EMB_ATOMIC_POOL 8u

/* Device pointers to the grouping arrays held in a workspace (for tests and
 * tools), all int32, ids global over tables in table order:
 *  perm[nnz]          lookup positions sorted by (table, row, position);
 *  uniq_row[U]        row of each unique (table, row);
 *  uniq_start[U+1]    start of each unique row's run in perm;
 *  inv[nnz]           position -> unique id;
 *  grp_prefix[G]      prefix q = row div n3 of each group;
 *  grp_start[G+1]     first unique id of each group;
 *  tab_uniq_start[T+1], tab_grp_start[T+1]  per-table starts. */
typedef struct {
    int64_t nnz, num_unique, num_groups;
    const int32_t *perm, *uniq_row, *uniq_start, *inv, *grp_prefix, *grp_start;
    const int32_t *tab_uniq_start, *tab_grp_start;
    int64_t num_units, num_tiles, num_chunks, num_split_tiles;
    /* scheduling statistics of the last forward contraction */
    int64_t num_steals, num_ckpt_hits, num_ckpt_misses;
} tt_emb_grouping;

/* Create a handle for T tables (FlowTT section 2.4 problem statement: a TT
 * gather over sequential core contractions).  num_rows[T] = N_t; n[3T], d[3T]
 * = row and column factors; R[4T] = ranks with R0 = R3 = 1.  All are host
 * arrays, copied.  Returns TT_EMB_ERR_ARG for inconsistent shapes and
 * TT_EMB_ERR_UNSUPPORTED beyond this build's limits (T <= 64, sum N_t <= 2^31 - 2,
 * ranks <= 256, D_t <= 1024).  *out receives the handle. */
int tt_emb_create(int32_t T, const int64_t *num_rows, const int32_t *n, const int32_t *d,
                  const int32_t *R, const tt_emb_options *opt, tt_emb_t *out);

/* Tables of K TT cores, K = 3 .. 8, the same K for every table (FlowTT
 * section 2.4 states the lookup as sequential TT-core contractions; section
 * 3.3 reuses the intermediate of rows sharing their leading digits -- here
 * at every prefix length).  n, d are host [T][K] arrays, R is [T][K+1] with
 * R_0 = R_K = 1; core k is [n_k][R_k][d_k][R_{k+1}]; digits are big-endian
 * (i = ((i_0 n_1 + i_1) n_2 + ...) n_{K-1} + i_{K-1}) and so are output
 * columns.  K = 3 is exactly tt_emb_create.  For K >= 4 the forward takes a
 * host array of T*K core pointers and computes every distinct prefix of
 * length 2 .. K-1 once (plain fp32, no matrix cores).  tt_emb_backward takes
 * the same T*K core pointers and T*K gradient pointers (overwritten, shaped
 * like the cores): the chain is reversed with the same prefix sharing, each
 * group's intermediate gradient formed once from its children, and every core
 * slice's gradient summed from per-row / per-group partials in a fixed order
 * (no atomics, bit-reproducible); tt_emb_sgd_update updates the T*K cores.
 * The forward leaves every prefix intermediate in ws: a backward with
 * TT_EMB_REUSE_GROUPING | TT_EMB_REUSE_PREFIX right after a forward on the
 * same ws, grouping and cores uses them instead of recomputing (REUSE_PREFIX
 * alone gives TT_EMB_ERR_ARG).  The forward flags TT_EMB_KEEP_PREFIX /
 * TT_EMB_ATOMIC_POOL give TT_EMB_ERR_ARG.  Beyond the
 * three-core limits: TT_EMB_ERR_UNSUPPORTED when T*K > 192, K = 2, K > 8,
 * the leading K-1 digits of all tables span 2^31 or more prefixes, the
 * product n_1 .. n_{K-1} of some table exceeds 2^32 - 1, some n_k summed
 * over the tables exceeds 2^30 - 1, or an
 * intermediate or core slice of some level exceeds 8192 floats; K < 2 is
 * TT_EMB_ERR_ARG.  The grouping view of such a handle groups unique rows by
 * their leading K-1 digits (grp_prefix = row div n_{K-1}). */
int tt_emb_create_k(int32_t T, int32_t K, const int64_t *num_rows, const int32_t *n, const int32_t *d,
                    const int32_t *R, const tt_emb_options *opt, tt_emb_t *out);

/* Release a handle (NULL is accepted). */
int tt_emb_destroy(tt_emb_t h);

/* Bytes of device workspace that forward + backward need for B bags per table
 * and nnz lookups (an upper bound that does not depend on the index values). */
int tt_emb_workspace_size(tt_emb_t h, int64_t B, int64_t nnz, size_t *bytes);

/* Bytes of device workspace that an inference-only caller needs: the
 * grouping and a forward without TT_EMB_KEEP_PREFIX (the FlowTT page,
 * Abstract and Conclusion, reports the method's inference peak memory).  A
 * workspace of this size (smaller than tt_emb_workspace_size's) is accepted
 * by tt_emb_group, tt_emb_forward without TT_EMB_KEEP_PREFIX,
 * tt_emb_grouping_view, tt_emb_block_stats and tt_emb_poll_error; the
 * backward and a forward with TT_EMB_KEEP_PREFIX return TT_EMB_ERR_WORKSPACE
 * on it.  The forward part is a prefix of the full layout, so a full
 * workspace serves both. */
int tt_emb_forward_workspace_size(tt_emb_t h, int64_t B, int64_t nnz, size_t *bytes);

/* Build the grouping of (indices, offsets) into ws: validation and key build,
 * stable radix sort by (table, row), unique extraction, prefix run-length
 * encoding and the work list (FlowTT section 4, grouping breakdown). */
int tt_emb_group(tt_emb_t h, const int64_t *indices, const int64_t *offsets, int64_t B,
                 int64_t nnz, void *ws, size_t ws_bytes, void *stream);

/* Pooled forward (FlowTT section 3.2: C = A.B, E = C.D, then pooling).
 * cores: HOST array of 3T device pointers (G1_0, G2_0, G3_0, G1_1, ...);
 * indices [nnz], offsets [T*B+1] int64 device; out fp32 [B][sum D] device,
 * fully overwritten.  Builds the grouping first unless
 * flags & TT_EMB_REUSE_GROUPING. */
int tt_emb_forward(tt_emb_t h, const float *const *cores, const int64_t *indices,
                   const int64_t *offsets, int64_t B, int64_t nnz, float *out, void *ws,
                   size_t ws_bytes, uint32_t flags, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * forward of tt_emb_forward (same kernels, same results bit for bit) with no
 * workspace argument.  Its scratch is a fixed device array of
 * TT_EMB_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; the call itself allocates nothing (no hipMalloc, no
 * allocating library routine).  The input must fit: when the forward
 * workspace for (B, nnz) (tt_emb_forward_workspace_size) exceeds the array,
 * returns TT_EMB_ERR_TOO_LARGE without launching anything.  flags:
 * TT_EMB_REUSE_GROUPING (the array still holds the grouping of the same
 * indices and offsets from the previous call on this GPU) and
 * TT_EMB_ATOMIC_POOL; TT_EMB_KEEP_PREFIX is TT_EMB_ERR_ARG.  Every call on a
 * GPU shares that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (other streams, other threads, other handles) race
 * and must be serialised by the caller; tt_emb_poll_error does not apply
 * (device-detected errors of this call are not reported). */
#define TT_EMB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int tt_emb_forward_noalloc(tt_emb_t h, const float *const *cores, const int64_t *indices,
                           const int64_t *offsets, int64_t B, int64_t nnz, float *out, uint32_t flags,
                           void *stream);

/* Backward of out = forward(cores) for the loss sum(grad_out * out) (FlowTT
 * section 3.2: the backward reverses the forward).  grad_out fp32 [B][sum D]
 * device; core_grads: HOST array of 3T device pointers, each shaped like its
 * core and fully OVERWRITTEN (slices no lookup touches become 0).  The core
 * gradients are reduced in a fixed order with no floating-point atomics, so
 * results are bit-reproducible run to run. */
int tt_emb_backward(tt_emb_t h, const float *grad_out, const float *const *cores,
                    const int64_t *indices, const int64_t *offsets, int64_t B, int64_t nnz,
                    float *const *core_grads, void *ws, size_t ws_bytes, uint32_t flags,
                    void *stream);

/* In-place SGD step G_k <- G_k - lr * dG_k on every core (the training step
 * of the benchmark workloads).  Both arrays are HOST arrays of 3T device
 * pointers. */
int tt_emb_sgd_update(tt_emb_t h, float *const *cores, const float *const *core_grads,
                      float lr, void *stream);

/* Synchronise the stream, then fill *view with device pointers into ws and
 * the counts it holds (tests and tools only). */
int tt_emb_grouping_view(tt_emb_t h, const void *ws, size_t ws_bytes, int64_t B, int64_t nnz,
                         void *stream, tt_emb_grouping *view);

/* Per-block scheduling records of the persistent matrix-core kernels: the
 * evidence for how evenly the work-stealing scheduler (FlowTT section 3.4,
 * persistent blocks with chunk stealing; section 4 reports the load
 * imbalance it removes) spreads one launch over blocks and compute units.
 * kernel: 0..3 = forward contraction of the rank-8/16/32/64 tables,
 * 4..7 = backward contraction of the same classes.  Each record holds the
 * block's start and end on the device's constant-rate wall clock
 * (t_start, t_end in ticks of *clock_khz kHz), the chunks (forward) or
 * (table, i2) runs (backward) it processed (work), the unique rows
 * (forward) or chunks (backward) in them (rows), the compute unit it ran on
 * (cu: xcc id << 7 | shader engine << 5 | cu id << 1 | shader array) and
 * the grid size.
 * Synchronises the stream, then copies min(grid, cap, 2048) records of the
 * last launch of that kernel on this workspace into the host array out
 * (caller-owned) and sets *nblocks to that count (0 when the kernel has not
 * run since the last grouping of ws, or the last forward (kernels 0..3) or
 * backward (4..7) did not launch it; always 0 for K >= 4 cores).  Tools and
 * tests only; TT_EMB_ERR_ARG for a bad kernel id or null pointers. */
typedef struct {
    int64_t t_start, t_end;
    int32_t work, rows, cu, grid;
} tt_emb_block_stat;
int tt_emb_block_stats(tt_emb_t h, const void *ws, size_t ws_bytes, int64_t B, int64_t nnz, int32_t kernel,
                       void *stream, tt_emb_block_stat *out, int32_t cap, int32_t *nblocks,
                       int64_t *clock_khz);

/* Victim order of the persistent kernels' chunk stealing (FlowTT section 3.4:
 * a block that has finished its own range takes chunks from others).  For a
 * grid of nb blocks (nb a positive multiple of 8, as every persistent launch
 * of this library is: blocks per CU times a multiple of 8 CUs) writes
 * order[vi] = the vi-th block whose range block `me` claims from, vi = 0 ..
 * nb-1 (caller-owned host array of nb entries): itself first, then the blocks
 * of its own XCD, then those of the other XCDs.  The kernels use the same
 * function; host only, no device work.  TT_EMB_ERR_ARG for a null array,
 * nb < 8, nb not a multiple of 8, or me outside [0, nb). */
int tt_emb_victim_order(int32_t me, int32_t nb, int32_t *order);

/* Measurement aid (not part of the hot path): launches `blocks` blocks of
 * four waves, each wave running eight independent chains of `iters` FP32
 * matrix-core instructions (v_mfma_f32_16x16x4_f32, 2048 flops each) with no
 * memory traffic, and writes one float per block to out (device, caller-owned,
 * `blocks` floats).  Timing it on the stream gives the device's measured FP32
 * matrix peak: blocks * 4 * 8 * iters * 2048 flops per launch.  Stream-ordered,
 * no synchronisation; TT_EMB_ERR_ARG for non-positive sizes or a null out. */
int tt_emb_peak_mfma(int32_t blocks, int32_t iters, float *out, void *stream);

/* Synchronise the stream and report a device-detected error recorded in ws
 * since the last grouping (TT_EMB_OK, TT_EMB_ERR_INDEX or TT_EMB_ERR_OFFSETS). */
int tt_emb_poll_error(tt_emb_t h, const void *ws, void *stream);

/* Static text for a status code. */
const char *tt_emb_status_string(int status);

/* Phase timers (tracing of the grouping / contraction / pooling / backward
 * breakdown the FlowTT page reports in section 4).  When enabled, every call
 * records a pair of hipEvents around each phase on the caller's stream. */
enum {
    TT_EMB_TIMER_GROUP_SORT = 0, /* validation, key build and radix sort */
    TT_EMB_TIMER_GROUP_RLE,      /* unique extraction, prefix RLE, work list */
    TT_EMB_TIMER_CONTRACT,       /* fused prefix-shared contraction (E rows) */
    TT_EMB_TIMER_POOL,           /* bag pooling */
    TT_EMB_TIMER_BWD_GATHER,     /* per-row output-gradient gather */
    TT_EMB_TIMER_BWD_CONTRACT,   /* reverse contraction per (table, i2) run */
    TT_EMB_TIMER_BWD_REDUCE,     /* fixed-order dG1 / dG3 reductions */
    TT_EMB_TIMER_SGD,            /* in-place SGD update */
    /* single kernels inside CONTRACT and BWD_CONTRACT: the matrix-core
     * contraction of the tables of rank 8, 16, 32 and 64 (R1 = R2, d1, d2 <= 4,
     * d3 <= 16); one interval per launch */
    TT_EMB_TIMER_FWD_R8, TT_EMB_TIMER_FWD_R16, TT_EMB_TIMER_FWD_R32, TT_EMB_TIMER_FWD_R64,
    TT_EMB_TIMER_BWD_R8, TT_EMB_TIMER_BWD_R16, TT_EMB_TIMER_BWD_R32, TT_EMB_TIMER_BWD_R64,
    /* stages inside GROUP_SORT and GROUP_RLE (the grouping overhead the
     * FlowTT page breaks down in section 4): validation and key build, the
     * (table, row) sort, unique extraction, mixed-radix prefix extraction and
     * run-length encoding, the (table, i2) unit order, and the work list */
    TT_EMB_TIMER_STAGE_DECODE, TT_EMB_TIMER_STAGE_SORT, TT_EMB_TIMER_STAGE_UNIQUE,
    TT_EMB_TIMER_STAGE_PREFIX, TT_EMB_TIMER_STAGE_ORDER, TT_EMB_TIMER_STAGE_WORKLIST,
    TT_EMB_NUM_TIMERS
};

/* enable != 0 creates the events (up to 1024 calls are kept per timer);
 * enable == 0 stops recording.  Host-side only; allocates events. */
int tt_emb_timing_enable(tt_emb_t h, int32_t enable);

/* Synchronise the device, then add up the recorded intervals:
 * ms[TT_EMB_NUM_TIMERS] total milliseconds, count[TT_EMB_NUM_TIMERS] recorded
 * intervals per timer (either pointer may be NULL); clears the records. */
int tt_emb_timing_read(tt_emb_t h, double *ms, int32_t *count);

/* Static name of a timer id (NULL if out of range). */
const char *tt_emb_timer_name(int32_t id);

#ifdef __cplusplus
}
#endif

#endif /* TT_EMB_H */
