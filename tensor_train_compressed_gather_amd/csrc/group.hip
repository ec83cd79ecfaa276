// group.hip -- index grouping on gfx950.
//
// Stage order follows the grouping breakdown of the FlowTT page ("FlowTT:
// Exploiting Computation Flow Reuse in Irregular Tensor-Train Embedding",
// section 4): index sorting, unique extraction, mixed-radix conversion,
// prefix extraction and run-length encoding; prefixes are the shared
// high-order row digits (section 3.3).  Everything is deterministic: a stable
// LSD radix sort and scans with a fixed block decomposition, so every output
// array is bit-exact against a plain stable sort.
//
// After the canonical arrays, the same pass builds the work list of the
// contraction: units (groups, or unique rows in the unique-only ablation)
// re-sorted stably by (table, i2) so that units sharing the second core slice
// are adjacent (the slice stays resident in registers), cut into tiles of at
// most four units and then into chunks of at most chunk_rows rows.
#include "primitives.h"

namespace ttemb {

// ------------------------------------------------------------- set-up

__global__ __launch_bounds__(kThreads) void k_init_ctrl(Ws ws, int T)
{
    for (int i = threadIdx.x; i < CTRL_N; i += blockDim.x) ws.ctrl[i] = 0;
    for (int i = threadIdx.x; i <= T; i += blockDim.x) {
        ws.tab_uniq_start[i] = 0;
        ws.tab_grp_start[i] = 0;
    }
    if (threadIdx.x == 0) {
        ws.uniq_start[0] = 0;
        ws.grp_start[0] = 0;
    }
    // no persistent launch has left records on this grouping yet
    if (threadIdx.x < kStatKernels) ws.bstat[threadIdx.x * kStatBlocks].nb = 0;
}

// Offsets must start at 0, never decrease and end at nnz.  Malformed offsets
// set ERRB_OFFSETS; every later kernel clamps ranges so it stays in bounds.
__global__ __launch_bounds__(kThreads) void k_check_offsets(const int64_t *offsets, int64_t nbags,
                                                            int64_t nnz, int64_t B, int T, Ws ws)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int bad = 0;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nbags; b += stride) {
        int64_t o0 = offsets[b], o1 = offsets[b + 1];
        if (o1 < o0 || o0 < 0 || o1 > nnz) bad = 1;
        if (b == 0 && o0 != 0) bad = 1;
        if (b == nbags - 1 && o1 != nnz) bad = 1;
    }
    if (__any(bad) && lane_id() == 0) atomicOr(&ws.ctrl[CTRL_ERR], (int)ERRB_OFFSETS);
    if (blockIdx.x == 0) {
        // table starts, clamped into [0, nnz] and made non-decreasing so the
        // table ranges never overlap even when the offsets are malformed
        __shared__ int32_t st[kMaxTables + 1];
        for (int t = threadIdx.x; t <= T; t += blockDim.x) {
            int64_t o = nbags > 0 ? offsets[(int64_t)t * B] : 0;
            if (t == T) o = nnz;
            o = o < 0 ? 0 : (o > nnz ? nnz : o);
            st[t] = (int32_t)o;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t m = 0;
            for (int t = 0; t <= T; ++t) {
                m = st[t] > m ? st[t] : m;
                ws.tstart[t] = m;
            }
        }
    }
}

// Range check and sort key (table base + row) of every lookup.
__global__ __launch_bounds__(kThreads) void k_decode(const int64_t *indices, int64_t nnz,
                                                     const TableDesc *tab, int T, int check, Ws ws)
{
    __shared__ int32_t st[kMaxTables + 1];
    __shared__ uint32_t kb[kMaxTables];
    __shared__ int64_t nrows[kMaxTables];
    for (int t = threadIdx.x; t <= T; t += blockDim.x) {
        st[t] = ws.tstart[t];
        if (t < T) {
            kb[t] = tab[t].key_base;
            nrows[t] = tab[t].N;
        }
    }
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int bad = 0;
    for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l < nnz; l += stride) {
        int t = segment_of(st, T, l);
        int64_t i = indices[l];
        if (i < 0 || i >= nrows[t]) {
            bad |= check;
            i = i < 0 ? 0 : nrows[t] - 1;
        }
        ws.keys0[l] = kb[t] + (uint32_t)i;
        ws.vals0[l] = (int32_t)l;
    }
    if (__any(bad) && lane_id() == 0) atomicOr(&ws.ctrl[CTRL_ERR], (int)ERRB_INDEX);
}

// -------------------------------------------------------- radix sort
//
// Stable LSD radix sort of (u32 key, i32 value), digits of at most 8 bits.  Per pass:
// per-block digit counts (upsweep), one exclusive scan of the digit-major
// count matrix, then a downsweep that ranks keys inside the block without
// breaking ties (each wave owns a contiguous quarter of the tile and keeps
// running per-digit counts) and writes runs of equal digits contiguously.

constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;

// Tile of this block for n keys: the tiles that hold keys are laid out XCD by
// XCD (the blocks of one XCD take consecutive tiles), so the partial lines a
// tile scatters into each digit's run meet those of its neighbour tiles in
// one L2 (measured: 0.70 -> 0.65 ms for the 17.9M-key sort).  Blocks past the
// keys keep their own (empty) tile.
__device__ __forceinline__ int sort_tile(int64_t n)
{
    const int nt = (int)(((n + kSortTile - 1) / kSortTile + 7) & ~int64_t(7));
    return (int)blockIdx.x < nt ? xcd_slot(blockIdx.x, nt) : (int)blockIdx.x;
}

__global__ __launch_bounds__(kThreads) void k_sort_upsweep(const uint32_t *keys, int64_t n_max,
                                                           const int32_t *n_dev, int shift, int dbits,
                                                           uint32_t *hist, int nblk)
{
    __shared__ uint32_t cnt[kRadix];
    for (int i = threadIdx.x; i < kRadix; i += kThreads) cnt[i] = 0;
    __syncthreads();
    const int64_t nd = n_dev ? (int64_t)*n_dev : n_max, n = nd < n_max ? nd : n_max; // never past the buffers
    const int tile = sort_tile(n);
    const int64_t base = (int64_t)tile * kSortTile;
    const uint32_t dmask = (1u << dbits) - 1u;
    if (base < n) {
        // every key of the thread in flight at once: unconditional loads from
        // clamped positions (a load under a condition is waited for before
        // the next one is issued), the range test applied when counting
        uint32_t kk[kSortItems];
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const int64_t i = base + j * kThreads + threadIdx.x;
            kk[j] = keys[i < n ? i : n - 1];
        }
#pragma unroll
        for (int j = 0; j < kSortItems; ++j)
            if (base + j * kThreads + threadIdx.x < n) atomicAdd(&cnt[(kk[j] >> shift) & dmask], 1u);
    }
    __syncthreads();
    for (int d = threadIdx.x; d <= (int)dmask; d += kThreads) hist[(int64_t)d * nblk + tile] = cnt[d];
}

struct HistScanOp {
    uint32_t *hist;
    int64_t n;
    __device__ int64_t count() const { return n; }
    __device__ uint64_t value(int64_t i) const { return hist[i]; }
    __device__ void emit(int64_t i, uint64_t excl, uint64_t) const { hist[i] = (uint32_t)excl; }
    __device__ void total(uint64_t, int64_t) const {}
};

template <int DB>
__global__ __launch_bounds__(kThreads) void k_sort_downsweep(const uint32_t *kin, const int32_t *vin,
                                                             uint32_t *kout, int32_t *vout,
                                                             int64_t n_max, const int32_t *n_dev,
                                                             int shift, const uint32_t *hist,
                                                             int nblk)
{
    constexpr int W = kThreads / 64;
    constexpr int SUB = kSortTile / W;    // keys per wave
    constexpr int ROUNDS = SUB / 64;
    __shared__ uint32_t wcnt[W][kRadix];
    __shared__ uint32_t dstart[kRadix];
    __shared__ uint32_t gbase[kRadix];
    __shared__ uint32_t skey[kSortTile];
    __shared__ int32_t sval[kSortTile];
    __shared__ uint32_t ssum[W];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t nd = n_dev ? (int64_t)*n_dev : n_max, n = nd < n_max ? nd : n_max; // never past the buffers
    const int tile = sort_tile(n); // as in the upsweep
    const int64_t base = (int64_t)tile * kSortTile;
    if (base >= n) return;
    for (int i = tid; i < W * kRadix; i += kThreads) (&wcnt[0][0])[i] = 0;
    constexpr uint32_t dmask = (1u << DB) - 1u;
    for (int d = tid; d <= (int)dmask; d += kThreads) gbase[d] = hist[(int64_t)d * nblk + tile];
    __syncthreads();

    uint32_t key[ROUNDS];
    int32_t val[ROUNDS];
    uint32_t rank[ROUNDS];
    const uint64_t lt = (1ull << lane) - 1ull;
    // the tile's keys and values all in flight at once: unconditional loads
    // from clamped positions (a load under a condition is waited for before
    // the next one is issued, one memory round trip per round)
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int64_t i = base + w * SUB + r * 64 + lane, ic = i < n ? i : n - 1;
        key[r] = kin[ic];
        val[r] = vin[ic];
    }
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const int64_t i = base + w * SUB + r * 64 + lane;
        const bool valid = i < n;
        const uint32_t k = valid ? key[r] : 0xffffffffu;
        const uint32_t d = (k >> shift) & dmask;
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const uint32_t below = (uint32_t)__popcll(m & lt);
        const uint32_t prior = wcnt[w][d];
        __builtin_amdgcn_wave_barrier();
        if (valid && below == 0) wcnt[w][d] = prior + (uint32_t)__popcll(m);
        __builtin_amdgcn_wave_barrier();
        key[r] = k;
        rank[r] = valid ? prior + below : 0xffffffffu;
    }
    __syncthreads();
    // wave prefixes per digit and the tile total of each digit
    uint32_t tot_d = 0;
    const int d0 = tid; // kRadix == kThreads
    {
        uint32_t s = 0;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) {
            uint32_t c = wcnt[ww][d0];
            wcnt[ww][d0] = s;
            s += c;
        }
        tot_d = s;
    }
    // exclusive scan of the digit totals -> tile-local digit starts
    {
        uint32_t x = wave_inclusive_scan(tot_d);
        if (lane == 63) ssum[w] = x;
        __syncthreads();
        uint32_t pre = 0;
        for (int ww = 0; ww < w; ++ww) pre += ssum[ww];
        dstart[d0] = pre + x - tot_d;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        if (rank[r] != 0xffffffffu) {
            const uint32_t d = (key[r] >> shift) & dmask;
            const uint32_t pos = dstart[d] + wcnt[w][d] + rank[r];
            skey[pos] = key[r];
            sval[pos] = val[r];
        }
    }
    __syncthreads();
    const int cnt = (int)((n - base) < kSortTile ? (n - base) : kSortTile);
    for (int j = tid; j < cnt; j += kThreads) {
        const uint32_t k = skey[j];
        const uint32_t d = (k >> shift) & dmask;
        const uint32_t o = gbase[d] + (uint32_t)j - dstart[d];
        kout[o] = k;
        vout[o] = sval[j];
    }
}

hipError_t radix_sort_pairs(const Plan &p, uint32_t *k0, int32_t *v0, uint32_t *k1, int32_t *v1,
                            int64_t n_max, const int32_t *n_dev, int bits, bool *result_in_1,
                            hipStream_t s)
{
    static_assert(kRadix == kThreads, "downsweep assumes one digit per thread");
    *result_in_1 = false;
    if (n_max <= 0 || bits <= 0) return hipSuccess;
    const int nblk = (int)sort_blocks(n_max);
    // passes of at most 8 bits, the bits spread evenly over them (28-bit keys:
    // 4 x 7 bits, so a 4096-key tile meets 128 digits, 32 keys each on average,
    // and writes whole 128-byte runs)
    const int passes = (bits + kRadixBits - 1) / kRadixBits;
    const int wd = (bits + passes - 1) / passes;
    uint32_t *kin = k0, *kout = k1;
    int32_t *vin = v0, *vout = v1;
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = pass * wd, dbits = bits - shift < wd ? bits - shift : wd;
        hipLaunchKernelGGL(k_sort_upsweep, dim3(nblk), dim3(kThreads), 0, s, kin, n_max, n_dev,
                           shift, dbits, p.ws.hist, nblk);
        HistScanOp op{p.ws.hist, ((int64_t)1 << dbits) * nblk};
        hipError_t e = run_scan(op, p.ws.part, scan_blocks(op.n), s);
        if (e != hipSuccess) return e;
        switch (dbits) {
#define TT_SORT_DOWN(DB)                                                                                   \
    case DB:                                                                                               \
        hipLaunchKernelGGL(k_sort_downsweep<DB>, dim3(nblk), dim3(kThreads), 0, s, kin, vin, kout, vout, n_max, \
                           n_dev, shift, p.ws.hist, nblk);                                                 \
        break;
            TT_SORT_DOWN(1) TT_SORT_DOWN(2) TT_SORT_DOWN(3) TT_SORT_DOWN(4)
            TT_SORT_DOWN(5) TT_SORT_DOWN(6) TT_SORT_DOWN(7) TT_SORT_DOWN(8)
#undef TT_SORT_DOWN
        default: return hipErrorInvalidValue;
        }
        uint32_t *tk = kin;
        kin = kout;
        kout = tk;
        int32_t *tv = vin;
        vin = vout;
        vout = tv;
    }
    *result_in_1 = (passes & 1) != 0;
    return hipGetLastError();
}

// ------------------------------------------------------ unique rows

struct UniqueOp {
    const uint32_t *sk;
    const int32_t *perm;
    Ws ws;
    int64_t n;
    __device__ int64_t count() const { return n; }
    __device__ uint64_t value(int64_t k) const
    {
        const uint32_t a = sk[k], b = sk[k > 0 ? k - 1 : 0]; // both loads unconditional
        return (k == 0 || a != b) ? 1 : 0;
    }
    // the sorted key and original position of element k, loaded before any emit
    __device__ int2 aux(int64_t k) const { return make_int2((int)sk[k], perm[k]); }
    __device__ void emit(int64_t k, uint64_t excl, uint64_t v, int2 ax) const
    {
        const int32_t uid = (int32_t)(excl + v) - 1;
        if (v) {
            ws.ukey[uid] = (uint32_t)ax.x;
            ws.uniq_start[uid] = (int32_t)k;
        }
        ws.inv[ax.y] = uid;
    }
    __device__ void total(uint64_t tot, int64_t nn) const
    {
        ws.ctrl[CTRL_U] = (int32_t)tot;
        ws.uniq_start[tot] = (int32_t)nn;
    }
};

// ------------------------------------------ mixed radix + prefix RLE

struct GroupOp {
    const TableDesc *tab;
    int T;
    Ws ws;
    __device__ int64_t count() const { return ws.ctrl[CTRL_U]; }
    __device__ void info(int64_t u, int *t, int32_t *row, int32_t *q) const
    {
        const uint32_t key = ws.ukey[u];
        *t = table_of_key(tab, T, key);
        *row = (int32_t)(key - tab[*t].key_base);
        *q = *row / tab[*t].n3;
    }
    // (table, row, prefix) of unique row u and the table of row u - 1 (-1 for
    // the first), read unconditionally (row 0 stands in for row -1)
    struct Aux {
        int t, tprev;
        int32_t row, q;
    };
    __device__ Aux aux(int64_t u) const
    {
        Aux g;
        int32_t r0, q0;
        info(u, &g.t, &g.row, &g.q);
        info(u > 0 ? u - 1 : 0, &g.tprev, &r0, &q0);
        g.tprev = u > 0 ? g.tprev : -1;
        return g;
    }
    __device__ uint64_t value(int64_t u) const
    {
        int t0, t1;
        int32_t r0, r1, q0, q1;
        info(u > 0 ? u - 1 : 0, &t0, &r0, &q0);
        info(u, &t1, &r1, &q1);
        return (u == 0 || t0 != t1 || q0 != q1) ? 1 : 0;
    }
    __device__ void emit(int64_t u, uint64_t excl, uint64_t v, const Aux &g) const
    {
        const int32_t gid = (int32_t)(excl + v) - 1;
        ws.uniq_row[u] = g.row;
        if (v) {
            ws.grp_prefix[gid] = g.q;
            ws.grp_start[gid] = (int32_t)u;
        }
        for (int tt = g.tprev + 1; tt <= g.t; ++tt) {
            ws.tab_uniq_start[tt] = (int32_t)u;
            ws.tab_grp_start[tt] = gid;
        }
    }
    __device__ void total(uint64_t tot, int64_t U) const
    {
        ws.ctrl[CTRL_G] = (int32_t)tot;
        ws.grp_start[tot] = (int32_t)U;
        int tl = -1;
        if (U > 0) tl = table_of_key(tab, T, ws.ukey[U - 1]);
        for (int tt = tl + 1; tt <= T; ++tt) {
            ws.tab_uniq_start[tt] = (int32_t)U;
            ws.tab_grp_start[tt] = (int32_t)tot;
        }
    }
};

// Work units in the unique-only ablation: every unique row is its own unit.
__global__ __launch_bounds__(kThreads) void k_units_unique(const TableDesc *tab, int T, Ws ws)
{
    const int64_t U = ws.ctrl[CTRL_U];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < U; u += stride) {
        const int t = segment_of(ws.tab_uniq_start, T, u);
        ws.unit_prefix[u] = ws.uniq_row[u] / tab[t].n3;
        ws.unit_start[u] = (int32_t)u;
    }
    if (blockIdx.x == 0) {
        for (int t = threadIdx.x; t <= T; t += blockDim.x) ws.tab_unit_start[t] = ws.tab_uniq_start[t];
        if (threadIdx.x == 0) {
            ws.unit_start[U] = (int32_t)U;
            ws.ctrl[CTRL_UNITS] = (int32_t)U;
        }
    }
}

// Per-table bases of the E rows and of the backward partial buffers.
__global__ __launch_bounds__(64) void k_finalize_bases(const TableDesc *tab, int T, int unique_only, Ws ws)
{
    // one lane per table reads its figures (all loads in flight together, none
    // behind a store); lane 0 then forms the running sums from LDS
    __shared__ int64_t su[kMaxTables], sn[kMaxTables], sunits[kMaxTables];
    __shared__ int sdp[kMaxTables], sp3[kMaxTables], scls[kMaxTables], sr2[kMaxTables];
    const int t = threadIdx.x;
    if (t < T) {
        const TableDesc &d = tab[t];
        su[t] = ws.tab_uniq_start[t];
        sn[t] = ws.tab_uniq_start[t + 1] - ws.tab_uniq_start[t];
        sunits[t] = ws.tab_unit_start[t + 1] - ws.tab_unit_start[t];
        sdp[t] = d.Dp;
        sp3[t] = d.R2 * d.d3;
        scls[t] = d.cls;
        sr2[t] = d.R2;
    }
    __syncthreads();
    if (t != 0) return;
    if (!unique_only) ws.ctrl[CTRL_UNITS] = ws.ctrl[CTRL_G];
    int64_t e = 0, p3 = 0;
    for (int k = 0; k < T; ++k) {
        ws.ebase[k] = e - su[k] * sdp[k];
        e += sn[k] * sdp[k];
        ws.p3base[k] = p3 - su[k] * (int64_t)sp3[k];
        p3 += sn[k] * (int64_t)sp3[k];
    }
    // kept prefix intermediates: 16 x R2 per unit of a table of the kept rank
    // classes, by position in the work order.  That order is class-major (tables grouped
    // by rank class, in table order within a class, as their i2 bases), so a
    // table's units are contiguous there but not at tab_unit_start.
    int64_t cg = 0, pos = 0;
    for (int c = 0; c <= 4; ++c)
        for (int k = 0; k < T; ++k) {
            if ((scls[k] < 0 ? 4 : scls[k]) != c) continue;
            const int64_t per = scls[k] >= kKeepMinCls ? 16 * (int64_t)sr2[k] : 0;
            ws.cbase[k] = cg - pos * per;
            cg += sunits[k] * per;
            pos += sunits[k];
        }
}

// ------------------------------------------------ B-stationary work list

__global__ __launch_bounds__(kThreads) void k_unit_keys(const TableDesc *tab, int T, Ws ws)
{
    const int64_t Un = ws.ctrl[CTRL_UNITS];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < Un; k += stride) {
        const int t = segment_of(ws.tab_unit_start, T, k);
        ws.keys0[k] = tab[t].i2_base + (uint32_t)(ws.unit_prefix[k] % tab[t].n2);
        ws.uvals0[k] = (int32_t)k;
    }
}

// Position of every unit in the work order.
__global__ __launch_bounds__(kThreads) void k_uinv(Ws ws, const int32_t *uo)
{
    const int64_t Un = ws.ctrl[CTRL_UNITS];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < Un; k += stride) ws.uinv[uo[k]] = (int32_t)k;
}

struct RunOp {
    const uint32_t *k2;
    Ws ws;
    __device__ int64_t count() const { return ws.ctrl[CTRL_UNITS]; }
    __device__ uint64_t value(int64_t k) const
    {
        const uint32_t a = k2[k], b = k2[k > 0 ? k - 1 : 0]; // both loads unconditional
        return (k == 0 || a != b) ? 1 : 0;
    }
    __device__ void emit(int64_t k, uint64_t excl, uint64_t v) const
    {
        if (v) ws.run_start[excl] = (int32_t)k;
    }
    __device__ void total(uint64_t tot, int64_t n) const
    {
        ws.ctrl[CTRL_RUNS] = (int32_t)tot;
        ws.run_start[tot] = (int32_t)n;
    }
};

struct TileOp {
    Ws ws;
    __device__ int64_t count() const { return ws.ctrl[CTRL_RUNS]; }
    __device__ uint64_t value(int64_t r) const
    {
        const int64_t len = ws.run_start[r + 1] - ws.run_start[r];
        return (uint64_t)((len + kUnitsPerTile - 1) / kUnitsPerTile);
    }
    // the tiles themselves are filled by k_tile_fill, one thread per tile (a
    // run of a hot (table, i2) holds hundreds of units)
    __device__ void emit(int64_t r, uint64_t excl, uint64_t) const { ws.run_tile_start[r] = (int32_t)excl; }
    __device__ void total(uint64_t tot, int64_t nruns) const
    {
        ws.ctrl[CTRL_TILES] = (int32_t)tot;
        ws.run_tile_start[nruns] = (int32_t)tot;
    }
};

struct ChunkOp {
    Ws ws;
    int S;
    __device__ int64_t count() const { return ws.ctrl[CTRL_TILES]; }
    // unique rows of a tile: its units' row counts, read unconditionally
    // (units past the tile's count read its first unit and add nothing)
    __device__ int32_t rows(int64_t tile) const
    {
        const int32_t b = ws.tile_ubeg[tile], nu = ws.tile_nu[tile];
        int32_t r = 0;
#pragma unroll
        for (int j = 0; j < kUnitsPerTile; ++j) {
            const int32_t u = ws.uorder[b + (j < nu ? j : 0)];
            const int32_t len = ws.unit_start[u + 1] - ws.unit_start[u];
            r += j < nu ? len : 0;
        }
        return r;
    }
    __device__ int32_t aux(int64_t tile) const { return rows(tile); }
    __device__ uint64_t value(int64_t tile) const
    {
        const int32_t r = rows(tile);
        const uint64_t nch = r <= S ? 1 : (uint64_t)((r + S - 1) / S);
        return nch | (nch > 1 ? (1ull << 32) : 0ull);
    }
    __device__ void emit(int64_t tile, uint64_t excl, uint64_t v, int32_t r) const
    {
        const uint32_t nch = (uint32_t)(v & 0xffffffffu);
        const uint32_t lo = (uint32_t)(excl & 0xffffffffu), hi = (uint32_t)(excl >> 32);
        ws.tile_rows[tile] = r;
        ws.tile_cstart[tile] = (int32_t)lo;
        ws.tile_slot[tile] = (nch > 1 && hi < (uint32_t)ws.ckpt_slots) ? (int32_t)hi : -1;
        for (uint32_t c = 0; c < nch; ++c) {
            if ((int64_t)lo + c >= ws.chunk_cap) break; // reported by total()
            ws.chunk_tile[lo + c] = (int32_t)tile;
            ws.chunk_rbeg[lo + c] = (int32_t)(c * S);
            const int32_t e = (int32_t)((c + 1) * S);
            ws.chunk_rend[lo + c] = e < r ? e : r;
        }
    }
    __device__ void total(uint64_t tot, int64_t) const
    {
        int64_t c = (int64_t)(tot & 0xffffffffu);
        if (c > ws.chunk_cap) {
            atomicOr(&ws.ctrl[CTRL_ERR], (int)ERRB_CAPACITY);
            c = ws.chunk_cap;
        }
        ws.ctrl[CTRL_CHUNKS] = (int32_t)c;
        ws.ctrl[CTRL_SPLIT] = (int32_t)(tot >> 32);
        ws.tile_cstart[ws.ctrl[CTRL_TILES]] = (int32_t)c;
    }
};

// First unit and unit count of every tile: tile i lies in the run r with
// run_tile_start[r] <= i < run_tile_start[r + 1] and takes that run's units
// 4j .. 4j + 3, j = i - run_tile_start[r].
__global__ __launch_bounds__(kThreads) void k_tile_fill(Ws ws)
{
    const int64_t nt = ws.ctrl[CTRL_TILES], nr = ws.ctrl[CTRL_RUNS];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nt; i += stride) {
        int64_t lo = 0, hi = nr; // last r < nr with run_tile_start[r] <= i
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (ws.run_tile_start[mid] <= i) lo = mid;
            else hi = mid;
        }
        const int32_t j = (int32_t)(i - ws.run_tile_start[lo]);
        const int32_t b = ws.run_start[lo], len = ws.run_start[lo + 1] - b;
        const int32_t rem = len - j * kUnitsPerTile;
        ws.tile_ubeg[i] = b + j * kUnitsPerTile;
        ws.tile_nu[i] = rem < kUnitsPerTile ? rem : kUnitsPerTile;
    }
}

// One record per chunk: the digits, row ranges and per-row i3 the persistent
// contraction kernel needs, gathered here in parallel.  A block takes
// kThreads chunks: (A) a thread per chunk works out its header (dwords
// 0-31) into LDS, (B) the block fills the i3 digits of all its chunks with
// independent loads, (C) each wave copies 64 records out, one coalesced
// 256-byte store per record.
constexpr int kRecStride = 65; // dwords per record in LDS (odd: rows spread over the banks)

__global__ __launch_bounds__(kThreads) void k_chunk_records(const TableDesc *tab, int T, int S, Ws ws)
{
    static_assert(sizeof(ChunkRec) == 64 * sizeof(int32_t), "64 dwords per record");
    __shared__ int32_t rl[kThreads * kRecStride];
    __shared__ int32_t n3l[kThreads];
    __shared__ int32_t tus[kMaxTables + 1]; // table unit starts: the table search reads LDS
    const int64_t C = ws.ctrl[CTRL_CHUNKS];
    const int tid = threadIdx.x, lane = tid & 63;
    for (int t = tid; t <= T; t += kThreads) tus[t] = ws.tab_unit_start[t];
    __syncthreads();
    for (int64_t cb = (int64_t)blockIdx.x * kThreads; cb < C; cb += (int64_t)gridDim.x * kThreads) {
        // (A) header of chunk cb + tid
        const int64_t c = cb + tid;
        int32_t *r = rl + tid * kRecStride;
        int rank = 4;
        if (c < C) {
            const int tile = ws.chunk_tile[c];
            const int rbeg = ws.chunk_rbeg[c], rend = ws.chunk_rend[c];
            const int ubeg = ws.tile_ubeg[tile], nu = ws.tile_nu[tile];
            const int u0 = ws.uorder[ubeg];
            const int t = segment_of(tus, T, u0);
            const TableDesc &tb = tab[t];
            const int P = (tb.d3 > 0 && tb.d3 <= 16) ? 16 / tb.d3 : 1;
            r[0] = tile;
            r[1] = t;
            r[2] = nu;
            r[3] = rbeg;
            r[4] = rend;
            r[5] = ws.tile_slot[tile];
            r[6] = ws.unit_prefix[u0] % tb.n2;
            r[7] = tb.cls;
            r[30] = (ws.tile_rows[tile] + S - 1) / S;
            r[31] = ubeg;
            n3l[tid] = tb.n3;
            int off = 0, coff = 0, ps = 0;
            r[20] = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // units past the tile's count read its first unit (unconditional
                // loads, all in flight together) and contribute nothing
                const int u = ws.uorder[ubeg + (j < nu ? j : 0)];
                const int s0 = ws.unit_start[u], cnt = j < nu ? ws.unit_start[u + 1] - s0 : 0;
                const int pq = ws.unit_prefix[u];
                int i1 = 0, us = 0, cc = 0;
                if (j < nu) {
                    const int lo = rbeg > off ? rbeg : off;
                    const int hi = rend < off + cnt ? rend : off + cnt;
                    cc = hi > lo ? hi - lo : 0;
                    us = s0 + (lo - off);
                    i1 = pq / tb.n2;
                    off += cnt;
                }
                r[8 + j] = i1;
                r[12 + j] = us;
                r[16 + j] = cc;
                r[25 + j] = coff;
                coff += cc;
                ps += (cc + P - 1) / P;
                r[21 + j] = ps;
            }
            r[29] = coff;
            rank = tb.cls < 0 ? 4 : tb.cls;
        }
        // first chunk of each rank class (chunks are class-major; generic
        // tables rank 4, after the MFMA classes), found where the rank steps
        // up between neighbouring chunks; entry 5 is the chunk count
        int prev = __shfl_up(rank, 1, 64); // every lane active
        if (c < C) {
            if (lane == 0 && c > 0) {
                const int pt = segment_of(tus, T, ws.uorder[ws.tile_ubeg[ws.chunk_tile[c - 1]]]);
                prev = tab[pt].cls < 0 ? 4 : tab[pt].cls;
            }
            if (c == 0) prev = -1;
            for (int q = prev + 1; q <= rank; ++q) ws.ctrl[CTRL_CLS_START + q] = (int32_t)c;
            if (c == C - 1)
                for (int q = rank + 1; q <= 5; ++q) ws.ctrl[CTRL_CLS_START + q] = (int32_t)C;
        }
        __syncthreads();
        // (B) i3 of row e % 32 of chunk e / 32, e = i * kThreads + tid (zeros past
        // the chunk's rows).  Eight rows at a time, their loads all in flight:
        // the header fields are read whatever the row (LDS, always in range),
        // the load is unconditional (row 0 of the unique rows stands in past a
        // chunk's rows, and its digit modulo 1 is the zero stored there), and
        // the division's result is stored without a select (a select on it is
        // turned into a branch around the division and the load)
        static_assert(kMaxChunkRows % 8 == 0, "rows in groups of eight");
#pragma unroll
        for (int i0 = 0; i0 < kMaxChunkRows; i0 += 8) {
            int x[8], n3v[8];
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                const int e = (i0 + ii) * kThreads + tid, k = e >> 5, row = e & 31;
                const int32_t *rk = rl + k * kRecStride;
                const bool ok = (cb + k < C) & (row < rk[29]);
                const int j = (row >= rk[26]) + (row >= rk[27]) + (row >= rk[28]);
                const int idx = rk[12 + j] + (row - rk[25 + j]);
                x[ii] = ws.uniq_row[ok ? idx : 0];
                n3v[ii] = ok ? n3l[k] : 1;
            }
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                const int e = (i0 + ii) * kThreads + tid, k = e >> 5, row = e & 31;
                rl[k * kRecStride + 32 + row] = x[ii] % n3v[ii];
            }
        }
        __syncthreads();
        // (C) wave w writes records w*64 .. w*64+63 of the block, one per store
        const int w = tid >> 6;
        for (int k = w * 64; k < w * 64 + 64 && cb + k < C; ++k)
            reinterpret_cast<int32_t *>(&ws.crec[cb + k])[lane] = rl[k * kRecStride + lane];
        __syncthreads();
    }
}

hipError_t launch_grouping(const Plan &p, const int64_t *indices, const int64_t *offsets,
                           hipStream_t s)
{
    Ws ws = p.ws;
    const int T = p.T;
    const int64_t nnz = p.nnz, nbags = (int64_t)T * p.B;
    timer_begin(p.timing, TM_GROUP_SORT, s);
    timer_begin(p.timing, TM_STAGE_DECODE, s);
    hipLaunchKernelGGL(k_init_ctrl, dim3(1), dim3(kThreads), 0, s, ws, T);
    {
        int g = ceil_div(nbags > 0 ? nbags : 1, kThreads);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(k_check_offsets, dim3(g), dim3(kThreads), 0, s, offsets, nbags, nnz, p.B, T, ws);
    }
    if (nnz > 0) {
        int g = ceil_div(nnz, kThreads * 4);
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(k_decode, dim3(g), dim3(kThreads), 0, s, indices, nnz, p.dtab, T,
                           p.check_indices ? 1 : 0, ws);
    }
    timer_end(p.timing, TM_STAGE_DECODE, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 1. index sorting by (table, row), stable
    timer_begin(p.timing, TM_STAGE_SORT, s);
    bool in1 = false;
    e = radix_sort_pairs(p, ws.keys0, ws.vals0, ws.keys1, ws.vals1, nnz, nullptr, p.key_bits, &in1, s);
    if (e != hipSuccess) return e;
    const uint32_t *sk = in1 ? ws.keys1 : ws.keys0;
    const int32_t *sv = in1 ? ws.vals1 : ws.vals0;
    // the plan points skeys/perm at the buffers the sort ends in
    if (sk != ws.skeys || sv != ws.perm) return hipErrorInvalidValue;
    timer_end(p.timing, TM_STAGE_SORT, s);
    timer_end(p.timing, TM_GROUP_SORT, s);
    timer_begin(p.timing, TM_GROUP_RLE, s);
    // 2. unique extraction
    timer_begin(p.timing, TM_STAGE_UNIQUE, s);
    if (nnz > 0) {
        UniqueOp uop{sk, sv, ws, nnz};
        e = run_scan(uop, ws.part, scan_blocks(nnz), s);
        if (e != hipSuccess) return e;
    }
    timer_end(p.timing, TM_STAGE_UNIQUE, s);
    timer_begin(p.timing, TM_STAGE_PREFIX, s);
    if (nnz > 0) {
        // 3.-4. mixed-radix conversion, prefix extraction, run-length encoding
        GroupOp gop{p.dtab, T, ws};
        e = run_scan(gop, ws.part, scan_blocks(nnz), s);
        if (e != hipSuccess) return e;
    }
    const bool unique_only = p.group_mode == 2;
    if (unique_only) {
        int g = ceil_div(nnz > 0 ? nnz : 1, kThreads * 4);
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(k_units_unique, dim3(g), dim3(kThreads), 0, s, p.dtab, T, ws);
    }
    hipLaunchKernelGGL(k_finalize_bases, dim3(1), dim3(64), 0, s, p.dtab, T, unique_only ? 1 : 0, ws);
    timer_end(p.timing, TM_STAGE_PREFIX, s);
    if (p.kp.K > 0) { // K >= 4 cores: the prefix levels are built by the forward itself
        timer_end(p.timing, TM_GROUP_RLE, s);
        return hipGetLastError();
    }
    if (nnz > 0) {
        // B-stationary order of units: stable sort by (table, i2)
        timer_begin(p.timing, TM_STAGE_ORDER, s);
        int g = ceil_div(nnz, kThreads * 4);
        if (g > 8192) g = 8192;
        hipLaunchKernelGGL(k_unit_keys, dim3(g), dim3(kThreads), 0, s, p.dtab, T, ws);
        bool u1 = false;
        e = radix_sort_pairs(p, ws.keys0, ws.uvals0, ws.keys1, ws.uvals1, nnz, &ws.ctrl[CTRL_UNITS],
                             p.key2_bits, &u1, s);
        if (e != hipSuccess) return e;
        const uint32_t *k2 = u1 ? ws.keys1 : ws.keys0;
        const int32_t *uo = u1 ? ws.uvals1 : ws.uvals0;
        if (k2 != ws.ukey2 || uo != ws.uorder) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_uinv, dim3(g), dim3(kThreads), 0, s, ws, uo);
        timer_end(p.timing, TM_STAGE_ORDER, s);
        // 5. work list: runs of equal (table, i2), tiles of <= 4 units, chunks
        timer_begin(p.timing, TM_STAGE_WORKLIST, s);
        RunOp rop{k2, ws};
        e = run_scan(rop, ws.part, scan_blocks(nnz), s);
        if (e != hipSuccess) return e;
        TileOp top{ws};
        e = run_scan(top, ws.part, scan_blocks(nnz), s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_tile_fill, dim3(g), dim3(kThreads), 0, s, ws);
        ChunkOp cop{ws, p.chunk_rows};
        e = run_scan(cop, ws.part, scan_blocks(nnz), s);
        if (e != hipSuccess) return e;
        int gc = ceil_div(ws.chunk_cap, kThreads);
        if (gc > 4096) gc = 4096;
        hipLaunchKernelGGL(k_chunk_records, dim3(gc), dim3(kThreads), 0, s, p.dtab, T, p.chunk_rows, ws);
        timer_end(p.timing, TM_STAGE_WORKLIST, s);
    }
    timer_end(p.timing, TM_GROUP_RLE, s);
    return hipGetLastError();
}

} // namespace ttemb
