// api.hip -- host side of the C ABI declared in include/tt_emb.h: argument
// checks, the workspace plan, and stream-ordered launch sequencing.
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/tt_emb.h"
#include "internal.h"

using namespace ttemb;

namespace ttemb {
// Rings of (start, stop) event pairs, one ring per phase timer.
struct Timing {
    static constexpr int kRing = 1024;
    std::vector<hipEvent_t> ev[TM_COUNT][2];
    int used[TM_COUNT] = {};
    bool on = false;
};

void timer_begin(Timing *tm, int id, hipStream_t s)
{
    if (!tm || !tm->on || tm->used[id] >= Timing::kRing) return;
    (void)hipEventRecord(tm->ev[id][0][tm->used[id]], s);
}

void timer_end(Timing *tm, int id, hipStream_t s)
{
    if (!tm || !tm->on || tm->used[id] >= Timing::kRing) return;
    (void)hipEventRecord(tm->ev[id][1][tm->used[id]], s);
    ++tm->used[id];
}
} // namespace ttemb

struct tt_emb {
    Timing *timing = nullptr;
    int32_t T;
    std::vector<TableDesc> tabs;
    TableDesc *dtab = nullptr;
    int device = 0;
    int sched_mode, group_mode, chunk_rows, num_blocks, check_indices, force_generic, keep_prefix;
    bool any_generic;
    int key_bits, key2_bits, key3_bits;
    int Dmax, Dpmax, R2max, sumD;
    int sum_n[3];
    int64_t max_d1R1, max_R2d3, max_Dp;
    int64_t g3t_elems;
    int cls_mask, gcls_mask;
    int K = 3;                 // TT cores per table
    std::vector<KTab> ktabs;   // K >= 4 only
    std::vector<int32_t> kn;   // K >= 4 only: n_k of every table, [T*K]
    KTab *dkt = nullptr;
};

namespace {

// Scratch of tt_emb_forward_noalloc: one fixed array per GPU the library runs
// on.  In host code `scratch` only names the symbol; its device address on
// each GPU is looked up once (hipGetSymbolAddress with that GPU current) and
// kept in noalloc_ptr, which is what the launches receive.
static __device__ __align__(256) char scratch[TT_EMB_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void *noalloc_ptr[kMaxDevices] = {};
hipError_t noalloc_err[kMaxDevices] = {};
bool noalloc_done[kMaxDevices] = {};

// Called at create time with the handle's device current.
void noalloc_setup(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return;
    std::lock_guard<std::mutex> g(noalloc_mu);
    if (noalloc_done[dev]) return;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    noalloc_err[dev] = e;
    noalloc_ptr[dev] = e == hipSuccess ? ptr : nullptr;
    noalloc_done[dev] = true;
}

int bits_for(uint64_t max_value)
{
    int b = 0;
    while (b < 63 && (max_value >> b) != 0) ++b;
    return b;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

int sort_passes(int64_t n, int bits) { return (n <= 0 || bits <= 0) ? 0 : (bits + 7) / 8; }

// dG2 partial slots for split backward runs: split runs take fewer than
// 2 * tiles / kPieceTiles <= 2 * nnz / kPieceTiles slots, capped (the backward
// then cuts longer pieces).
int64_t g2p_slots_for(int64_t nnz)
{
    const int64_t n = nnz > 0 ? nnz : 1;
    const int64_t v = 2 * n / kPieceTiles + 1;
    return v < kMaxG2Slots ? v : kMaxG2Slots;
}

// Carve the workspace.  With base == nullptr only the size is computed.  The
// regions a forward without TT_EMB_KEEP_PREFIX uses come first; *fwd_bytes
// (optional) receives their size.  With fwd_only the backward's pointers in
// the plan are left null (the caller's buffer ends before them).
size_t plan_workspace(const tt_emb *h, int64_t B, int64_t nnz, char *base, Plan *p, size_t *fwd_bytes = nullptr,
                      bool fwd_only = false)
{
    size_t off = 0;
    auto take = [&](size_t bytes) -> char * {
        char *r = base ? base + off : nullptr;
        off += align_up(bytes > 0 ? bytes : 1);
        return r;
    };
    const int64_t n = nnz > 0 ? nnz : 1;
    const int T = h->T;
    Ws w{};
    w.ctrl = (int32_t *)take(sizeof(int32_t) * CTRL_N);
    w.keys0 = (uint32_t *)take(4 * n);
    w.keys1 = (uint32_t *)take(4 * n);
    w.vals0 = (int32_t *)take(4 * n);
    w.vals1 = (int32_t *)take(4 * n);
    w.uvals0 = (int32_t *)take(4 * n);
    w.uvals1 = (int32_t *)take(4 * n);
    // radix histograms: the largest sort is the lookups' or the backward's
    // pieces (at most min(nnz, sum n2) + 1 + g2p_slots_for(nnz) keys)
    const int64_t pieces_keys = (nnz < h->sum_n[1] ? nnz : h->sum_n[1]) + 1 + g2p_slots_for(nnz);
    const int64_t nblk = sort_blocks(n > pieces_keys ? n : pieces_keys);
    w.hist = (uint32_t *)take(4 * 256 * nblk);
    w.part = (uint64_t *)take(8 * (kScanBlocks + 1));
    w.tstart = (int32_t *)take(4 * (T + 1));
    w.inv = (int32_t *)take(4 * n);
    w.ukey = (uint32_t *)take(4 * n);
    w.uniq_row = (int32_t *)take(4 * n);
    w.uniq_start = (int32_t *)take(4 * (n + 1));
    w.grp_prefix = (int32_t *)take(4 * n);
    w.grp_start = (int32_t *)take(4 * (n + 1));
    w.tab_uniq_start = (int32_t *)take(4 * (T + 1));
    w.tab_grp_start = (int32_t *)take(4 * (T + 1));
    w.ebase = (int64_t *)take(8 * T);
    w.p3base = (int64_t *)take(8 * T);
    if (h->group_mode == TT_EMB_GROUP_UNIQUE_ONLY) {
        w.unit_prefix = (int32_t *)take(4 * n);
        w.unit_start = (int32_t *)take(4 * (n + 1));
        w.tab_unit_start = (int32_t *)take(4 * (T + 1));
    } else {
        w.unit_prefix = w.grp_prefix;
        w.unit_start = w.grp_start;
        w.tab_unit_start = w.tab_grp_start;
    }
    w.run_start = (int32_t *)take(4 * (n + 1));
    w.run_tile_start = (int32_t *)take(4 * (n + 1));
    w.tile_ubeg = (int32_t *)take(4 * n);
    w.tile_nu = (int32_t *)take(4 * n);
    w.tile_rows = (int32_t *)take(4 * n);
    w.tile_slot = (int32_t *)take(4 * n);
    // chunks <= rows/S + tiles, tiles <= units/4 + runs, runs <= sum n2
    int64_t units_bound = 0;
    for (int t = 0; t < T; ++t) {
        const TableDesc &d = h->tabs[t];
        const int64_t pre = (int64_t)d.n1 * d.n2;
        int64_t ub = h->group_mode == TT_EMB_GROUP_UNIQUE_ONLY ? d.N : (pre < d.N ? pre : d.N);
        units_bound += ub < n ? ub : n;
    }
    if (units_bound > n) units_bound = n;
    int64_t chunks = n / h->chunk_rows + 1 + units_bound / 4 + 1 + h->sum_n[1] + 1;
    if (chunks > 2 * n + 1) chunks = 2 * n + 1;
    w.tile_cstart = (int32_t *)take(4 * (n + 1));
    w.uinv = (int32_t *)take(4 * n);
    w.chunk_tile = (int32_t *)take(4 * chunks);
    w.chunk_rbeg = (int32_t *)take(4 * chunks);
    w.chunk_rend = (int32_t *)take(4 * chunks);
    w.crec = (ChunkRec *)take(sizeof(ChunkRec) * chunks);
    w.chunk_cap = chunks;
    w.g3t = (float *)take(4 * (size_t)h->g3t_elems);
    // 4 classes x up to kMaxWorkersPerCu workers per CU, one 128-byte line each
    w.heads = (int32_t *)take(4 * (size_t)h->num_blocks * 4 * kMaxWorkersPerCu * 32);
    // L2 checkpoint slots (stealing with checkpoints only): one per split
    // tile, and a split tile holds more than chunk_rows unique rows
    int64_t ckpt_slots = h->sched_mode == 3 ? n / (h->chunk_rows + 1) + 1 : 0;
    if (ckpt_slots > kMaxCkptSlots) ckpt_slots = kMaxCkptSlots;
    w.ckpt_slots = (int32_t)ckpt_slots;
    w.flags = (int32_t *)take(4 * (size_t)ckpt_slots);
    w.ckpt = (float *)take(4 * (size_t)ckpt_slots * (4 * (16 * 68 + 16)));
    // bounds on unique rows / units per table that do not depend on values
    int64_t e_elems = 0, p3_elems = 0;
    for (int t = 0; t < T; ++t) {
        const TableDesc &d = h->tabs[t];
        const int64_t urows = d.N < n ? d.N : n;
        const int64_t pre = (int64_t)d.n1 * d.n2;
        e_elems += urows * d.Dp;
        p3_elems += urows * (int64_t)d.R2 * d.d3;
        (void)pre;
    }
    if (e_elems > n * h->max_Dp) e_elems = n * h->max_Dp;
    if (p3_elems > n * h->max_R2d3) p3_elems = n * h->max_R2d3;
    // gradient gather: tasks of kGuTask sorted positions per table, two partial rows each
    const int64_t tasks = n / kGuTask + T + 1;
    const int64_t part_elems = tasks * 2 * h->Dpmax;
    w.E = (float *)take(4 * e_elems);
    w.sink = (float *)take(4 * (size_t)kSinkFloats);
    w.bstat = (BlockStat *)take(sizeof(BlockStat) * (size_t)kStatKernels * kStatBlocks);
    w.cbase = (int64_t *)take(8 * T);
    w.ftab = (FwdTab *)take(sizeof(FwdTab) * (size_t)T);
    w.lb = (int32_t *)take(4 * n);
    // K >= 4 cores: per prefix length m = 2..K-1, the group of each unique
    // row, the groups' first rows, and one intermediate per group (at most
    // min(prefixes of length m, rows, nnz) groups per table)
    KPlan kp{};
    if (h->K >= 4) {
        kp.K = h->K;
        kp.dkt = h->dkt;
        for (int m = 2; m <= h->K - 1; ++m) {
            int64_t gb = 0, sm = 1;
            for (int t = 0; t < T; ++t) {
                const KTab &kt = h->ktabs[t];
                int64_t prod = 1;
                for (int j = 0; j < m; ++j) prod = std::min<int64_t>(prod * kt.n[j], (int64_t)1 << 40);
                gb += std::min<int64_t>(std::min<int64_t>(prod, h->tabs[t].N), n);
                sm = std::max<int64_t>(sm, (int64_t)kt.P[m] * kt.R[m]);
            }
            gb = std::min<int64_t>(gb, n);
            kp.ugrp[m] = (int32_t *)take(4 * n);
            kp.gfirst[m] = (int32_t *)take(4 * (n + 1));
            kp.V[m] = (float *)take(4 * (size_t)(gb * sm));
            kp.smax[m] = sm;
        }
    }
    // everything a forward without TT_EMB_KEEP_PREFIX (and the grouping, its
    // views and the block records) touches lies before this point; the
    // backward's regions and the kept prefix intermediates follow
    const size_t fwd_end = off;
    // kept prefix intermediates (keep_prefix handles only): 16 x R2 floats per
    // unit of every table of the kept rank classes, at most min(units of the
    // table, nnz) units
    int64_t cg_elems = 0;
    if (h->keep_prefix) {
        for (int t = 0; t < T; ++t) {
            const TableDesc &d = h->tabs[t];
            if (d.cls < kKeepMinCls) continue;
            const int64_t pre = (int64_t)d.n1 * d.n2;
            int64_t ub = h->group_mode == TT_EMB_GROUP_UNIQUE_ONLY ? d.N : (pre < d.N ? pre : d.N);
            ub = ub < n ? ub : n;
            cg_elems += ub * 16 * (int64_t)d.R2;
        }
    }
    w.Cg = (float *)take(4 * (cg_elems > 0 ? cg_elems : 4));
    w.gu_ml = (int32_t *)take(4 * tasks);
    w.gu_mr = (int32_t *)take(4 * tasks);
    // gradient gather: sorted-order lookup metadata
    w.sm = (int2 *)take(8 * n);
    w.P3 = (float *)take(4 * (p3_elems > part_elems ? p3_elems : part_elems));
    // G1 partials are indexed by work position (< units) with a uniform stride
    w.G1P = (float *)take(4 * (size_t)units_bound * h->max_d1R1);
    // [first, last) unique-row range (in (table, i3) order) of every G3 slice
    w.g3rng = (int32_t *)take(4 * 2 * ((size_t)h->sum_n[2] + 1));
    // backward pieces and their claim order: runs <= min(nnz, sum n2); split
    // runs take at most 2 * tiles / kPieceTiles <= 2 * nnz / kPieceTiles slots
    // (the backward's launch computes the same bounds from nnz and sum n2)
    const int64_t runs_bound = (nnz < h->sum_n[1] ? nnz : h->sum_n[1]) + 1;
    const int64_t slots_cap = g2p_slots_for(nnz);
    const int64_t pieces_bound = runs_bound + slots_cap;
    w.run_pbase = (int32_t *)take(4 * runs_bound);
    w.run_sbase = (int32_t *)take(4 * runs_bound);
    w.piece_tb = (int32_t *)take(4 * pieces_bound);
    w.piece_te = (int32_t *)take(4 * pieces_bound);
    w.piece_slot = (int32_t *)take(4 * pieces_bound);
    w.G2P = (float *)take(4 * (size_t)slots_cap * kG2PStride);
    w.rkey0 = (uint32_t *)take(4 * pieces_bound);
    w.rkey1 = (uint32_t *)take(4 * pieces_bound);
    w.rval0 = (int32_t *)take(4 * pieces_bound);
    w.rval1 = (int32_t *)take(4 * pieces_bound);
    w.rorder = w.rval0;
    // buffers where the sorts end
    const int fm = sort_passes(nnz, h->key_bits) & 1;
    const int fu = sort_passes(nnz, h->key2_bits) & 1;
    w.skeys = fm ? w.keys1 : w.keys0;
    w.perm = fm ? w.vals1 : w.vals0;
    w.ukey2 = fu ? w.keys1 : w.keys0;
    w.uorder = fu ? w.uvals1 : w.uvals0;
    w.u3order = fm ? w.vals0 : w.vals1;
    w.uvals_free = fu ? w.uvals0 : w.uvals1;
    w.key3 = nullptr;
    if (p) {
        p->timing = (h->timing && h->timing->on) ? h->timing : nullptr;
        p->T = T;
        p->B = B;
        p->nnz = nnz;
        p->num_blocks = h->num_blocks;
        p->sched_mode = h->sched_mode;
        p->group_mode = h->group_mode;
        p->chunk_rows = h->chunk_rows;
        p->check_indices = h->check_indices;
        p->force_generic = h->force_generic;
        p->keep_c = p->reuse_c = p->pool_atomic = 0;
        p->any_generic = h->any_generic;
        p->cls_mask = h->cls_mask;
        p->gcls_mask = h->gcls_mask;
        p->key_bits = h->key_bits;
        p->key2_bits = h->key2_bits;
        p->key3_bits = h->key3_bits;
        p->Dmax = h->Dmax;
        p->Dpmax = h->Dpmax;
        p->R2max = h->R2max;
        p->sumD = h->sumD;
        for (int k = 0; k < 3; ++k) p->sum_n[k] = h->sum_n[k];
        p->g1stride = (int)h->max_d1R1;
        p->g2p_slots = (int)g2p_slots_for(nnz);
        p->dtab = h->dtab;
        p->ws = w;
    }
    if (h->K >= 4) {
        // backward: groups of the first digit, the intermediates' gradients and
        // the per-group / per-row core partials
        for (int m = 1; m <= h->K - 1; ++m) {
            int64_t gb = 0, sm = 1, qm = 1;
            for (int t = 0; t < T; ++t) {
                const KTab &kt = h->ktabs[t];
                int64_t prod = 1;
                for (int j = 0; j < m; ++j) prod = std::min<int64_t>(prod * kt.n[j], (int64_t)1 << 40);
                gb += std::min<int64_t>(std::min<int64_t>(prod, h->tabs[t].N), n);
                sm = std::max<int64_t>(sm, (int64_t)kt.P[m] * kt.R[m]);
                if (m >= 2) qm = std::max<int64_t>(qm, (int64_t)kt.R[m - 1] * kt.d[m - 1] * kt.R[m]);
            }
            gb = std::min<int64_t>(gb, n);
            if (m == 1) {
                kp.ugrp[1] = (int32_t *)take(4 * n);
                kp.gfirst[1] = (int32_t *)take(4 * (n + 1));
                kp.smax[1] = sm;
            }
            kp.dV[m] = (float *)take(4 * (size_t)(gb * sm));
            if (m >= 2) {
                kp.Q[m] = (float *)take(4 * (size_t)(gb * qm));
                kp.qmax[m] = qm;
                kp.Cc[m] = (float *)take(4 * (size_t)(gb * kp.smax[m - 1]));
            }
        }
        int64_t pk = 1;
        for (int t = 0; t < T; ++t) {
            const KTab &kt = h->ktabs[t];
            pk = std::max<int64_t>(pk, (int64_t)kt.R[h->K - 1] * kt.d[h->K - 1]);
        }
        kp.pkmax = pk;
        kp.PK = (float *)take(4 * (size_t)(n * pk));
        // split sums of the per-slice reduction: 16 per slice of the largest core
        int64_t red = 1;
        for (int t = 0; t < T; ++t) {
            const KTab &kt = h->ktabs[t];
            for (int k = 0; k < h->K; ++k)
                red = std::max<int64_t>(red, (int64_t)kt.n[k] * kt.R[k] * kt.d[k] * kt.R[k + 1] * 16);
        }
        kp.red = (float *)take(4 * (size_t)red);
        for (int k = 0; k < h->K; ++k) {
            int64_t tot = 0;
            for (int t = 0; t < T; ++t) tot += h->ktabs[t].n[k];
            int bits = 1;
            while (((int64_t)1 << bits) <= tot) ++bits;
            kp.key_bits[k] = bits;
        }
    }
    if (p) {
        p->kp = kp;
        p->kp_n = h->K >= 4 ? h->kn.data() : nullptr;
        if (fwd_only) {
            Ws &v = p->ws;
            v.Cg = nullptr;
            v.gu_ml = v.gu_mr = nullptr;
            v.sm = nullptr;
            v.P3 = v.G1P = v.G2P = nullptr;
            v.g3rng = v.run_pbase = v.run_sbase = v.piece_tb = v.piece_te = v.piece_slot = nullptr;
            v.rkey0 = v.rkey1 = nullptr;
            v.rval0 = v.rval1 = nullptr;
            v.rorder = nullptr;
            for (int m = 0; m < kMaxK; ++m) p->kp.dV[m] = p->kp.Q[m] = p->kp.Cc[m] = nullptr;
            p->kp.ugrp[1] = p->kp.gfirst[1] = nullptr;
            p->kp.PK = p->kp.red = nullptr;
        }
    }
    if (fwd_bytes) *fwd_bytes = fwd_end;
    return off;
}

bool bad_ptr(const void *ptr) { return ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

// full: the call needs the whole workspace (backward, or a forward that keeps
// the prefix intermediates); otherwise the forward part is enough.
int check_call(const tt_emb *h, int64_t B, int64_t nnz, const int64_t *indices, const int64_t *offsets,
               void *ws, size_t ws_bytes, Plan *p, bool full)
{
    if (!h || B < 0 || nnz < 0 || nnz >= (int64_t)0x7fffffff) return TT_EMB_ERR_ARG;
    if ((int64_t)h->T * B >= (int64_t)0x7fffffff) return TT_EMB_ERR_ARG;
    if (!offsets) return TT_EMB_ERR_ARG;
    if (nnz > 0 && !indices) return TT_EMB_ERR_ARG;
    if (nnz > 0 && B == 0) return TT_EMB_ERR_ARG; // lookups with no bag to belong to
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return TT_EMB_ERR_WORKSPACE;
    size_t fwd = 0;
    const size_t all = plan_workspace(h, B, nnz, nullptr, nullptr, &fwd);
    if (ws_bytes < (full ? all : fwd)) return TT_EMB_ERR_WORKSPACE;
    plan_workspace(h, B, nnz, static_cast<char *>(ws), p, nullptr, ws_bytes < all);
    return TT_EMB_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TT_EMB_OK : TT_EMB_ERR_HIP; }

int set_device(const tt_emb *h)
{
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return TT_EMB_ERR_HIP;
    if (cur != h->device && hipSetDevice(h->device) != hipSuccess) return TT_EMB_ERR_HIP;
    return TT_EMB_OK;
}

} // namespace

extern "C" {

int tt_emb_create(int32_t T, const int64_t *num_rows, const int32_t *n, const int32_t *d, const int32_t *R,
                  const tt_emb_options *opt, tt_emb_t *out)
{
    try {
        if (!out) return TT_EMB_ERR_ARG;
        *out = nullptr;
        if (T <= 0 || !num_rows || !n || !d || !R) return TT_EMB_ERR_ARG;
        if (T > kMaxTables) return TT_EMB_ERR_UNSUPPORTED;
        tt_emb_options o{};
        if (opt) o = *opt;
        if (o.sched_mode < 0 || o.sched_mode > 3 || o.group_mode < 0 || o.group_mode > 2) return TT_EMB_ERR_ARG;
        if (o.chunk_rows < 0 || o.chunk_rows > kMaxChunkRows || o.num_blocks < 0) return TT_EMB_ERR_ARG;
        tt_emb *h = new (std::nothrow) tt_emb();
        if (!h) return TT_EMB_ERR_NOMEM;
        h->T = T;
        h->sched_mode = o.sched_mode; // 0: the per-rank-class default of the forward launch
        h->group_mode = o.group_mode == 0 ? TT_EMB_GROUP_PREFIX : o.group_mode;
        h->chunk_rows = o.chunk_rows == 0 ? kMaxChunkRows : o.chunk_rows;
        h->g3t_elems = 0;
        h->check_indices = o.check_indices >= 0 ? 1 : 0;
        h->force_generic = o.force_generic ? 1 : 0;
        h->keep_prefix = o.keep_prefix ? 1 : 0;
        uint64_t key = 0, b1 = 0, b2 = 0, b3 = 0;
        int col = 0;
        h->any_generic = false;
        h->Dmax = h->Dpmax = h->R2max = 0;
        h->max_d1R1 = h->max_R2d3 = h->max_Dp = 1;
        int rc = TT_EMB_OK;
        for (int t = 0; t < T && rc == TT_EMB_OK; ++t) {
            const int32_t *nt = n + 3 * t, *dt = d + 3 * t, *Rt = R + 4 * t;
            TableDesc td{};
            td.N = num_rows[t];
            td.n1 = nt[0];
            td.n2 = nt[1];
            td.n3 = nt[2];
            td.d1 = dt[0];
            td.d2 = dt[1];
            td.d3 = dt[2];
            td.R1 = Rt[1];
            td.R2 = Rt[2];
            if (td.N <= 0 || td.n1 <= 0 || td.n2 <= 0 || td.n3 <= 0 || td.d1 <= 0 || td.d2 <= 0 || td.d3 <= 0 ||
                Rt[0] != 1 || Rt[3] != 1 || td.R1 <= 0 || td.R2 <= 0) {
                rc = TT_EMB_ERR_ARG;
                break;
            }
            if ((int64_t)td.n1 * td.n2 * td.n3 < td.N) {
                rc = TT_EMB_ERR_ARG;
                break;
            }
            const int64_t D = (int64_t)td.d1 * td.d2 * td.d3;
            if (D > 1024 || td.R1 > 256 || td.R2 > 256 || (int64_t)td.d1 * td.d2 * td.R2 > 4096 ||
                (int64_t)td.R1 * td.d2 * td.R2 > 16384 || (int64_t)td.n1 * td.n2 >= (int64_t)0x7fffffff) {
                rc = TT_EMB_ERR_UNSUPPORTED;
                break;
            }
            td.D = (int32_t)D;
            td.Dp = (int32_t)((D + 3) & ~int64_t(3));
            td.col_off = col;
            col += td.D;
            td.key_base = (uint32_t)key;
            key += (uint64_t)td.N;
            td.i1_base = (uint32_t)b1;
            b1 += (uint64_t)td.n1;
            td.i2_base = (uint32_t)b2;
            b2 += (uint64_t)td.n2;
            td.i3_base = (uint32_t)b3;
            b3 += (uint64_t)td.n3;
            int cls = -1;
            if (td.R1 == td.R2 && td.d1 <= 4 && td.d2 <= 4 && td.d3 <= 16) {
                if (td.R1 == 8) cls = 0;
                else if (td.R1 == 16) cls = 1;
                else if (td.R1 == 32) cls = 2;
                else if (td.R1 == 64) cls = 3;
            }
            td.cls = cls;
            td.g3t_off = h->g3t_elems;
            if (cls >= 0) h->g3t_elems += (int64_t)td.n3 * td.R2 * td.d3;
            if (cls < 0) h->any_generic = true;
            if (td.D > h->Dmax) h->Dmax = td.D;
            if (td.Dp > h->Dpmax) h->Dpmax = td.Dp;
            if (td.R2 > h->R2max) h->R2max = td.R2;
            h->max_d1R1 = std::max<int64_t>(h->max_d1R1, (int64_t)td.d1 * td.R1);
            h->max_R2d3 = std::max<int64_t>(h->max_R2d3, (int64_t)td.R2 * td.d3);
            h->max_Dp = std::max<int64_t>(h->max_Dp, td.Dp);
            h->tabs.push_back(td);
        }
        if (rc == TT_EMB_OK && (key >= 0x7fffffffull || b2 >= 0x7fffffffull || b3 >= 0x7fffffffull || b1 >= 0x7fffffffull))
            rc = TT_EMB_ERR_UNSUPPORTED;
        if (rc != TT_EMB_OK) {
            delete h;
            return rc;
        }
        // work order is class-major: i2 bases follow the tables grouped by MFMA
        // rank class (generic tables last), so each class owns a contiguous
        // range of chunks and runs
        h->cls_mask = 0;
        {
            uint64_t base = 0;
            for (int c = 0; c <= 4; ++c)
                for (auto &td : h->tabs) {
                    const int rank = td.cls < 0 ? 4 : td.cls;
                    if (rank != c) continue;
                    td.i2_base = (uint32_t)base;
                    base += (uint64_t)td.n2;
                    if (td.cls >= 0) h->cls_mask |= 1 << td.cls;
                }
        }
        h->sumD = col;
        // gradient-gather class: rows move as float4 when every row of the
        // table's columns starts 16-byte aligned; lanes per row = columns
        // (float4 or float) rounded up to a power of two, at most 64
        h->gcls_mask = 0;
        for (auto &td : h->tabs) {
            const bool vec = ((col | td.col_off) & 3) == 0;
            const int cn = vec ? (td.D + 3) / 4 : td.D;
            int lg = 0;
            while (lg < 6 && (1 << lg) < cn) ++lg;
            td.gcls = lg + (vec ? 8 : 0);
            h->gcls_mask |= 1 << td.gcls;
        }
        h->sum_n[0] = (int)b1;
        h->sum_n[1] = (int)b2;
        h->sum_n[2] = (int)b3;
        h->key_bits = bits_for(key - 1);
        h->key2_bits = bits_for(b2 - 1);
        h->key3_bits = bits_for(b3 - 1);
        if (hipGetDevice(&h->device) != hipSuccess) {
            delete h;
            return TT_EMB_ERR_HIP;
        }
        if (o.num_blocks > 0) {
            h->num_blocks = (o.num_blocks + 7) / 8 * 8;
        } else {
            int cus = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess || cus <= 0)
                cus = 256;
            // one resident persistent block per CU: the contraction kernels
            // need more than 256 registers per lane (one wave per SIMD)
            h->num_blocks = (cus + 7) / 8 * 8;
        }
        // the no-allocation forward's scratch on this device (looked up once per device)
        noalloc_setup(h->device);
        if (hipMalloc((void **)&h->dtab, sizeof(TableDesc) * T) != hipSuccess) {
            delete h;
            return TT_EMB_ERR_NOMEM;
        }
        if (hipMemcpy(h->dtab, h->tabs.data(), sizeof(TableDesc) * T, hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(h->dtab);
            delete h;
            return TT_EMB_ERR_HIP;
        }
        *out = h;
        return TT_EMB_OK;
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

static void free_timing(tt_emb *h)
{
    if (!h->timing) return;
    for (int id = 0; id < TM_COUNT; ++id)
        for (int k = 0; k < 2; ++k)
            for (hipEvent_t e : h->timing->ev[id][k]) (void)hipEventDestroy(e);
    delete h->timing;
    h->timing = nullptr;
}

int tt_emb_create_k(int32_t T, int32_t K, const int64_t *num_rows, const int32_t *n, const int32_t *d,
                    const int32_t *R, const tt_emb_options *opt, tt_emb_t *out)
{
    try {
        if (!out) return TT_EMB_ERR_ARG;
        *out = nullptr;
        if (T <= 0 || !num_rows || !n || !d || !R) return TT_EMB_ERR_ARG;
        if (K == 3) return tt_emb_create(T, num_rows, n, d, R, opt, out);
        if (K < 2) return TT_EMB_ERR_ARG;
        if (K < 4 || K > kMaxK || T > kMaxTables || T * K > kMaxKPtrs) return TT_EMB_ERR_UNSUPPORTED;
        std::vector<KTab> kts((size_t)T);
        std::vector<int32_t> n3(3 * (size_t)T), d3(3 * (size_t)T, 1), R3(4 * (size_t)T, 1);
        int rc = TT_EMB_OK;
        for (int t = 0; t < T; ++t) {
            const int32_t *nt = n + (size_t)K * t, *dt = d + (size_t)K * t, *Rt = R + (size_t)(K + 1) * t;
            KTab &kt = kts[t];
            kt = KTab{};
            kt.K = K;
            if (num_rows[t] <= 0 || Rt[0] != 1 || Rt[K] != 1) return TT_EMB_ERR_ARG;
            int64_t prod = 1, D = 1;
            for (int k = 0; k < K; ++k) {
                if (nt[k] <= 0 || dt[k] <= 0 || Rt[k + 1] <= 0) return TT_EMB_ERR_ARG;
                kt.n[k] = nt[k];
                kt.d[k] = dt[k];
                kt.R[k] = Rt[k];
                prod = std::min<int64_t>(prod * nt[k], (int64_t)1 << 40);
                D *= dt[k];
                if (D > 1024) rc = TT_EMB_ERR_UNSUPPORTED;
                if (Rt[k + 1] > 256) rc = TT_EMB_ERR_UNSUPPORTED;
            }
            kt.R[K] = 1;
            if (prod < num_rows[t]) return TT_EMB_ERR_ARG;
            if (prod >= ((int64_t)1 << 40)) rc = TT_EMB_ERR_UNSUPPORTED;
            int64_t dv = 1;
            for (int k = K - 1; k >= 0; --k) {
                kt.div[k] = dv;
                dv = std::min<int64_t>(dv * nt[k], (int64_t)1 << 40);
            }
            // digit strides fit 32 bits (the kernels decode rows < 2^31 with
            // 32-bit division; div[0] is the largest stride)
            if (kt.div[0] > (int64_t)0xffffffff) rc = TT_EMB_ERR_UNSUPPORTED;
            kt.P[0] = 1;
            for (int m = 1; m <= K; ++m) kt.P[m] = kt.P[m - 1] * dt[m - 1];
            for (int k = 0; k < K; ++k) kt.nbase[k] = t == 0 ? 0 : kts[t - 1].nbase[k] + kts[t - 1].n[k];
            // staged operands of every level must fit in LDS
            for (int m = 2; m <= K - 1; ++m)
                if ((int64_t)kt.P[m - 1] * kt.R[m - 1] > kKLds || (int64_t)kt.R[m - 1] * dt[m - 1] * Rt[m] > kKLds)
                    rc = TT_EMB_ERR_UNSUPPORTED;
            if ((int64_t)kt.P[K - 1] * kt.R[K - 1] > kKLds) rc = TT_EMB_ERR_UNSUPPORTED;
            // the three-core view the grouping uses: digits (1, leading, last)
            const int64_t lead = kt.div[0] * nt[0] / nt[K - 1];
            if (lead >= 0x7fffffff) rc = TT_EMB_ERR_UNSUPPORTED;
            n3[3 * t] = 1;
            n3[3 * t + 1] = (int32_t)std::min<int64_t>(lead, 0x7fffffff);
            n3[3 * t + 2] = nt[K - 1];
            d3[3 * t + 2] = (int32_t)std::min<int64_t>(D, 1 << 20);
        }
        for (int k = 0; k < K; ++k) // backward sort keys of core-k slices fit 31 bits
            if ((int64_t)kts[T - 1].nbase[k] + kts[T - 1].n[k] > 0x3fffffff) rc = TT_EMB_ERR_UNSUPPORTED;
        if (rc != TT_EMB_OK) return rc;
        if ((rc = tt_emb_create(T, num_rows, n3.data(), d3.data(), R3.data(), opt, out)) != TT_EMB_OK) return rc;
        tt_emb *h = *out;
        h->K = K;
        h->ktabs = kts;
        h->kn.assign(n, n + (size_t)T * K);
        if (hipMalloc((void **)&h->dkt, sizeof(KTab) * T) != hipSuccess ||
            hipMemcpy(h->dkt, kts.data(), sizeof(KTab) * T, hipMemcpyHostToDevice) != hipSuccess) {
            tt_emb_destroy(h);
            *out = nullptr;
            return TT_EMB_ERR_HIP;
        }
        return TT_EMB_OK;
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

int tt_emb_destroy(tt_emb_t h)
{
    if (!h) return TT_EMB_OK;
    int rc = TT_EMB_OK;
    free_timing(h);
    if (h->dtab && hipFree(h->dtab) != hipSuccess) rc = TT_EMB_ERR_HIP;
    if (h->dkt && hipFree(h->dkt) != hipSuccess) rc = TT_EMB_ERR_HIP;
    delete h;
    return rc;
}

int tt_emb_workspace_size(tt_emb_t h, int64_t B, int64_t nnz, size_t *bytes)
{
    if (!h || !bytes || B < 0 || nnz < 0 || nnz >= (int64_t)0x7fffffff) return TT_EMB_ERR_ARG;
    *bytes = plan_workspace(h, B, nnz, nullptr, nullptr);
    return TT_EMB_OK;
}

int tt_emb_forward_workspace_size(tt_emb_t h, int64_t B, int64_t nnz, size_t *bytes)
{
    if (!h || !bytes || B < 0 || nnz < 0 || nnz >= (int64_t)0x7fffffff) return TT_EMB_ERR_ARG;
    plan_workspace(h, B, nnz, nullptr, nullptr, bytes);
    return TT_EMB_OK;
}

int tt_emb_group(tt_emb_t h, const int64_t *indices, const int64_t *offsets, int64_t B, int64_t nnz, void *ws,
                 size_t ws_bytes, void *stream)
{
    try {
        Plan p;
        int rc = check_call(h, B, nnz, indices, offsets, ws, ws_bytes, &p, false);
        if (rc) return rc;
        if ((rc = set_device(h))) return rc;
        return hip_status(launch_grouping(p, indices, offsets, (hipStream_t)stream));
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

static int kcore_ptrs(const tt_emb *h, const float *const *cores, KCorePtrs *cp)
{
    if (!cores) return TT_EMB_ERR_ARG;
    for (int i = 0; i < h->T * h->K; ++i) {
        if (bad_ptr(cores[i])) return TT_EMB_ERR_ARG;
        cp->g[i] = cores[i];
    }
    return TT_EMB_OK;
}

static int core_ptrs(const tt_emb *h, const float *const *cores, CorePtrs *cp)
{
    if (!cores) return TT_EMB_ERR_ARG;
    for (int t = 0; t < h->T; ++t)
        for (int k = 0; k < 3; ++k) {
            const float *c = cores[3 * t + k];
            if (bad_ptr(c)) return TT_EMB_ERR_ARG;
            cp->g[t][k] = c;
        }
    return TT_EMB_OK;
}

int tt_emb_forward(tt_emb_t h, const float *const *cores, const int64_t *indices, const int64_t *offsets,
                   int64_t B, int64_t nnz, float *out, void *ws, size_t ws_bytes, uint32_t flags, void *stream)
{
    try {
        Plan p;
        int rc = check_call(h, B, nnz, indices, offsets, ws, ws_bytes, &p, (flags & TT_EMB_KEEP_PREFIX) != 0);
        if (rc) return rc;
        if (B > 0 && !out) return TT_EMB_ERR_ARG;
        if (h->K >= 4) {
            // tables of K >= 4 cores: prefix reuse at every prefix length
            if (flags & (TT_EMB_KEEP_PREFIX | TT_EMB_ATOMIC_POOL)) return TT_EMB_ERR_ARG;
            KCorePtrs kc{};
            if ((rc = kcore_ptrs(h, cores, &kc))) return rc;
            if ((rc = set_device(h))) return rc;
            hipStream_t s = (hipStream_t)stream;
            if (!(flags & TT_EMB_REUSE_GROUPING)) {
                if ((rc = hip_status(launch_grouping(p, indices, offsets, s)))) return rc;
            }
            return hip_status(launch_forward_k(p, kc, offsets, out, s));
        }
        CorePtrs cp{};
        if ((rc = core_ptrs(h, cores, &cp))) return rc;
        if ((flags & TT_EMB_KEEP_PREFIX) && !h->keep_prefix) return TT_EMB_ERR_ARG;
        if ((flags & TT_EMB_KEEP_PREFIX) && (flags & TT_EMB_ATOMIC_POOL)) return TT_EMB_ERR_ARG;
        p.keep_c = (flags & TT_EMB_KEEP_PREFIX) ? 1 : 0;
        p.pool_atomic = (flags & TT_EMB_ATOMIC_POOL) ? 1 : 0;
        if ((rc = set_device(h))) return rc;
        hipStream_t s = (hipStream_t)stream;
        if (!(flags & TT_EMB_REUSE_GROUPING)) {
            if ((rc = hip_status(launch_grouping(p, indices, offsets, s)))) return rc;
        }
        return hip_status(launch_forward(p, cp, offsets, out, s));
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

int tt_emb_forward_noalloc(tt_emb_t h, const float *const *cores, const int64_t *indices, const int64_t *offsets,
                           int64_t B, int64_t nnz, float *out, uint32_t flags, void *stream)
{
    try {
        if (!h || B < 0 || nnz < 0 || nnz >= (int64_t)0x7fffffff) return TT_EMB_ERR_ARG;
        if (flags & TT_EMB_KEEP_PREFIX) return TT_EMB_ERR_ARG;
        size_t need = 0;
        plan_workspace(h, B, nnz, nullptr, nullptr, &need);
        if (need > TT_EMB_NOALLOC_SCRATCH_BYTES) return TT_EMB_ERR_TOO_LARGE;
        int rc = set_device(h);
        if (rc) return rc;
        if (h->device < 0 || h->device >= kMaxDevices || !noalloc_done[h->device]) return TT_EMB_ERR_HIP;
        void *ws = noalloc_ptr[h->device];
        if (!ws) return TT_EMB_ERR_HIP;
        return tt_emb_forward(h, cores, indices, offsets, B, nnz, out, ws, TT_EMB_NOALLOC_SCRATCH_BYTES, flags,
                              stream);
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

int tt_emb_backward(tt_emb_t h, const float *grad_out, const float *const *cores, const int64_t *indices,
                    const int64_t *offsets, int64_t B, int64_t nnz, float *const *core_grads, void *ws,
                    size_t ws_bytes, uint32_t flags, void *stream)
{
    try {
        Plan p;
        int rc = check_call(h, B, nnz, indices, offsets, ws, ws_bytes, &p, true);
        if (rc) return rc;
        if (B > 0 && !grad_out) return TT_EMB_ERR_ARG;
        if (h->K >= 4) {
            // tables of K >= 4 cores: the chain reversed with prefix sharing;
            // REUSE_PREFIX: the level intermediates in ws are the forward's
            if ((flags & TT_EMB_REUSE_PREFIX) && !(flags & TT_EMB_REUSE_GROUPING)) return TT_EMB_ERR_ARG;
            p.reuse_c = (flags & TT_EMB_REUSE_PREFIX) ? 1 : 0;
            KCorePtrs kc{};
            if ((rc = kcore_ptrs(h, cores, &kc))) return rc;
            if (!core_grads) return TT_EMB_ERR_ARG;
            for (int i = 0; i < h->T * h->K; ++i)
                if (bad_ptr(core_grads[i])) return TT_EMB_ERR_ARG;
            if ((rc = set_device(h))) return rc;
            hipStream_t s = (hipStream_t)stream;
            if (!(flags & TT_EMB_REUSE_GROUPING)) {
                if ((rc = hip_status(launch_grouping(p, indices, offsets, s)))) return rc;
            }
            return hip_status(launch_backward_k(p, grad_out, kc, offsets, core_grads, s));
        }
        CorePtrs cp{};
        if ((rc = core_ptrs(h, cores, &cp))) return rc;
        if (!core_grads) return TT_EMB_ERR_ARG;
        GradPtrs gp{};
        for (int t = 0; t < h->T; ++t)
            for (int k = 0; k < 3; ++k) {
                float *g = core_grads[3 * t + k];
                if (bad_ptr(g)) return TT_EMB_ERR_ARG;
                gp.g[t][k] = g;
            }
        if ((flags & TT_EMB_REUSE_PREFIX) && (!h->keep_prefix || !(flags & TT_EMB_REUSE_GROUPING)))
            return TT_EMB_ERR_ARG;
        p.reuse_c = (flags & TT_EMB_REUSE_PREFIX) ? 1 : 0;
        if ((rc = set_device(h))) return rc;
        hipStream_t s = (hipStream_t)stream;
        if (!(flags & TT_EMB_REUSE_GROUPING)) {
            if ((rc = hip_status(launch_grouping(p, indices, offsets, s)))) return rc;
        }
        return hip_status(launch_backward(p, grad_out, cp, offsets, gp, s));
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

int tt_emb_sgd_update(tt_emb_t h, float *const *cores, const float *const *core_grads, float lr, void *stream)
{
    if (!h || !cores || !core_grads) return TT_EMB_ERR_ARG;
    const int nc = h->K * h->T; // cores of the handle (three per table, or K)
    for (int i = 0; i < nc; ++i)
        if (bad_ptr(cores[i]) || bad_ptr(core_grads[i])) return TT_EMB_ERR_ARG;
    int rc = set_device(h);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    Timing *tm = (h->timing && h->timing->on) ? h->timing : nullptr;
    timer_begin(tm, TM_SGD, s);
    std::vector<int64_t> cnt((size_t)nc);
    for (int t = 0; t < h->T; ++t) {
        if (h->K >= 4) {
            const KTab &kt = h->ktabs[t];
            for (int k = 0; k < h->K; ++k) cnt[(size_t)h->K * t + k] = (int64_t)kt.n[k] * kt.R[k] * kt.d[k] * kt.R[k + 1];
            continue;
        }
        const TableDesc &d = h->tabs[t];
        cnt[3 * t + 0] = (int64_t)d.n1 * d.d1 * d.R1;
        cnt[3 * t + 1] = (int64_t)d.n2 * d.R1 * d.d2 * d.R2;
        cnt[3 * t + 2] = (int64_t)d.n3 * d.R2 * d.d3;
    }
    if (launch_sgd(cores, core_grads, cnt.data(), nc, lr, s) != hipSuccess) return TT_EMB_ERR_HIP;
    timer_end(tm, TM_SGD, s);
    return TT_EMB_OK;
}

int tt_emb_timing_enable(tt_emb_t h, int32_t enable)
{
    if (!h) return TT_EMB_ERR_ARG;
    try {
        if (!enable) {
            if (h->timing) h->timing->on = false;
            return TT_EMB_OK;
        }
        int rc = set_device(h);
        if (rc) return rc;
        if (!h->timing) {
            h->timing = new Timing();
            for (int id = 0; id < TM_COUNT; ++id)
                for (int k = 0; k < 2; ++k) {
                    h->timing->ev[id][k].resize(Timing::kRing);
                    for (auto &e : h->timing->ev[id][k])
                        if (hipEventCreate(&e) != hipSuccess) {
                            free_timing(h);
                            return TT_EMB_ERR_HIP;
                        }
                }
        }
        h->timing->on = true;
        return TT_EMB_OK;
    } catch (...) {
        return TT_EMB_ERR_NOMEM;
    }
}

int tt_emb_timing_read(tt_emb_t h, double *ms, int32_t *count)
{
    if (!h) return TT_EMB_ERR_ARG;
    int rc = set_device(h);
    if (rc) return rc;
    if (hipDeviceSynchronize() != hipSuccess) return TT_EMB_ERR_HIP;
    for (int id = 0; id < TM_COUNT; ++id) {
        double tot = 0.0;
        int n = h->timing ? h->timing->used[id] : 0;
        for (int k = 0; k < n; ++k) {
            float x = 0.f;
            if (hipEventElapsedTime(&x, h->timing->ev[id][0][k], h->timing->ev[id][1][k]) != hipSuccess)
                return TT_EMB_ERR_HIP;
            tot += x;
        }
        if (ms) ms[id] = tot;
        if (count) count[id] = n;
        if (h->timing) h->timing->used[id] = 0;
    }
    return TT_EMB_OK;
}

const char *tt_emb_timer_name(int32_t id)
{
    static const char *names[TM_COUNT] = {"group_sort", "group_rle", "contract", "pool",
                                          "bwd_gather", "bwd_contract", "bwd_reduce", "sgd",
                                          "fwd_r8", "fwd_r16", "fwd_r32", "fwd_r64",
                                          "bwd_r8", "bwd_r16", "bwd_r32", "bwd_r64",
                                          "stage_decode", "stage_sort", "stage_unique", "stage_prefix",
                                          "stage_order", "stage_worklist"};
    static_assert(TM_COUNT == TT_EMB_NUM_TIMERS, "one name per timer");
    return (id >= 0 && id < TM_COUNT) ? names[id] : nullptr;
}

int tt_emb_grouping_view(tt_emb_t h, const void *ws, size_t ws_bytes, int64_t B, int64_t nnz, void *stream,
                         tt_emb_grouping *view)
{
    if (!view) return TT_EMB_ERR_ARG;
    Plan p;
    int64_t dummy_off[1] = {0};
    int rc = check_call(h, B, nnz, nnz > 0 ? dummy_off : nullptr, dummy_off, const_cast<void *>(ws), ws_bytes, &p, false);
    if (rc) return rc;
    if ((rc = set_device(h))) return rc;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TT_EMB_ERR_HIP;
    int32_t ctrl[CTRL_N];
    if (hipMemcpy(ctrl, p.ws.ctrl, sizeof(ctrl), hipMemcpyDeviceToHost) != hipSuccess) return TT_EMB_ERR_HIP;
    view->nnz = nnz;
    view->num_unique = ctrl[CTRL_U];
    view->num_groups = ctrl[CTRL_G];
    view->perm = p.ws.perm;
    view->uniq_row = p.ws.uniq_row;
    view->uniq_start = p.ws.uniq_start;
    view->inv = p.ws.inv;
    view->grp_prefix = p.ws.grp_prefix;
    view->grp_start = p.ws.grp_start;
    view->tab_uniq_start = p.ws.tab_uniq_start;
    view->tab_grp_start = p.ws.tab_grp_start;
    view->num_units = ctrl[CTRL_UNITS];
    view->num_tiles = ctrl[CTRL_TILES];
    view->num_chunks = ctrl[CTRL_CHUNKS];
    view->num_split_tiles = ctrl[CTRL_SPLIT];
    view->num_steals = ctrl[CTRL_STEALS];
    view->num_ckpt_hits = ctrl[CTRL_CKPT_HIT];
    view->num_ckpt_misses = ctrl[CTRL_CKPT_MISS];
    return TT_EMB_OK;
}

int tt_emb_block_stats(tt_emb_t h, const void *ws, size_t ws_bytes, int64_t B, int64_t nnz, int32_t kernel,
                       void *stream, tt_emb_block_stat *out, int32_t cap, int32_t *nblocks, int64_t *clock_khz)
{
    static_assert(sizeof(tt_emb_block_stat) == sizeof(BlockStat), "public block record mirrors BlockStat");
    if (!out || !nblocks || !clock_khz || cap < 0 || kernel < 0 || kernel >= kStatKernels) return TT_EMB_ERR_ARG;
    Plan p;
    int64_t dummy_off[1] = {0};
    int rc = check_call(h, B, nnz, nnz > 0 ? dummy_off : nullptr, dummy_off, const_cast<void *>(ws), ws_bytes, &p, false);
    if (rc) return rc;
    if ((rc = set_device(h))) return rc;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TT_EMB_ERR_HIP;
    int rate = 0;
    if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, h->device) != hipSuccess) return TT_EMB_ERR_HIP;
    *clock_khz = rate;
    const BlockStat *src = p.ws.bstat + (size_t)kernel * kStatBlocks;
    BlockStat first;
    if (hipMemcpy(&first, src, sizeof(first), hipMemcpyDeviceToHost) != hipSuccess) return TT_EMB_ERR_HIP;
    int n = first.nb < 0 ? 0 : first.nb;
    if (n > kStatBlocks) n = kStatBlocks;
    if (n > cap) n = cap;
    *nblocks = n;
    if (n > 0 && hipMemcpy(out, src, sizeof(BlockStat) * (size_t)n, hipMemcpyDeviceToHost) != hipSuccess)
        return TT_EMB_ERR_HIP;
    return TT_EMB_OK;
}

int tt_emb_victim_order(int32_t me, int32_t nb, int32_t *order)
{
    if (!order || nb < 8 || (nb & 7) || me < 0 || me >= nb) return TT_EMB_ERR_ARG;
    for (int vi = 0; vi < nb; ++vi) order[vi] = victim_of(me, vi, nb);
    return TT_EMB_OK;
}

int tt_emb_poll_error(tt_emb_t h, const void *ws, void *stream)
{
    if (!h || !ws) return TT_EMB_ERR_ARG;
    int rc = set_device(h);
    if (rc) return rc;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TT_EMB_ERR_HIP;
    int32_t err = 0;
    if (hipMemcpy(&err, ws, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return TT_EMB_ERR_HIP;
    if (err & ERRB_CAPACITY) return TT_EMB_ERR_WORKSPACE;
    if (err & ERRB_OFFSETS) return TT_EMB_ERR_OFFSETS;
    if (err & ERRB_INDEX) return TT_EMB_ERR_INDEX;
    return TT_EMB_OK;
}

const char *tt_emb_status_string(int status)
{
    switch (status) {
    case TT_EMB_OK: return "ok";
    case TT_EMB_ERR_ARG: return "invalid argument";
    case TT_EMB_ERR_INDEX: return "index out of range";
    case TT_EMB_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TT_EMB_ERR_UNSUPPORTED: return "shape not supported by this build";
    case TT_EMB_ERR_HIP: return "HIP runtime error";
    case TT_EMB_ERR_NOMEM: return "out of memory";
    case TT_EMB_ERR_OFFSETS: return "malformed offsets";
    case TT_EMB_ERR_TOO_LARGE: return "input too large for the fixed scratch of the no-allocation forward";
    default: return "unknown status";
    }
}

} // extern "C"
