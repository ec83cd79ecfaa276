"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Bars: grouping arrays bit-exact; pooled outputs, core gradients and SGD
updates within max|gpu - oracle| <= 1e-4 * max|oracle|, the max taken per
table slice of the output and per core; the GPU path must also be
bit-reproducible run to run and across scheduling modes.
"""

import numpy as np
import pytest
import torch

import oracle
import tensor_train_compressed_gather_amd as tt
from tensor_train_compressed_gather_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-4


def _opts(**kw):
    o = tt.tt_emb_options()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


class Run:
    """Upload a workload and drive the library on it."""

    def __init__(self, w, **opt):
        print(f"[case] {w.name} T={w.T} B={w.B} nnz={w.nnz} opts={opt}", flush=True)
        self.w = w
        self.emb = tt.TTEmbeddingBag(w.tables, DEV, _opts(**opt) if opt else None)
        self.cores = [torch.from_numpy(c).to(DEV) for c in w.cores]
        self.idx = torch.from_numpy(w.indices).to(DEV)
        self.off = torch.from_numpy(w.offsets).to(DEV)

    def forward(self, flags=0):
        out = self.emb.forward(self.cores, self.idx, self.off, self.w.B, flags=flags)
        torch.cuda.synchronize()
        return out

    def backward(self, grad_out, flags=0):
        g = torch.from_numpy(grad_out).to(DEV)
        grads = self.emb.backward(g, self.cores, self.idx, self.off, self.w.B, flags=flags)
        torch.cuda.synchronize()
        return grads

    def grouping(self):
        g = self.emb.grouping(self.w.B, self.w.nnz)
        return {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in g.items()}


def assert_out_close(w, got, ref):
    col = w.col_offsets()
    for t in range(w.T):
        r = ref[:, col[t]:col[t + 1]]
        g = got[:, col[t]:col[t + 1]]
        scale = np.abs(r).max()
        err = np.abs(g.astype(np.float64) - r).max() if r.size else 0.0
        assert err <= TOL * max(scale, 1e-30), (t, err, scale)


def assert_grads_close(got, ref):
    for k, (g, r) in enumerate(zip(got, ref)):
        scale = np.abs(r).max()
        err = np.abs(g.astype(np.float64) - r).max()
        assert err <= TOL * max(scale, 1e-30), (k, err, scale)


def check_grouping(run):
    ref = oracle.grouping(run.w)
    got = run.grouping()
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k
    return got


SMALL = [(1, None), (2, 4096), (3, 512), (4, 128)]


@pytest.mark.parametrize("cfg,bags", SMALL)
def test_grouping_is_bit_exact(cfg, bags):
    run = Run(W.make_workload(cfg, bags=bags))
    run.forward()
    check_grouping(run)
    assert run.emb.poll_error() == 0


@pytest.mark.parametrize("cfg,bags", SMALL)
def test_forward_matches_oracle(cfg, bags):
    w = W.make_workload(cfg, bags=bags)
    run = Run(w)
    out = run.forward().cpu().numpy()
    assert_out_close(w, out, oracle.forward(w))


@pytest.mark.parametrize("opt", [
    dict(sched_mode=1), dict(sched_mode=2), dict(sched_mode=3, chunk_rows=1), dict(sched_mode=3, chunk_rows=3),
    dict(num_blocks=8), dict(group_mode=2), dict(sched_mode=1, num_blocks=8, chunk_rows=2),
    # the smallest grids: a num_blocks of 1 or 3 is rounded up to 8 (one
    # round over the 8 XCDs), so each class kernel runs 8 x its blocks per CU
    dict(num_blocks=1), dict(num_blocks=1, sched_mode=2), dict(num_blocks=3, sched_mode=1),
    dict(num_blocks=3, sched_mode=3, chunk_rows=2),
])
def test_scheduling_modes_are_bit_identical(opt):
    # every mode matches the oracle on its own, and the default path bit for bit
    w = W.make_workload(4, bags=64)
    base = Run(w).forward().cpu().numpy()
    other = Run(w, **opt).forward().cpu().numpy()
    assert_out_close(w, other, oracle.forward(w))
    assert np.array_equal(base, other)


def test_l2_checkpoints_are_consumed_at_full_size():
    # stealing with L2 checkpoints on the 26-table batch with short chunks (many
    # split prefix tiles): some chunks of split tiles must find a published
    # checkpoint and use it, and the output must still match the oracle and
    # the default path
    w = W.make_workload(4)
    base = Run(w).forward().cpu().numpy()
    run = Run(w, sched_mode=3, chunk_rows=4)
    out = run.forward().cpu().numpy()
    c = run.grouping()["counts"]
    print(f"[ckpt] split tiles {c['num_split_tiles']} steals {c['num_steals']} "
          f"hits {c['num_ckpt_hits']} misses {c['num_ckpt_misses']}", flush=True)
    assert c["num_split_tiles"] > 0 and c["num_ckpt_hits"] > 0
    assert np.array_equal(base, out)
    rng = np.random.default_rng(44)
    bags = np.unique(np.concatenate([[0, w.B - 1], rng.integers(0, w.B, 300)]))
    assert_out_close(w, out[bags], oracle.forward(w, bags=bags))


def test_generic_kernels_match_oracle():
    w = W.make_workload(4, bags=32)
    run = Run(w, force_generic=1)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward(w))


def test_shapes_outside_the_mfma_classes():
    tables = [W.Table(57, (3, 4, 5), (2, 3, 2), (1, 3, 2, 1), 0.3, "uniform"),
              W.Table(30, (2, 3, 5), (3, 1, 2), (1, 2, 4, 1), 0.3, "uniform"),
              W.Table(1000, (10, 10, 10), (4, 4, 16), (1, 16, 16, 1), 0.1, "uniform"),
              W.Table(500, (8, 8, 8), (1, 3, 5), (1, 24, 40, 1), 0.1, "uniform")]
    rng = np.random.default_rng(5)
    lens = [rng.integers(0, 9, size=40) for _ in tables]
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    w = W.make_custom(tables, lens, idx, seed=5)
    run = Run(w)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward(w))
    check_grouping(run)
    go = np.random.default_rng(6).standard_normal((w.B, w.sum_D)).astype(np.float32)
    w.grad_out = go
    got = [g.cpu().numpy() for g in run.backward(go)]
    assert_grads_close(got, oracle.backward(w))


def test_backward_with_split_runs():
    # n2 = 2 and n1 = 200: each (table, i2) run holds ~200 prefix units (~50
    # tiles), more than a backward piece (16 tiles), so the rank-16 and
    # rank-32 runs are cut into pieces whose dG2 partials are summed in order;
    # the rank-64 table keeps whole runs
    tables = [W.Table(3200, (200, 2, 8), (4, 4, 4), (1, R, R, 1), 0.1, "uniform") for R in (16, 32, 64)]
    rng = np.random.default_rng(11)
    lens = [rng.integers(16, 33, size=256) for _ in tables]
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    w = W.make_custom(tables, lens, idx, seed=11)
    w.grad_out = np.random.default_rng(12).standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward(w))
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))
    # the split classes ran more pieces than runs (2 runs per table)
    for r in (16, 32):
        st = run.emb.block_stats(w.B, w.nnz, f"bwd_r{r}")
        assert int(st["work"].sum()) > 2, (r, int(st["work"].sum()))
    assert int(run.emb.block_stats(w.B, w.nnz, "bwd_r64")["work"].sum()) == 2
    again = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    for g0, g1 in zip(got, again):
        assert np.array_equal(g0, g1)


def test_edge_cases_empty_bags_single_prefix_and_no_lookups():
    tab = W.Table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1), 0.1, "uniform")
    rows = (3 * 10 + 7) * 10 + np.arange(10)
    lens = [np.array([0, 4, 0, 300, 1, 0])]
    idx = [np.random.default_rng(7).choice(rows, size=int(lens[0].sum()))]
    w = W.make_custom([tab], lens, idx, seed=7)
    for opt in ({}, dict(chunk_rows=1), dict(group_mode=2)):
        run = Run(w, **opt)
        out = run.forward().cpu().numpy()
        assert_out_close(w, out, oracle.forward(w))
        assert not out[[0, 2, 5]].any()
        check_grouping(run)
    w0 = W.make_custom([tab], [np.array([0, 0, 0])], [np.zeros(0, np.int64)], seed=8)
    run = Run(w0)
    out = run.forward().cpu().numpy()
    assert out.shape == (3, 16) and not out.any()
    go = np.ones((3, 16), np.float32)
    grads = run.backward(go)
    assert all(not g.any().item() for g in grads)


def test_hot_row_longer_than_a_gather_task():
    tab = W.Table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1), 0.1, "uniform")
    rng = np.random.default_rng(9)
    lens = [rng.integers(20, 60, size=64)]
    n = int(lens[0].sum())
    idx = [np.where(rng.random(n) < 0.7, 421, rng.integers(0, 1000, n))]
    w = W.make_custom([tab], lens, idx, seed=9)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward(w))
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))


def test_gradient_gather_runs_at_task_edges():
    # Sorted lookup runs (one per distinct row) laid against the 256-position
    # gather tasks: a run ending exactly on a task edge, one filling a task, one
    # crossing two edges (a whole task in the middle), single lookups; plus a
    # 512-column table whose rows take two column passes of a lane group.
    counts = [100, 156, 256, 600, 1, 300, 3, 255, 2]
    tab_a = W.Table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1), 0.1, "uniform")
    tab_b = W.Table(64, (4, 4, 4), (4, 4, 32), (1, 4, 4, 1), 0.1, "uniform")
    rng = np.random.default_rng(11)
    rows_a = np.repeat(np.arange(len(counts)) * 37, counts)
    rng.shuffle(rows_a)
    B = 64
    cut = np.sort(rng.choice(np.arange(1, rows_a.size), size=B - 1, replace=False))
    len_a = np.diff(np.concatenate([[0], cut, [rows_a.size]]))
    len_b = rng.integers(0, 30, size=B)
    nb = int(len_b.sum())
    rows_b = np.where(rng.random(nb) < 0.5, 13, rng.integers(0, 64, nb))
    w = W.make_custom([tab_a, tab_b], [len_a, len_b], [rows_a, rows_b], seed=11)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward(w))
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))
    again = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert all(np.array_equal(a, b) for a, b in zip(got, again))


@pytest.mark.parametrize("cfg,bags", [(1, None), (3, 256), (5, 64)])
def test_backward_matches_oracle(cfg, bags):
    w = W.make_workload(cfg, bags=bags)
    if w.grad_out is None:
        w.grad_out = W.make_grad_out(w, 100 + cfg)
    run = Run(w)
    run.forward()
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))


def test_backward_on_the_finite_difference_instance():
    w = W.make_fd_instance()
    run = Run(w)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out)]
    assert_grads_close(got, oracle.backward(w))


def test_sgd_update_matches_oracle_delta():
    w = W.make_workload(5, bags=32)
    run = Run(w)
    before = [c.clone() for c in run.cores]
    run.forward()
    grads = run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)
    run.emb.sgd_update(run.cores, grads, w.lr)
    torch.cuda.synchronize()
    dG = oracle.backward(w)
    for k in range(3 * w.T):
        delta = (run.cores[k] - before[k]).cpu().numpy().astype(np.float64)
        ref = oracle.sgd_delta(dG[k], w.lr)
        scale = np.abs(ref).max()
        # the update is rounded to the fp32 grid of the core values
        ulp = np.spacing(np.abs(before[k].cpu().numpy())).max()
        assert np.abs(delta - ref).max() <= TOL * scale + ulp, k


def test_kernel_timers_record_every_launch():
    # the per-kernel timers behind the bench's roofline: one interval per call
    # of each rank class present, inside its phase
    w = W.make_workload(5, bags=64)
    run = Run(w)
    h = run.emb.handle
    tt.tt_emb_timing_read(h)
    tt.tt_emb_timing_enable(h, True)
    for _ in range(3):
        run.forward()
        run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)
    tt.tt_emb_timing_enable(h, False)
    ph = tt.tt_emb_timing_read(h)
    ranks = {t.R[1] for t in w.tables}
    for r in (8, 16, 32, 64):
        for p in ("fwd", "bwd"):
            ms, n = ph[f"{p}_r{r}"]
            assert n == (3 if r in ranks else 0), (p, r, n)
            if n:
                assert 0 < ms <= ph["contract" if p == "fwd" else "bwd_contract"][0]
    assert ph["contract"][1] == 3 and ph["bwd_contract"][1] == 3


@pytest.mark.parametrize("sched", [1, 3])
def test_block_records_account_for_every_chunk(sched):
    # the per-block scheduling records: one per block of each persistent
    # launch, and between them every forward chunk and unique row (each is
    # computed exactly once) and every backward chunk
    w = W.make_workload(5, bags=64)
    run = Run(w, sched_mode=sched)
    run.forward()
    run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)
    cnt = run.grouping()["counts"]
    ranks = {t.R[1] for t in w.tables}
    fwork = frows = bchunks = 0
    for r in (8, 16, 32, 64):
        for p in ("fwd", "bwd"):
            st = run.emb.block_stats(w.B, w.nnz, f"{p}_r{r}")
            assert (st is not None) == (r in ranks), (p, r)
            if st is None:
                continue
            n = len(st["work"])
            assert n == st["grid"] and n >= 256, (p, r, n)
            assert np.all(st["t1_us"] >= st["t0_us"]) and st["clock_khz"] > 0
            assert np.all(st["work"] >= 0) and np.all(st["rows"] >= 0)
            # hardware ids decode into at most 8 XCDs of 4 engines
            assert np.all((st["cu"] >> 7) < 8)
            if p == "fwd":
                fwork += int(st["work"].sum())
                frows += int(st["rows"].sum())
            else:
                bchunks += int(st["rows"].sum())
            bal = tt.block_balance(st)
            assert 0 < bal["eff_blocks"] <= 1 and 0 < bal["eff_cus"] <= 1
    assert fwork == cnt["num_chunks"] and bchunks == cnt["num_chunks"]
    assert frows == cnt["num_unique"]
    with pytest.raises(tt.TTEmbError):
        run.emb.block_stats(w.B, w.nnz, 8)


def test_bit_reproducible_forward_and_backward():
    w = W.make_workload(5, bags=64)
    run = Run(w)
    o1 = run.forward().cpu().numpy()
    g1 = [g.cpu().numpy() for g in run.backward(w.grad_out)]
    for _ in range(3):
        assert np.array_equal(run.forward().cpu().numpy(), o1)
        g2 = [g.cpu().numpy() for g in run.backward(w.grad_out)]
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("opt", [dict(), dict(sched_mode=2), dict(sched_mode=3, chunk_rows=4),
                                 dict(num_blocks=16, sched_mode=2)])
def test_bit_identical_over_ten_runs(opt):
    # the whole training step (kept prefix intermediates, split backward runs,
    # stealing or not) hashed over ten runs of each configuration
    import hashlib

    w = W.make_workload(5, bags=96)
    run = Run(w, keep_prefix=1, **opt)
    go = torch.from_numpy(w.grad_out).to(DEV)
    digests = set()
    for _ in range(10):
        out = run.emb.forward(run.cores, run.idx, run.off, w.B, flags=tt.TT_EMB_KEEP_PREFIX)
        grads = run.emb.backward(go, run.cores, run.idx, run.off, w.B,
                                 flags=tt.TT_EMB_REUSE_GROUPING | tt.TT_EMB_REUSE_PREFIX)
        torch.cuda.synchronize()
        h = hashlib.sha256(out.cpu().numpy().tobytes())
        for g in grads:
            h.update(g.cpu().numpy().tobytes())
        digests.add(h.hexdigest())
    assert len(digests) == 1


def test_device_detected_errors():
    w = W.make_workload(1)
    bad = w.indices.copy()
    bad[17] = 1000
    run = Run(w)
    run.idx = torch.from_numpy(bad).to(DEV)
    run.forward()
    assert run.emb.poll_error() == tt.TT_EMB_ERR_INDEX
    run.idx = torch.from_numpy(w.indices).to(DEV)
    run.forward()
    assert run.emb.poll_error() == 0
    off = w.offsets.copy()
    off[5] = off[7] + 3
    run.off = torch.from_numpy(off).to(DEV)
    run.forward()
    assert run.emb.poll_error() == tt.TT_EMB_ERR_OFFSETS


def test_host_detected_errors():
    w = W.make_workload(1)
    run = Run(w)
    ws = run.emb.workspace(w.B, w.nnz)
    out = torch.empty((w.B, w.sum_D), device=DEV)
    with pytest.raises(tt.TTEmbError) as e:
        tt.tt_emb_forward(run.emb.handle, run.cores, run.idx, run.off, w.B, out, ws[:1024])
    assert e.value.status == tt.TT_EMB_ERR_WORKSPACE
    cores = list(run.cores)
    cores[1] = cores[1].view(-1)[1:]
    with pytest.raises(tt.TTEmbError) as e:
        tt.tt_emb_forward(run.emb.handle, cores, run.idx, run.off, w.B, out, ws)
    assert e.value.status == tt.TT_EMB_ERR_ARG
    # lookups but no bags (offsets [0], nnz > 0)
    off0 = torch.zeros(1, dtype=torch.int64, device=DEV)
    with pytest.raises(tt.TTEmbError) as e:
        tt.tt_emb_forward(run.emb.handle, run.cores, run.idx, off0, 0, out[:0], ws)
    assert e.value.status == tt.TT_EMB_ERR_ARG


# ------------------------------------------------ fused atomic pooling

def _close_to(a, b, rel):
    scale = np.abs(b).max()
    assert np.abs(a.astype(np.float64) - b).max() <= rel * max(scale, 1e-30)


@pytest.mark.parametrize("cfg,bags,opt", [
    (1, None, {}), (2, 4096, {}), (3, 512, {}), (4, 128, {}),
    (4, 128, {"chunk_rows": 2}),                  # split tiles
    (4, 128, {"group_mode": 2, "sched_mode": 1}),  # one unit per unique row, static ranges
])
def test_fused_atomic_pooling_matches_oracle(cfg, bags, opt):
    # the non-deterministic fast mode: rows pooled inside the contraction with
    # float atomics; equal to the bag-major result up to summation order
    w = W.make_workload(cfg, bags=bags)
    run = Run(w, **opt)
    fused = run.forward(flags=tt.TT_EMB_ATOMIC_POOL).cpu().numpy()
    assert_out_close(w, fused, oracle.forward(w))
    det = run.forward(flags=tt.TT_EMB_REUSE_GROUPING).cpu().numpy()
    _close_to(fused, det, 1e-5)
    assert run.emb.poll_error() == 0


def test_fused_atomic_pooling_with_generic_tables_and_empty_bags():
    tables = [W.Table(57, (3, 4, 5), (2, 3, 2), (1, 3, 2, 1), 0.3, "uniform"),      # generic kernels
              W.Table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1), 0.1, "zipf", 1.1),
              W.Table(1000, (10, 10, 10), (4, 4, 16), (1, 16, 16, 1), 0.1, "uniform")]  # D = 256
    rng = np.random.default_rng(11)
    lens = [rng.integers(0, 9, size=48) for _ in tables]
    lens[1][:5] = 0
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    idx[1] = rng.integers(0, 12, size=idx[1].size)  # hot rows, repeated within bags
    w = W.make_custom(tables, lens, idx, seed=11)
    for opt in ({}, {"force_generic": 1}):
        run = Run(w, **opt)
        out = run.forward(flags=tt.TT_EMB_ATOMIC_POOL).cpu().numpy()
        assert_out_close(w, out, oracle.forward(w))
        col = w.col_offsets()
        assert not out[:5, col[1]:col[2]].any()
    with pytest.raises(tt.TTEmbError) as e:  # not with kept prefixes
        Run(w, keep_prefix=1).forward(flags=tt.TT_EMB_ATOMIC_POOL | tt.TT_EMB_KEEP_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_ARG


# ------------------------------------------------ kept prefix intermediates

REUSE = tt.TT_EMB_REUSE_GROUPING | tt.TT_EMB_REUSE_PREFIX


@pytest.mark.parametrize("cfg,bags,opt", [
    (3, 256, {}),
    (5, 64, {}),
    (5, 64, {"chunk_rows": 3}),                   # many tiles split over chunks (checkpoints)
    (5, 64, {"chunk_rows": 2, "sched_mode": 1}),  # split tiles, static ranges
    (4, 128, {"group_mode": 2}),                  # one unit per unique row
])
def test_kept_prefix_backward_matches_oracle(cfg, bags, opt):
    # training mode: the forward keeps every prefix unit's C_p, the backward
    # reads it instead of recomputing it
    w = W.make_workload(cfg, bags=bags)
    if w.grad_out is None:
        w.grad_out = W.make_grad_out(w, 200 + cfg)
    run = Run(w, keep_prefix=1, **opt)
    out = run.forward(flags=tt.TT_EMB_KEEP_PREFIX).cpu().numpy()
    assert_out_close(w, out, oracle.forward(w))
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=REUSE)]
    assert_grads_close(got, oracle.backward(w))
    # the recomputing backward on the same grouping sums C in another order:
    # equal to rounding
    rec = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    for k, (a, b) in enumerate(zip(got, rec)):
        scale = np.abs(b).max()
        assert np.abs(a.astype(np.float64) - b).max() <= 1e-5 * max(scale, 1e-30), k
    again = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=REUSE)]
    for a, b in zip(got, again):
        assert np.array_equal(a, b)


def test_prefix_flags_need_a_keep_prefix_handle():
    w = W.make_workload(1)
    w.grad_out = W.make_grad_out(w, 7)
    run = Run(w)
    with pytest.raises(tt.TTEmbError) as e:
        run.forward(flags=tt.TT_EMB_KEEP_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_ARG
    run = Run(w, keep_prefix=1)
    run.forward(flags=tt.TT_EMB_KEEP_PREFIX)
    with pytest.raises(tt.TTEmbError) as e:  # the kept prefixes need the kept grouping
        run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_ARG
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=REUSE)]
    assert_grads_close(got, oracle.backward(w))


# ------------------------------------------------------------ full sizes

@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_forward_sampled_bags(cfg):
    w = W.make_workload(cfg)
    run = Run(w)
    out = run.forward().cpu().numpy()
    g = check_grouping(run)
    print(f"[full] cfg{cfg} counts={g['counts']}", flush=True)
    rng = np.random.default_rng(cfg)
    bags = np.unique(np.concatenate([[0, w.B - 1], rng.integers(0, w.B, 600)]))
    ref = oracle.forward(w, bags=bags)
    assert_out_close(w, out[bags], ref)


@pytest.mark.parametrize("keep", [False, True])
def test_full_size_training_step_sampled_slices(keep):
    w = W.make_workload(5)
    run = Run(w, keep_prefix=1) if keep else Run(w)
    run.forward(flags=tt.TT_EMB_KEEP_PREFIX if keep else 0)
    grads = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=REUSE if keep else tt.TT_EMB_REUSE_GROUPING)]
    rng = np.random.default_rng(55)
    tabs = [0, 7, 13, 25]
    sel = np.full((w.T, 3), -2, np.int64)
    for t in tabs:
        lo = w.offsets[t * w.B]
        i = int(w.indices[lo + rng.integers(0, 100)])
        sel[t] = np.unravel_index(i, w.tables[t].n)
    ref = oracle.backward(w, sel=sel)
    for t in tabs:
        for k in range(3):
            s = sel[t, k]
            r = ref[3 * t + k][s]
            g = grads[3 * t + k][s]
            scale = np.abs(r).max()
            assert scale > 0
            assert np.abs(g - r).max() <= TOL * scale, (t, k)


# ------------------------------------------------------ K >= 4 TT cores

def _three_digit_view(w):
    """The same lookups over tables whose rows split into (1, leading K-1
    digits, last digit): the grouping a K-core table set is sorted by."""
    tabs = []
    for t in w.tables:
        lead = int(np.prod(t.n[:-1]))
        tabs.append(W.Table(t.N, (1, lead, t.n[-1]), (1, 1, t.D), (1, 1, 1, 1), t.sigma, t.dist, t.alpha))
    return W.Workload(name=w.name + "_view", tables=tabs, B=w.B, cores=[], indices=w.indices,
                      offsets=w.offsets)


def _sub_bags(w, bags):
    """The lookups of the chosen bags of every table, as a workload of its own."""
    lens, idx = [], []
    for t in range(w.T):
        lo = w.offsets[t * w.B + bags]
        hi = w.offsets[t * w.B + bags + 1]
        lens.append(hi - lo)
        idx.append(np.concatenate([w.indices[a:b] for a, b in zip(lo, hi)]) if len(bags) else
                   np.zeros(0, np.int64))
    off = np.zeros(w.T * len(bags) + 1, np.int64)
    np.cumsum(np.concatenate(lens), out=off[1:])
    return W.Workload(name=w.name + "_sub", tables=w.tables, B=len(bags), cores=w.cores,
                      indices=np.concatenate(idx), offsets=off)


def _check_kcore(w, run):
    out = run.forward().cpu().numpy()
    assert out.shape == (w.B, w.sum_D)
    assert_out_close(w, out, oracle.forward_k(w))
    ref = oracle.grouping(_three_digit_view(w))
    got = run.grouping()
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k
    return out


@pytest.mark.parametrize("name,bags", [("k4", 256), ("k5", 256), ("k4", 3)])
def test_kcore_forward_matches_oracle(name, bags):
    w = W.make_kcore_workload(name, bags=bags)
    run = Run(w)
    out = _check_kcore(w, run)
    # bit-reproducible, and the same again from the kept grouping
    assert np.array_equal(out, run.forward().cpu().numpy())
    assert np.array_equal(out, run.forward(flags=tt.TT_EMB_REUSE_GROUPING).cpu().numpy())


def test_kcore_mixed_shapes_empty_bags_and_no_lookups():
    # K = 4 tables of unequal ranks and widths: a wide row (D = 512), ranks
    # that are no MFMA class, a table with a single leading prefix, empty bags
    tables = [W.Table(5000, (4, 5, 6, 50), (4, 4, 4, 8), (1, 8, 24, 12, 1), 0.2, "uniform"),
              W.Table(77, (2, 3, 2, 7), (3, 1, 2, 5), (1, 5, 3, 7, 1), 0.3, "uniform"),
              W.Table(999, (10, 10, 10, 1), (2, 2, 2, 2), (1, 16, 16, 16, 1), 0.2, "uniform"),
              W.Table(40000, (20, 20, 20, 5), (2, 4, 4, 4), (1, 32, 32, 32, 1), 0.05, "zipf", 1.1)]
    rng = np.random.default_rng(41)
    lens = [rng.integers(0, 12, size=50) for _ in tables]
    lens[1][:] = 0
    lens[2][5:] = 0
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    idx[0][: len(idx[0]) // 2] = 4321  # one hot row
    idx[3] = np.minimum(idx[3], 37)    # a single leading prefix (rows 0..37)
    w = W.make_custom(tables, lens, idx, seed=41)
    run = Run(w)
    out = _check_kcore(w, run)
    col = w.col_offsets()
    assert not out[:, col[1]:col[2]].any()
    assert not out[5:, col[2]:col[3]].any()
    w0 = W.make_custom(tables[:2], [np.zeros(4, np.int64)] * 2, [np.zeros(0, np.int64)] * 2, seed=42)
    run0 = Run(w0)
    out0 = run0.forward().cpu().numpy()
    assert out0.shape == (4, w0.sum_D) and not out0.any()


def test_kcore_full_size_sampled_bags():
    w = W.make_kcore_workload("k4")
    run = Run(w)
    out = run.forward().cpu().numpy()
    rng = np.random.default_rng(44)
    bags = np.unique(np.concatenate([[0, w.B - 1], rng.integers(0, w.B, 300)]))
    sub = _sub_bags(w, bags)
    assert_out_close(sub, out[bags], oracle.forward_k(sub))


def test_block_records_empty_before_any_persistent_launch():
    # a grouping clears the records; a K-core handle never launches the
    # persistent class kernels
    w = W.make_workload(5, bags=16)
    run = Run(w)
    ws = run.emb.workspace(w.B, w.nnz)
    tt.tt_emb_group(run.emb.handle, run.idx, run.off, w.B, ws)
    for k in tt.BLOCK_STAT_KERNELS:
        assert run.emb.block_stats(w.B, w.nnz, k) is None, k
    wk = W.make_kcore_workload("k4", bags=16)
    runk = Run(wk)
    runk.forward()
    runk.backward(np.zeros((wk.B, wk.sum_D), np.float32), flags=tt.TT_EMB_REUSE_GROUPING)
    for k in tt.BLOCK_STAT_KERNELS:
        assert runk.emb.block_stats(wk.B, wk.nnz, k) is None, k


def test_kcore_unsupported_calls_are_rejected():
    w = W.make_kcore_workload("k5", bags=8)
    run = Run(w)
    with pytest.raises(tt.TTEmbError) as e:
        run.forward(flags=tt.TT_EMB_KEEP_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_ARG
    with pytest.raises(tt.TTEmbError) as e:
        run.forward(flags=tt.TT_EMB_ATOMIC_POOL)
    assert e.value.status == tt.TT_EMB_ERR_ARG
    run.forward()
    with pytest.raises(tt.TTEmbError) as e:
        run.backward(np.zeros((w.B, w.sum_D), np.float32), flags=tt.TT_EMB_REUSE_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_ARG


@pytest.mark.parametrize("name,bags", [("k4", 256), ("k5", 256)])
def test_kcore_backward_matches_oracle(name, bags):
    w = W.make_kcore_workload(name, bags=bags)
    w.grad_out = np.random.default_rng(51).standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    run.forward()
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert len(got) == len(w.cores)
    assert_grads_close(got, oracle.backward_k(w))
    # bit-reproducible, with or without the kept grouping, and with the
    # forward's prefix intermediates in place of recomputed ones
    again = [g.cpu().numpy() for g in run.backward(w.grad_out)]
    for a, b in zip(got, again):
        assert np.array_equal(a, b)
    run.forward(flags=tt.TT_EMB_REUSE_GROUPING)
    kept = [g.cpu().numpy() for g in run.backward(w.grad_out,
                                                  flags=tt.TT_EMB_REUSE_GROUPING | tt.TT_EMB_REUSE_PREFIX)]
    for a, b in zip(got, kept):
        assert np.array_equal(a, b)


def test_kcore_backward_mixed_shapes_and_sgd():
    tables = [W.Table(5000, (4, 5, 6, 50), (4, 4, 4, 8), (1, 8, 24, 12, 1), 0.2, "uniform"),
              W.Table(77, (2, 3, 2, 7), (3, 1, 2, 5), (1, 5, 3, 7, 1), 0.3, "uniform"),
              W.Table(999, (10, 10, 10, 1), (2, 2, 2, 2), (1, 16, 16, 16, 1), 0.2, "uniform"),
              W.Table(40000, (20, 20, 20, 5), (2, 4, 4, 4), (1, 32, 32, 32, 1), 0.05, "zipf", 1.1)]
    rng = np.random.default_rng(52)
    lens = [rng.integers(0, 12, size=50) for _ in tables]
    lens[1][:] = 0  # a table with no lookups: zero gradients
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    idx[0][: len(idx[0]) // 2] = 4321
    w = W.make_custom(tables, lens, idx, seed=52)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out)]
    ref = oracle.backward_k(w)
    assert_grads_close(got, ref)
    for k in range(4):
        assert not got[4 + k].any()
    # SGD on the T*K cores: the applied update is -lr * dG
    before = [c.cpu().numpy().astype(np.float64) for c in run.cores]
    grads = run.emb.backward(torch.from_numpy(w.grad_out).to(DEV), run.cores, run.idx, run.off, w.B)
    run.emb.sgd_update(run.cores, grads, 0.01)
    torch.cuda.synchronize()
    for c, b0, r in zip(run.cores, before, ref):
        delta = c.cpu().numpy().astype(np.float64) - b0
        want = oracle.sgd_delta(r, 0.01)
        ulp = np.spacing(np.abs(b0).astype(np.float32)).max()  # the update lands on the fp32 grid
        assert np.abs(delta - want).max() <= TOL * np.abs(want).max() + ulp
    # no lookups at all: every gradient is zero
    w0 = W.make_custom(tables[:2], [np.zeros(4, np.int64)] * 2, [np.zeros(0, np.int64)] * 2, seed=53)
    run0 = Run(w0)
    g0 = run0.backward(np.zeros((4, w0.sum_D), np.float32))
    assert all(not g.cpu().numpy().any() for g in g0)


def test_kcore_full_size_backward_sampled_bags():
    # the gradient is linear in grad_out: with grad_out zero outside a sample
    # of bags, the full-size backward equals the oracle's on those bags alone
    w = W.make_kcore_workload("k4")
    rng = np.random.default_rng(54)
    bags = np.unique(np.concatenate([[0, w.B - 1], rng.integers(0, w.B, 200)]))
    go = np.zeros((w.B, w.sum_D), np.float32)
    go[bags] = rng.standard_normal((len(bags), w.sum_D)).astype(np.float32)
    run = Run(w)
    got = [g.cpu().numpy() for g in run.backward(go)]
    sub = _sub_bags(w, bags)
    sub.grad_out = go[bags]
    assert_grads_close(got, oracle.backward_k(sub))


def test_largest_row_space():
    # Rows summed over the tables at the handle's limit (2^31 - 2), so that the
    # (table, row) sort keys fill 31 bits and the first table's row numbers
    # reach 2^31 - 1003: lookups at the first and last rows of each table,
    # rows near the top of the first and uniform rows, with empty bags.
    big = 2 ** 31 - 2 - 1000
    tabs = [W.Table(big, (2048, 1024, 1024), (2, 2, 4), (1, 8, 8, 1), 0.1, "uniform"),
            W.Table(1000, (10, 10, 10), (4, 4, 4), (1, 16, 16, 1), 0.1, "uniform")]
    rng = np.random.default_rng(31)
    B = 64
    lens, idx = [], []
    for t in tabs:
        ln = rng.integers(0, 40, size=B)
        ln[[3, 17]] = 0
        n = int(ln.sum())
        pick = rng.integers(0, 3, n)
        ix = np.where(pick == 0, rng.integers(max(t.N - 2 ** 20, 0), t.N, n), rng.integers(0, t.N, n))
        ix[:4] = [0, t.N - 1, t.N - 2, 0]
        lens.append(ln)
        idx.append(ix.astype(np.int64))
    w = W.make_custom(tabs, lens, idx, seed=31)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    out = run.forward().cpu().numpy()
    assert_out_close(w, out, oracle.forward(w))
    assert not out[[3, 17]].any()
    check_grouping(run)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))


def test_largest_supported_shapes():
    # Tables at the create-time shape limits, all outside the matrix-core
    # classes: D = 1024 columns with R1 d2 R2 = 16384 (the whole dG2 slice of a
    # unit in the generic backward's registers), R1 = 256 and R2 = 256, each
    # against the oracle forward and backward, with empty bags.
    tables = [W.Table(500, (8, 8, 8), (4, 4, 64), (1, 64, 64, 1), 0.05, "uniform"),
              W.Table(300, (7, 7, 7), (2, 2, 4), (1, 256, 32, 1), 0.05, "uniform"),
              W.Table(300, (7, 7, 7), (4, 2, 4), (1, 32, 256, 1), 0.05, "uniform")]
    rng = np.random.default_rng(41)
    lens = [rng.integers(0, 9, size=40) for _ in tables]
    for ln in lens:
        ln[[0, 7]] = 0
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    w = W.make_custom(tables, lens, idx, seed=41)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    out = run.forward().cpu().numpy()
    assert_out_close(w, out, oracle.forward(w))
    assert not out[[0, 7]].any()
    check_grouping(run)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))


def test_kcore_eight_cores():
    # K = 8, the largest core count: unequal ranks and digit widths (some
    # d_k = 1), a hot row, forward and backward against the oracle, each
    # with the level intermediates kept from the forward and recomputed.
    tables = [W.Table(2000, (2, 3, 2, 3, 2, 3, 2, 5), (2, 1, 2, 1, 2, 1, 2, 2), (1, 4, 6, 8, 5, 7, 3, 4, 1), 0.3,
                      "uniform"),
              W.Table(60000, (4, 4, 4, 4, 4, 4, 4, 4), (1, 2, 1, 2, 1, 2, 1, 2), (1, 8, 8, 8, 8, 8, 8, 8, 1), 0.3,
                      "uniform")]
    rng = np.random.default_rng(61)
    lens = [rng.integers(0, 16, size=48) for _ in tables]
    lens[0][5] = 0
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    idx[1][::3] = 59999
    w = W.make_custom(tables, lens, idx, seed=61)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    out = run.forward().cpu().numpy()
    assert_out_close(w, out, oracle.forward_k(w))
    assert not out[5, :w.col_offsets()[1]].any()
    ref = oracle.backward_k(w)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out,
                                                  flags=tt.TT_EMB_REUSE_GROUPING | tt.TT_EMB_REUSE_PREFIX)]
    assert_grads_close(got, ref)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out)]
    assert_grads_close(got, ref)


def test_sixty_four_tables():
    # T = 64, the most tables a handle takes: every matrix-core rank class and
    # generic shapes side by side, some tables without lookups, forward,
    # grouping and backward against the oracle.
    shapes = [((10, 10, 10), (2, 2, 4), (1, 8, 8, 1)), ((10, 10, 10), (4, 4, 4), (1, 16, 16, 1)),
              ((10, 10, 10), (4, 4, 4), (1, 32, 32, 1)), ((10, 10, 10), (4, 4, 4), (1, 64, 64, 1)),
              ((9, 9, 9), (3, 2, 5), (1, 6, 10, 1))]
    tables = [W.Table(600 + 2 * i, *shapes[i % 5], 0.1, "uniform") for i in range(64)]
    rng = np.random.default_rng(64)
    lens = [rng.integers(0, 7, size=16) for _ in tables]
    for t in (5, 33, 63):
        lens[t][:] = 0
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    w = W.make_custom(tables, lens, idx, seed=64)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward(w))
    check_grouping(run)
    got = [g.cpu().numpy() for g in run.backward(w.grad_out, flags=tt.TT_EMB_REUSE_GROUPING)]
    assert_grads_close(got, oracle.backward(w))


def test_kcore_most_cores_per_handle():
    # T * K = 192, the most cores a handle takes (48 tables of four cores),
    # with ranks and widths that differ between tables and tables without
    # lookups: forward and backward against the oracle.
    shapes = [((6, 6, 6, 6), (2, 2, 2, 2), (1, 8, 8, 8, 1)), ((5, 5, 5, 8), (2, 4, 4, 4), (1, 16, 16, 16, 1)),
              ((4, 6, 5, 7), (3, 1, 2, 5), (1, 5, 3, 7, 1))]
    tables = [W.Table(780 + i, *shapes[i % 3], 0.2, "uniform") for i in range(48)]
    rng = np.random.default_rng(192)
    lens = [rng.integers(0, 6, size=12) for _ in tables]
    for t in (0, 47):
        lens[t][:] = 0
    idx = [rng.integers(0, t.N, size=int(l.sum())) for t, l in zip(tables, lens)]
    w = W.make_custom(tables, lens, idx, seed=192)
    w.grad_out = rng.standard_normal((w.B, w.sum_D)).astype(np.float32)
    run = Run(w)
    assert_out_close(w, run.forward().cpu().numpy(), oracle.forward_k(w))
    got = [g.cpu().numpy() for g in run.backward(w.grad_out,
                                                  flags=tt.TT_EMB_REUSE_GROUPING | tt.TT_EMB_REUSE_PREFIX)]
    assert_grads_close(got, oracle.backward_k(w))


# ------------------------------------------------ inference-only workspace

def test_forward_only_workspace():
    # a forward without kept prefix intermediates runs in the smaller forward
    # workspace and matches the oracle; calls that need the backward's
    # regions are refused on it
    w = W.make_workload(5, bags=64)
    emb = tt.TTEmbeddingBag(w.tables, DEV, forward_only=True)
    full = tt.tt_emb_workspace_size(emb.handle, w.B, w.nnz)
    fwd = tt.tt_emb_forward_workspace_size(emb.handle, w.B, w.nnz)
    print(f"[ws] forward {fwd} of {full} bytes", flush=True)
    assert 0 < fwd < full
    cores = [torch.from_numpy(c).to(DEV) for c in w.cores]
    idx = torch.from_numpy(w.indices).to(DEV)
    off = torch.from_numpy(w.offsets).to(DEV)
    out = emb.forward(cores, idx, off, w.B)
    torch.cuda.synchronize()
    assert emb.workspace(w.B, w.nnz).numel() == fwd
    assert_out_close(w, out.cpu().numpy(), oracle.forward(w))
    assert emb.poll_error() == 0
    g = emb.grouping(w.B, w.nnz)
    ref = oracle.grouping(w)
    for k in ref:
        assert np.array_equal(g[k].cpu().numpy(), ref[k]), k
    with pytest.raises(tt.TTEmbError) as e:
        emb.backward(torch.from_numpy(w.grad_out).to(DEV), cores, idx, off, w.B, flags=tt.TT_EMB_REUSE_GROUPING)
    assert e.value.status == tt.TT_EMB_ERR_WORKSPACE
    o = tt.tt_emb_options()
    o.keep_prefix = 1
    embk = tt.TTEmbeddingBag(w.tables, DEV, o, forward_only=True)
    with pytest.raises(tt.TTEmbError) as e:
        embk.forward(cores, idx, off, w.B, flags=tt.TT_EMB_KEEP_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_WORKSPACE
