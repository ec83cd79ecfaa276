"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties an oracle function to a closed form, a library routine
(numpy/torch), an invariant the FlowTT summary states, brute force on tiny
inputs, or exact finite differences.  A plausible mistake in the oracle (a
transposed core operand, a swapped digit, a dropped term, a wrong sign, a
wrong tie-break) fails at least one of them.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_gather_amd import workloads as W

RNG = np.random.default_rng(12345)


def _table(N, n, d, R, sigma=0.1):
    return W.Table(N, tuple(n), tuple(d), tuple(R), sigma, "uniform")


def _random_workload(tables, B, seed, max_len=8, allow_empty=True):
    rng = np.random.default_rng(seed)
    lens, idx = [], []
    for tab in tables:
        lo = 0 if allow_empty else 1
        ln = rng.integers(lo, max_len + 1, size=B)
        lens.append(ln)
        idx.append(rng.integers(0, tab.N, size=int(ln.sum())))
    return W.make_custom(tables, lens, idx, seed=seed)


def _dense_table(tab, G1, G2, G3):
    """Full table [N][D] materialised by numpy einsum (a different code path
    and contraction order from the oracle)."""
    T = np.einsum("axpr,brqs,cstz->abcpqt", G1.astype(np.float64), G2.astype(np.float64),
                  G3.astype(np.float64))
    n1, n2, n3 = tab.n
    return T.reshape(n1 * n2 * n3, tab.D)[: tab.N]


ASYM = _table(57, (3, 4, 5), (2, 3, 2), (1, 3, 2, 1))
CFG1 = _table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1))


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("n", [(10, 10, 10), (3, 4, 5), (200, 200, 250), (342, 342, 342), (7, 1, 3)])
def test_decode_matches_unravel_index(n):
    N = n[0] * n[1] * n[2]
    pts = np.unique(np.concatenate([np.arange(min(N, 300)), RNG.integers(0, N, 300), [N - 1]]))
    for i in pts:
        got = oracle.decode(int(i), n)
        ref = tuple(int(x) for x in np.unravel_index(int(i), n))
        assert got == ref
        assert (got[0] * n[1] + got[1]) * n[2] + got[2] == i


# -------------------------------------------------------------- contraction

def test_rank1_rows_are_kronecker_products():
    tab = _table(60, (3, 4, 5), (2, 3, 4), (1, 1, 1, 1))
    rng = np.random.default_rng(1)
    G = [rng.standard_normal(s).astype(np.float32) for s in tab.core_shapes()]
    for i in range(tab.N):
        i1, i2, i3 = np.unravel_index(i, tab.n)
        ref = np.kron(G[0][i1, 0, :, 0].astype(np.float64),
                      np.kron(G[1][i2, 0, :, 0].astype(np.float64), G[2][i3, 0, :, 0].astype(np.float64)))
        got = oracle.row(tab, *G, i)
        np.testing.assert_allclose(got, ref, rtol=1e-15, atol=0)


def test_rank_diagonal_closed_form():
    """G1 constant over r1, G2 = x2 * delta(r1, r2), G3 constant over r2:
    every row is R * kron(x1, x2, x3)."""
    R = 5
    tab = _table(24, (2, 3, 4), (3, 2, 2), (1, R, R, 1))
    rng = np.random.default_rng(2)
    x = [rng.integers(-4, 5, size=(tab.n[k], tab.d[k])).astype(np.float32) for k in range(3)]
    G1 = np.repeat(x[0][:, None, :, None], R, axis=3)
    G2 = np.zeros((tab.n[1], R, tab.d[1], R), np.float32)
    for r in range(R):
        G2[:, r, :, r] = x[1]
    G3 = np.repeat(x[2][:, None, :, None], R, axis=1)
    for i in range(tab.N):
        i1, i2, i3 = np.unravel_index(i, tab.n)
        ref = R * np.kron(x[0][i1], np.kron(x[1][i2], x[2][i3])).astype(np.float64)
        assert np.array_equal(oracle.row(tab, G1, G2, G3, i), ref)


def test_all_ones_cores_pool_to_length_times_ranks():
    tab = _table(60, (3, 4, 5), (2, 2, 3), (1, 6, 7, 1))
    G = [np.ones(s, np.float32) for s in tab.core_shapes()]
    lens = [np.array([0, 1, 5, 2, 9])]
    idx = [RNG.integers(0, tab.N, size=int(lens[0].sum()))]
    w = W.make_custom([tab], lens, idx, cores=G)
    out = oracle.forward(w)
    ref = np.repeat((lens[0] * 6 * 7).astype(np.float64)[:, None], tab.D, axis=1)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("tab", [CFG1, ASYM, _table(30, (2, 3, 5), (3, 1, 2), (1, 2, 4, 1))])
def test_rows_match_dense_einsum_table(tab):
    rng = np.random.default_rng(3)
    G = [(rng.standard_normal(s) * 0.3).astype(np.float32) for s in tab.core_shapes()]
    dense = _dense_table(tab, *G)
    got = np.stack([oracle.row(tab, *G, i) for i in range(tab.N)])
    scale = np.abs(dense).max()
    assert np.abs(got - dense).max() <= 1e-13 * scale


def test_pooled_forward_matches_torch_embedding_bag():
    tables = [CFG1, ASYM, _table(30, (2, 3, 5), (3, 1, 2), (1, 2, 4, 1))]
    w = _random_workload(tables, B=37, seed=4)
    out = oracle.forward(w)
    col = w.col_offsets()
    for t, tab in enumerate(tables):
        dense = torch.from_numpy(_dense_table(tab, *w.cores[3 * t:3 * t + 3]))
        lo, hi = w.offsets[t * w.B], w.offsets[(t + 1) * w.B]
        idx = torch.from_numpy(w.indices[lo:hi])
        offs = torch.from_numpy(w.offsets[t * w.B:(t + 1) * w.B] - lo)
        ref = torch.nn.functional.embedding_bag(idx, dense, offs, mode="sum").numpy()
        got = out[:, col[t]:col[t + 1]]
        assert np.abs(got - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1e-300)
    # empty bags pool to zero
    lens = np.diff(w.offsets).reshape(len(tables), w.B)
    for t in range(len(tables)):
        for b in np.nonzero(lens[t] == 0)[0]:
            assert not out[b, col[t]:col[t + 1]].any()


def test_selected_bags_match_full_forward():
    w = W.make_workload(3, bags=64)
    full = oracle.forward(w)
    sel = np.array([5, 0, 63, 17, 17])
    part = oracle.forward(w, bags=sel)
    assert np.array_equal(part, full[sel])


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("cfg,bags", [(1, None), (2, 2048), (3, 128), (4, 32)])
def test_grouped_forward_bit_identical_to_ungrouped(cfg, bags):
    w = W.make_workload(cfg, bags=bags)
    a = oracle.forward(w)
    b = oracle.forward_grouped(w)
    assert np.array_equal(a, b)


def test_grouped_bit_identical_on_edge_cases():
    tab = _table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1))
    # every lookup in one prefix group (i1, i2) = (3, 7), plus empty bags
    rows = (3 * 10 + 7) * 10 + np.arange(10)
    lens = [np.array([0, 4, 0, 30, 1, 0])]
    idx = [RNG.choice(rows, size=int(lens[0].sum()))]
    w = W.make_custom([tab], lens, idx, seed=6)
    assert np.array_equal(oracle.forward(w), oracle.forward_grouped(w))


def test_pooling_is_linear():
    w = W.make_workload(3, bags=64)
    lens = np.diff(w.offsets)
    single = W.make_custom(w.tables, [np.ones(w.nnz, np.int64)], [w.indices], cores=w.cores)
    per_index = oracle.forward(single)
    summed = np.zeros((w.B, w.sum_D))
    np.add.at(summed, np.repeat(np.arange(w.B), lens), per_index)
    ref = oracle.forward(w)
    assert np.abs(summed - ref).max() <= 1e-12 * np.abs(ref).max()


def _round_mantissa(x, bits):
    m, e = np.frexp(x.astype(np.float64))
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e).astype(np.float32)


def test_forward_is_multilinear_in_the_cores():
    """Scaling one core scales the output; splitting one core into two parts
    splits the output.  Cores are rounded to 12 mantissa bits so that 3*G and
    the two parts are exact in fp32."""
    w = W.make_workload(4, bags=8)
    w.cores = [_round_mantissa(c, 12) for c in w.cores]
    base = oracle.forward(w)
    scale = np.abs(base).max()
    for k in range(3):
        cores = [c.copy() for c in w.cores]
        for t in range(w.T):
            cores[3 * t + k] = cores[3 * t + k] * np.float32(3.0)
        out = oracle.forward(w, cores=cores)
        assert np.abs(out - 3.0 * base).max() <= 1e-12 * scale
        hi = [c.copy() for c in w.cores]
        lo = [c.copy() for c in w.cores]
        for t in range(w.T):
            h = _round_mantissa(w.cores[3 * t + k], 5)
            hi[3 * t + k] = h
            lo[3 * t + k] = (w.cores[3 * t + k] - h).astype(np.float32)
        split = oracle.forward(w, cores=hi) + oracle.forward(w, cores=lo)
        assert np.abs(split - base).max() <= 1e-12 * scale
    cores = [c * np.float32(0.5) for c in w.cores]
    assert np.array_equal(oracle.forward(w, cores=cores), base * 0.125)


# ------------------------------------------------------------------ grouping

def _numpy_grouping(w):
    T, B = w.T, w.B
    tab_of = np.repeat(np.arange(T), np.diff(w.offsets[::B]))
    base = np.concatenate([[0], np.cumsum([t.N for t in w.tables])])
    key = base[tab_of] + w.indices
    perm = np.argsort(key, kind="stable")
    ks = key[perm]
    ukeys, first, inv_sorted = np.unique(ks, return_index=True, return_inverse=True)
    inv = np.empty(w.nnz, np.int64)
    inv[perm] = inv_sorted
    utab = np.searchsorted(base, ukeys, side="right") - 1
    urow = ukeys - base[utab]
    n3 = np.array([t.n[2] for t in w.tables])
    q = urow // n3[utab]
    pkey = utab.astype(np.int64) * (1 << 40) + q
    _, gfirst = np.unique(pkey, return_index=True)
    return {
        "perm": perm,
        "uniq_row": urow,
        "uniq_start": np.append(first, w.nnz),
        "inv": inv,
        "grp_prefix": q[gfirst],
        "grp_start": np.append(gfirst, len(ukeys)),
        "tab_uniq_start": np.searchsorted(utab, np.arange(T + 1), side="left"),
        "tab_grp_start": np.searchsorted(utab[gfirst], np.arange(T + 1), side="left"),
    }


@pytest.mark.parametrize("cfg,bags", [(1, None), (2, 4096), (3, 512), (4, 64)])
def test_grouping_matches_numpy_sort_and_unique(cfg, bags):
    w = W.make_workload(cfg, bags=bags)
    got = oracle.grouping(w)
    ref = _numpy_grouping(w)
    for k in ref:
        assert np.array_equal(got[k], np.asarray(ref[k])), k


def test_grouping_matches_python_brute_force_on_tiny_input():
    tables = [ASYM, _table(8, (2, 2, 2), (1, 1, 2), (1, 2, 2, 1))]
    w = _random_workload(tables, B=6, seed=7)
    got = oracle.grouping(w)
    T, B = w.T, w.B
    tab_of = [t for t in range(T) for _ in range(w.offsets[(t + 1) * B] - w.offsets[t * B])]
    order = sorted(range(w.nnz), key=lambda l: (tab_of[l], int(w.indices[l]), l))
    assert list(got["perm"]) == order
    uniq = []
    for l in order:
        kk = (tab_of[l], int(w.indices[l]))
        if not uniq or uniq[-1] != kk:
            uniq.append(kk)
    assert list(got["uniq_row"]) == [r for _, r in uniq]
    assert [int(got["inv"][l]) for l in range(w.nnz)] == [uniq.index((tab_of[l], int(w.indices[l]))) for l in range(w.nnz)]
    groups = []
    for t, r in uniq:
        kk = (t, r // tables[t].n[2])
        if not groups or groups[-1] != kk:
            groups.append(kk)
    assert list(got["grp_prefix"]) == [q for _, q in groups]


def test_grouping_edge_cases():
    tab = _table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1))
    # all identical indices; an empty bag; a bag that is the whole input
    w = W.make_custom([tab], [np.array([0, 7, 0])], [np.full(7, 999)])
    g = oracle.grouping(w)
    assert list(g["perm"]) == list(range(7))
    assert list(g["uniq_row"]) == [999] and list(g["uniq_start"]) == [0, 7]
    assert list(g["grp_prefix"]) == [99] and list(g["grp_start"]) == [0, 1]
    # no lookups at all
    w = W.make_custom([tab], [np.array([0, 0])], [np.zeros(0, np.int64)])
    g = oracle.grouping(w)
    assert g["perm"].size == 0 and list(g["uniq_start"]) == [0] and list(g["grp_start"]) == [0]


def test_invalid_inputs_are_rejected():
    tab = _table(57, (3, 4, 5), (2, 3, 2), (1, 3, 2, 1))
    w = W.make_custom([tab], [np.array([2, 1])], [np.array([0, 56, 3])])
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(w, indices=np.array([0, 57, 3]))
    assert e.value.rc == oracle.ERR_INDEX
    with pytest.raises(oracle.OracleError) as e:
        oracle.grouping(w, indices=np.array([0, -1, 3]))
    assert e.value.rc == oracle.ERR_INDEX
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(w, offsets=np.array([0, 3, 2]))
    assert e.value.rc == oracle.ERR_ARG
    bad = W.make_custom([_table(61, (3, 4, 5), (2, 3, 2), (1, 3, 2, 1))], [np.array([1])],
                        [np.array([0])], cores=w.cores)
    with pytest.raises(oracle.OracleError):
        oracle.forward(bad)


# ------------------------------------------------------------------ backward

def _torch_grads(w):
    """Gradients of sum(grad_out * out) through a dense einsum table and
    torch.nn.functional.embedding_bag, in float64 on the CPU."""
    grads = []
    col = w.col_offsets()
    go = torch.from_numpy(w.grad_out.astype(np.float64))
    for t, tab in enumerate(w.tables):
        G = [torch.tensor(c.astype(np.float64), requires_grad=True) for c in w.cores[3 * t:3 * t + 3]]
        dense = torch.einsum("axpr,brqs,cstz->abcpqt", *G)
        n1, n2, n3 = tab.n
        dense = dense.reshape(n1 * n2 * n3, tab.D)[: tab.N]
        lo, hi = w.offsets[t * w.B], w.offsets[(t + 1) * w.B]
        out = torch.nn.functional.embedding_bag(torch.from_numpy(w.indices[lo:hi]), dense,
                                                torch.from_numpy(w.offsets[t * w.B:(t + 1) * w.B] - lo),
                                                mode="sum")
        (out * go[:, col[t]:col[t + 1]]).sum().backward()
        grads.extend(g.grad.numpy() for g in G)
    return grads


def test_backward_matches_torch_autograd_dense():
    tables = [CFG1, ASYM, _table(30, (2, 3, 5), (3, 1, 2), (1, 2, 4, 1))]
    w = _random_workload(tables, B=23, seed=8)
    w.grad_out = np.random.default_rng(9).standard_normal((w.B, w.sum_D)).astype(np.float32)
    got = oracle.backward(w)
    ref = _torch_grads(w)
    for g, r in zip(got, ref):
        assert g.shape == r.shape
        assert np.abs(g - r).max() <= 1e-12 * max(np.abs(r).max(), 1e-300)


def test_backward_matches_exact_finite_differences():
    """The pooled loss is affine in each single core entry, so a central
    difference over the actually stored fp32 perturbation is exact up to
    fp64 rounding."""
    w = W.make_fd_instance()
    dG = oracle.backward(w)
    go = w.grad_out.astype(np.float64)
    rng = np.random.default_rng(10)
    for k in range(3):
        c = w.cores[k]
        flat = rng.choice(c.size, size=min(c.size, 60), replace=False)
        for f in flat:
            pos = np.unravel_index(int(f), c.shape)
            cp, cm = [x.copy() for x in w.cores], [x.copy() for x in w.cores]
            cp[k][pos] = np.float32(c[pos] + np.float32(0.01))
            cm[k][pos] = np.float32(c[pos] - np.float32(0.01))
            step = float(cp[k][pos]) - float(cm[k][pos])
            Lp = (oracle.forward(w, cores=cp, threads=1) * go).sum()
            Lm = (oracle.forward(w, cores=cm, threads=1) * go).sum()
            fd = (Lp - Lm) / step
            assert abs(fd - dG[k][pos]) <= 1e-9 * max(1.0, abs(dG[k][pos])), (k, pos)


def test_backward_selected_slices_match_full():
    w = W.make_workload(4, bags=16)
    w.grad_out = W.make_grad_out(w, 11)
    full = oracle.backward(w)
    sel = np.full((w.T, 3), -2, np.int64)
    picks = []
    for t in (0, 5, 25):
        tab = w.tables[t]
        lo = w.offsets[t * w.B]
        i1, i2, i3 = np.unravel_index(int(w.indices[lo]), tab.n)
        sel[t] = (i1, i2, i3)
        picks.append((t, (i1, i2, i3)))
    part = oracle.backward(w, sel=sel)
    for t, ii in picks:
        for k in range(3):
            assert np.array_equal(part[3 * t + k][ii[k]], full[3 * t + k][ii[k]])
            assert part[3 * t + k][ii[k]].any()


def test_untouched_gradient_slices_are_zero():
    w = _random_workload([CFG1], B=3, seed=12, max_len=2)
    w.grad_out = np.ones((w.B, w.sum_D), np.float32)
    dG = oracle.backward(w)
    used = [set(), set(), set()]
    for i in w.indices:
        for k, v in enumerate(np.unravel_index(int(i), CFG1.n)):
            used[k].add(int(v))
    for k in range(3):
        for s in range(CFG1.n[k]):
            assert dG[k][s].any() == (s in used[k])


def test_sgd_delta_matches_torch_sgd_step():
    # an independent statement of plain SGD: one torch.optim.SGD step (no
    # momentum, no weight decay) on an fp64 parameter whose gradient is dG;
    # the oracle's delta must be the parameter's change, sign and scale
    # included, for several learning rates and gradient scales
    import torch

    rng = np.random.default_rng(13)
    for lr, scale in ((0.01, 1.0), (0.5, 1e-3), (3.0, 1e4)):
        p0 = rng.standard_normal((5, 7))
        dG = rng.standard_normal((5, 7)) * scale
        p = torch.nn.Parameter(torch.from_numpy(p0.copy()))
        p.grad = torch.from_numpy(dG.copy())
        torch.optim.SGD([p], lr=lr).step()
        moved = p.detach().numpy() - p0
        got = oracle.sgd_delta(dG, lr)
        assert np.allclose(got, moved, rtol=1e-12, atol=1e-15 * np.abs(p0).max()), lr
        # descent direction: the step never increases the linear loss <dG, p>
        assert float(np.sum(got * dG)) < 0


# ----------------------------------------------------------------- generator

def test_generator_matches_the_recorded_digests():
    # sha256 of every generated array of each workload, recorded by
    # tests/golden/make_workload_digests.py: any change to the seeded inputs
    # (draw order, distributions, shapes) shows up here
    import json
    import os
    import sys

    golden = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, golden)
    import make_workload_digests as mk

    want = json.load(open(os.path.join(golden, "workload_digests.json")))
    assert mk.digests() == want


def test_generator_is_reproducible_and_shaped():
    a, b = W.make_workload(3, bags=256), W.make_workload(3, bags=256)
    assert a.digest() == b.digest()
    w4 = W.make_workload(4, bags=16)
    assert w4.T == 26
    for tab in w4.tables:
        assert tab.n[0] * tab.n[1] * tab.n[2] >= tab.N
        assert tab.R[1] in (16, 32, 64) and tab.R[1] == tab.R[2]
        assert 1000 <= tab.N <= 4 * 10 ** 7
    lens = np.diff(w4.offsets)
    assert lens.min() >= 1
    for t, tab in enumerate(w4.tables):
        seg = w4.indices[w4.offsets[t * 16]:w4.offsets[(t + 1) * 16]]
        assert seg.min() >= 0 and seg.max() < tab.N


# ------------------------------------------------------- K >= 4 TT cores

def _dense_table_k(tab, cores):
    """Full table [N][D] of a K-core table by one numpy einsum over the whole
    cores (a different route from the oracle's per-row chain)."""
    K = len(cores)
    I, J, Rl = "abcdefgh"[:K], "ijklmnop"[:K], "qrstuvwxy"[: K + 1]
    subs = ",".join(f"{I[k]}{Rl[k]}{J[k]}{Rl[k + 1]}" for k in range(K))
    full = np.einsum(f"{subs}->{I}{J}", *[c.astype(np.float64) for c in cores])
    n = [c.shape[0] for c in cores]
    d = [c.shape[2] for c in cores]
    return full.reshape(int(np.prod(n)), int(np.prod(d)))[: tab.N]


@pytest.mark.parametrize("n,d,R", [
    ((3, 2, 4, 2), (2, 3, 2, 2), (1, 3, 2, 4, 1)),
    ((2, 3, 2, 2, 3), (2, 2, 1, 3, 2), (1, 2, 3, 2, 2, 1)),
])
def test_kcore_forward_matches_dense_table(n, d, R):
    tab = _table(int(np.prod(n)) - 1, n, d, R, sigma=0.4)
    w = _random_workload([tab], 24, seed=31)
    dense = _dense_table_k(tab, w.cores)
    ref = np.zeros((w.B, tab.D))
    for b in range(w.B):
        for l in range(w.offsets[b], w.offsets[b + 1]):
            ref[b] += dense[w.indices[l]]
    got = oracle.forward_k(w)
    assert np.abs(got - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1.0)


def test_kcore_rank1_rows_are_kronecker_products():
    n, d, R = (3, 2, 2, 3), (2, 3, 2, 2), (1, 1, 1, 1, 1)
    tab = _table(36, n, d, R, sigma=0.5)
    lens = [np.ones(36, np.int64)]
    w = W.make_custom([tab], lens, [np.arange(36)], seed=32)
    got = oracle.forward_k(w)
    for i in range(36):
        dig = np.unravel_index(i, n)
        v = np.ones(1)
        for k in range(4):
            v = np.kron(v, w.cores[k][dig[k], 0, :, 0].astype(np.float64))
        assert np.allclose(got[i], v, rtol=0, atol=1e-14)


def test_kcore_with_three_cores_equals_the_three_core_oracle():
    w = W.make_workload(3, bags=64)
    a = oracle.forward_k(w)
    b = oracle.forward(w)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()


@pytest.mark.parametrize("name,bags", [("k4", 64), ("k5", 64)])
def test_kcore_grouped_is_bit_identical_to_ungrouped(name, bags):
    w = W.make_kcore_workload(name, bags=bags)
    assert np.array_equal(oracle.forward_k(w, grouped=True), oracle.forward_k(w))


def test_kcore_workload_factors_cover_the_rows():
    for name in ("k4", "k5"):
        w = W.make_kcore_workload(name, bags=8)
        t = w.tables[0]
        assert np.prod(t.n) >= t.N and len(t.n) == t.K == len(t.d) == len(t.R) - 1
        assert [c.shape for c in w.cores] == t.core_shapes()
        assert w.indices.min() >= 0 and w.indices.max() < t.N


def _torch_grads_k(w):
    """Gradients of sum(grad_out * out) for K-core tables through a dense
    torch.einsum table and embedding_bag, float64 on the CPU."""
    K = len(w.tables[0].n)
    I, J, Rl = "abcdefgh"[:K], "ijklmnop"[:K], "qrstuvwxy"[: K + 1]
    subs = ",".join(f"{I[k]}{Rl[k]}{J[k]}{Rl[k + 1]}" for k in range(K))
    grads = []
    col = w.col_offsets()
    go = torch.from_numpy(w.grad_out.astype(np.float64))
    for t, tab in enumerate(w.tables):
        G = [torch.tensor(c.astype(np.float64), requires_grad=True) for c in w.cores[K * t:K * t + K]]
        dense = torch.einsum(f"{subs}->{I}{J}", *G).reshape(int(np.prod(tab.n)), tab.D)[: tab.N]
        lo, hi = w.offsets[t * w.B], w.offsets[(t + 1) * w.B]
        out = torch.nn.functional.embedding_bag(torch.from_numpy(w.indices[lo:hi]), dense,
                                                torch.from_numpy(w.offsets[t * w.B:(t + 1) * w.B] - lo),
                                                mode="sum")
        (out * go[:, col[t]:col[t + 1]]).sum().backward()
        grads.extend(g.grad.numpy() for g in G)
    return grads


@pytest.mark.parametrize("n,d,R", [
    ((3, 2, 4, 2), (2, 3, 2, 2), (1, 3, 2, 4, 1)),
    ((2, 3, 2, 2, 3), (2, 2, 1, 3, 2), (1, 2, 3, 2, 2, 1)),
])
def test_kcore_backward_matches_torch_autograd_dense(n, d, R):
    tabs = [_table(int(np.prod(n)) - 1, n, d, R, sigma=0.4), _table(int(np.prod(n)) // 2, n, d, R, sigma=0.3)]
    w = _random_workload(tabs, 19, seed=41)
    w.grad_out = np.random.default_rng(42).standard_normal((w.B, w.sum_D)).astype(np.float32)
    got = oracle.backward_k(w)
    ref = _torch_grads_k(w)
    assert len(got) == len(ref) == 2 * len(n)
    for g, r in zip(got, ref):
        assert g.shape == r.shape
        assert np.abs(g - r).max() <= 1e-12 * max(np.abs(r).max(), 1e-300)


def test_kcore_backward_matches_exact_finite_differences():
    """The pooled loss is affine in each core entry: a central difference over
    the stored fp32 perturbation equals the gradient up to fp64 rounding."""
    n, d, R = (3, 2, 4, 2), (2, 3, 2, 2), (1, 3, 2, 4, 1)
    w = _random_workload([_table(40, n, d, R, sigma=0.4)], 12, seed=43)
    w.grad_out = np.random.default_rng(44).standard_normal((w.B, w.sum_D)).astype(np.float32)
    dG = oracle.backward_k(w)
    go = w.grad_out.astype(np.float64)
    rng = np.random.default_rng(45)
    for k in range(4):
        c = w.cores[k]
        for f in rng.choice(c.size, size=min(c.size, 25), replace=False):
            pos = np.unravel_index(int(f), c.shape)
            cp, cm = [x.copy() for x in w.cores], [x.copy() for x in w.cores]
            cp[k][pos] = np.float32(c[pos] + np.float32(0.01))
            cm[k][pos] = np.float32(c[pos] - np.float32(0.01))
            step = float(cp[k][pos]) - float(cm[k][pos])
            fd = ((oracle.forward_k(w, cores=cp) - oracle.forward_k(w, cores=cm)) * go).sum() / step
            assert abs(fd - dG[k][pos]) <= 1e-9 * max(1.0, abs(dG[k][pos])), (k, pos)


def test_kcore_backward_with_three_cores_equals_the_three_core_oracle():
    w = W.make_workload(5, bags=8)
    a = oracle.backward_k(w)
    b = oracle.backward(w)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-12 * max(np.abs(y).max(), 1e-300)
