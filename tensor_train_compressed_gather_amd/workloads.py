"""Seeded synthetic inputs for the TT-EmbeddingBag path.

This module only draws random inputs (table shapes, TT cores, bag lengths,
indices, output gradients).  It holds none of the method's arithmetic, so it can
feed both the GPU path and the CPU oracle without coupling them.

Recipe (every draw comes from one ``numpy.random.Generator(PCG64(seed))`` with
``seed = 20260 + config``, in this order):

1. per-table parameters (multi-table configs only): for each table, the row
   count ``N = round(exp(U(ln 1e3, ln 4e7)))``, the TT rank ``R`` uniform over
   {16, 32, 64} (``R1 = R2 = R``) and the Zipf exponent ``alpha = U(0.8, 1.3)``;
2. TT cores for each table, ``G1, G2, G3`` in that order, each
   ``standard_normal * sigma`` cast to fp32, stored ``[n_k][R_{k-1}][d_k][R_k]``;
3. bag lengths for each table (1, ``U{1..64}`` or ``Poisson(20) + 1``);
4. indices for each table: uniform rows, or a truncated Zipf law over ranks
   ``1..N`` (``P(k) ~ k^-alpha``, sampled by float64 inverse CDF) mapped through
   a seeded random permutation of the rows, so hot rows are scattered;
5. for the training configuration, ``grad_out ~ N(0, 1)`` in fp32.

Row counts that are not given as a product are factored into three near-equal
factors ``n1 = n2 = ceil(N^(1/3))``, ``n3 = ceil(N / (n1 n2))``.
The workloads stand in for the Meta synthetic recommendation benchmarks of the
FlowTT evaluation, whose shapes are not published.
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260


@dataclass
class Table:
    N: int
    n: tuple
    d: tuple
    R: tuple  # (1, R1, R2, 1)
    sigma: float
    dist: str  # "uniform" or "zipf"
    alpha: float = 0.0

    @property
    def K(self) -> int:
        return len(self.n)

    @property
    def D(self) -> int:
        return int(np.prod(self.d))

    def core_shapes(self):
        n, d, R = self.n, self.d, self.R
        return [(n[k], R[k], d[k], R[k + 1]) for k in range(len(n))]


@dataclass
class Workload:
    name: str
    tables: list
    B: int  # bags per table
    cores: list  # 3*T fp32 arrays, table-major: G1_t, G2_t, G3_t
    indices: np.ndarray  # int64 [nnz]
    offsets: np.ndarray  # int64 [T*B + 1], table-major CSR
    grad_out: np.ndarray | None = None  # fp32 [B][sum D_t]
    lr: float = 0.01
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return len(self.tables)

    @property
    def nnz(self) -> int:
        return int(self.indices.shape[0])

    @property
    def sum_D(self) -> int:
        return int(sum(t.D for t in self.tables))

    def col_offsets(self):
        off = [0]
        for t in self.tables:
            off.append(off[-1] + t.D)
        return off

    def arrays(self):
        """Flat shape arrays in the layout the C interfaces take."""
        N = np.array([t.N for t in self.tables], dtype=np.int64)
        n = np.array([t.n for t in self.tables], dtype=np.int32).reshape(-1)
        d = np.array([t.d for t in self.tables], dtype=np.int32).reshape(-1)
        R = np.array([t.R for t in self.tables], dtype=np.int32).reshape(-1)
        return N, n, d, R

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in self.cores + [self.indices, self.offsets]:
            h.update(np.ascontiguousarray(a).tobytes())
        if self.grad_out is not None:
            h.update(self.grad_out.tobytes())
        return h.hexdigest()


def near_equal_factors(N: int):
    """Three factors with n1 = n2 = ceil(N^(1/3)) and n1*n2*n3 >= N."""
    c = max(1, int(round(N ** (1.0 / 3.0))))
    while c ** 3 < N:
        c += 1
    while c > 1 and (c - 1) ** 3 >= N:
        c -= 1
    n3 = -(-N // (c * c))
    return (c, c, int(n3))


def _zipf_ranks(rng, N: int, alpha: float, m: int) -> np.ndarray:
    """m draws of 0-based ranks k-1 with P(k) ~ k^-alpha on k = 1..N."""
    w = np.arange(1, N + 1, dtype=np.float64)
    np.power(w, -alpha, out=w)
    np.cumsum(w, out=w)
    u = rng.random(m) * w[-1]
    k = np.searchsorted(w, u, side="right")
    np.minimum(k, N - 1, out=k)
    return k


def _draw_cores(rng, tab: Table):
    out = []
    for shp in tab.core_shapes():
        g = rng.standard_normal(int(np.prod(shp))) * tab.sigma
        out.append(g.astype(np.float32).reshape(shp))
    return out


def _draw_lengths(rng, kind: str, B: int) -> np.ndarray:
    if kind == "one":
        return np.ones(B, dtype=np.int64)
    if kind == "u1_64":
        return rng.integers(1, 65, size=B).astype(np.int64)
    if kind == "poisson20":
        return (rng.poisson(20.0, size=B) + 1).astype(np.int64)
    raise ValueError(kind)


def _draw_indices(rng, tab: Table, m: int) -> np.ndarray:
    if tab.dist == "uniform":
        return rng.integers(0, tab.N, size=m).astype(np.int64)
    perm = rng.permutation(tab.N)
    ranks = _zipf_ranks(rng, tab.N, tab.alpha, m)
    return perm[ranks].astype(np.int64)


def _assemble(name, tables, B, lens_kind, rng, meta):
    cores = []
    for tab in tables:
        cores.extend(_draw_cores(rng, tab))
    lens = [_draw_lengths(rng, lens_kind, B) for _ in tables]
    idx = []
    for tab, ln in zip(tables, lens):
        idx.append(_draw_indices(rng, tab, int(ln.sum())))
    all_len = np.concatenate(lens)
    offsets = np.zeros(len(tables) * B + 1, dtype=np.int64)
    np.cumsum(all_len, out=offsets[1:])
    indices = np.concatenate(idx) if idx else np.zeros(0, np.int64)
    return Workload(name=name, tables=tables, B=B, cores=cores, indices=indices,
                    offsets=offsets, meta=meta)


def _multi_table_params(rng, T=26):
    tables = []
    for _ in range(T):
        N = int(round(math.exp(rng.uniform(math.log(1e3), math.log(4e7)))))
        R = int((16, 32, 64)[int(rng.integers(0, 3))])
        alpha = float(rng.uniform(0.8, 1.3))
        tables.append(Table(N=N, n=near_equal_factors(N), d=(4, 4, 4), R=(1, R, R, 1),
                            sigma=0.05, dist="zipf", alpha=alpha))
    return tables


CONFIG_NAMES = {
    1: "tt1k_d16_r8_b256x1_uniform",
    2: "tt1m_d64_r32_b32768x1_zipf1.05",
    3: "tt10m_d128_r32_b32768_len1-64_zipf1.2",
    4: "26tables_d64_r16-64_b32768_poisson20_zipf0.8-1.3",
    5: "26tables_d64_r16-64_b32768_poisson20_train_sgd0.01",
}

FULL_BAGS = {1: 256, 2: 32768, 3: 32768, 4: 32768, 5: 32768}


def make_workload(cfg: int, bags: int | None = None) -> Workload:
    """Seeded workload for configuration ``cfg`` (1..5); ``bags`` overrides the
    number of bags per table (all other draws keep their recipe)."""
    rng = np.random.default_rng(np.random.PCG64(SEED_BASE + cfg))
    B = FULL_BAGS[cfg] if bags is None else int(bags)
    meta = {"config": cfg, "seed": SEED_BASE + cfg}
    if cfg == 1:
        tables = [Table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1), 0.1, "uniform")]
        w = _assemble(CONFIG_NAMES[1], tables, B, "one", rng, meta)
    elif cfg == 2:
        tables = [Table(10 ** 6, (100, 100, 100), (4, 4, 4), (1, 32, 32, 1), 0.05, "zipf", 1.05)]
        w = _assemble(CONFIG_NAMES[2], tables, B, "one", rng, meta)
    elif cfg == 3:
        tables = [Table(10 ** 7, (200, 200, 250), (4, 4, 8), (1, 32, 32, 1), 0.05, "zipf", 1.2)]
        w = _assemble(CONFIG_NAMES[3], tables, B, "u1_64", rng, meta)
    elif cfg in (4, 5):
        tables = _multi_table_params(rng)
        w = _assemble(CONFIG_NAMES[cfg], tables, B, "poisson20", rng, meta)
        if cfg == 5:
            w.grad_out = rng.standard_normal((B, w.sum_D), dtype=np.float32)
            w.lr = 0.01
    else:
        raise ValueError(f"unknown config {cfg}")
    return w


def make_grad_out(w: Workload, seed: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.PCG64(seed))
    return rng.standard_normal((w.B, w.sum_D), dtype=np.float32)


def make_custom(tables, lengths, indices, seed: int = 1, cores=None, name="custom") -> Workload:
    """Workload with explicit per-table bag lengths and indices.

    ``lengths`` and ``indices`` are lists (one entry per table) of int arrays;
    every table must have the same number of bags.  Cores are drawn from
    ``seed`` unless given.
    """
    rng = np.random.default_rng(np.random.PCG64(seed))
    B = len(lengths[0])
    if any(len(l) != B for l in lengths):
        raise ValueError("every table needs the same number of bags")
    if cores is None:
        cores = []
        for tab in tables:
            cores.extend(_draw_cores(rng, tab))
    all_len = np.concatenate([np.asarray(l, dtype=np.int64) for l in lengths])
    offsets = np.zeros(len(tables) * B + 1, dtype=np.int64)
    np.cumsum(all_len, out=offsets[1:])
    idx = np.concatenate([np.asarray(i, dtype=np.int64) for i in indices])
    if idx.shape[0] != offsets[-1]:
        raise ValueError("indices do not match the bag lengths")
    return Workload(name=name, tables=list(tables), B=B, cores=list(cores), indices=idx,
                    offsets=offsets, meta={"seed": seed})


def make_fd_instance(seed: int = SEED_BASE + 55) -> Workload:
    """Small instance for finite-difference checks of the backward: the
    1000-row rank-8 table (10x10x10 rows, D = 2x2x4) with 64 bags of
    Poisson(20)+1 uniform indices."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    tab = Table(1000, (10, 10, 10), (2, 2, 4), (1, 8, 8, 1), 0.1, "uniform")
    w = _assemble("fd_1000rows_rank8", [tab], 64, "poisson20", rng, {"seed": seed})
    w.grad_out = rng.standard_normal((w.B, w.sum_D), dtype=np.float32)
    return w


# --------------------------------------------------------- K >= 4 TT cores

def near_equal_factors_k(N: int, K: int):
    """K factors, the first K-1 equal to ceil(N^(1/K)) (then lowered while the
    product still covers N), the last covering the rest."""
    c = max(1, int(round(N ** (1.0 / K))))
    while c ** K < N:
        c += 1
    while c > 1 and (c - 1) ** K >= N:
        c -= 1
    last = -(-N // (c ** (K - 1)))
    return tuple([c] * (K - 1) + [int(last)])


KCORE_NAMES = {
    "k4": "tt10m_k4_d128_r32_b32768_len1-64_zipf1.2",
    "k5": "tt10m_k5_d64_r16_b32768_len1-64_zipf1.2",
}


def make_kcore_workload(name: str, bags: int | None = None) -> Workload:
    """Seeded K-core workloads (more than three TT cores per table): the
    10^7-row, Zipf(1.2), bag length U[1, 64] shape of the single-table
    workload with K = 4 (d = 2x4x4x4 = 128, ranks 32) or K = 5 (d = 2x2x2x2x4
    = 64, ranks 16), sigma 0.05; same draw order as the 3-core recipe, seed
    20270 + K."""
    K = {"k4": 4, "k5": 5}[name]
    rng = np.random.default_rng(np.random.PCG64(SEED_BASE + 10 + K))
    B = 32768 if bags is None else int(bags)
    N = 10 ** 7
    if K == 4:
        d, R = (2, 4, 4, 4), (1, 32, 32, 32, 1)
    else:
        d, R = (2, 2, 2, 2, 4), (1, 16, 16, 16, 16, 1)
    tab = Table(N, near_equal_factors_k(N, K), d, R, 0.05, "zipf", 1.2)
    return _assemble(KCORE_NAMES[name], [tab], B, "u1_64", rng, {"kcores": K, "seed": SEED_BASE + 10 + K})
