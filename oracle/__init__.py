"""CPU oracle for the TT-EmbeddingBag path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code: this wrapper loads ``liboracle_tt.so`` built from
``tt_oracle.c`` with plain gcc (fp64, ``-ffp-contract=off``).

Every function follows the FlowTT summary page (sections 2.4, 3.2, 3.3 and the
grouping breakdown of section 4) and the TT-Rec abstract; the C file states
which passage each function follows.  All functions are pinned by the CPU
tests in ``tests/test_oracle_pins.py`` (closed forms, a library dense-table
computation, invariants and finite differences); none is "parity unpinned".
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tt_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_tt.so")
_lock = threading.Lock()
_lib = None

OK, ERR_ARG, ERR_INDEX, ERR_NOMEM = 0, -1, -2, -6


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """The same oracle built for the CPU sanitizer check: AddressSanitizer and
    UndefinedBehaviorSanitizer (any report aborts), same fp64
    arithmetic flags."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-o", path, _SRC]
    subprocess.run(cmd, check=True)
    return path


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # TT_ORACLE_LIB: a sanitizer build of the same source (CPU tests only)
            path = os.environ.get("TT_ORACLE_LIB")
            if not path:
                build()
                path = _LIB
            lib = C.CDLL(path)
            p = C.c_void_p
            i32, i64 = C.c_int32, C.c_int64
            lib.orc_decode.argtypes = [i64, p, p]
            lib.orc_row.argtypes = [p, p, p, p, p, p, i64, p]
            lib.orc_forward.argtypes = [i32, p, p, p, p, p, p, p, i64, i64, p, i64, p, i32]
            lib.orc_grouping.argtypes = [i32, p, p, p, p, i64, i64, p, p, p, p, p, p, p, p, p]
            lib.orc_forward_grouped.argtypes = [i32, p, p, p, p, p, p, p, i64, i64, p]
            lib.orc_backward.argtypes = [i32, p, p, p, p, p, p, p, i64, i64, p, p, p, i32]
            lib.orc_forward_k.argtypes = [i32, i32, p, p, p, p, p, p, p, i64, i64, p, i32]
            lib.orc_forward_k_grouped.argtypes = [i32, i32, p, p, p, p, p, p, p, i64, i64, p]
            lib.orc_backward_k.argtypes = [i32, i32, p, p, p, p, p, p, p, i64, i64, p, p]
            lib.orc_sgd_delta.argtypes = [p, i64, C.c_double, p]
            lib.orc_sgd_delta.restype = None
            lib.orc_max_threads.restype = C.c_int
            _lib = lib
    return _lib


class OracleError(RuntimeError):
    def __init__(self, rc):
        super().__init__(f"oracle returned {rc}")
        self.rc = rc


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _shape_args(w):
    N, n, d, R = w.arrays()
    return N, n, d, R


def _cores_arg(cores):
    cs = [np.ascontiguousarray(c, dtype=np.float32) for c in cores]
    arr = (C.c_void_p * len(cs))(*[c.ctypes.data for c in cs])
    return cs, arr


def max_threads() -> int:
    return int(_load().orc_max_threads())


def decode(i: int, n) -> tuple:
    lib = _load()
    nn = np.asarray(n, dtype=np.int32)
    out = np.zeros(3, dtype=np.int64)
    rc = lib.orc_decode(int(i), _ptr(nn), _ptr(out))
    if rc:
        raise OracleError(rc)
    return tuple(int(x) for x in out)


def row(table, G1, G2, G3, i: int) -> np.ndarray:
    """One row rebuilt per index, fp64 [D]."""
    lib = _load()
    n = np.asarray(table.n, dtype=np.int32)
    d = np.asarray(table.d, dtype=np.int32)
    R = np.asarray(table.R, dtype=np.int32)
    gs = [np.ascontiguousarray(g, dtype=np.float32) for g in (G1, G2, G3)]
    E = np.zeros(table.D, dtype=np.float64)
    rc = lib.orc_row(_ptr(gs[0]), _ptr(gs[1]), _ptr(gs[2]), _ptr(n), _ptr(d), _ptr(R), int(i), _ptr(E))
    if rc:
        raise OracleError(rc)
    return E


def forward(w, bags=None, threads: int = 0, cores=None, indices=None, offsets=None) -> np.ndarray:
    """Pooled forward, no reuse; fp64 [len(bags) or B][sum D]."""
    lib = _load()
    N, n, d, R = _shape_args(w)
    cs, carr = _cores_arg(w.cores if cores is None else cores)
    idx = np.ascontiguousarray(w.indices if indices is None else indices, dtype=np.int64)
    off = np.ascontiguousarray(w.offsets if offsets is None else offsets, dtype=np.int64)
    sel = None if bags is None else np.ascontiguousarray(bags, dtype=np.int64)
    nb = w.B if sel is None else sel.shape[0]
    out = np.zeros((nb, w.sum_D), dtype=np.float64)
    rc = lib.orc_forward(w.T, _ptr(N), _ptr(n), _ptr(d), _ptr(R), carr, _ptr(idx), _ptr(off),
                         w.B, idx.shape[0], None if sel is None else _ptr(sel),
                         0 if sel is None else sel.shape[0], _ptr(out), int(threads))
    if rc:
        raise OracleError(rc)
    return out


def forward_grouped(w) -> np.ndarray:
    """Pooled forward with prefix-group reuse; fp64 [B][sum D]."""
    lib = _load()
    N, n, d, R = _shape_args(w)
    cs, carr = _cores_arg(w.cores)
    out = np.zeros((w.B, w.sum_D), dtype=np.float64)
    rc = lib.orc_forward_grouped(w.T, _ptr(N), _ptr(n), _ptr(d), _ptr(R), carr, _ptr(w.indices),
                                 _ptr(w.offsets), w.B, w.nnz, _ptr(out))
    if rc:
        raise OracleError(rc)
    return out


def grouping(w, indices=None, offsets=None) -> dict:
    """Canonical grouping arrays (all int32, ids global over tables)."""
    lib = _load()
    N, n, d, R = _shape_args(w)
    idx = np.ascontiguousarray(w.indices if indices is None else indices, dtype=np.int64)
    off = np.ascontiguousarray(w.offsets if offsets is None else offsets, dtype=np.int64)
    nnz = idx.shape[0]
    cap = max(nnz, 1)
    perm = np.zeros(cap, np.int32)
    urow = np.zeros(cap, np.int32)
    ustart = np.zeros(cap + 1, np.int32)
    inv = np.zeros(cap, np.int32)
    gpre = np.zeros(cap, np.int32)
    gstart = np.zeros(cap + 1, np.int32)
    tu = np.zeros(w.T + 1, np.int32)
    tg = np.zeros(w.T + 1, np.int32)
    counts = np.zeros(2, np.int64)
    rc = lib.orc_grouping(w.T, _ptr(N), _ptr(n), _ptr(idx), _ptr(off), w.B, nnz, _ptr(perm),
                          _ptr(urow), _ptr(ustart), _ptr(inv), _ptr(gpre), _ptr(gstart), _ptr(tu),
                          _ptr(tg), _ptr(counts))
    if rc:
        raise OracleError(rc)
    U, G = int(counts[0]), int(counts[1])
    return {
        "perm": perm[:nnz].copy(),
        "uniq_row": urow[:U].copy(),
        "uniq_start": ustart[:U + 1].copy(),
        "inv": inv[:nnz].copy(),
        "grp_prefix": gpre[:G].copy(),
        "grp_start": gstart[:G + 1].copy(),
        "tab_uniq_start": tu.copy(),
        "tab_grp_start": tg.copy(),
    }


def backward(w, grad_out=None, sel=None, threads: int = 0, cores=None) -> list:
    """Core gradients of sum(grad_out * out), fp64, shaped like the cores.

    ``sel`` optionally maps (table, core) -> slice index (a [T,3] int array,
    -1 = every slice, -2 = none) to compute only sampled slices."""
    lib = _load()
    N, n, d, R = _shape_args(w)
    cs, carr = _cores_arg(w.cores if cores is None else cores)
    g = np.ascontiguousarray(w.grad_out if grad_out is None else grad_out, dtype=np.float32)
    if g.shape != (w.B, w.sum_D):
        raise ValueError("grad_out must be [B][sum D]")
    dG = [np.zeros(c.shape, dtype=np.float64) for c in cs]
    darr = (C.c_void_p * len(dG))(*[x.ctypes.data for x in dG])
    s = None if sel is None else np.ascontiguousarray(np.asarray(sel).reshape(-1), dtype=np.int64)
    rc = lib.orc_backward(w.T, _ptr(N), _ptr(n), _ptr(d), _ptr(R), carr, _ptr(w.indices),
                          _ptr(w.offsets), w.B, w.nnz, _ptr(g), None if s is None else _ptr(s),
                          darr, int(threads))
    if rc:
        raise OracleError(rc)
    return dG


def sgd_delta(dG: np.ndarray, lr: float) -> np.ndarray:
    """Update of one plain SGD step, -lr * dG (fp64)."""
    lib = _load()
    src = np.ascontiguousarray(dG, dtype=np.float64)
    out = np.empty_like(src)
    lib.orc_sgd_delta(_ptr(src), src.size, float(lr), _ptr(out))
    return out


def forward_k(w, grouped: bool = False, threads: int = 0, cores=None) -> np.ndarray:
    """Pooled forward of K-core tables (every table of w has K = len(n)
    cores), fp64 [B][sum D]: per-index chains, or (grouped) every distinct
    leading-digit prefix computed once and reused."""
    lib = _load()
    K = len(w.tables[0].n)
    assert all(len(t.n) == K for t in w.tables)
    N, n, d, R = _shape_args(w)
    cs, carr = _cores_arg(w.cores if cores is None else cores)
    out = np.zeros((w.B, w.sum_D), dtype=np.float64)
    idx = np.ascontiguousarray(w.indices, dtype=np.int64)
    off = np.ascontiguousarray(w.offsets, dtype=np.int64)
    if grouped:
        rc = lib.orc_forward_k_grouped(w.T, K, _ptr(N), _ptr(n), _ptr(d), _ptr(R), carr, _ptr(idx), _ptr(off),
                                       w.B, idx.shape[0], _ptr(out))
    else:
        rc = lib.orc_forward_k(w.T, K, _ptr(N), _ptr(n), _ptr(d), _ptr(R), carr, _ptr(idx), _ptr(off),
                               w.B, idx.shape[0], _ptr(out), int(threads))
    if rc:
        raise OracleError(rc)
    return out


def backward_k(w, grad_out=None) -> list:
    """Core gradients of sum(grad_out * out) for K-core tables, fp64, shaped
    like the cores (T*K of them): every index's chain reversed on its own,
    lookups in CSR order."""
    lib = _load()
    K = len(w.tables[0].n)
    assert all(len(t.n) == K for t in w.tables)
    N, n, d, R = _shape_args(w)
    cs, carr = _cores_arg(w.cores)
    g = np.ascontiguousarray(w.grad_out if grad_out is None else grad_out, dtype=np.float32)
    if g.shape != (w.B, w.sum_D):
        raise ValueError("grad_out must be [B][sum D]")
    dG = [np.zeros(c.shape, dtype=np.float64) for c in cs]
    darr = (C.c_void_p * len(dG))(*[x.ctypes.data for x in dG])
    idx = np.ascontiguousarray(w.indices, dtype=np.int64)
    off = np.ascontiguousarray(w.offsets, dtype=np.int64)
    rc = lib.orc_backward_k(w.T, K, _ptr(N), _ptr(n), _ptr(d), _ptr(R), carr, _ptr(idx), _ptr(off), w.B,
                            idx.shape[0], _ptr(g), darr)
    if rc:
        raise OracleError(rc)
    return dG
