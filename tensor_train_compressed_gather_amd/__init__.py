"""MI355X (gfx950) TT-EmbeddingBag with prefix-shared reuse.

Python binding of ``libtt_emb.so`` (C ABI in ``include/tt_emb.h``).  This
module only marshals arguments: torch supplies device memory and the current
HIP stream; every step of the path runs in the library's HIP kernels.  There
is no CPU fallback -- if the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes as C
import math
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# TT_EMB_LIB names another build of the same library (the host-sanitizer build
# the CPU tests make); there is no fallback either way
LIB_PATH = os.environ.get("TT_EMB_LIB") or os.path.join(_HERE, "libtt_emb.so")

TT_EMB_OK = 0
TT_EMB_ERR_ARG = -1
TT_EMB_ERR_INDEX = -2
TT_EMB_ERR_WORKSPACE = -3
TT_EMB_ERR_UNSUPPORTED = -4
TT_EMB_ERR_HIP = -5
TT_EMB_ERR_NOMEM = -6
TT_EMB_ERR_OFFSETS = -7
TT_EMB_ERR_TOO_LARGE = -8

TT_EMB_SCHED_DEFAULT, TT_EMB_SCHED_STATIC, TT_EMB_SCHED_STEAL, TT_EMB_SCHED_STEAL_L2 = 0, 1, 2, 3
TT_EMB_GROUP_DEFAULT, TT_EMB_GROUP_PREFIX, TT_EMB_GROUP_UNIQUE_ONLY = 0, 1, 2
TT_EMB_REUSE_GROUPING = 1
TT_EMB_KEEP_PREFIX = 2
TT_EMB_REUSE_PREFIX = 4
TT_EMB_ATOMIC_POOL = 8

EXPORTED = (
    "tt_emb_create", "tt_emb_create_k", "tt_emb_destroy", "tt_emb_workspace_size", "tt_emb_forward_workspace_size",
    "tt_emb_group", "tt_emb_forward", "tt_emb_forward_noalloc",
    "tt_emb_backward", "tt_emb_sgd_update", "tt_emb_grouping_view", "tt_emb_poll_error",
    "tt_emb_status_string", "tt_emb_timing_enable", "tt_emb_timing_read", "tt_emb_timer_name",
    "tt_emb_block_stats", "tt_emb_victim_order", "tt_emb_peak_mfma",
)
BLOCK_STAT_KERNELS = ("fwd_r8", "fwd_r16", "fwd_r32", "fwd_r64", "bwd_r8", "bwd_r16", "bwd_r32", "bwd_r64")
TIMER_NAMES = ("group_sort", "group_rle", "contract", "pool", "bwd_gather", "bwd_contract",
               "bwd_reduce", "sgd", "fwd_r8", "fwd_r16", "fwd_r32", "fwd_r64",
               "bwd_r8", "bwd_r16", "bwd_r32", "bwd_r64",
               "stage_decode", "stage_sort", "stage_unique", "stage_prefix", "stage_order", "stage_worklist")


class tt_emb_options(C.Structure):
    _fields_ = [("sched_mode", C.c_int32), ("group_mode", C.c_int32), ("chunk_rows", C.c_int32),
                ("num_blocks", C.c_int32), ("check_indices", C.c_int32), ("force_generic", C.c_int32),
                ("keep_prefix", C.c_int32), ("reserved", C.c_int32)]


class tt_emb_grouping(C.Structure):
    _fields_ = [("nnz", C.c_int64), ("num_unique", C.c_int64), ("num_groups", C.c_int64),
                ("perm", C.c_void_p), ("uniq_row", C.c_void_p), ("uniq_start", C.c_void_p),
                ("inv", C.c_void_p), ("grp_prefix", C.c_void_p), ("grp_start", C.c_void_p),
                ("tab_uniq_start", C.c_void_p), ("tab_grp_start", C.c_void_p),
                ("num_units", C.c_int64), ("num_tiles", C.c_int64), ("num_chunks", C.c_int64),
                ("num_split_tiles", C.c_int64), ("num_steals", C.c_int64),
                ("num_ckpt_hits", C.c_int64), ("num_ckpt_misses", C.c_int64)]


class tt_emb_block_stat(C.Structure):
    _fields_ = [("t_start", C.c_int64), ("t_end", C.c_int64), ("work", C.c_int32), ("rows", C.c_int32),
                ("cu", C.c_int32), ("grid", C.c_int32)]


_lib = None
_lock = threading.Lock()


def lib():
    """Load libtt_emb.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                  "or python -m tensor_train_compressed_gather_amd.build")
            L = C.CDLL(LIB_PATH)
            p, i32, i64, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
            L.tt_emb_create.argtypes = [i32, p, p, p, p, C.POINTER(tt_emb_options), C.POINTER(p)]
            L.tt_emb_create_k.argtypes = [i32, i32, p, p, p, p, C.POINTER(tt_emb_options), C.POINTER(p)]
            L.tt_emb_destroy.argtypes = [p]
            L.tt_emb_workspace_size.argtypes = [p, i64, i64, C.POINTER(C.c_size_t)]
            L.tt_emb_forward_workspace_size.argtypes = [p, i64, i64, C.POINTER(C.c_size_t)]
            L.tt_emb_group.argtypes = [p, p, p, i64, i64, p, C.c_size_t, p]
            L.tt_emb_forward.argtypes = [p, p, p, p, i64, i64, p, p, C.c_size_t, u32, p]
            L.tt_emb_forward_noalloc.argtypes = [p, p, p, p, i64, i64, p, u32, p]
            L.tt_emb_backward.argtypes = [p, p, p, p, p, i64, i64, p, p, C.c_size_t, u32, p]
            L.tt_emb_sgd_update.argtypes = [p, p, p, C.c_float, p]
            L.tt_emb_grouping_view.argtypes = [p, p, C.c_size_t, i64, i64, p, C.POINTER(tt_emb_grouping)]
            L.tt_emb_poll_error.argtypes = [p, p, p]
            L.tt_emb_block_stats.argtypes = [p, p, C.c_size_t, i64, i64, i32, p, p, i32, p, p]
            L.tt_emb_victim_order.argtypes = [i32, i32, p]
            L.tt_emb_peak_mfma.argtypes = [i32, i32, p, p]
            L.tt_emb_status_string.argtypes = [C.c_int]
            L.tt_emb_status_string.restype = C.c_char_p
            L.tt_emb_timing_enable.argtypes = [p, i32]
            L.tt_emb_timing_read.argtypes = [p, p, p]
            L.tt_emb_timer_name.argtypes = [i32]
            L.tt_emb_timer_name.restype = C.c_char_p
            for name in EXPORTED:
                if name not in ("tt_emb_status_string", "tt_emb_timer_name"):
                    getattr(L, name).restype = C.c_int
            _lib = L
    return _lib


class TTEmbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tt_emb_status_string(status)} ({status})")


def _check(rc: int, where: str):
    if rc != TT_EMB_OK:
        raise TTEmbError(rc, where)


def _stream(stream):
    if stream is None:
        import torch

        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(0 if t is None else t.data_ptr())


def _need(specs):
    """Reject tensors the kernels would misread: the library takes raw
    pointers and cannot tell an int32 index array, a strided view or a host
    tensor from the int64 / fp32 contiguous device buffers it expects (reading
    8 bytes per index from a 4-byte array would run past the allocation).
    specs: (tensor or list of tensors, name, dtype name).  Types and layouts
    are checked first, then that every tensor is on one and the same GPU."""
    import torch

    kinds = {"int64": torch.int64, "float32": torch.float32, "uint8": torch.uint8}
    flat = []
    for ts, what, dtype in specs:
        if isinstance(ts, (list, tuple)):
            flat += [(t, f"{what}[{i}]", dtype) for i, t in enumerate(ts)]
        else:
            flat.append((ts, what, dtype))
    for t, what, dtype in flat:
        if not torch.is_tensor(t):
            raise TTEmbError(TT_EMB_ERR_ARG, f"{what}: expected a torch tensor, got {type(t).__name__}")
        if t.dtype != kinds[dtype]:
            raise TTEmbError(TT_EMB_ERR_ARG, f"{what}: dtype {t.dtype}, expected {kinds[dtype]}")
        if not t.is_contiguous():
            raise TTEmbError(TT_EMB_ERR_ARG, f"{what}: not contiguous")
    device = None
    for t, what, _ in flat:
        if t.device.type != "cuda":
            raise TTEmbError(TT_EMB_ERR_ARG, f"{what}: on {t.device}, expected a GPU tensor")
        if device is not None and t.device != device:
            raise TTEmbError(TT_EMB_ERR_ARG, f"{what}: on {t.device}, expected {device} like the others")
        device = t.device


def _ptr_array(tensors):
    arr = (C.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    return arr


def tt_emb_status_string(status: int) -> str:
    return lib().tt_emb_status_string(int(status)).decode()


def tt_emb_create_k(K: int, num_rows, n, d, R, options: tt_emb_options | None = None):
    """K-core tables: num_rows [T], n [T][K], d [T][K], R [T][K+1] -> handle."""
    import numpy as np

    N = np.ascontiguousarray(np.asarray(num_rows, dtype=np.int64).reshape(-1))
    nn = np.ascontiguousarray(np.asarray(n, dtype=np.int32).reshape(-1))
    dd = np.ascontiguousarray(np.asarray(d, dtype=np.int32).reshape(-1))
    RR = np.ascontiguousarray(np.asarray(R, dtype=np.int32).reshape(-1))
    T = N.shape[0]
    if nn.shape[0] != K * T or dd.shape[0] != K * T or RR.shape[0] != (K + 1) * T:
        raise ValueError("shape arrays must have KT, KT and (K+1)T entries")
    h = C.c_void_p()
    rc = lib().tt_emb_create_k(T, int(K), N.ctypes.data, nn.ctypes.data, dd.ctypes.data, RR.ctypes.data,
                               C.byref(options) if options is not None else None, C.byref(h))
    _check(rc, "tt_emb_create_k")
    return h


def tt_emb_create(num_rows, n, d, R, options: tt_emb_options | None = None):
    """num_rows [T], n [T][3], d [T][3], R [T][4] (host sequences) -> handle."""
    import numpy as np

    N = np.ascontiguousarray(np.asarray(num_rows, dtype=np.int64).reshape(-1))
    nn = np.ascontiguousarray(np.asarray(n, dtype=np.int32).reshape(-1))
    dd = np.ascontiguousarray(np.asarray(d, dtype=np.int32).reshape(-1))
    RR = np.ascontiguousarray(np.asarray(R, dtype=np.int32).reshape(-1))
    T = N.shape[0]
    if nn.shape[0] != 3 * T or dd.shape[0] != 3 * T or RR.shape[0] != 4 * T:
        raise ValueError("shape arrays must have 3T, 3T and 4T entries")
    h = C.c_void_p()
    rc = lib().tt_emb_create(T, N.ctypes.data, nn.ctypes.data, dd.ctypes.data, RR.ctypes.data,
                             C.byref(options) if options is not None else None, C.byref(h))
    _check(rc, "tt_emb_create")
    return h


def tt_emb_destroy(h):
    _check(lib().tt_emb_destroy(h), "tt_emb_destroy")


def tt_emb_workspace_size(h, B: int, nnz: int) -> int:
    out = C.c_size_t()
    _check(lib().tt_emb_workspace_size(h, int(B), int(nnz), C.byref(out)), "tt_emb_workspace_size")
    return int(out.value)


def tt_emb_forward_workspace_size(h, B: int, nnz: int) -> int:
    out = C.c_size_t()
    _check(lib().tt_emb_forward_workspace_size(h, int(B), int(nnz), C.byref(out)), "tt_emb_forward_workspace_size")
    return int(out.value)


def tt_emb_group(h, indices, offsets, B: int, ws, stream=None):
    _need([(indices, "indices", "int64"), (offsets, "offsets", "int64"), (ws, "workspace", "uint8")])
    rc = lib().tt_emb_group(h, _ptr(indices), _ptr(offsets), int(B), int(indices.numel()), _ptr(ws),
                            ws.numel(), _stream(stream))
    _check(rc, "tt_emb_group")


def tt_emb_forward(h, cores, indices, offsets, B: int, out, ws, flags: int = 0, stream=None):
    _need([(indices, "indices", "int64"), (offsets, "offsets", "int64"), (cores, "cores", "float32"),
           (out, "out", "float32"), (ws, "workspace", "uint8")])
    rc = lib().tt_emb_forward(h, _ptr_array(cores), _ptr(indices), _ptr(offsets), int(B),
                              int(indices.numel()), _ptr(out), _ptr(ws), ws.numel(), int(flags),
                              _stream(stream))
    _check(rc, "tt_emb_forward")


def tt_emb_forward_noalloc(h, cores, indices, offsets, B: int, out, flags: int = 0, stream=None):
    """The forward with the library's fixed per-GPU scratch instead of a
    workspace (allocates nothing; calls on one GPU must not overlap)."""
    _need([(indices, "indices", "int64"), (offsets, "offsets", "int64"), (cores, "cores", "float32"),
           (out, "out", "float32")])
    rc = lib().tt_emb_forward_noalloc(h, _ptr_array(cores), _ptr(indices), _ptr(offsets), int(B),
                                      int(indices.numel()), _ptr(out), int(flags), _stream(stream))
    _check(rc, "tt_emb_forward_noalloc")


def tt_emb_backward(h, grad_out, cores, indices, offsets, B: int, core_grads, ws, flags: int = 0,
                    stream=None):
    _need([(indices, "indices", "int64"), (offsets, "offsets", "int64"), (grad_out, "grad_out", "float32"),
           (cores, "cores", "float32"), (core_grads, "core_grads", "float32"), (ws, "workspace", "uint8")])
    rc = lib().tt_emb_backward(h, _ptr(grad_out), _ptr_array(cores), _ptr(indices), _ptr(offsets),
                               int(B), int(indices.numel()), _ptr_array(core_grads), _ptr(ws),
                               ws.numel(), int(flags), _stream(stream))
    _check(rc, "tt_emb_backward")


def tt_emb_sgd_update(h, cores, core_grads, lr: float, stream=None):
    _need([(cores, "cores", "float32"), (core_grads, "core_grads", "float32")])
    rc = lib().tt_emb_sgd_update(h, _ptr_array(cores), _ptr_array(core_grads), float(lr), _stream(stream))
    _check(rc, "tt_emb_sgd_update")


def tt_emb_poll_error(h, ws, stream=None) -> int:
    """Synchronises the stream; returns the device-side status (0 = ok)."""
    return int(lib().tt_emb_poll_error(h, _ptr(ws), _stream(stream)))


def tt_emb_grouping_view(h, ws, B: int, nnz: int, T: int, stream=None) -> dict:
    """Grouping arrays held in ws, as int32 torch views into ws, plus counts."""
    import torch

    v = tt_emb_grouping()
    rc = lib().tt_emb_grouping_view(h, _ptr(ws), ws.numel(), int(B), int(nnz), _stream(stream), C.byref(v))
    _check(rc, "tt_emb_grouping_view")
    base = ws.data_ptr()
    i32 = ws.view(torch.int32) if ws.numel() % 4 == 0 else None

    def arr(ptr, count):
        off = (ptr - base)
        assert off % 4 == 0
        return i32[off // 4: off // 4 + int(count)]

    U, G = v.num_unique, v.num_groups
    return {
        "perm": arr(v.perm, nnz), "uniq_row": arr(v.uniq_row, U), "uniq_start": arr(v.uniq_start, U + 1),
        "inv": arr(v.inv, nnz), "grp_prefix": arr(v.grp_prefix, G), "grp_start": arr(v.grp_start, G + 1),
        "tab_uniq_start": arr(v.tab_uniq_start, T + 1), "tab_grp_start": arr(v.tab_grp_start, T + 1),
        "counts": {k: int(getattr(v, k)) for k in ("num_unique", "num_groups", "num_units", "num_tiles",
                                                    "num_chunks", "num_split_tiles", "num_steals",
                                                    "num_ckpt_hits", "num_ckpt_misses")},
    }


def tt_emb_block_stats(h, ws, B: int, nnz: int, kernel, stream=None):
    """Per-block records of the last launch of a persistent matrix-core kernel
    (kernel: index or name in BLOCK_STAT_KERNELS) as numpy arrays (t0, t1 in
    microseconds from the earliest start, work, rows, cu); None when it did
    not run.  Synchronises the stream."""
    import numpy as np

    k = BLOCK_STAT_KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    cap = 2048
    recs = (tt_emb_block_stat * cap)()
    n = C.c_int32()
    khz = C.c_int64()
    rc = lib().tt_emb_block_stats(h, _ptr(ws), ws.numel(), int(B), int(nnz), k, _stream(stream), recs, cap,
                                  C.byref(n), C.byref(khz))
    _check(rc, "tt_emb_block_stats")
    if n.value == 0:
        return None
    m = n.value
    t0 = np.array([recs[i].t_start for i in range(m)], dtype=np.int64)
    t1 = np.array([recs[i].t_end for i in range(m)], dtype=np.int64)
    us = 1e3 / float(khz.value)
    base = t0.min()
    return {"t0_us": (t0 - base) * us, "t1_us": (t1 - base) * us,
            "work": np.array([recs[i].work for i in range(m)], dtype=np.int64),
            "rows": np.array([recs[i].rows for i in range(m)], dtype=np.int64),
            "cu": np.array([recs[i].cu for i in range(m)], dtype=np.int64),
            "grid": int(recs[0].grid), "clock_khz": int(khz.value)}


def block_balance(st) -> dict | None:
    """Load-balance summary of one launch's per-block records (host logic).

    eff_blocks = total block busy time / (blocks x launch span): 1.0 when
    every block works until the launch ends; eff_cus = the same over compute
    units (busy time of the blocks a CU ran, against the busiest CU);
    work_max_over_mean / rows_max_over_mean = how unevenly the chunks and
    rows were handed out."""
    if st is None:
        return None
    import numpy as np

    t0, t1 = st["t0_us"], st["t1_us"]
    busy = t1 - t0
    span = float(t1.max() - t0.min())
    n = len(busy)
    cus, inv = np.unique(st["cu"], return_inverse=True)
    cu_busy = np.bincount(inv, weights=busy)
    work, rows = st["work"].astype(np.float64), st["rows"].astype(np.float64)
    return {"blocks": n, "cus": int(len(cus)), "span_us": round(span, 2),
            "eff_blocks": round(float(busy.sum() / (n * span)), 4) if span > 0 else None,
            "eff_cus": round(float(cu_busy.mean() / cu_busy.max()), 4) if cu_busy.max() > 0 else None,
            "busy_us_min_mean_max": [round(float(busy.min()), 2), round(float(busy.mean()), 2),
                                     round(float(busy.max()), 2)],
            "start_spread_us": round(float(t0.max() - t0.min()), 2),
            "work_max_over_mean": round(float(work.max() / work.mean()), 3) if work.mean() > 0 else None,
            "rows_max_over_mean": round(float(rows.max() / rows.mean()), 3) if rows.mean() > 0 else None}


def tt_emb_victim_order(me: int, nb: int):
    """Blocks that block `me` of an nb-block persistent grid claims chunks
    from, in order (host-side; the kernels use the same function)."""
    import numpy as np

    order = np.empty(max(int(nb), 0), dtype=np.int32)
    _check(lib().tt_emb_victim_order(int(me), int(nb), order.ctypes.data if order.size else None),
           "tt_emb_victim_order")
    return order


def tt_emb_peak_mfma(blocks: int, iters: int, out, stream=None):
    """Launch the FP32 matrix-core peak kernel (measurement aid): blocks x 4
    waves x 8 chains x iters instructions of 2048 flops."""
    _need([(out, "out", "float32")])
    _check(lib().tt_emb_peak_mfma(int(blocks), int(iters), _ptr(out), _stream(stream)), "tt_emb_peak_mfma")


def tt_emb_timing_enable(h, enable: bool = True):
    _check(lib().tt_emb_timing_enable(h, 1 if enable else 0), "tt_emb_timing_enable")


def tt_emb_timing_read(h) -> dict:
    """Synchronises; returns {timer name: (total ms, intervals)} and clears."""
    n = len(TIMER_NAMES)
    ms = (C.c_double * n)()
    cnt = (C.c_int32 * n)()
    _check(lib().tt_emb_timing_read(h, ms, cnt), "tt_emb_timing_read")
    return {TIMER_NAMES[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


def tt_emb_timer_name(i: int):
    r = lib().tt_emb_timer_name(int(i))
    return None if r is None else r.decode()


class TTEmbeddingBag:
    """Owns a handle and a workspace for one table set (marshalling only).

    ``cores`` is the list of 3T fp32 device tensors shaped
    [n_k][R_{k-1}][d_k][R_k]; indices/offsets are int64 device tensors in
    table-major CSR (T*B+1 offsets)."""

    def __init__(self, tables, device="cuda", options: tt_emb_options | None = None, forward_only: bool = False):
        self.tables = list(tables)
        self.T = len(self.tables)
        self.K = len(self.tables[0].n)
        if self.K == 3:
            self.handle = tt_emb_create([t.N for t in self.tables], [t.n for t in self.tables],
                                        [t.d for t in self.tables], [t.R for t in self.tables], options)
        else:
            self.handle = tt_emb_create_k(self.K, [t.N for t in self.tables], [t.n for t in self.tables],
                                          [t.d for t in self.tables], [t.R for t in self.tables], options)
        self.device = device
        self.sum_D = sum(int(math.prod(t.d)) for t in self.tables)
        self._ws = None
        self._ws_key = None
        # inference only: the smaller forward workspace (no backward, no
        # TT_EMB_KEEP_PREFIX)
        self.forward_only = bool(forward_only)

    def workspace(self, B: int, nnz: int):
        import torch

        key = (int(B), int(nnz))
        if self._ws_key != key:
            size = tt_emb_forward_workspace_size if self.forward_only else tt_emb_workspace_size
            need = size(self.handle, B, nnz)
            if self._ws is None or self._ws.numel() < need:
                self._ws = None
                self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self._ws_key = key
        return self._ws

    def _core_sizes(self):
        sizes = []
        for t in self.tables:
            for k in range(self.K):
                sizes.append(int(t.n[k]) * int(t.R[k]) * int(t.d[k]) * int(t.R[k + 1]))
        return sizes

    def _check_shapes(self, cores, indices, offsets, B: int, out=None, grad_out=None, core_grads=None):
        """Sizes the kernels index by: K*T cores of n_k*R_k*d_k*R_{k+1}
        elements, T*B+1 offsets, [B][sum D] outputs and output gradients."""
        sizes = self._core_sizes()
        if len(cores) != len(sizes):
            raise TTEmbError(TT_EMB_ERR_ARG, f"cores: {len(cores)} tensors, expected {len(sizes)}")
        for i, (c, n) in enumerate(zip(cores, sizes)):
            if c.numel() != n:
                raise TTEmbError(TT_EMB_ERR_ARG, f"cores[{i}]: {c.numel()} elements, expected {n}")
        if core_grads is not None:
            if len(core_grads) != len(sizes):
                raise TTEmbError(TT_EMB_ERR_ARG, f"core_grads: {len(core_grads)} tensors, expected {len(sizes)}")
            for i, (g, n) in enumerate(zip(core_grads, sizes)):
                if g.numel() != n:
                    raise TTEmbError(TT_EMB_ERR_ARG, f"core_grads[{i}]: {g.numel()} elements, expected {n}")
        if offsets.numel() != self.T * int(B) + 1:
            raise TTEmbError(TT_EMB_ERR_ARG, f"offsets: {offsets.numel()} entries, expected T*B+1 = "
                                             f"{self.T * int(B) + 1}")
        for name, x in (("out", out), ("grad_out", grad_out)):
            if x is not None and x.numel() != int(B) * self.sum_D:
                raise TTEmbError(TT_EMB_ERR_ARG, f"{name}: {x.numel()} elements, expected B*sum(D) = "
                                                 f"{int(B) * self.sum_D}")

    def forward(self, cores, indices, offsets, B: int, out=None, flags: int = 0, stream=None):
        import torch

        if out is None:
            out = torch.empty((B, self.sum_D), dtype=torch.float32, device=self.device)
        self._check_shapes(cores, indices, offsets, B, out=out)
        ws = self.workspace(B, indices.numel())
        tt_emb_forward(self.handle, cores, indices, offsets, B, out, ws, flags, stream)
        return out

    def backward(self, grad_out, cores, indices, offsets, B: int, core_grads=None, flags: int = 0,
                 stream=None):
        import torch

        if core_grads is None:
            core_grads = [torch.empty_like(c) for c in cores]
        self._check_shapes(cores, indices, offsets, B, grad_out=grad_out, core_grads=core_grads)
        ws = self.workspace(B, indices.numel())
        tt_emb_backward(self.handle, grad_out, cores, indices, offsets, B, core_grads, ws, flags, stream)
        return core_grads

    def sgd_update(self, cores, core_grads, lr: float, stream=None):
        sizes = self._core_sizes()
        if len(cores) != len(sizes) or len(core_grads) != len(sizes) or any(
                c.numel() != n or g.numel() != n for c, g, n in zip(cores, core_grads, sizes)):
            raise TTEmbError(TT_EMB_ERR_ARG, "sgd_update: cores and gradients must match the tables' core sizes")
        tt_emb_sgd_update(self.handle, cores, core_grads, lr, stream)

    def poll_error(self, stream=None) -> int:
        return tt_emb_poll_error(self.handle, self._ws, stream)

    def grouping(self, B: int, nnz: int, stream=None) -> dict:
        return tt_emb_grouping_view(self.handle, self._ws, B, nnz, self.T, stream)

    def block_stats(self, B: int, nnz: int, kernel, stream=None):
        return tt_emb_block_stats(self.handle, self._ws, B, nnz, kernel, stream)

    def close(self):
        if self.handle is not None:
            tt_emb_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
