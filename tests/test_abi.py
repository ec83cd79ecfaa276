"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, and rejects bad shapes before touching
the device."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import tensor_train_compressed_gather_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "tt_emb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_emb_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert "tt_emb_forward" in names and "tt_emb_backward" in names
    L = tt.lib()
    for name in names:
        assert hasattr(L, name), name
    assert sorted(names) == sorted(tt.EXPORTED)


def test_status_strings():
    for code in range(-8, 1):
        s = tt.tt_emb_status_string(code)
        assert s and s != "unknown status"
    assert tt.tt_emb_status_string(-99) == "unknown status"


def test_timer_names_match_the_binding():
    n = len(tt.TIMER_NAMES)
    assert [tt.tt_emb_timer_name(i) for i in range(n)] == list(tt.TIMER_NAMES)
    assert tt.tt_emb_timer_name(n) is None and tt.tt_emb_timer_name(-1) is None
    # one timer per matrix-core contraction kernel, forward and backward
    assert all(f"{p}_r{r}" in tt.TIMER_NAMES for p in ("fwd", "bwd") for r in (8, 16, 32, 64))


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _create(N, n, d, R, opt=None):
    h = C.c_void_p()
    NN = np.asarray(N, np.int64)
    nn = np.asarray(n, np.int32).reshape(-1)
    dd = np.asarray(d, np.int32).reshape(-1)
    RR = np.asarray(R, np.int32).reshape(-1)
    rc = tt.lib().tt_emb_create(len(NN), NN.ctypes.data, nn.ctypes.data, dd.ctypes.data, RR.ctypes.data,
                                C.byref(opt) if opt is not None else None, C.byref(h))
    return rc, h


@pytest.mark.parametrize("N,n,d,R,code", [
    ([1000], [10, 10, 10], [2, 2, 4], [2, 8, 8, 1], tt.TT_EMB_ERR_ARG),      # R0 != 1
    ([1000], [10, 10, 10], [2, 2, 4], [1, 8, 8, 2], tt.TT_EMB_ERR_ARG),      # R3 != 1
    ([1001], [10, 10, 10], [2, 2, 4], [1, 8, 8, 1], tt.TT_EMB_ERR_ARG),      # n1 n2 n3 < N
    ([0], [10, 10, 10], [2, 2, 4], [1, 8, 8, 1], tt.TT_EMB_ERR_ARG),         # empty table
    ([1000], [10, 10, 10], [0, 2, 4], [1, 8, 8, 1], tt.TT_EMB_ERR_ARG),      # zero dim
    ([1000], [10, 10, 10], [16, 16, 8], [1, 8, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),  # D > 1024
    ([1000], [10, 10, 10], [2, 2, 4], [1, 512, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),  # rank > 256
    ([2 ** 31], [2 ** 11, 2 ** 10, 2 ** 10], [2, 2, 4], [1, 8, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),
    ([2 ** 31 - 1000, 999], [2 ** 11, 2 ** 10, 2 ** 10, 10, 10, 10], [2, 2, 4, 2, 2, 4], [1, 8, 8, 1, 1, 8, 8, 1],
     tt.TT_EMB_ERR_UNSUPPORTED),  # rows summed over the tables = 2^31 - 1
])
def test_create_rejects_bad_shapes_before_touching_the_device(N, n, d, R, code):
    rc, h = _create(N, n, d, R)
    assert rc == code
    assert not h.value


def _create_k(K, N, n, d, R):
    h = C.c_void_p()
    NN = np.asarray(N, np.int64)
    nn = np.asarray(n, np.int32).reshape(-1)
    dd = np.asarray(d, np.int32).reshape(-1)
    RR = np.asarray(R, np.int32).reshape(-1)
    rc = tt.lib().tt_emb_create_k(len(NN), K, NN.ctypes.data, nn.ctypes.data, dd.ctypes.data, RR.ctypes.data,
                                  None, C.byref(h))
    return rc, h


@pytest.mark.parametrize("K,N,n,d,R,code", [
    (1, [10], [10], [4], [1, 1], tt.TT_EMB_ERR_ARG),                                   # K < 2
    (2, [100], [10, 10], [2, 4], [1, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),                # two cores
    (9, [512], [2] * 9, [1] * 9, [1] * 10, tt.TT_EMB_ERR_UNSUPPORTED),                 # K > 8
    (3, [1000], [10, 10, 10], [2, 2, 4], [2, 8, 8, 1], tt.TT_EMB_ERR_ARG),             # K = 3 -> 3-core checks
    (4, [1000], [5, 5, 5, 8], [2, 2, 2, 2], [2, 8, 8, 8, 1], tt.TT_EMB_ERR_ARG),       # R0 != 1
    (4, [1000], [5, 5, 5, 8], [2, 2, 2, 2], [1, 8, 8, 8, 3], tt.TT_EMB_ERR_ARG),       # RK != 1
    (4, [1001], [5, 5, 5, 8], [2, 2, 2, 2], [1, 8, 8, 8, 1], tt.TT_EMB_ERR_ARG),       # prod n < N
    (4, [1000], [5, 5, 5, 8], [2, 0, 2, 2], [1, 8, 8, 8, 1], tt.TT_EMB_ERR_ARG),       # zero dim
    (4, [1000], [5, 5, 5, 8], [8, 8, 8, 4], [1, 8, 8, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),  # D > 1024
    (4, [1000], [5, 5, 5, 8], [2, 2, 2, 2], [1, 8, 300, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),  # rank > 256
    (4, [1000], [5, 5, 5, 8], [16, 4, 4, 4], [1, 8, 256, 8, 1], tt.TT_EMB_ERR_UNSUPPORTED),  # LDS
])
def test_create_k_rejects_bad_shapes_before_touching_the_device(K, N, n, d, R, code):
    rc, h = _create_k(K, N, n, d, R)
    assert rc == code
    assert not h.value


def test_create_rejects_bad_options():
    opt = tt.tt_emb_options()
    opt.sched_mode = 7
    rc, _ = _create([1000], [10, 10, 10], [2, 2, 4], [1, 8, 8, 1], opt)
    assert rc == tt.TT_EMB_ERR_ARG
    opt = tt.tt_emb_options()
    opt.chunk_rows = 5000
    rc, _ = _create([1000], [10, 10, 10], [2, 2, 4], [1, 8, 8, 1], opt)
    assert rc == tt.TT_EMB_ERR_ARG
    rc = tt.lib().tt_emb_create(65, None, None, None, None, None, C.byref(C.c_void_p()))
    assert rc == tt.TT_EMB_ERR_ARG


def test_null_handles_are_rejected():
    L = tt.lib()
    out = C.c_size_t()
    assert L.tt_emb_workspace_size(None, 1, 1, C.byref(out)) == tt.TT_EMB_ERR_ARG
    assert L.tt_emb_forward(None, None, None, None, 1, 1, None, None, 0, 0, None) == tt.TT_EMB_ERR_ARG
    assert L.tt_emb_backward(None, None, None, None, None, 1, 1, None, None, 0, 0, None) == tt.TT_EMB_ERR_ARG
    assert L.tt_emb_sgd_update(None, None, None, C.c_float(0.1), None) == tt.TT_EMB_ERR_ARG
    assert L.tt_emb_poll_error(None, None, None) == tt.TT_EMB_ERR_ARG
    assert L.tt_emb_destroy(None) == tt.TT_EMB_OK


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "tensor_train_compressed_gather_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "tt_oracle" not in text and "liboracle" not in text, f


def test_block_balance_summary():
    # host-side summary of per-block records: two CUs, one busy twice as long
    st = {"t0_us": np.array([0.0, 0.0, 0.0, 0.0]), "t1_us": np.array([10.0, 10.0, 5.0, 5.0]),
          "work": np.array([4, 4, 2, 2]), "rows": np.array([8, 8, 4, 4]), "cu": np.array([1, 1, 2, 2])}
    b = tt.block_balance(st)
    assert b["blocks"] == 4 and b["cus"] == 2 and b["span_us"] == 10.0
    assert b["eff_blocks"] == 0.75          # 30 busy of 40 block-microseconds
    assert b["eff_cus"] == 0.75             # CU busy 20 and 10: mean 15 over max 20
    assert b["work_max_over_mean"] == round(4 / 3, 3) and b["rows_max_over_mean"] == round(8 / 6, 3)
    assert tt.block_balance(None) is None


def test_block_stats_rejects_bad_arguments_on_the_host():
    # argument checks come before any device work
    L = tt.lib()
    recs = (tt.tt_emb_block_stat * 4)()
    n, khz = C.c_int32(), C.c_int64()
    for kernel in (-1, 8):
        rc = L.tt_emb_block_stats(None, None, 0, 1, 1, kernel, None, recs, 4, C.byref(n), C.byref(khz))
        assert rc == tt.TT_EMB_ERR_ARG
    rc = L.tt_emb_block_stats(None, None, 0, 1, 1, 0, None, None, 4, C.byref(n), C.byref(khz))
    assert rc == tt.TT_EMB_ERR_ARG
    rc = L.tt_emb_block_stats(None, None, 0, 1, 1, 0, None, recs, 4, C.byref(n), C.byref(khz))
    assert rc == tt.TT_EMB_ERR_ARG  # no handle


def test_victim_order_is_a_permutation_for_every_grid():
    # every persistent grid is a multiple of 8 blocks; for each such size up
    # to 4096 and every block, the stealing order starts with the block's own
    # range, visits every block exactly once, and keeps to the block's own XCD
    # (block mod 8) for its first nb/8 victims (the thieves' range)
    for nb in range(8, 4097, 8):
        mes = range(nb) if nb <= 256 else sorted({0, 1, 7, 8, nb // 2, nb - 9, nb - 1})
        for me in mes:
            order = tt.tt_emb_victim_order(me, nb)
            assert order[0] == me
            assert np.array_equal(np.sort(order), np.arange(nb)), (nb, me)
            assert np.all(order[: nb // 8] % 8 == me % 8), (nb, me)
    for nb, me in ((0, 0), (4, 0), (12, 0), (16, 16), (16, -1)):
        with pytest.raises(tt.TTEmbError) as e:
            tt.tt_emb_victim_order(me, nb)
        assert e.value.status == tt.TT_EMB_ERR_ARG


def test_binding_rejects_wrong_dtype_layout_or_device():
    # the library takes raw pointers: the binding must refuse what the
    # kernels would misread before any call reaches it
    import torch

    idx64 = torch.zeros(4, dtype=torch.int64)
    off64 = torch.zeros(3, dtype=torch.int64)
    core = torch.zeros(8, dtype=torch.float32)
    out = torch.zeros(2, 4, dtype=torch.float32)
    ws = torch.zeros(256, dtype=torch.uint8)
    cases = [
        dict(indices=idx64.to(torch.int32), msg="dtype"),
        dict(offsets=off64.to(torch.int32), msg="dtype"),
        dict(cores=[core.double()], msg="dtype"),
        dict(cores=[torch.zeros(4, 4)[:, 1]], msg="contiguous"),
        dict(out=out.t(), msg="contiguous"),
        dict(msg="GPU"),  # host tensors throughout
    ]
    for c in cases:
        args = dict(indices=idx64, offsets=off64, cores=[core], out=out)
        args.update({k: v for k, v in c.items() if k != "msg"})
        with pytest.raises(tt.TTEmbError) as e:
            tt.tt_emb_forward(None, args["cores"], args["indices"], args["offsets"], 2, args["out"], ws)
        assert e.value.status == tt.TT_EMB_ERR_ARG and c["msg"] in str(e.value), c
    with pytest.raises(tt.TTEmbError):
        tt.tt_emb_backward(None, out.double(), [core], idx64, off64, 2, [core], ws)
    with pytest.raises(tt.TTEmbError):
        tt.tt_emb_sgd_update(None, [core.double()], [core], 0.01)


def test_binding_module_names_resolve():
    # every global name the binding reads is defined in it or a builtin (a
    # static check: the marshalling paths that reach the library need a GPU)
    import ast
    import builtins

    src = open(os.path.join(ROOT, "tensor_train_compressed_gather_amd", "__init__.py")).read()
    tree = ast.parse(src)
    defined = set(dir(builtins)) | {"__file__"}
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            defined.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            defined |= {(a.asname or a.name).split(".")[0] for a in node.names}
        elif isinstance(node, ast.arg):
            defined.add(node.arg)
        elif isinstance(node, ast.Name) and isinstance(node.ctx, ast.Store):
            defined.add(node.id)
        elif isinstance(node, ast.ExceptHandler) and node.name:
            defined.add(node.name)
    used = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert not (used - defined), sorted(used - defined)
