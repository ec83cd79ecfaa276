"""The forward that allocates nothing (tt_emb_forward_noalloc), for callers
that cannot allocate: through the C ABI it must give the workspace forward's
output bit for bit (the same kernels), on consecutive calls sharing the
library's fixed scratch, and refuse inputs that do not fit that scratch."""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import tensor_train_compressed_gather_amd as tt
from tensor_train_compressed_gather_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH = 64 << 20  # TT_EMB_NOALLOC_SCRATCH_BYTES


def _close(w, got, ref):
    col = w.col_offsets()
    for t in range(w.T):
        r = ref[:, col[t]:col[t + 1]]
        g = got[:, col[t]:col[t + 1]]
        assert np.abs(g.astype(np.float64) - r).max() <= 1e-4 * max(np.abs(r).max(), 1e-30), t


def test_no_alloc_forward_matches_the_workspace_forward():
    emb = None
    # two calls in a row on one handle, the second with a smaller input, then a
    # single-table workload on another handle: each must see only its own data
    for cfg, bags in ((4, 96), (4, 24), (1, None)):
        w = W.make_workload(cfg, bags=bags)
        if emb is None or cfg == 1:
            emb = tt.TTEmbeddingBag(w.tables, DEV)
        need = tt.tt_emb_forward_workspace_size(emb.handle, w.B, w.nnz)
        print(f"[case] no-alloc cfg{cfg} B={w.B} nnz={w.nnz} forward workspace {need} bytes", flush=True)
        assert need <= SCRATCH
        cores = [torch.from_numpy(c).to(DEV) for c in w.cores]
        idx = torch.from_numpy(w.indices).to(DEV)
        off = torch.from_numpy(w.offsets).to(DEV)
        ref = emb.forward(cores, idx, off, w.B)
        out = torch.full_like(ref, float("nan"))
        tt.tt_emb_forward_noalloc(emb.handle, cores, idx, off, w.B, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        _close(w, out.cpu().numpy(), oracle.forward(w))
        # the scratch still holds this grouping: reusing it gives the same output
        out2 = torch.full_like(ref, float("nan"))
        tt.tt_emb_forward_noalloc(emb.handle, cores, idx, off, w.B, out2, flags=tt.TT_EMB_REUSE_GROUPING)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_no_alloc_forward_refuses_what_does_not_fit():
    w = W.make_workload(4, bags=8)
    emb = tt.TTEmbeddingBag(w.tables, DEV)
    cores = [torch.from_numpy(c).to(DEV) for c in w.cores]
    idx = torch.from_numpy(w.indices).to(DEV)
    off = torch.from_numpy(w.offsets).to(DEV)
    out = torch.zeros((w.B, w.sum_D), dtype=torch.float32, device=DEV)
    L = tt.lib()
    ptrs = (C.c_void_p * len(cores))(*[c.data_ptr() for c in cores])
    # sizes of the 26-table batch of 32768 bags: refused before any launch
    rc = L.tt_emb_forward_noalloc(emb.handle, ptrs, C.c_void_p(idx.data_ptr()), C.c_void_p(off.data_ptr()),
                                  32768, 17_900_000, C.c_void_p(out.data_ptr()), 0, None)
    assert rc == tt.TT_EMB_ERR_TOO_LARGE
    assert tt.tt_emb_forward_workspace_size(emb.handle, 32768, 17_900_000) > SCRATCH
    with pytest.raises(tt.TTEmbError) as e:
        tt.tt_emb_forward_noalloc(emb.handle, cores, idx, off, w.B, out, flags=tt.TT_EMB_KEEP_PREFIX)
    assert e.value.status == tt.TT_EMB_ERR_ARG
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0  # nothing ran
