#!/usr/bin/env python
"""Throughput of the TT-EmbeddingBag hot path on one MI355X.

One step = the whole hot path on one batch: index grouping (validation, sort,
unique extraction, prefix run-length encoding, work list), the fused
prefix-shared forward contraction, bag pooling, the backward to every TT core
and the in-place SGD update (lr 0.01), on the 26-table workload at batch
32,768 (rows log-uniform in [1e3, 4e7], D = 64, ranks in {16, 32, 64},
Poisson(20)+1 bag lengths, per-table Zipf skew).  Inputs are seeded and
synthetic and resident in HBM before the timed region.

Prints one JSON line.  Forward-only throughput of the same 26-table workload
and of the 10^7-row D = 128 workload are reported alongside, with the phase
breakdown measured by the library's HIP-event timers on the launch stream.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "pooled TT-embedding lookups/sec at batch 32768 (fwd, fwd+bwd); % of roofline"
PEAK_FP32_TFLOPS = 157.3   # MI355X dense FP32 (matrix cores; also the vector figure)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def mfma_rank(tb):
    """Rank of the matrix-core kernel class a table falls in (R1 = R2 in
    {8, 16, 32, 64}, d1, d2 <= 4, d3 <= 16), else None (generic kernels)."""
    R1, R2 = tb.R[1], tb.R[2]
    d1, d2, d3 = tb.d
    if R1 == R2 and R1 in (8, 16, 32, 64) and d1 <= 4 and d2 <= 4 and d3 <= 16:
        return R1
    return None


def kernel_flops(tabs, U_r, U_p, kept=False):
    """Algorithmic flops of each matrix-core contraction kernel: forward
    (C once per prefix unit, E once per unique row) and backward (dG1 and dG2
    per unit, plus C again unless the forward kept it; dC and the dG3 partial
    per unique row)."""
    out = {}
    for tb, ur, up in zip(tabs, U_r, U_p):
        R = mfma_rank(tb)
        if R is None:
            continue
        n1 = 2 if kept and R >= 32 else 3  # the library keeps C_p at ranks >= 32
        d1, d2, d3 = tb.d
        step1 = 2.0 * d1 * R * d2 * R
        step2 = 2.0 * d1 * d2 * d3 * R
        out[f"fwd_r{R}"] = out.get(f"fwd_r{R}", 0.0) + up * step1 + ur * step2
        out[f"bwd_r{R}"] = out.get(f"bwd_r{R}", 0.0) + up * n1 * step1 + ur * 2 * step2
    return out


def phase_flops(tabs, U_r, U_p, nnz_t, kept=False):
    """Algorithmic flops of the contraction phases (prefix reuse counted once)."""
    fwd = bwd = pool = 0.0
    for tb, ur, up, nz in zip(tabs, U_r, U_p, nnz_t):
        n1 = 2 if kept and mfma_rank(tb) is not None and mfma_rank(tb) >= 32 else 3
        d1, d2, d3 = tb.d
        R1, R2 = tb.R[1], tb.R[2]
        D = d1 * d2 * d3
        step1 = 2.0 * d1 * R1 * d2 * R2
        step2 = 2.0 * D * R2
        fwd += up * step1 + ur * step2
        # dG1 and dG2 (and C unless kept) per unit; dC and the dG3 term per unique row
        bwd += up * n1 * step1 + ur * 2 * step2
        pool += nz * D
    return fwd, bwd, pool


def phase_bytes(w, U_r):
    """Compulsory HBM bytes of pooling: read each unique row once, the inverse
    map and offsets, write the pooled output."""
    e = sum(ur * tb.D * 4 for tb, ur in zip(w.tables, U_r))
    return e + 4 * w.nnz + 8 * (w.T * w.B + 1) + 4 * w.B * w.sum_D


def split_timers(per_step):
    """Per-step timer readings -> (phases, single-kernel timers, grouping
    stages).  Kernel timers (names ending in the rank) and grouping stages
    (stage_*) are nested inside the phases."""
    phases = {k: round(v[0], 4) for k, v in per_step.items()
              if not k[-1].isdigit() and not k.startswith("stage_")}
    kern = {k: v[0] for k, v in per_step.items() if k[-1].isdigit()}
    stages = {k[6:]: round(v[0], 4) for k, v in per_step.items() if k.startswith("stage_")}
    return phases, kern, stages


def kernel_sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "tensor_train_compressed_gather_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, sha):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(kernel, {})
    if r.get("workload") != workload or r.get("src_sha") != sha:
        return None
    return r.get("bytes_per_launch")


# kernel symbol -> (timer name, sources it is built from)
TRAFFIC_KERNELS = {  # (the training step runs one instantiation per rank)
    "k_bwd_class<64,": ("bwd_r64", ["backward.hip", "internal.h"]),
    "k_bwd_class<32,": ("bwd_r32", ["backward.hip", "internal.h"]),
    "k_bwd_class<16,": ("bwd_r16", ["backward.hip", "internal.h"]),
    "k_contract_t<64,": ("fwd_r64", ["forward.hip", "internal.h"]),
    "k_contract_t<32,": ("fwd_r32", ["forward.hip", "internal.h"]),
    "k_contract_w<16,": ("fwd_r16", ["forward.hip", "internal.h"]),
    "k_pool<": ("pool", ["forward.hip", "internal.h"]),
    "k_gu_gather": ("bwd_gather", ["backward.hip", "internal.h"]),
    "k_sorted_meta": ("bwd_sorted_meta", ["backward.hip", "internal.h"]),
}


def write_traffic(d):
    """HBM bytes per launch of the contraction and pooling kernels from four
    rocprofv3 counter runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
    training step, and the same counters on a plain 1 GiB device copy, whose
    readings fix the scale of each counter (bytes moved / bytes counted)."""
    import csv

    def per_kernel(sub):
        acc = {}
        with open(os.path.join(d, sub, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    def copy_scale(sub):
        vals = [v for k, vs in per_kernel(sub).items() if "copyBuffer" in k for v in vs]
        return (1 << 30) / (sum(vals) / len(vals))

    fs, ws = copy_scale("cfetch"), copy_scale("cwrite")
    fetch, write = per_kernel("fetch"), per_kernel("write")
    from tensor_train_compressed_gather_amd import workloads as W
    out = {"_calibration": {"fetch_scale": fs, "write_scale": ws,
                            "copy": "1 GiB fp32 device-to-device copy (bench.py --mode copy)"}}
    for sym, (name, srcs) in TRAFFIC_KERNELS.items():
        fk = [k for k in fetch if sym in k]
        wk = [k for k in write if sym in k]
        if not fk or not wk:
            continue
        fb = sum(fetch[fk[0]]) / len(fetch[fk[0]]) * fs
        wb = sum(write[wk[0]]) / len(write[wk[0]]) * ws
        out[name] = {"workload": W.CONFIG_NAMES[5], "src_sha": kernel_sources_sha(srcs), "fetch_bytes": fb,
                     "write_bytes": wb, "bytes_per_launch": fb + wb}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))


COUNTER_KERNELS = (("k_contract_w<16", "fwd_r16"), ("k_contract_t<32", "fwd_r32"), ("k_contract_t<64", "fwd_r64"),
                   ("k_bwd_class<16", "bwd_r16"), ("k_bwd_class<32", "bwd_r32"), ("k_bwd_class<64", "bwd_r64"),
                   ("k_pool<", "pool"), ("k_gu_gather", "bwd_gather"))


def write_counters(d, trace_csv=None):
    """Per-kernel hardware counters of the training step from two rocprofv3
    --pmc runs (lds/: LdsBankConflict = bank-conflict cycles per conflict-free
    indexed LDS cycle, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE; mfma/: MfmaUtil =
    % of SIMD cycles the matrix core is busy, MfmaFlopsF32 = fp32 MFMA flops
    issued), averaged over the dispatches of each kernel, as a markdown table.
    With the kernel-trace csv, issued flops are also divided by the average
    launch duration."""
    import csv

    vals = {}
    # busy/ (optional): SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE, OccupancyPercent;
    # stallA/, stallB/ (optional): the sequencer's wave-cycle counters (where
    # the waves' time goes: issuing each instruction type, waiting on
    # s_waitcnt / barriers, waiting for an issue slot) and the matrix-core busy
    # cycles
    for sub in ("lds", "mfma", "busy", "stallA", "stallB"):
        path = os.path.join(d, sub, "run_counter_collection.csv")
        if sub not in ("lds", "mfma") and not os.path.exists(path):
            continue
        with open(path) as f:
            for r in csv.DictReader(f):
                vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    dur = {}
    if trace_csv and os.path.exists(trace_csv):
        with open(trace_csv) as f:
            for r in csv.DictReader(f):
                dur.setdefault(r["Kernel_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)

    def avg(sym, counter):
        xs = [v for (k, c), vs in vals.items() if sym in k and c == counter for v in vs]
        return sum(xs) / len(xs) if xs else None

    rows = []
    for sym, name in COUNTER_KERNELS:
        ds = [v for k, vs in dur.items() if sym in k for v in vs]
        t = sum(ds) / len(ds) if ds else None
        fl = avg(sym, "MfmaFlopsF32")
        busy, gui = avg(sym, "SQ_BUSY_CU_CYCLES"), avg(sym, "GRBM_GUI_ACTIVE")
        rows.append({"kernel": name, "lds_bank_conflict_ratio": avg(sym, "LdsBankConflict"),
                     # busy cycles of the CUs summed, against the launch's GPU-active
                     # cycles (GRBM_GUI_ACTIVE, summed over the 8 XCDs) x 256 CUs; on
                     # gfx950 the counter reads cycles (its description says
                     # quad-cycles, which would put every kernel near 390 %)
                     "cu_busy_pct": 100.0 * busy / (gui / 8 * 256) if (busy and gui) else None,
                     "occupancy_pct": avg(sym, "OccupancyPercent"),
                     "lds_conflict_cycles": avg(sym, "SQ_LDS_BANK_CONFLICT"),
                     "lds_active_cycles": avg(sym, "SQ_LDS_IDX_ACTIVE"),
                     "mfma_util_pct": avg(sym, "MfmaUtil"), "mfma_f32_flops": fl,
                     "launch_ms": t * 1e3 if t else None,
                     "mfma_issued_tflops": fl / t / 1e12 if (fl and t) else None})
        wc = avg(sym, "SQ_WAVE_CYCLES")
        if wc:
            # fractions of the waves' resident cycles
            for key, ctr in (("wait_any", "SQ_WAIT_ANY"), ("wait_issue", "SQ_WAIT_INST_ANY"),
                             ("active_any", "SQ_ACTIVE_INST_ANY"), ("active_valu", "SQ_ACTIVE_INST_VALU"),
                             ("active_salu", "SQ_ACTIVE_INST_SCA"), ("active_lds", "SQ_ACTIVE_INST_LDS"),
                             ("active_vmem", "SQ_ACTIVE_INST_VMEM"), ("active_misc", "SQ_ACTIVE_INST_MISC"),
                             ("wait_lds_issue", "SQ_WAIT_INST_LDS")):
                v = avg(sym, ctr)
                rows[-1]["frac_" + key] = v / wc if v is not None else None
            mb, gui2 = avg(sym, "SQ_VALU_MFMA_BUSY_CYCLES"), avg(sym, "GRBM_GUI_ACTIVE")
            # matrix-core busy cycles over (GPU-active cycles per XCD x 1024 SIMDs)
            rows[-1]["mfma_busy_pct_sq"] = 100.0 * mb / (gui2 / 8 * 1024) if (mb and gui2) else None
            for key, ctr in (("insts_mfma", "SQ_INSTS_MFMA"), ("insts_vmem", "SQ_INSTS_VMEM"),
                             ("insts_lds", "SQ_INSTS_LDS"), ("insts_salu", "SQ_INSTS_SALU")):
                rows[-1][key] = avg(sym, ctr)
    print(json.dumps(rows, indent=1))
    return rows


def kcore_flops(tables, indices, offsets, B):
    """Contraction flops of the K-core forward with prefix reuse at every
    length (one intermediate per distinct prefix of length 2..K-1, one last
    contraction per distinct row) and without it (the chain per lookup)."""
    import numpy as np

    grouped = dense = 0
    for t, tab in enumerate(tables):
        K, n, d, R = len(tab.n), tab.n, tab.d, tab.R
        rows = indices[offsets[t * B]:offsets[(t + 1) * B]]
        u = np.unique(rows)
        P = [1]
        for k in range(K):
            P.append(P[-1] * d[k])
        for m in range(2, K + 1):
            per = 2 * P[m - 1] * R[m - 1] * d[m - 1] * R[m]
            div = int(np.prod(n[m:])) if m < K else 1
            grouped += per * (np.unique(u // div).size if m < K else u.size)
            dense += per * rows.size
    return float(grouped), float(dense)


def kcore_extras(torch, tt, W, opts, args):
    out = {}
    for name in ("k4", "k5"):
        wk = W.make_kcore_workload(name)
        wk.grad_out = W.make_grad_out(wk, 20300 + len(wk.tables[0].n))
        bk = Bench(wk, torch, tt, opts)
        # training step on the K-core tables: forward, backward to all K cores, SGD
        tms, _, tph = bk.timed(bk.train_step, args.steps, args.warmup)
        tphase, _, _ = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in tph.items() if v[1]})
        ms, _, ph = bk.timed(bk.fwd, args.steps, args.warmup)
        phase, _, stages = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in ph.items() if v[1]})
        fg, fd = kcore_flops(wk.tables, wk.indices, wk.offsets, wk.B)
        cms = phase.get("contract", 0)
        post = cms + phase.get("pool", 0)
        out[wk.name] = {
            "K": len(wk.tables[0].n), "lookups_per_s": wk.nnz / (ms * 1e-3), "ms": ms, "nnz": wk.nnz,
            "post_grouping_ms": post, "phases_ms": phase, "grouping_stages_ms": stages,
            "contract_flops": fg, "contract_flops_without_reuse": fd,
            "contract_tflops": fg / (cms * 1e-3) / 1e12 if cms else None,
            "contract_frac_fp32_peak": fg / (cms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS if cms else None,
            "train_step": {"ms": tms, "lookups_per_s": wk.nnz / (tms * 1e-3), "phases_ms": tphase},
        }
        del bk
        torch.cuda.empty_cache()
    return out


class Bench:
    def __init__(self, w, torch, tt, options=None, keep=False, forward_only=False):
        self.w, self.torch, self.tt = w, torch, tt
        self.keep = keep
        if keep:
            options = options or tt.tt_emb_options()
            options.keep_prefix = 1
        dev = "cuda"
        self.emb = tt.TTEmbeddingBag(w.tables, dev, options, forward_only=forward_only)
        self.cores = [torch.from_numpy(c).to(dev) for c in w.cores]
        self.idx = torch.from_numpy(w.indices).to(dev)
        self.off = torch.from_numpy(w.offsets).to(dev)
        self.out = torch.empty((w.B, w.sum_D), dtype=torch.float32, device=dev)
        self.grads = None if forward_only else [torch.empty_like(c) for c in self.cores]
        self.gout = torch.from_numpy(w.grad_out).to(dev) if (w.grad_out is not None and not forward_only) else None
        self.emb.workspace(w.B, w.nnz)

    def fwd(self):
        self.emb.forward(self.cores, self.idx, self.off, self.w.B, out=self.out)

    def fwd_post(self):
        # contraction + pooling only: the grouping of the same inputs is already in the workspace
        self.emb.forward(self.cores, self.idx, self.off, self.w.B, out=self.out, flags=self.tt.TT_EMB_REUSE_GROUPING)

    def fwd_fused(self):
        # pooling inside the contraction with float atomics (not bit-reproducible)
        self.emb.forward(self.cores, self.idx, self.off, self.w.B, out=self.out, flags=self.tt.TT_EMB_ATOMIC_POOL)

    def train_step(self):
        tt = self.tt
        kcore = len(self.w.tables[0].n) > 3  # K-core forwards always leave their intermediates in ws
        self.emb.forward(self.cores, self.idx, self.off, self.w.B, out=self.out,
                         flags=tt.TT_EMB_KEEP_PREFIX if (self.keep and not kcore) else 0)
        self.emb.backward(self.gout, self.cores, self.idx, self.off, self.w.B, core_grads=self.grads,
                          flags=tt.TT_EMB_REUSE_GROUPING | (tt.TT_EMB_REUSE_PREFIX if (self.keep or kcore) else 0))
        self.emb.sgd_update(self.cores, self.grads, self.w.lr)

    def timed(self, fn, steps, warmup):
        """Time `steps` calls with the library's phase timers off (each timer
        event on the stream costs a few microseconds), then run `steps` more
        with them on for the per-phase and per-kernel breakdown."""
        torch, tt = self.torch, self.tt
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = ev0.elapsed_time(ev1) / steps
        tt.tt_emb_timing_read(self.emb.handle)          # clear
        tt.tt_emb_timing_enable(self.emb.handle, True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(steps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        self.ms_with_timers = ev0.elapsed_time(ev1) / steps
        tt.tt_emb_timing_enable(self.emb.handle, False)
        phases = tt.tt_emb_timing_read(self.emb.handle)
        assert self.emb.poll_error() == 0
        return ms, wall, phases

    def balance(self):
        tt = self.tt
        out = {}
        for k in tt.BLOCK_STAT_KERNELS:
            r = tt.block_balance(self.emb.block_stats(self.w.B, self.w.nnz, k))
            if r is not None:
                out[k] = r
        return out

    def counts(self):
        g = self.emb.grouping(self.w.B, self.w.nnz)
        tu = g["tab_uniq_start"].cpu().numpy()
        tg = g["tab_grp_start"].cpu().numpy()
        offs = self.w.offsets[:: self.w.B]
        return [int(x) for x in tu[1:] - tu[:-1]], [int(x) for x in tg[1:] - tg[:-1]], \
            [int(x) for x in offs[1:] - offs[:-1]], g["counts"]


def cpu_baseline(w, target_s=12.0):
    """The oracle (per-index fp64 contraction, no reuse) on the host cores, on
    the first S bags of every table, forward + backward when the workload has
    output gradients."""
    import numpy as np

    import oracle
    from tensor_train_compressed_gather_amd import workloads as W

    def sub(S):
        lens, idx = [], []
        for t in range(w.T):
            lo, hi = w.offsets[t * w.B], w.offsets[t * w.B + S]
            lens.append(np.diff(w.offsets[t * w.B: t * w.B + S + 1]))
            idx.append(w.indices[lo:hi])
        s = W.make_custom(w.tables, lens, idx, cores=w.cores)
        if w.grad_out is not None:
            s.grad_out = np.ascontiguousarray(w.grad_out[:S])
        return s

    def run(s):
        t0 = time.perf_counter()
        oracle.forward(s)
        if s.grad_out is not None:
            oracle.backward(s)
        return time.perf_counter() - t0

    S = 4
    s = sub(S)
    t = run(s)
    for _ in range(3):  # grow the sample until it takes about target_s
        if t >= 0.5 * target_s or S >= w.B:
            break
        S = int(min(w.B, max(2 * S, S * target_s / max(t, 1e-3))))
        s = sub(S)
        t = run(s)
    kind = "fwd+bwd" if s.grad_out is not None else "fwd"
    return {"value": s.nnz / t, "unit": "lookups/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"first {S} of {w.B} bags of each of the {w.T} tables ({s.nnz} lookups), "
                      f"{kind}, per-index fp64, {t:.1f} s",
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_single_thread(W):
    """The oracle's pooled forward on one host thread over the whole of the
    three single-table workloads (1000 rows; 10^6 rows, bags of one; 10^7
    rows, bags of 1-64): lookups/s and seconds."""
    import oracle

    out = {}
    for cfg in (1, 2, 3):
        w = W.make_workload(cfg)
        t0 = time.perf_counter()
        oracle.forward(w, threads=1)
        dt = time.perf_counter() - t0
        out[W.CONFIG_NAMES[cfg]] = {"lookups": w.nnz, "s": round(dt, 3), "lookups_per_s": w.nnz / dt,
                                    "kind": "oracle fwd, per-index fp64, 1 thread"}
    return out


def measure_peaks(torch, tt):
    """The device's own FP32 matrix-core rate (tt_emb_peak_mfma: independent
    MFMA chains, no memory traffic) and device-to-device copy bandwidth (1 GiB
    fp32 copy, read + write), timed on the current stream."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus * 4, 20000
    buf = torch.empty(blocks, dtype=torch.float32, device="cuda")
    tt.tt_emb_peak_mfma(blocks, 200, buf)  # warm-up
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    tt.tt_emb_peak_mfma(blocks, iters, buf)
    ev1.record()
    torch.cuda.synchronize()
    mfma = blocks * 4 * 8 * iters * 2048.0 / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev0.record()
    for _ in range(5):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    copy = 5 * 8.0 * n / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst, buf
    return {"mfma_f32_tflops": round(mfma, 2), "copy_gbs": round(copy, 1),
            "datasheet": {"fp32_tflops": PEAK_FP32_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}}


def run_ablation(args, torch, tt, W):
    """The scheduling / reuse ablation of the FlowTT evaluation (static prefix
    mapping, persistent blocks with stealing, stealing plus L2 checkpoints;
    prefix reuse against unique-row-only reuse) on the 26-table forward at
    batch 32768: latency normalised to the static mode, and how evenly each
    persistent launch spread over blocks and compute units."""
    w = W.make_workload(4)
    modes = [("static", 1, 1), ("steal", 2, 1), ("steal_l2", 3, 1), ("default", 0, 1),
             ("default_unique_only", 0, 2)]
    res = {}
    for name, sched, group in modes:
        o = tt.tt_emb_options()
        o.sched_mode, o.group_mode = sched, group
        bf = Bench(w, torch, tt, o)
        fms, _, fph = bf.timed(bf.fwd, args.steps, args.warmup)
        fphase, fkern, _ = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in fph.items() if v[1]})
        _, _, _, fc = bf.counts()
        res[name] = {"ms": round(fms, 4), "contract_ms": fphase.get("contract"), "kernels_ms": fkern,
                     "sched_stats": fc, "balance": bf.balance()}
        del bf
        torch.cuda.empty_cache()
    base, cbase = res["static"]["ms"], res["static"]["contract_ms"]
    for r in res.values():
        r["norm_latency"] = round(r["ms"] / base, 4)
        r["norm_contract"] = round(r["contract_ms"] / cbase, 4) if cbase else None
    print(json.dumps({"mode": "ablation", "workload": W.CONFIG_NAMES[4], "nnz": w.nnz, "steps": args.steps,
                      "results": res}), flush=True)


def run_sweep(args, torch, tt, W, opts):
    """Batch sweep on the 26-table shapes (same tables, bag-length law and
    index laws as the training workload, B bags per table): training step
    (group + forward + backward + SGD) and forward-only (group + forward)
    throughput, the grouping share of each, the workspace the library asks
    for (upper bounds that do not depend on index values) and the peak device
    memory of the step (inputs, cores, gradients, output and workspace)."""
    rows = []
    for B in [int(x) for x in args.batches.split(",") if x]:
        w = W.make_workload(5, bags=B)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        b = Bench(w, torch, tt, opts, keep=args.prefix == "keep")
        ws_bytes = tt.tt_emb_workspace_size(b.emb.handle, w.B, w.nnz)
        tms, _, tph = b.timed(b.train_step, args.steps, args.warmup)
        fms, _, fph = b.timed(b.fwd, args.steps, args.warmup)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del b
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        # inference only: a forward-only workspace, no gradients
        base_i = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        bi = Bench(w, torch, tt, opts, forward_only=True)
        fws_bytes = tt.tt_emb_forward_workspace_size(bi.emb.handle, w.B, w.nnz)
        ims, _, _ = bi.timed(bi.fwd, args.steps, args.warmup)
        torch.cuda.synchronize()
        ipeak = torch.cuda.max_memory_allocated() - base_i
        del bi
        tphase, _, tst = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in tph.items() if v[1]})
        fphase, _, fst = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in fph.items() if v[1]})
        tgroup = tphase.get("group_sort", 0) + tphase.get("group_rle", 0)
        fgroup = fphase.get("group_sort", 0) + fphase.get("group_rle", 0)
        row = {"batch": B, "nnz": w.nnz,
               "train_ms": round(tms, 4), "train_lookups_per_s": w.nnz / (tms * 1e-3),
               "fwd_ms": round(fms, 4), "fwd_lookups_per_s": w.nnz / (fms * 1e-3),
               "grouping_share_train": round(tgroup / tms, 4), "grouping_share_fwd": round(fgroup / fms, 4),
               "train_phases_ms": tphase, "fwd_phases_ms": fphase, "grouping_stages_ms": fst,
               "workspace_bytes": ws_bytes, "peak_device_bytes_train": int(peak),
               "inference": {"fwd_ms": round(ims, 4), "workspace_bytes": fws_bytes,
                             "peak_device_bytes": int(ipeak)}}
        rows.append(row)
        print(f"[sweep] B={B} nnz={w.nnz} train {tms:.3f} ms fwd {fms:.3f} ms ws {ws_bytes / 2**30:.2f} GiB "
              f"inference ws {fws_bytes / 2**30:.2f} GiB peak {ipeak / 2**30:.2f} GiB", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "sweep", "workload": "26 tables (the training workload's shapes), B bags per table",
                      "data": "synthetic", "steps": args.steps, "warmup": args.warmup, "sweep": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the forward-only workloads")
    ap.add_argument("--sched", type=int, default=0, help="0 default, 1 static, 2 steal, 3 steal+L2")
    ap.add_argument("--group", type=int, default=0, help="0 default, 1 prefix, 2 unique-only")
    ap.add_argument("--mode", default="train", choices=("train", "fwd", "copy", "traffic", "counters", "sweep", "kcores",
                                                     "ablation"),
                    help="train: the full step (default); fwd: forward only on --config; "
                         "copy: a plain 1 GiB device copy (counter calibration); "
                         "traffic: turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/traffic.json; "
                         "counters: summarise the LDS bank-conflict and MFMA-utilisation counter runs; "
                         "sweep: training step and forward over --batches on the 26-table shapes; "
                         "kcores: forward of the 4- and 5-core 10^7-row tables; "
                         "ablation: the 26-table forward under each scheduling and grouping mode")
    ap.add_argument("--pmc-dir", default="gpurun_out/m",
                    help="traffic: directory with the fetch/, write/, cfetch/, cwrite/ counter runs")
    ap.add_argument("--config", type=int, default=4, help="workload of --mode fwd (1..4)")
    ap.add_argument("--prefix", default="keep", choices=("keep", "recompute"),
                    help="training step: the forward keeps C_p for the backward (default) or the "
                         "backward recomputes it")
    ap.add_argument("--batches", default="2048,4096,8192,16384,32768,65536,131072",
                    help="sweep: bags per table, comma separated")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.mode == "traffic":
        write_traffic(args.pmc_dir)
        return
    if args.mode == "counters":
        write_counters(args.pmc_dir, os.path.join(args.pmc_dir, "trace", "run_kernel_trace.csv"))
        return

    import torch

    import tensor_train_compressed_gather_amd as tt
    from tensor_train_compressed_gather_amd import workloads as W

    if args.mode == "copy":
        n = 1 << 28  # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"mode": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n, "ms": dt * 1e3,
                          "GBps": 8 * n / dt / 1e9}), flush=True)
        return

    opts = None
    if args.sched or args.group:
        opts = tt.tt_emb_options()
        opts.sched_mode = args.sched
        opts.group_mode = args.group

    if args.mode == "sweep":
        run_sweep(args, torch, tt, W, opts)
        return

    if args.mode == "ablation":
        run_ablation(args, torch, tt, W)
        return

    if args.mode == "kcores":
        print(json.dumps({"mode": "kcores", "fwd_kcores": kcore_extras(torch, tt, W, opts, args)}), flush=True)
        return

    if args.mode == "fwd":
        wf = W.make_workload(args.config)
        bf = Bench(wf, torch, tt, opts)
        fms, _, fph = bf.timed(bf.fwd, args.steps, args.warmup)
        post, _, _ = bf.timed(bf.fwd_post, args.steps, args.warmup)
        ur, up, nz, fc = bf.counts()
        ff, _, _ = phase_flops(wf.tables, ur, up, nz)
        fphase, fkern, fstages = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in fph.items() if v[1]})
        roof = ff / (PEAK_FP32_TFLOPS * 1e12) * 1e3
        print(json.dumps({"mode": "fwd", "workload": W.CONFIG_NAMES[args.config], "ms": fms,
                          "post_grouping_ms": post, "post_grouping_frac_of_roofline": roof / post,
                          "lookups_per_s": wf.nnz / (fms * 1e-3), "phases_ms": fphase,
                          "grouping_stages_ms": fstages, "kernels_ms": fkern,
                          "contract_flops": ff, "unique_rows": sum(ur), "prefix_groups": sum(up),
                          "sched_stats": fc}), flush=True)
        return

    keep = args.prefix == "keep"
    w = W.make_workload(5)
    b = Bench(w, torch, tt, opts, keep=keep)
    ms, wall, ph = b.timed(b.train_step, args.steps, args.warmup)
    U_r, U_p, nnz_t, cnt = b.counts()
    F_fwd, F_bwd, F_pool = phase_flops(w.tables, U_r, U_p, nnz_t, kept=keep)
    value = w.nnz / (ms * 1e-3)
    per_step = {k: (v[0] / max(v[1], 1), v[1]) for k, v in ph.items() if v[1]}
    # single-kernel timers: one HIP event pair per launch, on the library's stream
    phases, kern_ms, stages = split_timers(per_step)
    kern_ms["pool"] = per_step["pool"][0]  # the pooling phase is one kernel
    kflops = kernel_flops(w.tables, U_r, U_p, kept=keep)
    wl = W.CONFIG_NAMES[5]
    # dominant kernel of the step and its roofline
    dom = max(kern_ms, key=kern_ms.get)
    if dom != "pool":
        flops = kflops[dom]
        src = "forward.hip" if dom.startswith("fwd") else "backward.hip"
        achieved = flops / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS, "algorithmic_flops": flops,
                "launch_ms": kern_ms[dom],
                "traffic": load_traffic(dom, wl, kernel_sources_sha([src, "internal.h"]))}
    else:
        byts = phase_bytes(w, U_r)
        achieved = byts / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "algorithmic_bytes": byts, "launch_ms": kern_ms[dom],
                "traffic": load_traffic(dom, wl, kernel_sources_sha(["forward.hip", "internal.h"]))}
    kernels = {k: {"ms": round(v, 4), "tflops": round(kflops[k] / (v * 1e-3) / 1e12, 2) if k in kflops else None}
               for k, v in sorted(kern_ms.items(), key=lambda kv: -kv[1])}
    # how evenly the last step's persistent launches spread over blocks and CUs
    balance = b.balance()
    res = {
        "metric": METRIC, "value": value, "unit": "lookups/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl, "step": "group+fwd+bwd+sgd", "tables": w.T, "batch": w.B, "nnz": w.nnz,
                   "unique_rows": sum(U_r), "prefix_groups": sum(U_p),
                   "prefix_intermediates": "kept by the forward" if keep else "recomputed by the backward",
                   "sched": args.sched,
                   "group": args.group, "wall_s": wall,
                   "ms_per_step_with_phase_timers": b.ms_with_timers},
        "phases_ms": phases,
        "grouping_stages_ms": stages,
        "kernels": kernels,
        "flops": {"fwd_contract": F_fwd, "bwd_contract": F_bwd, "pool_adds": F_pool},
        "sched_stats": cnt,
        "balance": balance,
        "roofline": roof,
    }
    del b
    torch.cuda.empty_cache()

    if not args.no_extra:
        fwd = {}
        for cfg in (4, 3, 2):
            wf = W.make_workload(cfg)
            bf = Bench(wf, torch, tt, opts)
            fms, _, fph = bf.timed(bf.fwd, args.steps, args.warmup)
            ur, up, nz, fc = bf.counts()
            ff, _, _ = phase_flops(wf.tables, ur, up, nz)
            fphase, fkern, fstages = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in fph.items() if v[1]})
            # the forward after grouping (contraction + pooling), timed on its own
            # with the phase timers off (their events would add to it)
            post, _, _ = bf.timed(bf.fwd_post, args.steps, args.warmup)
            cms = fphase.get("contract", 0)
            ws_fwd = tt.tt_emb_forward_workspace_size(bf.emb.handle, wf.B, wf.nnz)
            fwd[W.CONFIG_NAMES[cfg]] = {
                "lookups_per_s": wf.nnz / (fms * 1e-3), "ms": fms, "forward_workspace_bytes": ws_fwd,
                "post_grouping_ms": post, "post_grouping_lookups_per_s": wf.nnz / (post * 1e-3) if post else None,
                "phases_ms": fphase, "kernels_ms": {k: round(v, 4) for k, v in fkern.items()},
                "grouping_stages_ms": fstages, "nnz": wf.nnz, "unique_rows": sum(ur),
                "prefix_groups": sum(up),
                "contract_tflops": ff / (cms * 1e-3) / 1e12 if cms else None,
                "contract_frac_fp32_peak": ff / (cms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS if cms else None,
                "roofline_ms_fp32": ff / (PEAK_FP32_TFLOPS * 1e12) * 1e3,
                "post_grouping_frac_of_roofline": (ff / (PEAK_FP32_TFLOPS * 1e12) * 1e3) / post if post else None,
                "sched_stats": fc,
                "balance": bf.balance(),
            }
            # the non-deterministic fast mode: pooling fused into the contraction
            ums, _, uph = bf.timed(bf.fwd_fused, args.steps, args.warmup)
            uphase, _, _ = split_timers({k: (v[0] / max(v[1], 1), v[1]) for k, v in uph.items() if v[1]})
            upost = uphase.get("contract", 0) + uphase.get("pool", 0)
            fwd[W.CONFIG_NAMES[cfg]]["fused_atomic_pool"] = {
                "ms": ums, "lookups_per_s": wf.nnz / (ums * 1e-3), "post_grouping_ms": round(upost, 4),
                "post_grouping_frac_of_roofline": (ff / (PEAK_FP32_TFLOPS * 1e12) * 1e3) / upost if upost else None,
                "bit_reproducible": False}
            del bf
            torch.cuda.empty_cache()
        res["fwd"] = fwd
        res["fwd_kcores"] = kcore_extras(torch, tt, W, opts, args)

    peaks = measure_peaks(torch, tt)
    res["measured_peaks"] = peaks
    if roof["unit"] == "TFLOP/s":
        roof["frac_of_measured_peak"] = roof["achieved"] / peaks["mfma_f32_tflops"]
    else:
        roof["frac_of_measured_peak"] = roof["achieved"] / peaks["copy_gbs"]
    if "fwd" in res:
        for v in res["fwd"].values():
            if v.get("post_grouping_ms"):
                v["post_grouping_frac_of_measured_roofline"] = (
                    v["roofline_ms_fp32"] * PEAK_FP32_TFLOPS / peaks["mfma_f32_tflops"] / v["post_grouping_ms"])
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
        res["cpu_single_thread"] = cpu_single_thread(W)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
