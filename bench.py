#!/usr/bin/env python3
"""Benchmark of tree-masked verify attention on one MI355X.

One step = one tv_verify_attn call (mask packing + split attention + LSE merge)
over one batch of seeded synthetic inputs already resident in HBM, with cold
caches: before each step a 1 GiB fill kernel (outside the timed events) evicts
the pool, indices and mask from the 256 MB MALL and the L2s.  Each timed step's
call is bracketed by events on its stream, and its split-attention kernel's own
dispatch stamps a second event pair with its start and end
(tv_verify_attn_timed).  The warm-up steps are the same, untimed.  Beside it:
the same call back to back with warm caches, and replayed from a captured HIP
graph.  Default workload: 1 request, 32 draft tokens, 32768-key prefix, 16
heads (the 32k-prefix configuration the metric is quoted at), with the
library's own split plan (`--splits 32` gives the configuration's literal
split count; outputs do not depend on it).

Prints one JSON line: throughput as gathered-KV GB/s (sum over requests of
L_b * 1152 bytes per call / median cold call time), the roofline of the split
kernel from its event-timed average over the timed steps, and the fp64 CPU
oracle timed on a bounded sample.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
# every WARM_STRIDE-th call of the warm back-to-back figure carries the split
# kernel's event pair (every timed, cold-cache step carries one)
WARM_STRIDE = 8
sys.path.insert(0, ROOT)

import tv_workload as W  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


class HipEvents:
    """Raw hipEvent_t handles (torch's events cannot be handed to the C ABI)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return e.value

    def record(self, ev: int, stream: int):
        rc = self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_ms(self, a: int, b: int) -> float:
        self.lib.hipEventSynchronize(ctypes.c_void_p(b))
        f = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(f.value)

    def destroy(self, ev: int):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


def workload(cfg: str, poison: bool, prefix_visible: bool = False, placement: str = "random",
             contiguous_prefix: bool = False):
    """The workload of a configuration; placement "contiguous" lays each prefix
    out as one run of the pool, and contiguous_prefix (which needs it) passes
    the run by its first slot only (TV_FLAG_CONTIGUOUS_PREFIX)."""
    if contiguous_prefix:
        placement = "contiguous"
    w, desc, splits = _workload(cfg, poison, placement)
    if prefix_visible:
        w = W.prefix_visible_form(w)
        desc += "; mask in the prefix-visible form (draft keys only)"
    if placement == "contiguous":
        desc += "; each prefix one contiguous run of the pool"
    if contiguous_prefix:
        w = W.contiguous_prefix_form(w)
        desc += ", passed by its first slot (contiguous-prefix form)"
    return w, desc, splits


def _workload(cfg: str, poison: bool, placement: str = "random"):
    if cfg in W.EXTRA_DESC:
        return W.extra(cfg, poison=poison, placement=placement), W.EXTRA_DESC[cfg], None
    if cfg.startswith("S"):
        k = int(cfg[1:])
        w = W.sweep(k, poison=poison, placement=placement)
        desc = "S%d: 1 request, n_draft=9, prefix %d, H=8 (live shape at long prefix)" % (
            k, W.SWEEP_PREFIX[k])
        return w, desc, None
    k = int(cfg)
    return (W.config(k, poison=poison, placement=placement), W.CONFIG_DESC[k],
            W.CONFIG_SPLITS.get(k))


def flags_for(args):
    import tree_verify_mla_paged_amd as tv
    return ((tv.FLAG_PRECISE_P if args.precise else 0) |
            (tv.FLAG_PREFIX_VISIBLE if args.prefix_visible else 0) |
            (tv.FLAG_CONTIGUOUS_PREFIX if args.contiguous_prefix else 0))


def bench_workload(args, poison=False):
    return workload(args.config, poison=poison, prefix_visible=args.prefix_visible,
                    placement=args.placement, contiguous_prefix=args.contiguous_prefix)


def key_slots(w):
    """Every key's pool slot in key order (the contiguous-prefix form expanded)."""
    if not w.contiguous_prefix:
        return w.kv_indices
    out = w.kv_indices.astype(np.int64).copy()
    for b in range(w.batch):
        k0 = int(w.kv_indptr[b])
        P = int(w.kv_lens[b] - w.q_lens[b])
        out[k0:k0 + P] = out[k0] + np.arange(P)
    return out.astype(np.int32)


def index_entries(w):
    """kv_indices entries the call reads: every key's, or with the
    contiguous-prefix form each request's first prefix entry and its drafts'."""
    if not w.contiguous_prefix:
        return int(w.kv_lens.sum())
    P = w.kv_lens - w.q_lens
    return int(w.q_lens.sum() + (P > 0).sum())


def algorithmic(w):
    """Bytes the call must move and flops it must do (visible pairs only)."""
    H = w.num_heads
    kv_bytes = w.gathered_kv_bytes()
    nq = w.total_q
    total_bytes = (kv_bytes + nq * H * 576 * 2 + nq * H * 512 * 2 + nq * H * 4 +
                   index_entries(w) * 4 + int(w.mask.size))
    flops = 2.0 * (576 + 512) * H * w.visible_pairs()
    return kv_bytes, total_bytes, flops


def code_text(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed: what
    the compiler sees of it (the kernel sources hold no string with // or /*)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def source_hash():
    """The split kernel's code and the parameter structs it is launched with
    (comments and layout excluded)."""
    h = hashlib.sha256()
    for f in ("tv_split.hip", "tv_kernels.h"):
        text = open(os.path.join(ROOT, "tree_verify_mla_paged_amd", "csrc", f)).read()
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def plan_for(args):
    """The library's launch plan for the benchmark configuration."""
    import tree_verify_mla_paged_amd as tv
    w, _, cfg_splits = bench_workload(args)
    splits = args.splits if args.splits >= 0 else (cfg_splits or 0)
    p = tv.make_problem(w.batch, w.num_heads, w.total_q, w.max_q_len, w.max_kv_len, w.num_slots,
                        int(w.kv_indices.size), int(w.mask.size), splits,
                        tv.OUT_F32 if args.out_f32 else tv.OUT_BF16,
                        flags_for(args))
    return launch_shape(tv.plan(p))


def launch_shape(plan: dict) -> dict:
    """The part of a plan that fixes the split kernel's launch and traffic."""
    return {k: plan[k] for k in ("split_keys", "max_splits", "row_blocks")}


def measured_traffic(cfg: str, splits: int, precise: bool, plan: dict):
    """HBM bytes per split-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current split-kernel source with the same
    launch plan; else None."""
    path = os.path.join(ROOT, "profiles", "split_kernel_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    e = d.get("workloads", {}).get("%s/splits=%d/precise=%d" % (cfg, splits, int(precise)))
    if not e or e.get("source_hash") != source_hash() or e.get("plan") != plan:
        return None
    return e.get("bytes_per_launch")


COPY_BYTES = 256 * 1024 * 1024  # the calibration copy of the counter runs


def counter_workload(args):
    """For the two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE): a plain
    elementwise copy of COPY_BYTES (its counter reading calibrates the counter
    to bytes), then `--counter-workload` calls of the benchmark configuration."""
    import torch
    import tree_verify_mla_paged_amd as tv
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    w, _, cfg_splits = bench_workload(args)
    splits = args.splits if args.splits >= 0 else (cfg_splits or 0)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda") for k, v in dict(
        q=w.q.view(np.int16), kv=w.kv.view(np.int16), kv_indices=w.kv_indices,
        kv_indptr=w.kv_indptr, qo_indptr=w.qo_indptr, mask=w.mask,
        mask_indptr=w.mask_indptr).items()}
    p = tv.make_problem(w.batch, w.num_heads, w.total_q, w.max_q_len, w.max_kv_len, w.num_slots,
                        int(w.kv_indices.size), int(w.mask.size), splits,
                        tv.OUT_F32 if args.out_f32 else tv.OUT_BF16,
                        flags_for(args))
    out = torch.empty((w.total_q, w.num_heads, 512),
                      dtype=torch.float32 if args.out_f32 else torch.bfloat16, device="cuda")
    lse = torch.empty((w.total_q, w.num_heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tv.workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    for _ in range(args.counter_workload):
        tv.verify_attn(p, t["q"], t["kv"], t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                       t["mask"], t["mask_indptr"], float(w.sm_scale), out, lse, ws, ws.numel())
    torch.cuda.synchronize()
    print("counter workload: config %s, splits %d, %d calls" % (args.config, splits,
                                                             args.counter_workload))


def write_traffic(args):
    """profiles/split_kernel_hbm_traffic.json from the two counter csv files:
    per split-kernel dispatch, FETCH_SIZE and WRITE_SIZE (KiB) each scaled by
    COPY_BYTES / (the same counter's reading for the calibration copy)."""
    import csv
    fetch_csv, write_csv = args.write_traffic
    res = {}
    for f, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        vals = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        copy = [v for k, v in vals.items() if "elementwise" in k and "MulFunctor" in k]
        split = [v for k, v in vals.items() if "tv_split_kernel" in k]
        if len(copy) != 1 or len(split) != 1:
            raise SystemExit("%s: expected one copy and one split kernel, found %s"
                             % (f, sorted(vals)))
        copy_kib = float(np.mean(copy[0]))
        factor = COPY_BYTES / (copy_kib * 1024.0)
        split_kib = float(np.mean(split[0]))
        res[counter] = {"copy_kernel_kib": copy_kib, "factor": factor,
                        "split_kernel_kib_per_dispatch": split_kib, "dispatches": len(split[0]),
                        "bytes_per_launch": split_kib * 1024.0 * factor}
    path = os.path.join(ROOT, "profiles", "split_kernel_hbm_traffic.json")
    d = json.load(open(path)) if os.path.exists(path) else {}
    d["note"] = ("HBM bytes per tv_split_kernel dispatch: rocprofv3 --pmc FETCH_SIZE and "
                 "WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the same "
                 "counter read %d bytes for a plain copy of that size in the same run "
                 "(bench.py --counter-workload)." % COPY_BYTES)
    splits = args.splits if args.splits >= 0 else (workload(args.config, False)[2] or 0)
    key = "%s/splits=%d/precise=%d" % (args.config, splits, int(args.precise))
    d.setdefault("workloads", {})[key] = {
        "source_hash": source_hash(),
        "plan": plan_for(args),
        "commands": ["rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o fetch -- python3 bench.py "
                     "--config %s --splits %d%s --counter-workload %d" % (
                         args.config, splits, " --precise" if args.precise else "", 10),
                     "the same with --pmc WRITE_SIZE -o write",
                     "python3 bench.py --config %s --splits %d%s --write-traffic "
                     "<dir>/fetch_counter_collection.csv <dir>/write_counter_collection.csv" % (
                         args.config, splits, " --precise" if args.precise else "")],
        "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
        "bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] +
        res["WRITE_SIZE"]["bytes_per_launch"]}
    json.dump(d, open(path, "w"), indent=1)
    print(json.dumps(d["workloads"][key], indent=1))


def append_times(w, steps, prefix_visible):
    """tv_append_draft (draft rows into the pool, key lists, indptrs, tree mask)
    on the workload's pieces, timed back to back; algorithmic bytes: the draft
    rows read and written, the slot lists read, kv_indices and the mask
    written, the parents read."""
    import torch
    import tree_verify_mla_paged_amd as tv
    x = W.marshal_inputs(w)

    def dev(a, dt):
        a = np.ascontiguousarray(a, dtype=dt)
        a = a if a.size else np.zeros(1, dt)
        return torch.from_numpy(a.view(np.int16) if dt == np.uint16 else a).to("cuda")

    t = {k: dev(x[k], np.uint16 if k in ("kv_buf", "draft_kv") else np.int32)
         for k in ("kv_buf", "draft_kv", "out_cache_loc", "prefix_indices", "prefix_indptr",
                   "qo_indptr", "parents")}
    n, L = w.q_lens, w.kv_lens
    nmask = int((n * (n if prefix_visible else L)).sum())
    ki = torch.empty(int(L.sum()) + 1, dtype=torch.int32, device="cuda")
    kp = torch.empty(w.batch + 1, dtype=torch.int32, device="cuda")
    m = torch.empty(nmask + 1, dtype=torch.uint8, device="cuda")
    mp = torch.empty(w.batch + 1, dtype=torch.int32, device="cuda")
    p = tv.make_append_problem(w.batch, w.max_q_len, w.max_kv_len, w.total_q, w.num_slots,
                               int(x["prefix_indices"].size), int(L.sum()), nmask,
                               tv.FLAG_PREFIX_VISIBLE if prefix_visible else 0)

    def call():
        tv.append_draft(p, t["draft_kv"], t["out_cache_loc"], t["prefix_indices"],
                        t["prefix_indptr"], t["qo_indptr"], t["parents"], t["kv_buf"], ki, kp,
                        m, mp)
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / steps
    N = int(w.total_q)
    nbytes = 2 * N * 1152 + N * 4 + int((L - n).sum()) * 4 + int(L.sum()) * 4 + nmask + N * 4
    return {"us_per_call": us, "bytes": nbytes, "GB/s": nbytes / us / 1e3,
            "mask_form": "prefix-visible" if prefix_visible else "full"}


def calibration():
    """Achievable peaks on this GPU, for context beside the published ones: a
    1 GiB device-to-device copy (HBM read + write), a 1 GiB sum (read), and an
    8192^3 bf16 matrix product, all torch library code (not this path), each
    the median of 10."""
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda").contiguous()
    bm = torch.randn((n, n), dtype=torch.bfloat16, device="cuda").contiguous()
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")

    def med(fn, reps=10):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t_copy = med(lambda: dst.copy_(src))
    red = torch.empty((), dtype=torch.float32, device="cuda")
    src_f = src.view(torch.float32)
    t_read = med(lambda: torch.sum(src_f, dim=0, out=red))
    t_mm = med(lambda: torch.mm(a, bm, out=c))
    res = {"copy_GBs": 2 * nbytes / t_copy / 1e9, "read_GBs": nbytes / t_read / 1e9,
           "bf16_mm_TFLOPs": 2.0 * n ** 3 / t_mm / 1e12,
           "how": "median of 10: 1 GiB device copy (read + write bytes); torch.sum over "
                  "1 GiB of fp32 (read); torch.mm bf16 8192^3"}
    del src, dst, a, bm, c, red, src_f
    torch.cuda.synchronize()
    return res


def gather_calibration(kv, kv_indices, reps=10):
    """The same random 1152-byte pool rows gathered by library code
    (torch.index_select into a dense copy), warm and after a cache scrub: what
    plain row gathers reach on this GPU for this workload's slot pattern.
    Rates count the gathered bytes read (the copy also writes as many)."""
    import torch
    idx = kv_indices.long()
    out = torch.empty((idx.numel(), kv.shape[1]), dtype=kv.dtype, device="cuda")
    scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda")
    nbytes = idx.numel() * kv.shape[1] * kv.element_size()

    def timed(cold):
        ts = []
        for i in range(reps + 2):
            if cold:
                scrub.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.index_select(kv, 0, idx, out=out)
            e1.record()
            e1.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    tw, tc = timed(False), timed(True)
    del out, scrub
    torch.cuda.synchronize()
    return {"bytes_read": nbytes, "warm_us": tw * 1e6, "warm_read_GBs": nbytes / tw / 1e9,
            "cold_us": tc * 1e6, "cold_read_GBs": nbytes / tc / 1e9,
            "how": "torch.index_select of the workload's kv_indices rows, median of %d" % reps}


SCRUB_BYTES = 1 << 30  # larger than the 256 MB MALL plus every XCD's L2


def warm_times(call, ev, stream, n):
    """Secondary figure: n calls back to back on one stream (caches warm: the
    pool partly stays in the MALL between calls), wall clock over the n calls;
    every WARM_STRIDE-th call's split kernel stamps an event pair (event
    handling adds a few microseconds to a call, so the others carry none)."""
    import torch
    pairs = [(ev.create(), ev.create()) for _ in range(0, n, WARM_STRIDE)]
    with torch.cuda.stream(stream):
        for _ in range(5):
            call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(n):
            call(pairs[i // WARM_STRIDE] if i % WARM_STRIDE == 0 else None)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / n
    split = [ev.elapsed_ms(a, b) * 1e3 for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    return {"calls": n, "us_per_call": us, "split_kernel_avg_us": float(np.mean(split)),
            "split_kernel_timed_launches": len(split)}


def clean_cold_times(call, ev, stream, n):
    """Secondary figure: caches cold but clean.  Before each call a reduction
    reads a 1 GiB buffer that was written once, before any of these calls (the
    timed steps' scrub writes instead: the dirty lines it leaves in the MALL
    are written back while the call reads, which for a call that mostly reads
    adds about as much HBM traffic as the call's own).  Even calls are
    bracketed by events on the stream, odd calls carry the split kernel's own
    event pair, as in the timed steps."""
    import torch
    rbuf = torch.ones(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda")
    n_call = (n + 1) // 2
    pairs = [(ev.create(), ev.create()) for _ in range(n // 2)]
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_call)]
    with torch.cuda.stream(stream):
        rbuf.sum()  # its own fill's dirty lines leave the MALL here
        for _ in range(3):
            rbuf.sum()
            call()
        for i in range(n):
            rbuf.sum()
            if i % 2 == 0:
                calls[i // 2][0].record(stream)
                call()
                calls[i // 2][1].record(stream)
            else:
                call(pairs[i // 2])
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in calls]
    split = [ev.elapsed_ms(a, b) * 1e3 for a, b in pairs] or [float("nan")]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    del rbuf
    return {"calls_bracketed": len(us), "us_per_call": float(np.median(us)),
            "split_kernel_avg_us": float(np.mean(split)), "split_kernel_timed_launches": len(pairs)}


def graph_times(call, stream, n):
    """The call captured into a HIP graph: wall clock over n replays back to
    back, and 50 replays each bracketed by events outside the graph."""
    import torch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    for _ in range(5):
        graph.replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for _ in range(n):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - g0) * 1e6 / n
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(50)]
    with torch.cuda.stream(stream):
        for e0, e1 in gev:
            e0.record(stream)
            graph.replay()
            e1.record(stream)
    torch.cuda.synchronize()
    gus = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in gev])
    del graph
    return graph_us, {"replays": len(gev), "median_us": float(np.median(gus)),
                      "p10_us": float(np.percentile(gus, 10)),
                      "p90_us": float(np.percentile(gus, 90))}


def cpu_baseline(w, gpu_out, gpu_lse, kv_bytes, budget_s, out_f32):
    """Time the fp64 oracle on a bounded sample of rows and scale to the call."""
    import oracle
    H = w.num_heads
    total_rows = w.total_q * H
    threads = os.cpu_count() or 1
    rng = np.random.default_rng(123)
    order = rng.permutation(total_rows)
    # probe a few rows to size the sample for the time budget
    probe = np.sort(order[:min(total_rows, max(4, threads))])
    t0 = time.perf_counter()
    oracle.run(w, rows=probe, threads=threads)
    t_probe = time.perf_counter() - t0
    per_row = t_probe / len(probe)
    n = int(min(total_rows, max(len(probe), budget_s / max(per_row, 1e-9))))
    rows = np.sort(order[:n])
    t0 = time.perf_counter()
    ro, rl = oracle.run(w, rows=rows, threads=threads)
    t = time.perf_counter() - t0
    # the sampled rows see this share of the call's (row, key) pairs
    lens = np.repeat(w.kv_lens, w.q_lens * H).astype(np.float64)
    share = lens[rows].sum() / max(lens.sum(), 1.0)
    t_call = t / max(share, 1e-12)
    go = gpu_out.reshape(-1, 512)[rows]
    gl = gpu_lse.reshape(-1)[rows]
    d = np.abs(go - ro)
    fin = np.isfinite(rl)
    parity = {
        "rows": int(n), "max_abs_diff": float(d.max()),
        "mean_rel_err": float(d.sum() / max(np.abs(ro).sum(), 1e-300)),
        "max_lse_diff": float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0,
        "out_dtype": "f32" if out_f32 else "bf16",
    }
    res = {
        "value": kv_bytes / t_call / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "%d of %d rows (%.1f%% of row-key pairs), fp64 C/OpenMP, %.2f s measured, "
                  "%.2f s per full call" % (n, total_rows, 100 * share, t, t_call),
        "us_per_call": t_call * 1e6, "parity_vs_gpu": parity,
    }
    if n == total_rows and t_call * threads < 1.0:
        # a small call: also on one thread, median of 3 whole calls
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.run(w, threads=1)
            ts.append(time.perf_counter() - t0)
        res["one_thread_us_per_call"] = float(np.median(ts)) * 1e6
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="3",
                    help="1-5 (benchmark configurations), S1-S3 (long-prefix sweep), "
                         "D (plain decode) or K (chain verify)")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measured copy bandwidth and bf16 matrix-product peak")
    ap.add_argument("--append", action="store_true",
                    help="also time tv_append_draft (the marshaling step) on the same workload")
    ap.add_argument("--prefix-visible", action="store_true",
                    help="pass the mask in the prefix-visible form (draft keys only)")
    ap.add_argument("--splits", type=int, default=0,
                    help="KV split count (0 = the library's plan; -1 = the configuration's own "
                         "split count if it names one)")
    ap.add_argument("--placement", choices=("random", "contiguous"), default="random",
                    help="pool placement of the keys: random single slots (the configurations') "
                         "or each prefix one contiguous run")
    ap.add_argument("--contiguous-prefix", action="store_true",
                    help="contiguous placement, passed in the contiguous-prefix form (each prefix "
                         "by its first slot only)")
    ap.add_argument("--out-f32", action="store_true")
    ap.add_argument("--precise", action="store_true",
                    help="probabilities as a bf16 hi + lo pair in the P.V product")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timed-only", action="store_true",
                    help="only the warm-up and timed (cold-cache) steps, no warm, graph or "
                         "calibration runs: the command of the committed kernel traces")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--counter-workload", type=int, default=0, metavar="N",
                    help="run the calibration copy and N calls for rocprofv3 --pmc, no timing")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise the two counter runs into profiles/ (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU and has no multi-GPU path (requests and heads would "
              "shard across GPUs with no exchange between them).  Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.counter_workload > 0:
        counter_workload(args)
        return

    import torch
    import tree_verify_mla_paged_amd as tv

    w, desc, cfg_splits = bench_workload(args)
    splits = args.splits if args.splits >= 0 else (cfg_splits or 0)
    dev = "cuda"
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in dict(
        q=w.q.view(np.int16), kv=w.kv.view(np.int16), kv_indices=w.kv_indices,
        kv_indptr=w.kv_indptr, qo_indptr=w.qo_indptr, mask=w.mask,
        mask_indptr=w.mask_indptr).items()}
    p = tv.make_problem(w.batch, w.num_heads, w.total_q, w.max_q_len, w.max_kv_len, w.num_slots,
                        int(w.kv_indices.size), int(w.mask.size), splits,
                        tv.OUT_F32 if args.out_f32 else tv.OUT_BF16,
                        flags_for(args))
    plan = tv.plan(p)
    N, H = w.total_q, w.num_heads
    out = torch.empty((N, H, 512), dtype=torch.float32 if args.out_f32 else torch.bfloat16,
                      device=dev)
    lse = torch.empty((N, H), dtype=torch.float32, device=dev)
    nb = tv.workspace_bytes(p)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    sid = int(stream.cuda_stream)
    ev = HipEvents()

    def call(pair=None):
        if pair is None:
            tv.verify_attn(p, t["q"], t["kv"], t["kv_indices"], t["kv_indptr"], t["qo_indptr"],
                           t["mask"], t["mask_indptr"], float(w.sm_scale), out, lse, ws,
                           ws.numel(), stream=sid)
        else:
            tv.verify_attn_timed(p, t["q"], t["kv"], t["kv_indices"], t["kv_indptr"],
                                 t["qo_indptr"], t["mask"], t["mask_indptr"], float(w.sm_scale),
                                 out, lse, ws, ws.numel(), pair[0], pair[1], stream=sid)

    # The timed steps: inputs resident in HBM, caches cold.  Before each step a
    # 1 GiB fill kernel (outside the events, same stream) evicts the pool, the
    # indices and the mask from the 256 MB MALL and the L2s.  Even steps are
    # bracketed by events on the stream (the call time); odd steps carry
    # instead the event pair that the split kernel's own dispatch stamps (the
    # kernel time).  Each kind of event handling adds its own delay, so no step
    # carries both.  The warm-up steps are the same, untimed.
    scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=dev)
    n_call = (args.steps + 1) // 2
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps // 2)]
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_call)]
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            scrub.fill_(i & 0xFF)
            call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            scrub.fill_((i + 1) & 0xFF)
            if i % 2 == 0:
                calls[i // 2][0].record(stream)
                call()
                calls[i // 2][1].record(stream)
            else:
                call(pairs[i // 2])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in calls])
    split_ms = [ev.elapsed_ms(a, b) for a, b in pairs] or [float("nan")]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    del scrub
    split_avg_ms = float(np.mean(split_ms))
    ms_per_step = float(np.median(call_us)) * 1e-3
    timed_region_s = t1 - t0

    warm = clean = None
    graph_us = graph_events = None
    if not args.timed_only:
        warm = warm_times(call, ev, stream, max(args.steps, 50))
        clean = clean_cold_times(call, ev, stream, max(args.steps, 20))
        graph_us, graph_events = graph_times(call, stream, max(args.steps, 50))

    append = append_times(w, args.steps, args.prefix_visible) if args.append else None
    calib = calibration() if not (args.no_calibration or args.timed_only) else None
    if calib:
        calib["index_select_gather"] = gather_calibration(
            t["kv"], torch.from_numpy(key_slots(w)).to(dev))

    kv_bytes, total_bytes, flops = algorithmic(w)
    us_per_call = ms_per_step * 1e3
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    t_hbm = total_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        achieved = flops / (split_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
    else:
        achieved = total_bytes / (split_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    # the counter summary covers the full mask form and random placement only
    roof["traffic"] = (None if (args.prefix_visible or args.placement != "random" or
                                args.contiguous_prefix) else
                       measured_traffic(args.config, splits, bool(args.precise),
                                        launch_shape(plan)))
    roof["kernel"] = "tv_split_kernel"
    roof["kernel_avg_us"] = split_avg_ms * 1e3
    roof["kernel_timed_launches"] = len(pairs)
    roof["timing"] = ("cold cache: the split kernel of every odd timed step, stamped by its own "
                      "dispatch")
    if warm:
        # the same kernel with warm caches (back to back), for comparison
        w_ach = (flops if roof["bound"] == "mfma" else total_bytes) / (
            warm["split_kernel_avg_us"] * 1e-6) / (1e12 if roof["bound"] == "mfma" else 1e9)
        roof["warm"] = {"kernel_avg_us": warm["split_kernel_avg_us"], "achieved": w_ach,
                        "frac": w_ach / roof["peak"]}
    if clean:
        # and cold caches holding no dirty lines (see clean_cold_times)
        c_ach = (flops if roof["bound"] == "mfma" else total_bytes) / (
            clean["split_kernel_avg_us"] * 1e-6) / (1e12 if roof["bound"] == "mfma" else 1e9)
        roof["clean_cold"] = {"kernel_avg_us": clean["split_kernel_avg_us"], "achieved": c_ach,
                              "frac": c_ach / roof["peak"]}
    roof["algorithmic"] = {"bytes": total_bytes, "flops": flops,
                           "floor_us": max(t_hbm, t_mfma) * 1e6}
    if calib:
        # the same achieved rate against what this GPU reached on library code
        roof["frac_of_measured_peak"] = achieved / (
            calib["bf16_mm_TFLOPs"] if roof["bound"] == "mfma" else calib["copy_GBs"])

    res = {
        "metric": "verify-attn µs/call + gathered-KV GB/s (% of MI355X HBM peak) at 32k prefix",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, bf16-rounded N(0,1))",
        "us_per_call": us_per_call, "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "timing": ("value, ms_per_step and us_per_call: median over the even timed steps of "
                   "the event-bracketed call, each step after a %d-byte cache scrub (cold MALL "
                   "and L2); warm: back-to-back calls; clean_cold: each call after a read "
                   "of a 1 GiB buffer instead of the fill" % SCRUB_BYTES),
        "timed_steps": {"calls_bracketed": len(calls), "median_us": float(np.median(call_us)),
                        "p10_us": float(np.percentile(call_us, 10)),
                        "p90_us": float(np.percentile(call_us, 90)),
                        "mean_us": float(np.mean(call_us)),
                        "wall_s": timed_region_s},
        "warm": warm,
        "warm_GBs": (kv_bytes / (warm["us_per_call"] * 1e-6) / 1e9) if warm else None,
        "clean_cold": clean,
        "graph_us_per_call": graph_us,
        "graph_replay_events": graph_events,
        "append_draft": append,
        "calibration": calib,
        "floor_fraction": max(t_hbm, t_mfma) / (ms_per_step * 1e-3),
        "config": {"workload": desc, "requests": w.batch, "n_draft": int(w.max_q_len),
                   "max_kv_len": int(w.max_kv_len), "heads": H, "num_splits_arg": splits,
                   "plan": plan, "out_dtype": "f32" if args.out_f32 else "bf16",
                   "precise_p": bool(args.precise), "prefix_visible": bool(args.prefix_visible),
                   "placement": "contiguous" if args.contiguous_prefix else args.placement,
                   "contiguous_prefix": bool(args.contiguous_prefix),
                   "gathered_kv_bytes": kv_bytes, "visible_pairs_x_heads": w.visible_pairs() * H},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        o = out.float().cpu().numpy().astype(np.float64)
        l = lse.cpu().numpy().astype(np.float64)
        res["cpu_baseline"] = cpu_baseline(w, o, l, kv_bytes, args.cpu_budget_s, args.out_f32)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
