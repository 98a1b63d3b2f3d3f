#!/usr/bin/env python3
"""Benchmark of the variable-length attention forward on one MI355X.

A step is one call of the forward (work-partition pre-pass + attention
kernels) over one batch of seeded synthetic input already resident in HBM,
through the C ABI's out variant with preallocated out / lse / workspace.

Main workload: bf16 causal GQA prefill, 16 sequences with lengths drawn
uniformly from [128, 4096] (seed 1002, 33,781 tokens), 32 query heads,
8 kv heads, head_dim 128, scale 1/sqrt(128).  The value is mask-adjusted
TFLOP/s: 4 * head_dim FLOPs per unmasked (query, key) pair per head.

Also reported (same JSON line, key "also"): the full-attention Ulysses-shard
shape, the sliding-window + sinks MQA shape (bound by HBM) and the paged
decode shape (bound by HBM), each with its own step time and roofline;
(key "backward") one call of the backward on the main workload; and (key
"merge") the log-sum-exp merge of 8 float32 partials of the full-attention
shard (a ring of 8), bound by HBM; and (keys "sparse", "sparse_d512")
sliding-window + sparse compressed attention over shared K/V at head sizes
128 and 512.

Timing: the K timed steps of a workload run as one captured HIP graph of K
back-to-back calls (so host gaps between calls do not count), bracketed by
HIP events on the stream the kernels run on; the same K steps called
eagerly from Python are reported beside it.  The roofline figure is for the
dominant kernel: its average duration is the graph-timed call minus the
graph-timed pre-pass (the call-level fraction is reported too).
cpu_baseline times the fp64 oracle on this host: per workload, all rows
(configs 1, 4, 5) or a bounded sample of rows (configs 2, 3).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

# Kernel source files whose hash keys the committed HBM-traffic measurements
# (profiles/traffic.json): a measurement counts only for the exact sources
# it was taken with.
KERNEL_SOURCES = {
    "prefill_bf16": ["va_prefill_bf16.hip", "va_device.h", "va_plan.hip"],  # the item order sets L2 reuse
    "decode_bf16": ["va_decode.hip"],
    "f32": ["va_prefill_f32.hip"],
    "window_bf16": ["va_window.hip"],
    "sparse": ["va_sparse.hip"],
    "prefill512": ["va_prefill512.hip", "va_plan.hip"],
}
PATH_NAMES = ["prefill_bf16", "decode_bf16", "f32", "window_bf16", "prefill512"]  # index = varlen_attn_path


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work counts
def visible_pairs(case) -> np.ndarray:
    """Unmasked (query, key) pairs per query row (same for every head)."""
    INF = 1 << 40
    left = case["window_left"] if case["window_left"] >= 0 else INF
    right = 0 if case["causal"] else (case["window_right"] if case["window_right"] >= 0 else INF)
    lens_q = np.diff(case["cu_q"]).astype(np.int64)
    lens_k = (case["seqused_k"] if case["paged"] else np.diff(case["cu_k"])).astype(np.int64)
    out = np.zeros(case["T_q"], np.int64)
    for b in range(case["B"]):
        s = int(case["cu_q"][b])
        i = np.arange(lens_q[b], dtype=np.int64)
        p = i + lens_k[b] - lens_q[b]
        lo = np.maximum(0, p - left)
        hi = np.minimum(lens_k[b] - 1, p + right)
        out[s:s + lens_q[b]] = np.maximum(0, hi - lo + 1)
    return out


def flops(case) -> float:
    return float(4 * case["D"] * case["H"] * visible_pairs(case).sum())


def alg_bytes(case) -> float:
    es = 4 if case["dtype"] == "f32" else 2
    H, Hkv, D = case["H"], case["Hkv"], case["D"]
    qo = 2.0 * case["T_q"] * H * D * es
    lse = 4.0 * case["T_q"] * H
    if case["paged"]:
        kv_rows = float(np.sum(case["seqused_k"]))
        meta = 4.0 * (case["B"] + 1) + 4.0 * case["B"] + 4.0 * sum(
            (int(x) + case["block_size"] - 1) // case["block_size"] for x in case["seqused_k"])
    else:
        kv_rows = float(case["T_k"])
        meta = 8.0 * (case["B"] + 1)
    return qo + lse + 2.0 * kv_rows * Hkv * D * es + meta


# ---------------------------------------------------------------- GPU timing
def _dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def timed_eager(fn, n, w, torch):
    """ms per call of fn called n times from Python after w warm-up calls."""
    for _ in range(w):
        fn()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def timed_graph(fn, n, w, torch):
    """ms per call of n back-to-back calls of fn captured in one HIP graph
    (after w eager warm-up calls and one warm-up replay), timed by HIP
    events around one replay on the current stream.  Falls back to eager
    timing if capture is not available."""
    for _ in range(w):
        fn()
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
    except Exception as exc:  # pragma: no cover - depends on the runtime
        log(f"graph capture unavailable ({exc}); timing eagerly")
        return timed_eager(fn, n, 0, torch)
    e0, e1 = _events(torch)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_case(case, steps, warmup, torch):
    import variable_length_attention_amd as va
    q = _dev(case["q"], torch)
    cu_q = _dev(case["cu_q"], torch)
    sinks = _dev(case.get("sinks"), torch)
    win = (case["window_left"], case["window_right"])
    out = torch.empty_like(q)
    lse = torch.empty((case["T_q"], case["H"]), dtype=torch.float32, device="cuda")
    if case["paged"]:
        kc, vc = _dev(case["k_cache"], torch), _dev(case["v_cache"], torch)
        bt, su = _dev(case["block_table"], torch), _dev(case["seqused_k"], torch)
        prob = va.make_problem(q, kc.shape[2], 0, case["B"], case["max_q"], case["max_k"], case["scale"],
                               case["causal"], win, kc.shape[0], kc.shape[1], bt.shape[1])
        ws = torch.empty(va.workspace_size(prob, True), dtype=torch.uint8, device="cuda")

        def step():
            va.varlen_attn_paged(q, kc, vc, bt, cu_q, su, case["max_q"], case["max_k"],
                                 scale=case["scale"], causal=case["causal"], window=win, sinks=sinks,
                                 out=out, lse=lse, workspace=ws)
        seqlens = su
    else:
        k, v, cu_k = _dev(case["k"], torch), _dev(case["v"], torch), _dev(case["cu_k"], torch)
        prob = va.make_problem(q, k.shape[1], k.shape[0], case["B"], case["max_q"], case["max_k"],
                               case["scale"], case["causal"], win)
        ws = torch.empty(va.workspace_size(prob, False), dtype=torch.uint8, device="cuda")

        def step():
            va.varlen_attn_out(out, q, k, v, cu_q, cu_k, case["max_q"], case["max_k"], scale=case["scale"],
                               causal=case["causal"], window=win, sinks=sinks, lse=lse, workspace=ws)
        seqlens = cu_k
    path = va.kernel_path(prob, case["paged"])

    # pre-pass alone, through the plan entry point (count only)
    import ctypes
    from variable_length_attention_amd import _lib
    lib = _lib.load()

    def plan_step():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        _lib.check(lib.varlen_attn_plan(ctypes.byref(prob), 1 if case["paged"] else 0,
                                        ctypes.c_void_p(cu_q.data_ptr()), ctypes.c_void_p(seqlens.data_ptr()),
                                        None, 0, None,
                                        ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), stream))

    ms_eager = timed_eager(step, steps, warmup, torch)
    ms_step = timed_graph(step, steps, 1, torch)
    # the pre-pass alone (a few microseconds), the same way
    ms_plan = timed_graph(plan_step, max(steps, 20), 1, torch)
    return ms_step, ms_plan, path, ms_eager


def time_backward(case, steps, warmup, torch):
    """One call of the backward (pre-passes, dO.O row sums, dQ kernel, dK/dV
    kernel) on the workload, with out / lse from the forward and a seeded
    dO, all resident in HBM; returns ms per call."""
    import variable_length_attention_amd as va
    q, k, v = _dev(case["q"], torch), _dev(case["k"], torch), _dev(case["v"], torch)
    cu_q, cu_k = _dev(case["cu_q"], torch), _dev(case["cu_k"], torch)
    sinks = _dev(case.get("sinks"), torch)
    win = (case["window_left"], case["window_right"])
    out = torch.empty_like(q)
    lse = torch.empty((case["T_q"], case["H"]), dtype=torch.float32, device="cuda")
    va.varlen_attn_out(out, q, k, v, cu_q, cu_k, case["max_q"], case["max_k"], scale=case["scale"],
                       causal=case["causal"], window=win, sinks=sinks, lse=lse)
    g = torch.Generator().manual_seed(case["spec"].seed + 7)
    dout = torch.randn(tuple(q.shape), generator=g).to(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = va.make_problem(q, k.shape[1], k.shape[0], case["B"], case["max_q"], case["max_k"], case["scale"],
                           case["causal"], win)
    ws = torch.empty(va.bwd_workspace_size(prob), dtype=torch.uint8, device="cuda")

    def step():
        va.varlen_attn_bwd(dout, q, k, v, out, lse, cu_q, cu_k, case["max_q"], case["max_k"],
                           scale=case["scale"], causal=case["causal"], window=win, dq=dq, dk=dk, dv=dv,
                           workspace=ws)
    return timed_graph(step, steps, warmup, torch)


MERGE_SHAPE = dict(n=8, rows=32768, H=24, D=128)  # ring of 8 over the full-attention shard


def time_merge(steps, warmup, torch):
    """The log-sum-exp merge of 8 float32 partials (a ring of 8 ranks over
    the 32768-token, 24-head, d128 full-attention shard) into bf16 out +
    float32 lse; returns (ms per call, algorithmic bytes)."""
    import variable_length_attention_amd as va
    import workloads as W
    m = W.merge_inputs(MERGE_SHAPE["n"], MERGE_SHAPE["rows"], MERGE_SHAPE["H"], MERGE_SHAPE["D"], "f32", seed=2024)
    o_parts, lse_parts = _dev(m["o_parts"], torch), _dev(m["lse_parts"], torch)
    del m
    n, rows, H, D = (MERGE_SHAPE[k] for k in ("n", "rows", "H", "D"))
    out = torch.empty((rows, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, H), dtype=torch.float32, device="cuda")

    def step():
        va.varlen_attn_merge(o_parts, lse_parts, out=out, lse=lse)
    ms = timed_graph(step, steps, warmup, torch)
    nbytes = float(n * rows * H * (D * 4 + 4) + rows * H * (D * 2 + 4))
    return ms, nbytes


# third scenario: 512 distinct indices per sequence drawn, as the README
# example draws them, from the compressed keys every row of it sees
SPARSE_SHAPE = dict(lens_q=[1024] * 4, seqused_kv=[8192] * 4, H=64, Hkv=1, D=128, window=(127, 0), topk=512,
                    cmp_ratio=4, ori_bs=128, cmp_bs=128, seed=4600, visible_indices=True)
# the same at the Ascend operator's own head size
SPARSE_SHAPE_D512 = dict(SPARSE_SHAPE, D=512, seed=4601)
# second scenario at that head size: every compressed key the causal
# compressed mask admits (1025 to 2048 per row) plus the window
SPARSE_SHAPE_ALL_D512 = dict(SPARSE_SHAPE, D=512, topk=0, cmp_all=True, visible_indices=False, seed=4602)


def sparse_work(sc):
    """(FLOPs, algorithmic bytes) of sliding-window + compressed attention:
    4 * D FLOPs per (token, head, attended key); bytes = q, out, lse, the
    indices, block tables and each sequence's distinct original rows in some
    window and distinct attended compressed rows (read once).  Row i of a
    sequence sees compressed positions up to i + S3 - Lq."""
    cu = sc["cu_q"]
    left, right = sc["window"]
    g = sc["H"] // sc["Hkv"]
    keys, rows = 0, 0
    for b in range(sc["B"]):
        S2, Lq = int(sc["seqused_kv"][b]), int(cu[b + 1] - cu[b])
        if Lq == 0:
            continue
        S3 = S2 // sc["cmp_ratio"]
        p = np.arange(Lq) + S2 - Lq
        lo, hi = np.maximum(0, p - left), np.minimum(S2 - 1, p + right)
        nwin = np.maximum(0, hi - lo + 1)
        last = np.arange(Lq) + S3 - Lq
        seen = np.zeros(S2, bool)
        for a_, z in zip(lo, hi):
            if z >= a_:
                seen[a_:z + 1] = True
        rows += int(seen.sum()) * sc["Hkv"]
        keys += int(nwin.sum()) * sc["Hkv"]
        if sc.get("cmp_all"):
            ncmp = np.clip(last + 1, 0, S3)
            keys += int(ncmp.sum()) * sc["Hkv"]
            rows += int(ncmp.max()) * sc["Hkv"]
            continue
        idx = sc["indices"][cu[b]:cu[b + 1]] if sc["topk"] else np.zeros((Lq, sc["Hkv"], 0), np.int32)
        ok = (idx >= 0) & (idx <= last[:, None, None])
        keys += int(ok.sum())
        rows += sum(len(np.unique(idx[:, c][ok[:, c]])) for c in range(sc["Hkv"]))
    D, es = sc["D"], 2
    fl = 4.0 * D * g * keys
    by = (2.0 * sc["T"] * sc["H"] * D * es + 4.0 * sc["T"] * sc["H"] + 4.0 * sc["indices"].size
          + 4.0 * (sc["ori_table"].size + sc["cmp_table"].size) + rows * D * es)
    return fl, by


def time_sparse(steps, warmup, torch, shape=SPARSE_SHAPE):
    """Sliding-window + sparse compressed attention over shared K/V on
    shape; returns (ms per call, FLOPs, algorithmic bytes)."""
    import variable_length_attention_amd as va
    import workloads as W
    sc = W.sparse_case(**shape)
    args = [_dev(sc[k], torch) if sc["topk"] or k != "indices" else None
            for k in ("q", "ori_kv", "ori_table", "seqused_kv", "cmp_kv", "cmp_table", "indices", "cu_q")]
    sinks = _dev(sc["sinks"], torch)
    out = torch.empty_like(args[0])
    lse = torch.empty((sc["T"], sc["H"]), dtype=torch.float32, device="cuda")

    def step():
        va.varlen_attn_sparse_sharedkv(*args, sc["max_seqlen_kv"], scale=sc["scale"], window=sc["window"],
                                       cmp_ratio=sc["cmp_ratio"], cmp_attend_all=sc["cmp_all"], sinks=sinks, out=out,
                                       lse=lse)
    ms = timed_graph(step, steps, warmup, torch)
    fl, by = sparse_work(sc)
    return ms, fl, by


# ---------------------------------------------------------------- HBM traffic
def kernel_source_sha(path_name):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path_name]:
        with open(os.path.join(ROOT, "variable_length_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path_name, workload):
    """HBM bytes per launch of the dominant kernel from the committed
    counter runs, or None when there is none for the current sources."""
    fn = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as fh:
        rec = json.load(fh).get(f"{path_name}/{workload}")
    if not rec or rec.get("source_sha256") != kernel_source_sha(path_name):
        return None
    return rec["hbm_bytes_per_launch"]


def _profile_rows(csv_path, kernel_regex):
    import csv
    import re
    rx = re.compile(kernel_regex)
    with open(csv_path, newline="") as fh:
        for r in csv.DictReader(fh):
            if rx.search(r["Kernel_Name"]):
                yield r


def counter_means(csv_path, kernel_regex):
    """{counter: (mean per dispatch, dispatches)} over the dispatches of the
    kernels matching kernel_regex in a rocprofv3 counter_collection CSV."""
    per = {}
    for r in _profile_rows(csv_path, kernel_regex):
        d = per.setdefault(r["Counter_Name"], {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {c: (sum(v.values()) / len(v), len(v)) for c, v in per.items()}


def trace_summary(path, kernel_regex=".", last=20):
    """Per kernel (name, grid): dispatches and average / min / max duration
    in microseconds from a rocprofv3 kernel trace (its CSV, or the SQLite
    results database it writes by default), and the average over the last
    `last` dispatches (the timed graph replay of a benchmark step)."""
    import re
    rx = re.compile(kernel_regex)
    out = {}
    if path.endswith(".db"):
        import sqlite3
        con = sqlite3.connect(path)
        rows = con.execute("select name, grid_x, start, end from kernels order by start").fetchall()
        con.close()
        for name, grid, t0, t1 in rows:
            if rx.search(name):
                out.setdefault((name, int(grid)), []).append((t1 - t0) / 1e3)
    else:
        rows = sorted(_profile_rows(path, kernel_regex), key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            key = (r["Kernel_Name"], int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0))
            out.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: {"n": len(v), "avg_us": sum(v) / len(v), "min_us": min(v), "max_us": max(v),
                "last_avg_us": sum(v[-last:]) / len(v[-last:])} for k, v in out.items()}


def record_traffic(key, kernel_regex, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                   copy_bytes=1 << 30):
    """Stores in profiles/traffic.json the HBM bytes per launch of the
    kernels matching kernel_regex, from FETCH_SIZE and WRITE_SIZE runs
    (KiB per dispatch), each scaled by what the same counter reads for a
    plain device copy of copy_bytes (which reads and writes copy_bytes);
    keyed by the hash of the kernel's own sources (key = path/workload)."""
    path_name = key.split("/")[0]
    f = counter_means(fetch_csv, kernel_regex)["FETCH_SIZE"]
    w = counter_means(write_csv, kernel_regex)["WRITE_SIZE"]
    cf = counter_means(copy_fetch_csv, "copyBuffer")["FETCH_SIZE"][0]
    cw = counter_means(copy_write_csv, "copyBuffer")["WRITE_SIZE"][0]
    fs, ws = copy_bytes / 1024.0 / cf, copy_bytes / 1024.0 / cw
    rec = {"source_sha256": kernel_source_sha(path_name), "kernel_regex": kernel_regex,
           "fetch_kib_raw": f[0], "write_kib_raw": w[0], "fetch_scale": fs, "write_scale": ws,
           "fetch_bytes_per_launch": f[0] * fs * 1024.0, "write_bytes_per_launch": w[0] * ws * 1024.0,
           "dispatches": [f[1], w[1]]}
    rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    fn = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(fn):
        with open(fn) as fh:
            data = json.load(fh)
    data[key] = rec
    with open(fn, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return rec


def calibrate_copy(nbytes, reps):
    """A plain device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (each copy reads and writes nbytes)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def calibrate_attainable(steps):
    """Attainable references on this GPU, for context beside the datasheet
    peaks: a large bf16 GEMM through PyTorch (hipBLASLt) and a large
    read-only reduction (HBM read bandwidth)."""
    import torch
    torch.manual_seed(0)
    res = {}
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res["gemm_bf16_8192_tflops"] = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b
    x = torch.randn(4 * 1024 ** 3 // 2, device="cuda", dtype=torch.bfloat16)  # 4 GiB
    for _ in range(2):
        x.sum(dtype=torch.float32)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        x.sum(dtype=torch.float32)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res["read_4GiB_GBs"] = x.numel() * 2 / (ms * 1e-3) / 1e9
    print(json.dumps(res), flush=True)


def calibrate_mfma(iters):
    """Attainable matrix rate: a full-chip stream of 32x32x16 bf16 products
    (libva_probe.so), with random and with all-zero operands, and with 2..8
    vector instructions (v_exp_f32 / v_fma_f32) issued after every product,
    at one and two waves per SIMD.  Reports TFLOP/s, the fraction of the
    datasheet peak and the shader clock the waves ran at."""
    import ctypes
    import torch
    torch.cuda.init()
    lib = ctypes.CDLL(os.path.join(ROOT, "variable_length_attention_amd", "libva_probe.so"))
    d = ctypes.c_double
    lib.va_probe_mfma_stream.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(d)] * 3
    lib.va_probe_mfma_stream.restype = ctypes.c_int
    rows = []
    cases = [(wps, zero, 0, 0) for wps in (1, 2) for zero in (0, 1)]
    cases += [(wps, 0, k, op) for wps in (1, 2) for op in (0, 1) for k in (2, 4, 6, 8)]
    for wps, zero, k, op in cases:
        ms, tf, mhz = d(), d(), d()
        rc = lib.va_probe_mfma_stream(wps, iters, zero, k, op, ctypes.byref(ms), ctypes.byref(tf), ctypes.byref(mhz))
        if rc != 0:
            raise RuntimeError(f"va_probe_mfma_stream failed: hip error {rc}")
        rows.append({"waves_per_simd": wps, "data": "zero" if zero else "random",
                     "valu_per_mfma": k, "valu_op": ("v_exp_f32", "v_fma_f32")[op] if k else None,
                     "ms": round(ms.value, 4), "tflops": round(tf.value, 1),
                     "frac_of_peak": round(tf.value / PEAK_BF16_TFLOPS, 4), "shader_mhz": round(mhz.value)})
        print(json.dumps(rows[-1]), flush=True)


def calibrate_lds(iters):
    """LDS read rate per compute unit (libva_probe.so): 16-byte reads and
    transposing 8-byte reads, alone and supplying one operand of every
    32x32x16 bf16 product (1 KB per product per wave, the attention tile
    reads' ratio), at one and two workgroups of 4 waves per compute unit."""
    import ctypes
    import torch
    torch.cuda.init()
    lib = ctypes.CDLL(os.path.join(ROOT, "variable_length_attention_amd", "libva_probe.so"))
    d = ctypes.c_double
    lib.va_probe_lds_stream.argtypes = [ctypes.c_int] * 3 + [ctypes.POINTER(d)] * 4
    lib.va_probe_lds_stream.restype = ctypes.c_int
    names = ["ds_read_b128 -> product", "2 x ds_read_b64_tr_b16 -> product", "ds_read_b128 only",
             "ds_read_b64_tr_b16 only"]
    for wps in (1, 2):
        for mode in range(4):
            ms, tf, mhz, bpc = d(), d(), d(), d()
            rc = lib.va_probe_lds_stream(wps, iters, mode, ctypes.byref(ms), ctypes.byref(tf), ctypes.byref(mhz),
                                         ctypes.byref(bpc))
            if rc != 0:
                raise RuntimeError(f"va_probe_lds_stream failed: hip error {rc}")
            row = {"waves_per_simd": wps, "mode": names[mode], "ms": round(ms.value, 4),
                   "tflops": round(tf.value, 1) if mode <= 1 else None,
                   "frac_of_peak": round(tf.value / PEAK_BF16_TFLOPS, 4) if mode <= 1 else None,
                   "shader_mhz": round(mhz.value), "lds_bytes_per_clk_per_cu": round(bpc.value, 1)}
            print(json.dumps(row), flush=True)


def calibrate_hbm(gib):
    """Attainable HBM rate: a full-chip stream (libva_probe.so) over a
    buffer of `gib` GiB, read only, copy and write only, at 4, 8 and 16
    workgroups of 256 threads per CU and 4 or 16 16-byte accesses per lane
    in flight."""
    import ctypes
    import torch
    torch.cuda.init()
    lib = ctypes.CDLL(os.path.join(ROOT, "variable_length_attention_amd", "libva_probe.so"))
    d = ctypes.c_double
    lib.va_probe_hbm_stream.argtypes = [ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(d), ctypes.POINTER(d)]
    lib.va_probe_hbm_stream.restype = ctypes.c_int
    nbytes = int(gib * (1 << 30)) // 16 * 16
    for mode, name in ((0, "read"), (1, "copy"), (2, "write")):
        for deep in (0, 1):
            for bpc in (4, 8, 16):
                ms, gbs = d(), d()
                rc = lib.va_probe_hbm_stream(mode, nbytes, 5, bpc, deep, ctypes.byref(ms), ctypes.byref(gbs))
                if rc != 0:
                    raise RuntimeError(f"va_probe_hbm_stream failed: hip error {rc}")
                print(json.dumps({"stream": name, "bytes": nbytes, "workgroups_per_cu": bpc,
                                  "in_flight_per_lane": 16 if deep else 4, "ms_5_reps": round(ms.value, 3),
                                  "gbs": round(gbs.value, 1), "frac_of_peak": round(gbs.value / PEAK_HBM_GBS, 4)}),
                      flush=True)


# ---------------------------------------------------------------- CPU baseline
CPU_THREADS = 16  # the host-thread share of one GPU on the measurement boxes


def host_info():
    """Threads the oracle uses, the cores visible to this process, nproc and
    the CPU model."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"cores": min(CPU_THREADS, affinity), "affinity_cores": affinity, "nproc": os.cpu_count(),
            "cpu_model": model}


def cpu_baseline(case, budget_s=6.0, full=False):
    """The fp64 oracle on this host (as it stands, not tuned): every row of
    the workload when full, else random (token, head) rows for about
    budget_s seconds.  Rate in mask-adjusted TFLOP/s and query tokens/s."""
    import oracle
    info = host_info()
    threads = info["cores"]
    vis = visible_pairs(case)
    if full:
        t0 = time.perf_counter()
        oracle.forward(case, nthreads=threads)
        spent = time.perf_counter() - t0
        done_flops = flops(case)
        sample = f"all {case['T_q']} x {case['H']} (token, head) rows"
        tokens = case["T_q"]
    else:
        rng = np.random.default_rng(12345)
        done_flops, done_rows, spent = 0.0, 0, 0.0
        n = 64
        while spent < budget_s:
            toks = rng.integers(0, case["T_q"], n)
            heads = rng.integers(0, case["H"], n)
            t0 = time.perf_counter()
            oracle.forward_rows(case, toks, heads, nthreads=threads)
            dt = time.perf_counter() - t0
            spent += dt
            done_rows += n
            done_flops += float(4 * case["D"] * vis[toks].sum())
            if dt < budget_s / 4:
                n *= 2
        sample = f"{done_rows} random (token, head) rows"
        tokens = done_rows / case["H"]
    r = {"value": done_flops / spent / 1e12, "unit": "TFLOP/s", "kind": "oracle",
         "tokens_per_s": tokens / spent, "seconds": spent,
         "sample": f"{sample} of {case['spec'].name}, {done_flops / 1e9:.1f} mask-adjusted GFLOP in "
                   f"{spent:.1f} s (fp64, {threads} threads)"}
    r.update(info)
    return r


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only-main", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-merge", action="store_true", help="skip the log-sum-exp merge timing")
    ap.add_argument("--no-d512", action="store_true", help="skip the head-size-512 forward timing")
    ap.add_argument("--no-sparse", action="store_true", help="skip the sparse shared-KV attention timing")
    ap.add_argument("--sparse-shapes", default="sparse,sparse_d512,sparse_all_d512",
                    help="sparse shared-KV workloads to time (comma-separated keys)")
    ap.add_argument("--configs", default="2,3,4,5", help="workloads to time (first is the main one)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    ap.add_argument("--calibrate-attainable", action="store_true",
                    help="only measure a large bf16 GEMM and a large read-only reduction")
    ap.add_argument("--calibrate-hbm", type=float, default=0, metavar="GIB",
                    help="only run the HBM stream probe over a GIB-GiB buffer (read, copy, write)")
    ap.add_argument("--calibrate-mfma", type=int, default=0, metavar="ITERS",
                    help="only run the matrix-core stream probe (ITERS groups of 4 products per wave)")
    ap.add_argument("--calibrate-lds", type=int, default=0, metavar="ITERS",
                    help="only run the LDS stream probe (ITERS groups of 4 products or 8 reads per wave)")
    ap.add_argument("--record-traffic", nargs=6, metavar=("KEY", "KERNEL_REGEX", "FETCH_CSV", "WRITE_CSV",
                                                          "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="(no GPU) store a kernel's HBM bytes per launch from rocprofv3 counter CSVs")
    ap.add_argument("--counter-summary", nargs=2, metavar=("CSV", "KERNEL_REGEX"),
                    help="(no GPU) per-dispatch counter means of matching kernels, as JSON")
    ap.add_argument("--trace-summary", nargs=2, metavar=("CSV", "KERNEL_REGEX"),
                    help="(no GPU) dispatch durations of matching kernels from a kernel trace, as JSON lines")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic)))
        return
    if args.counter_summary:
        print(json.dumps(counter_means(*args.counter_summary)))
        return
    if args.trace_summary:
        for (name, grid), s in trace_summary(*args.trace_summary).items():
            print(json.dumps(dict(kernel=name, grid=grid, **s)))
        return
    if args.calibrate_mfma:
        calibrate_mfma(args.calibrate_mfma)
        return
    if args.calibrate_hbm:
        calibrate_hbm(args.calibrate_hbm)
        return
    if args.calibrate_lds:
        calibrate_lds(args.calibrate_lds)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return
    if args.calibrate_attainable:
        calibrate_attainable(max(1, args.steps))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the attention forward "
              "is measured per GPU; sharding across GPUs is not part of this library.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W

    torch.cuda.set_device(0)
    cfgs = [int(x) for x in args.configs.split(",")]
    if args.only_main:
        cfgs = cfgs[:1]
    results = {}
    main_case = None
    for n in cfgs:
        spec = W.config(n)
        log(f"config {n} ({spec.name}): generating input")
        case = W.make_case(spec)
        log(f"config {n}: timing {args.steps} steps after {args.warmup} warm-up")
        ms_step, ms_plan, path, ms_eager = time_case(case, args.steps, args.warmup, torch)
        fl, by = flops(case), alg_bytes(case)
        ms_kernel = max(ms_step - ms_plan, 1e-6)
        hbm_bound = path == 1 or (fl / by) < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        r = {"workload": spec.name, "ms_per_step": ms_step, "ms_per_step_eager": ms_eager,
             "ms_prepass": ms_plan, "ms_kernel": ms_kernel,
             "tflops": fl / (ms_step * 1e-3) / 1e12, "gbs": by / (ms_step * 1e-3) / 1e9,
             "tokens_per_s": case["T_q"] / (ms_step * 1e-3), "flop": fl, "bytes": by,
             "kernel_path": PATH_NAMES[path]}
        traffic = measured_traffic(r["kernel_path"], spec.name)
        if hbm_bound:
            ach = by / (ms_kernel * 1e-3) / 1e9
            r["roofline"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": ach / PEAK_HBM_GBS, "frac_call": r["gbs"] / PEAK_HBM_GBS,
                             "traffic": traffic}
        else:
            ach = fl / (ms_kernel * 1e-3) / 1e12
            r["roofline"] = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": ach / PEAK_BF16_TFLOPS, "frac_call": r["tflops"] / PEAK_BF16_TFLOPS,
                             "traffic": traffic}
        log(f"config {n}: {ms_step:.4f} ms/step in a graph ({ms_eager:.4f} eager; pre-pass {ms_plan:.4f} ms), "
            f"{r['tflops']:.1f} TFLOP/s, {r['gbs']:.0f} GB/s, roofline {r['roofline']['frac'] * 100:.1f}% "
            f"of {r['roofline']['bound']}")
        if not args.no_cpu_baseline:
            # one full run per workload (about 30 s for config 2), a sample
            # of rows for the 16k x 16k full-attention shard (5 minutes in full)
            cb = cpu_baseline(case, full=n in (2, 4, 5))
            r["cpu_baseline"] = cb
            log(f"config {n}: oracle {cb['value'] * 1e3:.1f} GFLOP/s on {cb['cores']} threads ({cb['sample']})")
        results[n] = r
        if main_case is None:
            main_case = case
        else:
            del case
    if not args.only_main and W.config(cfgs[0]).dtype == "bf16":
        # the main workload with float16 inputs (same kernels, f16 matrix instructions)
        import dataclasses
        spec16 = dataclasses.replace(W.config(cfgs[0]), dtype="f16", name=W.config(cfgs[0]).name + "_f16")
        log(f"{spec16.name}: generating input")
        case16 = W.make_case(spec16)
        ms16, mp16, _, _ = time_case(case16, args.steps, args.warmup, torch)
        fl16 = flops(case16)
        ach16 = fl16 / (max(ms16 - mp16, 1e-6) * 1e-3) / 1e12
        results["f16"] = {"workload": spec16.name, "ms_per_step": ms16, "ms_prepass": mp16,
                          "tflops": fl16 / (ms16 * 1e-3) / 1e12, "flop": fl16, "kernel_path": "prefill16",
                          "roofline": {"bound": "mfma", "achieved": ach16, "peak": PEAK_BF16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": ach16 / PEAK_BF16_TFLOPS, "traffic": None}}
        log(f"{spec16.name}: {ms16:.4f} ms/step, {results['f16']['tflops']:.1f} TFLOP/s")
        del case16
        cfgs = cfgs + ["f16"]
    n0 = cfgs[0]
    main = results[n0]
    spec0 = W.config(n0)
    line = {
        "metric": "varlen attn fwd TFLOP/s (mask-adjusted)",
        "value": main["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if spec0.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": spec0.name, "batch": main_case["B"], "total_tokens": main_case["T_q"],
                   "num_heads": spec0.H, "num_kv_heads": spec0.Hkv, "head_dim": spec0.D,
                   "causal": spec0.causal, "window": list(spec0.window), "sinks": spec0.sinks,
                   "paged": spec0.paged, "seed": spec0.seed},
        "roofline": main["roofline"],
        "tokens_per_s": main["tokens_per_s"],
        "ms_per_step_eager": main["ms_per_step_eager"],
        "ms_kernel": main["ms_kernel"],
        "timing": "K steps as one captured HIP graph of back-to-back calls, HIP events around the replay; "
                  "ms_per_step_eager: the same K calls issued from Python",
    }
    if not args.no_backward and spec0.dtype == "bf16" and not spec0.paged:
        log(f"backward on {spec0.name}: timing {args.steps} calls after {args.warmup} warm-up")
        ms_b = time_backward(main_case, args.steps, args.warmup, torch)
        # 5 matrix products (S, dP, dV, dK, dQ) of 2 * head_dim FLOPs per
        # unmasked pair and head: 10 * head_dim (the forward's 2.5x)
        fl_b = 2.5 * flops(main_case)
        tf_b = fl_b / (ms_b * 1e-3) / 1e12
        line["backward"] = {"workload": spec0.name, "ms_per_step": ms_b, "tflops": tf_b, "flop": fl_b,
                            "flop_convention": "10 * head_dim per unmasked (query, key) pair and head",
                            "roofline": {"bound": "mfma", "achieved": tf_b, "peak": PEAK_BF16_TFLOPS,
                                         "unit": "TFLOP/s", "frac": tf_b / PEAK_BF16_TFLOPS,
                                         "scope": "whole backward call", "traffic": None}}
        log(f"backward: {ms_b:.4f} ms/call, {tf_b:.1f} TFLOP/s")
    if not args.no_d512:
        # the forward at head size 512 (its own kernel) on a causal GQA prefill
        spec512 = W.D512_PREFILL
        log(f"{spec512.name} (4 x 2048 tokens, 32/8 heads, head size 512, causal): generating input")
        c512 = W.make_case(spec512)
        ms_s, ms_p, path_s, ms_e = time_case(c512, args.steps, args.warmup, torch)
        ms_k = max(ms_s - ms_p, 1e-6)
        fl = flops(c512)
        tf_k = fl / (ms_k * 1e-3) / 1e12
        line["prefill512"] = {
            "workload": "bf16 causal GQA prefill at head size 512: 4 x 2048 tokens, 32 heads / 8 kv heads",
            "kernel_path": PATH_NAMES[path_s], "ms_per_step": ms_s, "ms_per_step_eager": ms_e, "ms_kernel": ms_k,
            "tflops": fl / (ms_s * 1e-3) / 1e12, "flop": fl,
            "roofline": {"bound": "mfma", "achieved": tf_k, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf_k / PEAK_BF16_TFLOPS,
                         "traffic": measured_traffic(PATH_NAMES[path_s], spec512.name)}}
        log(f"prefill512: {ms_s:.4f} ms/step ({ms_e:.4f} eager), {tf_k:.1f} TFLOP/s kernel, "
            f"{tf_k / PEAK_BF16_TFLOPS * 100:.1f}% of mfma")
        del c512
    if not args.no_merge:
        log("merge of 8 float32 partials (32768 x 24 x 128): timing")
        ms_m, by_m = time_merge(args.steps, args.warmup, torch)
        gbs = by_m / (ms_m * 1e-3) / 1e9
        line["merge"] = {"workload": "ring of 8 float32 partials, 32768 rows x 24 heads x 128 -> bf16",
                         "ms_per_step": ms_m, "gbs": gbs, "bytes": by_m,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gbs / PEAK_HBM_GBS, "traffic": None}}
        log(f"merge: {ms_m:.4f} ms/call, {gbs:.0f} GB/s")
    if not args.no_sparse:
        shapes = {"sparse": SPARSE_SHAPE, "sparse_d512": SPARSE_SHAPE_D512, "sparse_all_d512": SPARSE_SHAPE_ALL_D512}
        for key in [k for k in args.sparse_shapes.split(",") if k]:
            shape = shapes[key]
            D = shape["D"]
            what = ("every visible compressed key (1025 to 2048) of 4x compressed keys" if shape.get("cmp_all") else
                    "512 selected of 4x compressed keys")
            log(f"sparse shared-KV attention (4 x 1024 tokens over 8192 keys, 64/1 heads, d{D}, "
                f"window 128 + {what})")
            ms_s, fl_s, by_s = time_sparse(args.steps, args.warmup, torch, shape)
            tf_s, gb_s = fl_s / (ms_s * 1e-3) / 1e12, by_s / (ms_s * 1e-3) / 1e9
            hbm = (fl_s / by_s) < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
            line[key] = {
                "workload": f"sliding window (127, 0) + {what}, shared K/V, "
                            f"4 x 1024 tokens over 8192 keys, 64 heads / 1 kv head, d{D}, bf16",
                "ms_per_step": ms_s, "tflops": tf_s, "gbs": gb_s, "flop": fl_s, "bytes": by_s,
                "roofline": ({"bound": "hbm", "achieved": gb_s, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": gb_s / PEAK_HBM_GBS, "traffic": measured_traffic("sparse", key)} if hbm else
                             {"bound": "mfma", "achieved": tf_s, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": tf_s / PEAK_BF16_TFLOPS, "traffic": measured_traffic("sparse", key)})}
            log(f"{key}: {ms_s:.4f} ms/call, {tf_s:.1f} TFLOP/s, {gb_s:.0f} GB/s (algorithmic)")
    if not args.no_cpu_baseline:
        # the main workload's oracle rate, and the oracle on every workload
        c1 = W.make_case(W.config(1))
        per = {W.config(1).name: cpu_baseline(c1, full=True)}
        for n in cfgs:
            if n in results and "cpu_baseline" in results[n]:
                per[results[n]["workload"]] = results[n].pop("cpu_baseline")
        line["cpu_baseline"] = dict(per[main["workload"]])
        line["cpu_baseline"]["per_workload"] = {k: {x: v[x] for x in ("value", "unit", "tokens_per_s", "seconds",
                                                                       "sample")} for k, v in per.items()}
    line["also"] = {results[n]["workload"]: {k: v for k, v in results[n].items() if k != "workload"}
                    for n in cfgs[1:]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
