"""Reference implementations of the variable-length attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the library under test imports,
loads or calls this package; only ``tests/``, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg do.  It shares no code with the HIP
path: the only common module is the seeded input generator ``workloads``,
which holds no attention arithmetic.

* ``backward`` -- the double-precision C backward (the steps of the boostr
  CPU backward ``varlen_attention_bwd``), given the forward's out and lse,
  threaded over (sequence, kv head) units so the GQA sums need no locks.
* ``forward`` / ``forward_rows`` -- the double-precision C implementation in
  ``varlen_oracle.c`` (a three-pass softmax per query row, in the order of
  the boostr CPU forward ``varlen_attention_fwd``), threaded over
  (sequence, head, 64-row) units.
* ``brute.dense_forward`` -- an independent dense numpy checker for small
  inputs (full score matrix, boolean mask, ``scipy.special.logsumexp``).
* ``backward_sampled`` -- the backward's definitions at chosen dq rows and
  dk / dv keys (numpy, float64), for workloads too large for ``backward``.
* ``sink_grad`` -- the gradient of the sink logits (the softmax chain rule
  for one more logit with a zero value row), written out in float64.
* ``merge`` -- the log-sum-exp merge of partial results over disjoint key
  sets (the combine step of ring / context-parallel attention that the
  vllm-omni Ulysses wrapper's ring path needs), written out in float64.
* ``sparse_sharedkv`` -- sliding-window + sparse compressed attention over
  shared K/V (the SparseAttnSharedkv README's third scenario), written out
  in float64 token by token.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "varlen_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libvarlen_oracle.so")
_lock = threading.Lock()
_lib = None


class _Args(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("wl", ctypes.c_int32), ("wr", ctypes.c_int32), ("scale", ctypes.c_double),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("cu_q", ctypes.c_void_p), ("cu_k", ctypes.c_void_p),
        ("seqused_k", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("sinks", ctypes.c_void_p), ("alibi", ctypes.c_void_p),
    ]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc into ``oracle/_build``."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                        "-pthread", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            lib.oracle_varlen_fwd.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int]
            lib.oracle_varlen_fwd.restype = ctypes.c_int
            lib.oracle_varlen_fwd_rows.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p,
                                                   ctypes.c_int64, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_int]
            lib.oracle_varlen_fwd_rows.restype = ctypes.c_int
            lib.oracle_varlen_bwd.argtypes = [ctypes.POINTER(_Args)] + [ctypes.c_void_p] * 6 + [ctypes.c_int]
            lib.oracle_varlen_bwd.restype = ctypes.c_int
            lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_half_to_double.restype = ctypes.c_double
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _make_args(case: dict, keep: list) -> _Args:
    def c(a, dt):
        if a is None:
            return None
        a = np.asarray(a)
        if a.dtype == np.float16:  # binary16 values go over as their bits
            a = a.view(np.uint16)
        a = np.ascontiguousarray(a, dtype=dt)
        keep.append(a)
        return a
    elt = np.uint16 if case["dtype"] in ("bf16", "f16") else np.float32
    a = _Args()
    a.dtype = {"f32": 0, "bf16": 1, "f16": 2}[case["dtype"]]
    a.B, a.H, a.Hkv, a.D = case["B"], case["H"], case["Hkv"], case["D"]
    a.causal = 1 if case["causal"] else 0
    a.wl, a.wr = case["window_left"], case["window_right"]
    a.scale = float(case["scale"])
    a.q = _ptr(c(case["q"], elt))
    a.cu_q = _ptr(c(case["cu_q"], np.int32))
    if case.get("paged"):
        a.k = _ptr(c(case["k_cache"], elt))
        a.v = _ptr(c(case["v_cache"], elt))
        a.seqused_k = _ptr(c(case["seqused_k"], np.int32))
        bt = c(case["block_table"], np.int32)
        a.block_table = _ptr(bt)
        a.bt_stride = bt.shape[1]
        a.block_size = case["block_size"]
    else:
        a.k = _ptr(c(case["k"], elt))
        a.v = _ptr(c(case["v"], elt))
        a.cu_k = _ptr(c(case["cu_k"], np.int32))
    a.sinks = _ptr(c(case.get("sinks"), np.float32))
    a.alibi = _ptr(c(case.get("alibi"), np.float32))
    return a


def forward(case: dict, nthreads: int | None = None):
    """All rows.  Returns (out float64 [T_q, H, D], lse float64 [T_q, H])."""
    lib = _load()
    keep: list = []
    a = _make_args(case, keep)
    out = np.zeros((case["T_q"], case["H"], case["D"]), dtype=np.float64)
    lse = np.zeros((case["T_q"], case["H"]), dtype=np.float64)
    rc = lib.oracle_varlen_fwd(ctypes.byref(a), out.ctypes.data, lse.ctypes.data,
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out, lse


def forward_rows(case: dict, tokens, heads, nthreads: int | None = None):
    """Selected (token, head) pairs.  Returns (out [n, D], lse [n]) in float64."""
    lib = _load()
    keep: list = []
    a = _make_args(case, keep)
    pairs = (np.asarray(tokens, dtype=np.int64) * case["H"]
             + np.asarray(heads, dtype=np.int64))
    pairs = np.ascontiguousarray(pairs)
    out = np.zeros((len(pairs), case["D"]), dtype=np.float64)
    lse = np.zeros(len(pairs), dtype=np.float64)
    rc = lib.oracle_varlen_fwd_rows(ctypes.byref(a), pairs.ctypes.data, len(pairs),
                                    out.ctypes.data, lse.ctypes.data,
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out, lse


def backward(case: dict, dout, out, lse, nthreads: int | None = None):
    """Gradients of sum(dout * O) for a contiguous case, given the forward's
    out [T_q, H, D] and lse [T_q, H] (any float arrays, used as float64).
    Returns (dq [T_q, H, D], dk [T_k, Hkv, D], dv [T_k, Hkv, D]) in float64."""
    if case.get("paged"):
        raise ValueError("the backward oracle takes contiguous K/V")
    lib = _load()
    keep: list = []
    a = _make_args(case, keep)
    f = [np.ascontiguousarray(x, dtype=np.float64) for x in (dout, out, lse)]
    T_k = int(np.asarray(case["cu_k"])[-1])
    dq = np.zeros((case["T_q"], case["H"], case["D"]), dtype=np.float64)
    dk = np.zeros((T_k, case["Hkv"], case["D"]), dtype=np.float64)
    dv = np.zeros_like(dk)
    rc = lib.oracle_varlen_bwd(ctypes.byref(a), f[0].ctypes.data, f[1].ctypes.data, f[2].ctypes.data,
                               dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return dq, dk, dv


def _wide(a, dtype):
    return _widen16(a, dtype) if dtype in ("bf16", "f16") else np.asarray(a, np.float64)


def _key_range(i, delta, Lk, case):
    """Visible keys [lo, hi] of query row i (p = i + delta): [p - left,
    p + right] within [0, Lk), with causal capping the right side at p and
    -1 meaning unbounded."""
    p = i + delta
    lo = 0 if case["window_left"] < 0 else max(0, p - case["window_left"])
    right = 0 if case["causal"] else case["window_right"]
    hi = Lk - 1 if right < 0 else min(Lk - 1, p + right)
    return lo, hi


def backward_sampled(case: dict, dout, out, lse, rows, keys):
    """The backward's definitions evaluated at chosen outputs only (for
    workloads too large for ``backward``): dq at query (token, head) pairs
    ``rows`` and dk, dv at key (token, kv head) pairs ``keys``.  With
    P_ij = exp(s_ij - lse_i), s_ij = scale <q_i, k_j> (+ ALiBi bias),
    Dv_i = <dout_i, out_i>, dS_ij = P_ij (<dout_i, v_j> - Dv_i):
    dq_i = scale sum_j dS_ij k_j over the keys row i sees; dk_j = scale
    sum_{i, h} dS_ij q_i and dv_j = sum_{i, h} P_ij dout_i over the rows and
    query heads of the kv head that see key j (the gradients the boostr CPU
    backward ``varlen_attention_bwd`` accumulates, here per output element).
    Contiguous K/V; float64."""
    if case.get("paged"):
        raise ValueError("the backward oracle takes contiguous K/V")
    dt, H, Hkv = case["dtype"], case["H"], case["Hkv"]
    g = H // Hkv
    cu_q, cu_k = np.asarray(case["cu_q"], np.int64), np.asarray(case["cu_k"], np.int64)
    q, k, v = (np.asarray(case[x]) for x in ("q", "k", "v"))
    dout, out, lse = (np.asarray(x) for x in (dout, out, lse))   # widened where read
    alibi = case.get("alibi")
    sc = float(case["scale"])

    def scores(qv, kv, h, p, js):
        s = sc * (kv @ qv)
        if alibi is not None:
            s = s - float(alibi[h]) * np.abs(p - js)
        return s

    dq = np.zeros((len(rows[0]), case["D"]))
    for n, (t, h) in enumerate(zip(*rows)):
        b = int(np.searchsorted(cu_q, t, side="right") - 1)
        i, Lq, Lk = t - cu_q[b], cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        lo, hi = _key_range(i, Lk - Lq, Lk, case)
        if hi < lo:
            continue
        js = np.arange(lo, hi + 1)
        c = h // g
        kb = _wide(k[cu_k[b] + js, c], dt)
        vb = _wide(v[cu_k[b] + js, c], dt)
        do_t, o_t = dout[t, h].astype(np.float64), out[t, h].astype(np.float64)
        pr = np.exp(scores(_wide(q[t, h], dt), kb, h, i + Lk - Lq, js) - float(lse[t, h]))
        ds = pr * (vb @ do_t - do_t @ o_t)
        dq[n] = sc * (ds @ kb)
    dk = np.zeros((len(keys[0]), case["D"]))
    dv = np.zeros_like(dk)
    for n, (u, c) in enumerate(zip(*keys)):
        b = int(np.searchsorted(cu_k, u, side="right") - 1)
        j, Lq, Lk = u - cu_k[b], cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        bounds = [_key_range(i, Lk - Lq, Lk, case) for i in range(Lq)]
        ii = np.array([i for i, (lo, hi) in enumerate(bounds) if lo <= j <= hi], np.int64)
        if ii.size == 0:
            continue
        kj, vj = _wide(k[u, c], dt), _wide(v[u, c], dt)
        for h in range(c * g, (c + 1) * g):
            t = cu_q[b] + ii
            qh = _wide(q[t, h], dt)
            s = sc * (qh @ kj)
            if alibi is not None:
                s = s - float(alibi[h]) * np.abs(ii + Lk - Lq - j)
            do_t, o_t = dout[t, h].astype(np.float64), out[t, h].astype(np.float64)
            pr = np.exp(s - lse[t, h].astype(np.float64))
            ds = pr * (do_t @ vj - np.sum(do_t * o_t, axis=1))
            dk[n] += sc * (ds @ qh)
            dv[n] += pr @ do_t
    return dq, dk, dv


def sink_grad(case: dict, dout, out, lse):
    """Gradient of sum(dout * O) with respect to the sink logits.  The sink of
    head h is one more logit of every query row's softmax whose value row is
    zero (SparseAttnSharedkv README, sinks parameter), so by the softmax's
    chain rule its dS term is exp(s_h - lse_i) (0 - sum_d dout_i,d O_i,d), and
    dsinks_h is the sum of those terms over every query row.  out and lse are
    the forward's (with the sinks); returns float64 [H]."""
    H = case["H"]
    d_vec = np.einsum("thd,thd->th", np.asarray(dout, np.float64), np.asarray(out, np.float64))
    lse64 = np.asarray(lse, np.float64)
    s = np.asarray(case["sinks"], np.float64)[None, :]
    p_sink = np.where(np.isneginf(lse64), 0.0, np.exp(s - lse64))
    return -(p_sink * d_vec).sum(axis=0).reshape(H)


def merge(o_parts, lse_parts, sinks=None):
    """Softmax over the union of disjoint key sets from per-set partials.

    o_parts [n, rows, H, D] and lse_parts [n, rows, H] (natural log; -inf for
    a part with no key) are the attention outputs and log-sum-exps of the
    same queries over n disjoint key sets; sinks [H] (or None) is the sink
    logit of each head, counted once.  For each (row, head):
    lse = log(sum_p exp(lse_p) + exp(sigma)), out = sum_p exp(lse_p - lse) o_p.
    Rows with nothing (every part empty, no sink) get out = 0, lse = -inf.
    Returns (out [rows, H, D], lse [rows, H]) in float64."""
    o = np.asarray(o_parts, dtype=np.float64)
    lp = np.asarray(lse_parts, dtype=np.float64)
    n, rows, H = lp.shape
    terms = lp
    if sinks is not None:
        sig = np.broadcast_to(np.asarray(sinks, dtype=np.float64)[None, None, :], (1, rows, H))
        terms = np.concatenate([lp, sig], axis=0)
    m = terms.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    total = np.exp(terms - m_safe[None]).sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, total, 1.0)), -np.inf)
    w = np.where(finite[None], np.exp(lp - np.where(finite, lse, 0.0)[None]), 0.0)
    out = (w[..., None] * o).sum(axis=0)
    return out, lse


def half_to_double(bits):
    """The oracle's binary16 widening (uint16 bit patterns -> float64)."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_half_to_double(int(x)) for x in b], dtype=np.float64)


def _widen16(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)  # float16 values


def sparse_sharedkv(case, tokens=None):
    """Attention of each query token over its sliding window of original
    keys plus compressed keys, in one softmax (sinks as extra logits; each
    key row is also its value row).  SparseAttnSharedkv README, formula
    section (K~ = V~ from ori_kv, cmp_kv, cmp_ratio and the indices) and its
    scenarios: with ``case["cmp_all"]`` false the compressed keys are those
    the indices select (third scenario; none when topk = 0), with it true
    every compressed key the mask admits (second scenario: ori_kv and cmp_kv
    given, no indices).
    Readings: the window is [p - left, p + right] with p = i + S2_b - Lq_b;
    sequence b has S3_b = S2_b / cmp_ratio compressed keys, and the
    compressed-key mask (cmp_mask_mode 3) is causal aligned to the
    bottom-right of the Lq_b x S3_b matrix: row i sees compressed position t
    iff t <= i + S3_b - Lq_b; an index outside [0, S3_b) or beyond that
    bound selects nothing; a repeated index is attended as often as it
    appears.
    Returns (out [n, H, D], lse [n, H]) in float64 for the given tokens (all
    tokens by default)."""
    cu_q = np.asarray(case["cu_q"], np.int64)
    T, H, Hkv, D = case["T"], case["H"], case["Hkv"], case["D"]
    g = H // Hkv
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    left, right = case["window"]
    cmp_all = bool(case.get("cmp_all", False))
    out = np.zeros((len(toks), H, D))
    lse = np.full((len(toks), H), -np.inf)

    def rows(cache, table, bs, b, positions, c):
        positions = np.asarray(positions, np.int64)
        phys = np.asarray(table)[b, positions // bs].astype(np.int64)
        return _widen16(np.asarray(cache)[phys, positions % bs, c], case["dtype"])

    for n, t in enumerate(toks):
        b = int(np.searchsorted(cu_q, t, side="right") - 1)
        i = t - cu_q[b]
        Lq = cu_q[b + 1] - cu_q[b]
        S2 = int(case["seqused_kv"][b])
        S3 = S2 // case["cmp_ratio"]
        p = i + S2 - Lq
        last = i + S3 - Lq  # last compressed position row i sees
        win = np.arange(max(0, p - left), min(S2 - 1, p + right) + 1)
        for c in range(Hkv):
            if cmp_all:
                sel = np.arange(0, max(0, min(S3, last + 1)))
            else:
                sel = np.asarray(case["indices"][t, c], np.int64)
                sel = sel[(sel >= 0) & (sel < S3) & (sel <= last)]
            kv = np.concatenate([rows(case["ori_kv"], case["ori_table"], case["ori_kv"].shape[1], b, win, c),
                                 rows(case["cmp_kv"], case["cmp_table"], case["cmp_kv"].shape[1], b, sel, c)])
            heads = np.arange(c * g, (c + 1) * g)
            qv = _widen16(np.asarray(case["q"])[t, heads], case["dtype"])
            logits = case["scale"] * (qv @ kv.T)                        # [g, keys]
            if case.get("sinks") is not None:
                logits = np.concatenate([logits, np.asarray(case["sinks"], np.float64)[heads][:, None]], axis=1)
            if logits.shape[1] == 0:
                continue
            m = logits.max(axis=1, keepdims=True)
            w = np.exp(logits - m)
            z = w.sum(axis=1, keepdims=True)
            lse[n, heads] = (m + np.log(z))[:, 0]
            out[n, heads] = (w[:, : kv.shape[0]] / z) @ kv
    return out, lse
