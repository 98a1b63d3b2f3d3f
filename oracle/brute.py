"""Dense brute-force checker (numpy float64), for small inputs only.

TEST INFRASTRUCTURE ONLY; independent of both the C oracle and the HIP path.
Per (sequence, head) it materialises the whole Lq x Lk score matrix, builds
the allowed-key mask by broadcasting index vectors, appends the sink logit
as one extra column whose value row is zero, and takes the log-sum-exp with
``scipy.special.logsumexp``.  It follows the formula of the SparseAttnSharedkv
README (softmax(Q K^T * scale) V) with the mask and sink readings stated in
``varlen_oracle.c``.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp

from workloads import bf16_bits_to_f32


def _f64(a, dtype):
    return (bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


def key_rows(case, b):
    """Logical K and V rows of sequence b as float64 [Lk, Hkv, D]."""
    dt = case["dtype"]
    if case.get("paged"):
        bs = case["block_size"]
        L = int(case["seqused_k"][b])
        idx = np.arange(L)
        blk = case["block_table"][b][idx // bs]
        k = case["k_cache"][blk, idx % bs]
        v = case["v_cache"][blk, idx % bs]
    else:
        s, e = int(case["cu_k"][b]), int(case["cu_k"][b + 1])
        k, v = case["k"][s:e], case["v"][s:e]
    return _f64(k, dt), _f64(v, dt)


def mask(Lq, Lk, causal, wl, wr):
    i = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    ok = np.ones((Lq, Lk), dtype=bool)
    if causal:
        ok &= j <= i
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


def dense_forward(case, return_probs=False):
    """Returns (out [T_q,H,D], lse [T_q,H]) and, optionally, per (b, h) the
    probability matrices including the sink column."""
    H, Hkv, D = case["H"], case["Hkv"], case["D"]
    g = H // Hkv
    q_all = _f64(case["q"], case["dtype"])
    out = np.zeros((case["T_q"], H, D))
    lse = np.full((case["T_q"], H), -np.inf)
    probs = {}
    sinks = case.get("sinks")
    alibi = case.get("alibi")
    for b in range(case["B"]):
        s, e = int(case["cu_q"][b]), int(case["cu_q"][b + 1])
        Lq = e - s
        k, v = key_rows(case, b)
        Lk = k.shape[0]
        ok = mask(Lq, Lk, case["causal"], case["window_left"], case["window_right"])
        for h in range(H):
            c = h // g
            S = (q_all[s:e, h, :] @ k[:, c, :].T) * case["scale"]
            if alibi is not None:
                pos = np.arange(Lq)[:, None] + (Lk - Lq)
                S = S - float(alibi[h]) * np.abs(pos - np.arange(Lk)[None, :])
            S = np.where(ok, S, -np.inf)
            V = v[:, c, :]
            if sinks is not None:
                S = np.concatenate([S, np.full((Lq, 1), float(sinks[h]))], axis=1)
                V = np.concatenate([V, np.zeros((1, D))], axis=0)
            L = logsumexp(S, axis=1) if S.shape[1] else np.full(Lq, -np.inf)
            with np.errstate(invalid="ignore"):
                P = np.where(np.isfinite(L)[:, None], np.exp(S - L[:, None]), 0.0)
            out[s:e, h, :] = P @ V
            lse[s:e, h] = L
            if return_probs:
                probs[(b, h)] = P
    if return_probs:
        return out, lse, probs
    return out, lse
