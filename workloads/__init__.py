"""Seeded synthetic inputs for variable-length packed attention.

This module is shared by the oracle's tests and the HIP path's tests and
benchmark.  It draws numbers and lays them out in memory; it holds none of
the attention arithmetic (no scores, masks, softmax or reductions).

Layouts follow the statement of the problem on the pages:

* packed "TND" tensors ``[T, N, D]`` with ``cu_seqlens`` prefix sums of
  ``B + 1`` non-decreasing int32 entries (SparseAttnSharedkv README,
  constraints section, TND layout bullet);
* paged "PA_ND" caches ``[num_blocks, block_size, KV_N, D]`` addressed
  through an int32 ``block_table[B, W]`` and per-sequence ``seqused_kv``
  (same README, PageAttention constraints bullet; parameter table rows
  ``ori_block_table`` and ``seqused_kv``);
* per-head fp32 sink logits ``sinks[H]`` (same README, parameter table row
  ``sinks``; its usage example draws one value per query head).

float16 ("f16") data is numpy's round-to-nearest-even cast of the same
float32 draws, carried as numpy float16 arrays.

Recipe (all configurations): ``rng = numpy.random.default_rng(seed)`` and,
in this order, (1) lengths, (2) ``q`` of shape ``[T_q, H, D]`` from
``standard_normal(float32)``, (3) per sequence in packing order ``k_b`` then
``v_b`` of shape ``[Lk_b, H_kv, D]``, (4) ``sinks`` when present, (5) the
block permutation when paged.  bf16 data is the round-to-nearest-even cast
of those float32 draws and is carried as its raw 16-bit patterns (uint16).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np

__all__ = [
    "Spec", "CONFIGS", "config", "scaled", "make_case", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "case_digest", "POISON_BF16", "POISON_F32", "merge_inputs", "sparse_case",
]

# Finite poison written into cache slots that no sequence owns.  Read by
# mistake it overflows the scores (|q.k| ~ 1e4 * sqrt(D)); multiplied by an
# exact zero it stays zero.
POISON_F32 = 1.0e4
POISON_BF16 = 0x461C  # bf16 bit pattern of 10000.0


@dataclasses.dataclass(frozen=True)
class Spec:
    """One synthetic workload.

    ``lens_q``: ("fixed", [..]) | ("uniform", lo, hi, B)  (inclusive bounds)
    ``lens_k``: "same" | ("uniform", lo, hi)               (inclusive bounds)
    ``window``: (left, right), -1 meaning unbounded on that side.
    """
    name: str
    seed: int
    dtype: str
    H: int
    Hkv: int
    D: int
    lens_q: tuple
    lens_k: object = "same"
    causal: bool = False
    window: tuple = (-1, -1)
    sinks: bool = False
    paged: bool = False
    block_size: int = 64
    scale: Optional[float] = None  # None -> 1/sqrt(D)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)


# The five workloads of this project (configs 1..5); seed = 1000 + number.
CONFIGS = {
    1: Spec("tiny_f32_causal_gqa", 1001, "f32", 4, 2, 64,
            ("fixed", [5, 17, 32]), causal=True),
    2: Spec("bf16_causal_gqa_prefill", 1002, "bf16", 32, 8, 128,
            ("uniform", 128, 4096, 16), causal=True),
    3: Spec("bf16_full_ulysses_shard", 1003, "bf16", 24, 24, 128,
            ("fixed", [16384, 16384])),
    4: Spec("bf16_swa_sinks_mqa", 1004, "bf16", 64, 1, 128,
            ("uniform", 1024, 8192, 8), window=(127, 0), sinks=True),
    5: Spec("bf16_paged_decode", 1005, "bf16", 32, 8, 128,
            ("uniform", 1, 4, 128), lens_k=("uniform", 1024, 32768),
            causal=True, paged=True, block_size=64),
}


def config(n: int) -> Spec:
    return CONFIGS[n]


# The head-size-512 forward workload (the SparseAttnSharedkv README's head
# size on the dense path): 4 x 2048 tokens, causal, 32 query / 8 kv heads.
D512_PREFILL = Spec("bf16_causal_gqa_d512", 1512, "bf16", 32, 8, 512, ("fixed", [2048] * 4), causal=True)


def scaled(spec: Spec, *, B: int = 6, max_len: int = 300, seed: Optional[int] = None,
           name: Optional[str] = None) -> Spec:
    """Same structure (heads, dims, mask, sinks, paging) at sizes a slow CPU
    implementation finishes in seconds: at most ``B`` sequences, lengths at
    most ``max_len``."""
    lq = spec.lens_q
    if lq[0] == "fixed":
        new_q = ("fixed", [min(x, max_len) for x in lq[1]][:B])
    else:
        lo, hi = lq[1], lq[2]
        hi2 = min(hi, max_len)
        new_q = ("uniform", min(lo, hi2), hi2, min(lq[3], B))
    lk = spec.lens_k
    if lk != "same":
        hi2 = min(lk[2], max_len)
        new_k = ("uniform", min(lk[1], hi2), hi2)
    else:
        new_k = "same"
    return dataclasses.replace(spec, lens_q=new_q, lens_k=new_k,
                               seed=spec.seed if seed is None else seed,
                               name=name or (spec.name + "_small"))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_lengths(spec: Spec, rng: np.random.Generator):
    lq = spec.lens_q
    if lq[0] == "fixed":
        lens_q = np.asarray(lq[1], dtype=np.int64)
    else:
        lens_q = rng.integers(lq[1], lq[2], size=lq[3], endpoint=True).astype(np.int64)
    if spec.lens_k == "same":
        lens_k = lens_q.copy()
    else:
        lens_k = rng.integers(spec.lens_k[1], spec.lens_k[2], size=len(lens_q),
                              endpoint=True).astype(np.int64)
    return lens_q, lens_k


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return np.ascontiguousarray(x, np.float32).astype(np.float16)  # round to nearest even
    return np.ascontiguousarray(x, np.float32)


def make_case(spec: Spec, *, lens_q=None, lens_k=None, poison: bool = True) -> dict:
    """Draw one case.  ``lens_q``/``lens_k`` override the drawn lengths (the
    draws are still made so that the value stream stays aligned)."""
    rng = np.random.default_rng(spec.seed)
    dq, dk = _draw_lengths(spec, rng)
    if lens_q is not None:
        dq = np.asarray(lens_q, dtype=np.int64)
        dk = dq.copy() if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    elif lens_k is not None:
        dk = np.asarray(lens_k, dtype=np.int64)
    B = len(dq)
    H, Hkv, D = spec.H, spec.Hkv, spec.D
    T_q = int(dq.sum())
    T_k = int(dk.sum())
    cu_q = np.zeros(B + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(dq)
    cu_k = np.zeros(B + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(dk)

    q = _cast(rng.standard_normal((T_q, H, D), dtype=np.float32), spec.dtype)
    elt = {"bf16": np.uint16, "f16": np.float16}.get(spec.dtype, np.float32)
    case = dict(spec=spec, B=B, H=H, Hkv=Hkv, D=D, dtype=spec.dtype,
                scale=spec.softmax_scale, causal=bool(spec.causal),
                window_left=int(spec.window[0]), window_right=int(spec.window[1]),
                lens_q=dq, lens_k=dk, T_q=T_q, T_k=T_k, cu_q=cu_q,
                max_q=int(dq.max()) if B else 0, max_k=int(dk.max()) if B else 0,
                q=q, paged=spec.paged)

    if not spec.paged:
        k = np.empty((T_k, Hkv, D), dtype=elt)
        v = np.empty((T_k, Hkv, D), dtype=elt)
        for b in range(B):
            s, e = int(cu_k[b]), int(cu_k[b + 1])
            k[s:e] = _cast(rng.standard_normal((e - s, Hkv, D), dtype=np.float32), spec.dtype)
            v[s:e] = _cast(rng.standard_normal((e - s, Hkv, D), dtype=np.float32), spec.dtype)
        case.update(k=k, v=v, cu_k=cu_k)
        if spec.sinks:
            case["sinks"] = rng.standard_normal(H, dtype=np.float32)
        else:
            case["sinks"] = None
        return case

    bs = spec.block_size
    nblk = [(int(x) + bs - 1) // bs for x in dk]
    n_used = int(sum(nblk))
    W = max(max(nblk) if nblk else 1, 1)
    poison_val = {"bf16": POISON_BF16, "f16": np.float16(POISON_F32)}.get(spec.dtype, np.float32(POISON_F32))
    # one spare physical block at the end holds only poison
    k_cache = np.empty((n_used + 1, bs, Hkv, D), dtype=elt)
    v_cache = np.empty((n_used + 1, bs, Hkv, D), dtype=elt)
    k_cache[n_used] = poison_val if poison else 0
    v_cache[n_used] = poison_val if poison else 0
    kv_draws = []
    for b in range(B):
        L = int(dk[b])
        kb = _cast(rng.standard_normal((L, Hkv, D), dtype=np.float32), spec.dtype)
        vb = _cast(rng.standard_normal((L, Hkv, D), dtype=np.float32), spec.dtype)
        kv_draws.append((kb, vb))
    sinks = rng.standard_normal(H, dtype=np.float32) if spec.sinks else None
    perm = rng.permutation(n_used).astype(np.int32)
    block_table = np.full((B, W), n_used, dtype=np.int32)
    off = 0
    for b in range(B):
        L = int(dk[b])
        kb, vb = kv_draws[b]
        for t in range(nblk[b]):
            phys = int(perm[off + t])
            block_table[b, t] = phys
            r0, r1 = t * bs, min(L, (t + 1) * bs)
            k_cache[phys, : r1 - r0] = kb[r0:r1]
            v_cache[phys, : r1 - r0] = vb[r0:r1]
            if r1 - r0 < bs:
                k_cache[phys, r1 - r0:] = poison_val if poison else 0
                v_cache[phys, r1 - r0:] = poison_val if poison else 0
        off += nblk[b]
        kv_draws[b] = None
    case.update(k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                seqused_k=dk.astype(np.int32), block_size=bs, num_blocks=n_used + 1,
                sinks=sinks, perm=perm)
    return case


def paged_to_contiguous(case: dict):
    """Logical K/V rows of a paged case gathered into packed TND order.
    (A memory re-layout only; used by tests to compare the two addressings.)"""
    bs = case["block_size"]
    ks, vs = [], []
    for b in range(case["B"]):
        L = int(case["seqused_k"][b])
        nb = (L + bs - 1) // bs
        ids = case["block_table"][b, :nb]
        ks.append(case["k_cache"][ids].reshape(nb * bs, case["Hkv"], case["D"])[:L])
        vs.append(case["v_cache"][ids].reshape(nb * bs, case["Hkv"], case["D"])[:L])
    cu_k = np.zeros(case["B"] + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(case["seqused_k"])
    return np.concatenate(ks, 0), np.concatenate(vs, 0), cu_k


def case_digest(case: dict) -> str:
    """SHA-256 over every array of a case, in a fixed key order."""
    h = hashlib.sha256()
    for key in ("q", "k", "v", "k_cache", "v_cache", "cu_q", "cu_k", "seqused_k",
                "block_table", "sinks"):
        a = case.get(key)
        if a is None:
            continue
        h.update(key.encode())
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def merge_inputs(n: int, rows: int, H: int, D: int, dtype: str = "f32", seed: int = 2000,
                 empty_frac: float = 0.0, empty_rows_every: int = 0) -> dict:
    """Partial results of the same queries over n disjoint key sets, for the
    log-sum-exp merge: ``o_parts`` [n, rows, H, D] (float32, or bf16 bit
    patterns when dtype is "bf16") from ``standard_normal``, ``lse_parts``
    float32 [n, rows, H] = 4 * ``standard_normal``; then a fraction
    ``empty_frac`` of the (part, row, head) entries gets lse = -inf (a part
    with no key for that row), and with ``empty_rows_every`` = k every k-th
    (row, head) vector gets -inf in every part.  Draw order: o, lse, empty
    mask."""
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((n, rows, H, D), dtype=np.float32)
    lse = (rng.standard_normal((n, rows, H), dtype=np.float32) * np.float32(4.0)).astype(np.float32)
    if empty_frac > 0:
        lse[rng.random((n, rows, H)) < empty_frac] = -np.inf
    if empty_rows_every > 0:
        flat = lse.reshape(n, rows * H)
        flat[:, ::empty_rows_every] = -np.inf
    if dtype == "bf16":
        o = f32_to_bf16_bits(o)
    return {"o_parts": o, "lse_parts": lse, "n": n, "rows": rows, "H": H, "D": D, "dtype": dtype}


def _paged(rng, rows_per_seq, bs, Hkv, D, dtype, poison_val):
    """Logical rows of each sequence placed in a block-permuted cache with one
    spare all-poison block; returns (cache, block_table)."""
    nblk = [(r.shape[0] + bs - 1) // bs for r in rows_per_seq]
    n_used = int(sum(nblk))
    W = max(max(nblk) if nblk else 1, 1)
    elt = {"bf16": np.uint16, "f16": np.float16}[dtype]
    cache = np.empty((n_used + 1, bs, Hkv, D), dtype=elt)
    cache[...] = poison_val
    perm = rng.permutation(n_used).astype(np.int32)
    table = np.full((len(rows_per_seq), W), n_used, dtype=np.int32)
    off = 0
    for b, rows in enumerate(rows_per_seq):
        for t in range(nblk[b]):
            phys = int(perm[off + t])
            table[b, t] = phys
            r0, r1 = t * bs, min(rows.shape[0], (t + 1) * bs)
            cache[phys, : r1 - r0] = rows[r0:r1]
        off += nblk[b]
    return cache, table


def sparse_case(lens_q, seqused_kv, *, H=64, Hkv=1, D=128, dtype="bf16", window=(127, 0), topk=512,
                cmp_ratio=4, ori_bs=128, cmp_bs=128, sinks=True, seed=4000, invalid_frac=0.0,
                shared_indices=False, scale=None, cmp_all=False, visible_indices=False) -> dict:
    """Inputs of sliding-window + compressed attention over shared K/V (the
    SparseAttnSharedkv README's second and third scenarios, its shapes: TND
    q, PA_ND caches through permuted block tables, int32 indices [T, H_kv,
    topk]).  ``cmp_all``: the second scenario (every compressed key the mask
    admits; topk must be 0).

    Draw order from ``default_rng(seed)``: q [T, H, D]; per sequence the
    original rows [S2_b, H_kv, D] then the compressed rows [S2_b / ratio,
    H_kv, D] (standard normal, cast to ``dtype``); sinks [H]; the two block
    permutations; the indices: uniform in [0, S3_b), drawn per token or once
    per sequence when ``shared_indices``; or, with ``visible_indices``, as
    the README example draws them: topk distinct positions of [0, S3_b -
    Lq_b] (the compressed keys every query row of the sequence sees), once
    per sequence; then a fraction ``invalid_frac`` of the indices replaced by
    out-of-range values (-1 or S3_b + k)."""
    if cmp_all and topk != 0:
        raise ValueError("the second scenario takes no indices (topk = 0)")
    rng = np.random.default_rng(seed)
    lens_q = np.asarray(lens_q, np.int64)
    S2 = np.asarray(seqused_kv, np.int64)
    B = len(lens_q)
    cu_q = np.zeros(B + 1, np.int32)
    cu_q[1:] = np.cumsum(lens_q)
    T = int(cu_q[-1])
    q = _cast(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
    ori_rows, cmp_rows = [], []
    for b in range(B):
        ori_rows.append(_cast(rng.standard_normal((int(S2[b]), Hkv, D), dtype=np.float32), dtype))
        cmp_rows.append(_cast(rng.standard_normal((int(S2[b]) // cmp_ratio, Hkv, D), dtype=np.float32), dtype))
    sk = rng.standard_normal(H, dtype=np.float32) if sinks else None
    poison = POISON_BF16 if dtype == "bf16" else np.float16(POISON_F32)
    ori_kv, ori_table = _paged(rng, ori_rows, ori_bs, Hkv, D, dtype, poison)
    cmp_kv, cmp_table = _paged(rng, cmp_rows, cmp_bs, Hkv, D, dtype, poison)
    idx = np.zeros((T, Hkv, topk), np.int32)
    for b in range(B):
        S3 = int(S2[b]) // cmp_ratio
        s, e = int(cu_q[b]), int(cu_q[b + 1])
        if e == s or topk == 0:
            continue
        hi = max(S3, 1)
        if visible_indices:
            span = S3 - (e - s) + 1
            if span < topk:
                raise ValueError(f"sequence {b}: only {max(span, 0)} compressed keys visible to every row, topk {topk}")
            for c in range(Hkv):
                idx[s:e, c] = rng.choice(span, topk, replace=False)[None, :]
        elif shared_indices:
            idx[s:e] = rng.integers(0, hi, (1, Hkv, topk))
        else:
            idx[s:e] = rng.integers(0, hi, (e - s, Hkv, topk))
        if S3 == 0:
            idx[s:e] = -1
    if invalid_frac > 0 and topk > 0:
        bad = rng.random(idx.shape) < invalid_frac
        alt = rng.integers(0, 2, idx.shape)
        seq_of = np.repeat(np.arange(B), lens_q)
        s3 = (S2 // cmp_ratio)[seq_of][:, None, None]
        idx = np.where(bad, np.where(alt == 0, -1, s3 + rng.integers(0, 5, idx.shape)), idx).astype(np.int32)
    return dict(B=B, T=T, H=H, Hkv=Hkv, D=D, dtype=dtype, cu_q=cu_q, seqused_kv=S2.astype(np.int32),
                q=q, ori_kv=ori_kv, ori_table=ori_table, cmp_kv=cmp_kv, cmp_table=cmp_table, indices=idx,
                sinks=sk, window=tuple(window), topk=topk, cmp_ratio=cmp_ratio, cmp_all=bool(cmp_all),
                scale=(1.0 / math.sqrt(D)) if scale is None else scale,
                max_seqlen_kv=int(S2.max()) if B else 0)
