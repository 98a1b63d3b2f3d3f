"""Host logic of the benchmark (no GPU): the mask-adjusted FLOP count behind
the headline metric, checked against brute-force counting of allowed
(query, key) pairs and against closed forms, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lengths_case(lens_q, lens_k, causal=False, window=(-1, -1), paged=False):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    c = dict(B=len(lens_q), H=4, D=64, cu_q=cu_q, cu_k=cu_k, T_q=int(cu_q[-1]), T_k=int(cu_k[-1]),
             causal=causal, window_left=window[0], window_right=window[1], paged=paged)
    if paged:
        c["seqused_k"] = np.asarray(lens_k, np.int32)
    return c


def _brute_pairs(case):
    """Allowed pairs per query row by testing every (row, key): key j of a
    sequence is allowed for row i (p = i + Lk - Lq) iff j <= p when causal,
    p - left <= j when left >= 0 and j <= p + right when right >= 0."""
    lens_q = np.diff(case["cu_q"])
    lens_k = case["seqused_k"] if case["paged"] else np.diff(case["cu_k"])
    wl, wr = case["window_left"], case["window_right"]
    out = []
    for Lq, Lk in zip(lens_q, lens_k):
        for i in range(Lq):
            p = i + Lk - Lq
            n = 0
            for j in range(Lk):
                ok = (not case["causal"] or j <= p) and (wl < 0 or j >= p - wl) and (wr < 0 or j <= p + wr)
                n += ok
            out.append(n)
    return np.asarray(out, np.int64)


@pytest.mark.parametrize("lens_q,lens_k,causal,window,paged", [
    ([5, 17, 32], [5, 17, 32], True, (-1, -1), False),
    ([7, 0, 40], [3, 9, 40], True, (-1, -1), False),        # more queries than keys; empty sequence
    ([30, 12], [50, 12], False, (6, 2), False),              # two-sided window
    ([30, 12], [50, 12], True, (6, 4), False),               # causal caps the right side
    ([1, 2, 3], [100, 40, 1], True, (-1, -1), True),         # decode-like, paged lengths
    ([25], [25], False, (-1, 0), False),                     # right = 0 without causal
])
def test_visible_pairs_equal_brute_force(lens_q, lens_k, causal, window, paged):
    case = _lengths_case(lens_q, lens_k, causal, window, paged)
    np.testing.assert_array_equal(bench.visible_pairs(case), _brute_pairs(case))


def test_flops_closed_forms():
    L = 1000
    full = _lengths_case([L], [L])
    causal = _lengths_case([L], [L], causal=True)
    win = _lengths_case([L], [L], window=(127, 0))
    assert bench.flops(full) == 4 * 64 * 4 * L * L
    assert bench.flops(causal) == 4 * 64 * 4 * L * (L + 1) // 2
    assert bench.flops(win) == 4 * 64 * 4 * sum(min(i + 1, 128) for i in range(L))


def test_flops_of_the_causal_gqa_prefill_workload():
    """16 sequences, causal, q = kv lengths: 4 D H sum L (L + 1) / 2."""
    case = W.make_case(W.config(2), poison=False)
    lens = np.diff(case["cu_q"]).astype(np.int64)
    assert bench.flops(case) == 4 * 128 * 32 * int(np.sum(lens * (lens + 1) // 2))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_price_16_bit_types_alike():
    """bf16 and fp16 elements are 2 bytes each, float32 4: the byte count of
    a workload depends only on the element size."""
    case = _lengths_case([5, 17, 32], [5, 17, 32], causal=True)
    case.update(Hkv=2, dtype="bf16")
    b16 = bench.alg_bytes(case)
    assert bench.alg_bytes(dict(case, dtype="f16")) == b16
    T, H, Hkv, D = case["T_q"], case["H"], 2, case["D"]
    expect16 = 2.0 * T * H * D * 2 + 4.0 * T * H + 2.0 * case["T_k"] * Hkv * D * 2 + 8.0 * (case["B"] + 1)
    assert b16 == expect16
    expect32 = 2.0 * T * H * D * 4 + 4.0 * T * H + 2.0 * case["T_k"] * Hkv * D * 4 + 8.0 * (case["B"] + 1)
    assert bench.alg_bytes(dict(case, dtype="f32")) == expect32


def test_sparse_work_counts_masked_keys_by_hand():
    # one sequence of 2 rows over 8 original keys, ratio 2 (4 compressed),
    # window (1, 0): row i sits at p = i + 6 and sees originals {5, 6} / {6, 7}
    # and compressed positions up to i + 4 - 2, i.e. {0..2} / {0..3}
    base = dict(lens_q=[2], seqused_kv=[8], H=4, Hkv=2, D=64, window=(1, 0), cmp_ratio=2, ori_bs=4, cmp_bs=4,
                seed=1)
    sc = W.sparse_case(**base, topk=0, cmp_all=True)
    fl, by = bench.sparse_work(sc)
    g, D, T, H = 2, 64, 2, 4
    keys = 2 * (4 + 7)                     # per kv head: 4 window + 7 compressed
    assert fl == 4.0 * D * g * keys
    rows = 2 * (3 + 4)                     # distinct originals {5, 6, 7}, compressed {0..3}
    tables = sc["ori_table"].size + sc["cmp_table"].size
    assert by == 2.0 * T * H * D * 2 + 4.0 * T * H + 4.0 * tables + rows * D * 2
    # indices: 3 for row 0 (one past its bound), 3 for row 1 (one invalid)
    sc = W.sparse_case(**base, topk=3)
    sc["indices"][0] = [[0, 3, 2], [1, 1, 0]]
    sc["indices"][1] = [[3, -1, 3], [4, 2, 0]]
    fl, by = bench.sparse_work(sc)
    # per kv head 0: row 0 {0, 2}, row 1 {3, 3}; kv head 1: row 0 {1, 1, 0}, row 1 {2, 0}
    keys = 2 * 4 + (2 + 2) + (3 + 2)
    assert fl == 4.0 * D * g * keys
    rows = 2 * 3 + len({0, 2, 3}) + len({0, 1, 2})
    assert by == 2.0 * T * H * D * 2 + 4.0 * T * H + 4.0 * sc["indices"].size + 4.0 * tables + rows * D * 2
