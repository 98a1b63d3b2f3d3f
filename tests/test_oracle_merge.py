"""Pins for the oracle's log-sum-exp merge (no GPU).

The merge is pinned to the (separately pinned) forward oracle through the
identity that defines it: attention over a union of disjoint key sets
equals the merge of the attentions over each set, with a sink counted
once.  Closed forms cover a single part, empty parts and sink-only rows.
"""
import numpy as np
import pytest

import oracle


def _case(lens_q, lens_k, H, Hkv, D, sinks=None, seed=0, scale=0.35):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    return dict(B=len(lens_q), H=H, Hkv=Hkv, D=D, dtype="f32", scale=scale, causal=False,
                window_left=-1, window_right=-1, T_q=Tq, T_k=Tk, cu_q=cu_q, cu_k=cu_k, paged=False,
                q=rng.standard_normal((Tq, H, D)).astype(np.float32),
                k=rng.standard_normal((Tk, Hkv, D)).astype(np.float32),
                v=rng.standard_normal((Tk, Hkv, D)).astype(np.float32),
                sinks=None if sinks is None else np.asarray(sinks, np.float32))


def _key_subset(case, cuts):
    """Cases with the same queries and, per sequence b, the keys
    [cuts[b][p], cuts[b][p+1]) of that sequence (part p)."""
    parts = []
    for p in range(len(cuts[0]) - 1):
        ks, lens = [], []
        for b in range(case["B"]):
            k0 = int(case["cu_k"][b])
            a, z = cuts[b][p], cuts[b][p + 1]
            ks.append(np.arange(k0 + a, k0 + z))
            lens.append(z - a)
        idx = np.concatenate(ks).astype(np.int64)
        c = dict(case)
        c["cu_k"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        c["T_k"] = int(c["cu_k"][-1])
        c["k"], c["v"] = case["k"][idx], case["v"][idx]
        c["sinks"] = None
        parts.append(c)
    return parts


PARTITIONS = {
    # (lens_q, lens_k, H, Hkv, D, per-sequence cut points)
    "two_even_halves": ([5, 3], [8, 6], 2, 2, 8, [[0, 4, 8], [0, 3, 6]]),
    "three_uneven_gqa": ([4, 6, 1], [9, 5, 7], 4, 2, 8, [[0, 1, 7, 9], [0, 5, 5, 5], [0, 0, 3, 7]]),
    "mqa_with_empty_parts": ([3, 2], [4, 6], 4, 1, 16, [[0, 0, 4, 4], [0, 6, 6, 6]]),
}


@pytest.mark.parametrize("sinks", [False, True])
@pytest.mark.parametrize("name", list(PARTITIONS))
def test_merge_of_key_partition_equals_attention_over_all_keys(name, sinks):
    lens_q, lens_k, H, Hkv, D, cuts = PARTITIONS[name]
    sk = np.linspace(-1.0, 1.5, H) if sinks else None
    case = _case(lens_q, lens_k, H, Hkv, D, sinks=sk, seed=len(name))
    want_o, want_l = oracle.forward(case, nthreads=2)
    outs = [oracle.forward(c, nthreads=2) for c in _key_subset(case, cuts)]
    o_parts = np.stack([o for o, _ in outs])
    l_parts = np.stack([l for _, l in outs])
    got_o, got_l = oracle.merge(o_parts, l_parts, case["sinks"])
    np.testing.assert_allclose(got_o, want_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got_l, want_l, rtol=0, atol=1e-12)


def test_single_part_without_sinks_is_identity():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((1, 5, 3, 8))
    lse = rng.standard_normal((1, 5, 3))
    got_o, got_l = oracle.merge(o, lse)
    np.testing.assert_array_equal(got_o, o[0])
    np.testing.assert_array_equal(got_l, lse[0])


def test_empty_parts_contribute_nothing():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((3, 4, 2, 8)) * 1e3  # finite values in the empty parts
    lse = rng.standard_normal((3, 4, 2))
    lse[1] = -np.inf
    got_o, got_l = oracle.merge(o, lse)
    ref_o, ref_l = oracle.merge(o[[0, 2]], lse[[0, 2]])
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got_l, ref_l, rtol=0, atol=1e-12)


def test_rows_with_nothing_and_sink_only_rows():
    o = np.ones((2, 2, 2, 8))
    lse = np.full((2, 2, 2), -np.inf)
    got_o, got_l = oracle.merge(o, lse)
    assert np.all(got_o == 0) and np.all(got_l == -np.inf)
    got_o, got_l = oracle.merge(o, lse, sinks=[0.25, -3.0])
    assert np.all(got_o == 0)
    np.testing.assert_array_equal(got_l, np.array([[0.25, -3.0], [0.25, -3.0]]))


def test_two_equal_parts_closed_form():
    # equal lse: weights 1/2 each and lse + log 2
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 3, 2, 8))
    lse = np.full((2, 3, 2), 0.7)
    got_o, got_l = oracle.merge(o, lse)
    np.testing.assert_allclose(got_o, 0.5 * (o[0] + o[1]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(got_l, 0.7 + np.log(2.0), rtol=0, atol=1e-14)
