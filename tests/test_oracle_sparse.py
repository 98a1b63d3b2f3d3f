"""Pins for the oracle of sliding-window + sparse compressed attention over
shared K/V (no GPU).

Pinned to the (separately pinned) forward oracle through identities of the
definition: with no selected keys it is window attention with K = V = the
original cache; when the compressed cache is the original cache (ratio 1)
and the indices select every key before the window, window + selection is
full causal attention; out-of-range indices are the same as absent ones;
with q = 0 every key weighs the same, so a repeated index doubles its
row's weight (closed form).
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _forward_case(sc, window, causal):
    """The same queries and original cache as a paged forward case (K = V)."""
    lens_q = np.diff(sc["cu_q"])
    return dict(B=sc["B"], H=sc["H"], Hkv=sc["Hkv"], D=sc["D"], dtype=sc["dtype"], scale=sc["scale"],
                causal=causal, window_left=window[0], window_right=window[1], T_q=sc["T"], cu_q=sc["cu_q"],
                max_q=int(lens_q.max()), max_k=sc["max_seqlen_kv"], q=sc["q"], paged=True,
                k_cache=sc["ori_kv"], v_cache=sc["ori_kv"], block_table=sc["ori_table"],
                seqused_k=sc["seqused_kv"], block_size=sc["ori_kv"].shape[1],
                num_blocks=sc["ori_kv"].shape[0], sinks=sc["sinks"])


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f16", 64), ("bf16", 512)])
def test_no_selection_is_window_attention(dtype, D):
    sc = W.sparse_case([5, 0, 9, 1], [40, 3, 200, 130], H=8, Hkv=2, D=D, dtype=dtype, window=(17, 3),
                       topk=0, ori_bs=32, cmp_bs=16, seed=4100)
    got_o, got_l = oracle.sparse_sharedkv(sc)
    ref_o, ref_l = oracle.forward(_forward_case(sc, (17, 3), causal=False))
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=0, atol=1e-12)


def test_window_plus_all_earlier_keys_is_causal_attention():
    w = 5
    sc = W.sparse_case([6, 4], [30, 25], H=4, Hkv=1, D=64, window=(w, 0), topk=0, cmp_ratio=1,
                       ori_bs=16, cmp_bs=16, sinks=True, seed=4200)
    # the compressed cache is the original one: select every key before the window
    sc["cmp_kv"], sc["cmp_table"] = sc["ori_kv"], sc["ori_table"]
    cu_q = sc["cu_q"]
    topk = int(max(sc["seqused_kv"])) - w
    idx = np.full((sc["T"], 1, topk), -1, np.int32)
    for b in range(sc["B"]):
        S2, Lq = int(sc["seqused_kv"][b]), int(cu_q[b + 1] - cu_q[b])
        for i in range(Lq):
            p = i + S2 - Lq
            before = np.arange(0, max(0, p - w))
            idx[cu_q[b] + i, 0, : len(before)] = before
    sc["indices"], sc["topk"] = idx, topk
    got_o, got_l = oracle.sparse_sharedkv(sc)
    ref_o, ref_l = oracle.forward(_forward_case(sc, (-1, -1), causal=True))
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got_l, ref_l, rtol=0, atol=1e-12)


def test_out_of_range_indices_are_absent():
    sc = W.sparse_case([4, 3], [64, 90], H=4, Hkv=2, D=64, window=(7, 0), topk=6, cmp_ratio=4,
                       ori_bs=16, cmp_bs=16, seed=4300)
    padded = dict(sc)
    S3 = (sc["seqused_kv"] // 4)
    extra = np.empty((sc["T"], 2, 3), np.int32)
    extra[..., 0] = -1
    extra[..., 1] = np.repeat(S3, np.diff(sc["cu_q"]))[:, None]       # == S3: out of range
    extra[..., 2] = -7
    padded["indices"] = np.concatenate([sc["indices"], extra], axis=2)
    padded["topk"] = 9
    o1, l1 = oracle.sparse_sharedkv(sc)
    o2, l2 = oracle.sparse_sharedkv(padded)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_repeated_index_closed_form():
    # q = 0: every logit is 0, so each occurrence of a key weighs 1 / count
    sc = W.sparse_case([1], [64], H=2, Hkv=1, D=64, dtype="f16", window=(3, 0), topk=4, cmp_ratio=4,
                       ori_bs=16, cmp_bs=16, sinks=False, seed=4400)
    sc["q"] = np.zeros_like(sc["q"])
    sc["indices"][0, 0] = [2, 2, 2, 5]
    out, lse = oracle.sparse_sharedkv(sc)
    ori = [sc["ori_kv"][sc["ori_table"][0, pos // 16], pos % 16, 0].astype(np.float64) for pos in range(60, 64)]
    cmp_ = [sc["cmp_kv"][sc["cmp_table"][0, j // 16], j % 16, 0].astype(np.float64) for j in (2, 2, 2, 5)]
    want = (np.sum(ori, axis=0) + np.sum(cmp_, axis=0)) / 8
    for h in range(2):
        np.testing.assert_allclose(out[0, h], want, rtol=0, atol=1e-12)
        assert abs(lse[0, h] - np.log(8.0)) < 1e-12
