"""Pins for the compressed-key part of the shared-KV oracle (no GPU): the
SparseAttnSharedkv README's second scenario (sliding window + every
compressed key the mask admits) and the compressed-key mask in the third.

Reading pinned here: sequence b has S3_b = S2_b / cmp_ratio compressed
keys, and query row i sees compressed position t iff t <= i + S3_b - Lq_b
(cmp_mask_mode 3: causal, aligned to the bottom-right of the Lq x S3
matrix; the README's example draws its indices from [0, S3 - Lq], the
positions every row sees).

* The window keys and the compressed keys are disjoint key sets, so the
  second scenario equals the log-sum-exp merge (oracle.merge) of window
  attention over the original cache and end-aligned causal attention over
  the compressed cache, both from the forward oracle, the sink counted once.
* Selecting every position in the third scenario equals the second one
  (the mask drops what a row cannot see).
* An index beyond a row's last visible position is the same as no index.
* With q = 0 every logit is 0: with constant original and compressed rows
  the output and LSE follow from the counts of visible keys (closed form).
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _paged_forward(sc, cache, table, seqused, window, causal):
    lens_q = np.diff(sc["cu_q"])
    return dict(B=sc["B"], H=sc["H"], Hkv=sc["Hkv"], D=sc["D"], dtype=sc["dtype"], scale=sc["scale"],
                causal=causal, window_left=window[0], window_right=window[1], T_q=sc["T"], cu_q=sc["cu_q"],
                max_q=int(lens_q.max()), max_k=int(max(int(x) for x in seqused)), q=sc["q"], paged=True,
                k_cache=cache, v_cache=cache, block_table=table, seqused_k=np.asarray(seqused, np.int32),
                block_size=cache.shape[1], num_blocks=cache.shape[0], sinks=None)


@pytest.mark.parametrize("ratio,lens_q,s2,window,sinks,dtype,D", [
    (4, [5, 40, 1, 16], [64, 200, 37, 16], (7, 0), True, "bf16", 64),
    (4, [128, 3], [512, 90], (127, 0), True, "bf16", 128),      # the README's window; S3 < Lq rows
    (1, [9, 30], [9, 45], (2, 1), False, "f16", 64),
    (128, [3, 5], [300, 1000], (4, 0), True, "bf16", 64),        # the README's other ratio
    (4, [6, 2], [20, 3], (0, 0), True, "bf16", 512),              # S3 = 0 for one sequence
])
def test_second_scenario_is_merge_of_window_and_causal_compressed(ratio, lens_q, s2, window, sinks, dtype, D):
    sc = W.sparse_case(lens_q, s2, H=8, Hkv=2, D=D, dtype=dtype, window=window, topk=0, cmp_ratio=ratio,
                       ori_bs=16, cmp_bs=16, sinks=sinks, seed=4700 + ratio, cmp_all=True)
    got_o, got_l = oracle.sparse_sharedkv(sc)
    s3 = [int(x) // ratio for x in sc["seqused_kv"]]
    win_o, win_l = oracle.forward(_paged_forward(sc, sc["ori_kv"], sc["ori_table"], sc["seqused_kv"], window,
                                                 causal=False))
    cmp_o, cmp_l = oracle.forward(_paged_forward(sc, sc["cmp_kv"], sc["cmp_table"], s3, (-1, -1), causal=True))
    ref_o, ref_l = oracle.merge(np.stack([win_o, cmp_o]), np.stack([win_l, cmp_l]), sc["sinks"])
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=0, atol=1e-12)


def test_selecting_every_position_is_the_second_scenario():
    kw = dict(H=4, Hkv=2, D=64, window=(5, 0), cmp_ratio=4, ori_bs=16, cmp_bs=16, seed=4800)
    all_ = W.sparse_case([7, 12], [80, 60], topk=0, cmp_all=True, **kw)
    S3max = int(max(all_["seqused_kv"])) // 4
    sel = dict(all_, cmp_all=False, topk=S3max,
               indices=np.broadcast_to(np.arange(S3max, dtype=np.int32), (all_["T"], 2, S3max)).copy())
    o1, l1 = oracle.sparse_sharedkv(all_)
    o2, l2 = oracle.sparse_sharedkv(sel)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_index_beyond_the_last_visible_position_is_absent():
    sc = W.sparse_case([6, 3], [64, 90], H=4, Hkv=2, D=64, window=(7, 0), topk=4, cmp_ratio=4, ori_bs=16,
                       cmp_bs=16, seed=4900, visible_indices=True)
    cu = sc["cu_q"]
    extra = np.empty((sc["T"], 2, 1), np.int32)
    inside = 0
    for b in range(sc["B"]):
        S3, Lq = int(sc["seqused_kv"][b]) // 4, int(cu[b + 1] - cu[b])
        for i in range(Lq):
            # one past the row's last visible position: below S3 except on
            # the last row, which sees every compressed key
            extra[cu[b] + i] = i + S3 - Lq + 1
            inside += i + S3 - Lq + 1 < S3
    assert inside == sc["T"] - sc["B"]
    padded = dict(sc, indices=np.concatenate([sc["indices"], extra], axis=2), topk=5)
    o1, l1 = oracle.sparse_sharedkv(sc)
    o2, l2 = oracle.sparse_sharedkv(padded)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_second_scenario_counts_closed_form():
    ratio, window = 4, (9, 2)
    sc = W.sparse_case([20, 5], [100, 12], H=2, Hkv=1, D=64, dtype="bf16", window=window, topk=0,
                       cmp_ratio=ratio, ori_bs=16, cmp_bs=16, sinks=True, seed=5000, cmp_all=True)
    sc["q"] = np.zeros_like(sc["q"])
    a, c = 0.5, 2.0  # exact in bf16: every original row a, every compressed row c
    sc["ori_kv"] = np.full_like(sc["ori_kv"], W.f32_to_bf16_bits(np.float32(a)))
    sc["cmp_kv"] = np.full_like(sc["cmp_kv"], W.f32_to_bf16_bits(np.float32(c)))
    out, lse = oracle.sparse_sharedkv(sc)
    cu = sc["cu_q"]
    for b in range(sc["B"]):
        S2, Lq = int(sc["seqused_kv"][b]), int(cu[b + 1] - cu[b])
        S3 = S2 // ratio
        for i in range(Lq):
            p = i + S2 - Lq
            n_win = min(S2 - 1, p + window[1]) - max(0, p - window[0]) + 1
            n_cmp = min(S3, max(0, i + S3 - Lq + 1))
            for h in range(2):
                z = n_win + n_cmp + np.exp(float(sc["sinks"][h]))
                assert abs(lse[cu[b] + i, h] - np.log(z)) < 1e-12
                np.testing.assert_allclose(out[cu[b] + i, h], (n_win * a + n_cmp * c) / z, rtol=0, atol=1e-12)
