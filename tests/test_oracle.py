"""Pins for the CPU oracle (no GPU).

The pages print no output values for this method, so the oracle is pinned to
things other than itself: hand-derived worked examples (tests/golden),
closed forms of special cases, exact counting tests for the mask, invariants
(GQA ratio 1, packing, paged addressing), an independent dense checker
(numpy + scipy.special.logsumexp) and PyTorch's CPU scaled_dot_product_attention
in float64.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, logsumexp

import oracle
from oracle import brute
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case_from_arrays(B, H, Hkv, D, q, k, v, cu_q, cu_k, scale, causal=False,
                      window=(-1, -1), sinks=None, dtype="f32"):
    cu_q = np.asarray(cu_q, np.int32)
    cu_k = np.asarray(cu_k, np.int32)
    return dict(B=B, H=H, Hkv=Hkv, D=D, dtype=dtype, scale=scale, causal=causal,
                window_left=window[0], window_right=window[1], T_q=int(cu_q[-1]),
                T_k=int(cu_k[-1]), cu_q=cu_q, cu_k=cu_k, paged=False,
                q=np.asarray(q, np.float32).reshape(int(cu_q[-1]), H, D),
                k=np.asarray(k, np.float32).reshape(int(cu_k[-1]), Hkv, D),
                v=np.asarray(v, np.float32).reshape(int(cu_k[-1]), Hkv, D),
                sinks=None if sinks is None else np.asarray(sinks, np.float32),
                lens_q=np.diff(cu_q), lens_k=np.diff(cu_k))


# --------------------------------------------------------------- worked examples
@pytest.mark.parametrize("name", ["gqa_causal", "window_sink_end_aligned"])
def test_hand_worked_examples(name):
    ex = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))[name]
    case = _case_from_arrays(ex["B"], ex["H"], ex["Hkv"], ex["D"], ex["q"], ex["k"], ex["v"],
                             ex["cu_q"], ex["cu_k"], ex["scale"], ex["causal"],
                             tuple(ex["window"]), ex["sinks"])
    for fn in (oracle.forward, brute.dense_forward):
        out, lse = fn(case)
        np.testing.assert_allclose(out, np.asarray(ex["out"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.asarray(ex["lse"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------- closed forms
def _random_causal(seed, lens, H=4, Hkv=2, D=16, scale=0.3):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    return _case_from_arrays(len(lens), H, Hkv, D, rng.standard_normal((T, H, D)),
                             rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D)),
                             cu, cu, scale, causal=True)


def test_single_key_rows_are_exact_value_rows():
    """Row 0 of a causal sequence sees one key: softmax weight 1, O = v_0,
    LSE = s_00."""
    case = _random_causal(1, [3, 7, 1])
    out, lse = oracle.forward(case)
    g = case["H"] // case["Hkv"]
    for b in range(case["B"]):
        t = case["cu_q"][b]
        for h in range(case["H"]):
            c = h // g
            np.testing.assert_array_equal(out[t, h], case["v"][t, c].astype(np.float64))
            s00 = case["scale"] * float(np.dot(case["q"][t, h].astype(np.float64),
                                              case["k"][t, c].astype(np.float64)))
            assert abs(lse[t, h] - s00) < 1e-12


def test_two_key_rows_closed_form():
    """Row 1 of a causal sequence: O = sigmoid(s0-s1) v0 + sigmoid(s1-s0) v1,
    LSE = log(e^s0 + e^s1)."""
    case = _random_causal(2, [4, 9])
    out, lse = oracle.forward(case)
    g = case["H"] // case["Hkv"]
    for b in range(case["B"]):
        t0 = case["cu_q"][b]
        t = t0 + 1
        for h in range(case["H"]):
            c = h // g
            qv = case["q"][t, h].astype(np.float64)
            s0 = case["scale"] * qv @ case["k"][t0, c].astype(np.float64)
            s1 = case["scale"] * qv @ case["k"][t0 + 1, c].astype(np.float64)
            expect = (expit(s0 - s1) * case["v"][t0, c] + expit(s1 - s0) * case["v"][t0 + 1, c])
            np.testing.assert_allclose(out[t, h], expect, rtol=0, atol=1e-12)
            assert abs(lse[t, h] - np.logaddexp(s0, s1)) < 1e-12


def test_identical_keys_give_uniform_weights():
    rng = np.random.default_rng(3)
    L, D = 11, 8
    k = np.tile(rng.standard_normal((1, 1, D)), (L, 1, 1))
    v = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((L, 1, D))
    case = _case_from_arrays(1, 1, 1, D, q, k, v, [0, L], [0, L], 0.7)
    out, lse = oracle.forward(case)
    vm = v.astype(np.float32).astype(np.float64)[:, 0].mean(0)
    np.testing.assert_allclose(out[:, 0], np.tile(vm, (L, 1)), atol=1e-12)
    s = 0.7 * (q.astype(np.float32).astype(np.float64)[:, 0] @ k.astype(np.float32).astype(np.float64)[0, 0])
    np.testing.assert_allclose(lse[:, 0], s + math.log(L), atol=1e-12)


# --------------------------------------------------------------- mask counting
def _counting_case(lens_q, lens_k, H, Hkv, causal, window, sinks=None, paged_bs=None, seed=0):
    """q == 0 so every allowed score is 0; v[j, c, 0] = j, v[j, c, 1] = c.
    Then LSE_i = ln |A(i)| (+ sink), O_i[0] = mean of A(i), O_i[1] = c."""
    D = 4
    lens_q, lens_k = list(lens_q), list(lens_k)
    B = len(lens_q)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    T_q, T_k = int(cu_q[-1]), int(cu_k[-1])
    q = np.zeros((T_q, H, D), np.float32)
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T_k, Hkv, D)).astype(np.float32)
    v = np.zeros((T_k, Hkv, D), np.float32)
    for b in range(B):
        for j in range(lens_k[b]):
            v[cu_k[b] + j, :, 0] = j
            v[cu_k[b] + j, :, 1] = np.arange(Hkv)
    case = _case_from_arrays(B, H, Hkv, D, q, k, v, cu_q, cu_k, 1.0, causal, window, sinks)
    if paged_bs:
        case = _to_paged(case, paged_bs, seed=seed + 17)
    return case


def _to_paged(case, bs, seed):
    """Scatter a contiguous case's K/V into a block cache with a random
    block permutation (memory layout only)."""
    rng = np.random.default_rng(seed)
    lens_k = np.diff(case["cu_k"])
    nblk = [(int(x) + bs - 1) // bs for x in lens_k]
    n = sum(nblk)
    perm = rng.permutation(n)
    Wd = max(max(nblk), 1)
    kc = np.full((n + 1, bs) + case["k"].shape[1:], 1e4, np.float32)
    vc = np.full((n + 1, bs) + case["v"].shape[1:], 1e4, np.float32)
    bt = np.full((case["B"], Wd), n, np.int32)
    off = 0
    for b in range(case["B"]):
        s = int(case["cu_k"][b])
        for t in range(nblk[b]):
            p = int(perm[off + t])
            bt[b, t] = p
            r0, r1 = t * bs, min(int(lens_k[b]), (t + 1) * bs)
            kc[p, : r1 - r0] = case["k"][s + r0:s + r1]
            vc[p, : r1 - r0] = case["v"][s + r0:s + r1]
        off += nblk[b]
    out = dict(case)
    for key in ("k", "v", "cu_k"):
        out.pop(key)
    out.update(paged=True, k_cache=kc, v_cache=vc, block_table=bt, block_size=bs,
               seqused_k=lens_k.astype(np.int32), num_blocks=n + 1)
    return out


def _check_counts(case, out, lse, lo_hi, sinks=None):
    g = case["H"] // case["Hkv"]
    for b in range(case["B"]):
        for i in range(int(case["lens_q"][b])):
            t = case["cu_q"][b] + i
            lo, hi = lo_hi(b, i)
            n = max(0, hi - lo + 1)
            for h in range(case["H"]):
                extra = 0.0 if sinks is None else math.exp(sinks[h])
                if n == 0 and sinks is None:
                    assert lse[t, h] == -np.inf
                    assert np.all(out[t, h] == 0)
                    continue
                assert abs(lse[t, h] - math.log(n + extra)) < 1e-12, (b, i, h)
                frac = n / (n + extra)
                mean = (lo + hi) / 2 if n else 0.0
                assert abs(out[t, h, 0] - mean * frac) < 1e-9, (b, i, h)
                assert abs(out[t, h, 1] - (h // g) * frac) < 1e-12, (b, i, h)


@pytest.mark.parametrize("paged", [None, 16])
def test_counting_causal_equal_lengths(paged):
    lens = [5, 1, 33, 0, 17]
    case = _counting_case(lens, lens, H=6, Hkv=3, causal=True, window=(-1, -1), paged_bs=paged)
    out, lse = oracle.forward(case)
    _check_counts(case, out, lse, lambda b, i: (0, i))  # |A| = i + 1


@pytest.mark.parametrize("paged", [None, 16])
def test_counting_end_aligned_causal_decode(paged):
    lq, lk = [1, 4, 3, 2], [9, 40, 2, 1]   # last two have more queries than keys
    case = _counting_case(lq, lk, H=4, Hkv=1, causal=True, window=(-1, -1), paged_bs=paged)
    out, lse = oracle.forward(case)
    # query i sits at key position i + Lk - Lq: keys 0 .. i + Lk - Lq
    _check_counts(case, out, lse, lambda b, i: (0, min(lk[b] - 1, i + lk[b] - lq[b])))


def test_counting_sliding_window_127_0():
    lens = [300, 128, 7]
    case = _counting_case(lens, lens, H=2, Hkv=1, causal=False, window=(127, 0))
    out, lse = oracle.forward(case)
    _check_counts(case, out, lse, lambda b, i: (max(0, i - 127), i))  # min(i,127)+1 keys


def test_counting_two_sided_window_and_full():
    lens = [50, 20]
    case = _counting_case(lens, lens, H=2, Hkv=2, causal=False, window=(3, 5))
    out, lse = oracle.forward(case)
    _check_counts(case, out, lse, lambda b, i: (max(0, i - 3), min(lens[b] - 1, i + 5)))
    case = _counting_case(lens, [60, 5], H=2, Hkv=2, causal=False, window=(-1, -1))
    out, lse = oracle.forward(case)
    _check_counts(case, out, lse, lambda b, i: (0, [60, 5][b] - 1))


def test_counting_causal_with_window():
    lens = [40]
    case = _counting_case(lens, lens, H=1, Hkv=1, causal=True, window=(4, 9))
    out, lse = oracle.forward(case)
    _check_counts(case, out, lse, lambda b, i: (max(0, i - 4), i))  # causal clips the right side


def test_counting_with_sinks():
    lq, lk = [6, 3], [6, 1]
    sinks = [0.5, -1.25, 2.0, 0.0]
    case = _counting_case(lq, lk, H=4, Hkv=2, causal=True, window=(-1, -1), sinks=sinks)
    out, lse = oracle.forward(case)
    # includes sink-only rows (second sequence, rows 0 and 1): O = 0, LSE = sigma
    _check_counts(case, out, lse, lambda b, i: (0, min(lk[b] - 1, i + lk[b] - lq[b])), sinks)
    assert lse[6, 1] == pytest.approx(-1.25, abs=1e-15)


def test_sink_minus_infinity_reduces_to_no_sink():
    case = _random_causal(5, [6, 13])
    base_out, base_lse = oracle.forward(case)
    case2 = dict(case, sinks=np.full(case["H"], -np.inf, np.float32))
    out, lse = oracle.forward(case2)
    np.testing.assert_array_equal(out, base_out)
    np.testing.assert_array_equal(lse, base_lse)


# --------------------------------------------------------------- brute force
def _sweep_cases():
    rng = np.random.default_rng(77)
    cases = []
    for n in range(14):
        g = [1, 2, 4, 8, 64][n % 5]
        Hkv = 1 if g == 64 else int(rng.integers(1, 3))
        H = g * Hkv
        D = [64, 128][n % 2]
        B = int(rng.integers(1, 5))
        lq = [int(x) for x in rng.choice([0, 1, 2, 3, 7, 31, 64, 65, 129], size=B)]
        decode = n % 3 == 0
        lk = [int(x) + (int(rng.integers(0, 90)) if decode else 0) for x in lq]
        kinds = [(True, (-1, -1)), (False, (-1, -1)), (False, (127, 0)), (True, (8, 3)),
                 (False, (2, 6))]
        causal, window = kinds[n % len(kinds)]
        sinks = (n % 2 == 1)
        spec = W.Spec(f"sweep{n}", 5000 + n, "bf16" if n % 4 else "f32", H, Hkv, D,
                      ("fixed", lq), causal=causal, window=window, sinks=sinks,
                      paged=(n % 4 == 2), block_size=[16, 64][n % 2])
        cases.append(W.make_case(spec, lens_q=lq, lens_k=lk))
    return cases


def test_oracle_matches_dense_bruteforce_tiny_f32_causal_gqa():
    case = W.make_case(W.config(1))
    out, lse = oracle.forward(case)
    out2, lse2 = brute.dense_forward(case)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_oracle_matches_dense_bruteforce_scaled_configs(n):
    spec = W.scaled(W.config(n), B=6 if n != 4 else 3, max_len=300)
    if n == 4:
        spec = W.Spec(**{**spec.__dict__, "H": 8})  # fewer heads, same MQA + window + sinks
    case = W.make_case(spec)
    out, lse = oracle.forward(case)
    out2, lse2 = brute.dense_forward(case)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_half_widening_matches_numpy_on_every_bit_pattern():
    # binary16 inputs: the oracle's widening against numpy's float16 -> float64
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.half_to_double(bits)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan]))


@pytest.mark.parametrize("n", [2, 4, 5])
def test_oracle_matches_dense_bruteforce_f16(n):
    # the same workloads in float16 (numpy's round-to-nearest-even cast)
    spec = W.scaled(W.config(n), B=4 if n != 4 else 2, max_len=200)
    spec = W.Spec(**{**spec.__dict__, "dtype": "f16", "name": spec.name + "_f16",
                     **({"H": 8} if n == 4 else {})})
    case = W.make_case(spec)
    assert case["q"].dtype == np.float16
    out, lse = oracle.forward(case)
    out2, lse2 = brute.dense_forward(case)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("idx", range(14))
def test_oracle_matches_dense_bruteforce_sweep(idx):
    case = _sweep_cases()[idx]
    out, lse = oracle.forward(case)
    out2, lse2 = brute.dense_forward(case)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lse2))
    fin = np.isfinite(lse2)
    np.testing.assert_allclose(lse[fin], lse2[fin], rtol=0, atol=1e-12)


def test_probability_rows_sum_to_one_minus_sink_share():
    spec = W.Spec("rows", 4242, "f32", 4, 1, 32, ("fixed", [40, 9]), causal=False,
                  window=(5, 2), sinks=True)
    case = W.make_case(spec)
    out, lse, probs = brute.dense_forward(case, return_probs=True)
    for (b, h), P in probs.items():
        s = int(case["cu_q"][b])
        # the last column is the sink: keys alone carry 1 - e^{sigma - LSE}
        np.testing.assert_allclose(P[:, :-1].sum(1), 1 - np.exp(case["sinks"][h] - lse[s:s + P.shape[0], h]),
                                   atol=1e-12)
        np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-12)
    o1, l1 = oracle.forward(case)
    np.testing.assert_allclose(o1, out, atol=1e-12)
    # LSE equals logsumexp of the masked scores together with the sink
    np.testing.assert_allclose(l1, lse, atol=1e-12)


# --------------------------------------------------------------- invariants
def test_gqa_equals_mha_with_repeated_kv_heads():
    spec = W.Spec("gqa", 31, "bf16", 8, 2, 64, ("fixed", [19, 70, 3]), causal=True, sinks=True)
    case = W.make_case(spec)
    out, lse = oracle.forward(case)
    g = case["H"] // case["Hkv"]
    mha = dict(case, Hkv=case["H"], k=np.repeat(case["k"], g, axis=1),
               v=np.repeat(case["v"], g, axis=1))
    out2, lse2 = oracle.forward(mha)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def _subcase(case, order):
    """Re-pack a contiguous case with sequences in the given order."""
    qs, ks, vs, lq, lk = [], [], [], [], []
    for b in order:
        qs.append(case["q"][case["cu_q"][b]:case["cu_q"][b + 1]])
        ks.append(case["k"][case["cu_k"][b]:case["cu_k"][b + 1]])
        vs.append(case["v"][case["cu_k"][b]:case["cu_k"][b + 1]])
        lq.append(int(case["lens_q"][b]))
        lk.append(int(case["lens_k"][b]))
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    return dict(case, B=len(order), q=np.concatenate(qs), k=np.concatenate(ks),
                v=np.concatenate(vs), cu_q=cu_q, cu_k=cu_k, T_q=int(cu_q[-1]),
                T_k=int(cu_k[-1]), lens_q=np.asarray(lq), lens_k=np.asarray(lk))


def test_packing_order_and_single_sequence_invariance():
    spec = W.Spec("pack", 9, "bf16", 4, 2, 64, ("fixed", [12, 0, 33, 5]),
                  lens_k=("uniform", 30, 40), causal=True, window=(20, -1))
    case = W.make_case(spec)
    out, lse = oracle.forward(case)
    order = [2, 0, 3, 1]
    perm = _subcase(case, order)
    out_p, lse_p = oracle.forward(perm)
    for new_b, b in enumerate(order):
        s, e = case["cu_q"][b], case["cu_q"][b + 1]
        s2, e2 = perm["cu_q"][new_b], perm["cu_q"][new_b + 1]
        np.testing.assert_array_equal(out[s:e], out_p[s2:e2])
        np.testing.assert_array_equal(lse[s:e], lse_p[s2:e2])
        one = _subcase(case, [b])
        o1, l1 = oracle.forward(one)
        np.testing.assert_array_equal(out[s:e], o1)
        np.testing.assert_array_equal(lse[s:e], l1)


def test_paged_addressing_equals_contiguous():
    spec = W.scaled(W.config(5), B=5, max_len=200)
    case = W.make_case(spec)
    out, lse = oracle.forward(case)
    k, v, cu_k = W.paged_to_contiguous(case)
    cont = dict(case, paged=False, k=k, v=v, cu_k=cu_k)
    out2, lse2 = oracle.forward(cont)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)
    # another physical arrangement of the same logical cache
    case3 = _to_paged(dict(cont, q=W.bf16_bits_to_f32(case["q"]), k=W.bf16_bits_to_f32(k),
                           v=W.bf16_bits_to_f32(v), dtype="f32"),
                      case["block_size"], seed=123)
    out3, lse3 = oracle.forward(case3)
    np.testing.assert_array_equal(out, out3)
    np.testing.assert_array_equal(lse, lse3)


def test_rows_mode_matches_full_mode():
    spec = W.scaled(W.config(2), B=4, max_len=150)
    case = W.make_case(spec)
    out, lse = oracle.forward(case)
    rng = np.random.default_rng(0)
    toks = rng.integers(0, case["T_q"], 40)
    heads = rng.integers(0, case["H"], 40)
    o, l = oracle.forward_rows(case, toks, heads)
    np.testing.assert_array_equal(o, out[toks, heads])
    np.testing.assert_array_equal(l, lse[toks, heads])


# --------------------------------------------------------------- library special case
def test_matches_torch_sdpa_float64_without_sinks():
    torch = pytest.importorskip("torch")
    spec = W.Spec("sdpa", 55, "bf16", 6, 3, 64, ("fixed", [17, 40]), lens_k=("uniform", 40, 50),
                  causal=True)
    case = W.make_case(spec)
    out, _ = oracle.forward(case)
    g = case["H"] // case["Hkv"]
    q = torch.from_numpy(W.bf16_bits_to_f32(case["q"]).astype(np.float64))
    k = torch.from_numpy(W.bf16_bits_to_f32(case["k"]).astype(np.float64))
    v = torch.from_numpy(W.bf16_bits_to_f32(case["v"]).astype(np.float64))
    for b in range(case["B"]):
        s, e = case["cu_q"][b], case["cu_q"][b + 1]
        ks, ke = case["cu_k"][b], case["cu_k"][b + 1]
        Lq, Lk = e - s, ke - ks
        m = torch.from_numpy(brute.mask(Lq, Lk, True, -1, -1))
        qb = q[s:e].transpose(0, 1)
        kb = k[ks:ke].repeat_interleave(g, dim=1).transpose(0, 1)
        vb = v[ks:ke].repeat_interleave(g, dim=1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=m,
                                                               scale=case["scale"])
        np.testing.assert_allclose(out[s:e], ref.transpose(0, 1).numpy(), atol=1e-12)


# --------------------------------------------------------------- generator
def test_generator_reproduces_seeded_lengths():
    rng = np.random.default_rng(1002)
    lens = rng.integers(128, 4096, size=16, endpoint=True)
    assert list(lens) == [2528, 1639, 3210, 1545, 3678, 3095, 2556, 1673, 3166, 1466, 362,
                          2330, 1551, 871, 3509, 602]
    assert int(lens.sum()) == 33781
    case1 = W.make_case(W.config(1))
    assert case1["q"].shape == (54, 4, 64) and case1["k"].shape == (54, 2, 64)
    assert W.case_digest(case1) == W.case_digest(W.make_case(W.config(1)))


def test_oracle_rejects_indivisible_heads():
    case = _random_causal(9, [3], H=3, Hkv=2)
    with pytest.raises(ValueError):
        oracle.forward(case)
