"""Pins for the oracle's ALiBi term (no GPU).

Reading: a per-head slope s_h adds -s_h * |i + Lk - Lq - j| to the scaled
score of query i and key j (the distance to the query's end-aligned
position, the alignment the causal mask uses); sinks are unaffected.

Closed forms: with q = 0 every score is the bias alone, so a row that sees
keys at distances 0..n has weights r^d (r = e^-s) and
  LSE = log((1 - r^(n+1)) / (1 - r)),
  sum_d d r^d / sum_d r^d = r (1 - (n+1) r^n + n r^(n+1)) / ((1 - r)(1 - r^(n+1))).
"""
import numpy as np
import pytest

import oracle
from oracle import brute
import workloads as W


def _zero_q_case(lens_q, lens_k, H, slopes, causal=True, window=(-1, -1), D=8):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    v = np.zeros((Tk, 1, D), np.float32)
    for b in range(len(lens_k)):
        v[cu_k[b]:cu_k[b + 1], 0, 0] = np.arange(lens_k[b])  # v[j, 0] = key position j
    return dict(B=len(lens_q), H=H, Hkv=1, D=D, dtype="f32", scale=1.0, causal=causal,
                window_left=window[0], window_right=window[1], T_q=Tq, T_k=Tk, cu_q=cu_q, cu_k=cu_k,
                paged=False, q=np.zeros((Tq, H, D), np.float32), k=np.ones((Tk, 1, D), np.float32),
                v=v, sinks=None, alibi=np.asarray(slopes, np.float32))


def _geometric(s, n):
    r = np.exp(-s)
    lse = np.log((1 - r ** (n + 1)) / (1 - r))
    mean_d = r * (1 - (n + 1) * r ** n + n * r ** (n + 1)) / ((1 - r) * (1 - r ** (n + 1)))
    return lse, mean_d


@pytest.mark.parametrize("lens", [([9], [9]), ([3, 5], [10, 5])])
def test_causal_zero_query_closed_form(lens):
    lq, lk = lens
    slopes = [0.5, 0.125]
    case = _zero_q_case(lq, lk, 2, slopes)
    out, lse = oracle.forward(case)
    for b in range(len(lq)):
        for i in range(lq[b]):
            t = int(case["cu_q"][b]) + i
            p = i + lk[b] - lq[b]  # keys 0..p at distances p..0
            for h, s in enumerate(np.asarray(slopes, np.float32).astype(np.float64)):
                want_lse, mean_d = _geometric(s, p)
                assert abs(lse[t, h] - want_lse) < 1e-12
                assert abs(out[t, h, 0] - (p - mean_d)) < 1e-11


def test_two_sided_window_is_symmetric_sum():
    # window (2, 2), no causal, Lq = Lk = 9: row 4 sees distances 0, 1, 1, 2, 2
    s = 0.75
    case = _zero_q_case([9], [9], 1, [s], causal=False, window=(2, 2))
    out, lse = oracle.forward(case)
    s = float(np.float32(s))
    want = np.log(1 + 2 * np.exp(-s) + 2 * np.exp(-2 * s))
    assert abs(lse[4, 0] - want) < 1e-12
    assert abs(out[4, 0, 0] - 4.0) < 1e-12  # symmetric weights around key 4


def test_zero_slopes_equal_no_alibi():
    case = W.make_case(W.scaled(W.config(2), B=3, max_len=150))
    ref_o, ref_l = oracle.forward(case)
    case["alibi"] = np.zeros(case["H"], np.float32)
    o, l = oracle.forward(case)
    np.testing.assert_array_equal(o, ref_o)
    np.testing.assert_array_equal(l, ref_l)


@pytest.mark.parametrize("n", [2, 4, 5])
def test_alibi_oracle_matches_dense_checker(n):
    spec = W.scaled(W.config(n), B=4 if n != 4 else 2, max_len=200)
    if n == 4:
        spec = W.Spec(**{**spec.__dict__, "H": 8})
    case = W.make_case(spec)
    case["alibi"] = (2.0 ** -np.arange(1, case["H"] + 1, dtype=np.float64) * 8 / case["H"]).astype(np.float32)
    out, lse = oracle.forward(case)
    out2, lse2 = brute.dense_forward(case)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    fin = np.isfinite(lse2)
    np.testing.assert_allclose(lse[fin], lse2[fin], rtol=0, atol=1e-12)
