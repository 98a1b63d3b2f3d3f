"""Pins for the oracle's sink-logit gradient (no GPU).

dsinks_h is checked against central finite differences of the forward
oracle: L(s) = sum(dout * O(s)) with the sink of head h moved up and down
(by the float32-rounded steps the oracle actually receives), for causal,
windowed and end-aligned cases, with GQA; and against the closed form of a
row whose only logit besides the sink is one key: O = w v, w = e^x / (e^x +
e^s), so dL/ds = -w (1 - w) (dout . v).
"""
import copy

import numpy as np
import pytest

import oracle
import workloads as W


def _loss_and_grad(case, dout):
    out, lse = oracle.forward(case)
    return float(np.sum(dout * out)), oracle.sink_grad(case, dout, out, lse)


@pytest.mark.parametrize("causal,window,lens_k", [(True, (-1, -1), None), (False, (5, 3), None),
                                                   (True, (-1, -1), [30, 12, 9])])
def test_sink_grad_matches_finite_differences(causal, window, lens_k):
    spec = W.Spec("sinkgrad", 8100, "f32", 6, 2, 64, ("fixed", [17, 12, 1]), causal=causal, window=window,
                  sinks=True)
    case = W.make_case(spec, lens_q=[17, 12, 1], lens_k=lens_k)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal(case["q"].shape)
    _, g = _loss_and_grad(case, dout)
    for h in range(case["H"]):
        vals = []
        for sign in (1, -1):
            c = copy.deepcopy(case)
            c["sinks"] = c["sinks"].copy()
            c["sinks"][h] = np.float32(c["sinks"][h] + sign * 1e-3)
            vals.append((float(c["sinks"][h]), _loss_and_grad(c, dout)[0]))
        (sp, lp), (sm, lm) = vals
        fd = (lp - lm) / (sp - sm)
        assert abs(g[h] - fd) <= 1e-5 * max(1.0, abs(fd)), (h, g[h], fd)


def test_sink_grad_single_key_closed_form():
    spec = W.Spec("sinkgrad1", 8200, "f32", 2, 1, 64, ("fixed", [1]), causal=True, sinks=True)
    case = W.make_case(spec, lens_q=[1], lens_k=[1])
    rng = np.random.default_rng(6)
    dout = rng.standard_normal(case["q"].shape)
    out, lse = oracle.forward(case)
    g = oracle.sink_grad(case, dout, out, lse)
    q = case["q"].astype(np.float64)[0]
    v = case["v"].astype(np.float64)[0, 0]
    k = case["k"].astype(np.float64)[0, 0]
    for h in range(2):
        x = case["scale"] * float(q[h] @ k)
        w = np.exp(x) / (np.exp(x) + np.exp(float(case["sinks"][h])))
        want = -w * (1 - w) * float(dout[0, h] @ v)
        assert abs(g[h] - want) <= 1e-12 * max(1.0, abs(want))
