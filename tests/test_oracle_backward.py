"""Pins for the backward oracle (no GPU).

The backward oracle follows the steps of the boostr CPU backward.  It is
pinned here to things other than itself: central finite differences of the
(separately pinned) forward oracle, a closed form for single-key rows, and
two invariants of the softmax (value weights sum to one minus the sink
share; a shift common to all keys of a sequence changes nothing).
"""
import numpy as np
import pytest

import oracle


def _case(lens_q, lens_k, H, Hkv, D, *, causal, window=(-1, -1), sinks=None, seed=0, scale=0.4):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    # values on a 1/64 grid: exact in float32, and so are the +-h perturbations
    q = np.round(rng.standard_normal((Tq, H, D)) * 64) / 64
    k = np.round(rng.standard_normal((Tk, Hkv, D)) * 64) / 64
    v = np.round(rng.standard_normal((Tk, Hkv, D)) * 64) / 64
    return dict(B=len(lens_q), H=H, Hkv=Hkv, D=D, dtype="f32", scale=scale, causal=causal,
                window_left=window[0], window_right=window[1], T_q=Tq, T_k=Tk, cu_q=cu_q, cu_k=cu_k,
                paged=False, q=q.astype(np.float32), k=k.astype(np.float32), v=v.astype(np.float32),
                sinks=None if sinks is None else np.asarray(sinks, np.float32))


def _loss(case, dout):
    out, _ = oracle.forward(case, nthreads=1)
    return float(np.sum(dout * out))


def _finite_difference(case, dout, name, h=2.0 ** -10):
    base = case[name]
    grad = np.zeros(base.shape, np.float64)
    for idx in np.ndindex(base.shape):
        vals = []
        for sgn in (1.0, -1.0):
            x = base.copy()
            x[idx] = np.float32(float(base[idx]) + sgn * h)
            c = dict(case)
            c[name] = x
            vals.append(_loss(c, dout))
        grad[idx] = (vals[0] - vals[1]) / (2 * h)
    return grad


FD_CASES = {
    "causal_gqa": dict(lens_q=[3, 5], lens_k=[3, 5], H=4, Hkv=2, D=8, causal=True),
    "end_aligned_decode_like": dict(lens_q=[2, 1], lens_k=[6, 4], H=2, Hkv=1, D=8, causal=True),
    "window_sinks": dict(lens_q=[6], lens_k=[6], H=2, Hkv=2, D=4, causal=False, window=(2, 1),
                         sinks=[0.3, -0.8]),
    "full_ragged_with_empty": dict(lens_q=[4, 0, 3], lens_k=[5, 2, 3], H=2, Hkv=1, D=4, causal=False),
}


@pytest.mark.parametrize("name", list(FD_CASES))
def test_backward_matches_finite_differences(name):
    case = _case(**FD_CASES[name], seed=len(name))
    rng = np.random.default_rng(7)
    dout = rng.standard_normal((case["T_q"], case["H"], case["D"]))
    out, lse = oracle.forward(case, nthreads=1)
    dq, dk, dv = oracle.backward(case, dout, out, lse, nthreads=2)
    for got, nm in ((dq, "q"), (dk, "k"), (dv, "v")):
        fd = _finite_difference(case, dout, nm)
        # central differences: error O(h^2) (h = 2^-10) plus rounding of the loss
        np.testing.assert_allclose(got, fd, rtol=0, atol=2e-5 * max(1.0, np.abs(fd).max()),
                                   err_msg=f"d{nm}")


def test_single_key_rows_closed_form():
    # one key per sequence and no sink: every weight is 1 and O = v, so
    # dP - D = <dout, v> - <dout, v> = 0: dq = dk = 0 and dv = the sum of dout
    # over the rows and query heads that share the kv head
    case = _case([3, 2], [1, 1], H=4, Hkv=2, D=8, causal=False, seed=3)
    dout = np.random.default_rng(1).standard_normal((case["T_q"], 4, 8))
    out, lse = oracle.forward(case)
    dq, dk, dv = oracle.backward(case, dout, out, lse)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)
    for b, (q0, q1) in enumerate([(0, 3), (3, 5)]):
        for c in range(2):
            want = dout[q0:q1, 2 * c:2 * c + 2].sum(axis=(0, 1))
            np.testing.assert_allclose(dv[b, c], want, atol=1e-12)


@pytest.mark.parametrize("sinks", [None, [0.5, -1.0, 2.0, 0.0]])
def test_value_gradient_sums_to_rows_times_kept_mass(sinks):
    # sum_j dv_j = sum_i (sum_j p_ij) dout_i, and sum_j p_ij = 1 - exp(sigma - lse)
    case = _case([7, 4], [7, 9], H=4, Hkv=2, D=8, causal=True, window=(3, 0), sinks=sinks, seed=11)
    dout = np.random.default_rng(2).standard_normal((case["T_q"], 4, 8))
    out, lse = oracle.forward(case)
    dq, dk, dv = oracle.backward(case, dout, out, lse)
    kept = np.ones_like(lse) if sinks is None else 1.0 - np.exp(np.asarray(sinks)[None, :] - lse)
    for b in range(2):
        qs = slice(case["cu_q"][b], case["cu_q"][b + 1])
        ks = slice(case["cu_k"][b], case["cu_k"][b + 1])
        for c in range(2):
            heads = slice(2 * c, 2 * c + 2)
            want = (kept[qs, heads][..., None] * dout[qs, heads]).sum(axis=(0, 1))
            np.testing.assert_allclose(dv[ks, c].sum(axis=0), want, atol=1e-10)


def test_common_key_shift_has_zero_gradient():
    # adding one vector to every key of a sequence adds a per-row constant to
    # its scores, which the softmax ignores (no sinks): sum_j dk_j = 0
    case = _case([6, 5], [6, 8], H=4, Hkv=2, D=8, causal=True, window=(4, 0), seed=5)
    dout = np.random.default_rng(3).standard_normal((case["T_q"], 4, 8))
    out, lse = oracle.forward(case)
    _, dk, _ = oracle.backward(case, dout, out, lse)
    for b in range(2):
        ks = slice(case["cu_k"][b], case["cu_k"][b + 1])
        np.testing.assert_allclose(dk[ks].sum(axis=0), 0, atol=1e-10)


def test_backward_rejects_paged_cases():
    case = _case([2], [2], H=1, Hkv=1, D=4, causal=True)
    case["paged"] = True
    with pytest.raises(ValueError):
        oracle.backward(case, np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), np.zeros((2, 1)))



@pytest.mark.parametrize("causal,window,alibi", [(True, (-1, -1), False), (False, (6, 2), True)])
def test_sampled_backward_equals_full_backward(causal, window, alibi):
    """The per-output evaluation agrees with the full C backward at every
    row and key (ragged lengths, queries shorter than keys, GQA, an empty
    sequence)."""
    case = _case([11, 1, 0, 17], [20, 3, 4, 17], 6, 2, 16, causal=causal, window=window,
                 sinks=[0.3, -1.0, 0.0, 2.0, 0.5, -0.2], seed=91)
    if alibi:
        case["alibi"] = (2.0 ** (-8.0 * np.arange(1, 7) / 6)).astype(np.float32)
    out, lse = oracle.forward(case)
    dout = np.random.default_rng(4).standard_normal(out.shape)
    dq, dk, dv = oracle.backward(case, dout, out, lse)
    T, Tk, D = case["T_q"], case["T_k"], case["D"]
    rows = (np.repeat(np.arange(T), case["H"]), np.tile(np.arange(case["H"]), T))
    keys = (np.repeat(np.arange(Tk), case["Hkv"]), np.tile(np.arange(case["Hkv"]), Tk))
    sq, sk, sv = oracle.backward_sampled(case, dout, out, lse, rows, keys)
    np.testing.assert_allclose(sq, dq.reshape(-1, D), rtol=0, atol=1e-12)
    np.testing.assert_allclose(sk, dk.reshape(-1, D), rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dv.reshape(-1, D), rtol=0, atol=1e-12)
