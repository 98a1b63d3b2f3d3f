"""Parity of the HIP backward (through the C ABI) with the fp64 backward oracle.

Both sides take the same inputs: q, k, v, a seeded dout (bf16), and the
forward's out (bf16) and lse (fp32) as computed by the HIP forward.  The
oracle follows the steps of the boostr CPU backward in float64.

Tolerance: the kernels round P and dS to bf16 for the matrix cores (relative
error <= 2^-9 each), accumulate in fp32 and round the results to bf16
(2^-9); a few such roundings on the largest terms stay below 1e-2 of the
largest gradient element, so each of dq, dk, dv must satisfy
max|got - ref| <= 2e-2 * max|ref| (the forward's bf16 bound of 2e-2, taken
relative to the gradient's scale, which grows with the number of summed rows).
Keys that no query sees must get exactly zero gradients.

fp16 inputs run the same kernels with the fp16 matrix instructions; their
roundings are 2^-11 instead of 2^-9, so the bound is 5e-3 of max |ref| (the
forward's fp16 bound on O).  With ALiBi slopes (geometric, 2^(-8 (h+1) / H))
both sides add the forward's bias to the recomputed scores.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import announce, dev, run_case, sample_pairs, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
REL_TOL = {"bf16": 2e-2, "f16": 5e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import variable_length_attention_amd._lib as L
    L.load()
    yield


def _dout(case, seed=99):
    """Seeded dout in the case's 16-bit type (bf16 as bits, fp16 as float16)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((case["T_q"], case["H"], case["D"]), dtype=np.float32)
    return x.astype(np.float16) if case["dtype"] == "f16" else W.f32_to_bf16_bits(x)


def _dout_f64(case, dout):
    return dout.astype(np.float64) if case["dtype"] == "f16" else W.bf16_bits_to_f32(dout)


def _run(case, dout_bits=None):
    import variable_length_attention_amd as va
    out, lse = run_case(case, torch)
    dout_bits = _dout(case) if dout_bits is None else dout_bits
    dout = dev(dout_bits, torch)
    q, k, v = dev(case["q"], torch), dev(case["k"], torch), dev(case["v"], torch)
    cu_q, cu_k = dev(case["cu_q"], torch), dev(case["cu_k"], torch)
    dq, dk, dv = va.varlen_attn_bwd(dout, q, k, v, out, lse, cu_q, cu_k, case["max_q"], case["max_k"],
                                    scale=case["scale"], causal=case["causal"],
                                    window=(case["window_left"], case["window_right"]),
                                    alibi_slopes=dev(case.get("alibi"), torch))
    torch.cuda.synchronize()
    return out, lse, dout_bits, dq, dk, dv


def _structural_zeros(case):
    """Query rows with no allowed key and key rows no query sees (from the
    mask definition: key j allowed for row i iff i + delta - wl <= j <=
    i + delta + wr, 0 <= j < Lk, with wr = 0 when causal)."""
    lq, lk = np.diff(case["cu_q"]), np.diff(case["cu_k"])
    wl = case["window_left"] if case["window_left"] >= 0 else 1 << 40
    wr = 0 if case["causal"] else (case["window_right"] if case["window_right"] >= 0 else 1 << 40)
    row_zero = np.zeros(case["T_q"], bool)
    key_zero = np.zeros(int(case["cu_k"][-1]), bool)
    for b in range(len(lq)):
        Lq, Lk = int(lq[b]), int(lk[b])
        i = np.arange(Lq)
        lo = np.maximum(0, i + Lk - Lq - wl)
        hi = np.minimum(Lk - 1, i + Lk - Lq + wr)
        row_zero[case["cu_q"][b]:case["cu_q"][b + 1]] = hi < lo
        seen = np.zeros(Lk, bool)
        for a_, z in zip(lo, hi):
            if z >= a_:
                seen[a_:z + 1] = True
        key_zero[case["cu_k"][b]:case["cu_k"][b + 1]] = ~seen
    return row_zero, key_zero


def _check(case, what):
    announce(f"backward {what}")
    out, lse, dout_bits, dq, dk, dv = _run(case)
    ref = oracle.backward(case, _dout_f64(case, dout_bits), to_f64(out), to_f64(lse))
    row_zero, key_zero = _structural_zeros(case)
    errs = {}
    for nm, got, r, zero in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, (row_zero, key_zero, key_zero)):
        g = to_f64(got)
        assert np.all(np.isfinite(g)), f"{what}: {nm} has non-finite values"
        scale = max(np.abs(r).max(), 1e-30)
        err = np.abs(g - r).max() / scale
        errs[nm] = err
        assert err <= REL_TOL[case["dtype"]], f"{what}: {nm} max error {err:.3e} of max |ref| {scale:.3e}"
        # rows with nothing to attend / keys nobody sees: exactly zero
        if zero.any():
            assert np.all(r.reshape(r.shape[0], -1)[zero] == 0)
            assert np.all(g.reshape(g.shape[0], -1)[zero] == 0), f"{what}: {nm} not zero where required"
    announce(f"backward {what}: relative errors " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    return errs


def test_backward_bf16_causal_gqa_prefill_scaled():
    _check(W.make_case(W.scaled(W.config(2), B=6, max_len=700)), "bf16_causal_gqa_prefill scaled (B=6, lengths <= 700)")


def test_backward_bf16_full_mha_scaled():
    _check(W.make_case(W.scaled(W.config(3), B=2, max_len=600)), "bf16_full_ulysses_shard scaled (B=2, lengths <= 600)")


def test_backward_bf16_swa_sinks_mqa_scaled():
    _check(W.make_case(W.scaled(W.config(4), B=3, max_len=700)), "bf16_swa_sinks_mqa scaled (B=3, lengths <= 700)")


SWEEP = [
    # name, H, Hkv, D, lens_q, lens_k, causal, window, sinks
    ("d64_causal_gqa", 8, 2, 64, [300, 77, 129], None, True, (-1, -1), False),
    ("end_aligned_q_shorter", 4, 4, 128, [40, 3, 130], [300, 64, 200], True, (-1, -1), False),
    ("two_sided_window", 8, 8, 128, [257, 64], None, False, (31, 17), False),
    ("sinks_full", 4, 2, 64, [100, 200], None, False, (-1, -1), True),
    ("queries_without_keys", 4, 2, 128, [50, 70, 30], [0, 90, 30], False, (-1, -1), False),
    ("keys_without_queries", 4, 2, 128, [0, 70, 129], [65, 70, 129], True, (-1, -1), False),
    ("single_rows", 4, 1, 128, [1, 1, 1, 2], [1, 5, 130, 2], True, (-1, -1), False),
    # GQA ratios 4 and 16 (quarter work units of the dQ kernel) with more
    # queries than keys, causal and end-aligned: leading rows and whole
    # leading quarters see no key
    ("q_longer_causal_g4", 8, 2, 128, [70, 40, 130], [30, 0, 100], True, (-1, -1), False),
    ("q_longer_causal_g4_sinks", 8, 2, 128, [70, 40, 130], [30, 0, 100], True, (-1, -1), True),
    ("q_longer_causal_g16", 32, 2, 128, [70, 40], [30, 10], True, (-1, -1), False),
    ("q_longer_causal_g16_sinks", 32, 2, 128, [70, 40], [30, 10], True, (-1, -1), True),
]


@pytest.mark.parametrize("row", SWEEP, ids=[r[0] for r in SWEEP])
def test_backward_sweep(row):
    name, H, Hkv, D, lq, lk, causal, win, sinks = row
    spec = W.Spec(f"bwd_{name}", 4242 + len(name), "bf16", H, Hkv, D, ("fixed", lq),
                  causal=causal, window=win, sinks=sinks)
    case = W.make_case(spec, lens_q=lq, lens_k=lk)
    _check(case, name)


def test_backward_is_deterministic():
    case = W.make_case(W.scaled(W.config(2), B=4, max_len=500))
    announce("backward run-to-run")
    a = _run(case)
    b = _run(case, dout_bits=a[2])
    for x, y in zip(a[3:], b[3:]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def _f16(spec):
    return dataclasses.replace(spec, dtype="f16", name=spec.name + "_f16")


def test_backward_f16_causal_gqa_prefill_scaled():
    case = W.make_case(_f16(W.scaled(W.config(2), B=5, max_len=600, seed=W.config(2).seed + 500)))
    assert case["q"].dtype == np.float16
    _check(case, "f16 bf16_causal_gqa_prefill scaled (B=5, lengths <= 600)")


def test_backward_f16_window_sinks_d64():
    spec = _f16(W.Spec("bwd_f16_window_d64", 4343, "bf16", 8, 2, 64, ("fixed", [200, 90, 1]),
                       window=(40, 9), sinks=True))
    _check(W.make_case(spec, lens_q=[200, 90, 1], lens_k=[260, 90, 5]), "f16 two-sided window, sinks, d64")


def _slopes(H):
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


def test_backward_alibi_causal_gqa_prefill_scaled():
    case = W.make_case(W.scaled(W.config(2), B=5, max_len=600, seed=W.config(2).seed + 600))
    case["alibi"] = _slopes(case["H"])
    _check(case, "alibi bf16_causal_gqa_prefill scaled (B=5, lengths <= 600)")


def test_backward_alibi_f16_window_end_aligned_d64():
    spec = _f16(W.Spec("bwd_alibi_f16_d64", 4444, "bf16", 8, 2, 64, ("fixed", [120, 33, 200]),
                       window=(50, 5), sinks=True))
    case = W.make_case(spec, lens_q=[120, 33, 200], lens_k=[300, 33, 210])
    case["alibi"] = _slopes(case["H"])
    _check(case, "alibi f16 two-sided window, sinks, end-aligned, d64")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_sink_gradient(dtype):
    """dsinks from the forward's out / lse against the oracle's sink gradient
    (same bound as the other gradients, relative to max |ref|), and the same
    bits on a second run (fixed-order sums)."""
    import variable_length_attention_amd as va
    spec = W.scaled(W.config(4), B=3, max_len=500, seed=W.config(4).seed + 700)
    spec = dataclasses.replace(spec, dtype=dtype, name=spec.name + "_" + dtype)
    case = W.make_case(spec)
    announce(f"sink gradient {dtype}")
    out, lse = run_case(case, torch)
    dout_bits = _dout(case, seed=101)
    dout, sinks = dev(dout_bits, torch), dev(case["sinks"], torch)
    g1 = va.varlen_attn_bwd_sinks(dout, out, lse, sinks)
    g2 = va.varlen_attn_bwd_sinks(dout, out, lse, sinks)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    ref = oracle.sink_grad(case, _dout_f64(case, dout_bits), to_f64(out), to_f64(lse))
    got = g1.double().cpu().numpy()
    err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    announce(f"sink gradient {dtype}: relative error {err:.2e}")
    assert err <= REL_TOL[dtype]


def test_backward_full_size_causal_gqa_prefill_sampled():
    """The benchmark's backward workload at full size (16 sequences of 128 to
    4096 tokens, 32 query heads on 8 kv heads, d128, causal) in the
    benchmark's launch configuration (preallocated dq / dk / dv and
    workspace): dq on sampled (token, head) pairs and dk, dv on sampled
    (key, kv head) pairs against the oracle's per-output evaluation, with
    the scaled tests' bound taken relative to the sample's largest gradient
    element; every element finite."""
    import variable_length_attention_amd as va
    case = W.make_case(W.config(2))
    announce("backward full size: forward")
    out, lse = run_case(case, torch)
    dout_bits = _dout(case, seed=123)
    q, k, v = dev(case["q"], torch), dev(case["k"], torch), dev(case["v"], torch)
    cu_q, cu_k = dev(case["cu_q"], torch), dev(case["cu_k"], torch)
    win = (case["window_left"], case["window_right"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = va.make_problem(q, k.shape[1], k.shape[0], case["B"], case["max_q"], case["max_k"], case["scale"],
                           case["causal"], win)
    ws = torch.empty(va.bwd_workspace_size(prob), dtype=torch.uint8, device="cuda")
    announce("backward full size: running")
    va.varlen_attn_bwd(dev(dout_bits, torch), q, k, v, out, lse, cu_q, cu_k, case["max_q"], case["max_k"],
                       scale=case["scale"], causal=case["causal"], window=win, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for nm, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(x).all()), f"{nm} has non-finite values"
    toks, heads = sample_pairs(case, 64, seed=5)
    rng = np.random.default_rng(6)
    T_k = int(case["cu_k"][-1])
    ktoks = np.concatenate([rng.integers(0, T_k, 64), case["cu_k"][:-1], case["cu_k"][1:] - 1]).astype(np.int64)
    kheads = rng.integers(0, case["Hkv"], len(ktoks))
    announce(f"backward full size: oracle on {len(toks)} rows and {len(ktoks)} keys")
    ref = oracle.backward_sampled(case, W.bf16_bits_to_f32(dout_bits), out.float().cpu().numpy(),
                                  lse.cpu().numpy(),
                                  (toks, heads), (ktoks, kheads))
    got = (dq[torch.from_numpy(toks).cuda(), torch.from_numpy(heads).cuda()],
           dk[torch.from_numpy(ktoks).cuda(), torch.from_numpy(kheads).cuda()],
           dv[torch.from_numpy(ktoks).cuda(), torch.from_numpy(kheads).cuda()])
    for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
        scale = max(np.abs(r).max(), 1e-30)
        err = np.abs(to_f64(g) - r).max() / scale
        announce(f"backward full size {nm}: max error {err:.2e} of max |ref| {scale:.3e}")
        assert err <= REL_TOL["bf16"], f"{nm} max error {err:.3e} of max |ref| {scale:.3e}"
