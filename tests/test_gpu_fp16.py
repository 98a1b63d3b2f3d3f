"""Parity of the float16 path (called through the C ABI) with the fp64 oracle.

float16 inputs run the bf16 kernels' templates with the f16 matrix
instructions; the oracle widens the same binary16 values exactly.

Tolerance (max-abs): O 5e-3, LSE 1e-3.  Derivation: the output rounding is
half a float16 ulp, <= 2^-10 for |O| < 2 and 2^-9 for |O| < 4 (|O| stays
below 4 here: a convex combination of standard-normal rows); the
probabilities are rounded to float16 for P V, relative error <= 2^-11 per
term, <= 2^-11 * max|v| ~ 2.2e-3 in total; scores accumulate exact products
in fp32, so the LSE error stays ~1e-6, and 1e-3 is the bf16 bar kept.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import announce, assert_close, run_case, sample_pairs, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import variable_length_attention_amd._lib as L
    L.load()
    yield


def _f16(spec, **kw):
    return dataclasses.replace(spec, dtype="f16", name=spec.name + "_f16", **kw)


def _check_full(case, what):
    announce(what)
    out, lse = run_case(case, torch)
    assert out.dtype == torch.float16
    ref_out, ref_lse = oracle.forward(case)
    e = assert_close(case, to_f64(out), to_f64(lse), ref_out, ref_lse, what)
    announce(f"{what}: O error {e[0]:.2e}, LSE error {e[1]:.2e}")
    return e


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_f16_scaled_configs(n):
    spec = _f16(W.scaled(W.config(n), B=4, max_len=700, seed=W.config(n).seed + 300))
    if n == 5:
        spec = dataclasses.replace(spec, lens_k=("uniform", 300, 2000))  # paged split-KV decode
    _check_full(W.make_case(spec), f"f16 {spec.name}")


SHAPES = [
    # name, H, Hkv, D, lens_q, lens_k, causal, window, sinks, paged
    ("d64_two_sided_window_sinks", 8, 2, 64, [200, 65, 1], None, False, (31, 17), True, False),
    ("d128_decode_contiguous", 32, 8, 128, [1, 3, 4, 2], [900, 1500, 40, 2100], True, (-1, -1), False, False),
    ("d128_paged_prefill_long_queries", 16, 2, 128, [150, 40, 129], [400, 40, 300], True, (-1, -1), True, True),
    ("d64_paged_decode_mqa_window", 16, 1, 64, [2, 1, 4], [700, 64, 1000], True, (127, 0), True, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_f16_shapes(shape):
    name, H, Hkv, D, lq, lk, causal, window, sinks, paged = shape
    spec = W.Spec(f"f16_{name}", 7000 + len(name), "f16", H, Hkv, D, ("fixed", lq), causal=causal,
                  window=window, sinks=sinks, paged=paged, block_size=32)
    case = W.make_case(spec, lens_q=lq, lens_k=lk if lk is not None else lq)
    _check_full(case, f"f16 {name}")


def test_f16_single_key_rows_are_value_rows_bitwise():
    spec = W.Spec("f16_onekey", 7100, "f16", 8, 2, 128, ("uniform", 1, 300, 5), causal=True)
    case = W.make_case(spec)
    announce("f16 single-key rows")
    out, _ = run_case(case, torch)
    o = out.cpu().numpy()
    g = case["H"] // case["Hkv"]
    for b in range(case["B"]):
        t = int(case["cu_q"][b])
        for h in range(case["H"]):
            np.testing.assert_array_equal(o[t, h].view(np.uint16), case["v"][t, h // g].view(np.uint16))


def test_f16_full_size_causal_gqa_prefill_sampled():
    """The 33,781-token causal GQA prefill workload in float16, in the
    benchmark's launch configuration; sampled rows against the oracle."""
    spec = _f16(W.config(2))
    announce("f16 causal GQA prefill full size: generating")
    case = W.make_case(spec)
    out, lse = run_case(case, torch)
    toks, heads = sample_pairs(case, 192, seed=11)
    ref_o, ref_l = oracle.forward_rows(case, toks, heads)
    ti, hi = torch.from_numpy(toks).cuda(), torch.from_numpy(heads).cuda()
    e = assert_close(case, to_f64(out[ti, hi]), to_f64(lse[ti, hi]), ref_o, ref_l, "f16 full sampled")
    announce(f"f16 full size sampled: O error {e[0]:.2e}, LSE error {e[1]:.2e}")
    assert bool(torch.isfinite(out).all())
