"""Parity of the ALiBi path (through the C ABI) with the fp64 oracle.

Reading (also in the header): with slopes s_h, the score of query i and key
j gets -s_h * |i + Lk - Lq - j| after the scale; sinks are unaffected.  The
slopes are the usual geometric ones, s_h = 2^(-8 (h + 1) / H).  Tolerances
are those of each dtype (the bias is computed in fp32 like the scores).
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


def _slopes(H):
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


def _check_full(case, what):
    announce(what)
    out, lse = run_case(case, torch)
    ref_o, ref_l = oracle.forward(case)
    e = assert_close(case, to_f64(out), to_f64(lse), ref_o, ref_l, what)
    announce(f"{what}: O error {e[0]:.2e}, LSE error {e[1]:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_alibi_scaled_configs(n, dtype):
    spec = W.scaled(W.config(n), B=4, max_len=600, seed=W.config(n).seed + 500)
    if n == 5:
        spec = dataclasses.replace(spec, lens_k=("uniform", 300, 2000))
    spec = dataclasses.replace(spec, dtype=dtype, name=f"{spec.name}_{dtype}_alibi")
    case = W.make_case(spec)
    case["alibi"] = _slopes(case["H"])
    _check_full(case, f"alibi {spec.name}")


def test_alibi_f32_path():
    spec = W.Spec("f32_alibi_window_sinks", 7300, "f32", 4, 2, 64, ("uniform", 20, 200, 4),
                  causal=False, window=(40, 12), sinks=True)
    case = W.make_case(spec)
    case["alibi"] = _slopes(case["H"])
    _check_full(case, "alibi f32 window + sinks")
    case = W.make_case(W.config(1))
    case["alibi"] = _slopes(case["H"])
    _check_full(case, "alibi tiny f32 causal GQA")


def test_zero_slopes_match_no_slopes():
    for n in (2, 5):
        case = W.make_case(W.scaled(W.config(n), B=3, max_len=300))
        o0, l0 = run_case(case, torch)
        o0, l0 = o0.clone(), l0.clone()
        case["alibi"] = np.zeros(case["H"], np.float32)
        o1, l1 = run_case(case, torch)
        if n == 5:  # decode: the same kernel, the bias adds -0
            assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
        else:       # prefill: the ALiBi instantiation, same arithmetic
            assert float((o0.float() - o1.float()).abs().max()) <= 2 ** -7
            assert float((l0 - l1).abs().max()) <= 1e-5


def test_alibi_full_size_causal_gqa_prefill_sampled():
    case = W.make_case(W.config(2))
    case["alibi"] = _slopes(case["H"])
    announce("alibi causal GQA prefill full size")
    out, lse = run_case(case, torch)
    toks, heads = sample_pairs(case, 192, seed=21)
    ref_o, ref_l = oracle.forward_rows(case, toks, heads)
    ti, hi = torch.from_numpy(toks).cuda(), torch.from_numpy(heads).cuda()
    e = assert_close(case, to_f64(out[ti, hi]), to_f64(lse[ti, hi]), ref_o, ref_l, "alibi full sampled")
    announce(f"alibi full size sampled: O error {e[0]:.2e}, LSE error {e[1]:.2e}")
