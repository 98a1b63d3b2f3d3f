"""Parity of the forward at head size 512 (its own kernel, called through the
C ABI) with the fp64 oracle: causal GQA with ragged and single-row
sequences, the SparseAttnSharedkv README's first scenario shape on the dense
path (64 heads on one kv head, window (127, 0), sinks), a two-sided window
without causality, paged K/V for prefill and decode shapes, fp16, ALiBi,
rows that see no key (with and without sinks), the out variant, and the
benchmark's head-size-512 workload at full size, every row.

Tolerances are the forward's (bf16: 2e-2 on O, 1e-3 on LSE; f16: 5e-3,
1e-3): the kernel accumulates the 512-term scores and P V in fp32, so the
longer dot products add ~sqrt(512) fp32 roundings (~1e-5 relative) to the
scores, far below the LSE bound, and O carries the same rounding of the
probabilities to the input type as at the other head sizes.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ORACLE_THREADS, announce, assert_close, assert_close_blocks, run_case, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import variable_length_attention_amd._lib as L
    L.load()
    yield


SHAPES = [
    # name, dtype, H, Hkv, lens_q, lens_k, causal, window, sinks, paged, block_size
    ("causal_gqa_ragged", "bf16", 8, 2, [300, 129, 1, 64], None, True, (-1, -1), False, False, 64),
    ("readme_first_scenario_mqa_window_sinks", "bf16", 64, 1, [200, 37], None, False, (127, 0), True, False, 64),
    ("two_sided_window_mha", "bf16", 4, 4, [257, 64], None, False, (31, 17), False, False, 64),
    ("paged_prefill_f16_sinks", "f16", 16, 4, [150, 40], [400, 40], True, (-1, -1), True, True, 32),
    ("paged_decode_gqa", "bf16", 32, 8, [1, 3, 4], [900, 1500, 40], True, (-1, -1), False, True, 64),
    ("rows_without_keys_sinks", "bf16", 8, 2, [40, 20, 5], [10, 1, 5], True, (-1, -1), True, False, 64),
    ("rows_without_keys_no_sinks", "f16", 8, 2, [40, 20], [10, 1], True, (-1, -1), False, False, 64),
]


def _case(shape, seed):
    name, dtype, H, Hkv, lq, lk, causal, window, sinks, paged, bs = shape
    spec = W.Spec(f"d512_{name}", seed, dtype, H, Hkv, 512, ("fixed", lq), causal=causal, window=window,
                  sinks=sinks, paged=paged, block_size=bs)
    return W.make_case(spec, lens_q=lq, lens_k=lk if lk is not None else lq)


def _check(case, what):
    announce(what)
    out, lse = run_case(case, torch)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.forward(case)
    e = assert_close(case, to_f64(out), to_f64(lse), ref_out, ref_lse, what)
    announce(f"{what}: O error {e[0]:.2e}, LSE error {e[1]:.2e}")
    return out, lse


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_d512_matches_oracle(shape):
    _check(_case(shape, 7700 + len(shape[0])), f"d512 {shape[0]}")


def test_d512_alibi_causal_gqa():
    case = _case(SHAPES[0], 7790)
    case["alibi"] = (2.0 ** (-8.0 * np.arange(1, case["H"] + 1) / case["H"])).astype(np.float32)
    _check(case, "d512 ALiBi causal GQA")


def test_d512_takes_its_own_kernel():
    import variable_length_attention_amd as va
    case = _case(SHAPES[1], 7791)
    q = torch.empty((case["T_q"], case["H"], 512), dtype=torch.bfloat16, device="cuda")
    p = va.make_problem(q, case["Hkv"], int(case["cu_k"][-1]), case["B"], case["max_q"], case["max_k"],
                        case["scale"], case["causal"], (case["window_left"], case["window_right"]))
    assert va.kernel_path(p) == 4


def test_d512_out_variant_matches_allocating_variant_bitwise():
    case = _case(SHAPES[0], 7792)
    out_a, lse_a = run_case(case, torch)
    buf = torch.full_like(out_a, float("nan"))
    out_b, lse_b = run_case(case, torch, out=buf)
    torch.cuda.synchronize()
    assert out_b.data_ptr() == buf.data_ptr()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_a, lse_b)


def test_d512_benchmark_workload_full_size_elementwise():
    """The benchmark's head-size-512 workload (4 x 2048 tokens, causal,
    32 / 8 heads, bf16) in its launch configuration, every (token, head) row
    against the fp64 oracle (5.5e11 oracle FLOPs, about 15 s on 16 host
    threads), compared in blocks of rows."""
    announce("d512 benchmark workload: generating")
    case = W.make_case(W.D512_PREFILL)
    announce("d512 benchmark workload: running")
    out, lse = run_case(case, torch)
    torch.cuda.synchronize()
    announce(f"d512 benchmark workload: oracle on all {case['T_q'] * case['H']} rows")
    ref_o, ref_l = oracle.forward(case, nthreads=ORACLE_THREADS)
    errs = assert_close_blocks(case, out, lse, ref_o, ref_l, "d512 benchmark workload")
    announce(f"d512 benchmark workload: max |dO| = {errs[0]:.3e}, max |dLSE| = {errs[1]:.3e}")
