"""Parity of the sliding-window kernel for wide GQA / MQA groups (32..64
query heads per kv head; path 3 of varlen_attn_path) with the fp64 oracle,
through the C ABI.

Tolerances are the forward's (bf16: 2e-2 on O, 1e-3 on LSE; f16: 5e-3,
1e-3): scores and softmax are computed as in the tile kernel (fp32
accumulation, probabilities rounded to the input type for P V).  Cases cover
the README's first scenario (64 heads on one kv head, window (127, 0),
sinks), 32 and 48 heads per kv head, d64, two-sided windows, windows that
leave room for only a few rows per work item, query / key lengths that
differ (end-aligned rows that see nothing), empty sequences, rows with one
visible key, and paged K/V (block sizes 128 and 48).
"""
import pytest

import oracle
import workloads as W
from helpers import announce, assert_close, dev, run_case, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import variable_length_attention_amd._lib as L
    L.load()
    yield


def _path(case):
    from variable_length_attention_amd import api
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[case["dtype"]]
    q = torch.empty((case["T_q"], case["H"], case["D"]), dtype=dt)   # shape and dtype only
    paged = bool(case.get("paged"))
    kw = dict(num_blocks=case["num_blocks"], block_size=case["block_size"],
              block_table_stride=case["block_table"].shape[1]) if paged else {}
    p = api.make_problem(q, case["Hkv"], case["T_k"], case["B"], case["max_q"], case["max_k"], case["scale"],
                         case["causal"], (case["window_left"], case["window_right"]), **kw)
    return api.kernel_path(p, paged)


CASES = {
    # name: Spec fields, lens_q, lens_k
    "readme_scenario1_64_heads_one_kv_head": (dict(H=64, Hkv=1, D=128, window=(127, 0), sinks=True),
                                              [300, 129, 1, 700], None),
    "g32_two_sided_window_empty_sequence": (dict(H=64, Hkv=2, D=128, window=(63, 10), sinks=False),
                                            [0, 50, 7, 260], None),
    "g48_d64_f16_wide_window": (dict(H=48, Hkv=1, D=64, dtype="f16", window=(200, 30), sinks=True),
                                [90, 400, 3], None),
    "queries_shorter_and_longer_than_keys": (dict(H=64, Hkv=1, D=128, window=(100, 0), sinks=False),
                                             [5, 40, 130], [300, 20, 130]),
    "diagonal_only_causal": (dict(H=32, Hkv=1, D=128, window=(0, -1), causal=True, sinks=True),
                             [70, 33], None),
    "window_leaves_four_rows": (dict(H=64, Hkv=1, D=128, window=(147, 1), sinks=True), [200, 17], None),
    "window_leaves_twelve_rows_f16": (dict(H=64, Hkv=1, D=128, dtype="f16", window=(140, 0), sinks=False),
                                      [333], None),
    # paged K/V (the README's PA_ND cache): 128-token blocks, and 48-token
    # blocks (not a power of two) with 32 heads per kv head; permuted tables
    "readme_scenario1_paged_blocks_128": (dict(H=64, Hkv=1, D=128, window=(127, 0), sinks=True, paged=True,
                                               block_size=128), [200, 33, 1], [700, 33, 90]),
    "paged_blocks_48_g32_d64_f16": (dict(H=64, Hkv=2, D=64, dtype="f16", window=(90, 3), sinks=True, paged=True,
                                         block_size=48), [60, 5, 130], [500, 5, 130]),
}


def _case(name):
    fields, lq, lk = CASES[name]
    fields = dict(fields)
    dtype = fields.pop("dtype", "bf16")
    spec = W.Spec("win_" + name, 5000 + len(name), dtype, lens_q=("fixed", lq),
                  lens_k="same" if lk is None else ("uniform", 1, 1), **fields)
    return W.make_case(spec, lens_q=lq, lens_k=lk)


@pytest.mark.parametrize("name", list(CASES))
def test_window_kernel_matches_oracle(name):
    case = _case(name)
    assert _path(case) == 3, "these shapes take the sliding-window kernel"
    announce(f"window {name}")
    out, lse = run_case(case, torch)
    ref_o, ref_l = oracle.forward(case)
    e = assert_close(case, to_f64(out), to_f64(lse), ref_o, ref_l, name)
    announce(f"window {name}: O error {e[0]:.2e}, LSE error {e[1]:.2e}")


def test_window_out_variant_bitwise_and_run_to_run():
    import variable_length_attention_amd as va
    case = _case("readme_scenario1_64_heads_one_kv_head")
    announce("window out-variant vs allocating, twice")
    o1, l1 = run_case(case, torch)
    q, k, v, cu_q, cu_k, sinks = (dev(case[x], torch) for x in ("q", "k", "v", "cu_q", "cu_k", "sinks"))
    o2, l2 = va.varlen_attn(q, k, v, cu_q, cu_k, case["max_q"], case["max_k"], scale=case["scale"],
                            window=(case["window_left"], case["window_right"]), sinks=sinks, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3 = va.varlen_attn(q, k, v, cu_q, cu_k, case["max_q"], case["max_k"], scale=case["scale"],
                        window=(case["window_left"], case["window_right"]), sinks=sinks)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
