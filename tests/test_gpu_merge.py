"""Parity of the HIP log-sum-exp merge (through the C ABI) with the oracle.

Element by element against ``oracle.merge`` (float64) on the same seeded
partials, and end to end: the HIP forward over a partition of each
sequence's keys, merged by the HIP merge, against the oracle forward over
all keys (the ring / context-parallel local step).

Tolerances.  Float32 output: every result is a weighted sum of n float32
values with float32 weights (relative error of a few ulp each), so
|got - ref| <= 1e-5 * max(1, |ref|) and lse within 1e-5 (|lse| < 30 here).
bf16 output: half a bf16 ulp of |O| < 8 is 0.0156, inside the forward's
2e-2; lse as above.  End to end (bf16 partials from the forward, each
already within the forward's bounds): the forward's 2e-2 on O and 1e-3 on
LSE.  Rows with no part and no sink must give O = 0 and LSE = -inf exactly.
"""
import numpy as np
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


def _parts_f64(m):
    o = m["o_parts"]
    return W.bf16_bits_to_f32(o).astype(np.float64) if m["dtype"] == "bf16" else o.astype(np.float64)


def _check(m, out_dtype, sinks, what, rows_sel=None):
    import variable_length_attention_amd as va
    o_parts, lse_parts = dev(m["o_parts"], torch), dev(m["lse_parts"], torch)
    s_dev = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device="cuda")
    out, lse = va.varlen_attn_merge(o_parts, lse_parts, sinks=s_dev, out_dtype=out_dtype)
    torch.cuda.synchronize()
    if rows_sel is not None:
        out, lse = out[torch.from_numpy(rows_sel).cuda()], lse[torch.from_numpy(rows_sel).cuda()]
        m = dict(m, o_parts=m["o_parts"][:, rows_sel], lse_parts=m["lse_parts"][:, rows_sel])
    got_o, got_l = to_f64(out), to_f64(lse)
    o64, l64 = _parts_f64(m), m["lse_parts"].astype(np.float64)
    ref_o, ref_l = oracle.merge(o64, l64, None if sinks is None else np.asarray(sinks, np.float32))
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    np.testing.assert_array_equal(np.isneginf(got_l), np.isneginf(ref_l), err_msg=f"{what}: -inf rows")
    empty = np.isneginf(ref_l)
    assert np.all(got_o[empty] == 0), f"{what}: rows with nothing must be 0"
    fin = ~empty
    if out_dtype == torch.bfloat16:
        err_o = float(np.max(np.abs(got_o - ref_o)))
        assert err_o <= 2e-2, f"{what}: max |O - ref| = {err_o:.3e}"
    else:
        err_o = float(np.max(np.abs(got_o - ref_o) / np.maximum(1.0, np.abs(ref_o))))
        assert err_o <= 1e-5, f"{what}: max relative |O - ref| = {err_o:.3e}"
    err_l = float(np.max(np.abs(got_l[fin] - ref_l[fin]))) if fin.any() else 0.0
    assert err_l <= 1e-5, f"{what}: max |LSE - ref| = {err_l:.3e}"
    announce(f"merge {what}: max O error {err_o:.2e}, max LSE error {err_l:.2e}")


CASES = [
    # name, n, rows, H, D, parts dtype, out dtype, sinks, empty fraction, empty-row period
    ("f32_to_f32_d128_n4_empties", 4, 300, 8, 128, "f32", torch.float32, False, 0.2, 7),
    ("bf16_to_bf16_d64_n2", 2, 257, 4, 64, "bf16", torch.bfloat16, False, 0.0, 0),
    ("bf16_to_f32_d128_n7_sinks", 7, 129, 6, 128, "bf16", torch.float32, True, 0.1, 11),
    ("f32_to_bf16_n1_identity", 1, 100, 3, 128, "f32", torch.bfloat16, False, 0.0, 5),
    ("f32_d8_n3_sinks_empty_rows", 3, 65, 5, 8, "f32", torch.float32, True, 0.3, 3),
    ("bf16_d512_n5", 5, 33, 2, 512, "bf16", torch.bfloat16, True, 0.05, 0),
    ("f32_n16_single_row", 16, 1, 1, 128, "f32", torch.float32, False, 0.5, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_merge_matches_oracle(case):
    name, n, rows, H, D, pdt, odt, sinks, ef, er = case
    announce(f"merge {name}")
    m = W.merge_inputs(n, rows, H, D, pdt, seed=3000 + len(name), empty_frac=ef, empty_rows_every=er)
    sk = np.linspace(-2.0, 3.0, H).astype(np.float32) if sinks else None
    _check(m, odt, sk, name)


def test_merge_at_ring_of_eight_size_sampled():
    # the benchmark's shape: 8 float32 partials of 32768 rows x 24 heads x 128
    announce("merge ring-of-8 size (32768 x 24 x 128, f32 parts, bf16 out), sampled rows")
    m = W.merge_inputs(8, 32768, 24, 128, "f32", seed=2024)
    rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, 32768, 600), [0, 32767]]))
    _check(m, torch.bfloat16, None, "ring-of-8 size", rows_sel=rows)


def _key_parts(case, cuts):
    parts = []
    for p in range(len(cuts[0]) - 1):
        idx, lens = [], []
        for b in range(case["B"]):
            k0 = int(case["cu_k"][b])
            a, z = cuts[b][p], cuts[b][p + 1]
            idx.append(np.arange(k0 + a, k0 + z))
            lens.append(z - a)
        idx = np.concatenate(idx).astype(np.int64)
        c = dict(case)
        c["cu_k"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        c["T_k"] = int(c["cu_k"][-1])
        c["max_k"] = max(1, max(lens))
        c["k"], c["v"] = case["k"][idx], case["v"][idx]
        c["sinks"] = None
        parts.append(c)
    return parts


@pytest.mark.parametrize("n_parts", [2, 3])
def test_forward_over_key_partition_then_merge_equals_full_forward(n_parts):
    import variable_length_attention_amd as va
    spec = W.scaled(W.config(3), B=3, max_len=700)
    case = W.make_case(spec)
    announce(f"merge end to end: {spec.name} scaled, keys split in {n_parts} parts")
    rng = np.random.default_rng(n_parts)
    lens = np.diff(case["cu_k"])
    cuts = []
    for L in lens:
        inner = np.sort(rng.integers(0, L + 1, n_parts - 1))
        cuts.append([0, *inner.tolist(), int(L)])
    cuts[0][1] = 0  # the first sequence gets an empty first part
    sinks = np.linspace(-1.0, 2.0, case["H"]).astype(np.float32)
    outs, lses = [], []
    for c in _key_parts(case, cuts):
        o, l = run_case(c, torch)
        outs.append(o)
        lses.append(l)
    o_parts = torch.stack(outs).contiguous()
    l_parts = torch.stack(lses).contiguous()
    out, lse = va.varlen_attn_merge(o_parts, l_parts, sinks=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    full = dict(case)
    full["sinks"] = sinks
    ref_o, ref_l = oracle.forward(full)
    e_o, e_l = assert_close(full, to_f64(out), to_f64(lse), ref_o, ref_l, f"{n_parts}-part merge")
    announce(f"merge end to end, {n_parts} parts: O error {e_o:.2e}, LSE error {e_l:.2e}")
