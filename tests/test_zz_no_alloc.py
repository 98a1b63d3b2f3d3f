"""The allocation-free out variant (varlen_attn_fwd_out_noalloc) against the
out variant with a caller workspace, through the C ABI: two calls in a row,
the second with a smaller input (the scratch keeps the first call's
contents), on the tile path and on the decode path (whose partials live in
the scratch too)."""
import numpy as np
import pytest

import workloads as W
from helpers import announce, dev

torch = pytest.importorskip("torch")


def _run_both(case):
    import variable_length_attention_amd as va
    q, k, v = dev(case["q"], torch), dev(case["k"], torch), dev(case["v"], torch)
    cu_q, cu_k = dev(case["cu_q"], torch), dev(case["cu_k"], torch)
    sinks = dev(case.get("sinks"), torch)
    win = (case["window_left"], case["window_right"])
    kw = dict(scale=case["scale"], causal=case["causal"], window=win, sinks=sinks)
    out_ref = torch.full_like(q, 7.0)
    lse_ref = torch.full((case["T_q"], case["H"]), 7.0, dtype=torch.float32, device="cuda")
    va.varlen_attn_out(out_ref, q, k, v, cu_q, cu_k, case["max_q"], case["max_k"], lse=lse_ref, **kw)
    out = torch.full_like(q, -3.0)
    lse = torch.full((case["T_q"], case["H"]), -3.0, dtype=torch.float32, device="cuda")
    va.varlen_attn_out_noalloc(out, q, k, v, cu_q, cu_k, case["max_q"], case["max_k"], lse=lse, **kw)
    torch.cuda.synchronize()
    return out, lse, out_ref, lse_ref


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_noalloc_equals_out_variant_on_two_calls(kind):
    if kind == "prefill":
        big = W.scaled(W.config(2), B=6, max_len=900)     # several 64-key tiles, ragged tails
        small = W.scaled(W.config(2), B=2, max_len=150)
    else:
        # decode-shaped contiguous calls: split-KV partials in the scratch
        big = W.Spec("na_dec_big", 771, "bf16", 32, 8, 128, ("uniform", 1, 4, 40), lens_k=("uniform", 500, 3000),
                     causal=True, paged=False)
        small = W.Spec("na_dec_small", 772, "bf16", 32, 8, 128, ("uniform", 1, 2, 5), lens_k=("uniform", 64, 400),
                       causal=True, paged=False)
    for spec in (big, small):
        case = W.make_case(spec)
        announce(f"noalloc {kind} {spec.name} T_q={case['T_q']}")
        out, lse, out_ref, lse_ref = _run_both(case)
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "O differs from the out variant"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), "LSE differs from the out variant"
        assert np.isfinite(out.float().cpu().numpy()).all()


@pytest.mark.gpu
def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    import variable_length_attention_amd as va
    # decode-shaped: partials for ~(4096 + B * Hkv) splits x 16 rows x (D + 2) floats exceed 64 MiB
    B, H, Hkv, D = 4096, 64, 64, 128
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    p = va.make_problem(q, Hkv, B, B, 1, 1, None, False, (-1, -1))
    assert va.workspace_size(p, False) > (64 << 20)
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="VA_ERR_WORKSPACE"):
        va.varlen_attn_out_noalloc(out, q, k, k, cu, cu, 1, 1)
