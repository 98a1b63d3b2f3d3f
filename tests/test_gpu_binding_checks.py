"""The Python binding checks every tensor against q and the problem before
calling the C ABI (the library sizes out, lse, dk, dv, ... from q's head_dim
and the descriptor): a mismatched tensor raises ValueError, nothing is
launched and the outputs keep their sentinel values."""
import pytest

from helpers import announce

torch = pytest.importorskip("torch")

T, H, HKV, D = 48, 4, 2, 128


def _base():
    g = torch.Generator().manual_seed(5)
    q = torch.randn((T, H, D), generator=g).to(torch.bfloat16).cuda()
    k = torch.randn((T, HKV, D), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((T, HKV, D), generator=g).to(torch.bfloat16).cuda()
    cu = torch.tensor([0, 20, 48], dtype=torch.int32, device="cuda")
    return q, k, v, cu


def _sentinel(shape, dtype):
    return torch.full(shape, 3.0, dtype=dtype, device="cuda")


FWD_CASES = ["out_dtype", "out_shape", "k_head_dim", "lse_dtype", "lse_shape", "sinks_size", "cu_k_size",
             "alibi_size", "v_shape"]


@pytest.mark.gpu
@pytest.mark.parametrize("which", FWD_CASES)
@pytest.mark.parametrize("entry", ["out", "noalloc"])
def test_out_variants_reject_mismatched_tensors(which, entry):
    import variable_length_attention_amd as va
    announce(f"binding check {entry} {which}")
    q, k, v, cu = _base()
    out = _sentinel((T, H, D), torch.bfloat16)
    lse = _sentinel((T, H), torch.float32)
    kw = dict(causal=True, lse=lse)
    cu_k = cu
    if which == "out_dtype":
        out = _sentinel((T, H, D), torch.float16)
    elif which == "out_shape":
        out = _sentinel((T, H, 64), torch.bfloat16)
    elif which == "k_head_dim":
        k, v = k[..., :64].contiguous(), v[..., :64].contiguous()
    elif which == "lse_dtype":
        kw["lse"] = lse = _sentinel((T, H), torch.float16)
    elif which == "lse_shape":
        kw["lse"] = lse = _sentinel((T, H + 1), torch.float32)
    elif which == "sinks_size":
        kw["sinks"] = torch.zeros(H + 1, dtype=torch.float32, device="cuda")
    elif which == "cu_k_size":
        cu_k = torch.tensor([0, 48], dtype=torch.int32, device="cuda")
    elif which == "alibi_size":
        kw["alibi_slopes"] = torch.zeros(H - 1, dtype=torch.float32, device="cuda")
    elif which == "v_shape":
        v = v[:, :1].contiguous()
    fn = va.varlen_attn_out if entry == "out" else va.varlen_attn_out_noalloc
    with pytest.raises(ValueError):
        fn(out, q, k, v, cu, cu_k, 28, 28, **kw)
    torch.cuda.synchronize()
    assert bool((out.float() == 3.0).all()) and bool((lse.float() == 3.0).all())


PAGED_CASES = ["cache_dtype", "cache_head_dim", "table_rows", "seqused_size", "out_shape", "lse_shape",
               "sinks_size"]


@pytest.mark.gpu
@pytest.mark.parametrize("which", PAGED_CASES)
def test_paged_rejects_mismatched_tensors(which):
    import variable_length_attention_amd as va
    announce(f"binding check paged {which}")
    q, _, _, cu = _base()
    kc = torch.zeros((8, 16, HKV, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    table = torch.arange(8, dtype=torch.int32, device="cuda").reshape(2, 4)
    used = torch.tensor([20, 28], dtype=torch.int32, device="cuda")
    out = _sentinel((T, H, D), torch.bfloat16)
    lse = _sentinel((T, H), torch.float32)
    kw = dict(causal=True, out=out, lse=lse)
    if which == "cache_dtype":
        kc = kc.to(torch.float16)
        vc = kc.clone()
    elif which == "cache_head_dim":
        kc = torch.zeros((8, 16, HKV, 64), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
    elif which == "table_rows":
        table = torch.arange(12, dtype=torch.int32, device="cuda").remainder(8).reshape(3, 4)
    elif which == "seqused_size":
        used = torch.tensor([20, 28, 0], dtype=torch.int32, device="cuda")
    elif which == "out_shape":
        kw["out"] = out = _sentinel((T, H, 64), torch.bfloat16)
    elif which == "lse_shape":
        kw["lse"] = lse = _sentinel((T + 1, H), torch.float32)
    elif which == "sinks_size":
        kw["sinks"] = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        va.varlen_attn_paged(q, kc, vc, table, cu, used, 28, 28, **kw)
    torch.cuda.synchronize()
    assert bool((out.float() == 3.0).all()) and bool((lse.float() == 3.0).all())


BWD_CASES = ["k_head_dim", "dk_shape", "dq_dtype", "lse_shape", "out_shape", "dout_dtype", "cu_k_size"]


@pytest.mark.gpu
@pytest.mark.parametrize("which", BWD_CASES)
def test_backward_rejects_mismatched_tensors(which):
    import variable_length_attention_amd as va
    announce(f"binding check backward {which}")
    q, k, v, cu = _base()
    out = torch.zeros_like(q)
    dout = torch.zeros_like(q)
    lse = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    dq = _sentinel((T, H, D), torch.bfloat16)
    dk = _sentinel((T, HKV, D), torch.bfloat16)
    dv = _sentinel((T, HKV, D), torch.bfloat16)
    cu_k = cu
    if which == "k_head_dim":
        k, v = k[..., :64].contiguous(), v[..., :64].contiguous()
        dk, dv = _sentinel((T, HKV, 64), torch.bfloat16), _sentinel((T, HKV, 64), torch.bfloat16)
    elif which == "dk_shape":
        dk = _sentinel((T, HKV, 64), torch.bfloat16)
    elif which == "dq_dtype":
        dq = _sentinel((T, H, D), torch.float16)
    elif which == "lse_shape":
        lse = torch.zeros((T, H - 1), dtype=torch.float32, device="cuda")
    elif which == "out_shape":
        out = torch.zeros((T, H, 64), dtype=torch.bfloat16, device="cuda")
    elif which == "dout_dtype":
        dout = dout.to(torch.float16)
    elif which == "cu_k_size":
        cu_k = torch.tensor([0, 48], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        va.varlen_attn_bwd(dout, q, k, v, out, lse, cu, cu_k, 28, 28, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool((t.float() == 3.0).all())
