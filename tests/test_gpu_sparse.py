"""Parity of sliding-window + compressed attention over shared K/V (the
SparseAttnSharedkv README's three scenarios, through the C ABI) with the fp64
oracle.  Key lists longer than the kernel's 1536-key LDS list (a long
window, many indices, or every visible compressed key of a long sequence)
are covered on purpose: the kernel takes them in chunks.

Tolerances are the forward's for each dtype (bf16: 2e-2 on O, 1e-3 on LSE;
f16: 5e-3, 1e-3): the kernel computes scores and the softmax the same way
(fp32 accumulation, probabilities rounded to the input type for P V).
Rows with no key and no sink must give O = 0 and LSE = -inf.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import TOL, announce, dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import variable_length_attention_amd._lib as L
    L.load()
    yield


def _run(sc):
    import variable_length_attention_amd as va
    idx = dev(sc["indices"], torch) if sc["topk"] > 0 else None
    out, lse = va.varlen_attn_sparse_sharedkv(
        dev(sc["q"], torch), dev(sc["ori_kv"], torch), dev(sc["ori_table"], torch), dev(sc["seqused_kv"], torch),
        dev(sc["cmp_kv"], torch), dev(sc["cmp_table"], torch), idx, dev(sc["cu_q"], torch),
        sc["max_seqlen_kv"], scale=sc["scale"], window=sc["window"], cmp_ratio=sc["cmp_ratio"],
        cmp_attend_all=sc["cmp_all"], sinks=dev(sc["sinks"], torch), return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _compare(sc, out, lse, ref_o, ref_l, what):
    tol_o, tol_l = TOL[sc["dtype"]]
    out, lse = np.asarray(out), np.asarray(lse)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_l), err_msg=f"{what}: -inf LSE rows")
    fin = np.isfinite(ref_l)
    e_o = float(np.max(np.abs(out - ref_o))) if out.size else 0.0
    e_l = float(np.max(np.abs(lse[fin] - ref_l[fin]))) if fin.any() else 0.0
    assert e_o <= tol_o, f"{what}: max |O - ref| = {e_o:.3e}"
    assert e_l <= tol_l, f"{what}: max |LSE - ref| = {e_l:.3e}"
    announce(f"sparse {what}: O error {e_o:.2e}, LSE error {e_l:.2e}")


CASES = {
    # the README example's structure at a small size: 64 heads over one kv head,
    # window (127, 0), 512 shared indices into a 4x compressed cache, sinks
    "readme_shape_shared_indices": dict(lens_q=[128, 128], seqused_kv=[4096, 4096], H=64, Hkv=1, D=128,
                                        window=(127, 0), topk=512, cmp_ratio=4, shared_indices=True),
    "per_token_indices_invalid_f16_gqa": dict(lens_q=[70, 33], seqused_kv=[900, 400], H=16, Hkv=2, D=128,
                                              dtype="f16", window=(31, 5), topk=100, cmp_ratio=4,
                                              invalid_frac=0.15, ori_bs=48, cmp_bs=16),
    "ragged_empty_and_keyless_no_sinks": dict(lens_q=[1, 0, 37, 5, 90], seqused_kv=[1, 50, 0, 20, 700], H=8,
                                              Hkv=1, D=128, window=(63, 0), topk=40, cmp_ratio=2, sinks=False,
                                              ori_bs=16, cmp_bs=32),
    "d64_two_sided_window": dict(lens_q=[64, 65], seqused_kv=[300, 129], H=32, Hkv=4, D=64, window=(20, 20),
                                 topk=64, cmp_ratio=3, invalid_frac=0.05, ori_bs=64, cmp_bs=64),
    "window_only_short_history": dict(lens_q=[16, 40], seqused_kv=[10, 40], H=64, Hkv=1, D=128,
                                      window=(127, 0), topk=0, cmp_ratio=4),
    # the README's head size: 64 heads over one kv head of 512, window (127, 0),
    # 512 indices per token, 128-token blocks, sinks
    "readme_config_d512": dict(lens_q=[64, 37], seqused_kv=[3000, 2100], H=64, Hkv=1, D=512,
                               window=(127, 0), topk=512, cmp_ratio=4, ori_bs=128, cmp_bs=128),
    # the README's first scenario at its head size: window (127, 0) only (topk 0), K = V
    "readme_scenario1_window_only_d512": dict(lens_q=[130, 7], seqused_kv=[900, 7], H=64, Hkv=1, D=512,
                                              window=(127, 0), topk=0, cmp_ratio=4, ori_bs=128, cmp_bs=128),
    "d512_f16_ragged_invalid_gqa_no_sinks": dict(lens_q=[5, 0, 40, 1], seqused_kv=[300, 7, 90, 1], H=24, Hkv=2,
                                                 D=512, dtype="f16", window=(20, 3), topk=50, cmp_ratio=2,
                                                 invalid_frac=0.2, sinks=False, ori_bs=32, cmp_bs=16),
    # the README usage example itself (third scenario): b = 4, 128 query rows
    # each over 4096 original keys, 64 / 1 heads of 512, window (127, 0), 512
    # distinct indices per sequence drawn from the keys every row sees
    "readme_example_scenario3_d512": dict(lens_q=[128] * 4, seqused_kv=[4096] * 4, H=64, Hkv=1, D=512,
                                          window=(127, 0), topk=512, cmp_ratio=4, visible_indices=True),
    # the same shapes in the second scenario: every compressed key the causal
    # compressed mask admits (up to 1024 per row, 1152 keys with the window)
    "readme_example_scenario2_d512": dict(lens_q=[128] * 4, seqused_kv=[4096] * 4, H=64, Hkv=1, D=512,
                                          window=(127, 0), topk=0, cmp_ratio=4, cmp_all=True),
    # second scenario with lists of up to 8320 keys (6 chunks), GQA, two
    # block sizes
    "scenario2_chunked_ratio1_gqa": dict(lens_q=[64, 33], seqused_kv=[8192, 7000], H=16, Hkv=2, D=128,
                                         window=(127, 0), topk=0, cmp_ratio=1, cmp_all=True, ori_bs=64,
                                         cmp_bs=256),
    # second scenario, ragged: an empty sequence, rows that see no compressed
    # key (Lq > S3), keyless rows without sinks, a two-sided window, d64, f16
    "scenario2_ragged_f16_d64_no_sinks": dict(lens_q=[1, 0, 50, 7, 12], seqused_kv=[5, 10, 3000, 0, 30], H=8,
                                              Hkv=1, D=64, dtype="f16", window=(20, 20), topk=0, cmp_ratio=3,
                                              cmp_all=True, sinks=False, ori_bs=16, cmp_bs=32),
    # an unbounded window (2^30 and above) over 2000 keys plus 500
    # compressed ones: two chunks, d512, GQA
    "scenario2_unbounded_window_d512": dict(lens_q=[40, 9], seqused_kv=[2000, 600], H=32, Hkv=2, D=512,
                                            window=(1 << 30, 0), topk=0, cmp_ratio=4, cmp_all=True),
    # third scenario with 2000 indices (2128 keys: two chunks), some of them
    # invalid, some past the compressed mask
    "scenario3_long_topk_chunked": dict(lens_q=[33, 70], seqused_kv=[5000, 2500], H=16, Hkv=1, D=128,
                                        window=(127, 0), topk=2000, cmp_ratio=2, invalid_frac=0.1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_matches_oracle(name):
    sc = W.sparse_case(**CASES[name], seed=4500 + len(name))
    announce(f"sparse {name}")
    out, lse = _run(sc)
    ref_o, ref_l = oracle.sparse_sharedkv(sc)
    _compare(sc, to_f64(out), to_f64(lse), ref_o, ref_l, name)


# benchmark workloads: 4 sequences of 1024 query tokens over 8192 original
# keys each, 64 heads / 1 kv head, d128 and d512, window (127, 0), 512
# distinct indices per sequence (drawn from the compressed keys every row
# sees) into a 4x compressed cache, 128-token blocks, sinks
BENCH = dict(lens_q=[1024] * 4, seqused_kv=[8192] * 4, H=64, Hkv=1, D=128, window=(127, 0), topk=512,
             cmp_ratio=4, ori_bs=128, cmp_bs=128, seed=4600, visible_indices=True)


@pytest.mark.parametrize("D", [128, 512])
def test_sparse_benchmark_size_sampled(D):
    sc = W.sparse_case(**dict(BENCH, D=D, seed=4600 if D == 128 else 4601))
    announce(f"sparse benchmark size d{D}: running")
    out, lse = _run(sc)
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([rng.integers(0, sc["T"], 96), [0, 1023, 1024, sc["T"] - 1]]))
    ref_o, ref_l = oracle.sparse_sharedkv(sc, tokens=toks)
    ti = torch.from_numpy(toks).cuda()
    _compare(sc, to_f64(out[ti]), to_f64(lse[ti]), ref_o, ref_l, "benchmark size sampled")
    assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("D", [128, 512])
def test_sparse_scenario2_benchmark_size_sampled(D):
    # second scenario at the benchmark size: up to 2048 compressed keys plus
    # the window per row (two chunks)
    sc = W.sparse_case(**dict(BENCH, D=D, topk=0, cmp_all=True, visible_indices=False, seed=4610 + D))
    announce(f"sparse scenario 2 benchmark size d{D}: running")
    out, lse = _run(sc)
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([rng.integers(0, sc["T"], 64), [0, 1023, 1024, sc["T"] - 1]]))
    ref_o, ref_l = oracle.sparse_sharedkv(sc, tokens=toks)
    ti = torch.from_numpy(toks).cuda()
    _compare(sc, to_f64(out[ti]), to_f64(lse[ti]), ref_o, ref_l, "scenario 2 benchmark size sampled")
    assert bool(torch.isfinite(out).all())


def test_sparse_abi4_descriptor_reads_no_attend_all():
    # a descriptor of ABI 4 ends before cmp_attend_all: whatever follows it
    # in memory is not read, and the call is the third scenario
    import ctypes
    import variable_length_attention_amd._lib as L
    sc = W.sparse_case(**dict(CASES["per_token_indices_invalid_f16_gqa"], seed=4620))
    ref_o, ref_l = oracle.sparse_sharedkv(sc)
    t = {k: dev(sc[k], torch) for k in ("q", "ori_kv", "ori_table", "seqused_kv", "cmp_kv", "cmp_table",
                                        "indices", "cu_q", "sinks")}
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=out.device)
    p = L.VaSparseProblem()
    p.struct_size = L.VaSparseProblem.cmp_attend_all.offset
    p.cmp_attend_all = 1
    p.dtype = 2
    p.batch, p.total_q = len(sc["cu_q"]) - 1, sc["T"]
    p.num_heads, p.num_kv_heads, p.head_dim = sc["H"], sc["Hkv"], sc["D"]
    p.max_seqlen_kv = int(max(sc["seqused_kv"]))
    p.scale = sc["scale"]
    p.window_left, p.window_right = sc["window"]
    p.topk, p.cmp_ratio = sc["topk"], sc["cmp_ratio"]
    p.ori_num_blocks, p.ori_block_size, p.ori_block_table_stride = (*t["ori_kv"].shape[:2], t["ori_table"].shape[1])
    p.cmp_num_blocks, p.cmp_block_size, p.cmp_block_table_stride = (*t["cmp_kv"].shape[:2], t["cmp_table"].shape[1])
    vp = lambda x: ctypes.c_void_p(x.data_ptr())
    L.check(L.load().varlen_attn_sparse_sharedkv(
        ctypes.byref(p), vp(t["q"]), vp(t["ori_kv"]), vp(t["ori_table"]), vp(t["seqused_kv"]), vp(t["cmp_kv"]),
        vp(t["cmp_table"]), vp(t["indices"]), vp(t["cu_q"]), vp(t["sinks"]), vp(out), vp(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()
    _compare(sc, to_f64(out), to_f64(lse), ref_o, ref_l, "ABI 4 descriptor")
