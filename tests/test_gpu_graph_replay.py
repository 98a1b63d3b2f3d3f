"""The forward entry points under HIP graph capture (the benchmark times its
steps as a captured graph of back-to-back calls): a graph of two out-variant
prefill calls and one paged decode call is replayed several times, with the
program's own eager work and synchronisations between the replays, and every
replay must give bitwise the eager results."""
import pytest

import workloads as W
from helpers import announce, dev

torch = pytest.importorskip("torch")


@pytest.mark.gpu
def test_graph_replays_equal_eager_calls():
    import variable_length_attention_amd as va
    pre = W.make_case(W.scaled(W.config(2), B=5, max_len=700))
    dec = W.make_case(W.scaled(W.config(5), B=8, max_len=2000))
    q, k, v = dev(pre["q"], torch), dev(pre["k"], torch), dev(pre["v"], torch)
    cu_q, cu_k = dev(pre["cu_q"], torch), dev(pre["cu_k"], torch)
    qd, kc, vc = dev(dec["q"], torch), dev(dec["k_cache"], torch), dev(dec["v_cache"], torch)
    bt, su, cu_qd = dev(dec["block_table"], torch), dev(dec["seqused_k"], torch), dev(dec["cu_q"], torch)
    out1, out2, outd = torch.empty_like(q), torch.empty_like(q), torch.empty_like(qd)
    lse1 = torch.empty((pre["T_q"], pre["H"]), dtype=torch.float32, device="cuda")
    lse2, lsed = torch.empty_like(lse1), torch.empty((dec["T_q"], dec["H"]), dtype=torch.float32, device="cuda")
    pp = va.make_problem(q, k.shape[1], k.shape[0], pre["B"], pre["max_q"], pre["max_k"], pre["scale"], True,
                         (-1, -1))
    pd = va.make_problem(qd, kc.shape[2], 0, dec["B"], dec["max_q"], dec["max_k"], dec["scale"], True, (-1, -1),
                         kc.shape[0], kc.shape[1], bt.shape[1])
    ws1 = torch.empty(va.workspace_size(pp, False), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws1)
    wsd = torch.empty(va.workspace_size(pd, True), dtype=torch.uint8, device="cuda")

    def calls():
        va.varlen_attn_out(out1, q, k, v, cu_q, cu_k, pre["max_q"], pre["max_k"], scale=pre["scale"],
                           causal=True, lse=lse1, workspace=ws1)
        va.varlen_attn_out(out2, q, k, v, cu_q, cu_k, pre["max_q"], pre["max_k"], scale=pre["scale"],
                           causal=True, lse=lse2, workspace=ws2)
        va.varlen_attn_paged(qd, kc, vc, bt, cu_qd, su, dec["max_q"], dec["max_k"], scale=dec["scale"],
                             causal=True, out=outd, lse=lsed, workspace=wsd)

    announce("graph replay: eager reference")
    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out1, lse1, outd, lsed)]
    announce("graph replay: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        # eager work of the program between replays: overwrite the outputs
        for t in (out1, out2, outd):
            t.fill_(1.5)
        lse1.fill_(-2.0)
        lsed.fill_(-2.0)
        torch.cuda.synchronize()
        announce(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = (out1, lse1, outd, lsed)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"replay {rep} differs"
        assert torch.equal(out2.view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(lse2, ref[1])
