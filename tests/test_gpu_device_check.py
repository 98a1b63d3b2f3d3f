"""The opt-in device-side argument check (VARLEN_ATTN_DEVICE_CHECK=1).

With the check on, a valid call gives bitwise the same results as without
it, and each violated device-resident precondition (the list in the
library header) returns VA_ERR_DEVICE_CHECK before anything else runs, with
out and lse untouched.  Every call with contents that would be unsafe to
compute on is preceded, under the same environment, by a harmless violation
(a max_seqlen_k below the true maximum, which only affects launch sizing)
that must be reported, so an unsafe input never reaches the kernels if the
switch were not honoured.  The paged violations are also safe to compute on
by themselves: the caches are views into allocations with one spare block
before and after (block ids -1 and num_blocks land in mapped memory) and
the block table has a spare row of valid ids (a key count beyond a row reads
the next row's first entry), so a regression in one condition of the check
gives a wrong result, not an access outside the allocations.
"""
import numpy as np
import pytest

import workloads as W
from helpers import announce, dev, run_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import variable_length_attention_amd._lib as L
    L.load()
    yield


def _contig():
    return W.make_case(W.scaled(W.config(2), B=4, max_len=300))


def _paged():
    return W.make_case(W.scaled(W.config(5), B=6, max_len=900))


def _expect_check_error(case, what):
    """Runs case with sentinel out / lse; expects VA_ERR_DEVICE_CHECK and untouched outputs."""
    import variable_length_attention_amd as va
    announce(f"device check: {what}")
    q = dev(case["q"], torch)
    out = torch.full_like(q, 3.0)
    before = out.clone()
    win = (case["window_left"], case["window_right"])
    cu_q = dev(case["cu_q"], torch)
    with pytest.raises(RuntimeError, match="VA_ERR_DEVICE_CHECK"):
        if case.get("paged"):
            va.varlen_attn_paged(q, _padded_cache(case["k_cache"]), _padded_cache(case["v_cache"]),
                                 _padded_table(case["block_table"]), cu_q, dev(case["seqused_k"], torch),
                                 case["max_q"], case["max_k"], scale=case["scale"], causal=case["causal"],
                                 window=win, sinks=dev(case.get("sinks"), torch), out=out)
        else:
            va.varlen_attn_out(out, q, dev(case["k"], torch), dev(case["v"], torch), cu_q,
                               dev(case["cu_k"], torch), case["max_q"], case["max_k"], scale=case["scale"],
                               causal=case["causal"], window=win, sinks=dev(case.get("sinks"), torch))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), before.view(torch.int16)), "out was written"


def _padded_cache(a):
    """The cache as a contiguous view with one spare (zero) block before and after it."""
    t = dev(a, torch)
    big = torch.zeros((t.shape[0] + 2,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    big[1:-1] = t
    return big[1:-1]


def _padded_table(a):
    """The block table as a contiguous view with a spare row of block id 0 after it."""
    t = dev(a, torch)
    big = torch.zeros((t.shape[0] + 1, t.shape[1]), dtype=t.dtype, device=t.device)
    big[:-1] = t
    return big[:-1]


def _canary(case):
    bad = dict(case)
    bad["max_k"] = int(case["max_k"]) - 1  # below the true maximum: launch sizing only
    _expect_check_error(bad, "canary max_seqlen_k below the true maximum")


def test_valid_call_unchanged_by_the_check(monkeypatch):
    for case in (_contig(), _paged()):
        announce("device check: valid call, check off / on")
        o0, l0 = run_case(case, torch)
        monkeypatch.setenv("VARLEN_ATTN_DEVICE_CHECK", "1")
        o1, l1 = run_case(case, torch)
        monkeypatch.delenv("VARLEN_ATTN_DEVICE_CHECK")
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(l0, l1)


def test_harmless_violation_reported(monkeypatch):
    monkeypatch.setenv("VARLEN_ATTN_DEVICE_CHECK", "1")
    _canary(_contig())
    _canary(_paged())


@pytest.mark.parametrize("which", ["cu_q_start", "cu_q_order", "cu_q_total", "cu_k_start", "cu_k_order",
                                   "cu_k_total", "len_q"])
def test_contiguous_violations(monkeypatch, which):
    monkeypatch.setenv("VARLEN_ATTN_DEVICE_CHECK", "1")
    case = _contig()
    _canary(case)
    bad = dict(case)
    cu_q, cu_k = case["cu_q"].copy(), case["cu_k"].copy()
    if which == "cu_q_start":
        cu_q[0] = 1
    elif which == "cu_q_order":
        cu_q[1], cu_q[2] = cu_q[2] + 5, cu_q[1]
    elif which == "cu_q_total":
        cu_q[-1] -= 1
    elif which == "cu_k_start":
        cu_k[0] = 2
    elif which == "cu_k_order":
        cu_k[2] = cu_k[1] - 1
    elif which == "cu_k_total":
        cu_k[-1] -= 3
    elif which == "len_q":
        bad["max_q"] = int(np.diff(cu_q).max()) - 1
    bad["cu_q"], bad["cu_k"] = cu_q, cu_k
    _expect_check_error(bad, which)


@pytest.mark.parametrize("which", ["block_id_high", "block_id_negative", "seqused_beyond_row",
                                   "seqused_negative"])
def test_paged_violations(monkeypatch, which):
    monkeypatch.setenv("VARLEN_ATTN_DEVICE_CHECK", "1")
    case = _paged()
    _canary(case)
    bad = dict(case)
    bt, su = case["block_table"].copy(), case["seqused_k"].copy()
    bs = int(case["block_size"])
    b = int(np.argmax(su))
    if which == "block_id_high":
        bt[b, (int(su[b]) - 1) // bs] = int(case["num_blocks"])
    elif which == "block_id_negative":
        bt[b, 0] = -1
    elif which == "seqused_beyond_row":
        su[b] = bt.shape[1] * bs + 1  # beyond the row (and above max_seqlen_k)
    elif which == "seqused_negative":
        su[b] = -1
    bad["block_table"], bad["seqused_k"] = bt, su
    _expect_check_error(bad, which)
