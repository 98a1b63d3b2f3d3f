"""Shared helpers of the GPU tests: move seeded cases to the device, run the
HIP path through the C ABI, compare with the oracle."""
import sys

import numpy as np

import workloads as W

# max-abs tolerances on (O, LSE): float32 inputs 1e-5 / 1e-5; bf16 inputs
# 2e-2 / 1e-3 with fp32 accumulation
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3), "f16": (5e-3, 1e-3)}

# host threads for oracle runs inside GPU tests: a GPU machine's CPU share
ORACLE_THREADS = 16


def announce(msg: str) -> None:
    sys.stderr.write(f"[gpu-case] {msg}\n")
    sys.stderr.flush()


def dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def run_case(case, torch, *, out=None, workspace=None, return_lse=True):
    import variable_length_attention_amd as va
    q = dev(case["q"], torch)
    cu_q = dev(case["cu_q"], torch)
    sinks = dev(case.get("sinks"), torch)
    alibi = dev(case.get("alibi"), torch)
    win = (case["window_left"], case["window_right"])
    if case.get("paged"):
        kc, vc = dev(case["k_cache"], torch), dev(case["v_cache"], torch)
        bt, su = dev(case["block_table"], torch), dev(case["seqused_k"], torch)
        o, lse = va.varlen_attn_paged(q, kc, vc, bt, cu_q, su, case["max_q"], case["max_k"],
                                      scale=case["scale"], causal=case["causal"], window=win,
                                      sinks=sinks, out=out, return_lse=True, workspace=workspace,
                                      alibi_slopes=alibi)
    else:
        k, v, cu_k = dev(case["k"], torch), dev(case["v"], torch), dev(case["cu_k"], torch)
        if out is None:
            out = torch.empty_like(q)
        lse = va.varlen_attn_out(out, q, k, v, cu_q, cu_k, case["max_q"], case["max_k"],
                                 scale=case["scale"], causal=case["causal"], window=win,
                                 sinks=sinks, return_lse=True, workspace=workspace, alibi_slopes=alibi)
        o = out
    torch.cuda.synchronize()
    return o, lse


def to_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def assert_close(case, out, lse, ref_out, ref_lse, what=""):
    tol_o, tol_l = TOL[case["dtype"]]
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert not np.any(np.isnan(lse)), f"{what}: NaN LSE"
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_lse), err_msg=f"{what}: -inf LSE rows")
    fin = np.isfinite(ref_lse)
    err_o = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert err_o <= tol_o, f"{what}: max |O - O_ref| = {err_o:.3e} > {tol_o}"
    assert err_l <= tol_l, f"{what}: max |LSE - LSE_ref| = {err_l:.3e} > {tol_l}"
    return err_o, err_l


def assert_close_blocks(case, out_t, lse_t, ref_out, ref_lse, what="", rows=2048):
    """assert_close over all rows, taken in blocks of rows (the GPU tensors
    are copied block by block); returns the largest (O, LSE) errors."""
    import torch
    worst_o, worst_l = 0.0, 0.0
    for r0 in range(0, int(out_t.shape[0]), rows):
        r1 = min(r0 + rows, int(out_t.shape[0]))
        o = out_t[r0:r1].to(torch.float64).cpu().numpy()
        l = lse_t[r0:r1].to(torch.float64).cpu().numpy()
        eo, el = assert_close(case, o, l, ref_out[r0:r1], ref_lse[r0:r1], f"{what} rows {r0}..{r1}")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    return worst_o, worst_l


def sample_pairs(case, n, seed):
    """Random (token, head) pairs plus the first and last row of every
    sequence and the rows around 128-row tile edges."""
    rng = np.random.default_rng(seed)
    toks = list(rng.integers(0, case["T_q"], n))
    for b in range(case["B"]):
        s, e = int(case["cu_q"][b]), int(case["cu_q"][b + 1])
        if e > s:
            toks += [s, e - 1]
            for edge in range(s + 127, e, 128):
                toks += [edge, min(edge + 1, e - 1)]
    toks = np.asarray(toks, np.int64)
    heads = rng.integers(0, case["H"], len(toks))
    return toks, heads


def sweep_cases():
    """Randomised structural sweep: lengths 0/1/odd/tile edges, GQA ratios
    1..64, D 64/128, every mask kind, sinks on/off, paged with block sizes
    16/64, float32 and bf16."""
    rng = np.random.default_rng(77)
    cases = []
    for n in range(14):
        g = [1, 2, 4, 8, 64][n % 5]
        Hkv = 1 if g == 64 else int(rng.integers(1, 3))
        H = g * Hkv
        D = [64, 128][n % 2]
        B = int(rng.integers(1, 5))
        lq = [int(x) for x in rng.choice([0, 1, 2, 3, 7, 31, 64, 65, 129], size=B)]
        decode = n % 3 == 0
        lk = [int(x) + (int(rng.integers(0, 90)) if decode else 0) for x in lq]
        kinds = [(True, (-1, -1)), (False, (-1, -1)), (False, (127, 0)), (True, (8, 3)),
                 (False, (2, 6))]
        causal, window = kinds[n % len(kinds)]
        sinks = (n % 2 == 1)
        spec = W.Spec(f"sweep{n}", 5000 + n, "bf16" if n % 4 else "f32", H, Hkv, D,
                      ("fixed", lq), causal=causal, window=window, sinks=sinks,
                      paged=(n % 4 == 2), block_size=[16, 64][n % 2])
        cases.append(W.make_case(spec, lens_q=lq, lens_k=lk))
    return cases
