"""Host-side tests of the C ABI (no GPU): the library loads, exports every
function include/varlen_attn.h declares, sizes workspaces, picks kernel
paths, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

from variable_length_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "varlen_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(varlen_attn_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_exactly_the_bound_functions():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.varlen_attn_abi_version() == 6


def test_problem_struct_matches_header(tmp_path):
    # the ctypes mirror against the header itself, compiled by the host C compiler
    import subprocess
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "varlen_attn.h"\n'
                   'int main(void) { printf("%zu %zu %zu\\n", sizeof(va_problem), '
                   'offsetof(va_problem, block_table_stride), offsetof(va_problem, alibi_slopes)); return 0; }\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    size, bts, alibi = map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split())
    assert ctypes.sizeof(_lib.VaProblem) == size
    assert _lib.VaProblem.block_table_stride.offset == bts
    assert _lib.VaProblem.alibi_slopes.offset == alibi


def test_version_one_problem_struct_is_accepted():
    # a caller built against version 1 (struct ends after block_table_stride)
    # (host checks only: the size queries launch nothing)
    lib = _lib.load()
    # 64 heads on one kv head, window (127, 0): slopes send it to the tile kernel
    p = _prob(num_heads=64, num_kv_heads=1, causal=0, window_left=127, window_right=0)
    p.alibi_slopes = 0x1234
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == 0
    p.struct_size = _lib.VaProblem.block_table_stride.offset + 4
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == 3                 # beyond the struct: not read
    assert lib.varlen_attn_workspace_size(ctypes.byref(p), 0) > 0
    assert lib.varlen_attn_bwd_workspace_size(ctypes.byref(p)) > 0
    p.struct_size -= 4
    assert lib.varlen_attn_workspace_size(ctypes.byref(p), 0) == 0      # shorter than version 1


def _prob(**kw):
    p = _lib.VaProblem()
    p.struct_size = ctypes.sizeof(_lib.VaProblem)
    defaults = dict(dtype=1, batch=2, total_q=100, total_k=100, num_heads=8, num_kv_heads=2,
                    head_dim=128, max_seqlen_q=60, max_seqlen_k=60, scale=0.088, causal=1,
                    window_left=-1, window_right=-1, num_blocks=0, block_size=0, block_table_stride=0)
    defaults.update(kw)
    for k, v in defaults.items():
        setattr(p, k, v)
    return p


# fake, aligned, never-dereferenced device addresses: every call below must
# fail validation before anything is enqueued
A = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(12)]


def _fwd_out(p, q=A[0], k=A[1], v=A[2], cuq=A[3], cuk=A[4], sinks=None, out=A[5], lse=None,
             ws=A[6], ws_bytes=1 << 30):
    lib = _lib.load()
    return lib.varlen_attn_fwd_out(ctypes.byref(p), q, k, v, cuq, cuk, sinks, out, lse, ws,
                                   ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=6, num_kv_heads=4), 2),        # H % H_kv != 0
    (dict(dtype=7), 3),
    (dict(dtype=3), 3),
    (dict(head_dim=96), 4),
    (dict(head_dim=256), 4),
    (dict(dtype=0, head_dim=512), 4),             # head size 512 takes 16-bit inputs
    (dict(batch=0), 2),
    (dict(total_q=0), 2),                          # empty tensors are not accepted
    (dict(total_k=0), 2),
    (dict(window_left=-2), 4),
    (dict(max_seqlen_q=0), 2),
    (dict(struct_size=8), 2),
    (dict(scale=float("nan")), 4),
])
def test_invalid_problems_are_rejected(kw, code):
    st = _fwd_out(_prob(**kw))
    assert st == code
    assert _lib.load().varlen_attn_last_error()


def test_null_pointers_alignment_aliasing_workspace():
    p = _prob()
    assert _fwd_out(p, q=None) == 1
    assert _fwd_out(p, cuk=None) == 1
    assert _fwd_out(p, out=None) == 1
    assert _fwd_out(p, q=ctypes.c_void_p(0x10000008)) == 6       # not 16-byte aligned
    assert _fwd_out(p, out=A[0]) == 5                            # out aliases q
    assert _fwd_out(p, lse=ctypes.c_void_p(A[5].value + 64)) == 5  # lse inside out
    assert _fwd_out(p, ws=None) == 7
    assert _fwd_out(p, ws_bytes=16) == 7


def test_paged_block_size_and_stride_validation():
    lib = _lib.load()

    p = _prob(num_blocks=10, block_size=40, block_table_stride=8)
    assert lib.varlen_attn_fwd_paged(ctypes.byref(p), A[0], A[1], A[2], A[7], A[3], A[8], None,
                                     A[5], None, A[6], ctypes.c_size_t(1 << 30), None) == 4
    p = _prob(num_blocks=10, block_size=64, block_table_stride=1, max_seqlen_k=200)
    assert lib.varlen_attn_fwd_paged(ctypes.byref(p), A[0], A[1], A[2], A[7], A[3], A[8], None,
                                     A[5], None, A[6], ctypes.c_size_t(1 << 30), None) == 2
    p = _prob(num_blocks=10, block_size=2048, block_table_stride=8)
    assert lib.varlen_attn_fwd_paged(ctypes.byref(p), A[0], A[1], A[2], A[7], A[3], A[8], None,
                                     A[5], None, A[6], ctypes.c_size_t(1 << 30), None) == 4


def test_allocating_entry_rejects_before_allocating():
    lib = _lib.load()
    out = ctypes.c_void_p(123)
    p = _prob(num_heads=5, num_kv_heads=2)
    st = lib.varlen_attn_fwd(ctypes.byref(p), A[0], A[1], A[2], A[3], A[4], None, ctypes.byref(out),
                             None, None)
    assert st == 2 and out.value is None


def test_workspace_size_and_kernel_path():
    lib = _lib.load()
    # causal bf16 prefill, GQA 4 -> tile path
    p = _prob(num_heads=32, num_kv_heads=8, total_q=33781, total_k=33781, batch=16,
              max_seqlen_q=4096, max_seqlen_k=4096)
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == 0
    ws = lib.varlen_attn_workspace_size(ctypes.byref(p), 0)
    n_max = (33781 + 16 * 127) // 128
    assert ws >= 16 * n_max * 2 + 4 * n_max
    # decode shape: g * max_q = 4 * 4 = 16 -> split-KV path with partials
    p = _prob(num_heads=32, num_kv_heads=8, total_q=327, batch=128, max_seqlen_q=4,
              max_seqlen_k=32768, num_blocks=33690, block_size=64, block_table_stride=512)
    assert lib.varlen_attn_path(ctypes.byref(p), 1) == 1
    assert lib.varlen_attn_workspace_size(ctypes.byref(p), 1) > 16 * 128 * 4
    # float32 always takes the float32 kernels
    p = _prob(dtype=0, head_dim=64, num_heads=4, num_kv_heads=2)
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == 2
    # 64 query heads on one kv head, window (127, 0): the sliding-window kernel
    c4 = dict(num_heads=64, num_kv_heads=1, total_q=25750, total_k=25750, batch=8, max_seqlen_q=8192,
              max_seqlen_k=8192, causal=0, window_left=127, window_right=0)
    p = _prob(**c4)
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == 3
    assert lib.varlen_attn_workspace_size(ctypes.byref(p), 0) > 0
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, dtype=2))), 0) == 3       # f16
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, num_heads=32))), 0) == 3  # 32 per kv head
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, causal=1, window_right=-1))), 0) == 3
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, head_dim=64, window_left=280))), 0) == 3
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, num_blocks=400, block_size=64,
                                                             block_table_stride=128))), 1) == 3  # paged
    # not taken: 16 heads per kv head, unbounded sides, no room for 4 rows
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, num_heads=16))), 0) == 0
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, window_left=-1))), 0) == 0
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, window_right=-1))), 0) == 0
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, window_left=149))), 0) == 0
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, dtype=0, head_dim=64))), 0) == 2
    # head size 512: its own kernel for every shape (here the window shape)
    assert lib.varlen_attn_path(ctypes.byref(_prob(**dict(c4, head_dim=512))), 0) == 4
    p = _prob(**c4)
    p.alibi_slopes = 0x10000000                                                          # ALiBi: tile kernel
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == 0
    # invalid -> 0 bytes / -1
    p = _prob(head_dim=80)
    assert lib.varlen_attn_workspace_size(ctypes.byref(p), 0) == 0
    assert lib.varlen_attn_path(ctypes.byref(p), 0) == -1


def test_binding_raises_value_error_with_message():
    with pytest.raises(ValueError, match="VA_ERR_SHAPE"):
        _lib.check(2)
    with pytest.raises(RuntimeError, match="VA_ERR_HIP"):
        _lib.check(8)


def _bwd(p, dout=A[0], q=A[1], k=A[2], v=A[3], out=A[4], lse=A[5], cuq=A[6], cuk=A[7], dq=A[8],
         dk=A[9], dv=A[10], ws=A[11], ws_bytes=1 << 30):
    lib = _lib.load()
    return lib.varlen_attn_bwd(ctypes.byref(p), dout, q, k, v, out, lse, cuq, cuk, dq, dk, dv, ws,
                               ctypes.c_size_t(ws_bytes), None)


def test_backward_rejects_before_launching():
    lib = _lib.load()
    p = _prob()
    assert lib.varlen_attn_bwd_workspace_size(ctypes.byref(p)) > 4 * 100 * 8  # includes Dv [T_q, H]
    assert lib.varlen_attn_bwd_workspace_size(ctypes.byref(_prob(dtype=0))) == 0
    assert _bwd(_prob(dtype=0)) == 4                                   # float32: unsupported
    assert _bwd(_prob(head_dim=96)) == 4
    assert _bwd(_prob(head_dim=512)) == 4                              # the forward only
    assert _bwd(_prob(dtype=2), ws_bytes=64) == 7                      # float16 accepted (then: workspace)
    assert _bwd(p, dout=None) == 1
    assert _bwd(p, lse=None) == 1
    assert _bwd(p, dq=A[1]) == 5                                       # dq aliases q
    assert _bwd(p, dv=ctypes.c_void_p(A[9].value + 256)) == 5          # dv inside dk
    assert _bwd(p, dk=ctypes.c_void_p(A[9].value + 8)) == 6            # not 16-byte aligned
    assert _bwd(p, ws_bytes=64) == 7
    assert _bwd(p, ws=None) == 7


def _merge(n=2, rows=10, H=4, D=128, pdt=1, odt=1, o=1 << 20, l=2 << 20, s=None, out=3 << 20, lse=4 << 20):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.load().varlen_attn_merge(n, rows, H, D, pdt, odt, vp(o), vp(l), vp(s), vp(out), vp(lse), None)


def test_merge_rejects_before_launching():
    # fake, never dereferenced addresses: every call fails its host checks
    assert _merge(n=0) == 2
    assert _merge(n=5000) == 2
    assert _merge(rows=0) == 2
    assert _merge(H=0) == 2
    assert _merge(D=12) == 4
    assert _merge(D=2048) == 4
    assert _merge(pdt=2) == 3
    assert _merge(odt=7) == 3
    assert _merge(pdt=2) == 3                                             # float16 partials are not taken
    assert _merge(o=None) == 1
    assert _merge(l=None) == 1
    assert _merge(out=None) == 1
    assert _merge(out=(3 << 20) + 8) == 6                                # out not 16-byte aligned
    assert _merge(l=(2 << 20) + 2) == 6                                   # lse_parts not 4-byte aligned
    assert _merge(out=(1 << 20) + 256) == 5                               # out inside o_parts
    assert _merge(lse=(2 << 20) + 4) == 5                                 # lse inside lse_parts
    assert _merge(lse=(3 << 20) + 64) == 5                                # lse inside out


def _sparse(**kw):
    p = _lib.VaSparseProblem()
    p.struct_size = ctypes.sizeof(_lib.VaSparseProblem)
    d = dict(dtype=1, batch=2, total_q=10, num_heads=64, num_kv_heads=1, head_dim=128, max_seqlen_kv=4096,
             scale=0.088, window_left=127, window_right=0, topk=512, cmp_ratio=4, ori_num_blocks=64,
             ori_block_size=128, ori_block_table_stride=32, cmp_num_blocks=16, cmp_block_size=128,
             cmp_block_table_stride=8)
    ptrs = dict(q=A[0], ori=A[1], ot=A[2], su=A[3], cmp=A[4], ct=A[5], idx=A[6], cuq=A[7], sinks=None,
                out=A[8], lse=A[9])
    for k, v in kw.items():
        (ptrs if k in ptrs else d)[k] = v
    for k, v in d.items():
        setattr(p, k, v)
    return _lib.load().varlen_attn_sparse_sharedkv(ctypes.byref(p), ptrs["q"], ptrs["ori"], ptrs["ot"], ptrs["su"],
                                                   ptrs["cmp"], ptrs["ct"], ptrs["idx"], ptrs["cuq"], ptrs["sinks"],
                                                   ptrs["out"], ptrs["lse"], None)


def test_sparse_rejects_before_launching():
    # fake, never dereferenced addresses: each call fails one host check
    assert _sparse(dtype=0) == 3                      # float32 not taken
    assert _sparse(num_heads=128) == 4                # 128 query heads per kv head
    assert _sparse(head_dim=96) == 4
    assert _sparse(head_dim=256) == 4
    assert _sparse(window_left=-1) == 4               # negative window side
    assert _sparse(topk=-1) == 2
    assert _sparse(cmp_attend_all=1) == 2             # every visible key takes no indices
    assert _sparse(cmp_attend_all=1, topk=0) == 2     # ... nor an indices pointer
    assert _sparse(cmp_attend_all=2, topk=0, idx=None) == 2
    assert _sparse(struct_size=4 * 18) == 2           # ends before the last field of ABI 4
    assert _sparse(cmp_ratio=0) == 2
    assert _sparse(ori_block_table_stride=31) == 2    # 4096 / 128 = 32 needed
    assert _sparse(cmp_block_table_stride=7) == 2     # 1024 / 128 = 8 needed
    assert _sparse(idx=None) == 1                     # topk > 0 needs indices
    assert _sparse(q=ctypes.c_void_p(A[0].value + 8)) == 6
    assert _sparse(out=A[1]) == 5                     # out aliases the original cache
    assert _sparse(lse=ctypes.c_void_p(A[8].value + 64)) == 5  # lse inside out
    assert _sparse(scale=0.0) == 4


def test_sink_gradient_rejects_before_launching():
    # fake, never dereferenced addresses: each call fails one host check
    lib = _lib.load()
    p = _prob()
    need = lib.varlen_attn_bwd_sinks_workspace_size(ctypes.byref(p))
    assert need >= 100 * 8 * 4                                          # one float per (row, head)
    assert lib.varlen_attn_bwd_sinks_workspace_size(ctypes.byref(_prob(dtype=0))) == 0

    def call(p, dout=A[0], out=A[1], lse=A[2], sinks=A[3], dsinks=A[4], ws=A[5], ws_bytes=1 << 20):
        return lib.varlen_attn_bwd_sinks(ctypes.byref(p), dout, out, lse, sinks, dsinks, ws,
                                         ctypes.c_size_t(ws_bytes), None)
    assert call(_prob(dtype=0)) == 4                                    # float32: unsupported
    assert call(_prob(head_dim=96)) == 4
    assert call(p, sinks=None) == 1
    assert call(p, dsinks=None) == 1
    assert call(p, ws_bytes=64) == 7
    assert call(p, out=ctypes.c_void_p(A[1].value + 8)) == 6            # not 16-byte aligned
    assert call(p, dsinks=ctypes.c_void_p(A[2].value + 16)) == 5        # dsinks inside lse
