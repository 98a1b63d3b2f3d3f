"""Python binding of the C ABI in include/varlen_attn.h.

Argument marshalling only: tensor shapes become a ``va_problem``, tensor
storage becomes device pointers, and the current torch stream becomes the
``hipStream_t``.  Every step of the computation runs in the HIP library.
PyTorch is used for device memory and streams only.

Entry points (names follow the C ABI and the out-variant API of the pull
request "[varlen_attn for inference] add out variant"):
  varlen_attn        allocating: returns out (and lse)
  varlen_attn_out    writes a caller-provided ``out``; returns lse or None
  varlen_attn_paged  paged K/V through a block table (SparseAttnSharedkv
                     README, PageAttention constraints)
  varlen_attn_fwd    the library-allocating C entry point, results copied
                     into torch tensors (for ABI tests)
  varlen_attn_bwd    backward (dq, dk, dv) for bf16 / fp16 contiguous K/V
  varlen_attn_bwd_sinks
                     gradient of the per-head sink logits
  varlen_attn_merge  merge of partial results over disjoint key sets
                     through their log-sum-exp (ring / context parallel)
  varlen_attn_sparse_sharedkv
                     sliding-window + sparse compressed attention over shared
                     K/V (SparseAttnSharedkv README, third scenario)
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

__all__ = ["varlen_attn", "varlen_attn_out", "varlen_attn_paged", "varlen_attn_fwd", "varlen_attn_bwd",
           "bwd_workspace_size", "varlen_attn_bwd_sinks", "varlen_attn_merge", "varlen_attn_sparse_sharedkv",
           "workspace_size", "plan", "kernel_path", "output_shapes", "make_problem"]

_DTYPES = {torch.float32: _lib.VA_F32, torch.bfloat16: _lib.VA_BF16, torch.float16: _lib.VA_F16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def output_shapes(q: torch.Tensor):
    """Shape inference (the analog of the op's meta function): out has q's
    shape and dtype, lse is float32 [total_q, num_heads]."""
    return tuple(q.shape), (q.shape[0], q.shape[1])


def make_problem(q, num_kv_heads, total_k, batch, max_seqlen_q, max_seqlen_k, scale, causal,
                 window, num_blocks=0, block_size=0, block_table_stride=0, alibi_slopes=None) -> _lib.VaProblem:
    _need(q.dim() == 3, "q must be [total_q, num_heads, head_dim]")
    _need(q.dtype in _DTYPES, f"dtype {q.dtype} not supported (float32, bfloat16 or float16)")
    p = _lib.VaProblem()
    p.struct_size = ctypes.sizeof(_lib.VaProblem)
    p.dtype = _DTYPES[q.dtype]
    p.batch = int(batch)
    p.total_q, p.num_heads, p.head_dim = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    p.total_k = int(total_k)
    p.num_kv_heads = int(num_kv_heads)
    p.max_seqlen_q, p.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    p.scale = float(1.0 / math.sqrt(q.shape[2]) if scale is None else scale)
    p.causal = 1 if causal else 0
    p.window_left, p.window_right = int(window[0]), int(window[1])
    p.num_blocks, p.block_size, p.block_table_stride = int(num_blocks), int(block_size), int(block_table_stride)
    if alibi_slopes is not None:
        _need(alibi_slopes.dtype == torch.float32 and alibi_slopes.numel() == q.shape[1] and
              alibi_slopes.is_cuda and alibi_slopes.is_contiguous(), "alibi_slopes must be float32 [num_heads] on the GPU")
        p.alibi_slopes = alibi_slopes.data_ptr()
    return p


def _check_tensors(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        _need(t.is_cuda, "all tensors must be on a GPU")
        _need(t.is_contiguous(), "all tensors must be contiguous")
        dev = dev or t.device
        _need(t.device == dev, "all tensors must be on the same device")
    return dev


def _check_rows_f32(t, rows, heads, what):
    if t is not None:
        _need(t.dtype == torch.float32 and tuple(t.shape) == (rows, heads),
              f"{what} must be float32 [total_q, num_heads] = [{rows}, {heads}]")


def _check_heads_f32(t, heads, what):
    if t is not None:
        _need(t.dtype == torch.float32 and t.dim() == 1 and t.numel() == heads,
              f"{what} must be float32 [num_heads] = [{heads}]")


def _check_forward(q, out, lse, sinks, alibi_slopes, cu_seqlens_q):
    """Checks shared by the forward bindings: the C library sizes every
    buffer from q and the problem description, so each tensor handed over
    must match them (nothing is launched otherwise)."""
    _need(q.dim() == 3, "q must be [total_q, num_heads, head_dim]")
    if out is not None:
        _need(out.dtype == q.dtype and out.shape == q.shape, "out must have q's shape and dtype")
    _check_rows_f32(lse, q.shape[0], q.shape[1], "lse")
    _check_heads_f32(sinks, q.shape[1], "sinks")
    _check_heads_f32(alibi_slopes, q.shape[1], "alibi_slopes")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.dim() == 1 and cu_seqlens_q.numel() >= 2,
          "cu_seqlens_q must be int32 [batch + 1]")


def _check_contiguous_kv(q, k, v, cu_seqlens_q, cu_seqlens_k):
    _need(k.dim() == 3 and v.shape == k.shape, "k and v must be [total_k, num_kv_heads, head_dim]")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share a dtype")
    _need(k.shape[2] == q.shape[2], "k and v must have q's head_dim")
    _need(cu_seqlens_k.dtype == torch.int32 and cu_seqlens_k.dim() == 1
          and cu_seqlens_k.numel() == cu_seqlens_q.numel(), "cu_seqlens_k must be int32 [batch + 1], like cu_seqlens_q")


def workspace_size(problem: _lib.VaProblem, paged: bool = False) -> int:
    return int(_lib.load().varlen_attn_workspace_size(ctypes.byref(problem), 1 if paged else 0))


def kernel_path(problem: _lib.VaProblem, paged: bool = False) -> int:
    """0 = prefill tiles, 1 = split-KV decode + combine, 2 = float32 path,
    3 = sliding-window kernel for 32..64 query heads per kv head, 4 = head
    size 512."""
    return int(_lib.load().varlen_attn_path(ctypes.byref(problem), 1 if paged else 0))


def _workspace(problem, paged, dev, workspace):
    need = workspace_size(problem, paged)
    if need == 0:  # invalid problem: let the call report why
        return workspace
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace


def varlen_attn_out(out: torch.Tensor, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    max_seqlen_k: int, *, scale: Optional[float] = None, causal: bool = False,
                    window: Tuple[int, int] = (-1, -1), sinks=None, lse=None,
                    return_lse: bool = False, workspace=None, alibi_slopes=None):
    """Writes attention over contiguous packed K/V into ``out``; returns the
    float32 LSE when ``return_lse`` (or an ``lse`` buffer is given), else None.
    ``alibi_slopes`` (float32 [num_heads]) adds -slope * |i + Lk - Lq - j|."""
    dev = _check_tensors(out, q, k, v, cu_seqlens_q, cu_seqlens_k, sinks, lse, workspace, alibi_slopes)
    _need(out is not None, "out must be given")
    _check_forward(q, out, lse, sinks, alibi_slopes, cu_seqlens_q)
    _check_contiguous_kv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    p = make_problem(q, k.shape[1], k.shape[0], cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k,
                     scale, causal, window, alibi_slopes=alibi_slopes)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=dev)
    ws = _workspace(p, False, dev, workspace)
    st = _lib.load().varlen_attn_fwd_out(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(sinks),
        _ptr(out), _ptr(lse), _ptr(ws), ctypes.c_size_t(0 if ws is None else ws.numel()), _stream(dev))
    _lib.check(st)
    return lse


def varlen_attn_out_noalloc(out: torch.Tensor, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                            max_seqlen_k: int, *, scale: Optional[float] = None, causal: bool = False,
                            window: Tuple[int, int] = (-1, -1), sinks=None, lse=None, alibi_slopes=None):
    """varlen_attn_out without a workspace (the library's per-device scratch
    array instead): for callers that cannot allocate.  ``lse`` (float32
    [total_q, num_heads]) is filled when given; calls that overlap in time on
    one device race."""
    dev = _check_tensors(out, q, k, v, cu_seqlens_q, cu_seqlens_k, sinks, lse, alibi_slopes)
    _need(out is not None, "out must be given")
    _check_forward(q, out, lse, sinks, alibi_slopes, cu_seqlens_q)
    _check_contiguous_kv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    p = make_problem(q, k.shape[1], k.shape[0], cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k,
                     scale, causal, window, alibi_slopes=alibi_slopes)
    st = _lib.load().varlen_attn_fwd_out_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(sinks),
        _ptr(out), _ptr(lse), _stream(dev))
    _lib.check(st)


def varlen_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
                scale: Optional[float] = None, causal: bool = False,
                window: Tuple[int, int] = (-1, -1), sinks=None, return_lse: bool = False, alibi_slopes=None):
    """Allocating form: returns out, or (out, lse) when ``return_lse``."""
    out = torch.empty_like(q)
    lse = varlen_attn_out(out, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          scale=scale, causal=causal, window=window, sinks=sinks,
                          return_lse=return_lse, alibi_slopes=alibi_slopes)
    return (out, lse) if return_lse else out


def varlen_attn_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqused_k, max_seqlen_q: int,
                      max_seqlen_k: int, *, scale: Optional[float] = None, causal: bool = False,
                      window: Tuple[int, int] = (-1, -1), sinks=None, out=None, lse=None,
                      return_lse: bool = False, workspace=None, alibi_slopes=None):
    """Paged K/V: caches [num_blocks, block_size, num_kv_heads, head_dim],
    block_table int32 [batch, stride], seqused_k int32 [batch]."""
    dev = _check_tensors(q, k_cache, v_cache, block_table, cu_seqlens_q, seqused_k, sinks, out, lse,
                         workspace, alibi_slopes)
    _check_forward(q, out, lse, sinks, alibi_slopes, cu_seqlens_q)
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
          "caches must be [num_blocks, block_size, num_kv_heads, head_dim]")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q and the caches must share a dtype")
    _need(k_cache.shape[3] == q.shape[2], "the caches must have q's head_dim")
    batch = cu_seqlens_q.numel() - 1
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == batch,
          "block_table must be int32 [batch, stride]")
    _need(seqused_k.dtype == torch.int32 and seqused_k.dim() == 1 and seqused_k.numel() == batch,
          "seqused_k must be int32 [batch]")
    p = make_problem(q, k_cache.shape[2], 0, cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k, scale,
                     causal, window, k_cache.shape[0], k_cache.shape[1], block_table.shape[1],
                     alibi_slopes=alibi_slopes)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=dev)
    ws = _workspace(p, True, dev, workspace)
    st = _lib.load().varlen_attn_fwd_paged(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cu_seqlens_q),
        _ptr(seqused_k), _ptr(sinks), _ptr(out), _ptr(lse), _ptr(ws),
        ctypes.c_size_t(0 if ws is None else ws.numel()), _stream(dev))
    _lib.check(st)
    return (out, lse) if (return_lse or lse is not None) else out


_hip = None


def _hip_rt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    return _hip


def varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
                    scale=None, causal=False, window=(-1, -1), sinks=None, return_lse=False):
    """Calls the library-allocating C entry point ``varlen_attn_fwd`` and
    copies its buffers into torch tensors before releasing them."""
    dev = _check_tensors(q, k, v, cu_seqlens_q, cu_seqlens_k, sinks)
    _check_forward(q, None, None, sinks, None, cu_seqlens_q)
    _check_contiguous_kv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    p = make_problem(q, k.shape[1], k.shape[0], cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k,
                     scale, causal, window)
    lib = _lib.load()
    o_ptr, l_ptr = ctypes.c_void_p(), ctypes.c_void_p()
    s = _stream(dev)
    st = lib.varlen_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                             _ptr(cu_seqlens_k), _ptr(sinks), ctypes.byref(o_ptr),
                             ctypes.byref(l_ptr) if return_lse else None, s)
    _lib.check(st)
    out = torch.empty_like(q)
    hip = _hip_rt()
    D2D = 3
    rc = hip.hipMemcpyAsync(ctypes.c_void_p(out.data_ptr()), o_ptr, out.numel() * out.element_size(), D2D, s)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=dev)
        rc |= hip.hipMemcpyAsync(ctypes.c_void_p(lse.data_ptr()), l_ptr, lse.numel() * 4, D2D, s)
        _lib.check(lib.varlen_attn_free(l_ptr, s))
    _lib.check(lib.varlen_attn_free(o_ptr, s))
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
    return (out, lse) if return_lse else out


def plan(cu_seqlens_q, seqlens_k, *, num_heads, num_kv_heads, head_dim, dtype, total_q, total_k,
         max_seqlen_q, max_seqlen_k, causal=False, window=(-1, -1), paged=False, num_blocks=0,
         block_size=0, block_table_stride=0):
    """Runs only the work-partition pre-pass; returns (items int32 [n, 4],
    path) with items in execution order."""
    dev = _check_tensors(cu_seqlens_q, seqlens_k)
    fake_q = torch.empty((total_q, num_heads, head_dim), dtype=dtype, device="meta")
    p = make_problem(fake_q, num_kv_heads, total_k, cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k,
                     None, causal, window, num_blocks, block_size, block_table_stride)
    ws = _workspace(p, paged, dev, None)
    cap = max(1, ws.numel() // 16)
    items = torch.empty((cap, 4), dtype=torch.int32, device=dev)
    count = torch.zeros(1, dtype=torch.int32, device=dev)
    st = _lib.load().varlen_attn_plan(ctypes.byref(p), 1 if paged else 0, _ptr(cu_seqlens_q),
                                      _ptr(seqlens_k), _ptr(items), ctypes.c_int32(cap), _ptr(count),
                                      _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    _lib.check(st)
    n = int(count.item())
    return items[:n].clone(), kernel_path(p, paged)


def bwd_workspace_size(problem: _lib.VaProblem) -> int:
    return int(_lib.load().varlen_attn_bwd_workspace_size(ctypes.byref(problem)))


def varlen_attn_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    max_seqlen_k: int, *, scale: Optional[float] = None, causal: bool = False,
                    window: Tuple[int, int] = (-1, -1), dq=None, dk=None, dv=None, workspace=None,
                    alibi_slopes=None):
    """Backward of varlen_attn for bf16 / fp16 contiguous K/V: returns (dq,
    dk, dv) (allocated when not given) from dout and the forward's out / lse
    (``alibi_slopes``: the forward's slopes, when it had them)."""
    dev = _check_tensors(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace, alibi_slopes)
    _check_forward(q, out, lse, None, alibi_slopes, cu_seqlens_q)
    _need(lse is not None, "lse of the forward call must be given")
    _need(dout.shape == q.shape and dout.dtype == q.dtype, "dout must have q's shape and dtype")
    _check_contiguous_kv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
          and all(t.dtype == q.dtype for t in (dq, dk, dv)), "dq must be like q, dk and dv like k")
    p = make_problem(q, k.shape[1], k.shape[0], cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k,
                     scale, causal, window, alibi_slopes=alibi_slopes)
    need = bwd_workspace_size(p)
    if need == 0:
        _lib.check(_lib.load().varlen_attn_bwd(ctypes.byref(p), *([None] * 12), ctypes.c_size_t(0), None))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = _lib.load().varlen_attn_bwd(
        ctypes.byref(p), _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
        _stream(dev))
    _lib.check(st)
    return dq, dk, dv


def varlen_attn_bwd_sinks(dout, out, lse, sinks, *, dsinks=None, workspace=None):
    """Gradient of the per-head sink logits of a forward call (bf16 / fp16):
    dsinks[h] = -sum_i exp(sinks[h] - lse[i, h]) * sum_d dout[i, h, d] out[i, h, d].
    Returns dsinks (float32 [num_heads]; allocated when not given)."""
    dev = _check_tensors(dout, out, lse, sinks, dsinks, workspace)
    _need(dout.dim() == 3 and out.shape == dout.shape and out.dtype == dout.dtype,
          "dout and out must be [total_q, num_heads, head_dim] of one dtype")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (out.shape[0], out.shape[1]),
          "lse must be float32 [total_q, num_heads]")
    _need(sinks.dtype == torch.float32 and sinks.numel() == out.shape[1], "sinks must be float32 [num_heads]")
    dsinks = torch.empty_like(sinks) if dsinks is None else dsinks
    _need(dsinks.dtype == torch.float32 and dsinks.numel() == out.shape[1], "dsinks must be float32 [num_heads]")
    p = make_problem(out, 1, 1, 1, 1, 0, None, False, (-1, -1))
    p.num_kv_heads = p.num_heads
    need = int(_lib.load().varlen_attn_bwd_sinks_workspace_size(ctypes.byref(p)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = _lib.load().varlen_attn_bwd_sinks(ctypes.byref(p), _ptr(dout), _ptr(out), _ptr(lse), _ptr(sinks),
                                           _ptr(dsinks), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                           _stream(dev))
    _lib.check(st)
    return dsinks


def varlen_attn_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, sinks: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None, return_lse: bool = True):
    """Merges n partial results over disjoint key sets: o_parts [n, rows, H, D]
    (float32 or bfloat16), lse_parts float32 [n, rows, H]; sinks (float32 [H])
    are counted once here.  Returns out [rows, H, D] (and lse [rows, H])."""
    _need(o_parts.dim() == 4, "o_parts must be [n_parts, rows, num_heads, head_dim]")
    n, rows, H, D = o_parts.shape
    _need(o_parts.dtype in (torch.float32, torch.bfloat16), "o_parts must be float32 or bfloat16")
    _need(lse_parts.dtype == torch.float32 and tuple(lse_parts.shape) == (n, rows, H),
          "lse_parts must be float32 [n_parts, rows, num_heads]")
    _need(sinks is None or (sinks.dtype == torch.float32 and tuple(sinks.shape) == (H,)),
          "sinks must be float32 [num_heads]")
    dev = _check_tensors(o_parts, lse_parts, sinks, out, lse)
    if out is None:
        out = torch.empty((rows, H, D), dtype=out_dtype or o_parts.dtype, device=dev)
    _need(tuple(out.shape) == (rows, H, D) and out.dtype in _DTYPES, "out must be [rows, num_heads, head_dim]")
    if lse is None and return_lse:
        lse = torch.empty((rows, H), dtype=torch.float32, device=dev)
    _need(lse is None or (lse.dtype == torch.float32 and tuple(lse.shape) == (rows, H)),
          "lse must be float32 [rows, num_heads]")
    _lib.check(_lib.load().varlen_attn_merge(n, rows, H, D, _DTYPES[o_parts.dtype], _DTYPES[out.dtype],
                                             _ptr(o_parts), _ptr(lse_parts), _ptr(sinks), _ptr(out), _ptr(lse),
                                             _stream(dev)))
    return (out, lse) if return_lse else out


def varlen_attn_sparse_sharedkv(q, ori_kv, ori_block_table, seqused_kv, cmp_kv, cmp_block_table,
                                cmp_sparse_indices, cu_seqlens_q, max_seqlen_kv: int, *,
                                scale: Optional[float] = None, window: Tuple[int, int] = (127, 0),
                                cmp_ratio: int = 4, cmp_attend_all: bool = False, sinks=None, out=None, lse=None,
                                return_lse: bool = False):
    """Sliding-window + compressed attention over shared K/V (the three
    scenarios of the SparseAttnSharedkv README).
    q [total_q, H, D] bf16 / f16; ori_kv / cmp_kv paged caches
    [blocks, block_size, H_kv, D]; block tables int32 [batch, stride];
    seqused_kv int32 [batch]; cmp_sparse_indices int32 [total_q, H_kv, topk]
    (or None); cu_seqlens_q int32 [batch + 1].  cmp_attend_all=True (indices
    None) attends to every compressed key the causal compressed mask admits;
    otherwise to the indexed ones it admits (none: window only)."""
    dev = _check_tensors(q, ori_kv, ori_block_table, seqused_kv, cmp_kv, cmp_block_table, cmp_sparse_indices,
                         cu_seqlens_q, sinks, out, lse)
    _need(q.dim() == 3 and q.dtype in (torch.bfloat16, torch.float16), "q must be bf16 / f16 [total_q, H, D]")
    _need(ori_kv.dim() == 4 and cmp_kv.dim() == 4 and ori_kv.dtype == q.dtype and cmp_kv.dtype == q.dtype,
          "caches must be [blocks, block_size, num_kv_heads, head_dim] in q's dtype")
    _need(ori_kv.shape[2] == cmp_kv.shape[2] and ori_kv.shape[3] == q.shape[2] and cmp_kv.shape[3] == q.shape[2],
          "caches must share num_kv_heads and q's head_dim")
    for name, t in (("ori_block_table", ori_block_table), ("cmp_block_table", cmp_block_table),
                    ("seqused_kv", seqused_kv), ("cu_seqlens_q", cu_seqlens_q)):
        _need(t.dtype == torch.int32, f"{name} must be int32")
    topk = 0 if cmp_sparse_indices is None else int(cmp_sparse_indices.shape[-1])
    if cmp_sparse_indices is not None:
        _need(cmp_sparse_indices.dtype == torch.int32 and cmp_sparse_indices.dim() == 3 and
              tuple(cmp_sparse_indices.shape[:2]) == (q.shape[0], ori_kv.shape[2]),
              "cmp_sparse_indices must be int32 [total_q, num_kv_heads, topk]")
    _need(not (cmp_attend_all and cmp_sparse_indices is not None),
          "cmp_attend_all attends to every visible compressed key: pass no cmp_sparse_indices")
    p = _lib.VaSparseProblem()
    p.struct_size = ctypes.sizeof(_lib.VaSparseProblem)
    p.dtype = _DTYPES[q.dtype]
    p.batch, p.total_q = cu_seqlens_q.numel() - 1, int(q.shape[0])
    p.num_heads, p.num_kv_heads, p.head_dim = int(q.shape[1]), int(ori_kv.shape[2]), int(q.shape[2])
    p.max_seqlen_kv = int(max_seqlen_kv)
    p.scale = float(1.0 / math.sqrt(q.shape[2]) if scale is None else scale)
    p.window_left, p.window_right = int(window[0]), int(window[1])
    p.topk, p.cmp_ratio, p.cmp_attend_all = topk, int(cmp_ratio), int(bool(cmp_attend_all))
    p.ori_num_blocks, p.ori_block_size, p.ori_block_table_stride = (int(ori_kv.shape[0]), int(ori_kv.shape[1]),
                                                                    int(ori_block_table.shape[1]))
    p.cmp_num_blocks, p.cmp_block_size, p.cmp_block_table_stride = (int(cmp_kv.shape[0]), int(cmp_kv.shape[1]),
                                                                    int(cmp_block_table.shape[1]))
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=dev)
    _lib.check(_lib.load().varlen_attn_sparse_sharedkv(
        ctypes.byref(p), _ptr(q), _ptr(ori_kv), _ptr(ori_block_table), _ptr(seqused_kv), _ptr(cmp_kv),
        _ptr(cmp_block_table), _ptr(cmp_sparse_indices), _ptr(cu_seqlens_q), _ptr(sinks), _ptr(out), _ptr(lse),
        _stream(dev)))
    return (out, lse) if (return_lse or lse is not None) else out
