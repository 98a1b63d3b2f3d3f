"""Variable-length packed attention forward for AMD Instinct MI355X (gfx950).

softmax(Q K^T * scale) V over ragged sequences packed in TND layout and
delimited by cu_seqlens, with GQA, causal / sliding-window masks, per-head
sink logits and an optional paged KV cache; writes O into a caller buffer and
returns the float32 log-sum-exp; an out variant that allocates nothing; its
backward (dq, dk, dv, and the sink-logit gradient) for bf16 / fp16
contiguous K/V; the log-sum-exp merge of partial results over disjoint key
sets; and sliding-window + compressed attention over shared K/V.  Head sizes
64 and 128 (and 512 for the 16-bit forward and the shared-KV op).  The
computation runs in hand-written HIP kernels behind the C ABI of
include/varlen_attn.h; this package only binds it.
"""
from .api import (bwd_workspace_size, kernel_path, make_problem, output_shapes, plan, varlen_attn,
                  varlen_attn_bwd, varlen_attn_bwd_sinks, varlen_attn_fwd, varlen_attn_merge, varlen_attn_out,
                  varlen_attn_out_noalloc, varlen_attn_paged, varlen_attn_sparse_sharedkv, workspace_size)

__all__ = ["varlen_attn", "varlen_attn_out", "varlen_attn_out_noalloc", "varlen_attn_paged", "varlen_attn_fwd", "varlen_attn_bwd",
           "varlen_attn_bwd_sinks", "varlen_attn_merge", "varlen_attn_sparse_sharedkv", "workspace_size", "bwd_workspace_size", "plan", "kernel_path", "output_shapes", "make_problem"]
