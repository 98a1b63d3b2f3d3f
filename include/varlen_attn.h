/*
 * varlen_attn.h -- C ABI of the variable-length packed attention forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (SparseAttnSharedkv README, formula section; boostr
 * varlen_attention.rs, varlen_attention_fwd):
 *
 *   for every sequence b, query row i < Lq_b and query head h
 *     c     = h / (H / H_kv)                       kv head shared by a GQA group
 *     s_j   = scale * <q[cu_q[b]+i, h, :], k_j[c, :]>
 *     A(i)  = { j < Lk_b : causal -> j <= p, window_left  >= 0 -> j >= p - window_left,
 *                                          window_right >= 0 -> j <= p + window_right }
 *             with p = i + Lk_b - Lq_b  (queries aligned to the end of the keys)
 *     m     = max( {s_j : j in A(i)} U {sinks[h]} )
 *     Z     = sum_{j in A(i)} exp(s_j - m) + exp(sinks[h] - m)
 *     out[cu_q[b]+i, h, :] = sum_{j in A(i)} exp(s_j - m) / Z * v_j[c, :]
 *     lse[cu_q[b]+i, h]    = m + ln Z                       (natural log, fp32)
 *
 *   The sink terms are dropped when `sinks` is NULL.  A row with no allowed
 *   key and no sink gets out = 0 and lse = -inf (never NaN).
 *
 * Layouts (all row-major, contiguous, element strides implied by the shapes):
 *   q, out        [total_q, H, D]                 "TND" packing
 *   k, v          [total_k, H_kv, D]              contiguous mode
 *   k_cache, v_cache [num_blocks, block_size, H_kv, D]   paged mode ("PA_ND")
 *   block_table   int32 [batch, block_table_stride]; key j of sequence b is
 *                 row (j % block_size) of block block_table[b][j / block_size]
 *   cu_seqlens_q  int32 [batch + 1] prefix sums (cu[0] = 0, non-decreasing,
 *                 cu[batch] = total_q); cu_seqlens_k likewise for keys
 *   seqused_k     int32 [batch] key count per sequence (paged mode)
 *   sinks         float32 [H] or NULL
 *   lse           float32 [total_q, H] or NULL when not wanted
 *   q, k, v, out share one dtype (VA_F32, VA_BF16 or VA_F16 -- the
 *   SparseAttnSharedkv README lists BF16 and FP16 inputs); out is rounded to
 *   nearest-even.  bf16 and fp16 run the same kernels (matrix cores, fp32
 *   accumulation, probabilities rounded to the input type for P V).
 *
 * Ownership and streams: every pointer handed in is caller-owned device
 * memory (except `va_problem`, which is host memory and only read during the
 * call).  Work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns without synchronising; buffers must stay alive
 * until the stream reaches the work.  The library keeps no pointer after a
 * call returns.  Only `out`, `lse` and `workspace` are written; bytes of `out`
 * outside [total_q, H, D] are never touched.
 *
 * Errors: every condition the host can check is checked before anything is
 * enqueued; a failing call launches nothing and writes nothing, returns a
 * non-zero va_status and leaves a message for varlen_attn_last_error().
 * Device-resident preconditions are not checked by default (checking needs
 * a synchronisation): cu_seqlens start at 0, never decrease and end at the
 * row totals, every length <= the max_seqlen given, 0 <= seqused_k[b] <=
 * block_table_stride * block_size, every block id used lies in
 * [0, num_blocks).  Violating them is undefined behaviour.  With the
 * environment variable VARLEN_ATTN_DEVICE_CHECK=1 (read on every call) each
 * forward call (varlen_attn_fwd, _fwd_out, _fwd_out_noalloc, _fwd_paged)
 * first runs a device-side check of exactly these conditions on its stream,
 * synchronises the stream, and returns VA_ERR_DEVICE_CHECK (nothing else
 * enqueued, out / lse untouched; the workspace may have been written) when
 * one fails.  The backward, the sink gradient, the merge and the sparse
 * shared-KV operator do not run this check.
 *
 * ABI rule: a shipped declaration never changes; a changed signature gets a
 * new _v2 name (the rule PyTorch applies to its stable C shim, per the pull
 * request "[varlen_attn for inference] add out variant").
 */
#ifndef VARLEN_ATTN_H
#define VARLEN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: forward, plan, backward.  2: adds VA_F16, va_problem.alibi_slopes,
 * varlen_attn_merge and varlen_attn_sparse_sharedkv (version 1 structs are
 * still accepted).  3: adds varlen_attn_bwd_sinks (+ its workspace size);
 * varlen_attn_bwd takes fp16 and alibi_slopes.  4: adds
 * varlen_attn_fwd_out_noalloc.  5: adds va_sparse_problem.cmp_attend_all (the
 * second scenario; version 4 descriptors are still accepted).  6: the
 * forward entry points take head_dim 512 (bf16 / fp16; varlen_attn_path 4). */
#define VARLEN_ATTN_ABI_VERSION 6

typedef enum {
    VA_OK = 0,
    VA_ERR_NULL = 1,         /* a required pointer is NULL                        */
    VA_ERR_SHAPE = 2,        /* inconsistent sizes (H % H_kv, batch < 1, totals 0) */
    VA_ERR_DTYPE = 3,        /* dtype not VA_F32 / VA_BF16 / VA_F16               */
    VA_ERR_UNSUPPORTED = 4,  /* head_dim not 64 / 128 / 512, window < -1, ...     */
    VA_ERR_ALIAS = 5,        /* out or lse overlaps an input or each other        */
    VA_ERR_ALIGN = 6,        /* a data pointer is not 16-byte aligned             */
    VA_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than required           */
    VA_ERR_HIP = 8,          /* a HIP runtime call or kernel launch failed        */
    VA_ERR_DEVICE_CHECK = 9  /* opt-in device-side argument check failed (below)  */
} va_status;

typedef enum { VA_F32 = 0, VA_BF16 = 1, VA_F16 = 2 } va_dtype;

/* Problem description, host memory.  Field meaning follows the argument list
 * of the out-variant op in the pull request "[varlen_attn for inference] add
 * out variant" (max_q / max_k, scale, window_size_left / right, seqused_k,
 * page_table) and the SparseAttnSharedkv README parameter table. */
typedef struct {
    uint32_t struct_size;     /* sizeof(va_problem); allows appending fields      */
    int32_t dtype;            /* va_dtype of q, k, v, out                          */
    int32_t batch;            /* B >= 1                                            */
    int32_t total_q;          /* rows of q / out (>= 1)                            */
    int32_t total_k;          /* rows of k / v (contiguous mode; ignored if paged) */
    int32_t num_heads;        /* H                                                 */
    int32_t num_kv_heads;     /* H_kv, divides H                                   */
    int32_t head_dim;         /* D: 64 or 128; 512 with bf16 / fp16 (forward)      */
    int32_t max_seqlen_q;     /* host upper bound of every Lq_b (grid sizing only) */
    int32_t max_seqlen_k;     /* host upper bound of every Lk_b                    */
    float scale;              /* multiplies q.k (not the sink); > 0                */
    int32_t causal;           /* 0 / 1; aligned to the end of the keys             */
    int32_t window_left;      /* keys before the query position, -1 = unbounded   */
    int32_t window_right;     /* keys after the query position, -1 = unbounded    */
    int32_t num_blocks;       /* paged: blocks in the cache                        */
    int32_t block_size;       /* paged: tokens per block, multiple of 16, <= 1024  */
    int32_t block_table_stride; /* paged: int32 entries per block_table row        */
    /* Fields below were appended in ABI version 2; a caller whose struct_size
     * ends before a field gets its default (NULL). */
    const float *alibi_slopes;  /* device float32 [H] or NULL: the score of query
                                 * i and key j of head h gets
                                 * - alibi_slopes[h] * |i + Lk - Lq - j|
                                 * (distance to the query's end-aligned position,
                                 * added after the scale; sinks unaffected).  The
                                 * pages list alibi_slopes in the op schema of the
                                 * pull request "[varlen_attn for inference] add
                                 * out variant" without its formula; this is the
                                 * reading taken.  Used by every forward kernel
                                 * and by varlen_attn_bwd (the slopes get no
                                 * gradient).                                     */
} va_problem;

/* Library helper (no passage of the pages defines it).  Bytes of device
 * workspace `varlen_attn_fwd_out` (paged = 0) or `varlen_attn_fwd_paged`
 * (paged = 1) needs for this problem; 0 if the problem is invalid (the entry
 * point then reports why). */
size_t varlen_attn_workspace_size(const va_problem *p, int paged);

/* Out variant, contiguous K/V: writes out [total_q, H, D] (and lse when not
 * NULL) into caller buffers.  `workspace` is device memory of at least
 * varlen_attn_workspace_size(p, 0) bytes, used only during the enqueued work;
 * its contents on entry do not matter.  (Pull request "[varlen_attn for
 * inference] add out variant": one implementation behind an allocating entry
 * point and an out entry point.) */
va_status varlen_attn_fwd_out(const va_problem *p, const void *q, const void *k,
                              const void *v, const int32_t *cu_seqlens_q,
                              const int32_t *cu_seqlens_k, const float *sinks,
                              void *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Allocating variant: same computation as varlen_attn_fwd_out (bitwise the
 * same results).  Allocates *out (total_q * H * D elements of the dtype) and,
 * when lse != NULL, *lse (total_q * H floats) stream-ordered on `stream`; the
 * caller releases them with varlen_attn_free.  The workspace is allocated and
 * released internally, stream-ordered.  On error nothing is allocated and
 * *out / *lse are set to NULL. */
va_status varlen_attn_fwd(const va_problem *p, const void *q, const void *k,
                          const void *v, const int32_t *cu_seqlens_q,
                          const int32_t *cu_seqlens_k, const float *sinks,
                          void **out, float **lse, void *stream);

/* Out variant for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and arguments as varlen_attn_fwd_out (bitwise the same results)
 * without a workspace argument.  The work list and the decode partials live
 * in a 64 MiB device array inside the library, one per device, held until the
 * process ends; its address is resolved on the first call on a device.  A
 * call whose workspace would exceed 64 MiB (varlen_attn_workspace_size(p, 0))
 * returns VA_ERR_WORKSPACE and enqueues nothing.  The call allocates nothing
 * and needs no cleared memory (the pre-pass rewrites everything it reads).
 * All calls on one device share that array: calls that overlap in time on
 * one device (on different streams, or from different threads without
 * stream ordering) race and give undefined results. */
va_status varlen_attn_fwd_out_noalloc(const va_problem *p, const void *q, const void *k,
                                      const void *v, const int32_t *cu_seqlens_q,
                                      const int32_t *cu_seqlens_k, const float *sinks,
                                      void *out, float *lse, void *stream);

/* Paged K/V (SparseAttnSharedkv README, PageAttention constraints; pull
 * request "[varlen_attn for inference] add out variant", page_table and
 * seqused_k arguments): key length of sequence b is seqused_k[b]; keys are
 * read through block_table.  Caches may alias each other (K == V). */
va_status varlen_attn_fwd_paged(const va_problem *p, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_table,
                                const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                                const float *sinks, void *out, float *lse,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Library helper (no passage of the pages defines it): releases memory
 * returned by varlen_attn_fwd, stream-ordered. */
va_status varlen_attn_free(void *ptr, void *stream);

/* Work partition of a call (the GPU pre-pass that maps ragged sequences to
 * tiles, in the role of the partition metadata operator that precedes
 * SparseAttnSharedkv): runs only that pre-pass and copies its list into
 * `items` (device int32 [capacity][4]: sequence, first query row or split
 * index, first key, end key) and the count into `count` (device int32 [1]),
 * in execution order.  `seqlens_k` is cu_seqlens_k (paged = 0) or seqused_k
 * (paged = 1).  With capacity 0, items and count may be NULL and only the
 * pre-pass runs (used to time it).  For tests of the partition. */
va_status varlen_attn_plan(const va_problem *p, int paged, const int32_t *cu_seqlens_q,
                           const int32_t *seqlens_k, int32_t *items, int32_t capacity,
                           int32_t *count, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Backward (bf16 or fp16, contiguous K/V), following the boostr CPU backward
 * varlen_attention_bwd: given dout [total_q, H, D] and the forward's out and
 * lse (lse carries any sink), writes
 *   dq [total_q, H, D] = scale * sum_j dS_ij k_j
 *   dk [total_k, H_kv, D] = scale * sum_i dS_ij q_i,  dv [total_k, H_kv, D] = sum_i P_ij dout_i
 * with P_ij = exp(scale <q_i, k_j> - lse_i) over the allowed keys of the
 * forward (same causal / window arguments), dS_ij = P_ij (<dout_i, v_j> -
 * sum_d dout_i,d out_i,d), and dk / dv of a kv head summed over the query
 * heads that share it; with p->alibi_slopes the scores carry the forward's
 * bias (-slope_h |i + Lk - Lq - j|, the slopes being an input like q).  dq,
 * dk, dv are in the input dtype (accumulated
 * in float32) and fully overwritten; keys no query sees get zero gradients.
 * The gradient of the sink logits is varlen_attn_bwd_sinks' output.  Same
 * ownership, stream and error rules as the forward (without the opt-in
 * device check); dq, dk, dv may not overlap any input, the
 * workspace or each other; p->dtype must be VA_BF16 or VA_F16 and head_dim
 * 64 or 128 (else VA_ERR_UNSUPPORTED).  `workspace` holds at least
 * varlen_attn_bwd_workspace_size(p) bytes (a library helper; 0 for an
 * invalid p). */
size_t varlen_attn_bwd_workspace_size(const va_problem *p);
va_status varlen_attn_bwd(const va_problem *p, const void *dout, const void *q, const void *k,
                          const void *v, const void *out, const float *lse,
                          const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, void *dq,
                          void *dk, void *dv, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Gradient of the sink logits (bf16 or fp16 forward, D in {64, 128}).  The
 * sink of head h is one more logit s_h of every query row's softmax with a
 * zero value row (SparseAttnSharedkv README, sinks parameter), so
 *   dsinks[h] = - sum_i exp(sinks[h] - lse[i][h]) * sum_d dout[i][h][d] out[i][h][d]
 * over all query rows i (the chain rule through the softmax; dq, dk, dv are
 * the ones varlen_attn_bwd writes, which the sinks enter only through lse).
 *   dout, out   [total_q, H, D] in p->dtype (out and lse from the forward
 *               call that had these sinks)
 *   lse         float32 [total_q, H];  sinks  float32 [H]
 *   dsinks      float32 [H], overwritten; summed in a fixed order, so the
 *               result is the same on every run
 * p is validated as for the forward; only its dtype, total_q, num_heads
 * and head_dim shape the work (the masks enter through out and lse).  `workspace` holds at least
 * varlen_attn_bwd_sinks_workspace_size(p) bytes (0 for an invalid p).  Same
 * ownership, stream and error rules as the forward; dsinks may not overlap
 * an input or the workspace. */
size_t varlen_attn_bwd_sinks_workspace_size(const va_problem *p);
va_status varlen_attn_bwd_sinks(const va_problem *p, const void *dout, const void *out, const float *lse,
                                const float *sinks, float *dsinks, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Merge of partial attention results computed over disjoint key sets of
 * the same queries: the local step of ring / context-parallel attention,
 * where each rank attends its queries to its share of the keys (the joint
 * K/V that the vllm-omni ulysses.py wrapper hands to its ring path) and the
 * partials are combined through their log-sum-exp.  For each (row, head),
 * with parts p = 0 .. n_parts-1 and sigma = sinks[head] (absent: -inf):
 *   m = max(max_p lse_p, sigma),  s = sum_p exp(lse_p - m) + exp(sigma - m),
 *   lse = m + log(s),             out = sum_p exp(lse_p - lse) o_p.
 * The result is the attention over the union of the key sets; a sink is
 * counted once here, so the partials must be computed without sinks.  A
 * part with lse_p = -inf contributes nothing; if every part is empty and
 * there is no sink, out = 0 and lse = -inf (with a sink: out = 0,
 * lse = sigma).
 *   o_parts    device [n_parts, rows, num_heads, head_dim], parts_dtype
 *   lse_parts  device float32 [n_parts, rows, num_heads], natural log
 *   sinks      device float32 [num_heads] or NULL
 *   out        device [rows, num_heads, head_dim], out_dtype (bf16: round to
 *              nearest even), fully overwritten
 *   lse        device float32 [rows, num_heads] or NULL
 * n_parts in [1, 4096]; head_dim a multiple of 8 in [8, 1024]; o_parts and
 * out 16-byte aligned, the float arrays 4-byte aligned; out and lse must not
 * overlap an input or each other.  Enqueued on `stream`; nothing is
 * allocated; a failing check returns before any launch. */
va_status varlen_attn_merge(int32_t n_parts, int32_t rows, int32_t num_heads, int32_t head_dim,
                            va_dtype parts_dtype, va_dtype out_dtype, const void *o_parts,
                            const float *lse_parts, const float *sinks, void *out, float *lse,
                            void *stream);

/* Sliding-window + compressed attention over shared K/V: the three
 * scenarios of the SparseAttnSharedkv README (K~ = V~ in its formula: one
 * tensor row serves as key and value).  For token t (row i of sequence b,
 * Lq_b rows, S2_b = seqused_kv[b] original keys, S3_b = S2_b / cmp_ratio
 * compressed keys) and each query head h of kv head c:
 *   window keys:   original positions j in [p - window_left, p + window_right]
 *                  and [0, S2_b), p = i + S2_b - Lq_b (aligned to the end),
 *                  read from ori_kv through ori_block_table;
 *   compressed keys, read from cmp_kv through cmp_block_table, visible up to
 *                  last = i + S3_b - Lq_b (its mask mode 3 read as causal,
 *                  aligned to the bottom-right corner of the Lq_b x S3_b
 *                  matrix, as mode 4 aligns the window to the end):
 *     cmp_attend_all = 1 (second scenario): every position 0 .. last;
 *     cmp_attend_all = 0 (third scenario):  the positions
 *                  cmp_sparse_indices[t][c][0 .. topk-1]; one outside
 *                  [0, last] selects nothing, a repeated one is attended as
 *                  often as it appears; topk = 0 gives the first scenario;
 *   out[t][h] = sum_j w_j kv_j,  w = softmax over the window and compressed
 *               keys of scale <q[t][h], kv_j>, with sinks[h] as an extra logit;
 *   lse[t][h] = natural log of that softmax's denominator.
 * The README does not define the compression operator: the compressed rows
 * are inputs.
 *   q, out            [total_q, H, D] dtype (VA_BF16 / VA_F16), TND
 *   ori_kv            [ori_num_blocks, ori_block_size, H_kv, D], PA_ND
 *   cmp_kv            [cmp_num_blocks, cmp_block_size, H_kv, D], PA_ND
 *   ori_block_table   int32 [batch, ori_block_table_stride]
 *   cmp_block_table   int32 [batch, cmp_block_table_stride]
 *   seqused_kv        int32 [batch], <= max_seqlen_kv
 *   cmp_sparse_indices int32 [total_q, H_kv, topk] (NULL iff topk = 0)
 *   cu_seqlens_q      int32 [batch + 1]; sinks float32 [H] or NULL;
 *   lse               float32 [total_q, H] or NULL
 * Limits: D in {64, 128, 512} (512 is the README's head size); H / H_kv <= 64;
 * window sides >= 0 (a side >= 2^30 is unbounded);
 * cmp_ratio >= 1; cmp_attend_all needs topk = 0.  A descriptor whose
 * struct_size ends before cmp_attend_all (ABI 4 callers) reads it as 0.  Same
 * ownership, stream, alignment and aliasing rules as the forward; nothing
 * is allocated and no workspace is needed. */
typedef struct {
    uint32_t struct_size;       /* sizeof(va_sparse_problem)                    */
    int32_t dtype;              /* VA_BF16 or VA_F16                            */
    int32_t batch, total_q;     /* B >= 1, rows of q (>= 1)                     */
    int32_t num_heads, num_kv_heads, head_dim;
    int32_t max_seqlen_kv;      /* host bound of every seqused_kv[b]            */
    float scale;                /* > 0                                          */
    int32_t window_left, window_right;
    int32_t topk;               /* selected compressed keys per (token, kv head) */
    int32_t cmp_ratio;          /* compressed keys of sequence b: S2_b / ratio  */
    int32_t ori_num_blocks, ori_block_size, ori_block_table_stride;
    int32_t cmp_num_blocks, cmp_block_size, cmp_block_table_stride;
    int32_t cmp_attend_all;     /* 1: every visible compressed key (no indices) */
} va_sparse_problem;

va_status varlen_attn_sparse_sharedkv(const va_sparse_problem *p, const void *q, const void *ori_kv,
                                      const int32_t *ori_block_table, const int32_t *seqused_kv,
                                      const void *cmp_kv, const int32_t *cmp_block_table,
                                      const int32_t *cmp_sparse_indices, const int32_t *cu_seqlens_q,
                                      const float *sinks, void *out, float *lse, void *stream);

/* Library helpers (no passage of the pages defines them).
 * Which kernel family a call with these arguments would use:
 * 0 = prefill tiles, 1 = split-KV decode with combine, 2 = float32 path,
 * 3 = sliding-window kernel (16-bit K/V, contiguous or paged, 32..64 query
 * heads per kv head, window bounded on both sides, no ALiBi), 4 = head size
 * 512 (every shape); -1 if invalid. */
int varlen_attn_path(const va_problem *p, int paged);

/* Thread-local text for the last non-OK status returned on this thread. */
const char *varlen_attn_last_error(void);

/* VARLEN_ATTN_ABI_VERSION of the built library. */
int varlen_attn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VARLEN_ATTN_H */
