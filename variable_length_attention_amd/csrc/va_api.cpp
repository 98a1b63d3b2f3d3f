// C ABI of the varlen attention library: argument validation, workspace
// layout, kernel choice and launches on the caller's stream.  No torch here;
// declarations and contracts are in include/varlen_attn.h.
//
// Structure follows the out-variant pull request for PyTorch's varlen
// attention ("[varlen_attn for inference] add out variant"): one core
// implementation (`run`) behind an out entry point and an allocating entry
// point, so the two are bitwise identical.
#include "../../include/varlen_attn.h"
#include "va_internal.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

va_status fail(va_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool log_enabled()
{
    static const bool on = [] {
        const char *e = std::getenv("VARLEN_ATTN_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

// VARLEN_ATTN_DEVICE_CHECK=1 turns on the device-side argument check (read
// on every call so that it can be switched within a process).
bool device_check_enabled()
{
    const char *e = std::getenv("VARLEN_ATTN_DEVICE_CHECK");
    return e && e[0] == '1';
}

enum Path { kPathPrefill = 0, kPathDecode = 1, kPathF32 = 2, kPathWindow = 3, kPath512 = 4 };

struct Layout {
    int path = -1;
    int hpw = 1;                 // prefill: query heads per workgroup
    int n_max = 0;
    int bm = 0, bn = 0;
    long long grid = 0;
    size_t off_count = 0, off_seq = 0, off_unsorted = 0, off_cost = 0, off_items = 0, off_seqinfo = 0;
    size_t off_part_ml = 0, off_part_o = 0, total = 0;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Size of the version-1 va_problem (fields up to block_table_stride); later
// fields take their defaults when struct_size ends before them.
constexpr size_t kProblemV1 = offsetof(va_problem, block_table_stride) + sizeof(int32_t);
const float *alibi_of(const va_problem *p)
{
    return p->struct_size >= offsetof(va_problem, alibi_slopes) + sizeof(p->alibi_slopes) ? p->alibi_slopes
                                                                                          : nullptr;
}

// Validation of the problem description alone (no pointers).
va_status check_problem(const va_problem *p, int paged)
{
    if (!p) return fail(VA_ERR_NULL, "problem descriptor is NULL");
    if (p->struct_size < kProblemV1)
        return fail(VA_ERR_SHAPE, "va_problem.struct_size %u is smaller than %zu", p->struct_size, kProblemV1);
    if (p->dtype != VA_F32 && p->dtype != VA_BF16 && p->dtype != VA_F16)
        return fail(VA_ERR_DTYPE, "dtype %d is not VA_F32 (0), VA_BF16 (1) or VA_F16 (2)", p->dtype);
    if (p->batch < 1) return fail(VA_ERR_SHAPE, "batch %d < 1", p->batch);
    if (p->total_q < 1) return fail(VA_ERR_SHAPE, "total_q %d < 1 (empty tensors are not accepted)", p->total_q);
    if (!paged && p->total_k < 1)
        return fail(VA_ERR_SHAPE, "total_k %d < 1 (empty tensors are not accepted)", p->total_k);
    if (p->num_heads < 1 || p->num_kv_heads < 1)
        return fail(VA_ERR_SHAPE, "num_heads %d / num_kv_heads %d must be >= 1", p->num_heads, p->num_kv_heads);
    if (p->num_heads % p->num_kv_heads != 0)
        return fail(VA_ERR_SHAPE, "num_heads %d is not a multiple of num_kv_heads %d", p->num_heads,
                    p->num_kv_heads);
    if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 512)
        return fail(VA_ERR_UNSUPPORTED, "head_dim %d is not 64, 128 or 512", p->head_dim);
    if (p->head_dim == 512 && p->dtype == VA_F32)
        return fail(VA_ERR_UNSUPPORTED, "head_dim 512 takes bf16 or fp16 inputs");
    if (p->max_seqlen_q < 1 || p->max_seqlen_q > va::kMaxSeqlen)
        return fail(VA_ERR_SHAPE, "max_seqlen_q %d outside [1, %d]", p->max_seqlen_q, va::kMaxSeqlen);
    if (p->max_seqlen_k < 0 || p->max_seqlen_k > va::kMaxSeqlen)
        return fail(VA_ERR_SHAPE, "max_seqlen_k %d outside [0, %d]", p->max_seqlen_k, va::kMaxSeqlen);
    if (!std::isfinite(p->scale) || !(p->scale > 0.f))
        return fail(VA_ERR_UNSUPPORTED, "scale must be finite and > 0");
    if (p->causal != 0 && p->causal != 1) return fail(VA_ERR_UNSUPPORTED, "causal must be 0 or 1");
    if (p->window_left < -1 || p->window_right < -1)
        return fail(VA_ERR_UNSUPPORTED, "window (%d, %d): values below -1 are not defined", p->window_left,
                    p->window_right);
    if (paged) {
        if (p->num_blocks < 1) return fail(VA_ERR_SHAPE, "num_blocks %d < 1", p->num_blocks);
        if (p->block_size < 16 || p->block_size > 1024 || p->block_size % 16 != 0)
            return fail(VA_ERR_UNSUPPORTED, "block_size %d is not a multiple of 16 in [16, 1024]", p->block_size);
        const long long need = ((long long)p->max_seqlen_k + p->block_size - 1) / p->block_size;
        if (p->block_table_stride < 1 || p->block_table_stride < need)
            return fail(VA_ERR_SHAPE, "block_table_stride %d < ceil(max_seqlen_k / block_size) = %lld",
                        p->block_table_stride, need);
    }
    return VA_OK;
}

// Query rows per work item of the sliding-window kernel, or 0 when it does
// not apply: 16-bit K/V (contiguous or paged), no ALiBi, 32..64 query heads
// per kv head, a window bounded on both sides (causal bounds the right
// side) that leaves room for at least 4 rows in the LDS window.  About 2048
// items per kv head fill the chip several times over; more rows per item
// share more of the window.
int window_rows(const va_problem *p)
{
    const int g = p->num_heads / p->num_kv_heads;
    const int right = p->causal ? 0 : p->window_right;
    if (p->dtype == VA_F32 || alibi_of(p) || g < 32 || g > 64 || p->window_left < 0 || right < 0)
        return 0;
    const long long room = (long long)va::win_cap(p->head_dim) - p->window_left - right;
    if (room < 4) return 0;
    const long long want = ((long long)p->total_q * p->num_kv_heads + 2047) / 2048;
    return (int)std::max<long long>(4, std::min<long long>({room, want, 32}));
}

va_status make_layout(const va_problem *p, int paged, Layout &L)
{
    const int g = p->num_heads / p->num_kv_heads;
    const int wrows = window_rows(p);
    if (p->head_dim == 512) {
        // every shape at head size 512: the prefill items, 32-key tiles
        L.path = kPath512;
        L.bm = va::kBM;
        L.bn = 32;
    } else if (p->dtype == VA_F32) {
        L.path = kPathF32;
        L.bm = va::kBMf32;
        L.bn = va::kBNf32;
    } else if ((long long)g * p->max_seqlen_q <= va::kDecRows) {
        L.path = kPathDecode;
    } else if (wrows > 0) {
        L.path = kPathWindow;
        L.bm = wrows;
        L.bn = va::kBN;
    } else {
        L.path = kPathPrefill;
        // GQA groups of a multiple of 4 heads: a workgroup takes 32 rows of
        // an item for 4 heads (the items stay 128 rows: the same pre-pass)
        L.hpw = g % 4 == 0 ? 4 : 1;
        L.bm = va::kBM;
        L.bn = va::kBN;
    }
    long long n_max;
    if (L.path == kPathDecode) {
        n_max = va::kDecTargetUnits / p->num_kv_heads + (long long)p->batch + 1;
        L.grid = n_max * p->num_kv_heads;
    } else if (L.path == kPathWindow) {
        n_max = ((long long)p->total_q + (long long)p->batch * (L.bm - 1)) / L.bm;
        L.grid = n_max * p->num_kv_heads;
    } else {
        n_max = ((long long)p->total_q + (long long)p->batch * (L.bm - 1)) / L.bm;
        L.grid = n_max * p->num_heads;
    }
    if (L.grid > 0x7fffffffLL || n_max > 0x7fffffffLL)
        return fail(VA_ERR_UNSUPPORTED, "problem needs %lld workgroups, above the launch limit", L.grid);
    L.n_max = (int)n_max;
    size_t off = 0;
    L.off_count = off; off = align_up(off + 4, 256);
    L.off_seq = off; off = align_up(off + 4 * ((size_t)p->batch + 1), 256);
    L.off_unsorted = off; off = align_up(off + 16 * (size_t)n_max, 256);
    L.off_cost = off; off = align_up(off + 4 * (size_t)n_max, 256);
    L.off_items = off; off = align_up(off + 16 * (size_t)n_max, 256);
    L.off_seqinfo = off; off = align_up(off + 16 * (size_t)n_max, 256);
    if (L.path == kPathDecode) {
        const size_t rows = (size_t)n_max * p->num_kv_heads * va::kDecRows;
        L.off_part_ml = off; off = align_up(off + 8 * rows, 256);
        L.off_part_o = off; off = align_up(off + 4 * rows * p->head_dim, 256);
    }
    L.total = off;
    return VA_OK;
}

struct Range {
    const void *p;
    size_t bytes;
};

bool overlaps(const Range &a, const Range &b)
{
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Call {
    const va_problem *p;
    int paged;
    const void *q, *k, *v;
    const int32_t *cu_q, *cu_k, *seqused_k, *block_table;
    const float *sinks;
    void *out;
    float *lse;
    void *ws;
    size_t ws_bytes;
};

va_status check_pointers(const Call &c, const Layout &L)
{
    const va_problem *p = c.p;
    if (!c.q || !c.k || !c.v) return fail(VA_ERR_NULL, "q, k and v must be non-NULL");
    if (!c.cu_q) return fail(VA_ERR_NULL, "cu_seqlens_q must be non-NULL");
    if (c.paged) {
        if (!c.block_table || !c.seqused_k) return fail(VA_ERR_NULL, "block_table and seqused_k must be non-NULL");
    } else if (!c.cu_k) {
        return fail(VA_ERR_NULL, "cu_seqlens_k must be non-NULL");
    }
    if (!c.out) return fail(VA_ERR_NULL, "out must be non-NULL");
    if (L.total > 0 && !c.ws) return fail(VA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
    if (c.ws_bytes < L.total)
        return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", c.ws_bytes, L.total);
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.out, 16) ||
        (c.ws && !aligned(c.ws, 16)))
        return fail(VA_ERR_ALIGN, "q, k, v, out and workspace must be 16-byte aligned");
    if (!aligned(c.cu_q, 4) || (c.cu_k && !aligned(c.cu_k, 4)) || (c.seqused_k && !aligned(c.seqused_k, 4)) ||
        (c.block_table && !aligned(c.block_table, 4)) || (c.sinks && !aligned(c.sinks, 4)) ||
        (c.lse && !aligned(c.lse, 4)) || (alibi_of(p) && !aligned(alibi_of(p), 4)))
        return fail(VA_ERR_ALIGN, "int32 / float32 arrays must be 4-byte aligned");

    const size_t es = p->dtype == VA_F32 ? 4 : 2;
    const size_t D = (size_t)p->head_dim;
    const size_t kv_rows = c.paged ? (size_t)p->num_blocks * p->block_size : (size_t)p->total_k;
    const Range out{c.out, (size_t)p->total_q * p->num_heads * D * es};
    const Range lse{c.lse, c.lse ? (size_t)p->total_q * p->num_heads * 4 : 0};
    const Range ins[] = {
        {c.q, (size_t)p->total_q * p->num_heads * D * es},
        {c.k, kv_rows * p->num_kv_heads * D * es},
        {c.v, kv_rows * p->num_kv_heads * D * es},
        {c.cu_q, 4 * ((size_t)p->batch + 1)},
        {c.cu_k, c.cu_k ? 4 * ((size_t)p->batch + 1) : 0},
        {c.seqused_k, c.seqused_k ? 4 * (size_t)p->batch : 0},
        {c.block_table, c.block_table ? 4 * (size_t)p->batch * p->block_table_stride : 0},
        {c.sinks, c.sinks ? 4 * (size_t)p->num_heads : 0},
        {alibi_of(p), alibi_of(p) ? 4 * (size_t)p->num_heads : 0},
        {c.ws, c.ws_bytes},
    };
    for (const Range &r : ins) {
        if (overlaps(out, r)) return fail(VA_ERR_ALIAS, "out overlaps an input, the workspace or lse");
        if (overlaps(lse, r)) return fail(VA_ERR_ALIAS, "lse overlaps an input or the workspace");
    }
    if (overlaps(out, lse)) return fail(VA_ERR_ALIAS, "out overlaps lse");
    return VA_OK;
}

va::AttnArgs make_args(const Call &c)
{
    const va_problem *p = c.p;
    va::AttnArgs a;
    a.q = c.q; a.k = c.k; a.v = c.v;
    a.out = c.out; a.lse = c.lse;
    a.cu_q = c.cu_q; a.cu_k = c.cu_k; a.seqused_k = c.seqused_k; a.block_table = c.block_table;
    a.sinks = c.sinks;
    a.alibi = alibi_of(p);
    a.B = p->batch; a.H = p->num_heads; a.Hkv = p->num_kv_heads; a.g = p->num_heads / p->num_kv_heads;
    a.bt_stride = c.paged ? p->block_table_stride : 0;
    a.block_size = c.paged ? p->block_size : 1;
    a.bs_shift = -1;
    for (int sh = 0; sh < 11; ++sh)
        if ((1 << sh) == a.block_size) a.bs_shift = sh;
    a.left = p->window_left >= 0 ? p->window_left : va::kInfOff;
    // causal caps the right side at the query position: min(window_right, 0)
    // with window_right >= -1 and -1 meaning unbounded is always 0
    if (p->causal) a.right = 0;
    else a.right = p->window_right >= 0 ? p->window_right : va::kInfOff;
    a.scale = p->scale;
    a.scale_log2 = p->scale * va::kLog2e;
    a.item_rows = 0;
    a.hpw = 1;
    return a;
}

va::PlanArgs make_plan(const Call &c, const Layout &L, const va::AttnArgs &a)
{
    char *ws = (char *)c.ws;
    va::PlanArgs pa;
    pa.cu_q = c.cu_q;
    pa.lens_k = c.paged ? c.seqused_k : c.cu_k;
    pa.lens_k_is_prefix = c.paged ? 0 : 1;
    pa.B = a.B; pa.Hkv = a.Hkv;
    pa.left = a.left; pa.right = a.right;
    pa.mode = L.path == kPathDecode ? va::kPlanDecode : L.path == kPathWindow ? va::kPlanWindow : va::kPlanPrefill;
    pa.bm = L.bm; pa.bn = L.bn;
    pa.n_max = L.n_max;
    pa.count = (int32_t *)(ws + L.off_count);
    pa.seq_off = (int32_t *)(ws + L.off_seq);
    pa.unsorted = (int4 *)(ws + L.off_unsorted);
    pa.cost = (int32_t *)(ws + L.off_cost);
    pa.items = (int4 *)(ws + L.off_items);
    pa.seqinfo = (int4 *)(ws + L.off_seqinfo);
    return pa;
}

// Device-side check of the argument contents; synchronises the stream.  The
// result word lives in the workspace's item-count slot, which the pre-pass
// overwrites afterwards.
va_status device_check(const Call &c, const Layout &L, hipStream_t s)
{
    const va_problem *p = c.p;
    va::CheckArgs ck;
    ck.cu_q = c.cu_q;
    ck.cu_k = c.paged ? nullptr : c.cu_k;
    ck.seqused_k = c.paged ? c.seqused_k : nullptr;
    ck.block_table = c.paged ? c.block_table : nullptr;
    ck.B = p->batch; ck.total_q = p->total_q; ck.total_k = p->total_k;
    ck.max_q = p->max_seqlen_q; ck.max_k = p->max_seqlen_k;
    ck.bt_stride = c.paged ? p->block_table_stride : 0;
    ck.block_size = c.paged ? p->block_size : 1;
    ck.num_blocks = c.paged ? p->num_blocks : 0;
    ck.flags = (uint32_t *)((char *)c.ws + L.off_count);
    uint32_t flags = 0;
    hipError_t e = va::launch_check(ck, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&flags, ck.flags, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "device check failed to run: %s", hipGetErrorString(e));
    if (!flags) return VA_OK;
    static const char *const what[] = {
        "cu_seqlens_q[0] != 0", "cu_seqlens_q decreases", "cu_seqlens_q[batch] != total_q",
        "a query length exceeds max_seqlen_q", "cu_seqlens_k[0] != 0", "cu_seqlens_k decreases",
        "cu_seqlens_k[batch] != total_k", "a key length exceeds max_seqlen_k",
        "seqused_k is negative or exceeds block_table_stride * block_size",
        "a used block id is outside [0, num_blocks)"};
    for (int i = 0; i < 10; ++i)
        if (flags & (1u << i)) return fail(VA_ERR_DEVICE_CHECK, "device check: %s (flags 0x%x)", what[i], flags);
    return fail(VA_ERR_DEVICE_CHECK, "device check failed (flags 0x%x)", flags);
}

// The one implementation behind every entry point.
va_status run(const Call &c, hipStream_t s)
{
    va_status st = check_problem(c.p, c.paged);
    if (st) return st;
    Layout L;
    if ((st = make_layout(c.p, c.paged, L))) return st;
    if ((st = check_pointers(c, L))) return st;
    va::AttnArgs a = make_args(c);
    a.item_rows = L.path == kPathWindow ? L.bm : 0;
    a.hpw = L.hpw;
    const va::PlanArgs pa = make_plan(c, L, a);
    if (device_check_enabled() && (st = device_check(c, L, s))) return st;
    if (log_enabled())
        fprintf(stderr, "[varlen_attn] path=%s D=%d paged=%d B=%d H=%d Hkv=%d total_q=%d grid=%lld ws=%zu\n",
                L.path == kPathPrefill ? "prefill16" : L.path == kPathDecode ? "decode16"
                                                   : L.path == kPathWindow ? "window16"
                                                   : L.path == kPath512    ? "prefill512" : "f32",
                c.p->head_dim, c.paged, a.B, a.H, a.Hkv, c.p->total_q, L.grid, L.total);
    hipError_t e = va::launch_plan(pa, s);
    if (e == hipSuccess) {
        if (L.path == kPathPrefill)
        {
            const size_t span = (size_t)c.p->max_seqlen_k * c.p->num_kv_heads * c.p->head_dim * 2;
            const int mode = c.paged ? va::kLoadPaged : (span < ((size_t)1 << 31) ? va::kLoadBuffer : va::kLoadGlobal);
            e = va::launch_prefill16(a, c.p->dtype == VA_F16, a.alibi != nullptr, c.p->head_dim, mode, pa.items,
                                     pa.seqinfo, pa.count, (int)L.grid, s);
        }
        else if (L.path == kPathWindow)
            e = va::launch_window16(a, c.p->dtype == VA_F16, c.p->head_dim, c.paged, pa.items, pa.seqinfo,
                                    pa.count, (int)L.grid, s);
        else if (L.path == kPathF32)
            e = va::launch_prefill_f32(a, c.p->head_dim, c.paged, pa.items, pa.seqinfo, pa.count, (int)L.grid, s);
        else if (L.path == kPath512)
            e = va::launch_prefill512(a, c.p->dtype == VA_F16, c.paged, pa.items, pa.seqinfo, pa.count, (int)L.grid, s);
        else {
            char *ws = (char *)c.ws;
            float *po = (float *)(ws + L.off_part_o);
            float2 *pml = (float2 *)(ws + L.off_part_ml);
            const bool f16 = c.p->dtype == VA_F16;
            e = va::launch_decode16(a, f16, c.p->head_dim, c.paged, pa.items, pa.seqinfo, pa.count, (int)L.grid, po,
                                    pml, s);
            if (e == hipSuccess) e = va::launch_decode_combine(a, f16, c.p->head_dim, pa.seq_off, po, pml, s);
        }
    }
    if (e != hipSuccess) return fail(VA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return VA_OK;
}

// ---------------------------------------------------------------- backward
// Workspace: the two pre-pass plans (query blocks for dQ, key blocks for
// dK / dV) and Dv [T_q, H] fp32.
struct PlanRegion {
    size_t count = 0, seq = 0, unsorted = 0, cost = 0, items = 0, seqinfo = 0;
    int n_max = 0;
    long long grid = 0;
};
struct BwdLayout {
    PlanRegion qp, kp;
    size_t dvec = 0;
    size_t total = 0;
};

size_t plan_region(size_t off, int B, int n_max, PlanRegion &r)
{
    r.n_max = n_max;
    r.count = off; off = align_up(off + 4, 256);
    r.seq = off; off = align_up(off + 4 * ((size_t)B + 1), 256);
    r.unsorted = off; off = align_up(off + 16 * (size_t)n_max, 256);
    r.cost = off; off = align_up(off + 4 * (size_t)n_max, 256);
    r.items = off; off = align_up(off + 16 * (size_t)n_max, 256);
    r.seqinfo = off; off = align_up(off + 16 * (size_t)n_max, 256);
    return off;
}

va_status bwd_layout(const va_problem *p, BwdLayout &L)
{
    va_status st = check_problem(p, 0);
    if (st) return st;
    if (p->dtype != VA_BF16 && p->dtype != VA_F16)
        return fail(VA_ERR_UNSUPPORTED, "the backward takes bf16 or fp16 inputs");
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(VA_ERR_UNSUPPORTED, "the backward takes head_dim 64 or 128, not %d", p->head_dim);
    const long long nq = ((long long)p->total_q + (long long)p->batch * (va::kBM - 1)) / va::kBM;
    const long long nk = ((long long)p->total_k + (long long)p->batch * (va::kBwdKeys - 1)) / va::kBwdKeys;
    const long long gq = nq * p->num_heads, gk = nk * p->num_kv_heads;
    if (gq > 0x7fffffffLL || gk > 0x7fffffffLL)
        return fail(VA_ERR_UNSUPPORTED, "problem needs %lld workgroups, above the launch limit", gq > gk ? gq : gk);
    size_t off = plan_region(0, p->batch, (int)nq, L.qp);
    off = plan_region(off, p->batch, (int)nk, L.kp);
    L.qp.grid = gq;
    L.kp.grid = gk;
    L.dvec = off; off = align_up(off + 4 * (size_t)p->total_q * p->num_heads, 256);
    L.total = off;
    return VA_OK;
}

va::PlanArgs bwd_plan(const va_problem *p, const int32_t *cu_q, const int32_t *cu_k, const va::BwdArgs &a,
                      char *ws, const PlanRegion &r, int mode)
{
    va::PlanArgs pa;
    pa.cu_q = cu_q;
    pa.lens_k = cu_k;
    pa.lens_k_is_prefix = 1;
    pa.B = p->batch; pa.Hkv = p->num_kv_heads;
    pa.left = a.left; pa.right = a.right;
    pa.mode = mode;
    pa.bm = mode == va::kPlanBwdKeys ? va::kBwdKeys : va::kBM;
    pa.bn = mode == va::kPlanBwdKeys ? va::kBwdQT : va::kBN;
    pa.n_max = r.n_max;
    pa.count = (int32_t *)(ws + r.count);
    pa.seq_off = (int32_t *)(ws + r.seq);
    pa.unsorted = (int4 *)(ws + r.unsorted);
    pa.cost = (int32_t *)(ws + r.cost);
    pa.items = (int4 *)(ws + r.items);
    pa.seqinfo = (int4 *)(ws + r.seqinfo);
    return pa;
}

// ---------------------------------------------------------------- scratch of the allocation-free entry point
// varlen_attn_fwd_out_noalloc keeps its workspace (work list, decode
// partials) in this array instead of a caller buffer.  Every device the
// library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

va_status scratch_of_current_device(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchDevices)
        return fail(VA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table covers", dev,
                    kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(VA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return VA_OK;
}

}  // namespace

extern "C" {

size_t varlen_attn_bwd_workspace_size(const va_problem *p)
{
    BwdLayout L;
    if (bwd_layout(p, L)) return 0;
    return L.total;
}

size_t varlen_attn_bwd_sinks_workspace_size(const va_problem *p)
{
    if (check_problem(p, 0)) return 0;
    if (p->dtype != VA_BF16 && p->dtype != VA_F16) return 0;
    return align_up((size_t)p->total_q * p->num_heads * 4, 256);
}

va_status varlen_attn_bwd_sinks(const va_problem *p, const void *dout, const void *out, const float *lse,
                                const float *sinks, float *dsinks, void *workspace, size_t workspace_bytes,
                                void *stream)
{
    va_status st = check_problem(p, 0);
    if (st) return st;
    if (p->dtype != VA_BF16 && p->dtype != VA_F16)
        return fail(VA_ERR_UNSUPPORTED, "the sink gradient takes bf16 or fp16 inputs");
    if (!dout || !out || !lse || !sinks || !dsinks)
        return fail(VA_ERR_NULL, "dout, out, lse, sinks and dsinks must be non-NULL");
    const size_t need = varlen_attn_bwd_sinks_workspace_size(p);
    if (!workspace || workspace_bytes < need)
        return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes,
                    need);
    if (!aligned(dout, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return fail(VA_ERR_ALIGN, "dout, out and the workspace must be 16-byte aligned");
    if (!aligned(lse, 4) || !aligned(sinks, 4) || !aligned(dsinks, 4))
        return fail(VA_ERR_ALIGN, "lse, sinks and dsinks must be 4-byte aligned");
    const size_t rows = (size_t)p->total_q * p->num_heads;
    const Range o{dsinks, 4 * (size_t)p->num_heads};
    const Range ins[] = {{dout, rows * p->head_dim * 2}, {out, rows * p->head_dim * 2}, {lse, rows * 4},
                         {sinks, 4 * (size_t)p->num_heads}, {workspace, workspace_bytes}};
    for (const Range &r : ins)
        if (overlaps(o, r)) return fail(VA_ERR_ALIAS, "dsinks must not overlap an input or the workspace");
    const hipError_t e = va::launch_sink_grad16(dout, out, lse, sinks, dsinks, (float *)workspace,
                                                p->dtype == VA_F16, p->head_dim, p->total_q, p->num_heads,
                                                (hipStream_t)stream);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return VA_OK;
}

va_status varlen_attn_bwd(const va_problem *p, const void *dout, const void *q, const void *k,
                          const void *v, const void *out, const float *lse,
                          const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, void *dq,
                          void *dk, void *dv, void *workspace, size_t workspace_bytes, void *stream)
{
    BwdLayout L;
    va_status st = bwd_layout(p, L);
    if (st) return st;
    if (!dout || !q || !k || !v || !out || !lse || !cu_seqlens_q || !cu_seqlens_k || !dq || !dk || !dv)
        return fail(VA_ERR_NULL, "dout, q, k, v, out, lse, cu_seqlens_q/k, dq, dk and dv must be non-NULL");
    if (!workspace || workspace_bytes < L.total)
        return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                    workspace_bytes, L.total);
    const void *al16[] = {dout, q, k, v, out, dq, dk, dv, workspace};
    for (const void *ptr : al16)
        if (!aligned(ptr, 16)) return fail(VA_ERR_ALIGN, "data pointers and the workspace must be 16-byte aligned");
    if (!aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(alibi_of(p), 4))
        return fail(VA_ERR_ALIGN, "lse, cu_seqlens and alibi_slopes must be 4-byte aligned");
    const size_t D = (size_t)p->head_dim;
    const size_t qb = (size_t)p->total_q * p->num_heads * D * 2;
    const size_t kb = (size_t)p->total_k * p->num_kv_heads * D * 2;
    const Range outs[] = {{dq, qb}, {dk, kb}, {dv, kb}};
    const Range ins[] = {{dout, qb}, {q, qb}, {k, kb}, {v, kb}, {out, qb},
                         {lse, (size_t)p->total_q * p->num_heads * 4},
                         {cu_seqlens_q, 4 * ((size_t)p->batch + 1)}, {cu_seqlens_k, 4 * ((size_t)p->batch + 1)},
                         {alibi_of(p), alibi_of(p) ? 4 * (size_t)p->num_heads : 0}, {workspace, workspace_bytes}};
    for (int i = 0; i < 3; ++i) {
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return fail(VA_ERR_ALIAS, "dq, dk and dv must not overlap an input or the workspace");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], outs[j])) return fail(VA_ERR_ALIAS, "dq, dk and dv must not overlap each other");
    }
    va::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.out = out; a.lse = lse;
    char *ws = (char *)workspace;
    a.dvec = (float *)(ws + L.dvec);
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.H = p->num_heads; a.Hkv = p->num_kv_heads; a.g = p->num_heads / p->num_kv_heads;
    a.hpw = a.g % 4 == 0 ? 4 : 1;
    a.left = p->window_left >= 0 ? p->window_left : va::kInfOff;
    if (p->causal) a.right = 0;
    else a.right = p->window_right >= 0 ? p->window_right : va::kInfOff;
    a.scale = p->scale;
    a.scale_log2 = p->scale * va::kLog2e;
    a.alibi = alibi_of(p);
    hipStream_t s = (hipStream_t)stream;
    const va::PlanArgs pq = bwd_plan(p, cu_seqlens_q, cu_seqlens_k, a, ws, L.qp, va::kPlanPrefill);
    const va::PlanArgs pk = bwd_plan(p, cu_seqlens_q, cu_seqlens_k, a, ws, L.kp, va::kPlanBwdKeys);
    hipError_t e = va::launch_plan(pq, s);
    if (e == hipSuccess) e = va::launch_plan(pk, s);
    if (e == hipSuccess)
        e = va::launch_backward16(a, p->dtype == VA_F16, a.alibi != nullptr, p->head_dim, p->total_q, pq.items,
                                  pq.seqinfo, pq.count,
                                  (int)L.qp.grid, pk.items, pk.seqinfo, pk.count, (int)L.kp.grid, s);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return VA_OK;
}


va_status varlen_attn_merge(int32_t n_parts, int32_t rows, int32_t num_heads, int32_t head_dim,
                            va_dtype parts_dtype, va_dtype out_dtype, const void *o_parts,
                            const float *lse_parts, const float *sinks, void *out, float *lse,
                            void *stream)
{
    if (n_parts < 1 || n_parts > 4096) return fail(VA_ERR_SHAPE, "n_parts %d outside [1, 4096]", n_parts);
    if (rows < 1 || num_heads < 1)
        return fail(VA_ERR_SHAPE, "rows %d and num_heads %d must be >= 1", rows, num_heads);
    if (head_dim < 8 || head_dim > 1024 || head_dim % 8 != 0)
        return fail(VA_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 8 in [8, 1024]", head_dim);
    if ((parts_dtype != VA_F32 && parts_dtype != VA_BF16) || (out_dtype != VA_F32 && out_dtype != VA_BF16))
        return fail(VA_ERR_DTYPE, "dtypes must be VA_F32 (0) or VA_BF16 (1)");
    if (!o_parts || !lse_parts || !out) return fail(VA_ERR_NULL, "o_parts, lse_parts and out must be non-NULL");
    if (!aligned(o_parts, 16) || !aligned(out, 16))
        return fail(VA_ERR_ALIGN, "o_parts and out must be 16-byte aligned");
    if (!aligned(lse_parts, 4) || (sinks && !aligned(sinks, 4)) || (lse && !aligned(lse, 4)))
        return fail(VA_ERR_ALIGN, "lse_parts, sinks and lse must be 4-byte aligned");
    const size_t vecs = (size_t)rows * num_heads;
    const size_t pe = parts_dtype == VA_BF16 ? 2 : 4, oe = out_dtype == VA_BF16 ? 2 : 4;
    const Range o_r{out, vecs * head_dim * oe}, l_r{lse, lse ? vecs * 4 : 0};
    const Range ins[] = {{o_parts, (size_t)n_parts * vecs * head_dim * pe},
                         {lse_parts, (size_t)n_parts * vecs * 4},
                         {sinks, sinks ? (size_t)num_heads * 4 : 0}};
    for (const Range &r : ins) {
        if (overlaps(o_r, r)) return fail(VA_ERR_ALIAS, "out overlaps an input");
        if (lse && overlaps(l_r, r)) return fail(VA_ERR_ALIAS, "lse overlaps an input");
    }
    if (lse && overlaps(o_r, l_r)) return fail(VA_ERR_ALIAS, "out overlaps lse");
    va::MergeArgs a;
    a.o_parts = o_parts; a.lse_parts = lse_parts; a.sinks = sinks; a.out = out; a.lse = lse;
    a.n = n_parts; a.rows = rows; a.H = num_heads; a.D = head_dim;
    const hipError_t e = va::launch_merge(a, parts_dtype == VA_BF16, out_dtype == VA_BF16, (hipStream_t)stream);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return VA_OK;
}

va_status varlen_attn_sparse_sharedkv(const va_sparse_problem *p, const void *q, const void *ori_kv,
                                      const int32_t *ori_block_table, const int32_t *seqused_kv,
                                      const void *cmp_kv, const int32_t *cmp_block_table,
                                      const int32_t *cmp_sparse_indices, const int32_t *cu_seqlens_q,
                                      const float *sinks, void *out, float *lse, void *stream)
{
    if (!p) return fail(VA_ERR_NULL, "problem descriptor is NULL");
    // descriptors of ABI 4 end before cmp_attend_all, which then reads as 0
    constexpr size_t kSparseV4Size = offsetof(va_sparse_problem, cmp_attend_all);
    if (p->struct_size < kSparseV4Size)
        return fail(VA_ERR_SHAPE, "va_sparse_problem.struct_size %u is smaller than %zu", p->struct_size,
                    kSparseV4Size);
    const int32_t attend_all = p->struct_size >= sizeof(va_sparse_problem) ? p->cmp_attend_all : 0;
    if (attend_all != 0 && attend_all != 1)
        return fail(VA_ERR_SHAPE, "cmp_attend_all %d is not 0 or 1", attend_all);
    if (attend_all && (p->topk != 0 || cmp_sparse_indices))
        return fail(VA_ERR_SHAPE, "cmp_attend_all takes no cmp_sparse_indices (topk %d)", p->topk);
    if (p->dtype != VA_BF16 && p->dtype != VA_F16)
        return fail(VA_ERR_DTYPE, "dtype %d is not VA_BF16 (1) or VA_F16 (2)", p->dtype);
    if (p->batch < 1 || p->total_q < 1) return fail(VA_ERR_SHAPE, "batch and total_q must be >= 1");
    if (p->num_heads < 1 || p->num_kv_heads < 1 || p->num_heads % p->num_kv_heads != 0)
        return fail(VA_ERR_SHAPE, "num_heads %d must be a positive multiple of num_kv_heads %d", p->num_heads,
                    p->num_kv_heads);
    if (p->num_heads / p->num_kv_heads > 64)
        return fail(VA_ERR_UNSUPPORTED, "more than 64 query heads per kv head");
    if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 512)
        return fail(VA_ERR_UNSUPPORTED, "head_dim %d is not 64, 128 or 512", p->head_dim);
    if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return fail(VA_ERR_UNSUPPORTED, "scale must be finite and > 0");
    if (p->window_left < 0 || p->window_right < 0)
        return fail(VA_ERR_UNSUPPORTED, "window sides (%d, %d) must be >= 0 (2^30 and above: unbounded)",
                    p->window_left, p->window_right);
    if (p->topk < 0) return fail(VA_ERR_SHAPE, "topk %d < 0", p->topk);
    if (p->cmp_ratio < 1) return fail(VA_ERR_SHAPE, "cmp_ratio %d < 1", p->cmp_ratio);
    if (p->max_seqlen_kv < 0 || p->max_seqlen_kv > va::kMaxSeqlen)
        return fail(VA_ERR_SHAPE, "max_seqlen_kv %d outside [0, %d]", p->max_seqlen_kv, va::kMaxSeqlen);
    if (p->ori_num_blocks < 1 || p->ori_block_size < 1 || p->cmp_num_blocks < 1 || p->cmp_block_size < 1)
        return fail(VA_ERR_SHAPE, "block counts and sizes must be >= 1");
    const long long ori_need = ((long long)p->max_seqlen_kv + p->ori_block_size - 1) / p->ori_block_size;
    const long long cmp_need = ((long long)(p->max_seqlen_kv / p->cmp_ratio) + p->cmp_block_size - 1) / p->cmp_block_size;
    if (p->ori_block_table_stride < ori_need || p->cmp_block_table_stride < cmp_need)
        return fail(VA_ERR_SHAPE, "block table strides (%d, %d) below (%lld, %lld) blocks", p->ori_block_table_stride,
                    p->cmp_block_table_stride, ori_need, cmp_need);
    if (!q || !ori_kv || !ori_block_table || !seqused_kv || !cmp_kv || !cmp_block_table || !cu_seqlens_q || !out ||
        (p->topk > 0 && !cmp_sparse_indices))
        return fail(VA_ERR_NULL, "a required pointer is NULL");
    const void *al16[] = {q, ori_kv, cmp_kv, out};
    for (const void *ptr : al16)
        if (!aligned(ptr, 16)) return fail(VA_ERR_ALIGN, "q, ori_kv, cmp_kv and out must be 16-byte aligned");
    const void *al4[] = {ori_block_table, seqused_kv, cmp_block_table, cmp_sparse_indices, cu_seqlens_q, sinks, lse};
    for (const void *ptr : al4)
        if (ptr && !aligned(ptr, 4)) return fail(VA_ERR_ALIGN, "int32 / float32 arrays must be 4-byte aligned");
    const size_t D = (size_t)p->head_dim, H = (size_t)p->num_heads, Hkv = (size_t)p->num_kv_heads;
    const size_t T = (size_t)p->total_q;
    const Range o_r{out, T * H * D * 2}, l_r{lse, lse ? T * H * 4 : 0};
    const Range ins[] = {
        {q, T * H * D * 2},
        {ori_kv, (size_t)p->ori_num_blocks * p->ori_block_size * Hkv * D * 2},
        {cmp_kv, (size_t)p->cmp_num_blocks * p->cmp_block_size * Hkv * D * 2},
        {ori_block_table, 4 * (size_t)p->batch * p->ori_block_table_stride},
        {cmp_block_table, 4 * (size_t)p->batch * p->cmp_block_table_stride},
        {seqused_kv, 4 * (size_t)p->batch},
        {cmp_sparse_indices, cmp_sparse_indices ? 4 * T * Hkv * p->topk : 0},
        {cu_seqlens_q, 4 * ((size_t)p->batch + 1)},
        {sinks, sinks ? 4 * H : 0},
    };
    for (const Range &r : ins) {
        if (overlaps(o_r, r)) return fail(VA_ERR_ALIAS, "out overlaps an input");
        if (overlaps(l_r, r)) return fail(VA_ERR_ALIAS, "lse overlaps an input");
    }
    if (overlaps(o_r, l_r)) return fail(VA_ERR_ALIAS, "out overlaps lse");
    va::SparseArgs a;
    a.q = q; a.ori_kv = ori_kv; a.ori_table = ori_block_table; a.seqused_kv = seqused_kv;
    a.cmp_kv = cmp_kv; a.cmp_table = cmp_block_table; a.indices = cmp_sparse_indices; a.cu_q = cu_seqlens_q;
    a.sinks = sinks; a.out = out; a.lse = lse;
    a.B = p->batch; a.T = p->total_q; a.H = p->num_heads; a.Hkv = p->num_kv_heads;
    a.g = p->num_heads / p->num_kv_heads; a.topk = p->topk; a.cmp_all = attend_all;
    a.ori_bs = p->ori_block_size; a.ori_stride = p->ori_block_table_stride;
    a.cmp_bs = p->cmp_block_size; a.cmp_stride = p->cmp_block_table_stride; a.cmp_ratio = p->cmp_ratio;
    a.ori_shift = a.cmp_shift = -1;
    for (int sh = 0; sh < 31; ++sh) {
        if ((1 << sh) == a.ori_bs) a.ori_shift = sh;
        if ((1 << sh) == a.cmp_bs) a.cmp_shift = sh;
    }
    a.left = std::min(p->window_left, va::kInfOff); a.right = std::min(p->window_right, va::kInfOff);
    a.scale_log2 = p->scale * va::kLog2e;
    // tokens per workgroup: the fewest that keep the grid within whole rounds
    // of 1024 workgroups (4 per CU of 2 waves each), 1 to kSpTokMax each
    const long long units = (long long)p->total_q * p->num_kv_heads;
    a.tok_per_wg = (int)std::min<long long>(va::kSpTokMax, std::max<long long>(1, (units + 1023) / 1024));
    const hipError_t e = va::launch_sparse16(a, p->dtype == VA_F16, p->head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return VA_OK;
}

int varlen_attn_abi_version(void) { return VARLEN_ATTN_ABI_VERSION; }

const char *varlen_attn_last_error(void) { return g_last_error.c_str(); }

size_t varlen_attn_workspace_size(const va_problem *p, int paged)
{
    if (check_problem(p, paged != 0)) return 0;
    Layout L;
    if (make_layout(p, paged != 0, L)) return 0;
    return L.total;
}

int varlen_attn_path(const va_problem *p, int paged)
{
    if (check_problem(p, paged != 0)) return -1;
    Layout L;
    if (make_layout(p, paged != 0, L)) return -1;
    return L.path;
}

va_status varlen_attn_fwd_out(const va_problem *p, const void *q, const void *k, const void *v,
                              const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                              const float *sinks, void *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    Call c{p, 0, q, k, v, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, sinks, out, lse, workspace,
           workspace_bytes};
    return run(c, (hipStream_t)stream);
}

va_status varlen_attn_fwd_out_noalloc(const va_problem *p, const void *q, const void *k, const void *v,
                                      const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                      const float *sinks, void *out, float *lse, void *stream)
{
    va_status st = check_problem(p, 0);
    if (st) return st;
    Layout L;
    if ((st = make_layout(p, 0, L))) return st;
    if (L.total > kScratchBytes)
        return fail(VA_ERR_WORKSPACE,
                    "the call needs %zu bytes of workspace, above the %zu-byte scratch of "
                    "varlen_attn_fwd_out_noalloc (varlen_attn_fwd_out takes a caller workspace)",
                    L.total, kScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    Call c{p, 0, q, k, v, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, sinks, out, lse, ws, kScratchBytes};
    return run(c, (hipStream_t)stream);
}

va_status varlen_attn_fwd_paged(const va_problem *p, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_table,
                                const int32_t *cu_seqlens_q, const int32_t *seqused_k,
                                const float *sinks, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    Call c{p, 1, q, k_cache, v_cache, cu_seqlens_q, nullptr, seqused_k, block_table, sinks, out, lse,
           workspace, workspace_bytes};
    return run(c, (hipStream_t)stream);
}

va_status varlen_attn_fwd(const va_problem *p, const void *q, const void *k, const void *v,
                          const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, const float *sinks,
                          void **out, float **lse, void *stream)
{
    if (!out) return fail(VA_ERR_NULL, "out (the address receiving the allocation) is NULL");
    *out = nullptr;
    if (lse) *lse = nullptr;
    va_status st = check_problem(p, 0);
    if (st) return st;
    Layout L;
    if ((st = make_layout(p, 0, L))) return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t es = p->dtype == VA_F32 ? 4 : 2;
    const size_t out_bytes = (size_t)p->total_q * p->num_heads * p->head_dim * es;
    const size_t lse_bytes = (size_t)p->total_q * p->num_heads * 4;
    void *o = nullptr, *l = nullptr, *w = nullptr;
    if (hipMallocAsync(&o, out_bytes, s) != hipSuccess ||
        (lse && hipMallocAsync(&l, lse_bytes, s) != hipSuccess) ||
        hipMallocAsync(&w, L.total, s) != hipSuccess) {
        if (o) (void)hipFreeAsync(o, s);
        if (l) (void)hipFreeAsync(l, s);
        if (w) (void)hipFreeAsync(w, s);
        return fail(VA_ERR_HIP, "stream-ordered allocation failed");
    }
    Call c{p, 0, q, k, v, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr, sinks, o, (float *)l, w, L.total};
    st = run(c, s);
    (void)hipFreeAsync(w, s);
    if (st) {
        (void)hipFreeAsync(o, s);
        if (l) (void)hipFreeAsync(l, s);
        return st;
    }
    *out = o;
    if (lse) *lse = (float *)l;
    return VA_OK;
}

va_status varlen_attn_free(void *ptr, void *stream)
{
    if (!ptr) return VA_OK;
    hipError_t e = hipFreeAsync(ptr, (hipStream_t)stream);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "hipFreeAsync failed: %s", hipGetErrorString(e));
    return VA_OK;
}

va_status varlen_attn_plan(const va_problem *p, int paged, const int32_t *cu_seqlens_q,
                           const int32_t *seqlens_k, int32_t *items, int32_t capacity, int32_t *count,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    va_status st = check_problem(p, paged != 0);
    if (st) return st;
    Layout L;
    if ((st = make_layout(p, paged != 0, L))) return st;
    if (!cu_seqlens_q || !seqlens_k)
        return fail(VA_ERR_NULL, "cu_seqlens_q and seqlens_k must be non-NULL");
    if ((capacity > 0 && !items) || (capacity > 0 && !count))
        return fail(VA_ERR_NULL, "items and count must be non-NULL when capacity > 0");
    if (!workspace || workspace_bytes < L.total)
        return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                    workspace_bytes, L.total);
    if (capacity < 0) return fail(VA_ERR_SHAPE, "capacity %d < 0", capacity);
    Call c{p, paged != 0, nullptr, nullptr, nullptr, cu_seqlens_q, paged ? nullptr : seqlens_k,
           paged ? seqlens_k : nullptr, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes};
    const va::AttnArgs a = make_args(c);
    const va::PlanArgs pa = make_plan(c, L, a);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = va::launch_plan(pa, s);
    const size_t n = (size_t)(capacity < L.n_max ? capacity : L.n_max);
    if (e == hipSuccess && n) e = hipMemcpyAsync(items, pa.items, n * 16, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && count) e = hipMemcpyAsync(count, pa.count, 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(VA_ERR_HIP, "plan failed: %s", hipGetErrorString(e));
    return VA_OK;
}

}  // extern "C"
