// Internal declarations shared by the HIP sources of the varlen attention
// library (kernels, work-partition pre-pass, host launcher).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace va {

// ---------------------------------------------------------------- constants
constexpr int kInfOff = 1 << 30;       // "unbounded" window offset
constexpr int kMaxSeqlen = 1 << 29;    // keeps i + delta +- offsets inside int32
constexpr int kBM = 128;               // bf16 prefill: query rows per workgroup
constexpr int kBN = 64;                // bf16 prefill: key rows per tile
constexpr int kBMf32 = 64;             // float32 path: query rows per workgroup
constexpr int kBNf32 = 32;             // float32 path: key rows per tile
constexpr int kDecRows = 16;           // decode: packed (head, query) rows per kv head
constexpr int kDecChunk = 64;          // decode: keys per wave step
constexpr int kDecQuantum = 256;       // decode: split sizes are multiples of this
constexpr int kDecTargetUnits = 4096;  // decode: aim for about this many (split, kv head) units
constexpr int kDecTableMax = 2048;     // decode: block ids of one split staged in LDS
constexpr int kPlanThreads = 512;
constexpr int kCostBins = 4096;        // cost classes of the pre-pass ordering
constexpr int kSortMax = 2048;         // pre-pass sorts up to this many items in LDS
constexpr int kRankSortMax = 1024;     // ... by ranking (no barriers) up to this many
constexpr int kPlanSeqs = 2048;        // pre-pass keeps up to this many sequences' lengths in LDS
constexpr int kBwdKeys = 128;          // backward: key rows per dK/dV workgroup
constexpr int kBwdQT = 64;             // backward: query rows per dK/dV tile

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- kernel arguments
struct AttnArgs {
    const void *q, *k, *v;
    void *out;
    float *lse;                  // may be null
    const int32_t *cu_q;         // [B+1]
    const int32_t *cu_k;         // [B+1] contiguous mode
    const int32_t *seqused_k;    // [B]   paged mode
    const int32_t *block_table;  // [B, bt_stride] paged mode
    const float *sinks;          // [H] or null
    const float *alibi;          // [H] slopes or null
    int32_t B, H, Hkv, g;
    int32_t bt_stride, block_size;
    int32_t bs_shift;            // log2(block_size) when a power of two, else -1
    int32_t left, right;         // visible keys of query position p: [p-left, p+right]
    float scale, scale_log2;     // scale and scale * log2(e)
    int32_t item_rows;           // sliding-window kernel: query rows per work item
    int32_t hpw;                 // prefill: query heads per workgroup (1, or 4 of one kv head)
};

// Sliding-window kernel for 32..64 query heads per kv head: LDS rows of the
// window (K and V each, 76 KB in all, two workgroups per CU); a work item of
// R query rows needs left + right + R <= win_cap(D).
constexpr int win_cap(int D) { return D == 128 ? 152 : 304; }

// Prefill: items are (sequence, block of bm query rows) with their key range.
// Decode: (sequence, split of the visible keys).  Backward key blocks:
// (sequence, block of bm key rows) with the range of query rows that see
// any of those keys.
// Window: the prefill's items of bm query rows, in index order (the
// sliding-window kernel's items cost about the same, no sort needed).
enum PlanMode : int32_t { kPlanPrefill = 0, kPlanDecode = 1, kPlanBwdKeys = 2, kPlanWindow = 3 };

// How the prefill kernel fetches K/V rows: buffer loads over one
// sequence's rows (contiguous, every sequence span below 2 GiB), plain
// global loads (contiguous, larger spans), or block-table gathers.
enum LoadMode : int32_t { kLoadBuffer = 0, kLoadGlobal = 1, kLoadPaged = 2 };

struct PlanArgs {
    const int32_t *cu_q;
    const int32_t *lens_k;       // cu_k (prefix sums) or seqused_k (counts)
    int32_t lens_k_is_prefix;    // 1: cu_k, 0: seqused_k
    int32_t B, Hkv;
    int32_t left, right;
    int32_t mode;                // PlanMode
    int32_t bm;                  // prefill: query rows per item; backward: key rows per item
    int32_t bn;                  // prefill: key rows per tile; backward: query rows per tile (cost unit)
    int32_t n_max;               // capacity of the item arrays
    int32_t *count;              // [1] number of items written
    int32_t *seq_off;            // [B+1] first item (prefill) / first split slot (decode)
    int4 *unsorted;              // [n_max]
    int32_t *cost;               // [n_max]
    int4 *items;                 // [n_max] sorted, execution order
    int4 *seqinfo;               // [n_max] per item: (first query row, query rows,
                                 //  first key row (contiguous; 0 paged), key rows)
};

// Backward (bf16, contiguous K/V).
struct BwdArgs {
    const void *q, *k, *v, *dout, *out;
    const float *lse;            // [T_q, H] from the forward
    float *dvec;                 // [T_q, H] workspace: sum_d dout * out
    void *dq, *dk, *dv;
    int32_t H, Hkv, g;
    int32_t left, right;         // as in AttnArgs
    float scale, scale_log2;
    const float *alibi;          // [H] slopes or null, as in AttnArgs
    int32_t hpw;                 // dQ kernel: query heads per workgroup (1, or 4 of one kv head)
};

// Sliding-window + sparse compressed attention over shared K/V (the
// third scenario of the SparseAttnSharedkv README).
constexpr int kSpTokMax = 16;    // tokens per workgroup, at most
constexpr int kSpListMax = 1536; // keys of one chunk of a token's list (a multiple of 128 and of the 64-key tile)
struct SparseArgs {
    const void *q;                   // [T_q, H, D]
    const void *ori_kv;              // [ori_blocks, ori_bs, Hkv, D], K = V
    const int32_t *ori_table;        // [B, ori_stride]
    const int32_t *seqused_kv;       // [B] original keys per sequence
    const void *cmp_kv;              // [cmp_blocks, cmp_bs, Hkv, D], K = V
    const int32_t *cmp_table;        // [B, cmp_stride]
    const int32_t *indices;          // [T_q, Hkv, topk] compressed positions
    const int32_t *cu_q;             // [B + 1]
    const float *sinks;              // [H] or null
    void *out;                       // [T_q, H, D]
    float *lse;                      // [T_q, H] or null
    int32_t B, T, H, Hkv, g, topk;
    int32_t cmp_all;                 // 1: every visible compressed key, no indices
    int32_t tok_per_wg;              // consecutive tokens per workgroup
    int32_t ori_bs, ori_stride, cmp_bs, cmp_stride, cmp_ratio;
    int32_t ori_shift, cmp_shift;    // log2 of ori_bs / cmp_bs when a power of two, else -1
    int32_t left, right;             // window on the original keys (kInfOff = unbounded)
    float scale_log2;
};

// Merge of partial results over disjoint key sets.
struct MergeArgs {
    const void *o_parts;         // [n, rows, H, D]
    const float *lse_parts;      // [n, rows, H]
    const float *sinks;          // [H] or null
    void *out;                   // [rows, H, D]
    float *lse;                  // [rows, H] or null
    int32_t n, rows, H, D;
};

// Opt-in device-side argument check (one bit per violated precondition).
enum CheckFlag : uint32_t {
    kChkCuQStart = 1u << 0,   // cu_seqlens_q[0] != 0
    kChkCuQOrder = 1u << 1,   // cu_seqlens_q decreases
    kChkCuQTotal = 1u << 2,   // cu_seqlens_q[B] != total_q
    kChkLenQ = 1u << 3,       // a query length exceeds max_seqlen_q
    kChkCuKStart = 1u << 4,   // cu_seqlens_k[0] != 0
    kChkCuKOrder = 1u << 5,   // cu_seqlens_k decreases
    kChkCuKTotal = 1u << 6,   // cu_seqlens_k[B] != total_k
    kChkLenK = 1u << 7,       // a key length exceeds max_seqlen_k
    kChkSeqused = 1u << 8,    // seqused_k < 0 or beyond its block-table row
    kChkBlockId = 1u << 9,    // a used block id outside [0, num_blocks)
};

struct CheckArgs {
    const int32_t *cu_q, *cu_k;        // cu_k null in paged mode
    const int32_t *seqused_k;          // null in contiguous mode
    const int32_t *block_table;
    int32_t B, total_q, total_k, max_q, max_k;
    int32_t bt_stride, block_size, num_blocks;
    uint32_t *flags;                   // [1] result
};

// ---------------------------------------------------------------- launchers
hipError_t launch_check(const CheckArgs &c, hipStream_t s);
hipError_t launch_backward16(const BwdArgs &a, bool f16, bool alibi, int head_dim, int total_q, const int4 *q_items,
                             const int4 *q_seqinfo, const int32_t *q_count, int q_grid, const int4 *k_items,
                             const int4 *k_seqinfo, const int32_t *k_count, int k_grid, hipStream_t s);
hipError_t launch_sink_grad16(const void *dout, const void *out, const float *lse, const float *sinks, float *dsinks,
                              float *terms, bool f16, int head_dim, int total_q, int H, hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, bool part_bf16, bool out_bf16, hipStream_t s);
hipError_t launch_sparse16(const SparseArgs &a, bool f16, int head_dim, hipStream_t s);
hipError_t launch_window16(const AttnArgs &a, bool f16, int head_dim, bool paged, const int4 *items,
                           const int4 *seqinfo, const int32_t *count, int grid, hipStream_t s);
hipError_t launch_plan(const PlanArgs &pa, hipStream_t s);
hipError_t launch_prefill16(const AttnArgs &a, bool f16, bool alibi, int head_dim, int mode, const int4 *items,
                            const int4 *seqinfo, const int32_t *count, int grid, hipStream_t s);
hipError_t launch_prefill512(const AttnArgs &a, bool f16, bool paged, const int4 *items, const int4 *seqinfo,
                             const int32_t *count, int grid, hipStream_t s);
hipError_t launch_prefill_f32(const AttnArgs &a, int head_dim, bool paged, const int4 *items,
                              const int4 *seqinfo, const int32_t *count, int grid, hipStream_t s);
hipError_t launch_decode16(const AttnArgs &a, bool f16, int head_dim, bool paged, const int4 *items,
                           const int4 *seqinfo, const int32_t *count, int grid, float *part_o,
                           float2 *part_ml, hipStream_t s);
hipError_t launch_decode_combine(const AttnArgs &a, bool f16, int head_dim, const int32_t *seq_off,
                                 const float *part_o, const float2 *part_ml, hipStream_t s);

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
// Visible keys [lo, hi] (inclusive, clipped to [0, Lk-1]) of query row i.
__device__ __forceinline__ void row_bounds(int i, int delta, int Lk, int left, int right,
                                           int &lo, int &hi)
{
    const int p = i + delta;
    lo = left >= kInfOff ? 0 : max(0, p - left);
    hi = right >= kInfOff ? Lk - 1 : min(Lk - 1, p + right);
}

// Element offset of key/value row j (logical position in its sequence) of
// kv head c: contiguous rows start at k0; paged rows go through the block
// table (block j / block_size, slot j % block_size).
template <int D, bool PAGED>
__device__ __forceinline__ size_t kv_row_offset(const AttnArgs &a, int b, int k0, int c, int j)
{
    size_t row;
    if (PAGED) {
        const int blk_i = a.bs_shift >= 0 ? (j >> a.bs_shift) : j / a.block_size;
        const int slot = a.bs_shift >= 0 ? (j & (a.block_size - 1)) : j % a.block_size;
        const int blk = a.block_table[(size_t)b * a.bt_stride + blk_i];
        row = (size_t)blk * a.block_size + slot;
    } else {
        row = (size_t)(k0 + j);
    }
    return (row * a.Hkv + c) * D;
}

// Workgroup -> (work item, head) with heads grouped per XCD: consecutive
// workgroup ids are dealt round-robin to the 8 XCDs, so giving each XCD a
// contiguous range of heads keeps one GQA group's K/V in one L2.
__device__ __forceinline__ void map_block(int bid, int nheads, int &item, int &head)
{
    if ((nheads & 7) == 0) {
        const int hpx = nheads >> 3;
        const int x = bid & 7, r = bid >> 3;
        item = r / hpx;
        head = x * hpx + r % hpx;
    } else {
        item = bid / nheads;
        head = bid % nheads;
    }
}

// Bijection of [0, n) that gives each XCD a contiguous range: workgroup id
// bid runs on XCD bid % 8, and XCD x takes ids x, x + 8, ... in turn, so
// ranges of about n / 8 consecutive items each share one L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int n)
{
    const int q = n >> 3, r = n & 7, x = bid & 7, j = bid >> 3;
    return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}
#endif

}  // namespace va
