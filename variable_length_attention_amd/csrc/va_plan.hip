// Work-partition pre-pass (one workgroup).
//
// Turns the device-resident cu_seqlens into the list of tiles the attention
// kernels process, so no host round-trip is needed.  It plays the role of
// the core-partition metadata that precedes SparseAttnSharedkv on Ascend
// (SparseAttnSharedkv README, parameter table row "metadata"), computed here
// on the GPU right before the attention kernels on the same stream.
//
// Prefill mode: one item per (sequence, block of bm query rows); the item
//   carries the union of the visible key ranges of its rows, and its cost is
//   the number of bn-row key tiles in that range.
// Decode mode:  one item per (sequence, split) where the visible key range of
//   the whole sequence is cut into splits of a common size chosen from the
//   total visible key count; the item carries its split slot.
// Items are ordered by descending cost (longest first), ties by ascending
// item index, so the result is deterministic.
#include "va_internal.h"

namespace va {

namespace {

__device__ __forceinline__ int q_len(const PlanArgs &a, int b)
{
    return a.cu_q[b + 1] - a.cu_q[b];
}

__device__ __forceinline__ int k_len(const PlanArgs &a, int b)
{
    return a.lens_k_is_prefix ? a.lens_k[b + 1] - a.lens_k[b] : a.lens_k[b];
}

// Visible key range [lo, hi) of query rows [i0, i1), i1 > i0.  Both bounds of
// a row are non-decreasing in the row index, so the first row gives the low
// end and the last row the high end (a superset when some rows are empty).
__device__ __forceinline__ void rows_range(int i0, int i1, int delta, int Lk, int left,
                                           int right, int &lo, int &hi)
{
    int l0, h0, l1, h1;
    row_bounds(i0, delta, Lk, left, right, l0, h0);
    row_bounds(i1 - 1, delta, Lk, left, right, l1, h1);
    lo = l0;
    hi = max(h1 + 1, lo);
}

// Exclusive scan of one value per thread over the workgroup; returns the
// prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int *s_tmp, int *total)
{
    const int tid = threadIdx.x;
    s_tmp[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        int x = tid >= off ? s_tmp[tid - off] : 0;
        __syncthreads();
        s_tmp[tid] += x;
        __syncthreads();
    }
    const int incl = s_tmp[tid];
    *total = s_tmp[kPlanThreads - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void k0_plan(PlanArgs a)
{
    __shared__ int s_bins[kCostBins];
    __shared__ uint32_t s_keys[kSortMax];   // (inverted cost, index) sort keys
    __shared__ int s_off[kSortMax + 1];     // per-sequence item offsets when B <= kSortMax
    __shared__ int s_tmp[kPlanThreads];
    __shared__ long long s_red[kPlanThreads];
    const int tid = threadIdx.x;
    const bool off_in_lds = a.B <= kSortMax;

    // 1. decode: split size from the total visible key count
    int split = 1;
    if (a.mode == kPlanDecode) {
        long long vis = 0;
        for (int b = tid; b < a.B; b += kPlanThreads) {
            const int Lq = q_len(a, b), Lk = k_len(a, b);
            if (Lq > 0 && Lk > 0) {
                int lo, hi;
                rows_range(0, Lq, Lk - Lq, Lk, a.left, a.right, lo, hi);
                vis += hi - lo;
            }
        }
        s_red[tid] = vis;
        __syncthreads();
        for (int off = kPlanThreads / 2; off > 0; off >>= 1) {
            if (tid < off) s_red[tid] += s_red[tid + off];
            __syncthreads();
        }
        const long long want = (s_red[0] * a.Hkv + kDecTargetUnits - 1) / kDecTargetUnits;
        long long sz = (want + kDecQuantum - 1) / kDecQuantum * kDecQuantum;
        if (sz < kDecQuantum) sz = kDecQuantum;
        if (sz > kMaxSeqlen) sz = kMaxSeqlen;
        split = (int)sz;
    }

    // 2. items per sequence and their prefix sums
    int carry = 0;
    for (int base = 0; base < a.B; base += kPlanThreads) {
        const int b = base + tid;
        int n = 0;
        if (b < a.B) {
            const int Lq = q_len(a, b);
            if (a.mode == kPlanPrefill) {
                n = (Lq + a.bm - 1) / a.bm;
            } else {
                const int Lk = k_len(a, b);
                int vis = 0;
                if (Lq > 0 && Lk > 0) {
                    int lo, hi;
                    rows_range(0, Lq, Lk - Lq, Lk, a.left, a.right, lo, hi);
                    vis = hi - lo;
                }
                n = max(1, (vis + split - 1) / split);
            }
        }
        int chunk_total;
        const int ex = block_exclusive_scan(n, s_tmp, &chunk_total);
        if (b < a.B) {
            a.seq_off[b] = carry + ex;
            if (off_in_lds) s_off[b] = carry + ex;
        }
        carry += chunk_total;
    }
    if (tid == 0) {
        a.seq_off[a.B] = carry;
        if (off_in_lds) s_off[a.B] = carry;
    }
    const int N = min(carry, a.n_max);
    const bool use_sort = N <= kSortMax;
    for (int i = tid; i < kCostBins; i += kPlanThreads) s_bins[i] = 0;
    __syncthreads();
    const int *offs = off_in_lds ? s_off : a.seq_off;

    // 3. unsorted items, costs and (for the large-N path) the cost histogram
    for (int idx = tid; idx < N; idx += kPlanThreads) {
        int lo_b = 0, hi_b = a.B - 1;  // last b with offs[b] <= idx
        while (lo_b < hi_b) {
            const int mid = (lo_b + hi_b + 1) >> 1;
            if (offs[mid] <= idx) lo_b = mid; else hi_b = mid - 1;
        }
        const int b = lo_b;
        const int s = idx - offs[b];
        const int Lq = q_len(a, b), Lk = k_len(a, b);
        int4 it;
        int cost;
        if (a.mode == kPlanPrefill) {
            const int i0 = s * a.bm, i1 = min(Lq, i0 + a.bm);
            int lo = 0, hi = 0;
            if (Lk > 0) rows_range(i0, i1, Lk - Lq, Lk, a.left, a.right, lo, hi);
            it = make_int4(b, i0, lo, hi);
            cost = (hi - lo + a.bn - 1) / a.bn;
        } else {
            int lo = 0, hi = 0;
            if (Lq > 0 && Lk > 0) rows_range(0, Lq, Lk - Lq, Lk, a.left, a.right, lo, hi);
            const int k_lo = min(hi, lo + s * split);
            const int k_hi = min(hi, k_lo + split);
            it = make_int4(b, idx, k_lo, k_hi);
            cost = (k_hi - k_lo + kDecQuantum - 1) / kDecQuantum;
        }
        const int cbin = min(cost, kCostBins - 1);
        a.unsorted[idx] = it;
        if (use_sort) {
            s_keys[idx] = ((uint32_t)(kCostBins - 1 - cbin) << 19) | (uint32_t)idx;
        } else {
            a.cost[idx] = cost;
            atomicAdd(&s_bins[cbin], 1);
        }
    }
    __syncthreads();

    if (use_sort) {
        // 4a. bitonic sort of the keys: ascending key = descending cost,
        // then ascending item index
        int P = 1;
        while (P < N) P <<= 1;
        for (int i = N + tid; i < P; i += kPlanThreads) s_keys[i] = 0xffffffffu;
        __syncthreads();
        for (int k = 2; k <= P; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int t = tid; t < P / 2; t += kPlanThreads) {
                    const int i = 2 * t - (t & (j - 1));  // lower element of the pair
                    const int l = i + j;
                    const uint32_t x = s_keys[i], y = s_keys[l];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) {
                        s_keys[i] = y;
                        s_keys[l] = x;
                    }
                }
                __syncthreads();
            }
        }
        for (int i = tid; i < N; i += kPlanThreads)
            a.items[i] = a.unsorted[s_keys[i] & ((1u << 19) - 1u)];
    } else {
        // 4b. bucket start positions, highest cost first
        constexpr int per = kCostBins / kPlanThreads;
        int local = 0;
        for (int k = 0; k < per; ++k) local += s_bins[kCostBins - 1 - (tid * per + k)];
        int total;
        int run = block_exclusive_scan(local, s_tmp, &total);
        for (int k = 0; k < per; ++k) {
            const int bin = kCostBins - 1 - (tid * per + k);
            const int c = s_bins[bin];
            s_bins[bin] = run;
            run += c;
        }
        __syncthreads();
        // 5. stable placement by one wave, 64 items at a time in index order
        if (tid < 64) {
            const int lane = tid;
            for (int base = 0; base < N; base += 64) {
                const int idx = base + lane;
                const bool active = idx < N;
                const int c = active ? min(a.cost[idx], kCostBins - 1) : -1;
                unsigned long long remaining = __ballot(active);
                while (remaining) {
                    const int leader = __ffsll((long long)remaining) - 1;
                    const int lc = __shfl(c, leader);
                    const unsigned long long peers = __ballot(active && c == lc);
                    int start = lane == leader ? s_bins[lc] : 0;
                    start = __shfl(start, leader);
                    if (active && c == lc) {
                        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
                        a.items[start + rank] = a.unsorted[idx];
                    }
                    if (lane == leader) s_bins[lc] = start + __popcll(peers);
                    remaining &= ~peers;
                }
            }
        }
    }
    if (tid == 0) *a.count = N;
}

}  // namespace

hipError_t launch_plan(const PlanArgs &pa, hipStream_t s)
{
    hipLaunchKernelGGL(k0_plan, dim3(1), dim3(kPlanThreads), 0, s, pa);
    return hipGetLastError();
}

}  // namespace va
