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
// Order (deterministic): prefill items sequence by sequence, the sequence
// with the most bn-key tiles first (ties: the later sequence first), and
// within a sequence its last query block first (under a causal mask its
// costliest): the workgroups running at one time then share one sequence's
// K/V in L2, and the list still ends with short work.  Decode and backward
// items by descending cost (longest first), ties by ascending item index.
#include "va_internal.h"

namespace va {

namespace {

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

constexpr int kWaves = kPlanThreads / 64;

// Exclusive scan of one value per thread over the workgroup (wave scans
// with cross-lane shuffles, then one pass over the wave totals); returns
// the prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int *s_w, int *total)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_w[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = s_w[i];
        before += i < w ? t : 0;
        tot += t;
    }
    *total = tot;
    __syncthreads();
    return before + x - v;
}

__global__ __launch_bounds__(kPlanThreads) void k0_plan(PlanArgs a)
{
    __shared__ int s_lq[kPlanSeqs], s_lk[kPlanSeqs];  // per-sequence lengths (B <= kPlanSeqs)
    __shared__ int s_q0[kPlanSeqs], s_k0[kPlanSeqs];  // per-sequence first query / key row
    __shared__ int s_off[kPlanSeqs + 1];              // first item of each sequence
    __shared__ uint32_t s_keys[kSortMax];             // (inverted cost, index) sort keys
    __shared__ int s_bins[kCostBins];                 // counting placement (large lists)
    __shared__ int s_w[kWaves];
    __shared__ long long s_w64[kWaves];
    const int tid = threadIdx.x;
    const bool seq_lds = a.B <= kPlanSeqs;

    // 0. per-sequence lengths into LDS once
    if (seq_lds)
        for (int b = tid; b < a.B; b += kPlanThreads) {
            const int q0 = a.cu_q[b], k0 = a.lens_k_is_prefix ? a.lens_k[b] : 0;
            s_q0[b] = q0;
            s_k0[b] = k0;
            s_lq[b] = a.cu_q[b + 1] - q0;
            s_lk[b] = a.lens_k_is_prefix ? a.lens_k[b + 1] - k0 : a.lens_k[b];
        }
    __syncthreads();
    auto q_len = [&](int b) { return seq_lds ? s_lq[b] : a.cu_q[b + 1] - a.cu_q[b]; };
    auto k_len = [&](int b) {
        return seq_lds ? s_lk[b] : (a.lens_k_is_prefix ? a.lens_k[b + 1] - a.lens_k[b] : a.lens_k[b]);
    };
    // (first query row, query rows, first key row, key rows) of sequence b
    auto seq_info = [&](int b) {
        if (seq_lds) return make_int4(s_q0[b], s_lq[b], s_k0[b], s_lk[b]);
        return make_int4(a.cu_q[b], q_len(b), a.lens_k_is_prefix ? a.lens_k[b] : 0, k_len(b));
    };
    auto vis_range = [&](int b, int &lo, int &hi) {  // keys any query row of b sees
        const int Lq = q_len(b), Lk = k_len(b);
        lo = hi = 0;
        if (Lq > 0 && Lk > 0) rows_range(0, Lq, Lk - Lq, Lk, a.left, a.right, lo, hi);
    };

    // 1. decode: split size from the total visible key count
    int split = 1;
    if (a.mode == kPlanDecode) {
        long long vis = 0;
        for (int b = tid; b < a.B; b += kPlanThreads) {
            int lo, hi;
            vis_range(b, lo, hi);
            vis += hi - lo;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) vis += __shfl_xor(vis, off);
        if ((tid & 63) == 0) s_w64[tid >> 6] = vis;
        __syncthreads();
        long long tot = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) tot += s_w64[i];
        const long long want = (tot * a.Hkv + kDecTargetUnits - 1) / kDecTargetUnits;
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
            if (a.mode == kPlanPrefill || a.mode == kPlanWindow) {
                n = (q_len(b) + a.bm - 1) / a.bm;
            } else if (a.mode == kPlanBwdKeys) {
                n = (k_len(b) + a.bm - 1) / a.bm;  // every key block, even with no query rows
            } else {
                int lo, hi;
                vis_range(b, lo, hi);
                n = max(1, (hi - lo + split - 1) / split);
            }
        }
        int chunk_total;
        const int ex = block_exclusive_scan(n, s_w, &chunk_total);
        if (b < a.B) {
            a.seq_off[b] = carry + ex;
            if (seq_lds) s_off[b] = carry + ex;
        }
        carry += chunk_total;
    }
    if (tid == 0) {
        a.seq_off[a.B] = carry;
        if (seq_lds) s_off[a.B] = carry;
    }
    const int N = min(carry, a.n_max);
    __syncthreads();
    const int *offs = seq_lds ? s_off : a.seq_off;

    // item idx: (sequence, first query row | split slot, key range) and cost
    auto make_item = [&](int idx, int &cost) -> int4 {
        int lo_b = 0, hi_b = a.B - 1;  // last b with offs[b] <= idx
        while (lo_b < hi_b) {
            const int mid = (lo_b + hi_b + 1) >> 1;
            if (offs[mid] <= idx) lo_b = mid; else hi_b = mid - 1;
        }
        const int b = lo_b;
        const int s = idx - offs[b];
        if (a.mode == kPlanPrefill || a.mode == kPlanWindow) {
            const int Lq = q_len(b), Lk = k_len(b);
            const int i0 = s * a.bm, i1 = min(Lq, i0 + a.bm);
            int lo = 0, hi = 0;
            if (Lk > 0) rows_range(i0, i1, Lk - Lq, Lk, a.left, a.right, lo, hi);
            cost = (hi - lo + a.bn - 1) / a.bn;
            return make_int4(b, i0, lo, hi);
        }
        if (a.mode == kPlanBwdKeys) {
            // query rows i that see a key of [j0, j1): i + delta + right >= j0
            // and i + delta - left <= j1 - 1 (right = 0 when causal)
            const int Lq = q_len(b), Lk = k_len(b);
            const int j0 = s * a.bm, j1 = min(Lk, j0 + a.bm);
            const long long delta = (long long)Lk - Lq;
            long long qlo = 0, qhi = Lq;
            if (a.right < kInfOff) qlo = max(qlo, (long long)j0 - delta - a.right);
            if (a.left < kInfOff) qhi = min(qhi, (long long)j1 - 1 - delta + a.left + 1);
            qlo = min(qlo, (long long)Lq);
            if (qhi < qlo) qhi = qlo;
            cost = (int)((qhi - qlo + a.bn - 1) / a.bn);
            return make_int4(b, j0, (int)qlo, (int)qhi);
        }
        int lo, hi;
        vis_range(b, lo, hi);
        const int k_lo = min(hi, lo + s * split);
        const int k_hi = min(hi, k_lo + split);
        cost = (k_hi - k_lo + kDecQuantum - 1) / kDecQuantum;
        return make_int4(b, idx, k_lo, k_hi);
    };

    // ordering key: a cost bin (higher first) and, for prefill items, the
    // index taken in reverse
    const bool by_seq = a.mode == kPlanPrefill;
    auto order_bin = [&](const int4 &itm, int cost) {
        return min(by_seq ? (k_len(itm.x) + a.bn - 1) / a.bn : cost, kCostBins - 1);
    };
    auto order_idx = [&](int idx) { return by_seq ? N - 1 - idx : idx; };  // an involution

    if (a.mode == kPlanWindow) {
        // 3w. index order
        for (int idx = tid; idx < N; idx += kPlanThreads) {
            int cost;
            const int4 itm = make_item(idx, cost);
            a.items[idx] = itm;
            a.seqinfo[idx] = seq_info(itm.x);
        }
    } else if (N <= kSortMax) {
        // 3a. sort keys in LDS: ascending key = descending bin, then index
        for (int idx = tid; idx < N; idx += kPlanThreads) {
            int cost;
            const int4 itm = make_item(idx, cost);
            s_keys[idx] = ((uint32_t)(kCostBins - 1 - order_bin(itm, cost)) << 19) | (uint32_t)order_idx(idx);
        }
        __syncthreads();
        if (N <= kRankSortMax) {
            // rank = number of smaller keys (keys are unique): a permutation
            for (int i = tid; i < N; i += kPlanThreads) {
                const uint32_t key = s_keys[i];
                int rank = 0;
                for (int j = 0; j < N; ++j) rank += s_keys[j] < key;
                int cost;
                const int4 itm = make_item(order_idx((int)(key & ((1u << 19) - 1u))), cost);
                a.items[rank] = itm;
                a.seqinfo[rank] = seq_info(itm.x);
            }
        } else {
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
                        if ((x > y) == ((i & k) == 0)) {
                            s_keys[i] = y;
                            s_keys[l] = x;
                        }
                    }
                    __syncthreads();
                }
            }
            for (int i = tid; i < N; i += kPlanThreads) {
                int cost;
                const int4 itm = make_item(order_idx((int)(s_keys[i] & ((1u << 19) - 1u))), cost);
                a.items[i] = itm;
                a.seqinfo[i] = seq_info(itm.x);
            }
        }
    } else {
        // 3b. large lists: counting placement, highest bin first, stable in
        // the order of order_idx
        for (int i = tid; i < kCostBins; i += kPlanThreads) s_bins[i] = 0;
        __syncthreads();
        for (int idx = tid; idx < N; idx += kPlanThreads) {
            int cost;
            const int4 itm = make_item(idx, cost);
            a.unsorted[idx] = itm;
            a.cost[idx] = order_bin(itm, cost);
            atomicAdd(&s_bins[order_bin(itm, cost)], 1);
        }
        __syncthreads();
        constexpr int per = kCostBins / kPlanThreads;
        int local = 0;
        for (int k = 0; k < per; ++k) local += s_bins[kCostBins - 1 - (tid * per + k)];
        int total;
        int run = block_exclusive_scan(local, s_w, &total);
        for (int k = 0; k < per; ++k) {
            const int bin = kCostBins - 1 - (tid * per + k);
            const int c = s_bins[bin];
            s_bins[bin] = run;
            run += c;
        }
        __syncthreads();
        if (tid < 64) {  // one wave, 64 items at a time in order_idx order
            const int lane = tid;
            for (int base = 0; base < N; base += 64) {
                const bool active = base + lane < N;
                const int idx = active ? order_idx(base + lane) : 0;
                const int c = active ? a.cost[idx] : -1;
                unsigned long long remaining = __ballot(active);
                while (remaining) {
                    const int leader = __ffsll((long long)remaining) - 1;
                    const int lc = __shfl(c, leader);
                    const unsigned long long peers = __ballot(active && c == lc);
                    int start = lane == leader ? s_bins[lc] : 0;
                    start = __shfl(start, leader);
                    if (active && c == lc) {
                        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
                        const int4 itm = a.unsorted[idx];
                        a.items[start + rank] = itm;
                        a.seqinfo[start + rank] = seq_info(itm.x);
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
