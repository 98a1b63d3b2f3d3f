// Sliding-window + sparse compressed attention over shared K/V on gfx950
// matrix cores (the third scenario of the SparseAttnSharedkv README: q
// attends to the original keys in its sliding window and to the compressed
// keys its sparse indices select, in one softmax, with per-head sinks; the
// same tensor rows serve as keys and values).
//
// Per token t (row i of sequence b), kv head c, the key list is
//   window:     original positions [p - left, p + right] within [0, S2_b),
//               p = i + S2_b - Lq_b (aligned to the end of the keys),
//   compressed: with cmp_all (the README's second scenario) every position
//               t' of the S3_b = S2_b / cmp_ratio compressed keys that the
//               mask admits, t' <= i + S3_b - Lq_b (causal, aligned to the
//               bottom-right of the Lq x S3 matrix); otherwise the positions
//               cmp_sparse_indices[t, c, 0 .. topk-1] (third scenario),
//               those outside [0, S3_b) or past that bound selecting nothing;
// and for each of the g query heads h of c
//   O[t, h] = softmax_j(scale <q[t, h], kv_j>, sink_h) . kv_j.
// Lists longer than the LDS list (kSpListMax keys) are taken in chunks of
// it, the running max / sum / O carried from chunk to chunk.
//
// One workgroup = 2 waves = up to 64 query heads of one kv head (heads on
// the MFMA N side: each lane owns one head), a few consecutive tokens in
// turn (chosen by the host so that the grid fills the chip).
// For each token the physical rows of its key list go to LDS, then 64-row
// tiles are gathered global -> LDS (double buffered, one barrier per tile).
// A tile is read row-wise as the K operand (S^T = K Q^T, keys on M) and
// through the transposing LDS read as the V^T operand (O^T += V^T P^T):
// one XOR swizzle of the 16-byte chunks serves both without bank
// conflicts.  Keys that select nothing carry a -inf bias.
#include "va_internal.h"

namespace va {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

template <typename T>
struct Elt;
template <>
struct Elt<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static __device__ __forceinline__ v4 read_tr(const char *p)
    {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)((__attribute__((address_space(3))) char *)(p)));
    }
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // acc += a b with acc held in AGPRs (see mfma_agpr_drain)
    static __device__ __forceinline__ void mfma_agpr(f32x16 &acc, v8 a, v8 b)
    {
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
};
template <>
struct Elt<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    static __device__ __forceinline__ v4 read_tr(const char *p)
    {
        return __builtin_bit_cast(
            v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)((__attribute__((address_space(3))) char *)(p))));
    }
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ void mfma_agpr(f32x16 &acc, v8 a, v8 b)
    {
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
};

// Wait states between the last matrix instruction into an AGPR accumulator
// and any other read of it (16-pass instructions need 18); the leading
// s_nop of mfma_agpr covers a VALU write of its A / B operand just before.
// The matrix instructions into AGPRs are written in assembly because the
// compiler selects one register form for all of a kernel's matrix
// instructions (this file is built with the VGPR form for the others).
__device__ __forceinline__ void mfma_agpr_drain(f32x16 &acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}
// Places acc in AGPRs here, so that values written by VALU code (the zero
// start, a rescale) do not carry the accumulators into VGPRs across the loop.
__device__ __forceinline__ void in_agpr(f32x16 &acc)
{
    asm volatile("" : "+a"(acc));
}

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r): the
// rows of a row-wise operand read and the 4 rows x 4 chunks of a
// transposing read land on distinct chunks (D = 128; D = 64 per pair of
// rows sharing a 256-byte bank line).  Rows of D = 512 are 4 bank lines:
// a chunk's bank depends on its index mod 16 only, which the D = 128
// pattern permutes the same way.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    return D >= 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// 16 bytes per lane, global -> LDS (lane i writes LDS bytes [lds + 16 i, +16));
// no register results, M0 carries the LDS address.  Ordered by the kernel's
// own vector-memory wait and barrier before a slot is read.
__device__ __forceinline__ void copy16_global(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// D = 512 (the README's head size): 32-key tiles (64 KB of double-buffered
// LDS), O accumulators (256 registers) in AGPRs, one wave per SIMD.
template <typename T, int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(D == 512 ? 1 : 2, D == 512 ? 1 : 2)))
void k5_sparse16(SparseArgs a)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr bool BIG = D == 512;
    constexpr int BN = BIG ? 32 : 64;  // keys per tile
    constexpr int NMB = BN / 32;       // 32-key blocks of a tile (MFMA M side)
    constexpr int NT4 = BN / 16;       // 16-key P V steps
    constexpr int NCH = D / 8;         // 16-byte chunks per row
    constexpr int KS = D / 16;         // QK^T k-steps
    constexpr int MD = D / 32;         // 32-wide blocks of the head dimension
    constexpr int RPI = 64 / NCH;      // rows one 64-lane copy fills
    constexpr int LPW = BN / RPI / 2;  // copies per wave per tile (2 waves)
    constexpr int ROWB = D * 2;
    constexpr int TILEB = BN * ROWB;
    constexpr int KPF = 4, VPF = 3;    // LDS operand reads in flight ahead of their product (K, V)
    __shared__ __attribute__((aligned(16))) char s_tile[2 * TILEB];
    __shared__ __attribute__((aligned(16))) int s_list[kSpListMax];  // physical row per key, -1: none

    // (kv head, token chunk) of this workgroup: each XCD walks a contiguous
    // stretch of tokens, whose windows and selected compressed rows (one
    // sequence's cache) stay in its L2
    const int nchunks = gridDim.x;
    const int wg = xcd_contiguous(blockIdx.x + blockIdx.y * nchunks, nchunks * gridDim.y);
    const int c = wg / nchunks;
    const int t0 = (wg - c * nchunks) * a.tok_per_wg;
    const int t_end = min(a.T, t0 + a.tok_per_wg);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;
    const int hrow = wave * 32 + n;           // head of the group this lane owns
    const bool head_ok = hrow < a.g;
    const int head = c * a.g + (head_ok ? hrow : 0);

    // sequence of the first token: the last b with cu_q[b] <= t0
    int b = 0;
    {
        int lo_b = 0, hi_b = a.B - 1;
        while (lo_b < hi_b) {
            const int mid = (lo_b + hi_b + 1) >> 1;
            if (a.cu_q[mid] <= t0) lo_b = mid;
            else hi_b = mid - 1;
        }
        b = lo_b;
    }

    // LDS offsets: row-wise K operand read of key row 32 mb + n, chunk
    // 2 ks + h2; transposing V^T read of rows 16 t4 + 4 h2 + q4 (+8), chunk
    // 4 md + 2 ((lane & 31) >> 4) + ((l16 & 3) >> 1).  The swizzle changes
    // the low 4 bits of a chunk index only, so chunks 16 and above are a
    // constant byte offset from a lane's address of the low ones (8 + 8
    // address registers at d512).
    auto koff = [&](int mb, int ks) -> uint32_t {
        const int r = mb * 32 + n;
        return r * ROWB + ((((ks & 7) * 2 + h2) ^ swz<D>(r)) << 4) + (ks >> 3) * 256;
    };
    auto toff = [&](int md, int half) -> uint32_t {
        const int r = h2 * 4 + q4 + half * 8;
        const int ch = (md & 3) * 4 + ((lane & 31) >> 4) * 2 + ((l16 & 3) >> 1);
        return r * ROWB + ((ch ^ swz<D>(r)) << 4) + (l16 & 1) * 8 + (md >> 2) * 256;
    };
    const float sink2 = (a.sinks && head_ok) ? a.sinks[head] * kLog2e : -INFINITY;

    for (int t = t0; t < t_end; ++t) {
        while (a.cu_q[b + 1] <= t) ++b;  // empty sequences are stepped over
        const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
        const int i = t - q0;
        const int S2 = a.seqused_kv[b];
        const int S3 = S2 / a.cmp_ratio;
        const int p = i + S2 - Lq;
        const int win_lo = a.left >= kInfOff ? 0 : max(0, p - a.left);
        const int win_hi = a.right >= kInfOff ? S2 - 1 : min(S2 - 1, p + a.right);
        const int nwin = max(0, win_hi - win_lo + 1);
        const int last = i + S3 - Lq;  // last compressed position row i sees (< S3)
        const int L = nwin + (a.cmp_all ? max(0, min(S3, last + 1)) : a.topk);

        // Q^T operand fragments: lane (head n, half h2) holds d = 16 ks + 8 h2 .. +8
        v8 qf[KS];
        {
            const uint16_t *qp = (const uint16_t *)a.q + ((size_t)t * a.H + head) * D + h2 * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 x = *(const u32x4 *)(qp + ks * 16);
                if (!head_ok) x = u32x4{0, 0, 0, 0};
                qf[ks] = __builtin_bit_cast(v8, x);
            }
        }
        f32x16 o[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) {
#pragma unroll
            for (int v = 0; v < 16; ++v) o[md][v] = 0.f;
            if constexpr (BIG) in_agpr(o[md]);
        }
        float m_run = sink2, l_run = (sink2 != -INFINITY && h2 == 0) ? 1.f : 0.f;
        bool o_acc = false;   // some P V step has accumulated into O (wave-uniform)

        // the key list in chunks of at most kSpListMax keys
        for (int base = 0; base < L; base += kSpListMax) {
        const int Lc = min(L - base, kSpListMax);
        const int ntiles = (Lc + BN - 1) / BN;

        // physical rows of the chunk's keys, in two rounds of independent
        // loads (the indices, then the block-table entries they name): thread
        // tid takes keys base + tid, base + tid + 128, ...
        constexpr int KPT = kSpListMax / 128;
        static_assert(kSpListMax % 128 == 0, "whole rounds of 128 keys");
        int pos[KPT];   // position within its cache, -1: selects nothing
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int kg = base + tid + 128 * k;
            pos[k] = -1;
            if (kg < nwin) pos[k] = win_lo + kg;
            else if (tid + 128 * k < Lc) {
                if (a.cmp_all) {
                    pos[k] = kg - nwin;
                } else {
                    const int idx = a.indices[((size_t)t * a.Hkv + c) * a.topk + (kg - nwin)];
                    pos[k] = (idx >= 0 && idx <= last) ? idx : -1;
                }
            }
        }
        // block and slot of a position: shifts for power-of-two block sizes
        // (an integer division is a long instruction sequence per key)
        auto blk_of = [&](int x, bool ori) {
            const int sh = ori ? a.ori_shift : a.cmp_shift;
            return sh >= 0 ? x >> sh : x / (ori ? a.ori_bs : a.cmp_bs);
        };
        auto slot_of = [&](int x, bool ori) {
            const int bs = ori ? a.ori_bs : a.cmp_bs;
            return (ori ? a.ori_shift : a.cmp_shift) >= 0 ? x & (bs - 1) : x % bs;
        };
        int blk[KPT];
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int kg = base + tid + 128 * k;
            blk[k] = 0;
            if (pos[k] >= 0)
                blk[k] = kg < nwin ? a.ori_table[(size_t)b * a.ori_stride + blk_of(pos[k], true)]
                                   : a.cmp_table[(size_t)b * a.cmp_stride + blk_of(pos[k], false)];
        }
        // entries up to the end of the chunk's last tile (-1 past its end);
        // whether any key of the chunk selects nothing decides if its tiles
        // are masked
        bool none_here = false;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int kk = tid + 128 * k, kg = base + kk;
            if (kk < ntiles * BN) {
                const int bs = kg < nwin ? a.ori_bs : a.cmp_bs;
                const int row = pos[k] >= 0 ? blk[k] * bs + slot_of(pos[k], kg < nwin) : -1;
                s_list[kk] = row;
                none_here |= row < 0;
            }
        }
        const bool masked = __syncthreads_or(none_here);  // the list is complete

        // tile tau's rows into slot
        auto issue = [&](int tau, int slot) {
            // all list entries first: one LDS round trip, not one per copy
            int rows[LPW];
#pragma unroll
            for (int u = 0; u < LPW; ++u) rows[u] = s_list[tau * BN + (wave * LPW + u) * RPI + lane / NCH];
#pragma unroll
            for (int u = 0; u < LPW; ++u) {
                const int r = (wave * LPW + u) * RPI + lane / NCH;
                const int kg = base + tau * BN + r;
                const int row = rows[u];
                const char *src = (const char *)(kg < nwin ? a.ori_kv : a.cmp_kv);
                const int chunk = (lane % NCH) ^ swz<D>(r);
                // a key that selects nothing re-reads row 0 of the original
                // cache (finite data under a -inf bias)
                const size_t off = ((size_t)(row >= 0 ? row : 0) * a.Hkv + c) * ROWB + chunk * 16;
                copy16_global((row >= 0 ? src : (const char *)a.ori_kv) + off,
                              lds_addr(s_tile + slot * TILEB + (wave * LPW + u) * 1024));
            }
        };

        issue(0, 0);
        wait_vmem();
        __syncthreads();
        for (int tau = 0; tau < ntiles; ++tau) {
            const int slot = tau & 1;
            if (tau + 1 < ntiles) issue(tau + 1, slot ^ 1);
            const char *kt = s_tile + slot * TILEB;
            // S^T = K Q^T: lane value v of block mb is key 32 mb + 8 (v/4) + 4 h2 + v%4
            // steps st = (ks, mb), mb fastest; K operands read KPF steps
            // ahead of their product.  With one 32-key block the even and
            // odd k-steps go to two accumulators (two independent chains).
            f32x16 S[NMB], S1;
#pragma unroll
            for (int v = 0; v < 16; ++v) S1[v] = 0.f;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[mb][v] = 0.f;
            {
                constexpr int NST = KS * NMB;
                v8 kb[KPF];
#pragma unroll
                for (int q = 0; q < KPF; ++q) kb[q] = *(const v8 *)(kt + koff(q % NMB, q / NMB));
#pragma unroll
                for (int st = 0; st < NST; ++st) {
                    const int ks = st / NMB, mb = st % NMB;
                    const v8 cur = kb[st % KPF];
                    if (st + KPF < NST) kb[st % KPF] = *(const v8 *)(kt + koff((st + KPF) % NMB, (st + KPF) / NMB));
                    if (NMB == 1 && (ks & 1)) S1 = E::mfma(cur, qf[ks], S1);
                    else S[mb] = E::mfma(cur, qf[ks], S[mb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (NMB == 1) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) S[0][v] += S1[v];
                }
            }
            // raw scores (scale > 0: the max of the raw scores scaled is the
            // max of the scaled ones; the scale rides in the exponent's FMA)
            float mx = -INFINITY;
            if (masked) {
                // keys that select nothing (list entry -1) drop out
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const int4 row = *(const int4 *)&s_list[tau * BN + mb * 32 + e4 * 8 + h2 * 4];
                        S[mb][e4 * 4 + 0] = row.x < 0 ? -INFINITY : S[mb][e4 * 4 + 0];
                        S[mb][e4 * 4 + 1] = row.y < 0 ? -INFINITY : S[mb][e4 * 4 + 1];
                        S[mb][e4 * 4 + 2] = row.z < 0 ? -INFINITY : S[mb][e4 * 4 + 2];
                        S[mb][e4 * 4 + 3] = row.w < 0 ? -INFINITY : S[mb][e4 * 4 + 3];
                    }
            }
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[mb][v]);
            // the running max moves only when a tile raises it by more than
            // 2^8 (log2 units) for some head: until then the probabilities
            // stay below 2^8 and the O / l rescale is skipped
            mx = halves_max(mx) * a.scale_log2;
            if (__ballot(mx > m_run + 8.f) != 0ull) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
                if (o_acc) {   // O is zero until the token's first P V step
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        if constexpr (BIG) mfma_agpr_drain(o[md]);
#pragma unroll
                        for (int v = 0; v < 16; ++v) o[md][v] *= alpha;
                        if constexpr (BIG) in_agpr(o[md]);
                    }
                }
                m_run = m_new;
            }
            const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
            float rs = 0.f;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float pr = __builtin_amdgcn_exp2f(fmaf(S[mb][v], a.scale_log2, neg_m));
                    S[mb][v] = pr;
                    rs += pr;
                }
            l_run += rs;
            // O^T += V^T P^T, steps st = (t4, md) of 16 keys; V^T operands
            // read VPF steps ahead of their product
            {
                v8 pb[NT4];
#pragma unroll
                for (int t4 = 0; t4 < NT4; ++t4) {
                    f32x8 pv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] = S[t4 >> 1][(t4 & 1) * 8 + e];
                    pb[t4] = __builtin_convertvector(pv, v8);
                }
                constexpr int NST = NT4 * MD;
                auto vread = [&](int st) __attribute__((always_inline)) -> v8 {
                    const int t4 = st / MD, md = st % MD;
                    const v4 va = E::read_tr(kt + toff(md, 0) + t4 * 16 * ROWB);
                    const v4 vb = E::read_tr(kt + toff(md, 1) + t4 * 16 * ROWB);
                    return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                };
                v8 vbuf[VPF];
#pragma unroll
                for (int q = 0; q < VPF; ++q) vbuf[q] = vread(q);
#pragma unroll
                for (int st = 0; st < NST; ++st) {
                    const v8 cur = vbuf[st % VPF];
                    if (st + VPF < NST) vbuf[st % VPF] = vread(st + VPF);
                    if constexpr (BIG) E::mfma_agpr(o[st % MD], cur, pb[st / MD]);
                    else o[st % MD] = E::mfma(cur, pb[st / MD], o[st % MD]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            o_acc = true;
            wait_vmem();
            __syncthreads();
        }
        }  // chunks of the key list

        // epilogue: lane (head n, half h2) holds O^T[32 md + 8 i + 4 h2 + j]
        if constexpr (BIG) {
#pragma unroll
            for (int md = 0; md < MD; ++md) mfma_agpr_drain(o[md]);
        }
        const float l = halves_sum(l_run);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (head_ok) {
            uint16_t *op = (uint16_t *)a.out + ((size_t)t * a.H + head) * D;
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    f32x4 x;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = o[md][ii * 4 + j] * inv;
                    *(u32x2 *)(op + md * 32 + ii * 8 + h2 * 4) =
                        __builtin_bit_cast(u32x2, __builtin_convertvector(x, v4));
                }
            if (a.lse && h2 == 0)
                a.lse[(size_t)t * a.H + head] = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_sparse16(const SparseArgs &a, bool f16, int head_dim, hipStream_t s)
{
    const dim3 g((a.T + a.tok_per_wg - 1) / a.tok_per_wg, a.Hkv), blk(128);
#define VA_DIMS(TT)                                                                      \
    do {                                                                                 \
        if (head_dim == 512) hipLaunchKernelGGL((k5_sparse16<TT, 512>), g, blk, 0, s, a); \
        else if (head_dim == 128) hipLaunchKernelGGL((k5_sparse16<TT, 128>), g, blk, 0, s, a); \
        else hipLaunchKernelGGL((k5_sparse16<TT, 64>), g, blk, 0, s, a);                 \
    } while (0)
    if (f16) VA_DIMS(_Float16);
    else VA_DIMS(__bf16);
#undef VA_DIMS
    return hipGetLastError();
}

}  // namespace va
