// Forward at head size 512 on the dense varlen path (512 is the head size
// of the SparseAttnSharedkv README's operator): the same computation as the
// other forward kernels -- for query row i of sequence b and head h, with
// p = i + Lk_b - Lq_b, keys j in [p - left, p + right] within [0, Lk_b),
//   O[i, h] = softmax_j(scale <q[i, h], k_j> - slope_h |p - j|, sink_h) . v_j
// (the ALiBi term only with slopes), LSE[i, h] = natural log of the
// softmax's denominator -- over contiguous or paged K/V.
//
// One workgroup = 4 waves = one prefill item (128 query rows of one
// sequence) for one head; each wave owns 32 rows, one per lane pair (keys
// on the MFMA M side: S^T = K Q^T; O^T += V^T P^T).  At D = 512 the O^T
// accumulators of a wave's rows fill 256 registers, so they live in AGPRs
// (one wave per SIMD) and the Q^T fragments take 128 VGPRs.  Per 32-key
// tile, K and V rows go global -> LDS (double buffered, 128 KB) and are
// read row-wise (K operand) and through the transposing LDS read (V^T
// operand), one XOR swizzle of the 16-byte chunks serving both.  The
// matrix instructions take their LDS operands several products after the
// reads are issued, and the exponentials of tile t run between the
// products of tile t + 1 (software pipeline, one barrier per tile).  Tiles
// a wave cannot see are skipped; masks are evaluated only on tiles that
// straddle a mask edge.
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
// transposing read land on distinct banks (a 1 KB row is 4 bank lines; a
// chunk's bank depends on its index mod 16 only).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// 16 bytes per lane, global -> LDS (lane i writes LDS bytes [lds + ldsoff
// + 16 i, +16)) from a wave-uniform base (SGPR pair) plus a 32-bit lane
// offset; no register results.  M0 (the LDS address) is formed here, so
// that the destinations of a tile's rows are not each held in a register.
// Ordered by the kernel's own vector-memory wait and barrier before a
// buffer is read.
__device__ __forceinline__ void copy16_global_sv(const void *sbase, uint32_t voff, uint32_t lds, uint32_t ldsoff)
{
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 : : "v"(voff), "s"(sbase), "s"(lds), "s"(ldsoff) : "m0", "scc");
}
// (lane16 ^ x) + y computed at the point of use (kept out of
// loop-invariant hoisting, which would hold one register per distinct x)
__device__ __forceinline__ uint32_t xor_add_here(uint32_t lane16, uint32_t x, uint32_t y)
{
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2\n\tv_add_u32 %0, %3, %0" : "=&v"(r) : "s"(x), "v"(lane16), "s"(y));
    return r;
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

template <typename T, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k8_prefill512(
    AttnArgs a, const int4 *__restrict__ items, const int4 *__restrict__ seqinfo, const int32_t *__restrict__ count)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr int D = 512;
    constexpr int BN = 32;             // keys per tile
    constexpr int KS = D / 16;         // QK^T k-steps
    constexpr int MD = D / 32;         // 32-wide blocks of the head dimension
    constexpr int ROWB = D * 2;        // bytes per row (one 64-lane copy)
    constexpr int TILEB = BN * ROWB;
    constexpr int CPW = 2 * BN / 4;
    constexpr int KPF = 4, VPF = 3;   // LDS operand reads in flight ahead of their product (K, V)    // copies per wave per tile: waves 0, 1 take K rows, 2, 3 V rows
    __shared__ __attribute__((aligned(16))) char s_k[2 * TILEB];
    __shared__ __attribute__((aligned(16))) char s_v[2 * TILEB];

    int item, head;
    map_block(blockIdx.x, a.H, item, head);
    const int n_items = *count;
    if (item >= n_items) return;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    const int b = it.x, i0 = it.y, kv_lo = it.z, kv_hi = it.w;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int delta = Lk - Lq;
    const int c = head / a.g;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;
    const int r0 = i0 + wave * 32;   // the wave's first row
    const int i = r0 + n;            // this lane's row
    const bool row_ok = i < Lq;
    int lo = 1, hi = 0;              // keys row i sees (none past the sequence)
    if (row_ok) row_bounds(i, delta, Lk, a.left, a.right, lo, hi);
    // keys some row of the wave sees (wlo..whi) and keys all of them see (flo..fhi)
    int wlo = 1, whi = 0, flo = 0x7fffffff, fhi = -1;
    if (r0 < Lq) {
        int l0, h0, l1, h1;
        row_bounds(r0, delta, Lk, a.left, a.right, l0, h0);
        row_bounds(min(r0 + 31, Lq - 1), delta, Lk, a.left, a.right, l1, h1);
        wlo = l0; whi = h1; flo = l1; fhi = h0;
    }
    const float sink2 = a.sinks ? a.sinks[head] * kLog2e : -INFINITY;
    // ALiBi on the raw scores: - slope / scale |pos - j| (0 without slopes)
    const float alibi_r = a.alibi ? a.alibi[head] / a.scale : 0.f;
    const float pos = (float)(i + delta);

    // Q^T operand fragments: lane (row n, half h2) holds d = 16 ks + 8 h2 .. +8
    // (rows past the sequence read the item's first row, zeroed)
    v8 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + (row_ok ? i : i0)) * a.H + head) * D + h2 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4 *)(qp + ks * 16);
            if (!row_ok) x = u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(v8, x);
        }
    }
    f32x16 o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int v = 0; v < 16; ++v) o[md][v] = 0.f;
        in_agpr(o[md]);
    }
    float m_run = sink2, l_run = (sink2 != -INFINITY && h2 == 0) ? 1.f : 0.f;

    // LDS offsets: row-wise K operand read of key row n, chunk 2 ks + h2;
    // transposing V^T read of rows 16 t4 + 4 h2 + q4 (+8), chunk
    // 4 md + 2 ((lane & 31) >> 4) + ((l16 & 3) >> 1).  The swizzle changes
    // the low 4 bits of a chunk index only, so chunks 16 and above are a
    // constant byte offset from a lane's address of the low ones.
    auto koff = [&](int ks) -> uint32_t {
        return n * ROWB + ((((ks & 7) * 2 + h2) ^ swz(n)) << 4) + (ks >> 3) * 256;
    };
    auto toff = [&](int md, int half) -> uint32_t {
        const int r = h2 * 4 + q4 + half * 8;
        const int ch = (md & 3) * 4 + ((lane & 31) >> 4) * 2 + ((l16 & 3) >> 1);
        return r * ROWB + ((ch ^ swz(r)) << 4) + (l16 & 1) * 8 + (md >> 2) * 256;
    };

    // tile tau's K rows (waves 0, 1) or V rows (waves 2, 3) into buffer
    // slot; one 64-lane copy per row.  Rows past the item's key range repeat
    // its last row (finite data under the mask).  Contiguous K/V: the rows
    // of a tile are a constant stride apart, so the tile has one base and a
    // row's offset joins the lane's chunk offset.  Paged K/V: the row of a
    // copy is the same for all its lanes, so its block-table entry is one
    // scalar load; the entries of 8 copies are read before those copies.
    const bool is_v = wave >= 2;
    auto issue = [&](int tau, int slot) __attribute__((always_inline)) {
        const char *src = (const char *)(is_v ? a.v : a.k);
        // LDS address of the wave's first row in the slot
        const uint32_t dst = lds_addr((is_v ? s_v : s_k) + slot * TILEB + (wave & 1) * CPW * ROWB);
        const int jt = kv_lo + tau * BN;   // the tile's first key (< kv_hi)
        if constexpr (!PAGED) {
            const char *tb = src + ((size_t)(k0 + jt) * a.Hkv + c) * (D * 2);
            const int rmax = kv_hi - 1 - jt;
            const uint32_t rstride = (uint32_t)a.Hkv * (D * 2);
#pragma unroll
            for (int u = 0; u < CPW; ++u) {
                const int r = (wave & 1) * CPW + u;
                const uint32_t roff = (uint32_t)min(r, rmax) * rstride;
                copy16_global_sv(tb, xor_add_here(lane * 16, swz(r) * 16, roff), dst, u * ROWB);
            }
        } else {
#pragma unroll
            for (int h = 0; h < CPW; h += 8) {
                const char *rb[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = (wave & 1) * CPW + h + u;
                    const int j = min(jt + r, kv_hi - 1);
                    const int bi = a.bs_shift >= 0 ? j >> a.bs_shift : j / a.block_size;
                    // the table is read-only here: through the constant
                    // address space the entry is a scalar load (its own
                    // counter, no wait on the copies in flight)
                    const int blk = ((const __attribute__((address_space(4))) int32_t *)a.block_table)[(size_t)b * a.bt_stride + bi];
                    const size_t row = (size_t)blk * a.block_size + (j - bi * a.block_size);
                    rb[u] = src + (row * a.Hkv + c) * (D * 2);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = (wave & 1) * CPW + h + u;
                    copy16_global_sv(rb[u], xor_add_here(lane * 16, swz(r) * 16, 0u), dst, (h + u) * ROWB);
                }
            }
        }
    };

    const int ntiles = kv_hi > kv_lo ? (kv_hi - kv_lo + BN - 1) / BN : 0;
    auto visible = [&](int tau) __attribute__((always_inline)) {   // some row of the wave sees a key of tile tau
        const int j0 = kv_lo + tau * BN;
        return j0 <= whi && j0 + BN - 1 >= wlo;
    };

    // S^T = K Q^T for the tile in kt: lane value v is key j0 + 8 (v/4) +
    // 4 h2 + v%4 of row n.  Two accumulators (even / odd k-steps); K
    // operands read KPF steps ahead of their product; hook(ks) runs after
    // step ks (independent vector work placed between the products).
    auto qk = [&](f32x16 &S, const char *kt, auto &&hook) __attribute__((always_inline)) {
        f32x16 S1;
#pragma unroll
        for (int v = 0; v < 16; ++v) { S[v] = 0.f; S1[v] = 0.f; }
        v8 kb[KPF];
#pragma unroll
        for (int p = 0; p < KPF; ++p) kb[p] = *(const v8 *)(kt + koff(p));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v8 cur = kb[ks % KPF];
            if (ks + KPF < KS) kb[ks % KPF] = *(const v8 *)(kt + koff(ks + KPF));
            if (ks & 1) S1 = E::mfma(cur, qf[ks], S1);
            else S = E::mfma(cur, qf[ks], S);
            hook(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] += S1[v];
    };
    // ALiBi and the mask on the raw scores of tile tau, their row max, and
    // the running max moved (O and l rescaled) only when the tile raises it
    // by more than 2^8 (log2 units) for some row: until then the
    // probabilities stay below 2^8.  The max is taken on raw scores (scale > 0).
    auto row_max = [&](f32x16 &S, int tau) __attribute__((always_inline)) {
        const int j0 = kv_lo + tau * BN;
        if (a.alibi) {
            const float base = pos - (float)(j0 + 4 * h2);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                S[v] = fmaf(-alibi_r, fabsf(base - (float)(8 * (v >> 2) + (v & 3))), S[v]);
        }
        if (!(j0 >= flo && j0 + BN - 1 <= fhi)) {
            // key j is visible iff (unsigned)(j - lo) <= (unsigned)(hi - lo);
            // rows that see nothing (hi < lo) get span 0 and offsets >= 1
            const bool none = hi < lo;
            const uint32_t span = none ? 0u : (uint32_t)(hi - lo);
            const int jb = none ? 1 : j0 + 4 * h2 - lo;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t d = (uint32_t)(jb + 8 * (v >> 2) + (v & 3));
                S[v] = d > span ? -INFINITY : S[v];
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[v]);
        mx = halves_max(mx) * a.scale_log2;
        if (__ballot(mx > m_run + 8.f) != 0ull) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            // rows whose running max is still -inf have O = 0: no rescale
            // while the whole wave is in that state (its first tile)
            if (__ballot(m_run != -INFINITY) != 0ull) {
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    mfma_agpr_drain(o[md]);
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[md][v] *= alpha;
                    in_agpr(o[md]);
                }
            }
            m_run = m_new;
        }
    };
    // probability v of the tile in S, in place: 2^(scale_log2 S - m)
    auto prob = [&](f32x16 &S, int v, float neg_m, float &rs) __attribute__((always_inline)) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(S[v], a.scale_log2, neg_m));
        S[v] = pr;
        rs += pr;
    };
    // O^T += V^T P^T over the tile in vt, step st = (t4, md) of 16 keys;
    // V^T operands read VPF steps ahead of their product
    auto pv = [&](const f32x16 &P, const char *vt) __attribute__((always_inline)) {
        v8 pb[BN / 16];
#pragma unroll
        for (int t4 = 0; t4 < BN / 16; ++t4) {
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = P[t4 * 8 + e];
            pb[t4] = __builtin_convertvector(x, v8);
        }
        constexpr int NST = BN / 16 * MD;
        auto vread = [&](int st) __attribute__((always_inline)) -> v8 {
            const int t4 = st / MD, md = st % MD;
            const v4 va = E::read_tr(vt + toff(md, 0) + t4 * 16 * ROWB);
            const v4 vb = E::read_tr(vt + toff(md, 1) + t4 * 16 * ROWB);
            return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        v8 vbuf[VPF];
#pragma unroll
        for (int p = 0; p < VPF; ++p) vbuf[p] = vread(p);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const v8 cur = vbuf[st % VPF];
            if (st + VPF < NST) vbuf[st % VPF] = vread(st + VPF);
            E::mfma_agpr(o[st % MD], cur, pb[st / MD]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Software pipeline over the tiles: K and V rings of two slots (tile t
    // in slot t & 1).  Iteration t computes S^T of tile t + 1 with the
    // exponentials of tile t placed between its products, then O^T +=
    // V^T P^T of tile t, then the row max of tile t + 1; its copies (issued
    // at the top, landed by its closing barrier) bring K(t + 2) into the slot
    // K(t) left and V(t + 1) into the slot V(t - 1) left.
    f32x16 sa, sb;
    if (ntiles > 0) {
        issue(0, 0);                           // K(0) by waves 0, 1; V(0) by waves 2, 3
        if (!is_v && ntiles > 1) issue(1, 1);  // K(1)
    }
    wait_vmem();
    __syncthreads();
    bool vc = ntiles > 0 && visible(0);
    if (vc) {
        qk(sa, s_k, [](int) {});
        row_max(sa, 0);
    }
    __syncthreads();  // K slot 0 is refilled by iteration 0

    auto iteration = [&](int t, auto BUFC, f32x16 &Sc, f32x16 &Sn) __attribute__((always_inline)) {
        constexpr int BUF = decltype(BUFC)::value;
        if (is_v) {
            if (t + 1 < ntiles) issue(t + 1, BUF ^ 1);
        } else {
            if (t + 2 < ntiles) issue(t + 2, BUF);
        }
        const bool vn = t + 1 < ntiles && visible(t + 1);
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        float rs = 0.f;
        if (vn) {
            qk(Sn, s_k + (BUF ^ 1) * TILEB, [&](int ks) {
                if (ks & 1) prob(Sc, ks >> 1, neg_m, rs);
            });
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) prob(Sc, v, neg_m, rs);
        }
        if (vc) {
            l_run += rs;
            pv(Sc, s_v + BUF * TILEB);
        }
        if (vn) row_max(Sn, t + 1);
        vc = vn;
        wait_vmem();
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        iteration(t, std::integral_constant<int, 0>{}, sa, sb);
        iteration(t + 1, std::integral_constant<int, 1>{}, sb, sa);
    }
    if (t < ntiles) iteration(t, std::integral_constant<int, 0>{}, sa, sb);

    // epilogue: lane (row n, half h2) holds O^T[32 md + 8 ii + 4 h2 + j]
#pragma unroll
    for (int md = 0; md < MD; ++md) mfma_agpr_drain(o[md]);
    const float l = halves_sum(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok) {
        uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + i) * a.H + head) * D;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                f32x4 x;
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = o[md][ii * 4 + j] * inv;
                *(u32x2 *)(op + md * 32 + ii * 8 + h2 * 4) = __builtin_bit_cast(u32x2, __builtin_convertvector(x, v4));
            }
        if (a.lse && h2 == 0)
            a.lse[(size_t)(q0 + i) * a.H + head] = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill512(const AttnArgs &a, bool f16, bool paged, const int4 *items, const int4 *seqinfo,
                             const int32_t *count, int grid, hipStream_t s)
{
    const dim3 g(grid), blk(256);
    if (f16) {
        if (paged) hipLaunchKernelGGL((k8_prefill512<_Float16, true>), g, blk, 0, s, a, items, seqinfo, count);
        else hipLaunchKernelGGL((k8_prefill512<_Float16, false>), g, blk, 0, s, a, items, seqinfo, count);
    } else {
        if (paged) hipLaunchKernelGGL((k8_prefill512<__bf16, true>), g, blk, 0, s, a, items, seqinfo, count);
        else hipLaunchKernelGGL((k8_prefill512<__bf16, false>), g, blk, 0, s, a, items, seqinfo, count);
    }
    return hipGetLastError();
}

}  // namespace va
