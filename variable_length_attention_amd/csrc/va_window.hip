// Sliding-window attention for wide GQA / MQA groups (32 to 64 query heads
// per kv head) on gfx950 matrix cores: the first scenario of the
// SparseAttnSharedkv README (window (127, 0) over the original keys, 64
// query heads on one kv head, per-head sinks) with separate K and V,
// contiguous or paged through a block table.
//
// Query row i of sequence b (p = i + Lk_b - Lq_b) sees keys
// [p - left, p + right] within [0, Lk_b); for each query head h
//   O[i, h] = softmax_j(scale <q[i, h], k_j>, sink_h) . v_j,
//   LSE[i, h] = natural log of that softmax's denominator.
//
// One workgroup = 4 waves = one block of R consecutive query rows of one
// sequence and one kv head.  The union of the block's windows (at most
// left + right + R rows of K and of V) is copied global -> LDS once; then
// every row of the block is computed against its own window slice, heads on
// the MFMA N side (S^T = K Q^T with keys on M, one lane per head; O^T +=
// V^T P^T through the transposing LDS read).  A row's 64-key tiles cover
// exactly its window, so a full window does no masked work, and the waves
// never wait for each other after the copy: 64 heads take 2 waves per row
// and 2 rows run at once (32 heads: 1 wave per row, 4 rows at once).
#include "va_internal.h"

#include <type_traits>

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
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ v4 read_tr(const char *p)
    {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)((__attribute__((address_space(3))) char *)(p)));
    }
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elt<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ v4 read_tr(const char *p)
    {
        return __builtin_bit_cast(
            v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)((__attribute__((address_space(3))) char *)(p))));
    }
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r): the
// rows of a row-wise operand read and the 4 rows x 4 chunks of a
// transposing read land on distinct chunks (D = 128; D = 64 per pair of
// rows sharing a 256-byte bank line).  It depends on r mod 16 only.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// 16 bytes per lane, global -> LDS (lane i writes LDS bytes [lds + 16 i, +16));
// no register results, M0 carries the LDS address.  Ordered by the vector
// memory wait and the barrier that follow the copies.
__device__ __forceinline__ void copy16_global(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Makes x available at this point of the instruction stream (an empty
// volatile statement that reads and writes it): operands read in one batch
// are waited for once, and the next batch's reads are issued while the
// matrix instructions that use this one run.
template <typename V>
__device__ __forceinline__ void pin(V &x)
{
    asm volatile("" : "+v"(x));
}

// The O accumulators hold O[head][d] with lane (n, h2) <-> d = 32 md + n and
// register v <-> head (v/4) 8 + 4 h2 + v%4.  Per-head scalars live one head
// per lane (lanes h and h + 32); this gives every lane register v's one: an
// LDS-crossbar permute (no LDS memory, no vector ALU work) from lane
// (v/4) 8 + 4 h2 + v%4.
__device__ __forceinline__ float head_value(float x, int v, int h2)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(h2 * 16 + 4 * ((v >> 2) * 8 + (v & 3)), __float_as_int(x)));
}

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

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k6_window16(
    AttnArgs a, const int4 *__restrict__ items, const int4 *__restrict__ seqinfo, const int32_t *__restrict__ count)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    typedef typename E::v2 v2;
    constexpr int CAP = win_cap(D);    // LDS rows of the window (K and V each)
    constexpr int NCH = D / 8;         // 16-byte chunks per row
    constexpr int KS = D / 16;         // QK^T k-steps
    constexpr int MD = D / 32;         // 32-wide blocks of the head dimension
    constexpr int RPI = 64 / NCH;      // rows one 64-lane copy fills
    constexpr int ROWB = 2 * D;        // bytes per LDS row
    static_assert(CAP % RPI == 0, "whole copies");
    __shared__ __attribute__((aligned(16))) char s_k[CAP * ROWB];
    __shared__ __attribute__((aligned(16))) char s_v[CAP * ROWB];

    // each XCD takes a contiguous range of items: neighbouring rows share
    // most of their window, which then stays in that XCD's L2
    const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
    const int c = wg % a.Hkv;
    const int item = wg / a.Hkv;
    const int n_items = *count;
    if (item >= n_items) return;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    const int b = it.x, i0 = it.y, kv_lo = it.z, kv_hi = it.w;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int delta = Lk - Lq;
    const int nwin = kv_hi - kv_lo;              // <= left + right + R <= CAP (host)
    const int rows_here = min(a.item_rows, Lq - i0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;

    // ---- the block's window: rows kv_lo .. kv_hi-1 (contiguous, or
    // through the block table) to LDS rows 0 .. nwin-1; rows past nwin (read
    // only as keys outside a row's window) repeat the last row, so every
    // value the products meet is finite
    if (nwin > 0) {
        const int nl = min(CAP, (nwin + 63 + RPI - 1) / RPI * RPI);
        for (int u = wave; u < nl / RPI; u += 4) {
            const int r = u * RPI + lane / NCH;
            const int chunk = (lane % NCH) ^ swz<D>(r);
            const size_t off = kv_row_offset<D, PAGED>(a, b, k0, c, kv_lo + min(r, nwin - 1)) * 2 + chunk * 16;
            copy16_global((const char *)a.k + off, lds_addr(s_k + u * 1024));
            copy16_global((const char *)a.v + off, lds_addr(s_v + u * 1024));
        }
    }

    // waves per row (1: up to 32 heads, 2: up to 64) and rows in flight
    const int wpr = a.g > 32 ? 2 : 1;
    const int rif = 4 / wpr;
    const int hrow = (wave % wpr) * 32 + n;      // head of the group this lane owns
    const bool head_ok = hrow < a.g;
    const int head = c * a.g + (head_ok ? hrow : 0);
    const float sink2 = (a.sinks && head_ok) ? a.sinks[head] * kLog2e : -INFINITY;

    // Q^T operand fragments of block row r (clamped to the block): lane
    // (head n, half h2) holds d = 16 ks + 8 h2 .. +8 (lanes past the group
    // read head 0; their results are never stored).  A row's fragments are
    // loaded when the wave starts its previous row, so their latency hides
    // behind a whole row of work; loads and stores share one counter, and
    // the wait for them leaves the stores issued after them in flight.
    auto load_q = [&](int r, v8 (&dst)[KS]) {
        const size_t tq = (size_t)q0 + i0 + min(r, rows_here - 1);
        const uint16_t *qp = (const uint16_t *)a.q + (tq * a.H + head) * D + h2 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dst[ks] = __builtin_bit_cast(v8, *(const u32x4 *)(qp + ks * 16));
    };
    v8 qf[KS];
    load_q(wave / wpr, qf);

    wait_vmem();
    __syncthreads();

    for (int r = wave / wpr; r < rows_here; r += rif) {
        v8 qn[KS];
        load_q(r + rif, qn);
        const int i = i0 + r;
        const int p = i + delta;
        const int kst = max(0, p - a.left);
        const int ken = min(Lk - 1, p + a.right);
        const int nk = max(0, ken - kst + 1);
        const int base = kst - kv_lo;            // LDS row of the row's first key
        const size_t t = (size_t)q0 + i;
        // byte offsets within a row: K operand chunk 2 ks + h2 of a row
        // congruent to base + n (mod 16); V^T chunk 4 md + 2 ((lane & 31) >> 4)
        // + ((l16 & 3) >> 1) of a row congruent to base + 4 h2 + q4 + 8 half.
        // A tile step of 64 rows keeps a row's residue mod 16, so these hold
        // for every tile of the row.
        const int kx = swz<D>(base + n);
        const int vx0 = swz<D>(base + h2 * 4 + q4), vx1 = swz<D>(base + h2 * 4 + q4 + 8);
        uint32_t kofs[KS], vofs[MD][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kofs[ks] = ((ks * 2 + h2) ^ kx) << 4;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ch = md * 4 + ((lane & 31) >> 4) * 2 + ((l16 & 3) >> 1);
                vofs[md][half] = ((ch ^ (half ? vx1 : vx0)) << 4) | ((l16 & 1) * 8);
            }

        f32x16 o[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[md][v] = 0.f;
        float m_run = sink2, l_run = (sink2 != -INFINITY && h2 == 0) ? 1.f : 0.f;

        // one 64-key tile at LDS row base + 64 tau.  FULL: all 64 keys are in
        // the row's window, so no key is masked and every row read is below
        // nwin <= CAP (whole-row offsets then fold into the instructions'
        // immediates).  Otherwise the window's last, partial tile: keys past
        // it get a -inf score and reads clamp to the allocation (a clamped
        // row only serves such keys).
        auto tile = [&](int tau, auto full) {
            constexpr bool FULL = decltype(full)::value == 1;
            const int tb = base + tau * 64;
            // the row's offsets enter each tile as they are (both kinds of
            // tile share them; a tile adds its own row base to each)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) pin(kofs[ks]);
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                pin(vofs[md][0]);
                pin(vofs[md][1]);
            }
            auto rowb = [&](int rr) -> uint32_t { return (uint32_t)min(rr, CAP - 1) * ROWB; };
            // operand addresses: in a full tile one register per K chunk and
            // per V^T chunk, the row steps within the tile in the
            // instructions' immediates; in the partial tile per clamped row
            const char *kp[KS], *vp[MD][2];
            if constexpr (FULL) {
                const char *kt = s_k + (tb + n) * ROWB;
                const char *vt = s_v + (tb + h2 * 4 + q4) * ROWB;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kp[ks] = kt + kofs[ks];
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    vp[md][0] = vt + vofs[md][0];
                    vp[md][1] = vt + vofs[md][1];
                }
            }
            // S^T = K Q^T: lane value v of block mb is key 64 tau + 32 mb + 8 (v/4) + 4 h2 + v%4
            f32x16 S[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) S[mb][v] = 0.f;
                // the block's K operands in one batch of reads, then the products
                v8 kf[KS];
                if constexpr (FULL) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const v8 *)(kp[ks] + mb * 32 * ROWB);
                } else {
                    const char *kr = s_k + rowb(tb + mb * 32 + n);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const v8 *)(kr + kofs[ks]);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) pin(kf[ks]);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) S[mb] = E::mfma(kf[ks], qf[ks], S[mb]);
            }
            if constexpr (!FULL) {
                const int lim = nk - tau * 64 - 4 * h2;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        S[mb][v] = mb * 32 + 8 * (v >> 2) + (v & 3) >= lim ? -INFINITY : S[mb][v];
            }
            // the max of the unscaled scores, scaled once (scale > 0 keeps
            // the order); the scale then rides in the exponent's FMA
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
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
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float av = head_value(alpha, v, h2);
#pragma unroll
                    for (int md = 0; md < MD; ++md) o[md][v] *= av;
                }
                m_run = m_new;
            }
            const float m_neg = m_run == -INFINITY ? 0.f : -m_run;
            float rs = 0.f;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][v], a.scale_log2, m_neg));
                    S[mb][v] = pr;
                    rs += pr;
                }
            l_run += rs;
            // O += P V, 16 keys per step: rows 16 t4 + 4 h2 + q4 (+8).  The
            // P fragment (heads on M) comes straight from the S^T
            // accumulators, the V fragment from the transposing read.
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                f32x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = S[t4 >> 1][(t4 & 1) * 8 + e];
                const v8 pb = __builtin_convertvector(pv, v8);
                v8 vf[MD];
                if constexpr (FULL) {
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        const v4 va = E::read_tr(vp[md][0] + t4 * 16 * ROWB);
                        const v4 vb = E::read_tr(vp[md][1] + (t4 * 16 + 8) * ROWB);
                        vf[md] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                } else {
                    const char *v0 = s_v + rowb(tb + t4 * 16 + h2 * 4 + q4);
                    const char *v1 = s_v + rowb(tb + t4 * 16 + h2 * 4 + q4 + 8);
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        const v4 va = E::read_tr(v0 + vofs[md][0]);
                        const v4 vb = E::read_tr(v1 + vofs[md][1]);
                        vf[md] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                }
#pragma unroll
                for (int md = 0; md < MD; ++md) pin(vf[md]);
#pragma unroll
                for (int md = 0; md < MD; ++md) o[md] = E::mfma(pb, vf[md], o[md]);
            }
        };
        // (the first full tile is written out on its own: the register
        // allocation of the loop then fits without spills)
        const int nfull = nk >> 6;
        if (nfull > 0) {
            tile(0, std::integral_constant<int, 1>{});
            for (int tau = 1; tau < nfull; ++tau) tile(tau, std::integral_constant<int, 1>{});
        }
        if (nk & 63) tile(nfull, std::integral_constant<int, 0>{});


        // epilogue: register v of lane (n, h2) holds O[head (v/4) 8 + 4 h2 +
        // v%4][32 md + n].  Each lane packs its two heads h, h + 1 at d = n
        // into one word, neighbour lanes trade the words and each keeps the
        // halves of one head (h at d = n, n + 1 on even lanes, h + 1 at
        // d = n - 1, n on odd ones): every store covers 64 contiguous bytes
        // of 4 heads.  Buffer
        // stores over this row's heads of the group: the range check drops
        // heads past the group (and every LSE lane when lse is NULL), so no
        // branch splits the stores from the loads above.
        const float l = halves_sum(l_run);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float iv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) iv[v] = head_value(inv, v, h2);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (char *)a.out + (t * a.H + (size_t)c * a.g) * D * 2, (short)0, a.g * D * 2, 0x00020000);
        const bool odd = n & 1;
        // byte selectors of v_perm (bytes 0-3: own word, 4-7: the neighbour's)
        const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
        // the lane's store offset (its head parity and half, its pair of d);
        // each store adds a constant (kept in the instruction and in an
        // SGPR offset rather than in a register per store across rows)
        uint32_t obase = (uint32_t)((((wave % wpr) * 32 + 4 * h2 + (odd ? 1 : 0)) * D + (n & ~1)) * 2);
        pin(obase);
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int vp = 0; vp < 8; ++vp) {
                const float x = o[md][2 * vp] * iv[2 * vp], y = o[md][2 * vp + 1] * iv[2 * vp + 1];
                const uint32_t own = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, v2));
                // quad_perm [1, 0, 3, 2]: the word of lane n ^ 1
                const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
                const uint32_t pk = __builtin_amdgcn_perm(nb, own, sel);
                // head (wave % wpr) 32 + 8 (vp / 2) + 4 h2 + 2 (vp % 2) + odd, d = 32 md + (n & ~1)
                __builtin_amdgcn_raw_buffer_store_b32(pk, ro, obase + (2 * (vp & 1) * D + md * 32) * 2,
                                                      (vp >> 1) * 8 * D * 2, 0);
            }
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
            a.lse ? (void *)(a.lse + t * a.H + (size_t)c * a.g) : nullptr, (short)0, a.lse ? a.g * 4 : 0, 0x00020000);
        const float lse = l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, h2 == 0 ? hrow * 4 : a.g * 4, 0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
    }
}

}  // namespace

hipError_t launch_window16(const AttnArgs &a, bool f16, int head_dim, bool paged, const int4 *items,
                           const int4 *seqinfo, const int32_t *count, int grid, hipStream_t s)
{
    const dim3 g(grid), blk(256);
#define VA_LAUNCH(TT, DD, PP) hipLaunchKernelGGL((k6_window16<TT, DD, PP>), g, blk, 0, s, a, items, seqinfo, count)
#define VA_DIMS(TT)                                                           \
    do {                                                                      \
        if (head_dim == 128) {                                                \
            if (paged) VA_LAUNCH(TT, 128, true); else VA_LAUNCH(TT, 128, false); \
        } else {                                                              \
            if (paged) VA_LAUNCH(TT, 64, true); else VA_LAUNCH(TT, 64, false);   \
        }                                                                     \
    } while (0)
    if (f16) VA_DIMS(_Float16);
    else VA_DIMS(__bf16);
#undef VA_DIMS
#undef VA_LAUNCH
    return hipGetLastError();
}

}  // namespace va
