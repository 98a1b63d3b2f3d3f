// bf16 / fp16 prefill forward on gfx950 matrix cores (one kernel template
// over the 16-bit input type).
//
// One workgroup = 4 waves = 128 query rows of one head (32 rows per wave);
// key/value tiles of 64 rows are staged in LDS (double buffered, one barrier
// per tile) and shared by the 4 waves.  Per wave and tile:
//   S^T = K * Q^T      8 (D=128) x 2 MFMA 32x32x16 bf16 / f16, fp32 accumulate.
//                      With keys on the MFMA M side, each lane ends up owning
//                      one query row: the row max needs one cross-lane step
//                      (lanes l and l^32) and the row sum none until the end.
//   scale, mask, online softmax in fp32 registers (exp2 domain);
//   O^T += V^T * P^T   4 x 4 MFMA 32x32x16; V^T operands come straight from
//                      the row-major V tile through the transposing LDS read
//                      ds_read_b64_tr_b16, P^T straight from the S^T
//                      accumulators (same lane, same key order).
// Tiles a wave cannot see are skipped; masks are evaluated only on tiles
// that straddle a mask edge.
//
// Method: the online-softmax form of softmax(Q K^T * scale) V
// (SparseAttnSharedkv README, formula section); it reaches the same value as
// the three-pass row softmax of the boostr CPU forward up to rounding.  The
// sink logit enters as the initial running max / sum (a key with a zero
// value row); the returned LSE is max + ln(sum) as in that CPU forward.
#include "va_device.h"

#include <type_traits>

namespace va {

namespace {

using namespace dev;

template <typename T, int D, int MODE, bool ALIBI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k1_prefill16(
    AttnArgs a, const int4 *__restrict__ items, const int4 *__restrict__ seqinfo, const int32_t *__restrict__ count)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr int BN = kBN;
    constexpr int NCH = D / 8;         // 16-byte chunks per row
    constexpr int NSEG = NCH / 4;      // 64-byte segments per row
    constexpr int KS = D / 16;         // QK^T k-steps
    constexpr int MD = D / 32;         // 32-wide blocks of the head dimension
    constexpr int RPI = 64 / NCH;      // rows one 64-lane load instruction fills
    constexpr int LPW = BN / RPI / 4;  // load instructions per wave per tile
    constexpr int ROWB = D * 2;        // bytes per LDS row
    constexpr int TILEB = BN * ROWB;   // bytes per K or V tile
    // LDS: K ring [K0 | K1] then V ring [V0 | V1]; tile t lives in slot t & 1
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILEB];
    char *const sbase = (char *)smem;
    char *const kring = sbase;
    char *const vring = sbase + 2 * TILEB;

    // a.hpw == 1: the item's 128 query rows of one head (32 per wave).
    // a.hpw == 4: a quarter of the item (32 rows) for 4 heads that share a kv
    // head (one head per wave): the waves see the same keys, and the quarter
    // spans fewer diagonal tiles than the whole item.  Either way the item
    // has a.H workgroups; map_block gives each XCD a contiguous range of them.
    int item, slot;
    map_block(blockIdx.x, a.H, item, slot);
    // the item, its sequence's offsets and the item count in one round trip
    // (item < capacity always holds, so the first two reads stay in bounds)
    const int n_items = *count;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    asm volatile("" ::"s"(it.x), "s"(si.x), "s"(n_items));
    if (item >= n_items) return;
    const int b = it.x;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int delta = Lk - Lq;
    int i0 = it.y, kv_lo = it.z, kv_hi = it.w;
    if (a.hpw != 1) {
        // this quarter's rows and the union of their visible keys
        i0 += (slot & 3) * 32;
        if (i0 >= Lq) return;
        int l0, h0, l1, h1;
        row_bounds(i0, delta, Lk, a.left, a.right, l0, h0);
        row_bounds(min(i0 + 31, Lq - 1), delta, Lk, a.left, a.right, l1, h1);
        kv_lo = Lk > 0 ? l0 : 0;
        kv_hi = Lk > 0 ? max(h1 + 1, kv_lo) : 0;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;
    const int wrow = a.hpw == 1 ? wave * 32 : 0;                // the wave's first row
    const int head = a.hpw == 1 ? slot : (slot >> 2) * 4 + wave;
    const int c = head / a.g;                                   // the same for every wave
    const int row = i0 + wrow + n;
    const bool row_ok = row < Lq;
    int lo = 1, hi = 0;
    if (row_ok) row_bounds(row, delta, Lk, a.left, a.right, lo, hi);
    // ALiBi in raw-score units (the scores are scaled after the max):
    // - (slope / scale) * |row + delta - j|
    float alibi_r = 0.f;
    if constexpr (ALIBI) alibi_r = a.alibi[head] / a.scale;
    const int pos = row + delta;

    // keys this wave can see (wlo..whi) and keys all its rows see (flo..fhi)
    int wlo = 1, whi = 0, flo = 0x7fffffff, fhi = -1;
    {
        const int w0 = i0 + wrow, w1 = min(w0 + 31, Lq - 1);
        if (w0 < Lq) {
            int l0, h0, l1, h1;
            row_bounds(w0, delta, Lk, a.left, a.right, l0, h0);
            row_bounds(w1, delta, Lk, a.left, a.right, l1, h1);
            wlo = l0; whi = h1; flo = l1; fhi = h0;
        }
    }
    const int ntiles = (kv_hi - kv_lo + BN - 1) / BN;
    auto visible = [&](int t) {
        const int j0 = kv_lo + t * BN;
        return wlo <= whi && j0 <= whi && j0 + BN - 1 >= wlo;
    };

    // ---- tile loads, global -> LDS without staging registers.  One load
    // instruction fills RPI consecutive rows (64 lanes x 16 bytes, lane-linear
    // in LDS); each lane fetches the logical chunk that belongs at its
    // physical slot.  K rows: chunk XOR (row mod NCH), so the rows of one MFMA
    // operand read hit distinct chunks; V rows: 64-byte segment XOR (row mod
    // NSEG), so the rows of one transposing read hit distinct segments.
    const size_t rowstride = (size_t)a.Hkv * D * 2;
    const char *kseq = (const char *)a.k + ((size_t)k0 * a.Hkv + c) * D * 2;
    const char *vseq = (const char *)a.v + ((size_t)k0 * a.Hkv + c) * D * 2;
    // lane's row / chunk for load instruction u
    auto ld_row = [&](int u) { return (wave * LPW + u) * RPI + lane / NCH; };
    auto ld_chunk = [&](int u, bool is_v) {
        const int r = ld_row(u), p = lane % NCH;
        return is_v ? p ^ ((r % NSEG) << 2) : p ^ (r % NCH);
    };
    // copy instruction u (rows (wave LPW + u) RPI ..) of tile t to dst.  A
    // tile past the end (t >= ntiles) is harmless: buffer mode reads an
    // empty range (zeros), the other modes re-read the last row; the
    // destination slot is a free one either way.
    // buffer mode: raw buffer over rows j0 .. min(kv_hi, j0 + BN) - 1 of tile
    // t (reads past the end return 0; at most BN rows, so the 32-bit byte
    // count cannot wrap for long key ranges)
    auto tile_rsrc = [&](int t, bool is_v) -> u32x4 {
        const int j0 = kv_lo + t * BN;
        const char *seq = is_v ? vseq : kseq;
        const uint32_t nrec = j0 < kv_hi ? (uint32_t)(min(kv_hi - j0, BN) * rowstride) : 0u;
        const uint64_t addr = (uint64_t)(uintptr_t)(seq + j0 * rowstride);
        return u32x4{(uint32_t)addr, (uint32_t)(addr >> 32) & 0xffffu, nrec, 0x00020000u};
    };
    auto issue_u = [&](int t, bool is_v, char *dst, int u, const u32x4 &rsrc) {
        if constexpr (MODE == kLoadBuffer) {
            (void)t;
            const uint32_t off = (uint32_t)(ld_row(u) * rowstride) + ld_chunk(u, is_v) * 16;
            copy16_buffer(rsrc, off, lds_addr(dst + (wave * LPW + u) * 1024));
        } else {
            (void)rsrc;
            const int j0 = kv_lo + t * BN;
            const uint16_t *base = (const uint16_t *)(is_v ? a.v : a.k);
            const int j = min(j0 + ld_row(u), kv_hi - 1);
            const size_t off = kv_row_offset<D, MODE == kLoadPaged>(a, b, k0, c, j) + ld_chunk(u, is_v) * 8;
            copy16_global((const void *)(base + off), lds_addr(dst + (wave * LPW + u) * 1024));
        }
    };
    auto issue = [&](int t, bool is_v, char *dst) {
        const u32x4 rsrc = MODE == kLoadBuffer ? tile_rsrc(t, is_v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < LPW; ++u) issue_u(t, is_v, dst, u, rsrc);
    };

    // Q^T operand fragments: lane (row n, half h2) holds d = 16 ks + 8 h2 .. +8
    v8 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + (row_ok ? row : 0)) * a.H + head) * D + h2 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // unconditional load (rows past the end read row 0), then zeroed
            u32x4 x = *(const u32x4 *)(qp + ks * 16);
            if (!row_ok) x = u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(v8, x);
        }
    }

    f32x16 o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[md][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // LDS byte offsets of this lane's MFMA operand reads
    auto koff = [&](int ks) -> uint32_t { return n * ROWB + ((((ks * 2 + h2) ^ (n % NCH))) << 4); };
    auto voff = [&](int md) -> uint32_t {
        const int col = md * 32 + ((lane & 31) >> 4) * 16 + (l16 & 3) * 4;
        const int seg = (col >> 3) ^ ((q4 % NSEG) << 2);
        return (h2 * 4 + q4) * ROWB + (seg << 4) + (col & 7) * 2;
    };

    // ---- the three pieces of work per tile
    // S^T = K Q^T: lane value v of block mb is key j0 + 32 mb + 8 (v/4) + 4 h2 + v%4
    auto qk = [&](f32x16 (&S)[2], const char *kt, auto &&hook) {
#pragma unroll
        for (int v = 0; v < 16; ++v) { S[0][v] = 0.f; S[1][v] = 0.f; }
        // K operands read one step ahead of their products
        v8 kf0 = *(const v8 *)(kt + koff(0));
        v8 kf1 = *(const v8 *)(kt + koff(0) + 32 * ROWB);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            v8 n0 = kf0, n1 = kf1;
            if (ks + 1 < KS) {
                n0 = *(const v8 *)(kt + koff(ks + 1));
                n1 = *(const v8 *)(kt + koff(ks + 1) + 32 * ROWB);
            }
            S[0] = E::mfma(kf0, qf[ks], S[0]);
            S[1] = E::mfma(kf1, qf[ks], S[1]);
            hook(ks);
            kf0 = n0;
            kf1 = n1;
        }
    };
    // mask (edge tiles only) and row max, then move the running max if the
    // tile raises it by more than the slack (raw scores; scale > 0)
    auto row_max = [&](f32x16 (&S)[2], int t) {
        const int j0 = kv_lo + t * BN;
        if constexpr (ALIBI) {
            // lane value v of block mb is key j0 + 32 mb + 8 (v/4) + 4 h2 + v%4
            const float base = (float)(pos - j0 - 4 * h2);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    S[mb][v] = fmaf(-alibi_r, fabsf(base - (float)(32 * mb + 8 * (v >> 2) + (v & 3))), S[mb][v]);
        }
        float mx = -INFINITY;
        if (j0 >= flo && j0 + BN - 1 <= fhi) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[mb][v]);
        } else {
            // key j is visible iff (unsigned)(j - lo) <= (unsigned)(hi - lo).
            // Rows that see nothing (hi < lo) get span 0 and offsets >= 1,
            // which hides every key.  Selects, no branches.
            const bool none = hi < lo;
            const uint32_t span = none ? 0u : (uint32_t)(hi - lo);
            const int jb = none ? 1 : j0 + h2 * 4 - lo;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const uint32_t d = (uint32_t)(jb + mb * 32 + (v >> 2) * 8 + (v & 3));
                    const float x = d > span ? -INFINITY : S[mb][v];
                    S[mb][v] = x;
                    mx = fmaxf(mx, x);
                }
        }
        const float mx_c = halves_max(mx) * a.scale_log2;
        if (__ballot(mx_c > m_run + kRescaleSlack) != 0ull) {
            const float m_new = fmaxf(m_run, mx_c);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[md][v] *= alpha;
        }
    };
    // one probability in place (element idx of the tile's 32 per lane),
    // pinned where it is computed
    auto prob_elem = [&](f32x16 (&S)[2], int idx, float neg_m, float &rs) {
        float x = fast_exp2(fmaf(S[idx >> 4][idx & 15], a.scale_log2, neg_m));
        pin(x);
        S[idx >> 4][idx & 15] = x;
        rs += x;
    };
    // bf16 operand of PV step t4 from probabilities computed in place
    auto cvt_step = [&](f32x16 (&S)[2], int t4) -> v8 {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = S[t4 >> 1][(t4 & 1) * 8 + e];
        return __builtin_convertvector(pv, v8);
    };
    // probabilities of PV step t4 (keys 16 t4 .. +16) in bf16, laid out as
    // that step's P^T operand
    auto probs = [&](f32x16 (&S)[2], int t4, float neg_m, float &rs) -> v8 {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = fast_exp2(fmaf(S[t4 >> 1][(t4 & 1) * 8 + e], a.scale_log2, neg_m));
            pv[e] = x;
            rs += x;
        }
        return __builtin_convertvector(pv, v8);
    };
    // V^T operand of block md for PV step t4 (transposing LDS reads)
    auto vread = [&](int t4, int md, const char *vt) -> v8 {
        const v4 va = E::read_tr((const uint16_t *)(vt + voff(md) + t4 * 16 * ROWB));
        const v4 vb = E::read_tr((const uint16_t *)(vt + voff(md) + (t4 * 16 + 8) * ROWB));
        return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // O^T += V^T P^T for one step of 16 keys; V^T operands read two
    // products ahead
    auto pv = [&](const v8 &P, int t4, const char *vt) {
        v8 vb0 = vread(t4, 0, vt), vb1 = vread(t4, 1, vt);
#pragma unroll
        for (int md = 0; md < MD; ++md) {
            const v8 vf = (md & 1) ? vb1 : vb0;
            if (md + 2 < MD) {
                if (md & 1) vb1 = vread(t4, md + 2, vt);
                else vb0 = vread(t4, md + 2, vt);
            }
            o[md] = E::mfma(vf, P, o[md]);
        }
    };

    // ---- software pipeline: iteration t runs QK^T of tile t+1 next to the
    // softmax of tile t, then PV of tile t next to the row max of tile t+1.
    // Loads issued at the top of iteration t (into slots freed by the
    // previous barrier) land before its closing barrier.
    f32x16 sa[2], sb[2];
    if (ntiles > 0) {
        issue(0, false, kring);
        issue(0, true, vring);
        if (ntiles > 1) issue(1, false, kring + TILEB);
    }
    // the sink logit is read after the first tiles are in flight, so that
    // its wait does not hold them back
    if (a.sinks) {
        m_run = a.sinks[head] * kLog2e;
        l_run = h2 == 0 ? 1.f : 0.f;
    }
    wait_vmem();
    __syncthreads();
    bool vc = ntiles > 0 && visible(0);
    if (vc) {
        qk(sa, kring, [](int) {});
        row_max(sa, 0);
    }
    __syncthreads();  // K slot 0 is refilled by iteration 0

    auto iteration = [&](int t, auto BUFC, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
        constexpr int BUF = decltype(BUFC)::value;
        char *k_next = kring + (BUF ^ 1) * TILEB;         // K(t+1)
        char *v_cur = vring + BUF * TILEB;                // V(t)
        char *k_dst = kring + BUF * TILEB;                // K(t+2) goes where K(t) was
        char *v_dst = vring + (BUF ^ 1) * TILEB;          // V(t+1) goes where V(t-1) was
        const bool vn = t + 1 < ntiles && visible(t + 1);
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        // the copies for the coming tiles go out one at a time between the
        // MFMA groups of this iteration (unconditionally: see issue_u)
        constexpr int KEVERY = KS / LPW;
        const u32x4 rs_k = MODE == kLoadBuffer ? tile_rsrc(t + 2, false) : u32x4{0u, 0u, 0u, 0u};
        const u32x4 rs_v = MODE == kLoadBuffer ? tile_rsrc(t + 1, true) : u32x4{0u, 0u, 0u, 0u};
        // the probabilities of PV steps 0 and 1 (16 per lane) are computed
        // between the QK^T products of the next tile (independent work), two
        // per K step; with no current tile they are computed and dropped
        float rs = 0.f;
        constexpr int PER_KS = 16 / KS;
        static_assert(PER_KS * KS == 16, "16 probabilities over the K steps");
        // matrix phases at a raised wave priority (the co-resident wave's
        // vector-only phases yield the issue slot to them)
        __builtin_amdgcn_s_setprio(1);
        if (vn) {
            qk(Sn, k_next, [&](int ks) {
                if (ks % KEVERY == KEVERY - 1) issue_u(t + 2, false, k_dst, ks / KEVERY, rs_k);
#pragma unroll
                for (int e = 0; e < PER_KS; ++e) prob_elem(Sc, ks * PER_KS + e, neg_m, rs);
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            issue(t + 2, false, k_dst);
#pragma unroll
            for (int e = 0; e < 16; ++e) prob_elem(Sc, e, neg_m, rs);
        }
        if (vc) {
            constexpr int VEVERY = 4 / LPW;
            auto vhook = [&](int t4) {
                if (t4 % VEVERY == VEVERY - 1) issue_u(t + 1, true, v_dst, t4 / VEVERY, rs_v);
            };
            const v8 p0 = cvt_step(Sc, 0);
            const v8 p1 = cvt_step(Sc, 1);
            pv(p0, 0, v_cur);
            vhook(0);
            const v8 p2 = probs(Sc, 2, neg_m, rs);
            pv(p1, 1, v_cur);
            vhook(1);
            const v8 p3 = probs(Sc, 3, neg_m, rs);
            pv(p2, 2, v_cur);
            vhook(2);
            pv(p3, 3, v_cur);
            vhook(3);
            l_run += rs;
        } else {
            issue(t + 1, true, v_dst);
        }
        __builtin_amdgcn_s_setprio(0);
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

    // epilogue: lane (row n, half h2) holds O[row][32 md + 8 i + 4 h2 + j].
    // The O tile goes through LDS (the K/V slots are free after the last
    // barrier) so that global stores write whole rows with 16-byte lanes:
    // a workgroup's stores then complete sooner, and it holds its slot until
    // they have.
    const float l_tot = halves_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char *ow = sbase + wave * 32 * ROWB;  // this wave's 32 rows, 16-byte chunk XOR (row mod NCH)
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = o[md][i * 4 + j] * inv;
            const v4 y = __builtin_convertvector(x, v4);
            const int phys = (md * 4 + i) ^ (n % NCH);
            *(u32x2 *)(ow + n * ROWB + phys * 16 + h2 * 8) = __builtin_bit_cast(u32x2, y);
        }
    if (row_ok && h2 == 0 && a.lse)
        a.lse[(size_t)(q0 + row) * a.H + head] =
            l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    __syncthreads();
    {
        constexpr int RPW = 64 / NCH;  // rows one 64-lane pass covers
        const int cidx = lane % NCH;
#pragma unroll
        for (int u = 0; u < 32 / RPW; ++u) {
            const int r = u * RPW + lane / NCH;
            const int orow = i0 + wrow + r;
            const u32x4 v = *(const u32x4 *)(ow + r * ROWB + ((cidx ^ (r % NCH)) << 4));
            if (orow < Lq)
                *(u32x4 *)((uint16_t *)a.out + ((size_t)(q0 + orow) * a.H + head) * D + cidx * 8) = v;
        }
    }
}

}  // namespace

hipError_t launch_prefill16(const AttnArgs &a, bool f16, bool alibi, int head_dim, int mode, const int4 *items,
                            const int4 *seqinfo, const int32_t *count, int grid, hipStream_t s)
{
    const dim3 g(grid), blk(256);
#define VA_LAUNCH(TT, DD, MM, AA) \
    hipLaunchKernelGGL((k1_prefill16<TT, DD, MM, AA>), g, blk, 0, s, a, items, seqinfo, count)
#define VA_MODES(TT, DD, AA)                                          \
    do {                                                              \
        if (mode == kLoadBuffer) VA_LAUNCH(TT, DD, kLoadBuffer, AA);  \
        else if (mode == kLoadGlobal) VA_LAUNCH(TT, DD, kLoadGlobal, AA); \
        else VA_LAUNCH(TT, DD, kLoadPaged, AA);                       \
    } while (0)
#define VA_DIMS(TT, AA)                          \
    do {                                         \
        if (head_dim == 128) VA_MODES(TT, 128, AA); \
        else VA_MODES(TT, 64, AA);               \
    } while (0)
    if (f16) {
        if (alibi) VA_DIMS(_Float16, true);
        else VA_DIMS(_Float16, false);
    } else {
        if (alibi) VA_DIMS(__bf16, true);
        else VA_DIMS(__bf16, false);
    }
#undef VA_DIMS
#undef VA_MODES
#undef VA_LAUNCH
    return hipGetLastError();
}

}  // namespace va
