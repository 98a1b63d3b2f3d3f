// bf16 prefill forward on gfx950 matrix cores.
//
// One workgroup = 4 waves = 128 query rows of one head (32 rows per wave);
// key/value tiles of 64 rows are staged in LDS (double buffered, one barrier
// per tile) and shared by the 4 waves.  Per wave and tile:
//   S^T = K * Q^T      8 (D=128) x 2 MFMA 32x32x16 bf16, fp32 accumulate.
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
#include "va_internal.h"

#include <type_traits>

namespace va {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)((__attribute__((address_space(3))) uint16_t *)(p)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Values of lanes l and l^32 combined (v_permlane32_swap exchanges the two
// 32-lane halves, no LDS round trip).
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

// A row's running max is only moved when a tile raises it by more than this
// (log2 units): until then probabilities exp2(s - m) stay below 2^8, far
// inside fp32 / bf16 range, and the O / l rescale is skipped.
constexpr float kRescaleSlack = 8.f;

template <int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k1_prefill_bf16(
    AttnArgs a, const int4 *__restrict__ items, const int32_t *__restrict__ count)
{
    constexpr int BN = kBN;
    constexpr int NCH = D / 8;         // 16-byte chunks per row
    constexpr int NSEG = NCH / 4;      // 64-byte segments per row
    constexpr int KS = D / 16;         // QK^T k-steps
    constexpr int MD = D / 32;         // 32-wide blocks of the head dimension
    constexpr int RSTEP = 256 / NCH;   // rows covered by one loader pass
    constexpr int LPT = BN / RSTEP;    // loader passes per tile
    constexpr int ROWB = D * 2;        // bytes per LDS row
    constexpr int TILEB = BN * ROWB;   // bytes per K or V tile
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILEB];  // K0 V0 K1 V1
    char *const sbase = (char *)smem;

    int item, head;
    map_block(blockIdx.x, a.H, item, head);
    if (item >= *count) return;
    const int4 it = items[item];
    const int b = it.x, i0 = it.y, kv_lo = it.z, kv_hi = it.w;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int Lk = MODE == kLoadPaged ? a.seqused_k[b] : a.cu_k[b + 1] - a.cu_k[b];
    const int k0 = MODE == kLoadPaged ? 0 : a.cu_k[b];
    const int delta = Lk - Lq;
    const int c = head / a.g;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;
    const int row = i0 + wave * 32 + n;
    const bool row_ok = row < Lq;
    int lo = 1, hi = 0;
    if (row_ok) row_bounds(row, delta, Lk, a.left, a.right, lo, hi);

    // keys this wave can see (wlo..whi) and keys all its rows see (flo..fhi)
    int wlo = 1, whi = 0, flo = 0x7fffffff, fhi = -1;
    {
        const int w0 = i0 + wave * 32, w1 = min(w0 + 31, Lq - 1);
        if (w0 < Lq) {
            int l0, h0, l1, h1;
            row_bounds(w0, delta, Lk, a.left, a.right, l0, h0);
            row_bounds(w1, delta, Lk, a.left, a.right, l1, h1);
            wlo = l0; whi = h1; flo = l1; fhi = h0;
        }
    }

    // Q^T operand fragments: lane (row n, half h2) holds d = 16 ks + 8 h2 .. +8
    bf16x8 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + (row_ok ? row : 0)) * a.H + head) * D + h2 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = row_ok ? *(const u32x4 *)(qp + ks * 16) : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[md][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    if (a.sinks) {
        m_run = a.sinks[head] * kLog2e;
        l_run = h2 == 0 ? 1.f : 0.f;
    }

    // LDS byte offsets, fixed per lane.  K rows: chunk index XOR (row mod NCH),
    // so the 16 rows one MFMA operand read touches hit 16 different chunks.
    // V rows: 64-byte segment XOR (row mod NSEG), so the 8 rows of one
    // transposing read spread over all segments.
    uint32_t koff[KS], voff[MD];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = n * ROWB + ((((ks * 2 + h2) ^ (n % NCH))) << 4);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
        const int col = md * 32 + ((lane & 31) >> 4) * 16 + (l16 & 3) * 4;
        const int seg = (col >> 3) ^ ((q4 % NSEG) << 2);
        voff[md] = (h2 * 4 + q4) * ROWB + (seg << 4) + (col & 7) * 2;
    }
    const int cc = tid % NCH, r_first = tid / NCH;
    const uint32_t st_k = r_first * ROWB + ((cc ^ (r_first % NCH)) << 4);
    const uint32_t st_v = r_first * ROWB + ((cc ^ ((r_first % NSEG) << 2)) << 4);

    // global -> register loader for one tile.  Rows at or past kv_hi are
    // never used unmasked: the buffer path reads them as zeros (out of the
    // descriptor's range), the other paths re-read the last valid row.
    const size_t rowstride = (size_t)a.Hkv * D * 2;
    const char *kseq = (const char *)a.k + ((size_t)k0 * a.Hkv + c) * D * 2;
    const char *vseq = (const char *)a.v + ((size_t)k0 * a.Hkv + c) * D * 2;
    u32x4 kr[LPT], vr[LPT];
    auto gload = [&](int t) {
        const int j0 = kv_lo + t * BN;
        if constexpr (MODE == kLoadBuffer) {
            const uint32_t nrec = (uint32_t)((kv_hi - j0) * rowstride);
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void *)(kseq + j0 * rowstride), (short)0, nrec, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void *)(vseq + j0 * rowstride), (short)0, nrec, 0x00020000);
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const uint32_t off = (uint32_t)((r_first + u * RSTEP) * rowstride) + cc * 16;
                kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
                vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const int j = min(j0 + r_first + u * RSTEP, kv_hi - 1);
                const size_t off = kv_row_offset<D, MODE == kLoadPaged>(a, b, k0, c, j) + cc * 8;
                kr[u] = *(const u32x4 *)((const uint16_t *)a.k + off);
                vr[u] = *(const u32x4 *)((const uint16_t *)a.v + off);
            }
        }
    };
    auto sstore = [&](auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        char *sk = sbase + BUF * 2 * TILEB;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            *(u32x4 *)(sk + st_k + u * RSTEP * ROWB) = kr[u];
            *(u32x4 *)(sk + TILEB + st_v + u * RSTEP * ROWB) = vr[u];
        }
    };

    auto compute = [&](int j0, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const char *kt = sbase + BUF * 2 * TILEB;
        const char *vt = kt + TILEB;
        // S^T = K Q^T, two independent 32-key accumulator chains
        f32x16 s[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) { s[0][v] = 0.f; s[1][v] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf0 = *(const bf16x8 *)(kt + koff[ks]);
            const bf16x8 kf1 = *(const bf16x8 *)(kt + koff[ks] + 32 * ROWB);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[ks], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[ks], s[1], 0, 0, 0);
        }
        // lane value v of block mb is key j0 + 32 mb + 8 (v/4) + 4 h2 + v%4;
        // raw scores here, the scale enters through one FMA before exp2
        float mx = -INFINITY;
        if (j0 >= flo && j0 + BN - 1 <= fhi) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mb][v]);
        } else {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = j0 + mb * 32 + (v >> 2) * 8 + h2 * 4 + (v & 3);
                    if (j < lo || j > hi) s[mb][v] = -INFINITY;
                    mx = fmaxf(mx, s[mb][v]);
                }
        }
        const float mx_c = halves_max(mx) * a.scale_log2;  // scale > 0
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
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        float rs = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(fmaf(s[mb][v], a.scale_log2, neg_m));
                s[mb][v] = p;
                rs += p;
            }
        l_run += rs;

        // O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int mb = t4 >> 1, ib = (t4 & 1) * 2;
            f32x8 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = s[mb][ib * 4 + e];
            const bf16x8 pf = __builtin_convertvector(pv, bf16x8);
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const bf16x4 va = lds_read_tr((const uint16_t *)(vt + voff[md] + t4 * 16 * ROWB));
                const bf16x4 vb = lds_read_tr((const uint16_t *)(vt + voff[md] + (t4 * 16 + 8) * ROWB));
                const bf16x8 vf = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[md], 0, 0, 0);
            }
        }
    };

    const int ntiles = (kv_hi - kv_lo + BN - 1) / BN;
    auto step = [&](int t, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const int j0 = kv_lo + t * BN;
        if (j0 <= whi && j0 + BN - 1 >= wlo) compute(j0, BUFC);
        if (t + 1 < ntiles) sstore(std::integral_constant<int, BUF ^ 1>{});
        if (t + 2 < ntiles) gload(t + 2);
        __syncthreads();
    };
    if (ntiles > 0) {
        gload(0);
        sstore(std::integral_constant<int, 0>{});
        if (ntiles > 1) gload(1);
    }
    __syncthreads();
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntiles) step(t, std::integral_constant<int, 0>{});

    // epilogue: lane (row n, half h2) holds O[row][32 md + 8 i + 4 h2 + j]
    const float l_tot = halves_sum(l_run);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + row) * a.H + head) * D + h2 * 4;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 x;
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = o[md][i * 4 + j] * inv;
                const bf16x4 y = __builtin_convertvector(x, bf16x4);
                *(u32x2 *)(op + md * 32 + i * 8) = __builtin_bit_cast(u32x2, y);
            }
        if (h2 == 0 && a.lse)
            a.lse[(size_t)(q0 + row) * a.H + head] =
                l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs &a, int head_dim, int mode, const int4 *items,
                               const int32_t *count, int grid, hipStream_t s)
{
    const dim3 g(grid), blk(256);
#define VA_LAUNCH(DD, MM) hipLaunchKernelGGL((k1_prefill_bf16<DD, MM>), g, blk, 0, s, a, items, count)
    if (head_dim == 128) {
        if (mode == kLoadBuffer) VA_LAUNCH(128, kLoadBuffer);
        else if (mode == kLoadGlobal) VA_LAUNCH(128, kLoadGlobal);
        else VA_LAUNCH(128, kLoadPaged);
    } else {
        if (mode == kLoadBuffer) VA_LAUNCH(64, kLoadBuffer);
        else if (mode == kLoadGlobal) VA_LAUNCH(64, kLoadGlobal);
        else VA_LAUNCH(64, kLoadPaged);
    }
#undef VA_LAUNCH
    return hipGetLastError();
}

}  // namespace va
