// Split-KV decode for short queries (g * Lq <= 16) against long, possibly
// paged, key/value sequences, plus the combine step.
//
// Partial kernel: one workgroup per (split, kv head).  All g heads of the
// GQA group and all Lq query rows of the sequence are packed into the 16
// rows of one MFMA 16x16x32 tile, so every K/V byte of the split is read
// from HBM exactly once.  The 4 waves take interleaved 64-key chunks of the
// split; per chunk a wave
//   loads K straight into MFMA operand registers (row-major K rows are the
//   A-operand layout), stages V in its own LDS slice,
//   S^T = K Q^T (4 x 4 MFMA), mask, online softmax in fp32 (exp2 domain),
//   O^T += V^T P^T (8 x 2 MFMA) with V^T read by ds_read_b64_tr_b16.
// The 4 wave states merge through LDS and the split writes an unnormalised
// fp32 partial O with its running (max, sum).
//
// Combine kernel: per (sequence, kv head) merges the splits' partials
// LSE-weighted and adds the sink term exactly once:
//   M = max(m_s, sigma), L = sum_s l_s 2^(m_s-M) + 2^(sigma-M),
//   O = sum_s O_s 2^(m_s-M) / L,  LSE = (M + log2 L) ln 2.
// This is the same softmax(Q K^T * scale) V (SparseAttnSharedkv README,
// formula section) regrouped over key splits; the returned LSE is what makes
// the regrouping exact (pull request "[varlen_attn for inference] add out
// variant": the op returns softmax_logsumexp).
#include "va_internal.h"

#include <type_traits>

namespace va {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

// The 16-bit input type's 16x16x32 matrix instruction and transposing LDS
// read (bf16 and fp16 share the data layout and the fp32 accumulation).
template <typename T>
struct Elt;
template <>
struct Elt<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static __device__ __forceinline__ v4 read_tr(const uint16_t *p)
    {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)((__attribute__((address_space(3))) uint16_t *)(p)));
    }
    static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elt<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    static __device__ __forceinline__ v4 read_tr(const uint16_t *p)
    {
        return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                          (lds_fp16x4 *)((__attribute__((address_space(3))) uint16_t *)(p))));
    }
    static __device__ __forceinline__ f32x4 mfma(v8 a, v8 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k2_decode16(AttnArgs a, const int4 *__restrict__ items,
                                                      const int4 *__restrict__ seqinfo,
                                                      const int32_t *__restrict__ count,
                                                      float *__restrict__ part_o,
                                                      float2 *__restrict__ part_ml)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr int CH = kDecChunk;        // keys per wave step
    constexpr int NCH = D / 8;           // 16-byte chunks per row
    constexpr int KS = D / 32;           // QK^T k-steps
    constexpr int MD = D / 16;           // 16-wide blocks of the head dimension
    constexpr int NKB = CH / 16;         // 16-key blocks per chunk
    constexpr int RPP = 64 / NCH;        // rows per V loader pass
    constexpr int VL = CH / RPP;         // V loader passes
    constexpr int ROWS = kDecRows;
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * CH * D];
    __shared__ int s_tbl[kDecTableMax];

    int item, c;
    map_block(blockIdx.x, a.Hkv, item, c);
    const int n_items = *count;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    asm volatile("" ::"s"(it.x), "s"(si.x), "s"(n_items));
    if (item >= n_items) return;
    const int b = it.x, slot = it.y, kv_lo = it.z, kv_hi = it.w;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int delta = Lk - Lq;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 15, kq = lane >> 4, l16 = lane & 15;
    const int rows = min(a.g * Lq, ROWS);
    const bool row_ok = n < rows;
    const int qi = n / a.g, head = c * a.g + n % a.g;
    int lo = 1, hi = 0;
    if (row_ok) row_bounds(qi, delta, Lk, a.left, a.right, lo, hi);
    // ALiBi: - slope * |qi + delta - j| in log2 units (0 without slopes,
    // which leaves every score unchanged)
    const float sl2 = (a.alibi && row_ok) ? a.alibi[head] * kLog2e : 0.f;
    const int pos = qi + delta;
    // keys every packed row sees: rows are ordered by query index
    int flo = 0x7fffffff, fhi = -1;
    if (rows > 0) {
        int l0, h0, l1, h1;
        row_bounds(0, delta, Lk, a.left, a.right, l0, h0);
        row_bounds((rows - 1) / a.g, delta, Lk, a.left, a.right, l1, h1);
        flo = l1; fhi = h0;
    }

    v8 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + (row_ok ? qi : 0)) * a.H + (row_ok ? head : 0)) * D + kq * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4 *)(qp + ks * 32);
            if (!row_ok) x = u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(v8, x);
        }
    }
    f32x4 o[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const uint16_t *kbase = (const uint16_t *)a.k;
    const uint16_t *vbase = (const uint16_t *)a.v;
    uint16_t *sv = smem + wave * CH * D;
    // Paged: the block ids of this split's keys are staged in LDS once, so
    // a row's address needs no dependent global load (a wait for one would
    // also drain every data load issued before it).
    int blk0 = 0;
    bool tbl = false;
    if constexpr (PAGED) {
        if (a.bs_shift >= 0 && kv_hi > kv_lo) {
            blk0 = kv_lo >> a.bs_shift;
            const int nblk = ((kv_hi - 1) >> a.bs_shift) - blk0 + 1;
            tbl = nblk <= kDecTableMax;
            if (tbl)
                for (int i = tid; i < nblk; i += 256) s_tbl[i] = a.block_table[(size_t)b * a.bt_stride + blk0 + i];
        }
        __syncthreads();
    }
    // Address modes of the chunk loop (chosen once per split):
    //  0  every 64-key chunk lies in one block (contiguous K/V, or paged with
    //     power-of-two blocks >= 64 keys and a chunk-aligned split): one
    //     buffer descriptor per chunk, per-lane offsets fixed, rows past
    //     kv_hi read as zeros (outside the descriptor's range)
    //  1  paged, power-of-two blocks: per-row block ids from the LDS table
    //  2  anything else: per-row block-table lookups
    const size_t rowstride = (size_t)a.Hkv * D * 2;  // bytes between key rows
    auto chunk_loop = [&](auto AMC) {
    constexpr int AM = decltype(AMC)::value;
    // element offset of key row j (modes 1, 2; clamped into the split: rows
    // past kv_hi are masked, so re-reading the last row is harmless)
    auto row_off = [&](int j) -> size_t {
        j = min(j, kv_hi - 1);
        if constexpr (AM == 1) {
            const int blk = s_tbl[(j >> a.bs_shift) - blk0];
            return ((((size_t)blk << a.bs_shift) + (j & (a.block_size - 1))) * a.Hkv + c) * D;
        } else {
            return kv_row_offset<D, PAGED>(a, b, k0, c, j);
        }
    };
    // mode 0 per-lane byte offsets (all in the range-checked vector offset):
    // K operand rows n (+16 kb), d = 8 kq (+32 ks); V rows lane / NCH
    // (+RPP u), chunk lane % NCH
    const uint32_t koff0 = n * (uint32_t)rowstride + kq * 16;
    const uint32_t voff0 = (lane / NCH) * (uint32_t)rowstride + (lane % NCH) * 16;

    for (int j0 = kv_lo + wave * CH; j0 < kv_hi; j0 += 4 * CH) {
        v8 kf[NKB][KS];
        u32x4 vr[VL];
        const int cc = lane % NCH;
        if constexpr (AM == 0) {
            size_t row0;  // first row of the chunk in the K/V arrays
            if constexpr (PAGED) {
                const int blk = __builtin_amdgcn_readfirstlane(s_tbl[(j0 >> a.bs_shift) - blk0]);
                row0 = ((size_t)blk << a.bs_shift) + (j0 & (a.block_size - 1));
            } else {
                row0 = (size_t)(k0 + j0);
            }
            const size_t base = (row0 * a.Hkv + c) * D * 2;
            const uint32_t nrec = (uint32_t)(min(kv_hi - j0, CH) * rowstride);
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const char *)a.k + base), (short)0, nrec, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const char *)a.v + base), (short)0, nrec, 0x00020000);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[kb][ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(
                        rk, koff0 + (uint32_t)(kb * 16 * rowstride) + ks * 64, 0, 0));
#pragma unroll
            for (int u = 0; u < VL; ++u)
                vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff0 + (uint32_t)(u * RPP * rowstride), 0, 0);
        } else {
            // K rows j0 + 16 kb + n as A operands (d = 32 ks + 8 kq .. +8)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const uint16_t *kp = kbase + row_off(j0 + kb * 16 + n) + kq * 8;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = __builtin_bit_cast(v8, *(const u32x4 *)(kp + ks * 32));
            }
            // V rows of the chunk, 16-byte chunk `cc` of row r
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int r = u * RPP + lane / NCH;
                vr[u] = *(const u32x4 *)(vbase + row_off(j0 + r) + cc * 8);
            }
        }
        // keep every load of the chunk ahead of the math that consumes them
        __builtin_amdgcn_sched_barrier(0);
        f32x4 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[kb] = E::mfma(kf[kb][ks], qf[ks], s[kb]);
        }
        // stage V: chunk index XOR 2 (row mod NCH/2) spreads the 16 rows of
        // one transposing read over all banks
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int r = u * RPP + lane / NCH;
            *(u32x4 *)(sv + r * D + ((cc ^ ((r % (NCH / 2)) << 1)) << 3)) = vr[u];
        }
        // lane value v of block kb is key j0 + 16 kb + 4 kq + v of row n
        float mx = -INFINITY;
        if (j0 >= flo && j0 + CH - 1 <= fhi && row_ok) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = j0 + kb * 16 + kq * 4 + v;
                    s[kb][v] = fmaf(-sl2, fabsf((float)(pos - j)), s[kb][v] * a.scale_log2);
                    mx = fmaxf(mx, s[kb][v]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = j0 + kb * 16 + kq * 4 + v;
                    const float x = (j >= lo && j <= hi) ? fmaf(-sl2, fabsf((float)(pos - j)), s[kb][v] * a.scale_log2)
                                                         : -INFINITY;
                    s[kb][v] = x;
                    mx = fmaxf(mx, x);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float p = __builtin_amdgcn_exp2f(s[kb][v] - m_use);
                s[kb][v] = p;
                rs += p;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md] *= alpha;

        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < CH / 32; ++t) {
            f32x8 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = s[2 * t][e];
                pv[4 + e] = s[2 * t + 1][e];
            }
            const v8 pf = __builtin_convertvector(pv, v8);
            const int rA = 32 * t + kq * 4 + (l16 >> 2);
            const int rB = rA + 16;
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const int col = md * 16 + (l16 & 3) * 4;
                const int chA = (col >> 3) ^ ((rA % (NCH / 2)) << 1);
                const int chB = (col >> 3) ^ ((rB % (NCH / 2)) << 1);
                const v4 va = E::read_tr(sv + rA * D + (chA << 3) + (col & 7));
                const v4 vb = E::read_tr(sv + rB * D + (chB << 3) + (col & 7));
                const v8 vf = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                o[md] = E::mfma(vf, pf, o[md]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    };
    const bool aligned_blocks = PAGED && tbl && a.bs_shift >= 6 && (kv_lo & (CH - 1)) == 0;
    if (!PAGED || aligned_blocks) chunk_loop(std::integral_constant<int, 0>{});
    else if (tbl) chunk_loop(std::integral_constant<int, 1>{});
    else chunk_loop(std::integral_constant<int, 2>{});

    // merge the 4 wave states (LDS reused)
    float l_w = l_run + __shfl_xor(l_run, 16);
    l_w += __shfl_xor(l_w, 32);
    __syncthreads();
    float *so = (float *)smem;                         // [4][ROWS][D]
    float2 *sml = (float2 *)(so + 4 * ROWS * D);       // [4][ROWS]
#pragma unroll
    for (int md = 0; md < MD; ++md)
        *(f32x4 *)(so + (wave * ROWS + n) * D + md * 16 + kq * 4) = o[md];
    if (kq == 0) sml[wave * ROWS + n] = make_float2(m_run, l_w);
    __syncthreads();
    {
        constexpr int DPT = D / 16;  // head-dim values per thread
        const int r = tid >> 4, d0 = (tid & 15) * DPT;
        float mw[4], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = sml[w * ROWS + r].x;
            M = fmaxf(M, mw[w]);
        }
        const float M_use = M == -INFINITY ? 0.f : M;
        float L = 0.f, acc[DPT];
#pragma unroll
        for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sc = __builtin_amdgcn_exp2f(mw[w] - M_use);
            L += sml[w * ROWS + r].y * sc;
#pragma unroll
            for (int i = 0; i < DPT; ++i) acc[i] += so[(w * ROWS + r) * D + d0 + i] * sc;
        }
        const size_t base = ((size_t)slot * a.Hkv + c) * ROWS + r;
        float *po = part_o + base * D + d0;
#pragma unroll
        for (int i = 0; i < DPT; i += 4)
            *(float4 *)(po + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
        if ((tid & 15) == 0) part_ml[base] = make_float2(M, L);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k3_combine(AttnArgs a, const int32_t *__restrict__ seq_off,
                                                  const float *__restrict__ part_o,
                                                  const float2 *__restrict__ part_ml)
{
    constexpr int ROWS = kDecRows, DPT = D / 16;
    const int b = blockIdx.x / a.Hkv, c = blockIdx.x % a.Hkv;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int rows = min(a.g * Lq, ROWS);
    const int r = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * DPT;
    if (r >= rows) return;
    const int qi = r / a.g, head = c * a.g + r % a.g;
    const int s0 = seq_off[b], ns = seq_off[b + 1] - s0;

    float M = a.sinks ? a.sinks[head] * kLog2e : -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[((size_t)(s0 + s) * a.Hkv + c) * ROWS + r].x);
    const float M_use = M == -INFINITY ? 0.f : M;
    float L = a.sinks ? __builtin_amdgcn_exp2f(a.sinks[head] * kLog2e - M_use) : 0.f;
    float acc[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
    for (int s = 0; s < ns; ++s) {
        const size_t base = ((size_t)(s0 + s) * a.Hkv + c) * ROWS + r;
        const float2 ml = part_ml[base];
        const float w = __builtin_amdgcn_exp2f(ml.x - M_use);
        L += ml.y * w;
        const float *po = part_o + base * D + d0;
#pragma unroll
        for (int i = 0; i < DPT; i += 4) {
            const float4 x = *(const float4 *)(po + i);
            acc[i] += w * x.x; acc[i + 1] += w * x.y; acc[i + 2] += w * x.z; acc[i + 3] += w * x.w;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + qi) * a.H + head) * D + d0;
#pragma unroll
    for (int i = 0; i < DPT; i += 4) {
        const f32x4 x = {acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
        const auto y = __builtin_convertvector(x, typename Elt<T>::v4);
        *(u32x2 *)(op + i) = __builtin_bit_cast(u32x2, y);
    }
    if ((threadIdx.x & 15) == 0 && a.lse)
        a.lse[(size_t)(q0 + qi) * a.H + head] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode16(const AttnArgs &a, bool f16, int head_dim, bool paged, const int4 *items,
                           const int4 *seqinfo, const int32_t *count, int grid, float *part_o,
                           float2 *part_ml, hipStream_t s)
{
    const dim3 g(grid), blk(256);
#define VA_LAUNCH(TT, DD, PP) \
    hipLaunchKernelGGL((k2_decode16<TT, DD, PP>), g, blk, 0, s, a, items, seqinfo, count, part_o, part_ml)
    if (f16) {
        if (head_dim == 128) { if (paged) VA_LAUNCH(_Float16, 128, true); else VA_LAUNCH(_Float16, 128, false); }
        else { if (paged) VA_LAUNCH(_Float16, 64, true); else VA_LAUNCH(_Float16, 64, false); }
    } else {
        if (head_dim == 128) { if (paged) VA_LAUNCH(__bf16, 128, true); else VA_LAUNCH(__bf16, 128, false); }
        else { if (paged) VA_LAUNCH(__bf16, 64, true); else VA_LAUNCH(__bf16, 64, false); }
    }
#undef VA_LAUNCH
    return hipGetLastError();
}

hipError_t launch_decode_combine(const AttnArgs &a, bool f16, int head_dim, const int32_t *seq_off,
                                 const float *part_o, const float2 *part_ml, hipStream_t s)
{
    const dim3 g(a.B * a.Hkv), blk(256);
    if (f16) {
        if (head_dim == 128) hipLaunchKernelGGL((k3_combine<_Float16, 128>), g, blk, 0, s, a, seq_off, part_o, part_ml);
        else hipLaunchKernelGGL((k3_combine<_Float16, 64>), g, blk, 0, s, a, seq_off, part_o, part_ml);
    } else {
        if (head_dim == 128) hipLaunchKernelGGL((k3_combine<__bf16, 128>), g, blk, 0, s, a, seq_off, part_o, part_ml);
        else hipLaunchKernelGGL((k3_combine<__bf16, 64>), g, blk, 0, s, a, seq_off, part_o, part_ml);
    }
    return hipGetLastError();
}

}  // namespace va
