// float32 forward (no down-conversion anywhere): 64 query rows of one head
// per workgroup, four lanes per row, each lane owning a quarter of the head
// dimension as float4 chunks; 32-row K/V tiles staged in LDS.  Per tile the
// 32 scores of a row are formed (quarter dot products summed over the four
// lanes), then one online-softmax rescale and the P V accumulation, all in
// fp32 with the exp2 / log2 hardware instructions.
//
// Method: online-softmax form of softmax(Q K^T * scale) V (SparseAttnSharedkv
// README, formula section), LSE = max + ln(sum) (boostr CPU forward).
#include "va_internal.h"

namespace va {

namespace {

template <int D, bool PAGED>
__global__ __launch_bounds__(256) void k1_prefill_f32(AttnArgs a, const int4 *__restrict__ items,
                                                      const int4 *__restrict__ seqinfo,
                                                      const int32_t *__restrict__ count)
{
    constexpr int BN = kBNf32;
    constexpr int NC4 = D / 16;  // float4 chunks per lane
    __shared__ float4 sk[BN][D / 4];
    __shared__ float4 sv[BN][D / 4];

    int item, head;
    map_block(blockIdx.x, a.H, item, head);
    const int n_items = *count;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    asm volatile("" ::"s"(it.x), "s"(si.x), "s"(n_items));
    if (item >= n_items) return;
    const int b = it.x, i0 = it.y, kv_lo = it.z, kv_hi = it.w;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int c = head / a.g;

    const int tid = threadIdx.x, part = tid & 3;
    const int row = i0 + (tid >> 2);
    const bool row_ok = row < Lq;
    int lo = 1, hi = 0;
    if (row_ok) row_bounds(row, Lk - Lq, Lk, a.left, a.right, lo, hi);
    // ALiBi: - slope * |row + Lk - Lq - j| in log2 units (0 without slopes,
    // which leaves every score unchanged)
    const float sl2 = a.alibi ? a.alibi[head] * kLog2e : 0.f;
    const int pos = row + Lk - Lq;

    // lane `part` owns float4 chunks part, part+4, part+8, ...
    float4 qv[NC4], ov[NC4];
    const float *qp = (const float *)a.q + ((size_t)(q0 + (row_ok ? row : 0)) * a.H + head) * D;
#pragma unroll
    for (int i = 0; i < NC4; ++i) {
        qv[i] = row_ok ? *(const float4 *)(qp + (part + 4 * i) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        ov[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float m_run = -INFINITY, l_run = 0.f;
    if (a.sinks) {
        m_run = a.sinks[head] * kLog2e;
        l_run = 1.f;
    }

    const float *kbase = (const float *)a.k, *vbase = (const float *)a.v;
    for (int j0 = kv_lo; j0 < kv_hi; j0 += BN) {
        __syncthreads();
        for (int e = tid; e < BN * (D / 4); e += 256) {
            const int r = e / (D / 4), ch = e % (D / 4);
            const int j = j0 + r;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (j < kv_hi) {
                const size_t off = kv_row_offset<D, PAGED>(a, b, k0, c, j);
                kx = *(const float4 *)(kbase + off + ch * 4);
                vx = *(const float4 *)(vbase + off + ch * 4);
            }
            sk[r][ch] = kx;
            sv[r][ch] = vx;
        }
        __syncthreads();

        float sc[BN];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < BN; ++jj) {
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < NC4; ++i) {
                const float4 kx = sk[jj][part + 4 * i];
                d = fmaf(qv[i].x, kx.x, d);
                d = fmaf(qv[i].y, kx.y, d);
                d = fmaf(qv[i].z, kx.z, d);
                d = fmaf(qv[i].w, kx.w, d);
            }
            d += __shfl_xor(d, 1);
            d += __shfl_xor(d, 2);
            const int j = j0 + jj;
            const float x = (j >= lo && j <= hi) ? fmaf(-sl2, fabsf((float)(pos - j)), d * a.scale_log2) : -INFINITY;
            sc[jj] = x;
            mx = fmaxf(mx, x);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NC4; ++i) {
            ov[i].x *= alpha; ov[i].y *= alpha; ov[i].z *= alpha; ov[i].w *= alpha;
        }
#pragma unroll
        for (int jj = 0; jj < BN; ++jj) {
            const float p = __builtin_amdgcn_exp2f(sc[jj] - m_use);
            l_run += p;
#pragma unroll
            for (int i = 0; i < NC4; ++i) {
                const float4 vx = sv[jj][part + 4 * i];
                ov[i].x = fmaf(p, vx.x, ov[i].x);
                ov[i].y = fmaf(p, vx.y, ov[i].y);
                ov[i].z = fmaf(p, vx.z, ov[i].z);
                ov[i].w = fmaf(p, vx.w, ov[i].w);
            }
        }
        m_run = m_new;
    }

    if (row_ok) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *op = (float *)a.out + ((size_t)(q0 + row) * a.H + head) * D;
#pragma unroll
        for (int i = 0; i < NC4; ++i)
            *(float4 *)(op + (part + 4 * i) * 4) =
                make_float4(ov[i].x * inv, ov[i].y * inv, ov[i].z * inv, ov[i].w * inv);
        if (part == 0 && a.lse)
            a.lse[(size_t)(q0 + row) * a.H + head] =
                l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const AttnArgs &a, int head_dim, bool paged, const int4 *items,
                              const int4 *seqinfo, const int32_t *count, int grid, hipStream_t s)
{
    const dim3 g(grid), blk(256);
    if (head_dim == 128) {
        if (paged) hipLaunchKernelGGL((k1_prefill_f32<128, true>), g, blk, 0, s, a, items, seqinfo, count);
        else hipLaunchKernelGGL((k1_prefill_f32<128, false>), g, blk, 0, s, a, items, seqinfo, count);
    } else {
        if (paged) hipLaunchKernelGGL((k1_prefill_f32<64, true>), g, blk, 0, s, a, items, seqinfo, count);
        else hipLaunchKernelGGL((k1_prefill_f32<64, false>), g, blk, 0, s, a, items, seqinfo, count);
    }
    return hipGetLastError();
}

}  // namespace va
