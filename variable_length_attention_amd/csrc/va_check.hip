// Opt-in device-side check of the argument contents the host cannot see
// without a synchronisation: cu_seqlens start at 0, never decrease and end
// at the row totals; lengths stay within max_seqlen; in paged mode each
// seqused_k fits its block-table row and every block id it uses names a
// block of the cache.  One workgroup; it reads only the arrays whose sizes
// the host has already validated, so it is safe on any contents.
#include "va_internal.h"

namespace va {

namespace {

__global__ __launch_bounds__(256) void k_check(CheckArgs c)
{
    __shared__ uint32_t s_flags;
    if (threadIdx.x == 0) s_flags = 0;
    __syncthreads();
    uint32_t f = 0;
    for (int b = threadIdx.x; b < c.B; b += blockDim.x) {
        const int q0 = c.cu_q[b], q1 = c.cu_q[b + 1];
        if (b == 0 && q0 != 0) f |= kChkCuQStart;
        if (q1 < q0) f |= kChkCuQOrder;
        if (b == c.B - 1 && q1 != c.total_q) f |= kChkCuQTotal;
        if (q1 - q0 > c.max_q) f |= kChkLenQ;
        if (c.cu_k) {
            const int k0 = c.cu_k[b], k1 = c.cu_k[b + 1];
            if (b == 0 && k0 != 0) f |= kChkCuKStart;
            if (k1 < k0) f |= kChkCuKOrder;
            if (b == c.B - 1 && k1 != c.total_k) f |= kChkCuKTotal;
            if (k1 - k0 > c.max_k) f |= kChkLenK;
        }
        if (c.seqused_k) {
            const int su = c.seqused_k[b];
            const long long cap = (long long)c.bt_stride * c.block_size;
            if (su < 0 || su > cap) f |= kChkSeqused;
            if (su > c.max_k) f |= kChkLenK;
            const int used = su <= 0 ? 0 : (int)min((long long)(su + c.block_size - 1) / c.block_size,
                                                     (long long)c.bt_stride);
            for (int i = 0; i < used; ++i) {
                const int blk = c.block_table[(size_t)b * c.bt_stride + i];
                if (blk < 0 || blk >= c.num_blocks) f |= kChkBlockId;
            }
        }
    }
    if (f) atomicOr(&s_flags, f);
    __syncthreads();
    if (threadIdx.x == 0) *c.flags = s_flags;
}

}  // namespace

hipError_t launch_check(const CheckArgs &c, hipStream_t s)
{
    hipLaunchKernelGGL(k_check, dim3(1), dim3(256), 0, s, c);
    return hipGetLastError();
}

}  // namespace va
