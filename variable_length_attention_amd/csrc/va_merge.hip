// Merge of partial attention results computed over disjoint key sets.
//
// The local step of ring / context-parallel attention (vllm-omni ulysses.py
// hands the ring path its joint K/V; every rank's partial result is an
// attention output over its own keys plus the log-sum-exp of those keys'
// scores): with partials (O_p, L_p) for one (row, head),
//   m = max(max_p L_p, sigma),  w_p = exp(L_p - m),  s = sum_p w_p + exp(sigma - m)
//   L = m + log(s),             O = sum_p (w_p / s) O_p
// where sigma is the head's sink logit (omitted when there are no sinks):
// the softmax over the union of the key sets, with the sink counted once.
// A part with L_p = -inf (no visible key) has weight 0; a row whose parts
// are all empty and has no sink gets O = 0, L = -inf.
//
// HBM bound: every partial is read once, the result written once.  One
// lane per 8 consecutive elements of a (row, head) vector (16- or 32-byte
// loads, the D / 8 lanes of a vector read one contiguous segment); the n
// log-sum-exp values of the vector are read by each of its lanes (the same
// cache line).
#include "va_internal.h"

namespace va {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load8(const void *base, size_t idx, bool bf16, float (&x)[8])
{
    if (bf16) {
        const u32x4 w = *(const u32x4 *)((const uint16_t *)base + idx);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)base + idx);
        const f32x4 b = *(const f32x4 *)((const float *)base + idx + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    }
}

// round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <bool PART_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void k4_merge(MergeArgs a)
{
    const int lpv = a.D >> 3;  // lanes per (row, head) vector
    const long long vecs = (long long)a.rows * a.H;
    const long long n_threads = vecs * lpv;
    const size_t part_stride = (size_t)vecs * a.D;  // elements between parts
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < n_threads;
         t += (long long)gridDim.x * blockDim.x) {
        const long long vec = t / lpv;
        const int c8 = (int)(t - vec * lpv);
        const int h = (int)(vec % a.H);
        const float sig = a.sinks ? a.sinks[h] : -INFINITY;
        float m = sig;
        for (int p = 0; p < a.n; ++p) m = fmaxf(m, a.lse_parts[(size_t)p * vecs + vec]);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        float lse_out = -INFINITY;
        if (m != -INFINITY) {
            float s = a.sinks ? __expf(sig - m) : 0.f;
            const size_t idx = (size_t)vec * a.D + c8 * 8;
            // four parts per round, their loads issued together; a part past
            // n re-reads the last one and an empty part (weight 0) is dropped
            // by a select after the product, so values stored in an empty
            // part never reach the result
            for (int p0 = 0; p0 < a.n; p0 += 4) {
                float x[4][8], w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = min(p0 + i, a.n - 1);
                    load8(a.o_parts, (size_t)p * part_stride + idx, PART_BF16, x[i]);
                    const float l = a.lse_parts[(size_t)p * vecs + vec];
                    w[i] = (p0 + i < a.n && l != -INFINITY) ? __expf(l - m) : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s += w[i];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += w[i] != 0.f ? w[i] * x[i][e] : 0.f;
                }
            }
            const float inv = 1.f / s;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= inv;
            lse_out = m + __logf(s);
        }
        const size_t o = (size_t)vec * a.D + c8 * 8;
        if (OUT_BF16) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = bf16_bits(acc[2 * e]) | (bf16_bits(acc[2 * e + 1]) << 16);
            *(u32x4 *)((uint16_t *)a.out + o) = w;
        } else {
            *(f32x4 *)((float *)a.out + o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *(f32x4 *)((float *)a.out + o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        }
        if (a.lse && c8 == 0) a.lse[vec] = lse_out;
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, bool part_bf16, bool out_bf16, hipStream_t s)
{
    const long long n_threads = (long long)a.rows * a.H * (a.D >> 3);
    const long long want = (n_threads + 255) / 256;
    const int grid = (int)(want < 65536 ? want : 65536);
    if (part_bf16 && out_bf16) hipLaunchKernelGGL((k4_merge<true, true>), dim3(grid), dim3(256), 0, s, a);
    else if (part_bf16) hipLaunchKernelGGL((k4_merge<true, false>), dim3(grid), dim3(256), 0, s, a);
    else if (out_bf16) hipLaunchKernelGGL((k4_merge<false, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k4_merge<false, false>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace va
