// Device helpers shared by the 16-bit attention kernels (matrix instruction
// and transposing LDS read per input type, global -> LDS copies, cross-lane
// reductions).  Internal; included by .hip sources only.
#pragma once

#include "va_internal.h"

namespace va {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

// The 16-bit input type's matrix instruction and transposing LDS read
// (bf16 and fp16 share the data layout and the fp32 accumulation).
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
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
    static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keeps the computation of x at this point of the instruction stream (an
// empty volatile statement that reads and writes it).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

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

// Global -> LDS copies of 16 bytes per lane (lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16)).  They are issued from inline assembly so
// that the compiler's wait-count analysis does not see them: it would make
// every transposing LDS read wait for all copies in flight.  The kernels
// order copies and reads themselves (a vector-memory wait and a barrier
// before a slot is read; copies never target a slot being read).  The
// instructions have no register results; M0 carries the LDS address
// (uniform per wave).
__device__ __forceinline__ void copy16_buffer(u32x4 rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "m0");
}
__device__ __forceinline__ void copy16_global(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p);
}

// Waits until at most N of this wave's vector-memory operations are still
// in flight (they complete in issue order); other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmem_keep()
{
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_keep<0>(); }

}  // namespace dev
}  // namespace va
