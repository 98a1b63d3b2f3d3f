// Attainable-rate probes for the roofline denominators (not part of the
// attention library; built as libva_probe.so and called by the benchmark).
//
// va_probe_mfma_stream: every wave of a full-chip grid runs a stream of
// v_mfma_f32_32x32x16_bf16 on four independent accumulators (consecutive
// products use different operands), optionally with K vector instructions
// (v_exp_f32 or v_fma_f32) issued between products, as an attention
// softmax interleaves them.  It reports the matrix rate the chip sustains
// with that data under its power limit, and the shader clock it ran at
// (s_memtime cycles against the 100 MHz s_memrealtime counter).
//
// va_probe_hbm_stream: a full-chip grid streams a buffer far larger than
// the caches, 16 bytes per lane per access, 4 or 16 independent accesses in
// flight per lane: read only, copy, or write only.  It reports the HBM rate
// the chip sustains for such plain streams, the attainable ceiling beside
// the 8 TB/s datasheet figure for the HBM-bound kernels.
//
// va_probe_lds_stream: the LDS read rate per compute unit (16-byte reads, or
// the transposing 8-byte reads), alone or supplying one operand of every
// product of a product stream, as the attention kernels' tile reads do.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t hash32(uint32_t x)
{
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
}

// a bf16 pair with random mantissa and sign, exponent near 1 (finite sums)
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t s)
{
    const uint32_t h = hash32(s);
    const uint32_t lo = 0x3f00u | (h & 0x807fu), hi = 0x3f00u | ((h >> 16) & 0x807fu);
    return lo | (hi << 16);
}

template <int K, int OP>
__global__ __launch_bounds__(256) void mfma_stream(int iters, int zero, float *sink, unsigned long long *clk)
{
    const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 x, y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[r] = zero ? 0u : rand_bf16x2(gid * 64 + j * 8 + r);
            y[r] = zero ? 0u : rand_bf16x2(gid * 64 + j * 8 + 4 + r + 0x9e3779b9u);
        }
        a[j] = __builtin_bit_cast(bf16x8, x);
        b[j] = __builtin_bit_cast(bf16x8, y);
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = 0.001f * (float)(i + (gid & 7));
    const float f1 = 0.999f, f2 = 0.0001f;

    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a[j]), "v"(b[j]));
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float &x = e[(j * K + k) & 7];
                if constexpr (OP == 0) asm volatile("v_exp_f32 %0, %0" : "+v"(x));
                else asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(f1), "v"(f2));
            }
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += e[i];
    sink[gid] = s;
    if ((threadIdx.x & 63) == 0) {
        const int w = gid >> 6;
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = r1 - r0;
    }
}

template <int K, int OP>
void launch(int grid, int iters, int zero, float *sink, unsigned long long *clk, hipStream_t s)
{
    hipLaunchKernelGGL((mfma_stream<K, OP>), dim3(grid), dim3(256), 0, s, iters, zero, sink, clk);
}

// mode 0: read src, 1: copy src -> dst, 2: write dst; n16 16-byte elements,
// U independent 16-byte accesses per lane in flight
template <int MODE, int U>
__global__ __launch_bounds__(256) void hbm_stream(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, long long n16,
                                                  uint32_t *sink)
{
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        if constexpr (MODE == 2) {
            const u32x4 v = {(uint32_t)i, 1u, 2u, 3u};
#pragma unroll
            for (int k = 0; k < U; ++k) dst[i + k * stride] = v;
        } else {
            u32x4 v[U];
#pragma unroll
            for (int k = 0; k < U; ++k) v[k] = src[i + k * stride];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                if constexpr (MODE == 1) dst[i + k * stride] = v[k];
                else acc ^= v[k];
            }
        }
    }
    for (; i < n16; i += stride) {
        if constexpr (MODE == 2) dst[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
        else if constexpr (MODE == 1) dst[i] = src[i];
        else acc ^= src[i];
    }
    if constexpr (MODE == 0) {
        // one word per thread, so the loads are not dropped
        sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    }
}

// LDS stream: MODE 0: one ds_read_b128 (1 KB per wave) supplies the first
// operand of every product (four products in flight, each operand read four
// products ahead of its use); MODE 1: two ds_read_b64_tr_b16 (2 x 512 B)
// supply it; MODE 2: ds_read_b128 only, eight in flight, no products;
// MODE 3: ds_read_b64_tr_b16 only.  32 KB of LDS per workgroup, every
// address inside it, consecutive lanes on consecutive banks.
template <int MODE>
__global__ __launch_bounds__(256) void lds_stream(int iters, float *sink, unsigned long long *clk)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[8192];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t gid = blockIdx.x * 256 + tid;
    for (int i = tid; i < 8192; i += 256) lds[i] = rand_bf16x2(gid * 131u + (uint32_t)i);
    __syncthreads();
    const char *base = (const char *)lds;
    bf16x8 a[4], b[4];
    f32x16 acc[4];
    u32x4 r[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 x, y;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[q] = rand_bf16x2(gid * 64 + j * 8 + q);
            y[q] = rand_bf16x2(gid * 64 + j * 8 + 4 + q + 0x9e3779b9u);
        }
        a[j] = __builtin_bit_cast(bf16x8, x);
        b[j] = __builtin_bit_cast(bf16x8, y);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = u32x4{0u, 0u, 0u, 0u};

    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int slot = (it * 4 + j) & 31;
            if constexpr (MODE == 0) {
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
                a[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(base + slot * 1024 + lane * 16));
            } else if constexpr (MODE == 1) {
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                typedef bf16x4 __attribute__((address_space(3))) lds_v4;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_v4 *)((__attribute__((address_space(3))) char *)(base + slot * 1024 + lane * 8)));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_v4 *)((__attribute__((address_space(3))) char *)(base + slot * 1024 + 512 + lane * 8)));
                a[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else if constexpr (MODE == 2) {
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    asm volatile("" ::"v"(r[j * 2 + k]));
                    r[j * 2 + k] = *(const u32x4 *)(base + ((slot * 2 + k) & 31) * 1024 + lane * 16);
                }
            } else {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                typedef bf16x4 __attribute__((address_space(3))) lds_v4;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    asm volatile("" ::"v"(r[j * 2 + k]));
                    const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_v4 *)((__attribute__((address_space(3))) char *)(base + slot * 1024 + k * 512 + lane * 8)));
                    const uint2 u = __builtin_bit_cast(uint2, x);
                    r[j * 2 + k] = u32x4{u.x, u.y, 0u, 0u};
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) asm volatile("" ::"v"(r[k]));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
        s += (float)a[j][0];
    }
    sink[gid] = s;
    if (lane == 0) {
        const int w = gid >> 6;
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = r1 - r0;
    }
}

}  // namespace

// Streams `bytes` (a multiple of 16) on the current device with
// blocks_per_cu workgroups of 256 threads per compute unit, 4 (16 if deep)
// accesses per lane in flight, reps times
// between HIP events: mode 0 reads a buffer, 1 copies it to a second one,
// 2 writes one.  Outputs: time of the reps (ms) and the rate counting every
// byte read and written (GB/s).  Allocates and frees its buffers.  Returns
// 0, or a hipError_t.
extern "C" int va_probe_hbm_stream(int mode, long long bytes, int reps, int blocks_per_cu, int deep, double *ms,
                                   double *gbs)
{
    int dev = 0;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return (int)e;
    if (mode < 0 || mode > 2 || bytes < 16 || bytes % 16 != 0 || reps < 1 || blocks_per_cu < 1 || blocks_per_cu > 64)
        return (int)hipErrorInvalidValue;
    const int grid = prop.multiProcessorCount * blocks_per_cu;
    const long long n16 = bytes / 16;
    u32x4 *src = nullptr, *dst = nullptr;
    uint32_t *sink = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (mode != 2) e = hipMalloc(&src, (size_t)bytes);
    if (e == hipSuccess && mode != 0) e = hipMalloc(&dst, (size_t)bytes);
    if (e == hipSuccess) e = hipMalloc(&sink, (size_t)grid * 256 * sizeof(uint32_t));
    if (e == hipSuccess && src) e = hipMemset(src, 0x3c, (size_t)bytes);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    auto run = [&]() {
        if (mode == 0 && deep) hipLaunchKernelGGL((hbm_stream<0, 16>), dim3(grid), dim3(256), 0, 0, src, dst, n16, sink);
        else if (mode == 0) hipLaunchKernelGGL((hbm_stream<0, 4>), dim3(grid), dim3(256), 0, 0, src, dst, n16, sink);
        else if (mode == 1 && deep) hipLaunchKernelGGL((hbm_stream<1, 16>), dim3(grid), dim3(256), 0, 0, src, dst, n16, sink);
        else if (mode == 1) hipLaunchKernelGGL((hbm_stream<1, 4>), dim3(grid), dim3(256), 0, 0, src, dst, n16, sink);
        else if (deep) hipLaunchKernelGGL((hbm_stream<2, 16>), dim3(grid), dim3(256), 0, 0, src, dst, n16, sink);
        else hipLaunchKernelGGL((hbm_stream<2, 4>), dim3(grid), dim3(256), 0, 0, src, dst, n16, sink);
    };
    if (e == hipSuccess) {
        run();  // warm-up
        e = hipEventRecord(e0, 0);
        for (int r = 0; r < reps && e == hipSuccess; ++r) run();
        if (e == hipSuccess) e = hipEventRecord(e1, 0);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
    }
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) {
        float t = 0.f;
        e = hipEventElapsedTime(&t, e0, e1);
        *ms = t;
        *gbs = (double)bytes * (mode == 1 ? 2.0 : 1.0) * reps / (t * 1e-3) / 1e9;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (src) (void)hipFree(src);
    if (dst) (void)hipFree(dst);
    if (sink) (void)hipFree(sink);
    return (int)e;
}

// Runs the stream on the current device: waves_per_simd waves on each SIMD
// of every compute unit, iters groups of 4 products per wave, K = valu
// vector instructions (op 0: v_exp_f32, 1: v_fma_f32) after every product.
// Outputs: kernel time (ms, HIP events), matrix rate (TFLOP/s) and the mean
// shader clock of the waves (MHz).  Returns 0, or a hipError_t.
extern "C" int va_probe_mfma_stream(int waves_per_simd, int iters, int zero_data, int valu, int op, double *ms,
                                    double *tflops, double *mhz)
{
    int dev = 0;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return (int)e;
    if (waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || valu < 0 || valu > 8 || (op != 0 && op != 1))
        return (int)hipErrorInvalidValue;
    const int grid = prop.multiProcessorCount * waves_per_simd;  // 4 waves per workgroup = one per SIMD
    const int waves = grid * 4;
    float *sink = nullptr;
    unsigned long long *clk = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    void (*fn)(int, int, int, float *, unsigned long long *, hipStream_t) = nullptr;
    switch (valu * 2 + op) {
    case 0: case 1: fn = launch<0, 0>; break;
    case 4: fn = launch<2, 0>; break;
    case 5: fn = launch<2, 1>; break;
    case 8: fn = launch<4, 0>; break;
    case 9: fn = launch<4, 1>; break;
    case 12: fn = launch<6, 0>; break;
    case 13: fn = launch<6, 1>; break;
    case 16: fn = launch<8, 0>; break;
    case 17: fn = launch<8, 1>; break;
    default: return (int)hipErrorInvalidValue;
    }
    e = hipMalloc(&sink, (size_t)grid * 256 * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&clk, (size_t)waves * 2 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        fn(grid, iters / 4 + 1, zero_data, sink, clk, 0);  // warm-up (clock ramp)
        e = hipEventRecord(e0, 0);
        if (e == hipSuccess) fn(grid, iters, zero_data, sink, clk, 0);
        if (e == hipSuccess) e = hipEventRecord(e1, 0);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
    }
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) {
        float t = 0.f;
        e = hipEventElapsedTime(&t, e0, e1);
        unsigned long long *h = new unsigned long long[(size_t)waves * 2]();
        if (e == hipSuccess) e = hipMemcpy(h, clk, (size_t)waves * 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
        double cyc = 0, real = 0;
        for (int w = 0; w < waves; ++w) { cyc += (double)h[2 * w]; real += (double)h[2 * w + 1]; }
        delete[] h;
        *ms = t;
        *tflops = (double)waves * iters * 4.0 * 32768.0 / (t * 1e-3) / 1e12;
        *mhz = real > 0 ? cyc / real * 100.0 : 0.0;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (sink) (void)hipFree(sink);
    if (clk) (void)hipFree(clk);
    return (int)e;
}

// Runs the LDS stream (mode 0..3, above) on the current device:
// waves_per_simd workgroups of 4 waves per compute unit, iters groups of 4
// products (modes 0, 1) or of 8 reads (modes 2, 3) per wave.  Outputs:
// kernel time (ms), matrix rate (TFLOP/s, modes 0 and 1), mean shader
// clock (MHz) and LDS bytes read per clock per compute unit (the waves'
// bytes over their mean cycle count).  Returns 0, or a hipError_t.
extern "C" int va_probe_lds_stream(int waves_per_simd, int iters, int mode, double *ms, double *tflops, double *mhz,
                                   double *bytes_per_clk)
{
    int dev = 0;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return (int)e;
    if (waves_per_simd < 1 || waves_per_simd > 4 || iters < 1 || mode < 0 || mode > 3)
        return (int)hipErrorInvalidValue;
    const int cus = prop.multiProcessorCount;
    const int grid = cus * waves_per_simd;
    const int waves = grid * 4;
    float *sink = nullptr;
    unsigned long long *clk = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    auto go = [&](int n) {
        if (mode == 0) hipLaunchKernelGGL((lds_stream<0>), dim3(grid), dim3(256), 0, 0, n, sink, clk);
        else if (mode == 1) hipLaunchKernelGGL((lds_stream<1>), dim3(grid), dim3(256), 0, 0, n, sink, clk);
        else if (mode == 2) hipLaunchKernelGGL((lds_stream<2>), dim3(grid), dim3(256), 0, 0, n, sink, clk);
        else hipLaunchKernelGGL((lds_stream<3>), dim3(grid), dim3(256), 0, 0, n, sink, clk);
    };
    e = hipMalloc(&sink, (size_t)grid * 256 * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&clk, (size_t)waves * 2 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        go(iters / 4 + 1);  // warm-up (clock ramp)
        e = hipEventRecord(e0, 0);
        if (e == hipSuccess) go(iters);
        if (e == hipSuccess) e = hipEventRecord(e1, 0);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
    }
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) {
        float t = 0.f;
        e = hipEventElapsedTime(&t, e0, e1);
        unsigned long long *h = new unsigned long long[(size_t)waves * 2]();
        if (e == hipSuccess) e = hipMemcpy(h, clk, (size_t)waves * 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
        double cyc = 0, real = 0;
        for (int w = 0; w < waves; ++w) { cyc += (double)h[2 * w]; real += (double)h[2 * w + 1]; }
        delete[] h;
        const double per_wave = mode == 2 ? 8192.0 : 4096.0;  // bytes per iteration
        *ms = t;
        *tflops = mode <= 1 ? (double)waves * iters * 4.0 * 32768.0 / (t * 1e-3) / 1e12 : 0.0;
        *mhz = real > 0 ? cyc / real * 100.0 : 0.0;
        *bytes_per_clk = cyc > 0 ? (double)waves * iters * per_wave / (cyc / waves) / cus : 0.0;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (sink) (void)hipFree(sink);
    if (clk) (void)hipFree(clk);
    return (int)e;
}
