// Backward of the varlen attention forward on gfx950 matrix cores, for bf16
// or fp16 inputs (one template over the 16-bit type, fp32 accumulation).
//
// Method: the steps of the boostr CPU backward varlen_attention_bwd, given
// the forward's out and lse (a sink enters only through lse):
//   Dv_i = sum_d dO_i,d O_i,d
//   P_ij = exp(scale <q_i, k_j> - lse_i)            (allowed keys only)
//   dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - Dv_i)
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
// with dK / dV of a kv head summed over the query heads that share it.
//
// Three kernels, none with atomics (results are deterministic):
//   B0 k_bwd_dot   Dv for every (row, head), fp32.
//   B1 k_bwd_dq    one workgroup per (128-row query block, head), the work
//                  items of the forward: per 64-key tile S^T = K Q^T and
//                  dP^T = V dO^T (Q^T, dO^T in registers), dS^T from them,
//                  dQ^T += K^T dS^T through transposing LDS reads.
//   B2 k_bwd_dkdv  one workgroup per (128-key block, kv head); each wave
//                  keeps its 32 keys' K and V operands in registers and
//                  streams 64-row Q / dO tiles of every query head of the
//                  GQA group: S = Q K^T, dP = dO V^T, dV^T += dO^T P and
//                  dK^T += Q^T dS (keys on the MFMA N side).
// K, V, Q and dO tiles are read both row-wise (16-byte operand reads) and
// transposed (ds_read_b64_tr_b16); one XOR swizzle of the 16-byte chunks
// serves both without bank conflicts.
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

// The 16-bit input type's transposing LDS read, matrix instruction (in the
// VGPR form, and into AGPR accumulators through assembly: the compiler
// selects one register form for all of a kernel's matrix instructions; the
// leading s_nop covers the two wait states after a VALU write of an A / B
// operand, which the compiler does not see into the block) and widening of
// the low / high half of a 32-bit word.
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
    static __device__ __forceinline__ void mfma_agpr(f32x16 &acc, v8 a, v8 b)
    {
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
    static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
    static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
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
    static __device__ __forceinline__ float lo(uint32_t x) { return (float)__builtin_bit_cast(_Float16, (uint16_t)x); }
    static __device__ __forceinline__ float hi(uint32_t x)
    {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
    }
};

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).
// For 256-byte rows (D = 128) the 16 rows of a row-wise operand read get 16
// distinct chunks, and the 4 consecutive rows x 4 consecutive chunks of a
// transposing read get 16 distinct chunks; for 128-byte rows (D = 64) the
// same holds per pair of rows sharing a 256-byte bank line.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Global -> LDS copies of 16 bytes per lane (lane i writes LDS bytes
// [lds + 16 i, +16)), issued from inline assembly so that the compiler's
// wait-count analysis does not make the transposing reads wait for copies
// of other slots; the kernels order copies and reads themselves (a
// vector-memory wait and a barrier before a slot is read).  No register
// results; M0 carries the LDS address (uniform per wave).
__device__ __forceinline__ void copy16_buffer(u32x4 rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(p);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// raw buffer over `rows` rows of `rowstride` bytes from base (reads past
// the end return 0)
__device__ __forceinline__ u32x4 rows_rsrc(const void *base, int rows, size_t rowstride)
{
    const uint32_t nrec = rows > 0 ? (uint32_t)((size_t)rows * rowstride) : 0u;
    const uint64_t addr = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)addr, (uint32_t)(addr >> 32) & 0xffffu, nrec, 0x00020000u};
}

// Copies a tile of 64 rows x D (row-major, `rowstride` bytes apart, rows
// past `rows` read as zero) into LDS at dst with the swizzle above; the 4
// waves take 16 rows each.
template <int D>
__device__ __forceinline__ void copy_tile(const char *src, int rows, size_t rowstride, char *dst, int wave, int lane)
{
    constexpr int NCH = D / 8, RPI = 64 / NCH, LPW = 64 / RPI / 4;
    const u32x4 rs = rows_rsrc(src, rows < 64 ? rows : 64, rowstride);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int r = (wave * LPW + u) * RPI + lane / NCH;
        const int chunk = (lane % NCH) ^ swz<D>(r);
        copy16_buffer(rs, (uint32_t)(r * rowstride) + chunk * 16, lds_addr(dst + (wave * LPW + u) * 1024));
    }
}

// The dK / dV kernel keeps its 256 accumulator registers in AGPRs
// (Elt::mfma_agpr) and everything else in VGPRs.  Wait states between the last matrix instruction into acc and any other
// read of it (VALU, LDS or memory instructions read AGPRs only after the
// matrix pipeline has written them back; 16 passes need 18).
__device__ __forceinline__ void mfma_agpr_drain(f32x16 &acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Keeps the computation of x at this point of the instruction stream (an
// empty volatile statement that reads and writes it; arithmetic without
// side effects is otherwise free to sink towards its uses).
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }


// ------------------------------------------------------------------ B0
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_dot(const uint16_t *__restrict__ dout, const uint16_t *__restrict__ out,
                                                 float *__restrict__ dvec, int rows)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr int LPR = D / 8;        // lanes per (row, head), 16 bytes each
    constexpr int RPB = 256 / LPR;    // (row, head) pairs per workgroup
    const int r = blockIdx.x * RPB + threadIdx.x / LPR;
    const int l = threadIdx.x % LPR;
    float acc = 0.f;
    if (r < rows) {
        const u32x4 x = *(const u32x4 *)(dout + (size_t)r * D + l * 8);
        const u32x4 y = *(const u32x4 *)(out + (size_t)r * D + l * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += E::lo(x[e]) * E::lo(y[e]) + E::hi(x[e]) * E::hi(y[e]);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (l == 0 && r < rows) dvec[r] = acc;
}

// ------------------------------------------------------------------ B3
// Gradient of the sink logits.  The sink of head h enters row i's softmax as
// one more logit s_h with a zero value row, so its dS term is
// P_sink (0 - Dv_i) with P_sink = exp(s_h - lse_i), and
//   dsinks_h = - sum_i exp(s_h - lse_i) sum_d dO_i,d O_i,d.
// Step 1: the term of every (row, head), into the workspace.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_sink_terms(const uint16_t *__restrict__ dout,
                                                        const uint16_t *__restrict__ out, const float *__restrict__ lse,
                                                        const float *__restrict__ sinks, float *__restrict__ terms,
                                                        int rows, int H)
{
    using E = Elt<T>;
    constexpr int LPR = D / 8;        // lanes per (row, head), 16 bytes each
    constexpr int RPB = 256 / LPR;    // (row, head) pairs per workgroup
    const int r = blockIdx.x * RPB + threadIdx.x / LPR;
    const int l = threadIdx.x % LPR;
    float acc = 0.f;
    if (r < rows) {
        const u32x4 x = *(const u32x4 *)(dout + (size_t)r * D + l * 8);
        const u32x4 y = *(const u32x4 *)(out + (size_t)r * D + l * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += E::lo(x[e]) * E::lo(y[e]) + E::hi(x[e]) * E::hi(y[e]);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (l == 0 && r < rows) {
        const float ls = lse[r];
        terms[r] = ls == -INFINITY ? 0.f : __expf(sinks[r % H] - ls) * acc;
    }
}

// Step 2: one workgroup per head sums its terms in a fixed order
// (deterministic): strided partial sums, then a tree in LDS.
__global__ __launch_bounds__(256) void k_bwd_sink_sum(const float *__restrict__ terms, float *__restrict__ dsinks,
                                                      int T, int H)
{
    __shared__ float part[256];
    const int h = blockIdx.x, tid = threadIdx.x;
    float acc = 0.f;
    for (int i = tid; i < T; i += 256) acc += terms[(size_t)i * H + h];
    part[tid] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) part[tid] += part[tid + w];
        __syncthreads();
    }
    if (tid == 0) dsinks[h] = -part[0];
}

// ------------------------------------------------------------------ B1
template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dq(
    BwdArgs a, const int4 *__restrict__ items, const int4 *__restrict__ seqinfo, const int32_t *__restrict__ count)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr int BN = 64;
    constexpr int NCH = D / 8;
    constexpr int KS = D / 16;
    constexpr int MD = D / 32;
    constexpr int ROWB = D * 2;
    constexpr int TILEB = BN * ROWB;
    // LDS: K ring [K0 | K1] then V ring [V0 | V1]; tile t in slot t & 1
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILEB];
    char *const kring = (char *)smem;
    char *const vring = kring + 2 * TILEB;

    // a.hpw == 1: the item's 128 query rows of one head (32 per wave).
    // a.hpw == 4: a quarter of the item (32 rows) for 4 heads that share a kv
    // head (one head per wave): the waves see the same keys, so none of them
    // waits through tiles only another wave's rows need.
    int item, slot;
    map_block(blockIdx.x, a.H, item, slot);
    const int n_items = *count;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    asm volatile("" ::"s"(it.x), "s"(si.x), "s"(n_items));
    if (item >= n_items) return;
    int i0 = it.y, kv_lo = it.z, kv_hi = it.w;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int delta = Lk - Lq;
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;
    const int wrow = a.hpw == 1 ? wave * 32 : 0;  // the wave's first row
    const int head = a.hpw == 1 ? slot : (slot >> 2) * 4 + wave;
    const int c = head / a.g;                     // the same for every wave
    const int row = i0 + wrow + n;
    const bool row_ok = row < Lq;
    int lo = 1, hi = 0;
    if (row_ok) row_bounds(row, delta, Lk, a.left, a.right, lo, hi);
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

    const size_t rowstride = (size_t)a.Hkv * D * 2;
    const char *kseq = (const char *)a.k + ((size_t)k0 * a.Hkv + c) * D * 2;
    const char *vseq = (const char *)a.v + ((size_t)k0 * a.Hkv + c) * D * 2;
    auto issue = [&](int t, char *kdst, char *vdst) {
        const int j0 = kv_lo + t * BN;
        copy_tile<D>(kseq + (size_t)j0 * rowstride, kv_hi - j0, rowstride, kdst, wave, lane);
        copy_tile<D>(vseq + (size_t)j0 * rowstride, kv_hi - j0, rowstride, vdst, wave, lane);
    };

    // Q^T and dO^T operand fragments: lane (row n, half h2) holds d = 16 ks + 8 h2 .. +8
    v8 qf[KS], df[KS];
    {
        const size_t off = ((size_t)(q0 + (row_ok ? row : 0)) * a.H + head) * D + h2 * 8;
        const uint16_t *qp = (const uint16_t *)a.q + off;
        const uint16_t *dp = (const uint16_t *)a.dout + off;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4 *)(qp + ks * 16);
            u32x4 y = *(const u32x4 *)(dp + ks * 16);
            if (!row_ok) { x = u32x4{0, 0, 0, 0}; y = u32x4{0, 0, 0, 0}; }
            qf[ks] = __builtin_bit_cast(v8, x);
            df[ks] = __builtin_bit_cast(v8, y);
        }
    }
    // lse in log2 units; rows without any allowed key (lse = -inf) and rows
    // past the end get +inf, which makes every probability 0
    float lse2 = INFINITY, dvr = 0.f;
    // ALiBi in log2 units: - slope log2(e) |row + delta - j|
    const float sl2 = ALIBI ? a.alibi[head] * kLog2e : 0.f;
    if (row_ok) {
        const size_t ri = (size_t)(q0 + row) * a.H + head;
        const float l = a.lse[ri];
        lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
        dvr = a.dvec[ri];
    }

    f32x16 dqa[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 16; ++v) dqa[md][v] = 0.f;

    // LDS byte offsets: row-wise operand read of row n, chunk 2 ks + h2; and
    // the transposing read of rows 16 t4 + 4 h2 + q4 (+8), 4 columns at
    // md * 32 + 16 ((lane & 31) >> 4) + 4 (l16 & 3)
    auto koff = [&](int ks) -> uint32_t { return n * ROWB + (((ks * 2 + h2) ^ swz<D>(n)) << 4); };
    auto toff = [&](int md, int half) -> uint32_t {
        const int r = h2 * 4 + q4 + half * 8;
        const int col = md * 32 + ((lane & 31) >> 4) * 16 + (l16 & 3) * 4;
        return r * ROWB + (((col >> 3) ^ swz<D>(r)) << 4) + (col & 7) * 2;
    };

    if (ntiles > 0) issue(0, kring, vring);
    wait_vmem();
    __syncthreads();

    auto tile = [&](int t, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const char *kt = kring + BUF * TILEB;
        const char *vt = vring + BUF * TILEB;
        if (t + 1 < ntiles) issue(t + 1, kring + (BUF ^ 1) * TILEB, vring + (BUF ^ 1) * TILEB);
        if (visible(t)) {
            const int j0 = kv_lo + t * BN;
            // S^T = K Q^T, dP^T = V dO^T: lane value v of block mb is key
            // j0 + 32 mb + 8 (v/4) + 4 h2 + v%4 of query row n
            f32x16 S[2], P[2];
#pragma unroll
            for (int v = 0; v < 16; ++v) { S[0][v] = 0.f; S[1][v] = 0.f; P[0][v] = 0.f; P[1][v] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const v8 k0f = *(const v8 *)(kt + koff(ks));
                const v8 k1f = *(const v8 *)(kt + koff(ks) + 32 * ROWB);
                const v8 v0f = *(const v8 *)(vt + koff(ks));
                const v8 v1f = *(const v8 *)(vt + koff(ks) + 32 * ROWB);
                S[0] = E::mfma(k0f, qf[ks], S[0]);
                S[1] = E::mfma(k1f, qf[ks], S[1]);
                P[0] = E::mfma(v0f, df[ks], P[0]);
                P[1] = E::mfma(v1f, df[ks], P[1]);
            }
            if (!(j0 >= flo && j0 + BN - 1 <= fhi)) {
                // key j is allowed iff (unsigned)(j - lo) <= (unsigned)(hi - lo)
                const bool none = hi < lo;
                const uint32_t span = none ? 0u : (uint32_t)(hi - lo);
                const int jb = none ? 1 : j0 + h2 * 4 - lo;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const uint32_t d = (uint32_t)(jb + mb * 32 + (v >> 2) * 8 + (v & 3));
                        S[mb][v] = d > span ? -INFINITY : S[mb][v];
                    }
            }
            // dS^T in the input type, laid out as the B operand of step t4 (keys 16 t4 ..)
            const float abase = (float)(row + delta - j0 - 4 * h2);
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ix = (t4 & 1) * 8 + e;
                    float y = fmaf(S[t4 >> 1][ix], a.scale_log2, -lse2);
                    if constexpr (ALIBI)
                        y = fmaf(-sl2, fabsf(abase - (float)(32 * (t4 >> 1) + 8 * (ix >> 2) + (ix & 3))), y);
                    const float p = __builtin_amdgcn_exp2f(y);
                    x[e] = p * (P[t4 >> 1][ix] - dvr);
                }
                const v8 dsb = __builtin_convertvector(x, v8);
                // dQ^T += K^T dS^T
#pragma unroll
                for (int md = 0; md < MD; ++md) {
                    const v4 ka = E::read_tr(kt + toff(md, 0) + t4 * 16 * ROWB);
                    const v4 kb = E::read_tr(kt + toff(md, 1) + t4 * 16 * ROWB);
                    const v8 kf = __builtin_shufflevector(ka, kb, 0, 1, 2, 3, 4, 5, 6, 7);
                    dqa[md] = E::mfma(kf, dsb, dqa[md]);
                }
            }
        }
        wait_vmem();
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        tile(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntiles) tile(t, std::integral_constant<int, 0>{});

    // epilogue: lane (row n, half h2) holds dQ^T[32 md + 8 i + 4 h2 + j][row];
    // rows leave through LDS as whole 16-byte-per-lane rows
    char *ow = kring + wave * 32 * ROWB;  // chunk XOR (row mod NCH)
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = dqa[md][i * 4 + j] * a.scale;
            const v4 y = __builtin_convertvector(x, v4);
            const int phys = (md * 4 + i) ^ (n % NCH);
            *(u32x2 *)(ow + n * ROWB + phys * 16 + h2 * 8) = __builtin_bit_cast(u32x2, y);
        }
    __syncthreads();
    {
        constexpr int RPW = 64 / NCH;
        const int cidx = lane % NCH;
#pragma unroll
        for (int u = 0; u < 32 / RPW; ++u) {
            const int r = u * RPW + lane / NCH;
            const int orow = i0 + wrow + r;
            const u32x4 v = *(const u32x4 *)(ow + r * ROWB + ((cidx ^ (r % NCH)) << 4));
            if (orow < Lq)
                *(u32x4 *)((uint16_t *)a.dq + ((size_t)(q0 + orow) * a.H + head) * D + cidx * 8) = v;
        }
    }
}

// ------------------------------------------------------------------ B2
template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_bwd_dkdv(
    BwdArgs a, const int4 *__restrict__ items, const int4 *__restrict__ seqinfo, const int32_t *__restrict__ count)
{
    using E = Elt<T>;
    typedef typename E::v8 v8;
    typedef typename E::v4 v4;
    constexpr int QT = 64;             // query rows per tile
    constexpr int KS = D / 16;
    constexpr int MD = D / 32;
    constexpr int ROWB = D * 2;
    constexpr int TILEB = QT * ROWB;
    // LDS: Q ring [Q0 | Q1], dO ring [O0 | O1], the block's 128 V rows, then
    // per slot 64 lse2 and 64 Dv
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILEB];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[kBwdKeys * D];
    __shared__ __attribute__((aligned(16))) float s_rows[2][2][QT];
    char *const qring = (char *)smem;
    char *const oring = qring + 2 * TILEB;
    char *const vt = (char *)s_v;

    int item, c;
    map_block(blockIdx.x, a.Hkv, item, c);
    const int n_items = *count;
    const int4 it = items[item];
    const int4 si = seqinfo[item];
    asm volatile("" ::"s"(it.x), "s"(si.x), "s"(n_items));
    if (item >= n_items) return;
    const int j0 = it.y, qlo = it.z, qhi = it.w;
    const int q0 = si.x, Lq = si.y, k0 = si.z, Lk = si.w;
    const int delta = Lk - Lq;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h2 = lane >> 5, l16 = lane & 15, q4 = l16 >> 2;
    // wave (kh, rh): keys j0 + 64 kh .. +64 (two MFMA column blocks kb), query
    // rows 32 rh .. +32 of every tile; the two waves of one kh add their
    // partial dK / dV at the end
    const int kh = wave & 1, rh = wave >> 1;
    int keyv[2];
    bool key_ok[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        keyv[kb] = j0 + kh * 64 + kb * 32 + n;
        key_ok[kb] = keyv[kb] < Lk;
    }

    // K^T operand fragments (B side) in registers: lane (key n, half h2)
    // holds d = 16 ks + 8 h2 .. +8; the V rows of the block go to LDS (the
    // dP products read them from there: registers are short)
    v8 kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const size_t off = ((size_t)(k0 + (key_ok[kb] ? keyv[kb] : 0)) * a.Hkv + c) * D + h2 * 8;
        const uint16_t *kp = (const uint16_t *)a.k + off;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4 *)(kp + ks * 16);
            if (!key_ok[kb]) x = u32x4{0, 0, 0, 0};
            kf[kb][ks] = __builtin_bit_cast(v8, x);
        }
    }
    {
        const size_t kvstride = (size_t)a.Hkv * D * 2;
        const char *vsrc = (const char *)a.v + ((size_t)(k0 + j0) * a.Hkv + c) * D * 2;
        copy_tile<D>(vsrc, Lk - j0, kvstride, vt, wave, lane);
        copy_tile<D>(vsrc + 64 * kvstride, Lk - j0 - 64, kvstride, vt + 64 * ROWB, wave, lane);
    }
    f32x16 dka[MD][2], dva[MD][2];
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) { dka[md][kb][v] = 0.f; dva[md][kb][v] = 0.f; }

    // allowed (query i, key j): j - i in [delta - left, delta + right], j < Lk;
    // for each of this lane's keys: rows [rlo, rlo + rspan] (none past Lk)
    const long long dlo = a.left >= kInfOff ? -(1ll << 40) : (long long)delta - a.left;
    const long long dhi = a.right >= kInfOff ? (1ll << 40) : (long long)delta + a.right;
    int rlo[2];
    uint32_t rspan[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        rlo[kb] = (int)max((long long)keyv[kb] - dhi, -1ll);
        const int rhi = (int)min((long long)keyv[kb] - dlo, (long long)kMaxSeqlen);
        rspan[kb] = (uint32_t)(rhi - rlo[kb]);
        if (!key_ok[kb] || rhi < rlo[kb]) { rlo[kb] = kMaxSeqlen + 1; rspan[kb] = 0; }  // rows < kMaxSeqlen
    }

    const size_t qstride = (size_t)a.H * D * 2;
    const int qtiles = (qhi - qlo + QT - 1) / QT;
    const int total = qtiles * a.g;  // (query tile, head of the group) steps
    // step s: query rows qlo + QT (qtiles - 1 - s / g) .., head c g + s % g:
    // the g heads of one tile in a row (their rows are adjacent in memory),
    // tiles from the last one down (measured 2-3% faster than head-major
    // ascending order on a causal GQA workload)
    // step s: copies of its Q / dO tiles into slot `slot`; its per-row lse
    // (log2 units; +inf for rows past the range or without keys) and Dv are
    // read into registers here and written to LDS by row_store() at the end
    // of the current step, so that waiting for them never waits for copies
    float st_l2 = INFINITY, st_dv = 0.f;
    // ALiBi slope (log2 units) of the next step's head and of this step's
    float sl_next = 0.f, sl_cur = 0.f;
    // step s = t g + h (t: query tile counted from the last, h: head offset),
    // tracked as the pair (t, h) so that no step divides by g
    auto tile_row = [&](int t) { return qlo + (qtiles - 1 - t) * QT; };
    // copies of step s's tiles: KS parts of one 16-byte-per-lane copy each
    // (Q rows, then dO rows), issued one at a time between the matrix
    // instructions of the previous step; with no step s the buffers are
    // empty (nothing is read, the slot gets zeros)
    constexpr int NCH = D / 8, RPI = 64 / NCH, LPW = 64 / RPI / 4;
    static_assert(2 * LPW == KS, "one copy part per K step");
    u32x4 rs_q = {0, 0, 0, 0}, rs_o = {0, 0, 0, 0};
    int cp_slot = 0;
    auto copy_setup = [&](bool valid, int t, int hoff, int slot) {
        const int rows = valid ? min(qhi - tile_row(t), QT) : 0;
        const size_t off = valid ? ((size_t)(q0 + tile_row(t)) * a.H + c * a.g + hoff) * D * 2 : 0;
        rs_q = rows_rsrc((const char *)a.q + off, rows, qstride);
        rs_o = rows_rsrc((const char *)a.dout + off, rows, qstride);
        cp_slot = slot;
    };
    auto copy_part = [&](int part) {
        const int u = part % LPW;
        const int r = (wave * LPW + u) * RPI + lane / NCH;
        const int chunk = (lane % NCH) ^ swz<D>(r);
        char *dst = (part < LPW ? qring : oring) + cp_slot * TILEB + (wave * LPW + u) * 1024;
        copy16_buffer(part < LPW ? rs_q : rs_o, (uint32_t)(r * qstride) + chunk * 16, lds_addr(dst));
    };
    auto issue = [&](int t, int hoff) {
        const int h = c * a.g + hoff;
        const int r0 = tile_row(t);
        st_l2 = INFINITY;
        st_dv = 0.f;
        if constexpr (ALIBI) sl_next = a.alibi[h] * kLog2e;
        const int r = r0 + tid;
        if (tid < QT && r < qhi) {
            const size_t ri = (size_t)(q0 + r) * a.H + h;
            const float l = a.lse[ri];
            st_l2 = l == -INFINITY ? INFINITY : l * kLog2e;
            st_dv = a.dvec[ri];
        }
    };
    auto row_store = [&](int slot) {
        if (tid < QT) {
            s_rows[slot][0][tid] = st_l2;
            s_rows[slot][1][tid] = st_dv;
        }
    };

    // LDS offsets: row-wise operand read of query row 32 rh + n, chunk
    // 2 ks + h2; transposing read of rows 16 t4 + 4 h2 + q4 (+8)
    auto roff = [&](int ks) -> uint32_t {
        const int r = rh * 32 + n;
        return r * ROWB + (((ks * 2 + h2) ^ swz<D>(r)) << 4);
    };
    auto toff = [&](int md, int half) -> uint32_t {
        const int r = h2 * 4 + q4 + half * 8;
        const int col = md * 32 + ((lane & 31) >> 4) * 16 + (l16 & 3) * 4;
        return r * ROWB + (((col >> 3) ^ swz<D>(r)) << 4) + (col & 7) * 2;
    };

    // V row-wise operand read of key kh 64 + kb 32 + n, chunk 2 ks + h2
    auto voff = [&](int kb, int ks) -> uint32_t {
        const int r = kh * 64 + kb * 32 + n;
        return r * ROWB + (((ks * 2 + h2) ^ swz<D>(r)) << 4);
    };
    // a query tile starting at row r0 needs no mask when every (row, key) of
    // it is allowed (rows past the range carry lse = +inf and drop out)
    const bool keys_full = j0 + kBwdKeys <= Lk;
    auto tile_full = [&](int r0) {
        return keys_full && (long long)j0 - (r0 + QT - 1) >= dlo && (long long)j0 + kBwdKeys - 1 - r0 <= dhi;
    };

    // one step: lane value v of block kb is row 32 rh + 8 (v/4) + 4 h2 + v%4
    // of the tile and key keyv[kb]
    auto step = [&](int slot, int r0, bool full) {
        const char *qt = qring + slot * TILEB;
        const char *ot = oring + slot * TILEB;
        const float *l2s = s_rows[slot][0];
        const float *dvs = s_rows[slot][1];
        // S = Q K^T
        f32x16 S[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) S[kb][v] = 0.f;
        // all Q operands first: one LDS latency for the 2 KS products
        v8 qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = *(const v8 *)(qt + roff(ks));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            S[0] = E::mfma(qa[ks], kf[0][ks], S[0]);
            S[1] = E::mfma(qa[ks], kf[1][ks], S[1]);
        }
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int base = r0 + rh * 32 + h2 * 4 - rlo[kb];
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    S[kb][v] = (uint32_t)(base + (v >> 2) * 8 + (v & 3)) <= rspan[kb] ? S[kb][v] : -INFINITY;
            }
        }
        f32x4 l2r[4], dvr[4];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            l2r[e4] = *(const f32x4 *)(l2s + rh * 32 + e4 * 8 + h2 * 4);
            dvr[e4] = *(const f32x4 *)(dvs + rh * 32 + e4 * 8 + h2 * 4);
        }
        // dP = dO V^T, interleaved with the probabilities (in place in S):
        // each matrix instruction is followed by 16 / KS exponentials; the
        // scheduling fences keep that order (one wave per SIMD: the overlap
        // of matrix and vector work has to come from the instruction order)
        f32x16 P[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) P[kb][v] = 0.f;
        // ALiBi: row 32 rh + 8 (v/4) + 4 h2 + v%4 of the tile against key keyv[kb]
        float abase[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) abase[kb] = (float)(r0 + rh * 32 + 4 * h2 + delta - keyv[kb]);
        auto prob = [&](int idx) {
            const int kb = idx >> 4, v = idx & 15;
            float y = fmaf(S[kb][v], a.scale_log2, -l2r[v >> 2][v & 3]);
            if constexpr (ALIBI) y = fmaf(-sl_cur, fabsf(abase[kb] + (float)(8 * (v >> 2) + (v & 3))), y);
            float p = __builtin_amdgcn_exp2f(y);
            pin(p);
            S[kb][v] = p;
        };
        v8 oa = *(const v8 *)(ot + roff(0));
        v8 v0 = *(const v8 *)(vt + voff(0, 0));
        v8 v1 = *(const v8 *)(vt + voff(1, 0));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const v8 oc = oa, vc0 = v0, vc1 = v1;
            if (ks + 1 < KS) {
                oa = *(const v8 *)(ot + roff(ks + 1));
                v0 = *(const v8 *)(vt + voff(0, ks + 1));
                v1 = *(const v8 *)(vt + voff(1, ks + 1));
            }
            // 32 values over 2 KS matrix instructions
            constexpr int EPS = 16 / KS;
            static_assert(2 * KS * EPS == 32, "every probability gets a slot");
            copy_part(ks);
            P[0] = E::mfma(oc, vc0, P[0]);
#pragma unroll
            for (int e = 0; e < EPS; ++e) prob((ks * 2) * EPS + e);
            __builtin_amdgcn_sched_barrier(0);
            P[1] = E::mfma(oc, vc1, P[1]);
#pragma unroll
            for (int e = 0; e < EPS; ++e) prob((ks * 2 + 1) * EPS + e);
            __builtin_amdgcn_sched_barrier(0);
        }
        // bf16 probabilities: the dV operand
        v8 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = S[kb][half * 8 + e];
                pb[kb][half] = __builtin_convertvector(x, v8);
            }
        // dV^T += dO^T P over this wave's 32 rows, interleaved with
        // dS = P (dP - Dv) (in place in P)
        auto dsm = [&](int idx) {
            const int kb = idx >> 4, v = idx & 15;
            float d = S[kb][v] * (P[kb][v] - dvr[v >> 2][v & 3]);
            pin(d);
            P[kb][v] = d;
        };
        // dO^T operand of step (half, md), read one step ahead of its products
        auto oread = [&](int step) __attribute__((always_inline)) -> v8 {
            const int t4 = rh * 2 + step / MD, md = step % MD;
            const v4 ta = E::read_tr(ot + toff(md, 0) + t4 * 16 * ROWB);
            const v4 tb = E::read_tr(ot + toff(md, 1) + t4 * 16 * ROWB);
            return __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        v8 ofn = oread(0);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const v8 of = ofn;
                if (half * MD + md + 1 < 2 * MD) ofn = oread(half * MD + md + 1);
                // 32 values over 4 MD matrix instructions
                constexpr int EPD = 8 / MD;
                static_assert(4 * MD * EPD == 32, "every dS value gets a slot");
                const int sl = (half * MD + md) * 2;
                E::mfma_agpr(dva[md][0], of, pb[0][half]);
#pragma unroll
                for (int e = 0; e < EPD; ++e) dsm(sl * EPD + e);
                __builtin_amdgcn_sched_barrier(0);
                E::mfma_agpr(dva[md][1], of, pb[1][half]);
#pragma unroll
                for (int e = 0; e < EPD; ++e) dsm((sl + 1) * EPD + e);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        v8 db[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = P[kb][half * 8 + e];
                db[kb][half] = __builtin_convertvector(x, v8);
            }
        // dK^T += Q^T dS
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int t4 = rh * 2 + half;
            v8 qf[MD];
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const v4 ta = E::read_tr(qt + toff(md, 0) + t4 * 16 * ROWB);
                const v4 tb = E::read_tr(qt + toff(md, 1) + t4 * 16 * ROWB);
                qf[md] = __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) E::mfma_agpr(dka[md][kb], qf[md], db[kb][half]);
        }
    };

    if (total > 0) {
        copy_setup(true, 0, 0, 0);
#pragma unroll
        for (int part = 0; part < KS; ++part) copy_part(part);
        issue(0, 0);
        row_store(0);
        sl_cur = sl_next;
    }
    wait_vmem();
    __syncthreads();
    int ct = 0;          // query tile of step s
    int nt = 0, nh = 1;  // query tile and head offset of step s + 1
    if (nh == a.g) { nh = 0; nt = 1; }
    for (int s = 0; s < total; ++s) {
        const int slot = s & 1;
        const bool more = s + 1 < total;
        copy_setup(more, nt, nh, slot ^ 1);
        if (more) issue(nt, nh);
        const int r0 = tile_row(ct);
        step(slot, r0, tile_full(r0));
        if (more) row_store(slot ^ 1);  // the next step's slot is not read in this step
        sl_cur = sl_next;
        ct = nt;
        if (++nh == a.g) { nh = 0; ++nt; }
        wait_vmem();
        __syncthreads();
    }

#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mfma_agpr_drain(dka[md][kb]);
            mfma_agpr_drain(dva[md][kb]);
        }

    // epilogue: the waves of rows 32..63 hand their dK partials to the waves
    // of rows 0..31 through LDS (then the reverse for dV); lane (key n, half
    // h2) holds d = 32 md + 8 i + 4 h2 .. +4 of its keys' dK^T / dV^T columns
    f32x4 *xch = (f32x4 *)smem + (size_t)kh * (MD * 2 * 4 * 64);  // [md][kb][i][lane]
    auto put = [&](f32x16 (&acc)[MD][2]) {
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xch[((md * 2 + kb) * 4 + i) * 64 + lane] =
                        f32x4{acc[md][kb][i * 4], acc[md][kb][i * 4 + 1], acc[md][kb][i * 4 + 2], acc[md][kb][i * 4 + 3]};
    };
    auto finish = [&](f32x16 (&acc)[MD][2], void *dst, float mul) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!key_ok[kb]) continue;
            const size_t base = ((size_t)(k0 + keyv[kb]) * a.Hkv + c) * D;
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 o = xch[((md * 2 + kb) * 4 + i) * 64 + lane];
                    f32x4 x;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = (acc[md][kb][i * 4 + j] + o[j]) * mul;
                    const int d = md * 32 + i * 8 + h2 * 4;
                    *(u32x2 *)((uint16_t *)dst + base + d) = __builtin_bit_cast(u32x2, __builtin_convertvector(x, v4));
                }
        }
    };
    if (rh == 1) put(dka);
    __syncthreads();
    if (rh == 0) finish(dka, a.dk, a.scale);
    __syncthreads();
    if (rh == 0) put(dva);
    __syncthreads();
    if (rh == 1) finish(dva, a.dv, 1.f);
}

}  // namespace

hipError_t launch_sink_grad16(const void *dout, const void *out, const float *lse, const float *sinks, float *dsinks,
                              float *terms, bool f16, int head_dim, int total_q, int H, hipStream_t s)
{
    const int rows = total_q * H;
#define VA_SG(TT, DD)                                                                                       \
    hipLaunchKernelGGL((k_bwd_sink_terms<TT, DD>), dim3((rows + 256 / (DD / 8) - 1) / (256 / (DD / 8))), dim3(256), 0, \
                       s, (const uint16_t *)dout, (const uint16_t *)out, lse, sinks, terms, rows, H)
    if (f16) {
        if (head_dim == 128) VA_SG(_Float16, 128);
        else VA_SG(_Float16, 64);
    } else {
        if (head_dim == 128) VA_SG(__bf16, 128);
        else VA_SG(__bf16, 64);
    }
#undef VA_SG
    hipLaunchKernelGGL(k_bwd_sink_sum, dim3(H), dim3(256), 0, s, terms, dsinks, total_q, H);
    return hipGetLastError();
}

hipError_t launch_backward16(const BwdArgs &a, bool f16, bool alibi, int head_dim, int total_q, const int4 *q_items,
                             const int4 *q_seqinfo, const int32_t *q_count, int q_grid, const int4 *k_items,
                             const int4 *k_seqinfo, const int32_t *k_count, int k_grid, hipStream_t s)
{
    const int rows = total_q * a.H;
#define VA_BWD2(TT, DD, AA)                                                                              \
    do {                                                                                                 \
        hipLaunchKernelGGL((k_bwd_dq<TT, DD, AA>), dim3(q_grid), dim3(256), 0, s, a, q_items, q_seqinfo, q_count); \
        hipLaunchKernelGGL((k_bwd_dkdv<TT, DD, AA>), dim3(k_grid), dim3(256), 0, s, a, k_items, k_seqinfo, k_count); \
    } while (0)
#define VA_BWD(TT, DD)                                                                                   \
    do {                                                                                                 \
        hipLaunchKernelGGL((k_bwd_dot<TT, DD>), dim3((rows + 256 / (DD / 8) - 1) / (256 / (DD / 8))), dim3(256), 0, s, \
                           (const uint16_t *)a.dout, (const uint16_t *)a.out, a.dvec, rows);          \
        if (alibi) VA_BWD2(TT, DD, true);                                                                \
        else VA_BWD2(TT, DD, false);                                                                     \
    } while (0)
    if (f16) {
        if (head_dim == 128) VA_BWD(_Float16, 128);
        else VA_BWD(_Float16, 64);
    } else {
        if (head_dim == 128) VA_BWD(__bf16, 128);
        else VA_BWD(__bf16, 64);
    }
#undef VA_BWD
#undef VA_BWD2
    return hipGetLastError();
}

}  // namespace va
