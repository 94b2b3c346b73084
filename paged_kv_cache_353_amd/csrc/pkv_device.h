// Device helpers shared by the decode kernels: element types, lane exchange,
// MFMA steps over 16-byte chunks, conversions, buffer loads and the coherent
// accesses partial results travel through.  Included by .hip sources only.
#pragma once

#include "pkv_internal.h"

#include <type_traits>

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr uint32_t kBufferFlags = 0x00020000u;  // gfx9 buffer descriptor word 3 (32-bit data)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Block Table and length reads go through the constant address space so they
// become scalar loads (their addresses are wave-uniform).
typedef const int32_t __attribute__((address_space(4))) *const_i32_ptr;

struct F32 { static constexpr int kBytes = 4; };
struct F16 { static constexpr int kBytes = 2; };
struct BF16 { static constexpr int kBytes = 2; };

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f.template operator()<I>();
        static_for<I + 1, N>(f);
    }
}
// f<I>(), f<I + 1>(), ... f<N - 1>() until one returns true; returns whether
// one did.  A loop `while (!static_any<0, N>(step))` leaves straight from the
// step that ends it, so its back edge is reached only after all N steps.
template <int I, int N, typename F>
__device__ __forceinline__ bool static_any(F &&f) {
    if constexpr (I < N) {
        if (f.template operator()<I>()) return true;
        return static_any<I + 1, N>(f);
    } else {
        return false;
    }
}

// Element reinterpretation goes through by-value helpers: hipcc (clang 22)
// miscompiles __builtin_bit_cast applied directly to an ext-vector element
// (it reads element 0 whatever the index).
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// Values the compiler cannot prove wave-uniform are pinned to scalar
// registers; a buffer descriptor built from a per-lane value would be
// wrapped in a waterfall loop around every load.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
    const uint64_t v = (uint64_t)x;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------ lane exchange
// Lane n of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}
// Lane n of each row broadcast to the row, taking `hi` in lanes 8..15 and
// `lo` in lanes 0..7 (the bank mask leaves banks 0 and 1 unwritten).
template <int N>
__device__ __forceinline__ float row_bcast_split(float lo, float hi) {
    const int l = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, lo), 0x150 + N, 0xF, 0xF, false);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        l, __builtin_bit_cast(int, hi), 0x150 + N, 0xF, 0xC, false));
}
// Lane c <-> c+8 (mod 16) inside each row (DPP row_ror:8).
__device__ __forceinline__ float row_ror8(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}
// floor(num / den) for 0 <= num < 2^52 and 0 < den < 2^52, given inv_den =
// 1.0 / den: the fp64 product is within one of the quotient, and one exact
// integer correction each way makes it exact (no 64-bit integer division).
__device__ __forceinline__ int64_t floor_div(int64_t num, int64_t den, double inv_den) {
    int64_t q = (int64_t)((double)num * inv_den);
    if (q * den > num) --q;
    else if ((q + 1) * den <= num) ++q;
    return q;
}

// Lane swaps between 16-lane rows (gfx950 VALU instructions, no LDS).
// swap_rows16(a, b): rows 1 and 3 of a trade places with rows 0 and 2 of b,
// so that with a == b == x afterwards a holds x of rows 0, 0, 2, 2 and b x of
// rows 1, 1, 3, 3.  swap_rows32(a, b): the upper half of a trades with the
// lower half of b (a: x of the lower half everywhere, b: of the upper).
// The leading s_nop covers the wait a VALU write needs before these read it.
__device__ __forceinline__ void swap_rows16(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows32(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// x summed over lanes l, l ^ 16, l ^ 32 and l ^ 48, as (r0 + r1) + (r2 + r3)
// of the four rows, in every lane.
__device__ __forceinline__ float rows_sum4(float x) {
    float a = x, b = x;
    swap_rows16(a, b);
    float c = a + b, d = c;
    swap_rows32(c, d);
    return c + d;
}
// Four values reduced over the four rows at once: afterwards row r holds the
// sum, over the rows, of the r-th argument, as (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float rows_scatter_sum4(float x, float y, float z, float w) {
    swap_rows16(x, y);   // x: x0, y0, x2, y2 by rows; y: x1, y1, x3, y3
    float s1 = x + y;    // rows 0..3: x0+x1, y0+y1, x2+x3, y2+y3
    swap_rows16(z, w);
    float s2 = z + w;    // rows 0..3: z0+z1, w0+w1, z2+z3, w2+w3
    swap_rows32(s1, s2);
    return s1 + s2;      // rows 0..3: x, y, z, w summed over the rows
}
__device__ __forceinline__ float rows_max4(float x) {
    float a = x, b = x;
    swap_rows16(a, b);
    float c = fmaxf(a, b), d = c;
    swap_rows32(c, d);
    return fmaxf(c, d);
}
__device__ __forceinline__ float xor16(float x) {  // lane ^ 16
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ float xor32(float x, int lane) {  // lane ^ 32
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ int wave_sum_i(int x, int lane) {
    for (int d = 1; d < kWave; d <<= 1) x += __builtin_amdgcn_ds_bpermute((lane ^ d) << 2, x);
    return x;
}
// Inclusive prefix sum over the wave with DPP: shifts by 1, 2, 4 and 8 inside
// each 16-lane row, then lane 15 of each row into the next row and lane 31
// into rows 2 and 3 (lanes without a source add the 0 given as `old`).
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
    (void)lane;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// ------------------------------------------------------------------ element types
// One MFMA step over a 16-byte chunk of K rows (A, 16 tokens) and of q (B, 16 heads).
template <typename DT>
__device__ __forceinline__ f32x4 mfma_chunk(const u32x4 &k, const u32x4 &q, f32x4 c) {
    if constexpr (std::is_same_v<DT, BF16>) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                        __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
    } else if constexpr (std::is_same_v<DT, F16>) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                       __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
    } else {
        static_for<0, 4>([&]<int i>() {
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(k[i]), as_f(q[i]), c, 0, 0, 0);
        });
        return c;
    }
}

template <typename DT>
__device__ __forceinline__ void chunk_to_f32(const u32x4 &v, float (&f)[16 / DT::kBytes]) {
    if constexpr (std::is_same_v<DT, BF16>) {
        static_for<0, 4>([&]<int i>() {
            f[2 * i] = as_f(v[i] << 16);
            f[2 * i + 1] = as_f(v[i] & 0xFFFF0000u);
        });
    } else if constexpr (std::is_same_v<DT, F16>) {
        static_for<0, 4>([&]<int i>() {
            const f16x2 h = as_h2(v[i]);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        });
    } else {
        static_for<0, 4>([&]<int i>() { f[i] = as_f(v[i]); });
    }
}

// Round-to-nearest-even conversion of one 16-byte chunk of output elements.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    const uint32_t u = as_u(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
template <typename DT>
__device__ __forceinline__ u32x4 pack_chunk(const float (&f)[16 / DT::kBytes]) {
    u32x4 r;
    if constexpr (std::is_same_v<DT, BF16>) {
        static_for<0, 4>([&]<int i>() { r[i] = bf16_rne(f[2 * i]) | (bf16_rne(f[2 * i + 1]) << 16); });
    } else if constexpr (std::is_same_v<DT, F16>) {
        static_for<0, 4>([&]<int i>() {
            f16x2 h;
            h[0] = (_Float16)f[2 * i];
            h[1] = (_Float16)f[2 * i + 1];
            r[i] = __builtin_bit_cast(uint32_t, h);
        });
    } else {
        static_for<0, 4>([&]<int i>() { r[i] = as_u(f[i]); });
    }
    return r;
}

__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
// Streaming read of K/V rows: the non-temporal policy bit (nt) marks the lines
// as read once, so they do not displace what the caches hold for other data.
// Measured on the Llama-8B-shaped batch it raised the delivered rate by ~10%.
constexpr int kStreamNT = 2;
__device__ __forceinline__ u32x4 load_stream(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kStreamNT);
}

// Partial results pass between waves that may sit on different XCDs, whose
// L2 caches are not coherent with each other for ordinary accesses.  They are
// written and read with the agent-coherence cache policy (sc1), the encoding
// of relaxed agent-scope atomic accesses, so that every access is coherent on
// its own and no whole-cache writeback or invalidate is needed.  The writer
// waits for its stores to complete before it bumps the arrival counter; the
// last arriver reads only after the counter told it so.
constexpr int kCoherentSC1 = 16;  // buffer cache-policy bit sc1
__device__ __forceinline__ void store_coherent(float *base, int bytes, int byte_off, const f32x4 &v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCoherentSC1);
}
__device__ __forceinline__ f32x4 load_coherent(const float *base, int bytes, int byte_off) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kBufferFlags);
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherentSC1));
}
__device__ __forceinline__ void store_coherent_f32(float *base, int bytes, int byte_off, float v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b32(as_u(v), r, byte_off, 0, kCoherentSC1);
}
// Plain 16-byte store through a buffer descriptor (outputs, cache slots).
__device__ __forceinline__ void store_chunk(void *base, int bytes, int byte_off, const u32x4 &v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}
// Plain 8- and 4-byte stores through a buffer descriptor.
__device__ __forceinline__ void store_b64(void *base, int bytes, int byte_off, uint32_t lo, uint32_t hi) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, r, byte_off, 0, 0);
}
__device__ __forceinline__ void store_b32(void *base, int bytes, int byte_off, uint32_t v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b32(v, r, byte_off, 0, 0);
}
// Relaxed agent-scope atomic add that returns the previous value, issued as
// a buffer instruction: the compiler then counts it in order with the
// stream's buffer loads, so it may stay in flight while they go on (a global
// atomic with return in flight makes every later wait a full drain).
__device__ __forceinline__ int atomic_add_counter(int32_t *ctr, int v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(ctr, 0, 4, kBufferFlags);
    return __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(v, r, 0, 0, 0);
}
__device__ __forceinline__ void store_counter(int32_t *ctr, int v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(ctr, 0, 4, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, 0, 0, kCoherentSC1);
}
__device__ __forceinline__ float load_coherent_f32(const float *base, int bytes, int byte_off) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kBufferFlags);
    return as_f(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCoherentSC1));
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum): every vector
// memory access issued so far has completed.  The empty asm with a memory
// clobber keeps the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void wait_vmem_done() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace pkv
