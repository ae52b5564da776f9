// fp_device.h -- device helpers for the gfx950 kernels: bf16 conversions,
// non-temporal 8- and 16-byte loads and stores (aligned and on any 2-byte
// boundary), realigning 16-byte copies, and wave / workgroup reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp_internal.h"

namespace fpk {

// bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32 one.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (gfx950 converts two values with one
// v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo;
    const __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 w, float f[8]) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

__device__ __forceinline__ uint4 f32x8_to_bf16(const float f[8]) {
    return make_uint4(bf16x2(f[0], f[1]), bf16x2(f[2], f[3]),
                      bf16x2(f[4], f[5]), bf16x2(f[6], f[7]));
}

// Four bf16 values (8 bytes) <-> fp32.
__device__ __forceinline__ void bf16x4_to_f32(const uint2 w, float f[4]) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
}

__device__ __forceinline__ uint2 f32x4_to_bf16(const float f[4]) {
    return make_uint2(bf16x2(f[0], f[1]), bf16x2(f[2], f[3]));
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Every stream lives in global memory.  Saying so (address space 1) matters
// for pointers the kernels read from memory (the multi-unit records): the
// compiler would otherwise emit flat accesses, which also count against the
// scalar-load counter, so each wait for a pointer would wait for every
// stream load in flight as well.
#define FP_GLOBAL __attribute__((address_space(1)))

// Aligned 16-byte load / store with the non-temporal hint: every stream of
// the step is touched once per step, so it should not displace other data
// in the caches (measured ~8% faster than plain accesses on cold HBM).
__device__ __forceinline__ uint4 ld16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load((const FP_GLOBAL u32x4_t*)(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, const uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (FP_GLOBAL u32x4_t*)(p));
}

// 8-byte forms of the above, for bf16 quads.
__device__ __forceinline__ uint2 ld8(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load((const FP_GLOBAL u32x2_t*)(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st8(void* p, const uint2 v) {
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, (FP_GLOBAL u32x2_t*)(p));
}

// The same accesses at addresses on any 2-byte boundary (bf16 streams that
// start off their natural grid: gradient rows, copy sources, the own slice
// of the full buffer).  gfx950 runs with unaligned global access enabled, so
// one dwordx2 / dwordx4 instruction serves a misaligned address; the
// compiler emits the same instructions for a plain memcpy of 2-byte-aligned
// data.  The types only tell the compiler the true alignment.  Gradient
// quads read this way, measured on MI355X against realigning two aligned
// loads with a byte funnel shift: the 64-rank step with every gradient row 38
// elements past a cache line 2.95 ms instead of 3.19, the 8-rank d=1024
// layer's step with rows 3 elements off 20.8 us instead of 24.1.  Copies keep
// the realignment below, which measured faster for them.
typedef unsigned int u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef unsigned int u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));

__device__ __forceinline__ uint4 ld16u(const void* p) {
    const u32x4_a2 v = __builtin_nontemporal_load((const FP_GLOBAL u32x4_a2*)(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8u(const void* p) {
    const u32x2_a2 v = __builtin_nontemporal_load((const FP_GLOBAL u32x2_a2*)(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st8u(void* p, const uint2 v) {
    const u32x2_a2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, (FP_GLOBAL u32x2_a2*)(p));
}

// A bf16 stream read as 16-byte words from a base that may sit anywhere on a
// 2-byte boundary.  The shift is a property of the base (uniform across the
// wave), so the realignment is branch-free: two aligned loads -- the second
// one repeats the first when the base is aligned, so no load touches a word
// outside the stream -- and a byte funnel shift (v_alignbyte_b32).
struct Src16 {
    const uint4* abase;  // aligned word holding the base's first byte
    uint32_t ds;         // dwords to skip in the 32-byte window
    uint32_t bs;         // then bytes to skip
    uint32_t step;       // 1 if misaligned (second load needed), else 0
};

__device__ __forceinline__ Src16 src16(const void* base) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(base);
    const uint32_t mis = static_cast<uint32_t>(a & 15u);
    Src16 r;
    r.abase = reinterpret_cast<const uint4*>(a - mis);
    r.ds = mis >> 2;
    r.bs = mis & 3u;
    r.step = mis != 0 ? 1u : 0u;
    return r;
}

__device__ __forceinline__ uint32_t pick(uint32_t i, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : a3;
}

// The 16 wanted bytes from the aligned words lo (holding the first wanted
// byte) and hi (the next word, or lo again when the base is aligned).
__device__ __forceinline__ uint4 realign16(const Src16& s, const uint4 lo, const uint4 hi) {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const uint32_t d = s.ds;
    const uint32_t w0 = pick(d, w[0], w[1], w[2], w[3]);
    const uint32_t w1 = pick(d, w[1], w[2], w[3], w[4]);
    const uint32_t w2 = pick(d, w[2], w[3], w[4], w[5]);
    const uint32_t w3 = pick(d, w[3], w[4], w[5], w[6]);
    const uint32_t w4 = pick(d, w[4], w[5], w[6], w[7]);
    return make_uint4(__builtin_amdgcn_alignbyte(w1, w0, s.bs), __builtin_amdgcn_alignbyte(w2, w1, s.bs),
                      __builtin_amdgcn_alignbyte(w3, w2, s.bs), __builtin_amdgcn_alignbyte(w4, w3, s.bs));
}

// The value of the next lane of the wave (lane i receives lane i + 1's;
// lane 63 receives `fallback`): a wave-shift DPP move, no memory access.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v, uint32_t fallback) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fallback, (int)v, 0x130 /* wave_shl:1 */, 0xF,
                                                 0xF, false);
}
__device__ __forceinline__ uint4 from_next_lane(const uint4 v, const uint4 fallback) {
    return make_uint4(from_next_lane(v.x, fallback.x), from_next_lane(v.y, fallback.y),
                      from_next_lane(v.z, fallback.z), from_next_lane(v.w, fallback.w));
}

__device__ __forceinline__ bool finite_f32(float x) {
    return (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u;
}

// Sum over the 64 lanes of a wave (butterfly; the same tree every call).
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over the workgroup in a fixed order; the result is valid in thread 0.
__device__ __forceinline__ double group_sum(double x) {
    __shared__ double lds[kWaves];
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = x;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) r += lds[w];
    }
    return r;
}

// OR bits into the overflow flag (a vector atomic): the flag is never
// cleared by a kernel, so bits set by earlier calls survive.
__device__ __forceinline__ void flag_or(int32_t* flag, int32_t bits) {
    __hip_atomic_fetch_or(flag, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raise the overflow flag (bit 0) if any lane of the wave saw a non-finite
// value: one atomic OR per wave, only on overflow.
__device__ __forceinline__ void flag_if_any(bool bad, int32_t* flag) {
    if (flag != nullptr && __ballot(bad) != 0ull && (threadIdx.x & 63) == 0) flag_or(flag, 1);
}

}  // namespace fpk
