// fp_device.h -- device helpers for the gfx950 kernels: bf16 conversions,
// realigning 16-byte loads, 16-byte stores to 2-byte-aligned addresses, and
// wave / workgroup reductions.
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

// A bf16 stream read as 8-byte quads from a base on any 2-byte boundary:
// the same branch-free scheme as Src16 below on an 8-byte grid (two aligned
// 8-byte loads, the second repeating the first when the base is aligned,
// then a byte funnel shift).
struct Src8 {
    const uint2* abase;  // aligned quad holding the base's first byte
    uint32_t ds;         // dwords to skip in the 16-byte window (0 or 1)
    uint32_t bs;         // then bytes to skip (0 or 2)
    uint32_t step;       // 1 if misaligned, else 0
};

__device__ __forceinline__ Src8 src8(const void* base) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(base);
    const uint32_t mis = static_cast<uint32_t>(a & 7u);
    Src8 r;
    r.abase = reinterpret_cast<const uint2*>(a - mis);
    r.ds = mis >> 2;
    r.bs = mis & 3u;
    r.step = mis != 0 ? 1u : 0u;
    return r;
}

// The 8 wanted bytes from the aligned quads lo (holding the first wanted
// byte) and hi (the next quad, or lo again when the base is aligned).
__device__ __forceinline__ uint2 realign8(const Src8& s, const uint2 lo, const uint2 hi) {
    const uint32_t w0 = s.ds ? lo.y : lo.x;
    const uint32_t w1 = s.ds ? hi.x : lo.y;
    const uint32_t w2 = s.ds ? hi.y : hi.x;
    return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, s.bs), __builtin_amdgcn_alignbyte(w2, w1, s.bs));
}

// 8 bytes to any 2-byte-aligned address, inside the 8 target bytes.
__device__ __forceinline__ void store8_any(void* p, const uint2 v) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if ((a & 7u) == 0) {
        const u32x2_t w = {v.x, v.y};
        *(FP_GLOBAL u32x2_t*)(p) = w;
    } else if ((a & 3u) == 0) {
        FP_GLOBAL uint32_t* q = (FP_GLOBAL uint32_t*)(p);
        q[0] = v.x; q[1] = v.y;
    } else {
        FP_GLOBAL uint16_t* q = (FP_GLOBAL uint16_t*)(p);
        q[0] = (uint16_t)v.x; q[1] = (uint16_t)(v.x >> 16);
        q[2] = (uint16_t)v.y; q[3] = (uint16_t)(v.y >> 16);
    }
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

// Word `word` (16 bytes at byte offset 16 * word from the base).
__device__ __forceinline__ uint4 ld16_realign(const Src16& s, int64_t word) {
    return realign16(s, ld16(s.abase + word), ld16(s.abase + word + s.step));
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

// 16 bytes starting at any 2-byte-aligned address.  A misaligned address is
// served by the two aligned 16-byte words that hold the wanted bytes (both
// hold at least one wanted byte, so neither leaves the mapped pages of the
// buffer) and a byte funnel shift (v_alignbyte_b32).
__device__ __forceinline__ uint4 load16_any(const void* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t mis = static_cast<uint32_t>(a & 15u);
    if (mis == 0) return *reinterpret_cast<const uint4*>(p);
    const uint4* base = reinterpret_cast<const uint4*>(a - mis);
    const uint4 lo = base[0];
    const uint4 hi = base[1];
    const uint32_t ds = mis >> 2;        // whole dwords to skip
    const uint32_t bs = mis & 3u;        // then bytes to skip
    uint32_t w0, w1, w2, w3, w4;
    if (ds == 0)      { w0 = lo.x; w1 = lo.y; w2 = lo.z; w3 = lo.w; w4 = hi.x; }
    else if (ds == 1) { w0 = lo.y; w1 = lo.z; w2 = lo.w; w3 = hi.x; w4 = hi.y; }
    else if (ds == 2) { w0 = lo.z; w1 = lo.w; w2 = hi.x; w3 = hi.y; w4 = hi.z; }
    else              { w0 = lo.w; w1 = hi.x; w2 = hi.y; w3 = hi.z; w4 = hi.w; }
    return make_uint4(__builtin_amdgcn_alignbyte(w1, w0, bs), __builtin_amdgcn_alignbyte(w2, w1, bs),
                      __builtin_amdgcn_alignbyte(w3, w2, bs), __builtin_amdgcn_alignbyte(w4, w3, bs));
}

// 16 bytes to any 2-byte-aligned address: one dwordx4 store when aligned,
// else four dword or eight short stores (all inside the 16 target bytes).
__device__ __forceinline__ void store16_any(void* p, const uint4 v) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if ((a & 15u) == 0) {
        *reinterpret_cast<uint4*>(p) = v;
    } else if ((a & 3u) == 0) {
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
        q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
    } else {
        uint16_t* q = reinterpret_cast<uint16_t*>(p);
        q[0] = (uint16_t)v.x; q[1] = (uint16_t)(v.x >> 16);
        q[2] = (uint16_t)v.y; q[3] = (uint16_t)(v.y >> 16);
        q[4] = (uint16_t)v.z; q[5] = (uint16_t)(v.z >> 16);
        q[6] = (uint16_t)v.w; q[7] = (uint16_t)(v.w >> 16);
    }
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

// Raise the overflow flag if any lane of the wave saw a non-finite value.
// The flag is only ever set to 1, so concurrent stores of 1 are benign.
__device__ __forceinline__ void flag_if_any(bool bad, int32_t* flag) {
    if (flag != nullptr && __ballot(bad) != 0ull && (threadIdx.x & 63) == 0) *flag = 1;
}

}  // namespace fpk
