// step_kernels.hip -- gfx950 kernels of the per-step path: reduce, AdamW with
// the bf16 cast, unshard, and the shard step's first phase.
//
// Every kernel is a grid-stride stream over 8-element chunks: each lane
// moves one 16-byte word per bf16 stream and two per fp32 stream, so every
// HBM access is a 128-bit (dwordx4) load or store and a wave touches 1 KiB
// (bf16) or 2 KiB (fp32) of contiguous memory per access.  Elements past
// the last whole chunk are handled one by one by workgroup 0.  Nothing here
// is a contraction, so there is no MFMA; the kernels are bound by HBM.
//
// Compiled with -ffp-contract=off: every fp32 / fp64 operation below is one
// IEEE round-to-nearest-even operation, in the order written.

#include "fp_device.h"

namespace fpk {

// ---------------------------------------------------------------- reduce
// Ascending-rank fp32 sum of the ranks' bf16 gradients at chunk j0.  The
// 8 loads of a rank group are issued before any add so that each lane has
// 128 bytes in flight.  "Infra: Data Parallel", ZeRO-1/ZeRO-2 paragraphs
// (reduce-scatter with averaging); "4.1 数据并行详解" section 2 (average of
// the local gradients).
template <class A>
__device__ __forceinline__ void sum_ranks8(const A& a, int64_t j0, float s[8]) {
    const int world = a.world;
    for (int q0 = 0; q0 < world; q0 += 8) {
        uint4 w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (q0 + k < world) w[k] = load16_any(a.grads[q0 + k] + j0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (q0 + k < world) {
                float f[8];
                bf16x8_to_f32(w[k], f);
                if (q0 + k == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] = f[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] = s[e] + f[e];
                }
            }
        }
    }
}

template <class A>
__device__ __forceinline__ float sum_ranks1(const A& a, int64_t j) {
    float s = bf16_lo(a.grads[0][j]);
    for (int q = 1; q < a.world; ++q) s = s + bf16_lo(a.grads[q][j]);
    return s;
}

__device__ __forceinline__ void load_f32x8(const float* p, float f[8]) {
    const float4 u = reinterpret_cast<const float4*>(p)[0];
    const float4 v = reinterpret_cast<const float4*>(p)[1];
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
    f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
}

__device__ __forceinline__ void store_f32x8(float* p, const float f[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// ---------------------------------------------------------------- AdamW
// One element of decoupled-weight-decay AdamW with bias correction,
// evaluated in fp64 in the order of its definition; master, exp_avg and
// exp_avg_sq are each rounded once to fp32.  "Infra: Data Parallel", ZeRO-1
// paragraph (elementwise update of the rank's slice) and ZeRO figure legend
// (fp32 master and moments, k = 12).
__device__ __forceinline__ void adamw_elem(const AdamCoef& c, float g, float& th, float& m,
                                           float& v) {
    const double gd = (double)g;
    double theta = (double)th;
    double md = (double)m;
    double vd = (double)v;
    theta = theta * c.decay;
    md = c.beta1 * md + c.one_m_beta1 * gd;
    vd = c.beta2 * vd + c.one_m_beta2 * gd * gd;
    const double m_hat = md / c.bias1;
    const double v_hat = vd / c.bias2;
    theta = theta - c.lr * m_hat / (sqrt(v_hat) + c.eps);
    th = (float)theta;
    m = (float)md;
    v = (float)vd;
}

// ---------------------------------------------------------------- unshard
// Shard q occupies full[qS, (q+1)S).  Its interior 16-byte words of `full`
// are copied with one aligned store each (the source word is realigned when
// qS is not a multiple of 8); the at most 14 edge elements that share a
// word with a neighbouring shard are copied one by one.
struct ShardSpan {
    int64_t lo, a, b, hi;  // [lo, a) head, [a, b) whole words, [b, hi) tail
};

__device__ __forceinline__ ShardSpan shard_span(const uint16_t* full, int64_t S, int q) {
    // element index e is 16-byte aligned in `full` when e % 8 == phase
    const int64_t phase = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(full) & 15u)) & 15u) >> 1);
    ShardSpan s;
    s.lo = (int64_t)q * S;
    s.hi = s.lo + S;
    const int64_t up = s.lo + (((phase - s.lo) % 8) + 8) % 8;         // first aligned >= lo
    s.a = up < s.hi ? up : s.hi;
    const int64_t down = s.hi - (((s.hi - phase) % 8) + 8) % 8;       // last aligned <= hi
    s.b = down > s.a ? down : s.a;
    return s;
}

__device__ __forceinline__ void unshard_words(const uint16_t* src, uint16_t* full, int64_t S, int q,
                                              int64_t t, int64_t stride) {
    const ShardSpan sp = shard_span(full, S, q);
    const int64_t n_words = (sp.b - sp.a) >> 3;
    for (int64_t w = t; w < n_words; w += stride) {
        const int64_t e0 = sp.a + (w << 3);
        *reinterpret_cast<uint4*>(full + e0) = load16_any(src + (e0 - sp.lo));
    }
}

__device__ __forceinline__ void unshard_edges(const uint16_t* src, uint16_t* full, int64_t S, int q,
                                              int t, int stride) {
    const ShardSpan sp = shard_span(full, S, q);
    const int64_t n_head = sp.a - sp.lo;
    const int64_t n_edge = n_head + (sp.hi - sp.b);
    for (int64_t k = t; k < n_edge; k += stride) {
        const int64_t e = k < n_head ? sp.lo + k : sp.b + (k - n_head);
        full[e] = src[e - sp.lo];
    }
}

// ---------------------------------------------------------------- kernels

template <bool kAccumulate, bool kNorm>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const ReduceArgs a) {
    const int64_t n_chunks = a.shard >> 3;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    bool bad = false;
    double sq = 0.0;
    for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < n_chunks; c += stride) {
        const int64_t j0 = c << 3;
        float y[8];
        sum_ranks8(a, j0, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = y[e] * a.scale;
        if (kAccumulate) {
            float p[8];
            load_f32x8(a.acc + j0, p);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = p[e] + y[e];
        }
        store_f32x8(a.acc + j0, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bad |= !finite_f32(y[e]);
            if (kNorm) sq += (double)y[e] * (double)y[e];
        }
    }
    const int64_t tail0 = n_chunks << 3;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        float y = sum_ranks1(a, j) * a.scale;
        if (kAccumulate) y = a.acc[j] + y;
        a.acc[j] = y;
        bad |= !finite_f32(y);
        if (kNorm) sq += (double)y * (double)y;
    }
    flag_if_any(bad, a.found_inf);
    if (kNorm) {
        const double t = group_sum(sq);
        if (threadIdx.x == 0) a.partials[blockIdx.x] = t;
    }
}

// Sums the per-workgroup partials in a fixed order (one workgroup).
__device__ __forceinline__ void finalize_norm(const double* partials, int n, double* out) {
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += kThreads) s += partials[i];
    const double t = group_sum(s);
    if (threadIdx.x == 0) *out = t;
}

__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(const double* partials, int n,
                                                                 double* out) {
    finalize_norm(partials, n, out);
}

__global__ __launch_bounds__(kThreads) void adamw_kernel(const AdamArgs a) {
    if (a.sq_norm != nullptr && blockIdx.x == 0) finalize_norm(a.partials, a.n_partials, a.sq_norm);
    const bool skip = a.found_inf != nullptr && *a.found_inf != 0;
    const int64_t n_chunks = a.shard >> 3;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < n_chunks; c += stride) {
        const int64_t j0 = c << 3;
        float th[8];
        load_f32x8(a.master + j0, th);
        if (!skip) {
            float g[8], m[8], v[8];
            load_f32x8(a.grad + j0, g);
            load_f32x8(a.exp_avg + j0, m);
            load_f32x8(a.exp_avg_sq + j0, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) adamw_elem(a.c, g[e], th[e], m[e], v[e]);
            store_f32x8(a.master + j0, th);
            store_f32x8(a.exp_avg + j0, m);
            store_f32x8(a.exp_avg_sq + j0, v);
        }
        if (a.param_bf16 != nullptr) store16_any(a.param_bf16 + j0, f32x8_to_bf16(th));
    }
    const int64_t tail0 = n_chunks << 3;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        float th = a.master[j];
        if (!skip) {
            float m = a.exp_avg[j], v = a.exp_avg_sq[j];
            adamw_elem(a.c, a.grad[j], th, m, v);
            a.master[j] = th;
            a.exp_avg[j] = m;
            a.exp_avg_sq[j] = v;
        }
        if (a.param_bf16 != nullptr) a.param_bf16[j] = (uint16_t)bf16x2(th, 0.0f);
    }
}

__global__ __launch_bounds__(kThreads) void unshard_kernel(const UnshardArgs a) {
    const int q = blockIdx.y;
    const uint16_t* src = a.shards[q];
    if (src == nullptr) return;
    unshard_words(src, a.full, a.shard, q, (int64_t)blockIdx.x * kThreads + threadIdx.x,
                  (int64_t)gridDim.x * kThreads);
    if (blockIdx.x == 0) unshard_edges(src, a.full, a.shard, q, threadIdx.x, kThreads);
}

// First phase of the shard step.  kFused = false: reduce into acc (the
// AdamW phase follows once the overflow flag of the whole shard is known).
// kFused = true: reduce, AdamW and the bf16 cast in one pass, no gate.
template <bool kFused>
__global__ __launch_bounds__(kThreads) void step_phase1_kernel(const StepArgs a) {
    if ((int)blockIdx.x < a.reduce_groups) {
        const int64_t n_chunks = a.shard >> 3;
        const int64_t stride = (int64_t)a.reduce_groups * kThreads;
        uint16_t* own = a.full + (int64_t)a.rank * a.shard;
        bool bad = false;
        double sq = 0.0;
        const bool want_sq = a.partials != nullptr;
        for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < n_chunks; c += stride) {
            const int64_t j0 = c << 3;
            float y[8];
            sum_ranks8(a, j0, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = y[e] * a.scale;
            if (a.accumulate) {
                float p[8];
                load_f32x8(a.acc + j0, p);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = p[e] + y[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bad |= !finite_f32(y[e]);
                if (want_sq) sq += (double)y[e] * (double)y[e];
            }
            if (!kFused || a.keep_grad) store_f32x8(a.acc + j0, y);
            if (kFused) {
                float th[8], m[8], v[8];
                load_f32x8(a.master + j0, th);
                load_f32x8(a.exp_avg + j0, m);
                load_f32x8(a.exp_avg_sq + j0, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) adamw_elem(a.c, y[e], th[e], m[e], v[e]);
                store_f32x8(a.master + j0, th);
                store_f32x8(a.exp_avg + j0, m);
                store_f32x8(a.exp_avg_sq + j0, v);
                store16_any(own + j0, f32x8_to_bf16(th));
            }
        }
        const int64_t tail0 = n_chunks << 3;
        if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
            const int64_t j = tail0 + threadIdx.x;
            float y = sum_ranks1(a, j) * a.scale;
            if (a.accumulate) y = a.acc[j] + y;
            bad |= !finite_f32(y);
            if (want_sq) sq += (double)y * (double)y;
            if (!kFused || a.keep_grad) a.acc[j] = y;
            if (kFused) {
                float th = a.master[j], m = a.exp_avg[j], v = a.exp_avg_sq[j];
                adamw_elem(a.c, y, th, m, v);
                a.master[j] = th;
                a.exp_avg[j] = m;
                a.exp_avg_sq[j] = v;
                own[j] = (uint16_t)bf16x2(th, 0.0f);
            }
        }
        flag_if_any(bad, a.found_inf);
        if (want_sq) {
            const double t = group_sum(sq);
            if (threadIdx.x == 0) a.partials[blockIdx.x] = t;
        }
    } else {
        const int u = (int)blockIdx.x - a.reduce_groups;
        const int n_u = (int)gridDim.x - a.reduce_groups;
        for (int q = 0; q < a.world; ++q) {
            const uint16_t* src = a.shards[q];
            if (src == nullptr) continue;
            unshard_words(src, a.full, a.shard, q, (int64_t)u * kThreads + threadIdx.x,
                          (int64_t)n_u * kThreads);
            if (u == 0) unshard_edges(src, a.full, a.shard, q, threadIdx.x, kThreads);
        }
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_reduce(const ReduceArgs& a, int grid, hipStream_t s) {
    const bool norm = a.partials != nullptr;
    if (a.accumulate) {
        if (norm) reduce_kernel<true, true><<<grid, kThreads, 0, s>>>(a);
        else reduce_kernel<true, false><<<grid, kThreads, 0, s>>>(a);
    } else {
        if (norm) reduce_kernel<false, true><<<grid, kThreads, 0, s>>>(a);
        else reduce_kernel<false, false><<<grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_norm_finalize(const double* partials, int n, double* out, hipStream_t s) {
    norm_finalize_kernel<<<1, kThreads, 0, s>>>(partials, n, out);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamArgs& a, int grid, hipStream_t s) {
    adamw_kernel<<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_unshard(const UnshardArgs& a, int grid_x, hipStream_t s) {
    unshard_kernel<<<dim3(grid_x, a.world), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_step_phase1(const StepArgs& a, int grid, bool fused_update, hipStream_t s) {
    if (fused_update) step_phase1_kernel<true><<<grid, kThreads, 0, s>>>(a);
    else step_phase1_kernel<false><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
