// local_kernels.hip -- the steps on either side of the reduce.
//
// Accumulation without communication ("Infra: Data Parallel", section
// "Naive Data Parallelism", gradient-accumulation paragraph; "PyTorch FSDP
// ...", section 3.4): a rank adds the bf16 gradients of its first
// micro-batches into an fp32 buffer over its whole unit, in micro-batch
// order, and on the last micro-batch rounds the sum (with that micro-batch's
// gradient) once to bf16, the row it contributes to the reduce-scatter.
// Both are elementwise streams in the quad layout of the step kernels.
//
// The consumers of the overflow flag and of the gradient norm ("PyTorch
// FSDP ...", section 3.5, sharded gradient scaler; the policy is not on the
// pages): one-lane kernels that turn the loss scale and the reduced
// gradient's sum of squares into the fp64 factor AdamW applies to the
// gradient (unscale, then clip to a global norm), and that advance the
// dynamic loss scale after a step's overflow decision.

#include "fp_extra.h"
#include "step_ops.h"

namespace fpk {

// local = (accumulate ? local : 0) + f32(grad), fp32, one rounding.
template <bool kAligned, bool kAcc>
__global__ __launch_bounds__(kThreads) void local_accumulate_kernel(const LocalArgs a) {
    constexpr int kU = kQuadsPerLane;
    const int64_t tile = blockIdx.x;
    const int64_t nq = a.n >> 2;
    if (nq > 0) {
        const Quads<kU> Q = lane_quads<kU>(tile, nq);
        uint2 g[kU];
        float l[kU][4];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            g[u] = ld_bf16q<kAligned>(a.grad, Q, u);
            if (kAcc) ld_f32q(a.local, Q, u, l[u]);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float f[4];
            bf16x4_to_f32(g[u], f);
#pragma unroll
            for (int e = 0; e < 4; ++e) l[u][e] = kAcc ? l[u][e] + f[e] : f[e];
            if (Q.ok[u]) st_f32q(a.local, Q, u, l[u]);
        }
    }
    const int64_t tail0 = nq << 2;
    if (tile == 0 && (int64_t)threadIdx.x < a.n - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        const float g = bf16_lo(a.grad[j]);
        a.local[j] = kAcc ? a.local[j] + g : g;
    }
}

// out = bf16(accumulate ? local + f32(grad) : f32(grad)), round to nearest even.
template <bool kAligned, bool kAcc>
__global__ __launch_bounds__(kThreads) void local_finish_kernel(const LocalArgs a) {
    constexpr int kU = kQuadsPerLane;
    const int64_t tile = blockIdx.x;
    const int64_t nq = a.n >> 2;
    if (nq > 0) {
        const Quads<kU> Q = lane_quads<kU>(tile, nq);
        uint2 g[kU];
        float l[kU][4];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            g[u] = ld_bf16q<kAligned>(a.grad, Q, u);
            if (kAcc) ld_f32q(a.local, Q, u, l[u]);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            float f[4];
            bf16x4_to_f32(g[u], f);
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = kAcc ? l[u][e] + f[e] : f[e];
            if (Q.ok[u]) st_bf16q<kAligned>(a.out, Q, u, f32x4_to_bf16(f));
        }
    }
    const int64_t tail0 = nq << 2;
    if (tile == 0 && (int64_t)threadIdx.x < a.n - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        const float g = bf16_lo(a.grad[j]);
        a.out[j] = (uint16_t)bf16x2(kAcc ? a.local[j] + g : g, 0.0f);
    }
}

// The fp64 factor of the loss-scaled reduced gradient: 1 / scale, times
// min(1, max_norm / (||g|| + 1e-6)) with ||g|| = sqrt(sq_norm) / scale when
// max_norm > 0.  One lane.
__global__ void grad_coef_kernel(const double* sq_norm, const float* loss_scale, double max_norm,
                                 double* coef) {
    if (threadIdx.x != 0) return;
    const double inv = 1.0 / (double)(loss_scale != nullptr ? *loss_scale : 1.0f);
    double k = inv;
    if (max_norm > 0.0) {
        const double norm = sqrt(*sq_norm) * inv;
        const double clip = max_norm / (norm + 1e-6);
        if (clip < 1.0) k = inv * clip;
    }
    *coef = k;
}

// Dynamic loss scaling after one step: an overflow multiplies the scale by
// the backoff factor and restarts the count of clean steps; growth_interval
// clean steps in a row multiply it by the growth factor.  One lane.
__global__ void scaler_update_kernel(const int32_t* found_inf, float* scale, int32_t* clean_steps,
                                     float growth_factor, float backoff_factor, int32_t growth_interval) {
    if (threadIdx.x != 0) return;
    if (*found_inf != 0) {
        *scale = *scale * backoff_factor;
        *clean_steps = 0;
        return;
    }
    const int32_t c = *clean_steps + 1;
    if (c == growth_interval) {
        *scale = *scale * growth_factor;
        *clean_steps = 0;
    } else {
        *clean_steps = c;
    }
}

hipError_t launch_local(const LocalArgs& a, bool finish, bool accumulate, bool aligned, hipStream_t s) {
    const int64_t t = tiles_of(a.n >> 2);
    const unsigned grid = (unsigned)(t > 0 ? t : 1);
    if (finish) {
        if (aligned) {
            if (accumulate) local_finish_kernel<true, true><<<grid, kThreads, 0, s>>>(a);
            else local_finish_kernel<true, false><<<grid, kThreads, 0, s>>>(a);
        } else {
            if (accumulate) local_finish_kernel<false, true><<<grid, kThreads, 0, s>>>(a);
            else local_finish_kernel<false, false><<<grid, kThreads, 0, s>>>(a);
        }
    } else {
        if (aligned) {
            if (accumulate) local_accumulate_kernel<true, true><<<grid, kThreads, 0, s>>>(a);
            else local_accumulate_kernel<true, false><<<grid, kThreads, 0, s>>>(a);
        } else {
            if (accumulate) local_accumulate_kernel<false, true><<<grid, kThreads, 0, s>>>(a);
            else local_accumulate_kernel<false, false><<<grid, kThreads, 0, s>>>(a);
        }
    }
    return hipGetLastError();
}

hipError_t launch_grad_coef(const double* sq_norm, const float* loss_scale, double max_norm, double* coef,
                            hipStream_t s) {
    grad_coef_kernel<<<1, 64, 0, s>>>(sq_norm, loss_scale, max_norm, coef);
    return hipGetLastError();
}

hipError_t launch_scaler_update(const int32_t* found_inf, float* scale, int32_t* clean_steps,
                                float growth_factor, float backoff_factor, int32_t growth_interval,
                                hipStream_t s) {
    scaler_update_kernel<<<1, 64, 0, s>>>(found_inf, scale, clean_steps, growth_factor, backoff_factor,
                                          growth_interval);
    return hipGetLastError();
}

}  // namespace fpk
