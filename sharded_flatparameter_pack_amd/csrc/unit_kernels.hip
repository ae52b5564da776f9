// unit_kernels.hip -- the per-step kernels over many units in one launch:
// e.g. the DDP buckets of a model, whose shards make up one rank's fp32
// partition ("Infra: Data Parallel", ZeRO-1/ZeRO-2 paragraphs: each rank
// keeps one slice of the whole optimizer state; "4.1 数据并行详解",
// section 4.2: gradients are reduced bucket by bucket).  Each workgroup
// finds its unit by a binary search over the plan's tile prefix table
// (scalar loads, cached), then runs the same tile bodies as the single-unit
// kernels on that unit's pointers.

#include "step_ops.h"

namespace fpk {

namespace {

// The unit whose workgroup range holds idx: the last u with
// start[u] <= idx (start ascending, start[0] = 0, idx < start[n]).
__device__ __forceinline__ int find_unit(const int64_t* start, int n, int64_t idx) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= idx) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// One unit as the tile bodies see it.
struct UnitView {
    const uint16_t* const* grads;
    const uint16_t* const* shards;
    uint16_t* full;
    float* acc;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    int64_t shard;
    AdamCoef c;
    float scale;
    int32_t world;
    int32_t rank;
    int32_t copy_tiles;
};

__device__ __forceinline__ UnitView unit_view(const UnitsArgs& a, int u) {
    const UnitDesc& d = a.units[u];
    UnitView v;
    v.grads = d.grads;
    v.shards = d.shards;
    v.full = d.full;
    v.acc = a.acc + d.offset;
    v.master = a.master + d.offset;
    v.exp_avg = a.exp_avg + d.offset;
    v.exp_avg_sq = a.exp_avg_sq + d.offset;
    v.shard = d.shard;
    v.c = a.c;
    v.scale = a.scale;
    v.world = a.world;
    v.rank = a.rank;
    v.copy_tiles = d.copy_tiles;
    return v;
}

__device__ __forceinline__ uint16_t* own_slice(const UnitView& v) {
    return v.full != nullptr ? v.full + (int64_t)v.rank * v.shard : nullptr;
}

}  // namespace

template <bool kAligned, bool kAccumulate, bool kNorm>
__global__ __launch_bounds__(kThreads) void units_reduce_kernel(const UnitsArgs a) {
    const int u = find_unit(a.tile_start, a.n_units, blockIdx.x);
    const UnitView v = unit_view(a, u);
    reduce_tile<kAligned, kAccumulate, kNorm>(v, (int64_t)blockIdx.x - a.tile_start[u], a.found_inf,
                                              kNorm ? a.partials + blockIdx.x : nullptr);
}

template <bool kAligned, bool kFused>
__global__ __launch_bounds__(kThreads) void units_phase1_kernel(const UnitsArgs a) {
    if ((int64_t)blockIdx.x >= a.reduce_groups) {
        const int64_t idx = (int64_t)blockIdx.x - a.reduce_groups;
        const int u = find_unit(a.copy_start, a.n_units, idx);
        const UnitView v = unit_view(a, u);
        copy_role<kAligned, kCopyWordsStream>(v, (unsigned)(idx - a.copy_start[u]));
        return;
    }
    const int u = find_unit(a.tile_start, a.n_units, blockIdx.x);
    const UnitView v = unit_view(a, u);
    step_reduce_tile<kAligned, kFused>(v, (int64_t)blockIdx.x - a.tile_start[u], a.accumulate != 0,
                                       a.keep_grad != 0, own_slice(v), a.found_inf,
                                       a.partials != nullptr ? a.partials + blockIdx.x : nullptr);
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void units_adamw_kernel(const UnitsArgs a) {
    if (a.sq_norm != nullptr && blockIdx.x == 0)
        finalize_norm(a.partials, (int)a.reduce_groups, a.sq_norm);
    const int u = find_unit(a.tile_start, a.n_units, blockIdx.x);
    const UnitView v = unit_view(a, u);
    adamw_tile<kAligned>(v, v.acc, (int64_t)blockIdx.x - a.tile_start[u], a.found_inf, own_slice(v));
}

hipError_t launch_units_reduce(const UnitsArgs& a, bool aligned, hipStream_t s) {
    const bool norm = a.partials != nullptr, acc = a.accumulate != 0;
    const dim3 g((unsigned)a.reduce_groups);
#define FP_UREDUCE(AL, AC, NO) units_reduce_kernel<AL, AC, NO><<<g, kThreads, 0, s>>>(a)
    if (aligned) {
        if (acc) { if (norm) FP_UREDUCE(true, true, true); else FP_UREDUCE(true, true, false); }
        else { if (norm) FP_UREDUCE(true, false, true); else FP_UREDUCE(true, false, false); }
    } else {
        if (acc) { if (norm) FP_UREDUCE(false, true, true); else FP_UREDUCE(false, true, false); }
        else { if (norm) FP_UREDUCE(false, false, true); else FP_UREDUCE(false, false, false); }
    }
#undef FP_UREDUCE
    return hipGetLastError();
}

hipError_t launch_units_phase1(const UnitsArgs& a, int64_t copy_groups, bool fused_update,
                               bool aligned, hipStream_t s) {
    const dim3 g((unsigned)(a.reduce_groups + copy_groups));
    if (aligned) {
        if (fused_update) units_phase1_kernel<true, true><<<g, kThreads, 0, s>>>(a);
        else units_phase1_kernel<true, false><<<g, kThreads, 0, s>>>(a);
    } else {
        if (fused_update) units_phase1_kernel<false, true><<<g, kThreads, 0, s>>>(a);
        else units_phase1_kernel<false, false><<<g, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_units_adamw(const UnitsArgs& a, bool aligned, hipStream_t s) {
    const dim3 g((unsigned)a.reduce_groups);
    if (aligned) units_adamw_kernel<true><<<g, kThreads, 0, s>>>(a);
    else units_adamw_kernel<false><<<g, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
