// unit_kernels.hip -- the per-step kernels over many units in one launch:
// e.g. the DDP buckets of a model, whose shards make up one rank's fp32
// partition ("Infra: Data Parallel", ZeRO-1/ZeRO-2 paragraphs: each rank
// keeps one slice of the whole optimizer state; "4.1 数据并行详解",
// section 4.2: gradients are reduced bucket by bucket).  Each workgroup
// finds its unit (by a division for equal units, else from the plan's
// per-workgroup table), reads the unit's record (header and rank pointers),
// and runs the same tile bodies as the single-unit kernels on that unit.

#include "step_ops.h"

namespace fpk {

namespace {

// One unit as the tile bodies see it.
struct UnitView {
    const uint16_t* const* grads;
    const uint16_t* const* shards;
    uint16_t* full;
    float* acc;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
    int64_t shard;
    int64_t tile0;
    int64_t copy0;
    AdamCoef c;
    const double* g_coef;
    float scale;
    int32_t world;
    int32_t rank;
    int32_t copy_tiles;
};

// The unit of workgroup `group`: arithmetic for equal units, else the
// per-workgroup table (one more dependent load before the unit's record).
__device__ __forceinline__ int unit_of_group(const UnitsArgs& a, int64_t group) {
    const bool copy = group >= a.reduce_groups;
    const uint32_t run = (uint32_t)(copy ? a.copy_run : a.tile_run);
    if (run != 0) {
        const uint32_t i = (uint32_t)(copy ? group - a.reduce_groups : group);
        const uint32_t u = i / run;
        return u < (uint32_t)a.n_units ? (int)u : a.n_units - 1;
    }
    return a.unit_of[group];
}

__device__ __forceinline__ UnitView unit_view_of(const UnitsArgs& a, int u) {
    const char* rec = a.records + (int64_t)u * a.record_bytes;
    const UnitDesc& d = *reinterpret_cast<const UnitDesc*>(rec);
    UnitView v;
    v.grads = reinterpret_cast<const uint16_t* const*>(rec + kUnitHeader);
    v.shards = v.grads + a.world;
    v.full = d.full;
    v.acc = a.acc + d.offset;
    v.master = a.master + d.offset;
    v.exp_avg = a.exp_avg + d.offset;
    v.exp_avg_sq = a.exp_avg_sq + d.offset;
    const bool out = a.master_out != nullptr;
    v.master_out = (out ? a.master_out : a.master) + d.offset;
    v.exp_avg_out = (out ? a.exp_avg_out : a.exp_avg) + d.offset;
    v.exp_avg_sq_out = (out ? a.exp_avg_sq_out : a.exp_avg_sq) + d.offset;
    v.shard = d.shard;
    v.tile0 = d.tile0;
    v.copy0 = d.copy0;
    v.c = a.c;
    v.g_coef = a.g_coef;
    v.scale = a.scale;
    v.world = a.world;
    v.rank = a.rank;
    v.copy_tiles = d.copy_tiles;
    return v;
}

__device__ __forceinline__ UnitView unit_view(const UnitsArgs& a, int64_t group) {
    return unit_view_of(a, unit_of_group(a, group));
}

__device__ __forceinline__ uint16_t* own_slice(const UnitView& v) {
    return v.full != nullptr ? v.full + (int64_t)v.rank * v.shard : nullptr;
}

// The fused update of a unit stores its state to the step's output
// partitions (found by argument-dependent lookup from the tile bodies).
__device__ __forceinline__ StateOut state_out(const UnitView& v) {
    return {v.master_out, v.exp_avg_out, v.exp_avg_sq_out};
}

}  // namespace

template <bool kAligned, bool kAccumulate, bool kNorm, int kG>
__global__ __launch_bounds__(kThreads) void units_reduce_kernel(const UnitsArgs a) {
    const UnitView v = unit_view(a, blockIdx.x);
    reduce_tile<kAligned, kAccumulate, kNorm, kG>(v, (int64_t)blockIdx.x - v.tile0, a.found_inf,
                                                  kNorm ? a.partials + blockIdx.x : nullptr);
}

template <bool kAligned, bool kCopyAligned, bool kFused, int kG>
__global__ __launch_bounds__(kThreads) void units_phase1_kernel(const UnitsArgs a) {
    const UnitView v = unit_view(a, blockIdx.x);
    if ((int64_t)blockIdx.x >= a.reduce_groups) {
        copy_role<kCopyAligned, kCopyWordsStream>(v, (unsigned)((int64_t)blockIdx.x - a.reduce_groups - v.copy0));
        return;
    }
    step_reduce_tile<kAligned, kFused, kG>(v, (int64_t)blockIdx.x - v.tile0, a.accumulate != 0,
                                           a.keep_grad != 0, own_slice(v), a.found_inf,
                                           a.partials != nullptr ? a.partials + blockIdx.x : nullptr);
}

// The copies of every unit's other shards in a launch of their own (the
// split form of the fused step): copy workgroup g is workgroup
// reduce_groups + g of the combined launch's numbering.
template <bool kCopyAligned>
__global__ __launch_bounds__(kThreads) void units_copy_kernel(const UnitsArgs a) {
    const int64_t group = a.reduce_groups + (int64_t)blockIdx.x;
    const UnitView v = unit_view(a, group);
    copy_role<kCopyAligned, kCopyWordsStream>(v, (unsigned)((int64_t)blockIdx.x - v.copy0));
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void units_adamw_kernel(const UnitsArgs a) {
    if (a.sq_norm != nullptr && blockIdx.x == 0)
        finalize_norm(a.partials, (int)a.reduce_groups, a.sq_norm);
    const UnitView v = unit_view(a, blockIdx.x);
    adamw_tile<kAligned>(v, v.acc, (int64_t)blockIdx.x - v.tile0, a.found_inf, own_slice(v));
}

// Last kernel of the speculative multi-unit step: if the flag (the OR over
// the step's micro-batches and all units) is set, every unit's output state
// takes its unchanged input state and its own slice of full the bf16 cast
// of the unchanged master, as a skipped step leaves them; otherwise every
// workgroup returns at once.  A grid-stride loop over each unit in turn: it
// only runs on a skipped step.
__global__ __launch_bounds__(kThreads) void units_resolve_kernel(const UnitsArgs a) {
    if (*a.found_inf == 0) return;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int u = 0; u < a.n_units; ++u) {
        const UnitView v = unit_view_of(a, u);
        uint16_t* own = own_slice(v);
        for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < v.shard; j += stride) {
            const float th = v.master[j];
            v.master_out[j] = th;
            v.exp_avg_out[j] = v.exp_avg[j];
            v.exp_avg_sq_out[j] = v.exp_avg_sq[j];
            if (own != nullptr) own[j] = (uint16_t)bf16x2(th, 0.0f);
        }
    }
}

namespace {
template <bool kAligned, bool kAcc, bool kNorm>
void units_reduce_launch(const UnitsArgs& a, dim3 g, unsigned lds, hipStream_t s) {
    if (wide_group(a.world)) units_reduce_kernel<kAligned, kAcc, kNorm, 16><<<g, kThreads, lds, s>>>(a);
    else units_reduce_kernel<kAligned, kAcc, kNorm, 8><<<g, kThreads, lds, s>>>(a);
}

// The last micro-batch's launch keeps 8 ranks' loads in flight per round
// trip whatever the group size, each group's row pointers read up front.
// Measured on MI355X at the bucketed 611M model (16 ranks): the fused launch
// 453 -> 436 us, the two-phase launch with its copies 641 -> 618 us (groups
// of 16 read their pointers rank by rank: sixteen held pointers cost
// occupancy).  The reduce-only launch keeps groups of 16 (245 us against
// 248 with 8).
template <bool kAligned, bool kCopyAligned, bool kFused>
void units_phase1_launch(const UnitsArgs& a, dim3 g, unsigned lds, hipStream_t s) {
    units_phase1_kernel<kAligned, kCopyAligned, kFused, 8><<<g, kThreads, lds, s>>>(a);
}

template <bool kAligned, bool kCopyAligned>
void units_phase1_launch(const UnitsArgs& a, dim3 g, bool fused, unsigned lds, hipStream_t s) {
    if (fused) units_phase1_launch<kAligned, kCopyAligned, true>(a, g, lds, s);
    else units_phase1_launch<kAligned, kCopyAligned, false>(a, g, lds, s);
}
}  // namespace

hipError_t launch_units_reduce(const UnitsArgs& a, bool aligned, bool capped, hipStream_t s) {
    const bool norm = a.partials != nullptr, acc = a.accumulate != 0;
    const dim3 g((unsigned)a.reduce_groups);
    const unsigned lds = capped ? kReduceCapLds : 0u;
#define FP_UREDUCE(AL, AC, NO) units_reduce_launch<AL, AC, NO>(a, g, lds, s)
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

hipError_t launch_units_phase1(const UnitsArgs& a, int64_t copy_groups, bool fused_update, bool capped,
                               bool aligned, bool copy_aligned, hipStream_t s) {
    const dim3 g((unsigned)(a.reduce_groups + copy_groups));
    const unsigned lds = capped ? kCapLds : 0u;
    if (aligned) {
        if (copy_aligned) units_phase1_launch<true, true>(a, g, fused_update, lds, s);
        else units_phase1_launch<true, false>(a, g, fused_update, lds, s);
    } else {
        if (copy_aligned) units_phase1_launch<false, true>(a, g, fused_update, lds, s);
        else units_phase1_launch<false, false>(a, g, fused_update, lds, s);
    }
    return hipGetLastError();
}

hipError_t launch_units_copy(const UnitsArgs& a, int64_t copy_groups, bool copy_aligned, hipStream_t s) {
    const dim3 g((unsigned)copy_groups);
    if (copy_aligned) units_copy_kernel<true><<<g, kThreads, 0, s>>>(a);
    else units_copy_kernel<false><<<g, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_units_adamw(const UnitsArgs& a, bool aligned, hipStream_t s) {
    const dim3 g((unsigned)a.reduce_groups);
    if (aligned) units_adamw_kernel<true><<<g, kThreads, 0, s>>>(a);
    else units_adamw_kernel<false><<<g, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_units_resolve(const UnitsArgs& a, hipStream_t s) {
    constexpr int64_t kMaxResolveGroups = 2048;
    int64_t grid = a.reduce_groups < kMaxResolveGroups ? a.reduce_groups : kMaxResolveGroups;
    if (grid < 1) grid = 1;
    units_resolve_kernel<<<(unsigned)grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
