// hybrid_kernels.hip -- the reduce of hybrid sharding.
//
// "PyTorch FSDP ...", section 3.3 and the sharding-factor bullet: with a
// sharding factor F, groups of F GPUs fully shard a unit and the W / F
// groups replicate it; "4.1 数据并行详解", HYBRID_SHARD: a reduce-scatter
// inside each group, an all-reduce across the groups.  The unit is split
// into F slices; rank (group g, position p) owns slice p, and its reduced
// gradient averages all W ranks' gradients of that slice in two levels:
// each group's F gradients summed in rank order, then the W / F group sums
// in group order, then one multiply by the scale.  Rank g * F + j of the
// pointer table is rank j of group g.
//
// The tile body is the flat reduce's (reduce_tile in step_ops.h): only the
// summation order differs, supplied here as overloads of sum_ranks and
// sum_ranks1 for HybridArgs, which the tile body picks up by argument type.
// The loads are issued as in the flat reduce, 8 ranks (16 beyond 8) at a
// time; the group boundaries only decide which running sum an element is
// added to.

#include "fp_extra.h"
#include "step_ops.h"

namespace fpk {

template <bool kAligned, int kG, int kU>
__device__ __forceinline__ void sum_ranks(const HybridArgs& a, const Quads<kU>& Q, float s[kU][4]) {
    const int world = a.world, group = a.group;
    float t[kU][4];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[u][e] = t[u][e] = 0.0f;   // both replaced by the first values
    }
    int j0 = 0;                      // position in its group of rank q0
    for (int q0 = 0; q0 < world; q0 += kG) {
        uint2 w[kG][kU];
        load_group<kAligned, kG, kU, false>(a.grads, q0, world, Q, w);
        int j = j0;
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            if (q0 + k < world) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    float f[4];
                    bf16x4_to_f32(w[k][u], f);
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[u][e] = j == 0 ? f[e] : t[u][e] + f[e];
                }
                if (j == group - 1) {        // the group's sum is complete
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[u][e] = q0 + k == group - 1 ? t[u][e] : s[u][e] + t[u][e];
                    }
                    j = 0;
                } else {
                    ++j;
                }
            }
        }
        j0 = j;
    }
}

__device__ __forceinline__ float sum_ranks1(const HybridArgs& a, int64_t j) {
    float s = 0.0f;
    for (int g = 0; g < a.world / a.group; ++g) {
        float t = bf16_lo(a.grads[g * a.group][j]);
        for (int k = 1; k < a.group; ++k) t = t + bf16_lo(a.grads[g * a.group + k][j]);
        s = g == 0 ? t : s + t;
    }
    return s;
}

template <bool kAligned, bool kAccumulate, bool kNorm, int kG>
__global__ __launch_bounds__(kThreads) void hybrid_reduce_kernel(const HybridArgs a) {
    reduce_tile<kAligned, kAccumulate, kNorm, kG>(a, blockIdx.x, a.found_inf,
                                                  kNorm ? a.partials + blockIdx.x : nullptr);
}

template <bool kAligned, bool kAcc, bool kNorm>
void hybrid_launch(const HybridArgs& a, dim3 g, bool wide, hipStream_t s) {
    const unsigned lds = capped_reduce_lds(a.shard);
    if (wide) hybrid_reduce_kernel<kAligned, kAcc, kNorm, 16><<<g, kThreads, lds, s>>>(a);
    else hybrid_reduce_kernel<kAligned, kAcc, kNorm, 8><<<g, kThreads, lds, s>>>(a);
}

hipError_t launch_reduce_hybrid(const HybridArgs& a, int64_t grid, bool aligned, hipStream_t s) {
    const bool norm = a.partials != nullptr, acc = a.accumulate != 0, wide = wide_group(a.world);
    const dim3 g((unsigned)grid);
#define FP_HYBRID(AL, AC, NO) hybrid_launch<AL, AC, NO>(a, g, wide, s)
    if (aligned) {
        if (acc) { if (norm) FP_HYBRID(true, true, true); else FP_HYBRID(true, true, false); }
        else { if (norm) FP_HYBRID(true, false, true); else FP_HYBRID(true, false, false); }
    } else {
        if (acc) { if (norm) FP_HYBRID(false, true, true); else FP_HYBRID(false, true, false); }
        else { if (norm) FP_HYBRID(false, false, true); else FP_HYBRID(false, false, false); }
    }
#undef FP_HYBRID
    return hipGetLastError();
}

}  // namespace fpk
