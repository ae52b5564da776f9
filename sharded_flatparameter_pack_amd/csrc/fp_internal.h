// fp_internal.h -- kernel argument blocks and launcher declarations shared by
// the host entry points (abi.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flatparam.h"

namespace fpk {

constexpr int kThreads = 256;          // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kElemsPerChunk = 8;      // one 16-byte bf16 word, two 16-byte fp32 words
constexpr int kMaxGrid = 4096;         // cap of grid-stride launches = norm partial slots
constexpr int64_t kWorkspaceBytes = 64 * 1024;   // >= kMaxGrid doubles
constexpr int kPackBlockElems = 8192;  // flat elements per pack workgroup
constexpr int kPackLdsTensors = 1024;  // tensor descriptors a pack workgroup stages in LDS

// fp64 coefficients of one AdamW step, all derived on the host in fp64.
struct AdamCoef {
    double decay;        // 1 - lr * weight_decay
    double beta1;
    double one_m_beta1;  // 1 - beta1
    double beta2;
    double one_m_beta2;  // 1 - beta2
    double bias1;        // 1 - beta1^t
    double bias2;        // 1 - beta2^t
    double lr;
    double eps;
};

struct ReduceArgs {
    const uint16_t* grads[FP_MAX_WORLD];  // rank q's bf16 gradient over this shard
    float* acc;                            // fp32[S]
    int32_t* found_inf;                    // may be null
    double* partials;                      // per-workgroup sum of squares, may be null
    int64_t shard;
    float scale;
    int32_t world;
    int32_t accumulate;
};

struct AdamArgs {
    const float* grad;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    uint16_t* param_bf16;       // may be null
    const int32_t* found_inf;   // may be null: never skip
    int64_t shard;
    AdamCoef c;
    // optional finalisation of the reduce's norm partials by workgroup 0
    const double* partials;
    double* sq_norm;
    int32_t n_partials;
};

struct UnshardArgs {
    const uint16_t* shards[FP_MAX_WORLD];  // null = leave that range untouched
    uint16_t* full;
    int64_t shard;
    int32_t world;
};

// One launch of the shard step's first phase: workgroups [0, reduce_groups)
// run the reduce (two-phase) or the fused reduce + AdamW (no-skip); the
// remaining workgroups copy the other ranks' shards into `full`.
struct StepArgs {
    const uint16_t* grads[FP_MAX_WORLD];
    const uint16_t* shards[FP_MAX_WORLD];  // entry `rank` is null
    float* acc;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    uint16_t* full;
    int32_t* found_inf;
    double* partials;
    int64_t shard;
    AdamCoef c;
    float scale;
    int32_t world;
    int32_t rank;
    int32_t accumulate;
    int32_t keep_grad;
    int32_t reduce_groups;
};

struct PackArgs {
    const int64_t* offsets;     // [n_tensors + 1] prefix sums, offsets[n] = T
    const int32_t* group_first; // [n_groups + 1] first tensor overlapping each group
    const void* const* src;     // [n_tensors] device pointers
    void* flat;
    int64_t total;              // T
    int64_t padded;             // P
    int32_t n_tensors;
};

// Launchers (return the HIP error of the launch).
hipError_t launch_reduce(const ReduceArgs& a, int grid, hipStream_t s);
hipError_t launch_norm_finalize(const double* partials, int n, double* out, hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, int grid, hipStream_t s);
hipError_t launch_unshard(const UnshardArgs& a, int grid_x, hipStream_t s);
hipError_t launch_step_phase1(const StepArgs& a, int grid, bool fused_update, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, int elem_size, int64_t n_groups, hipStream_t s);

}  // namespace fpk
