// fp_internal.h -- kernel argument blocks and launcher declarations shared by
// the host entry points (abi.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/flatparam.h"

namespace fpk {

constexpr int kThreads = 256;          // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
// Element streams move in quads of 4 elements (16 bytes of fp32, 8 of bf16).
// A workgroup of a streaming kernel owns one tile of kTileQuads consecutive
// quads, kQuadsPerLane per lane, and tiles are numbered in dispatch order,
// so the workgroups in flight cover one contiguous window of every stream --
// on MI355X this keeps HBM pages open far better than grid-stride loops,
// whose concurrent accesses spread over the whole buffer.  One quad per lane
// (1024 elements per workgroup) measured best for the two-kernel step: fewer
// registers, more waves in flight (against two: the d=12288 layer's step
// 2.92 ms vs 3.00, the 10k-tensor step at 64 ranks 3.00 ms vs 3.30).
constexpr int kQuadsPerLane = 1;
constexpr int64_t kTileQuads = (int64_t)kThreads * kQuadsPerLane;
// 16-byte words per lane of a copy workgroup.  Stand-alone copies and the
// two-pass step use one (consecutive waves then sweep consecutive addresses,
// the fastest pattern measured for long copies); the one-pass step uses four,
// all loads issued before the stores, so that its fewer copy workgroups fit
// beside the resident barrier workgroups from the start.
constexpr int kCopyWordsStream = 1;
constexpr int kCopyWordsCoop = 4;
constexpr int kMaxCoopQuads = 4;       // quads a lane keeps in registers in the one-pass step

// Streaming kernels with many loads in flight per lane (AdamW, the reduce)
// run shards of kCapElems elements and more with at most four workgroups
// resident per CU (the reduce-only kernels at three, below): the launch asks
// for kCapLds bytes of dynamic LDS, which the kernels never touch, so that
// 160 KiB of LDS admits four.  Measured on
// MI355X at full occupancy they lost bandwidth on the largest shards
// (fp_adamw_shard at 226.5M elements: 1231 us uncapped, 1154 us capped;
// fp_reduce_shard of 8 ranks: 906 vs 844 us; at 100M 508 vs 499 and 389
// vs 379 us), while from 42.6M elements down the cap cost up to 2.5 %.
// Copies (few loads per lane) lose under the cap, so launches that copy
// keep full occupancy.
constexpr int64_t kCapElems = (int64_t)1 << 26;
constexpr unsigned kCapLds = 40u << 10;
inline unsigned capped_lds(int64_t shard) { return shard >= kCapElems ? kCapLds : 0u; }
// The reduce-only kernels (single-unit and hybrid from kCapElems elements,
// multi-unit from kSplitElems partition elements) run with at most three
// workgroups per CU.  Measured on MI355X: the multi-unit reduce at the
// bucketed 611M model (16 ranks, 38.2M elements) 245 us at full occupancy,
// 241 at four workgroups per CU, 233 at three, 241 at two; fp_reduce_shard
// of 16 ranks at 226.5M elements 1326-1348 us at four, 1306-1309 at three.
// The fused step and AdamW kernels gained nothing from three over four.
constexpr unsigned kReduceCapLds = 53504u;
inline unsigned capped_reduce_lds(int64_t shard) { return shard >= kCapElems ? kReduceCapLds : 0u; }
// The fused no-skip step of shards from kSplitElems elements on runs its
// reduce + AdamW workgroups under the same cap and the copies of the other
// shards in a launch of their own (measured: the d=12288 layer at 8 ranks
// 2.64 -> 2.54 ms, the 10k-tensor group at 64 ranks, 42.6M elements, 2.97 ->
// 2.90 ms); smaller shards keep one launch.
constexpr int64_t kSplitElems = (int64_t)1 << 24;
constexpr int kSyncGroups = 32;        // first level of the grid barrier
constexpr int kLineWords = 32;         // 128-byte cache line in 32-bit words

// Grid-barrier state at the start of the workspace (zero-filled by the
// caller before first use; every completed barrier leaves the counters at
// 0).  Each counter and each copy of the generation word has a cache line
// of its own.
struct GridSync {
    unsigned int group[kSyncGroups * kLineWords];  // arrivals per group (+ overflow bit 16)
    unsigned int top[kLineWords];                  // groups complete (+ overflow bit 16)
    unsigned int gen[kSyncGroups * kLineWords];    // per-group copy: generation | flag << 31
    unsigned int timeouts;                         // waits that gave up
    unsigned int pad[kLineWords - 1];
};
constexpr int64_t kWorkspaceHeader = 16384;  // GridSync, then one double per workgroup
static_assert(sizeof(GridSync) <= kWorkspaceHeader, "barrier state exceeds the header");
static_assert(offsetof(GridSync, timeouts) == FP_WORKSPACE_TIMEOUTS_OFFSET, "timeouts offset");

// fp64 coefficients of one AdamW step, all derived on the host in fp64.
struct AdamCoef {
    double decay;        // 1 - lr * weight_decay
    double beta1;
    double one_m_beta1;  // 1 - beta1
    double beta2;
    double one_m_beta2;  // 1 - beta2
    double step_size;       // lr / (1 - beta1^t)
    double inv_sqrt_bias2;  // 1 / sqrt(1 - beta2^t)
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

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t tiles_of(int64_t quads) { return ceil_div64(quads, kTileQuads); }
// Copy tiles per shard: the whole 16-byte words of a shard number at most S/8 + 1.
inline int64_t copy_tiles_per_shard(int64_t S, int words) { return ceil_div64(S / 8 + 1, (int64_t)kThreads * words); }

// Shard q occupies full[qS, (q+1)S).  [lo, a) and [b, hi) are its edge
// elements that share a 16-byte word of `full` with a neighbouring shard;
// [a, b) are whole, aligned words of `full`.
struct ShardSpan {
    int64_t lo, a, b, hi;
};

// Elements [lo, lo + len) of a 2-byte stream at `base`, split into whole
// aligned 16-byte words [a, b) and edge elements [lo, a), [b, hi).
__host__ __device__ inline ShardSpan elem_span(const uint16_t* base, int64_t lo, int64_t len) {
    // element index e is 16-byte aligned in `base` when e % 8 == phase
    const int64_t phase = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(base) & 15u)) & 15u) >> 1);
    ShardSpan s;
    s.lo = lo;
    s.hi = lo + len;
    const int64_t up = s.lo + (((phase - s.lo) % 8) + 8) % 8;     // first aligned >= lo
    s.a = up < s.hi ? up : s.hi;
    const int64_t down = s.hi - (((s.hi - phase) % 8) + 8) % 8;   // last aligned <= hi
    s.b = down > s.a ? down : s.a;
    return s;
}

__host__ __device__ inline ShardSpan shard_span(const uint16_t* full, int64_t S, int q) {
    return elem_span(full, (int64_t)q * S, S);
}

// True when shard q's source, read from its first whole word of `full` on,
// is 16-byte aligned (then the copy needs no realignment).
inline bool copy_source_aligned(const uint16_t* src, const uint16_t* full, int64_t S, int q) {
    const ShardSpan sp = shard_span(full, S, q);
    return ((reinterpret_cast<uintptr_t>(src) + 2 * (uintptr_t)(sp.a - sp.lo)) & 15u) == 0;
}
// Norm partial slots the workspace provides for a shard of S elements (one
// per workgroup of any launch geometry used for that shard).
inline int64_t partial_slots(int64_t S) { return ceil_div64(S / 4, kTileQuads) + 1; }

struct AdamArgs {
    const float* grad;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    uint16_t* param_bf16;       // may be null
    const int32_t* found_inf;   // may be null: never skip
    int64_t shard;
    AdamCoef c;
    const double* g_coef;       // factor applied to the gradient, may be null (1)
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
    double* sq_norm;         // one-pass: finalised by workgroup 0 after the barrier
    int64_t shard;
    AdamCoef c;
    const double* g_coef;    // factor applied to the gradient, may be null (1)
    float scale;
    int32_t world;
    int32_t rank;
    int32_t accumulate;
    int32_t keep_grad;
    int32_t reduce_groups;   // workgroups of the reduce role (barrier members in one pass)
    int32_t copy_tiles;      // copy tiles per shard
    GridSync* sync;          // one-pass: barrier state in the workspace
    int32_t barrier_n;       // one-pass: members the barrier waits for
    uint32_t spin_limit;     // one-pass: polls before a wait gives up
    // Where the fused update stores the state: separate buffers for the
    // speculative step, else master / exp_avg / exp_avg_sq themselves.
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
};

// The speculative step's last kernel: if *found_inf is set, the output state
// takes the input state and own (the rank's slice of full) its bf16 cast.
struct ResolveArgs {
    const int32_t* found_inf;
    const float* master;
    const float* exp_avg;
    const float* exp_avg_sq;
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
    uint16_t* own;
    int64_t shard;
};

// One unit of a multi-unit launch: a device record of kUnitHeader bytes
// (this header) followed by the unit's world gradient row pointers and
// world shard pointers (entry rank null; all null without unshard), so that
// a workgroup reaches everything about its unit from one record address.
// The rank's fp32 partition (acc, master, moments) holds unit u at element
// `offset`, a multiple of 4, so every unit's fp32 shard is 16-byte aligned.
struct UnitDesc {
    int64_t shard;
    int64_t offset;
    int64_t tile0;       // first reduce / AdamW workgroup of the unit
    int64_t copy0;       // first copy workgroup of the unit, counted from reduce_groups
    uint16_t* full;      // bf16[world * shard], or null
    int32_t copy_tiles;  // copy workgroups per other shard
    int32_t pad[3];
};
constexpr int64_t kUnitHeader = 64;
static_assert(sizeof(UnitDesc) <= kUnitHeader, "unit header exceeds its slot");
inline int64_t unit_record_bytes(int world) { return kUnitHeader + 16 * (int64_t)world; }

// A launch over all units of a plan.  Workgroup i (reduce / AdamW tiles
// first, then copy tiles) belongs to unit u(i), whose record sits at
// records + u(i) * record_bytes.  When every unit but the last has the same
// number of reduce tiles (and of copy tiles) -- equal DDP buckets -- u(i)
// is computed (tile_run / copy_run > 0); otherwise it is read from unit_of.
struct UnitsArgs {
    const char* records;
    const int32_t* unit_of;      // [reduce_groups + copy_groups]
    int32_t tile_run;            // reduce tiles of each unit but the last, or 0
    int32_t copy_run;            // copy tiles of each unit but the last, or 0
    float* acc;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    int32_t* found_inf;
    double* partials;
    double* sq_norm;             // AdamW launch: finalised by workgroup 0
    AdamCoef c;
    const double* g_coef;        // factor applied to the gradient, may be null (1)
    int64_t reduce_groups;
    int64_t record_bytes;
    float scale;
    int32_t n_units;
    int32_t world;
    int32_t rank;
    int32_t accumulate;
    int32_t keep_grad;
    // Where the fused update stores the state: separate partitions for the
    // speculative step, else master / exp_avg / exp_avg_sq themselves.
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
};

// Ranks reduced per group of loads in flight: 16 when more than 8 ranks
// contribute (one round trip for up to 16 ranks), else 8.  The fused
// reduce + AdamW launches always take 8.
inline bool wide_group(int world) { return world > 8; }

// Reduce / AdamW workgroups of one unit: at least one, so that its tail
// elements and flag have an owner.
inline int64_t unit_tiles(int64_t S) {
    const int64_t t = tiles_of(S >> 2);
    return t > 0 ? t : 1;
}

// Host helpers of the entry points (abi.hip): set the calling thread's
// error message and return `status`; run fp_shard_step (give_up_test: the
// one-pass kernel with a barrier that always gives up).
fp_status report_error(fp_status status, const char* message);
fp_status shard_step_run(const fp_step_args* args, void* stream, bool give_up_test);

// Launchers (return the HIP error of the launch).
// `aligned`: every bf16 quad stream of the launch (gradients, own shard) is
// 8-byte aligned; `copy_aligned` (and `aligned` for fp_unshard's kernel):
// every copy source is 16-byte aligned at the words the kernel reads.  Then
// those streams take the aligned form of the accesses.
hipError_t launch_reduce(const ReduceArgs& a, int64_t grid, bool aligned, hipStream_t s);
hipError_t launch_norm_finalize(const double* partials, int n, double* out, hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, int64_t grid, bool aligned, hipStream_t s);
hipError_t launch_unshard(const UnshardArgs& a, int64_t grid_x, bool aligned, hipStream_t s);
// `capped`: the launch holds only the reduce workgroups (the copies run in a
// launch of their own), which then run at the occupancy cap.
hipError_t launch_step_phase1(const StepArgs& a, int64_t grid, bool fused_update, bool capped, bool aligned,
                              bool copy_aligned, hipStream_t s);
// One-pass exact-skip step: plan_step_coop picks the variant (lanes keep
// 2 or 4 quads in registers) and a grid that fits the device's co-resident
// capacity, or sets *variant = -1 when the shard is too large.
hipError_t plan_step_coop(int64_t shard, int* variant, int* grid);
// give_up_test: every barrier wait gives up (the cancelled decision), for
// testing that path from the host.
hipError_t launch_step_coop(const StepArgs& a, int variant, int grid, bool aligned, bool copy_aligned,
                            hipStream_t s, bool give_up_test = false);
hipError_t launch_step_resolve(const ResolveArgs& r, hipStream_t s);
// Multi-unit launches: one micro-batch's reduce over all units; the last
// micro-batch's reduce (+ AdamW when fused) with the copies of all units'
// other shards (copy_groups workgroups after the reduce tiles); AdamW over
// all units.
hipError_t launch_units_reduce(const UnitsArgs& a, bool aligned, bool capped, hipStream_t s);
// `capped`: only the reduce tiles (copy_groups = 0), at the occupancy cap.
hipError_t launch_units_phase1(const UnitsArgs& a, int64_t copy_groups, bool fused_update, bool capped,
                               bool aligned, bool copy_aligned, hipStream_t s);
// The copy workgroups of a units launch in a launch of their own.
hipError_t launch_units_copy(const UnitsArgs& a, int64_t copy_groups, bool copy_aligned, hipStream_t s);
hipError_t launch_units_adamw(const UnitsArgs& a, bool aligned, hipStream_t s);
// The speculative multi-unit step's last kernel: on overflow, every unit's
// output state takes its input state and its own slice the bf16 cast.
hipError_t launch_units_resolve(const UnitsArgs& a, hipStream_t s);

}  // namespace fpk
