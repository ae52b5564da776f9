// fp_extra.h -- argument blocks and launcher declarations of the operations
// around the step: the segment copy lists (FlatParameter pack, the per-
// parameter dim-0 layout, resharding), accumulation without communication,
// the loss-scaler and gradient-factor kernels, and the reduce of hybrid
// sharding.  Kept apart from fp_internal.h, which defines the step kernels'
// own blocks.
#pragma once

#include "fp_internal.h"

namespace fpk {

// The reduce of hybrid sharding: world = W ranks in groups of `group` = F
// consecutive ranks; the order is two-level (see hybrid_kernels.hip).
struct HybridArgs : ReduceArgs {
    int32_t group;
};

// One entry of a segment list, in 2-byte units.
// kind kSegCopy: dst[dst_off + k] = src[src_off + k] for k < len, or zeros
//   when src < 0; whole 16-byte words of the destination per lane.
// kind kSegStrided: a set of equal pieces of `piece` units, for groups of
//   small pieces that would otherwise share destination cache lines between
//   workgroups: for e < len, q = e / piece, k = e % piece,
//   dst[dst_off + q * dst_stride + k] = e < valid ? src[src_off + q * src_stride + k] : 0,
//   one unit per lane (len < 2^31).
constexpr int32_t kSegCopy = 0, kSegStrided = 1;
struct SegDesc {
    int64_t dst_off;
    int64_t src_off;
    int64_t len;
    int64_t tile0;                // first workgroup of the entry
    int64_t piece;
    int64_t valid;
    int64_t dst_stride;
    int64_t src_stride;
    int32_t dst;                  // index into the pointer table
    int32_t src;                  // index into the pointer table, -1: zeros
    int32_t kind;
    int32_t words;                // copy entries: 16-byte words per lane (1 or 2)
};

struct SegArgs {
    const SegDesc* segs;
    const int32_t* seg_of;        // entry of every workgroup
    void* const* dst_tab;         // per-call device pointers
    const void* const* src_tab;
};

// 16-byte words per lane of a copy tile (long entries; shorter ones set
// `words` to 2); units per workgroup of a strided entry; pieces below
// kSegSmallPiece units go to strided entries.
constexpr int kSegWords = 1;
constexpr int64_t kSegStridedTile = 4096;
constexpr int64_t kSegSmallPiece = 2048;
// Workgroups of one entry (at least one, for a copy's edges).
inline int64_t segment_tiles(const SegDesc& d) {
    if (d.kind == kSegStrided) return ceil_div64(d.len, kSegStridedTile);
    return ceil_div64(d.len / 8 + 1, (int64_t)kThreads * (d.words == 2 ? 2 : kSegWords));
}

// Local accumulation without communication over n elements of a rank's unit.
struct LocalArgs {
    const uint16_t* grad;   // bf16[n]
    float* local;           // fp32[n], 16-byte aligned (read only by the finish)
    uint16_t* out;          // bf16[n] (finish)
    int64_t n;
};

// Launchers (return the HIP error of the launch).
hipError_t launch_segments(const SegArgs& a, int64_t n_groups, hipStream_t s);
hipError_t launch_reduce_hybrid(const HybridArgs& a, int64_t grid, bool aligned, hipStream_t s);
hipError_t launch_local(const LocalArgs& a, bool finish, bool accumulate, bool aligned, hipStream_t s);
hipError_t launch_grad_coef(const double* sq_norm, const float* loss_scale, double max_norm, double* coef,
                            hipStream_t s);
hipError_t launch_scaler_update(const int32_t* found_inf, float* scale, int32_t* clean_steps,
                                float growth_factor, float backoff_factor, int32_t growth_interval,
                                hipStream_t s);

}  // namespace fpk
