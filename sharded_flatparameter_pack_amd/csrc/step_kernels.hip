// step_kernels.hip -- gfx950 kernels of one unit's per-step path: reduce,
// AdamW with the bf16 cast, unshard, and the shard step (one-pass or
// two-phase), with their launchers.  The building blocks and the stream
// layout are described in step_ops.h.

#include <atomic>

#include "step_ops.h"

namespace fpk {

__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(const double* partials, int n,
                                                                 double* out) {
    finalize_norm(partials, n, out);
}

// ---------------------------------------------------------------- kernels

template <bool kAligned, bool kAccumulate, bool kNorm, int kG>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const ReduceArgs a) {
    reduce_tile<kAligned, kAccumulate, kNorm, kG>(a, blockIdx.x, a.found_inf,
                                                  kNorm ? a.partials + blockIdx.x : nullptr);
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void adamw_kernel(const AdamArgs a) {
    if (a.sq_norm != nullptr && blockIdx.x == 0) finalize_norm(a.partials, a.n_partials, a.sq_norm);
    adamw_tile<kAligned>(a, a.grad, blockIdx.x, a.found_inf, a.param_bf16);
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void unshard_kernel(const UnshardArgs a) {
    const int q = blockIdx.y;
    const uint16_t* src = a.shards[q];
    if (src == nullptr) return;
    const ShardSpan sp = shard_span(a.full, a.shard, q);
    copy_tile<kAligned, kCopyWordsStream, false>(src, a.full, sp, blockIdx.x);
    if (blockIdx.x == 0) unshard_edges(src, a.full, a.shard, q, threadIdx.x, kThreads);
}

// First phase of the two-phase step (kFused = false) or the whole no-skip
// step (kFused = true).  Workgroups [0, reduce_groups) take reduce tiles;
// the others take (shard, tile) pairs of the copy of the other ranks'
// shards into `full`.
template <bool kAligned, bool kCopyAligned, bool kFused, int kG>
__global__ __launch_bounds__(kThreads) void step_phase1_kernel(const StepArgs a) {
    if (blockIdx.x >= (unsigned)a.reduce_groups) {
        copy_role<kCopyAligned, kCopyWordsStream>(a, blockIdx.x - (unsigned)a.reduce_groups);
        return;
    }
    step_reduce_tile<kAligned, kFused, kG>(a, blockIdx.x, a.accumulate != 0, a.keep_grad != 0,
                                       a.full + (int64_t)a.rank * a.shard, a.found_inf,
                                       a.partials != nullptr ? a.partials + blockIdx.x : nullptr);
}

// Last kernel of the speculative exact-skip step.  The fused pass before it
// stored the updated state to separate output buffers without waiting for
// the overflow check; the skip rule is applied here instead: if the flag
// (the OR over the step's micro-batches) is set, the outputs receive the
// unchanged input state and the rank's slice of full the bf16 cast of the
// unchanged master, as a skipped step leaves them.  Without overflow, the
// common case, every workgroup reads the flag and returns.  The copy is a
// plain grid-stride loop: it only runs on a skipped step.
__global__ __launch_bounds__(kThreads) void step_resolve_kernel(const ResolveArgs r) {
    if (*r.found_inf == 0) return;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < r.shard; j += stride) {
        const float th = r.master[j];
        r.master_out[j] = th;
        r.exp_avg_out[j] = r.exp_avg[j];
        r.exp_avg_sq_out[j] = r.exp_avg_sq[j];
        r.own[j] = (uint16_t)bf16x2(th, 0.0f);
    }
}

// One-pass exact-skip step.  Workgroups [0, reduce_groups) take part in a
// grid barrier and must be resident together (the grid is sized for it);
// each of their lanes loads, for its kQ quads, the fp32 master / moments and
// the ranks' gradient quads (none of which depends on the overflow flag),
// reduces, and computes the AdamW update into registers.  The workgroup ORs
// its overflow bit (and the flag left by earlier micro-batches) into the
// barrier and waits; the barrier returns the grid's decision, after which
// the lanes only store: the new state and its bf16 cast, or on overflow just
// the cast of the old master.  Should a wait give up (the members were not
// resident together), the barrier is cancelled for every member alike and
// nothing is stored: the state, acc (unless the reduced gradient is kept
// for a call without accumulation) and the own slice keep their contents,
// and bit 1 is OR-ed into the flag.  The flag is only ever OR-ed into.
// Workgroups past reduce_groups copy the other ranks' shards meanwhile and
// take no part in the barrier.  The reduced gradient never leaves the
// registers, so the step moves exactly the algorithmic bytes.  With separate
// output state (state_out differs from the input), the new state goes to
// the outputs, and on overflow the outputs receive the input state, read
// again after the barrier (the skipped step's result, with no restore
// launch).
template <bool kAligned, bool kCopyAligned, int kQ>
__global__ __launch_bounds__(kThreads) void step_coop_kernel(const StepArgs a) {
    FP_PHASE_MARK(0);
    if (blockIdx.x >= (unsigned)a.reduce_groups) {
        copy_role<kCopyAligned, kCopyWordsCoop>(a, blockIdx.x - (unsigned)a.reduce_groups);
        FP_PHASE_MARK(5);
        return;
    }
    __shared__ unsigned s_decision;
    const int64_t nq = a.shard >> 2;
    const bool want_sq = a.partials != nullptr;
    const bool acc_in = a.accumulate != 0;
    uint16_t* own = a.full + (int64_t)a.rank * a.shard;
    // Thread 0 takes the barrier ticket and reads the flag left by earlier
    // kernels (measured faster than having every lane read them).
    BarrierTicket ticket = {0u, 0u};
    int32_t prior = 0;
    if (threadIdx.x == 0) {
        ticket = grid_ticket(a.sync);
        prior = *a.found_inf;
    }

    // reduce and speculative update, all in registers
    const AdamCoef c = coef_for(a.c, a.g_coef);
    const Quads<kQ> Q = lane_quads<kQ>(blockIdx.x, nq > 0 ? nq : 1);
    State<kQ> st;
    uint2 old_bf16[kQ];
    bool bad = false;
    double sq = 0.0;
    if (nq > 0) {
        load_state<kQ>(a, Q, st);
        float y[kQ][4];
        reduce_quads<kAligned, false, 8, kQ>(a, Q, acc_in, y);
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
            old_bf16[u] = f32x4_to_bf16(st.th[u]);
            if (!Q.ok[u]) continue;
            check_quad(y[u], bad, sq, want_sq);
            // (the path is chosen so that acc is not an input here)
            if (a.keep_grad) st_f32q(a.acc, Q, u, y[u]);
        }
        adamw_quads<kQ>(c, y, st);
    }
    const int64_t tail0 = nq << 2;
    const bool has_tail = blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0;
    float tt = 0.0f, tm = 0.0f, tv = 0.0f, told = 0.0f;
    if (has_tail) {
        const int64_t j = tail0 + threadIdx.x;
        tt = told = a.master[j];
        tm = a.exp_avg[j];
        tv = a.exp_avg_sq[j];
        const float yt = reduce_elem(a, j, acc_in);
        bad |= !finite_f32(yt);
        if (want_sq) sq += (double)yt * (double)yt;
        if (a.keep_grad) a.acc[j] = yt;
        adamw_elem(c, yt, tt, tm, tv);
    }
    FP_PHASE_MARK(1);
    const int group_bad = __syncthreads_or(bad);
    if (want_sq) {
        const double t = group_sum(sq);
        if (threadIdx.x == 0) a.partials[blockIdx.x] = t;   // summed by a follow-up kernel
    }
    FP_PHASE_MARK(2);
    if (threadIdx.x == 0) {
        const unsigned n = (unsigned)a.barrier_n;
        grid_arrive(a.sync, ticket, (group_bad || prior != 0) ? 1u : 0u, n);
        FP_PHASE_MARK(3);
        s_decision = grid_wait(a.sync, ticket, n, a.spin_limit);
    }
    FP_PHASE_MARK(4);
    __syncthreads();
    const unsigned decision = s_decision;
    if (decision == kBarrierCancelled) {
        if (blockIdx.x == 0 && threadIdx.x == 0) flag_or(a.found_inf, 2);
        FP_PHASE_MARK(5);
        return;
    }
    const bool skip = decision == kBarrierOverflow;
    if (skip && blockIdx.x == 0 && threadIdx.x == 0) flag_or(a.found_inf, 1);
    const StateOut o = state_out(a);
    const bool out_of_place = o.master != a.master;

    // commit: stores only (and on an overflowed out-of-place step, the copy
    // of the input state)
    if (nq > 0) {
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
            if (!Q.ok[u]) continue;
            if (skip) {
                st_bf16q<kAligned>(own, Q, u, old_bf16[u]);
                if (out_of_place) {
                    float f[4];
                    ld_f32q(a.master, Q, u, f);
                    st_f32q(o.master, Q, u, f);
                    ld_f32q(a.exp_avg, Q, u, f);
                    st_f32q(o.exp_avg, Q, u, f);
                    ld_f32q(a.exp_avg_sq, Q, u, f);
                    st_f32q(o.exp_avg_sq, Q, u, f);
                }
            } else {
                st_f32q(o.master, Q, u, st.th[u]);
                st_f32q(o.exp_avg, Q, u, st.m[u]);
                st_f32q(o.exp_avg_sq, Q, u, st.v[u]);
                st_bf16q<kAligned>(own, Q, u, f32x4_to_bf16(st.th[u]));
            }
        }
    }
    if (has_tail) {
        const int64_t j = tail0 + threadIdx.x;
        if (skip) {
            own[j] = (uint16_t)bf16x2(told, 0.0f);
            if (out_of_place) {
                o.master[j] = told;
                o.exp_avg[j] = a.exp_avg[j];
                o.exp_avg_sq[j] = a.exp_avg_sq[j];
            }
        } else {
            o.master[j] = tt;
            o.exp_avg[j] = tm;
            o.exp_avg_sq[j] = tv;
            own[j] = (uint16_t)bf16x2(tt, 0.0f);
        }
    }
    FP_PHASE_MARK(5);
}

// ---------------------------------------------------------------- launchers

template <bool kAligned, bool kAcc, bool kNorm>
void reduce_launch(const ReduceArgs& a, dim3 g, bool wide, hipStream_t s) {
    const unsigned lds = capped_reduce_lds(a.shard);
    if (wide) reduce_kernel<kAligned, kAcc, kNorm, 16><<<g, kThreads, lds, s>>>(a);
    else reduce_kernel<kAligned, kAcc, kNorm, 8><<<g, kThreads, lds, s>>>(a);
}

hipError_t launch_reduce(const ReduceArgs& a, int64_t grid, bool aligned, hipStream_t s) {
    const bool norm = a.partials != nullptr, acc = a.accumulate != 0, wide = wide_group(a.world);
    const dim3 g((unsigned)grid);
#define FP_REDUCE(AL, AC, NO) reduce_launch<AL, AC, NO>(a, g, wide, s)
    if (aligned) {
        if (acc) { if (norm) FP_REDUCE(true, true, true); else FP_REDUCE(true, true, false); }
        else { if (norm) FP_REDUCE(true, false, true); else FP_REDUCE(true, false, false); }
    } else {
        if (acc) { if (norm) FP_REDUCE(false, true, true); else FP_REDUCE(false, true, false); }
        else { if (norm) FP_REDUCE(false, false, true); else FP_REDUCE(false, false, false); }
    }
#undef FP_REDUCE
    return hipGetLastError();
}

hipError_t launch_norm_finalize(const double* partials, int n, double* out, hipStream_t s) {
    norm_finalize_kernel<<<1, kThreads, 0, s>>>(partials, n, out);
    return hipGetLastError();
}

hipError_t launch_step_resolve(const ResolveArgs& r, hipStream_t s) {
    constexpr int64_t kMaxResolveGroups = 2048;
    int64_t grid = (r.shard + kThreads - 1) / kThreads;
    if (grid > kMaxResolveGroups) grid = kMaxResolveGroups;
    if (grid < 1) grid = 1;
    step_resolve_kernel<<<(unsigned)grid, kThreads, 0, s>>>(r);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamArgs& a, int64_t grid, bool aligned, hipStream_t s) {
    const unsigned lds = capped_lds(a.shard);
    if (aligned) adamw_kernel<true><<<(unsigned)grid, kThreads, lds, s>>>(a);
    else adamw_kernel<false><<<(unsigned)grid, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_unshard(const UnshardArgs& a, int64_t grid_x, bool aligned, hipStream_t s) {
    const dim3 g((unsigned)grid_x, a.world);
    if (aligned) unshard_kernel<true><<<g, kThreads, 0, s>>>(a);
    else unshard_kernel<false><<<g, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

namespace {
// The fused reduce + AdamW keeps 8 ranks' loads in flight per round trip
// whatever the group size: with 16 it ran slower at 64 ranks (the 10k-tensor
// group's fused launch 1175 -> 1141 us with 8) and no faster at 16.
template <bool kAligned, bool kCopyAligned, bool kFused>
void phase1_launch(const StepArgs& a, dim3 g, unsigned lds, hipStream_t s) {
    if (wide_group(a.world) && !kFused) step_phase1_kernel<kAligned, kCopyAligned, kFused, 16><<<g, kThreads, lds, s>>>(a);
    else step_phase1_kernel<kAligned, kCopyAligned, kFused, 8><<<g, kThreads, lds, s>>>(a);
}

template <bool kAligned, bool kCopyAligned>
void phase1_launch(const StepArgs& a, dim3 g, bool fused, unsigned lds, hipStream_t s) {
    if (fused) phase1_launch<kAligned, kCopyAligned, true>(a, g, lds, s);
    else phase1_launch<kAligned, kCopyAligned, false>(a, g, lds, s);
}
}  // namespace

hipError_t launch_step_phase1(const StepArgs& a, int64_t grid, bool fused_update, bool capped, bool aligned,
                              bool copy_aligned, hipStream_t s) {
    const dim3 g((unsigned)grid);
    const unsigned lds = capped ? kCapLds : 0u;
    if (aligned) {
        if (copy_aligned) phase1_launch<true, true>(a, g, fused_update, lds, s);
        else phase1_launch<true, false>(a, g, fused_update, lds, s);
    } else {
        if (copy_aligned) phase1_launch<false, true>(a, g, fused_update, lds, s);
        else phase1_launch<false, false>(a, g, fused_update, lds, s);
    }
    return hipGetLastError();
}

namespace {
// Resident workgroups per CU of each one-pass variant and the CU count, per
// device: fixed properties of the device and the code object, computed on
// first use and kept for the life of the process.  The smaller of the
// aligned and general forms' figures bounds both.
constexpr int kMaxDevices = 64;
constexpr int kVariants = 2;  // lanes keep 2 or kMaxCoopQuads quads
struct CoopLimits {
    std::atomic<int> state{0};  // 0 unknown, 1 computing, 2 ready
    int cus = 0;
    int per_cu[kVariants] = {0, 0};
};
CoopLimits g_limits[kMaxDevices];

template <bool kAligned, bool kCopyAligned>
const void* coop_fn(int variant) {
    return variant == 0 ? reinterpret_cast<const void*>(&step_coop_kernel<kAligned, kCopyAligned, 2>)
                        : reinterpret_cast<const void*>(&step_coop_kernel<kAligned, kCopyAligned, kMaxCoopQuads>);
}

const void* coop_fn(int variant, int form) {
    switch (form) {
        case 0: return coop_fn<true, true>(variant);
        case 1: return coop_fn<true, false>(variant);
        case 2: return coop_fn<false, true>(variant);
        default: return coop_fn<false, false>(variant);
    }
}

hipError_t coop_limits(int dev, const CoopLimits** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    CoopLimits& L = g_limits[dev];
    for (;;) {
        const int state = L.state.load(std::memory_order_acquire);
        if (state == 2) break;
        int expect = 0;
        if (state == 0 && L.state.compare_exchange_strong(expect, 1)) {
            hipError_t e = hipDeviceGetAttribute(&L.cus, hipDeviceAttributeMultiprocessorCount, dev);
            for (int i = 0; i < kVariants && e == hipSuccess; ++i) {
                int lo = 1 << 30;
                for (int form = 0; form < 4 && e == hipSuccess; ++form) {
                    int b = 0;
                    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, coop_fn(i, form), kThreads, 0);
                    lo = b < lo ? b : lo;
                }
                L.per_cu[i] = lo;
            }
            L.state.store(e == hipSuccess ? 2 : 0, std::memory_order_release);
            if (e != hipSuccess) return e;
        }
    }
    *out = &L;
    return hipSuccess;
}
}  // namespace

hipError_t plan_step_coop(int64_t shard, int* variant, int* grid) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const CoopLimits* L = nullptr;
    if ((e = coop_limits(dev, &L)) != hipSuccess) return e;
    *variant = -1;
    const int64_t nq = shard >> 2;
    const int quads[kVariants] = {2, kMaxCoopQuads};
    for (int i = 0; i < kVariants; ++i) {
        const int64_t g = nq > 0 ? ceil_div64(nq, (int64_t)kThreads * quads[i]) : 1;
        if (g <= (int64_t)L->per_cu[i] * L->cus) {
            *variant = i;
            *grid = (int)g;
            return hipSuccess;
        }
    }
    return hipSuccess;
}

hipError_t launch_step_coop(const StepArgs& a, int variant, int grid, bool aligned, bool copy_aligned,
                            hipStream_t s, bool give_up_test) {
    // A plain launch (a cooperative launch costs ~17 us more per launch on
    // MI355X).  The barrier workgroups [0, reduce_groups) fit the device's
    // resident capacity and are dispatched before the copy workgroups, which
    // never wait; so on a GPU not running other work they are resident
    // together, and otherwise they become so as the copy workgroups finish.
    // give_up_test: the barrier waits for one member more than the grid holds
    // and gives up after a few polls, so every wait ends in the cancelled
    // decision (the barrier never completes, and its counters are left
    // mid-generation: the caller zero-fills the workspace again).
    StepArgs b = a;
    b.reduce_groups = grid;
    b.barrier_n = give_up_test ? grid + 1 : grid;
    b.spin_limit = give_up_test ? 64u : kSpinLimit;
    b.copy_tiles = (int32_t)copy_tiles_per_shard(a.shard, kCopyWordsCoop);
    const dim3 g((unsigned)((int64_t)grid + (int64_t)(a.world - 1) * b.copy_tiles));
#define FP_COOP(AL, CA)                                                          \
    do {                                                                         \
        if (variant == 0) step_coop_kernel<AL, CA, 2><<<g, kThreads, 0, s>>>(b);    \
        else step_coop_kernel<AL, CA, kMaxCoopQuads><<<g, kThreads, 0, s>>>(b);     \
    } while (0)
    if (aligned) {
        if (copy_aligned) FP_COOP(true, true);
        else FP_COOP(true, false);
    } else {
        if (copy_aligned) FP_COOP(false, true);
        else FP_COOP(false, false);
    }
#undef FP_COOP
    return hipGetLastError();
}

}  // namespace fpk
