/*
 * flatparam.h -- C ABI of libflatparam.so: one rank's FSDP / ZeRO shard step
 * on an AMD Instinct MI355X (gfx950).
 *
 * The library implements, as hand-written HIP kernels, the per-rank data
 * path of sharded data parallelism:
 *   pack    -- build a FlatParameter from a unit's tensors,
 *   reduce  -- the arithmetic of the gradient reduce-scatter (average of the
 *              N ranks' bf16 gradients into this rank's fp32 shard, with
 *              micro-batch accumulation and an overflow check),
 *   adamw   -- the mixed-precision AdamW update of the shard,
 *   unshard -- the bf16 cast and the all-gather's copy of every rank's
 *              shard back into the full flat buffer,
 *   views   -- the original tensors as full, fragment or empty views.
 * Around that step: the per-parameter dim-0 layout (FSDP2), accumulation
 * without communication (no_sync), the loss scaler's update and the
 * gradient factor (unscale, global-norm clipping), the reduce of hybrid
 * sharding, and resharding a flat buffer to another rank count.
 * On one GPU the N "ranks" are buffers on that GPU.
 *
 * Pages the operations follow (cited by title and section):
 *   [DP]    "Infra: Data Parallel" (pufanyi.com)
 *   [FSDP]  "PyTorch FSDP: 大模型分布式训练的工业级分片并行方案" (2048ai.net,
 *           a summary of Zhao et al., PyTorch FSDP, VLDB 2023)
 *   [GUIDE] "4.1 数据并行详解" (AIInfraGuide)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: every device buffer belongs to the caller and is passed as a
 *   raw device pointer; the library never frees or keeps them.  Host arrays
 *   (pointer tables, shapes) are read during the call only.  An fp_plan is
 *   owned by the library until fp_plan_destroy.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Device work is enqueued on it asynchronously; no entry point
 *   waits for the device, except fp_pack as noted there.
 * Layout: bf16 values are passed as uint16_t bit patterns.  fp32 buffers
 *   (grad / acc, master, exp_avg, exp_avg_sq) must be 16-byte aligned;
 *   bf16 buffers need only their natural 2-byte alignment.
 * Errors: every call returns an fp_status.  On any error nothing has been
 *   enqueued, except FP_ERR_DEVICE after a failed launch.  Faults inside a
 *   kernel surface at the caller's next synchronisation.  fp_last_error()
 *   returns a message for the calling thread's most recent failure.
 * Sizes: a dispatch holds at most (2^32 - 1) / 256 = 16 777 215 workgroups
 *   of 256 lanes.  A call whose launch would need more returns FP_ERR_RANGE
 *   before enqueueing anything.  The streaming kernels (reduce, AdamW,
 *   no_sync) take 1024 elements per workgroup, so S up to about 1.7e10;
 *   fp_unshard takes 2048 per shard and workgroup.  The two-phase and
 *   no-skip shard step holds the reduce tiles and the N - 1 other shards'
 *   copy tiles in its first launch, which bounds S to about 3.8e9 at N = 8.
 *   The copy kernel of pack, the dim-0 layout and resharding counts the
 *   workgroups of its whole entry list against the same limit.
 * The library keeps no global mutable state apart from that message and a
 * per-device cache of occupancy figures (fixed properties of the device and
 * the code object, computed on first use).  Plans (fp_plan, fp_units,
 * fp_shard0_plan, fp_reshard_plan) own the device tables their calls build.
 * A host allocation failure inside a call returns FP_ERR_DEVICE; no C++
 * exception crosses this interface.
 */
#ifndef FLATPARAM_H
#define FLATPARAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp_status;

#define FP_OK 0
#define FP_ERR_INVALID (-1) /* null pointer, negative size, bad enum value  */
#define FP_ERR_RANGE (-2)   /* size, world, rank or count out of range      */
#define FP_ERR_ALIGN (-3)   /* pointer not aligned as required              */
#define FP_ERR_DEVICE (-4)  /* the HIP runtime reported an error            */

/* Largest N_d the device entry points accept (pointer tables travel as
 * kernel arguments).  Plans and views accept any world up to 1 << 20. */
#define FP_MAX_WORLD 128
#define FP_MAX_NDIM 8

/* ------------------------------------------------------------------ plan */

/* Immutable description of one FlatParameter: the unit's tensor shapes in
 * order and the world size N_d.  [DP] section "FSDP1: pack first, then
 * split" and its figure: the tensors are flattened (row-major) and
 * concatenated into one 1-D buffer that is split evenly over N_d ranks, a
 * shard boundary may cut a tensor.  [FSDP] section 2 (FlatParameter).
 * Geometry: T = sum of numels; P = T rounded up to a multiple of N_d (the
 * tail P - T elements are zero padding); S = P / N_d; rank q's shard is
 * flat[q*S, (q+1)*S).  [DP] ZeRO figure: GPU i holds slice i. */
typedef struct fp_plan fp_plan;

/* n_tensors >= 1 tensors; ndims[i] in [0, FP_MAX_NDIM] (0 = scalar);
 * shapes holds the dims of all tensors back to back (sum of ndims entries,
 * each >= 0); world in [1, 1 << 20].  Host only: touches no device.
 * On success *out receives a new plan.  FP_ERR_RANGE if T exceeds 2^62. */
fp_status fp_plan_create(int32_t n_tensors, const int32_t* ndims, const int64_t* shapes,
                         int32_t world, fp_plan** out);

/* Releases the plan and any device tables fp_pack attached to it.  The
 * caller must make sure no fp_pack on this plan is still running. */
void fp_plan_destroy(fp_plan* plan);

/* T, P and S of the plan (any output pointer may be NULL).  Host only. */
fp_status fp_plan_info(const fp_plan* plan, int64_t* numel, int64_t* padded, int64_t* shard);

/* ------------------------------------------------------------------ pack */

/* FlatParameter construction.  flat[o_i + k] = tensor_i[k] bit for bit,
 * o_i = sum of the numels before tensor i; flat[T, P) = 0.
 * elem_size: 2 (bf16 / fp16) or 4 (fp32); the copy is dtype-agnostic and
 * keeps every bit pattern (NaN payloads, -0).
 * src: host array of n_tensors device pointers, each to a contiguous
 *   row-major tensor aligned to elem_size; NULL only for empty tensors.
 * flat: device buffer of P elements, 16-byte aligned, not overlapping any
 *   source; NULL only when P = 0.
 * On its first call on a device the plan allocates and uploads its tensor
 * tables to that device (hipMalloc / pinned host staging; released by
 * fp_plan_destroy).  A call whose source pointers differ from the previous
 * call's uploads them on `stream` (waiting on the host only if that
 * previous upload has not finished); a call with the same pointers only
 * orders `stream` after it, and a call with the same arguments as the last
 * validated one skips the argument checks.  Calls that share a plan must be
 * ordered on one stream.  Not for graph capture.  A one-time set-up
 * operation per unit, not part of the per-step path. */
fp_status fp_pack(fp_plan* plan, int32_t elem_size, const void* const* src, void* flat,
                  void* stream);

/* ------------------------------------------------------------------ views */

/* Views of the original tensors on the flat buffer.  [DP] FSDP1 section,
 * use_orig_params paragraph: each original parameter points into the flat
 * buffer; on a rank it may be a piece of the tensor or empty.
 * rank == -1: the full view, buf_offset = o_i into the FlatParameter,
 *   numel = n_i, tensor_offset = 0, shape = the tensor's shape.
 * rank in [0, N_d): with lo = max(o_i, rank*S), hi = min(o_i + n_i,
 *   (rank+1)*S), a 1-D fragment when hi > lo: buf_offset = lo - rank*S
 *   into the shard, numel = hi - lo, tensor_offset = lo - o_i, ndim = 1,
 *   shape[0] = numel; otherwise an empty view (numel = 0, ndim = 1,
 *   shape[0] = 0, offsets 0).
 * One descriptor per tensor, in tensor order, written to out[0..n) where
 * n = number of tensors; FP_ERR_RANGE if cap < n (then *n_out = n and
 * nothing is written).  Host only. */
typedef struct fp_view {
    int32_t tensor;
    int32_t ndim;
    int64_t buf_offset;
    int64_t numel;
    int64_t tensor_offset;
    int64_t shape[FP_MAX_NDIM];
} fp_view;

fp_status fp_unpack_views(const fp_plan* plan, int32_t rank, fp_view* out, int32_t cap,
                          int32_t* n_out);

/* ------------------------------------------------------------------ reduce */

/* Size in bytes of the device workspace that fp_reduce_shard (for the
 * gradient norm) and fp_shard_step (norm and one-pass grid barrier) use for
 * a shard of S elements: a small header plus 8 bytes per 1024 elements.
 * The caller allocates it, zero-fills it once before its first use and then
 * passes it unchanged to later calls; every completed call leaves it
 * reusable.  Calls that may run concurrently need separate workspaces. */
int64_t fp_workspace_bytes(int64_t shard);

/* Byte offset, in the workspace, of a uint32 that counts grid-barrier waits
 * of the one-pass step that gave up (sticky: the library never clears it).
 * It stays 0 as long as the step's workgroups are co-resident, which the
 * library sizes the grid for; a caller that runs other kernels concurrently
 * on the GPU can check it, or pass FP_STEP_NO_COOP. */
#define FP_WORKSPACE_TIMEOUTS_OFFSET 8320

/* Bits of the device int32 overflow flag (found_inf).  Kernels only ever OR
 * bits into it; the caller zeroes it at the start of a step.  Any nonzero
 * value makes AdamW skip and counts as an overflow for fp_scaler_update.
 *   FP_FLAG_OVERFLOW -- a reduced gradient element was +-inf or NaN.
 *   FP_FLAG_GAVE_UP  -- the one-pass step's grid barrier gave up waiting
 *     (its workgroups were not resident together, e.g. because other
 *     kernels shared the GPU): that call stored no state, no own-shard
 *     element and no acc element that was an input, so the step was not
 *     taken.  The caller may clear this bit and run the call again with
 *     FP_STEP_NO_COOP. */
#define FP_FLAG_OVERFLOW 1
#define FP_FLAG_GAVE_UP 2

/* One micro-batch of the reduce-scatter arithmetic for this rank's shard.
 * [GUIDE] section 2 (equation for the averaged gradient): the synchronised
 * gradient is the mean of the N local gradients.  [DP] ZeRO-1 / ZeRO-2
 * paragraphs: reduce-scatter with averaging, each rank keeps its own
 * reduced slice.  [DP] Naive DP section: with n equal micro-batches each
 * loss is divided by n.  [FSDP] section 3.5: low-precision (bf16)
 * communication, high precision for the optimizer; sharded grad scaler.
 * For every i < S:
 *   s = bf16(grads[0][i]); s = s + bf16(grads[q][i]) for q = 1..N-1 in
 *   ascending order (fp32, round-to-nearest-even, no fused multiply-add);
 *   y = s * scale (fp32);  acc[i] = accumulate ? acc[i] + y : y.
 * Then FP_FLAG_OVERFLOW is OR-ed into *found_inf if any new acc[i] is
 * +-inf or NaN (it is never cleared: the caller zeroes it at the start of a
 * step, so the flag ORs over micro-batches), and, if sq_norm != NULL, *sq_norm = sum of
 * acc[i]^2 over the shard in fp64 (a fixed-order tree over a fixed grid:
 * bitwise reproducible run to run).
 * S >= 0; world in [1, FP_MAX_WORLD]; grads: host array of world device
 *   pointers to bf16[S] (rank q's gradient restricted to this shard's
 *   range); acc: device fp32[S], 16-byte aligned; found_inf: device int32,
 *   may be NULL; sq_norm: device double, may be NULL; workspace: device
 *   buffer of fp_workspace_bytes() bytes, needed only when sq_norm != NULL.
 *   scale is normally 1 / (N * n_micro). */
fp_status fp_reduce_shard(int64_t shard, int32_t world, const uint16_t* const* grads,
                          float scale, int32_t accumulate, float* acc, int32_t* found_inf,
                          double* sq_norm, void* workspace, void* stream);

/* The reduce of hybrid sharding with sharding factor F = group.  [FSDP]
 * section 3.3 and the sharding-factor bullet (groups of F GPUs fully shard,
 * the W / F groups replicate; F = 1 is DDP, F = W full sharding); [GUIDE]
 * HYBRID_SHARD row and tip (reduce-scatter inside the group, all-reduce
 * across groups).  The unit is planned with world = F (fp_plan_create), so
 * S = P / F and a rank at position p of its group owns slice p.  grads:
 * host array of world = W device pointers to the W ranks' bf16 gradients
 * over that slice; entry g * F + j is rank j of group g.  For each i:
 *   t_g = f32(g[gF][i]) + ... + f32(g[gF + F - 1][i])   (rank order, fp32)
 *   s = t_0 + t_1 + ... + t_{W/F - 1}                     (group order, fp32)
 *   y = s * scale (normally 1 / (W n)); acc as in fp_reduce_shard.
 * The two levels are the intra-group reduce-scatter and the inter-group
 * all-reduce, summed exactly in fp32 with no intermediate rounding; F = W
 * and F = 1 give fp_reduce_shard's order.  Everything else (flag, norm,
 * alignment, workspace) as fp_reduce_shard.  FP_ERR_RANGE unless F divides
 * W.  The AdamW, cast and unshard of a hybrid step are fp_adamw_shard and
 * fp_unshard with world = F. */
fp_status fp_reduce_shard_hybrid(int64_t shard, int32_t world, int32_t group, const uint16_t* const* grads,
                                 float scale, int32_t accumulate, float* acc, int32_t* found_inf,
                                 double* sq_norm, void* workspace, void* stream);

/* ------------------------------------------------------------------ adamw */

/* Hyperparameters in fp64; the library derives every coefficient in fp64. */
typedef struct fp_adamw_hparams {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int64_t step; /* t >= 1, the caller's count of steps taken (not skipped) */
} fp_adamw_hparams;

/* AdamW on the shard.  [DP] ZeRO-1 paragraph: AdamW is elementwise, so a
 * rank updates its slice from its averaged gradient and its own moments;
 * [DP] ZeRO figure legend and [GUIDE] section 7: fp32 master weights and
 * two fp32 moments (12 bytes per parameter).  For every i < S, evaluated in
 * fp64 from the fp32 values:
 *   theta = master[i] * (1 - lr * weight_decay)
 *   m = beta1 * exp_avg[i] + (1 - beta1) * g[i]
 *   v = beta2 * exp_avg_sq[i] + (1 - beta2) * g[i]^2
 *   theta = theta - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * (evaluated with the bias corrections folded into lr / (1 - beta1^t) and
 * 1 / sqrt(1 - beta2^t), derived once in fp64), and master, exp_avg,
 * exp_avg_sq are each rounded once to fp32.
 * If found_inf != NULL and *found_inf != 0 (read on the device) the update
 * is skipped: master / exp_avg / exp_avg_sq are left untouched.
 * If param_bf16 != NULL, param_bf16[i] = bf16 round-to-nearest-even of the
 * (new, or on a skip the unchanged) master[i] -- the low-precision copy
 * that the all-gather moves ([FSDP] section 3.5); usually full + rank * S.
 * If grad_coef != NULL (device double, read when the kernel starts), g[i]
 * above is grad[i] * *grad_coef: the unscale and clip factor of
 * fp_grad_coef ([FSDP] section 3.5, sharded gradient scaler).  It is
 * applied through the moment weights, (1 - beta1) k and (1 - beta2) k^2,
 * which equals multiplying the gradient up to fp64 rounding.
 * grad, master, exp_avg, exp_avg_sq: device fp32[S], 16-byte aligned,
 * master / exp_avg / exp_avg_sq distinct; param_bf16: device bf16[S]. */
fp_status fp_adamw_shard(int64_t shard, const fp_adamw_hparams* hp, const float* grad,
                         float* master, float* exp_avg, float* exp_avg_sq,
                         const int32_t* found_inf, uint16_t* param_bf16, const double* grad_coef,
                         void* stream);

/* ------------------------------------------------------------------ unshard */

/* The all-gather's data movement on one GPU: full[q*S + j] = shards[q][j]
 * for every q with shards[q] != NULL and every j < S (bit copy).  A NULL
 * entry leaves full[q*S, (q+1)*S) untouched (e.g. the rank's own shard,
 * already written by fp_adamw_shard).  [DP] ZeRO-1 paragraph (gather the
 * updated parameters) and ZeRO-3 paragraph (gather a unit before use);
 * [GUIDE] section 5.1 (all-gather shares the reduced chunks).
 * world in [1, FP_MAX_WORLD]; shards: host array of world device pointers
 * to bf16[S]; full: device bf16[world * S], not overlapping the sources. */
fp_status fp_unshard(int64_t shard, int32_t world, const uint16_t* const* shards,
                     uint16_t* full, void* stream);

/* ------------------------------------------------------------------ step */

#define FP_STEP_EXACT_SKIP 0 /* default: on overflow nothing is updated    */
#define FP_STEP_NO_SKIP 1    /* one fused pass; state updated regardless   */
#define FP_STEP_KEEP_GRAD 2  /* also leave the reduced gradient in acc     */
#define FP_STEP_NO_COOP 4    /* never use the cooperative one-pass kernel  */

/* One rank's whole shard step for the last micro-batch: reduce (as
 * fp_reduce_shard), AdamW with the bf16 cast into full + rank*S (as
 * fp_adamw_shard), and the copy of every other rank's shard into full (as
 * fp_unshard).  [DP] ZeRO-1 / ZeRO-2 step: reduce-scatter, update the
 * slice, all-gather the updated parameters; [FSDP] section 3.1.
 * flags:
 *   FP_STEP_EXACT_SKIP -- the overflow check over the whole shard (with the
 *     flag from earlier micro-batches) decides before any state is written;
 *     on overflow master / exp_avg / exp_avg_sq are untouched and full
 *     receives bf16 of the unchanged master.  When the shard fits the GPU's
 *     co-resident grid (S up to a few million elements) and a workspace
 *     is given, this runs as one kernel whose workgroups keep the reduced
 *     gradient in registers across a grid barrier (the overflow bit rides
 *     on the barrier's counters); otherwise as two kernels that pass the
 *     reduced gradient through acc.
 *   FP_STEP_NO_SKIP -- reduce and update in one pass without a gate; the
 *     flag is still reported (for callers without a loss scaler).
 *   FP_STEP_KEEP_GRAD (may be or-ed in) -- acc holds the reduced gradient
 *     afterwards; without it acc's contents afterwards are unspecified.
 *   FP_STEP_NO_COOP (may be or-ed in) -- use the two-kernel form even when
 *     the one-pass cooperative kernel would fit (for callers that share the
 *     GPU with concurrent kernels).
 * On return *found_inf is the OR of its input, this call's check
 * (FP_FLAG_OVERFLOW) and, from the one-pass kernel only, FP_FLAG_GAVE_UP
 * when its barrier gave up: then master / exp_avg / exp_avg_sq, full's own
 * slice and acc are as they were (the one-pass kernel is not chosen when
 * FP_STEP_KEEP_GRAD is combined with accumulate), the other shards may have
 * been copied, and the step can be run again with FP_STEP_NO_COOP after
 * clearing that bit.  The barrier decides for all workgroups alike, so no
 * call ever leaves a partly updated shard. */
typedef struct fp_step_args {
    int64_t shard;                 /* S */
    int32_t world;                 /* N_d, in [1, FP_MAX_WORLD] */
    int32_t rank;                  /* r, in [0, world) */
    const uint16_t* const* grads;  /* host array: world device ptrs, bf16[S] */
    float scale;                   /* normally 1 / (N_d * n_micro) */
    int32_t accumulate;            /* 1 if acc holds earlier micro-batches */
    float* acc;                    /* device fp32[S], 16-byte aligned */
    float* master;                 /* device fp32[S] */
    float* exp_avg;                /* device fp32[S] */
    float* exp_avg_sq;             /* device fp32[S] */
    fp_adamw_hparams hp;
    const uint16_t* const* shards; /* host array: world device ptrs, bf16[S]; entry rank unused */
    uint16_t* full;                /* device bf16[world * S] */
    int32_t* found_inf;            /* device int32, required */
    double* sq_norm;               /* device double, may be NULL */
    void* workspace;               /* device, fp_workspace_bytes(S), zero-filled before first
                                      use; NULL disables the norm and the one-pass path */
    int32_t flags;
    /* NULL, or a host array of FP_STEP_EVENTS hipEvent_t (as void*) that the
     * call records on `stream`: before its first kernel, between its first
     * and second kernel, and after its last kernel -- per-kernel timing. */
    void* const* profile_events;
    /* device double or NULL: the gradient factor of fp_adamw_shard, read
     * when the step's kernels start, so it cannot depend on this step's own
     * norm (for clipping by it, use fp_reduce_shard, fp_grad_coef and
     * fp_adamw_shard) -- the loss scaler's unscale factor, typically. */
    const double* grad_coef;
    /* All three NULL (the state is updated in place), or all three device
     * fp32[S], distinct from every other buffer of the call: the speculative
     * form of the step.  The new master / exp_avg / exp_avg_sq go to these
     * buffers and master / exp_avg / exp_avg_sq are only read, so the
     * update need not wait for the overflow check.  With FP_STEP_EXACT_SKIP,
     * on overflow the outputs receive the unchanged input state (and full
     * the bf16 of the unchanged master), which is the skipped step's result;
     * the caller swaps input and output buffers after each step either way.
     * With FP_STEP_NO_SKIP the outputs receive the update regardless.  A
     * shard that fits the one-pass kernel (workspace given) takes it with
     * the outputs as store targets (FP_PATH_SPECULATIVE_ONE_PASS). */
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
} fp_step_args;

#define FP_STEP_EVENTS 3

fp_status fp_shard_step(const fp_step_args* args, void* stream);

/* The kernels fp_shard_step launches for these arguments on the current
 * device, after the same argument checks (nothing is launched).  With the
 * output state buffers given, FP_STEP_EXACT_SKIP always takes one of the
 * speculative paths, FP_STEP_NO_SKIP the no-skip ones:
 *   FP_PATH_ONE_PASS  -- one kernel (then the norm finalisation if sq_norm);
 *   FP_PATH_TWO_PHASE -- reduce + copy kernel, then the AdamW kernel;
 *   FP_PATH_NO_SKIP   -- one fused kernel (then the norm finalisation if
 *                        sq_norm);
 *   FP_PATH_NO_SKIP_SPLIT -- the no-skip step of a shard of 2^24 elements
 *                        or more: the fused reduce + AdamW + cast kernel at
 *                        reduced occupancy, then the copy of the other
 *                        shards in a kernel of its own (then the norm
 *                        finalisation if sq_norm).
 *   FP_PATH_SPECULATIVE   -- exact skip with separate output state: the
 *                        kernels of FP_PATH_NO_SKIP writing the outputs,
 *                        then a kernel that, on overflow only, copies the
 *                        input state to the outputs and recasts the own
 *                        shard; the step moves the bytes of the no-skip
 *                        step plus one small launch.
 *   FP_PATH_SPECULATIVE_SPLIT -- the same from 2^24 elements on, with the
 *                        kernels of FP_PATH_NO_SKIP_SPLIT.
 *   FP_PATH_SPECULATIVE_ONE_PASS -- exact skip with separate output state
 *                        on the one-pass kernel (when it fits, as for
 *                        FP_PATH_ONE_PASS): after the barrier the kernel
 *                        stores the new state to the outputs, or on overflow
 *                        copies the input state to them; no restore launch.
 * The one-pass choice depends on the device's co-resident capacity, hence
 * on the device current at the call. */
#define FP_PATH_ONE_PASS 0
#define FP_PATH_TWO_PHASE 1
#define FP_PATH_NO_SKIP 2
#define FP_PATH_NO_SKIP_SPLIT 3
#define FP_PATH_SPECULATIVE 4
#define FP_PATH_SPECULATIVE_SPLIT 5
#define FP_PATH_SPECULATIVE_ONE_PASS 6
fp_status fp_step_path(const fp_step_args* args, int32_t* path);

/* For tests of the one-pass kernel's give-up path.  Runs fp_shard_step's
 * one-pass kernel (FP_ERR_INVALID unless fp_step_path would return
 * FP_PATH_ONE_PASS or FP_PATH_SPECULATIVE_ONE_PASS for these arguments)
 * with a grid barrier that waits for one workgroup more than the launch
 * holds and gives up after 64 polls, so every wait gives up and the kernel
 * ends normally: the result is the FP_FLAG_GAVE_UP outcome described above
 * (with output state buffers, the outputs are not written either).  The
 * barrier's counters are left mid-generation: zero-fill the workspace
 * before passing it to another call. */
fp_status fp_step_test_give_up(const fp_step_args* args, void* stream);

/* fp_shard_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same kernels and results as fp_shard_step with a workspace, but the
 * step's scratch (the one-pass grid barrier's state and the norm partials)
 * is a 2 MiB array inside the library, one per GPU, held until the process
 * ends; the call allocates nothing.  args->workspace must be NULL
 * (FP_ERR_INVALID otherwise).  With sq_norm, shards of more than
 * 266,337,283 elements need more partials than the array holds:
 * FP_ERR_RANGE before anything is enqueued.  The first call on a device
 * takes the array's device address and enqueues a small kernel that clears
 * the barrier state (again on later calls while that one was captured into
 * a graph).  Every call on a GPU shares that GPU's array: calls that may
 * overlap on one GPU (concurrent streams, graphs replayed concurrently)
 * race and must not be issued. */
fp_status fp_shard_step_noalloc(const fp_step_args* args, void* stream);

/* ------------------------------------------------------------------ units */

/* Many units (for example the ~25 MB DDP buckets of a model, or a model's
 * FSDP units) stepped together, one launch per stage for all of them.  A
 * rank's optimizer state is one fp32 partition holding every unit's shard:
 * [DP] ZeRO-1 / ZeRO-2 (each rank keeps one slice of the whole state);
 * [GUIDE] section 4.2 (gradients are reduced bucket by bucket).
 *
 * fp_units_create: n_units >= 1 units of one rank `rank` in a group of
 * `world`.  shard: host array of n_units shard sizes S_u >= 0.
 * grads: host array of n_units * world device pointers; entry u * world + q
 *   is rank q's bf16 gradient over this rank's shard of unit u (bf16[S_u]).
 * shards, full: both NULL (a plan that only reduces) or: shards a host array
 *   of n_units * world device pointers, entry u * world + q rank q's bf16
 *   shard of unit u (entry rank ignored); full a host array of n_units
 *   device pointers, unit u's gathered bf16[world * S_u].
 * The pointers are fixed for the plan's life (create one plan per set of
 * gradient buffers).  Unit u's fp32 shard sits in the partition at element
 * offset_u = sum over v < u of S_v rounded up to a multiple of 4
 * (fp_units_offsets); the partition has fp_units_info's `partition`
 * elements.  Creation allocates and fills a small device table on the
 * current device with a synchronous copy (a set-up call: not for graph
 * capture); calls must be made with that device current.
 * Errors: FP_ERR_RANGE (n_units, world, rank, sizes), FP_ERR_INVALID (NULL
 * pointers, a source overlapping its unit's full buffer), FP_ERR_ALIGN (bf16
 * pointers need 2-byte alignment), FP_ERR_DEVICE (allocation / copy). */
typedef struct fp_units fp_units;
fp_status fp_units_create(int32_t n_units, int32_t world, int32_t rank, const int64_t* shard,
                          const uint16_t* const* grads, const uint16_t* const* shards,
                          uint16_t* const* full, fp_units** out);
void fp_units_destroy(fp_units* units);
/* partition: elements of the rank's fp32 partition; workspace_bytes: the
 * workspace fp_units_reduce / fp_units_step need for the norm.  Either
 * output may be NULL. */
fp_status fp_units_info(const fp_units* units, int64_t* partition, int64_t* workspace_bytes);
/* offsets: host array of n_units elements, receives offset_u. */
fp_status fp_units_offsets(const fp_units* units, int64_t* offsets);

/* One micro-batch's reduce over all units in one launch: fp_reduce_shard's
 * arithmetic on every unit, into acc (device fp32[partition], 16-byte
 * aligned; unit u at offset_u).  found_inf, sq_norm, workspace as there
 * (workspace of fp_units_info's size). */
fp_status fp_units_reduce(const fp_units* units, float scale, int32_t accumulate, float* acc,
                          int32_t* found_inf, double* sq_norm, void* workspace, void* stream);

/* The last micro-batch's step over all units: fp_shard_step's arithmetic on
 * every unit, with one overflow flag for the whole step (a non-finite value
 * in any unit skips the update of every unit).  FP_STEP_EXACT_SKIP runs two
 * launches (reduce + copies of every unit's other shards, then AdamW and
 * the casts into each unit's full + rank * S_u); FP_STEP_NO_SKIP one fused
 * launch; FP_STEP_KEEP_GRAD may be or-ed in.  acc, master, exp_avg,
 * exp_avg_sq: device fp32[partition], 16-byte aligned.  profile_events as
 * in fp_step_args.  Requires a plan made with shards and full.
 * master_out / exp_avg_out / exp_avg_sq_out: all NULL (in place) or all
 * three device fp32[partition], 16-byte aligned, distinct from every other
 * buffer: the speculative form, as in fp_step_args -- the fused launch
 * writes the update of every unit to these partitions without waiting for
 * the overflow check and, with FP_STEP_EXACT_SKIP, a last kernel copies the
 * input state to them (and recasts every own slice) when the flag is set,
 * so the result is the exact-skip step's; the caller swaps input and output
 * partitions after each step.  The step then moves no reduced gradient
 * through acc (with FP_STEP_KEEP_GRAD it is still written there). */
typedef struct fp_units_step_args {
    float scale;
    int32_t accumulate;
    float* acc;
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    fp_adamw_hparams hp;
    int32_t* found_inf;            /* device int32, required */
    double* sq_norm;               /* device double, may be NULL */
    void* workspace;               /* device, needed with sq_norm */
    int32_t flags;
    void* const* profile_events;
    const double* grad_coef;       /* as in fp_step_args, may be NULL */
    float* master_out;             /* NULL, or with the next two the output partitions */
    float* exp_avg_out;
    float* exp_avg_sq_out;
} fp_units_step_args;
fp_status fp_units_step(const fp_units* units, const fp_units_step_args* args, void* stream);

/* The launches fp_units_step makes for these arguments, after the same
 * argument checks (host only, nothing launched): FP_PATH_TWO_PHASE (exact
 * skip in place), FP_PATH_NO_SKIP / FP_PATH_SPECULATIVE (one fused launch
 * with the copies of the other shards, then for the speculative form the
 * restore kernel), or FP_PATH_NO_SKIP_SPLIT / FP_PATH_SPECULATIVE_SPLIT for
 * partitions of 2^24 elements and more: the fused reduce + AdamW + cast
 * launch, then the copies in a launch of their own. */
fp_status fp_units_step_path(const fp_units* units, const fp_units_step_args* args, int32_t* path);

/* ------------------------------------------------------------------ dim-0 */

/* Per-parameter sharding along dim 0.  [DP] FSDP2 sections and the
 * FSDP1 / FSDP2 comparison figure: every parameter of a group is cut along
 * its first dimension over the N_d ranks and keeps its global shape; a
 * rank's pieces of the group's parameters travel together in one buffer.
 * Geometry, for parameter i of shape (d0, ...) with r_i = product of the
 * other dims (1 for a 0-d parameter, which counts as one row of one element):
 *   c_i = ceil(d0 / N_d) rows per rank; rank q holds rows
 *   [q c_i, min((q+1) c_i, d0)) of it, the rest of its c_i rows are zero;
 *   off_i = sum over j < i of c_j r_j;  S = sum of c_i r_i.
 * Rank q's buffer holds its chunk of parameter i at [off_i, off_i + c_i r_i)
 * (row-major, padding rows last); the gathered buffer is the N_d ranks'
 * buffers one after the other, bf16 or fp32 [N_d * S].  Padding rows are
 * the plainest reading where d0 is not a multiple of N_d (the pages show
 * only even splits). */
typedef struct fp_shard0_plan fp_shard0_plan;

/* n_params >= 1 parameters, ndims / shapes as in fp_plan_create; world in
 * [1, 1 << 20].  Host only.  FP_ERR_RANGE when a dim exceeds 2^40 or S
 * exceeds 2^40 elements. */
fp_status fp_shard0_plan_create(int32_t n_params, const int32_t* ndims, const int64_t* shapes,
                                int32_t world, fp_shard0_plan** out);
/* Releases the plan and the device tables its calls attached to it (the
 * caller makes sure none of its calls is still running). */
void fp_shard0_plan_destroy(fp_shard0_plan* plan);
/* shard: S; numel: sum of the parameters' numels (either may be NULL). */
fp_status fp_shard0_plan_info(const fp_shard0_plan* plan, int64_t* shard, int64_t* numel);
/* Rank `rank`'s local piece of every parameter, one descriptor per
 * parameter written to out[0..n): buf_offset = off_i into the rank's buffer,
 * numel = real rows * r_i, tensor_offset = q c_i r_i into the flattened
 * parameter (0 when empty), shape = (real rows, other dims...) -- the local
 * shape, 2-D or more kept (a 0-d parameter has ndim 1).  FP_ERR_RANGE if
 * cap < n (then *n_out = n) or rank outside [0, N_d).  Host only. */
fp_status fp_shard0_views(const fp_shard0_plan* plan, int32_t rank, fp_view* out, int32_t cap,
                          int32_t* n_out);

/* Rank `rank`'s buffer of the group from the full parameters:
 * dst[off_i + k] = param_i[q c_i r_i + k] for the real rows, 0 for the
 * padding rows.  rank == -1 writes every rank's buffer: dst is then the
 * gathered layout, [N_d * S].  elem_size 2 or 4, bits copied as they are.
 * params: host array of n_params device pointers (contiguous, row-major,
 * aligned to elem_size; NULL only for empty parameters); dst: device
 * buffer aligned to elem_size, not overlapping any parameter.
 * The first call of an (operation, elem_size, rank) on a device builds and
 * uploads that call's segment tables (hipMalloc, synchronous copies; kept
 * until fp_shard0_plan_destroy).  A call whose pointers differ from the
 * previous call's of the same table uploads them on `stream` from pinned
 * staging, waiting on the host only if that previous upload has not
 * finished; a call with the same pointers only orders `stream` after that
 * upload.  The device pointer table is shared by the calls of a table: order
 * the calls of one plan on one stream (a lock serialises the host side).
 * Not for graph capture. */
fp_status fp_shard0_pack(fp_shard0_plan* plan, int32_t elem_size, int32_t rank,
                         const void* const* params, void* dst, void* stream);

/* After the all-gather: every parameter at its global shape from the
 * gathered buffer: param_i[q c_i r_i + k] = full[q S + off_i + k] for every
 * rank q and real row (padding rows are dropped).  full: device [N_d * S],
 * aligned to elem_size; params as in fp_shard0_pack but written, none
 * overlapping full or each other.  Tables and staging as in
 * fp_shard0_pack. */
fp_status fp_shard0_unpack(fp_shard0_plan* plan, int32_t elem_size, const void* full,
                           void* const* params, void* stream);

/* ------------------------------------------------------------------ reshard */

/* Resharding a flat buffer from N to N' ranks: [DP] section
 * "Checkpoint：让各张卡保存自己的分片" (a sharded checkpoint may be loaded
 * into a different number of ranks).  The flat buffer of T elements is cut into N shards of
 * S = ceil(T / N) (old rank q holds flat[qS, (q+1)S), zeros past T) and is to
 * be cut into N' shards of S' = ceil(T / N').  New rank q' receives
 * flat[q'S' + k] for k < S', read from the old shards, and zeros past T
 * (the old shards' padding is never read).  The same copy serves the fp32
 * master and moments (elem_size 4) and the bf16 parameters (elem_size 2) of
 * a FlatParameter; the geometry is fp_plan's (T, world), so S and S' are the
 * shard sizes fp_plan_info reports for N and N'.
 * fp_reshard_plan_create: T in [0, 2^40], N and N' in [1, 2^20]; host only.
 * fp_reshard: new_rank in [0, N') writes that rank's S' elements to dst;
 *   new_rank = -1 writes every new rank's shard, dst = N' * S' elements.
 *   old_shards: host array of N device pointers to S elements each, aligned
 *   to elem_size (entries of old ranks that hold only padding may be NULL);
 *   dst: device, aligned to elem_size, not overlapping the old shards.
 *   Device tables, pointer uploads, validation caching and stream rules as
 *   in fp_shard0_pack. */
typedef struct fp_reshard_plan fp_reshard_plan;
fp_status fp_reshard_plan_create(int64_t numel, int32_t world_old, int32_t world_new, fp_reshard_plan** out);
void fp_reshard_plan_destroy(fp_reshard_plan* plan);
fp_status fp_reshard_plan_info(const fp_reshard_plan* plan, int64_t* shard_old, int64_t* shard_new);
fp_status fp_reshard(fp_reshard_plan* plan, int32_t elem_size, int32_t new_rank, const void* const* old_shards,
                     void* dst, void* stream);

/* ------------------------------------------------------------ no_sync, scaler */

/* Gradient accumulation without communication.  [DP] "Naive Data
 * Parallelism", gradient-accumulation paragraph: the first micro-batches'
 * gradients are accumulated locally and only the last micro-batch
 * synchronises (DDP's no_sync); [FSDP] section 3.4: accumulation without
 * communication trades memory for fewer exchanges.  A rank keeps an fp32
 * buffer `local` over its whole unit (n elements, 4 bytes each):
 *   fp_local_accumulate: local[i] = (accumulate ? local[i] : 0) + f32(grad[i])
 *     for each micro-batch but the last, in micro-batch order;
 *   fp_local_finish: out[i] = bf16(local[i] + f32(grad[i])) (or bf16 of
 *     grad[i] alone when accumulate == 0) for the last one, round to nearest
 *     even: the bf16 row this rank contributes to the reduce-scatter, which
 *     then runs as fp_reduce_shard / fp_shard_step with the usual scale
 *     1 / (N_d n).  With one micro-batch the row is the gradient itself and
 *     this call is not needed.
 * grad, out: device bf16[n] (2-byte aligned); local: device fp32[n], 16-byte
 * aligned; out may not overlap local or grad.  n >= 0. */
fp_status fp_local_accumulate(int64_t n, const uint16_t* grad, int32_t accumulate, float* local,
                              void* stream);
fp_status fp_local_finish(int64_t n, const uint16_t* grad, int32_t accumulate, const float* local,
                          uint16_t* out, void* stream);

/* The factor AdamW applies to a loss-scaled reduced gradient (device
 * double *coef): 1 / scale with scale = *loss_scale (1 when loss_scale is
 * NULL), times min(1, max_norm / (||g|| + 1e-6)) with ||g|| =
 * sqrt(*sq_norm) / scale when max_norm > 0 (global-norm clipping; sq_norm
 * then required: this rank's Sum g^2 from the reduce, or the sum over ranks
 * after their exchange).  [FSDP] section 3.5 (sharded gradient scaler); the
 * pages give no policy, so the usual unscale-then-clip rule is used.  One
 * lane, enqueued on `stream`. */
fp_status fp_grad_coef(const double* sq_norm, const float* loss_scale, double max_norm, double* coef,
                       void* stream);

/* Dynamic loss scaling after a step's overflow decision (device values):
 * if *found_inf != 0, *scale *= backoff_factor and *clean_steps = 0;
 * otherwise ++*clean_steps, and when it reaches growth_interval,
 * *scale *= growth_factor and *clean_steps = 0 (fp32 arithmetic).  The usual
 * defaults are 2.0, 0.5 and 2000.  [FSDP] section 3.5; the policy is not on
 * the pages.  growth_interval >= 1, factors > 0.  One lane, on `stream`. */
fp_status fp_scaler_update(const int32_t* found_inf, float* scale, int32_t* clean_steps, float growth_factor,
                           float backoff_factor, int32_t growth_interval, void* stream);

/* ------------------------------------------------------------------ helpers */

/* Model-state bytes per GPU.  [DP] ZeRO figure (one formula per row) and
 * [GUIDE] sections 6.1 and 7: parameters and gradients 2 bytes each,
 * optimizer state k bytes per parameter, N = world:
 *   stage 0 (replicated, DDP): 2psi + 2psi + k psi
 *   stage 1 (optimizer state sharded): 2psi + 2psi + k psi / N
 *   stage 2 (+ gradients): 2psi + (2psi + k psi) / N
 *   stage 3 (+ parameters, FSDP full shard): (2psi + 2psi + k psi) / N
 * FP_ERR_INVALID for another stage, psi < 0, k < 0 or world < 1. */
fp_status fp_state_bytes(double psi, int32_t world, double k, int32_t stage, double* out);

/* Static text for a status code. */
const char* fp_status_string(fp_status status);

/* Message of the calling thread's most recent failed call ("" if none). */
const char* fp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLATPARAM_H */
