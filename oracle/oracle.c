/*
 * oracle.c -- plain, serial CPU oracle for one rank's FSDP / ZeRO shard step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source with the GPU path.
 *
 * Every routine is the plainest loop that computes what the cited passage
 * defines: no blocking, no vectorisation by hand, no reordering.  Build with
 * -O2 -ffp-contract=off and no fast-math (oracle/build.py), so every float
 * operation below is one IEEE-754 round-to-nearest-even operation in the
 * type it is written in.
 *
 * Pages cited (by title, then section / figure / equation):
 *   [DP]   "Infra: Data Parallel" (pufanyi.com)
 *   [FSDP] "PyTorch FSDP: 大模型分布式训练的工业级分片并行方案" (2048ai.net,
 *          summary of Zhao et al., PyTorch FSDP, VLDB 2023)
 *   [GUIDE] "4.1 数据并行详解" (AIInfraGuide)
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes of the repository):
 *   - padding: zeros appended after the last tensor up to a multiple of the
 *     world size; no per-tensor alignment padding;
 *   - the N rank gradients are summed in ascending rank order in fp32,
 *     starting from rank 0's value, then multiplied by one fp32 scale
 *     (normally 1/(N * n_micro)) and, from the second micro-batch on, added
 *     to the fp32 accumulator;
 *   - AdamW is decoupled-weight-decay Adam with bias correction, the decay
 *     multiplied by the learning rate, epsilon added outside the square
 *     root; it is evaluated in fp64 from the fp32 state and the decimal
 *     hyperparameters, and each of master, exp_avg, exp_avg_sq is rounded
 *     once to fp32;
 *   - the cast to bf16 is round-to-nearest, ties to even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* FlatParameter geometry and packing.                                      */
/* [DP] section "FSDP1: pack first, then split" and its figure: the unit's  */
/* tensors are flattened and concatenated into one 1-D FlatParameter that   */
/* is split evenly over the ranks; a shard may cut through a tensor.        */
/* [DP] ZeRO figure: GPU i keeps slice i.                                   */
/* ------------------------------------------------------------------------ */

/* T = total elements, P = T rounded up to a multiple of world, S = P/world. */
void or_geometry(int32_t n_tensors, const int64_t* numel, int32_t world,
                 int64_t* total, int64_t* padded, int64_t* shard)
{
    int64_t t = 0;
    for (int32_t i = 0; i < n_tensors; ++i)
        t += numel[i];
    int64_t p = ((t + world - 1) / world) * world;
    *total = t;
    *padded = p;
    *shard = p / world;
}

/* flat[o_i + k] = tensor_i[k] bit for bit (row-major flatten), o_i the sum of
 * the sizes of the tensors before i; flat[T..P) = 0.  elem_size is 2 or 4. */
void or_pack(int32_t n_tensors, const int64_t* numel, int32_t elem_size,
             const void* const* src, int32_t world, void* flat)
{
    int64_t t, p, s;
    or_geometry(n_tensors, numel, world, &t, &p, &s);
    unsigned char* out = (unsigned char*)flat;
    int64_t pos = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        const unsigned char* in = (const unsigned char*)src[i];
        for (int64_t k = 0; k < numel[i] * elem_size; ++k)
            out[pos * elem_size + k] = in[k];
        pos += numel[i];
    }
    for (int64_t k = pos * elem_size; k < p * elem_size; ++k)
        out[k] = 0;
}

/* For flat positions pos[0..m) given in ascending order, the tensor that
 * holds each one and the element offset inside it; tensor = -1 marks a
 * padding position.  One merge pass over the tensors. */
void or_locate_sorted(int32_t n_tensors, const int64_t* numel, int64_t m,
                      const int64_t* pos, int32_t* tensor, int64_t* offset)
{
    int32_t i = 0;
    int64_t start = 0;
    for (int64_t j = 0; j < m; ++j) {
        while (i < n_tensors && pos[j] >= start + numel[i]) {
            start += numel[i];
            ++i;
        }
        if (i < n_tensors) {
            tensor[j] = i;
            offset[j] = pos[j] - start;
        } else {
            tensor[j] = -1;
            offset[j] = pos[j] - start;
        }
    }
}

/* Views of the original tensors.  [DP] FSDP1 section (use_orig_params): the
 * original parameters point into the flat buffer; on a rank they may be only
 * a piece of the tensor, or empty when the rank holds none of it.
 * rank == -1: the full view of tensor i is flat[o_i, o_i + n_i).
 * rank == q : lo = max(o_i, qS), hi = min(o_i + n_i, (q+1)S); a 1-D fragment
 *             at shard offset lo - qS holding tensor elements [lo-o_i, hi-o_i)
 *             when hi > lo, else an empty view (length 0, offsets 0).
 * Returns the number of descriptors written (= n_tensors). */
int32_t or_views(int32_t n_tensors, const int64_t* numel, int32_t world,
                 int32_t rank, int64_t* buf_offset, int64_t* length,
                 int64_t* tensor_offset)
{
    int64_t t, p, s;
    or_geometry(n_tensors, numel, world, &t, &p, &s);
    int64_t o = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (rank < 0) {
            buf_offset[i] = o;
            length[i] = numel[i];
            tensor_offset[i] = 0;
        } else {
            int64_t lo = o > (int64_t)rank * s ? o : (int64_t)rank * s;
            int64_t end = o + numel[i];
            int64_t shard_end = ((int64_t)rank + 1) * s;
            int64_t hi = end < shard_end ? end : shard_end;
            if (hi > lo) {
                buf_offset[i] = lo - (int64_t)rank * s;
                length[i] = hi - lo;
                tensor_offset[i] = lo - o;
            } else {
                buf_offset[i] = 0;
                length[i] = 0;
                tensor_offset[i] = 0;
            }
        }
        o += numel[i];
    }
    return n_tensors;
}

/* ------------------------------------------------------------------------ */
/* Per-parameter dim-0 sharding.  [DP] FSDP2 section and its figure: each   */
/* parameter is split along dim 0 over the ranks and keeps its global      */
/* shape; three (4,2) weights over 2 ranks give every rank the first (or    */
/* last) two rows of each weight, local shape (2,2), 12 elements per rank; */
/* [DP] "FSDP2: record each parameter's shard": an (8,4) weight over 4     */
/* ranks gives a local (2,4).  Parameters of one group still travel       */
/* together: a rank's shards of the group's parameters are concatenated    */
/* into one buffer for the group's collectives.                             */
/* Reading for splits the pages do not show: chunks of c = ceil(d0/world)  */
/* rows, rank q holding rows [q*c, min((q+1)*c, d0)); each rank's chunk is  */
/* padded with zero rows to c rows so that every rank's buffer has the same */
/* size S = sum_i c_i * r_i (r_i = elements per row, the product of the     */
/* other dimensions).  A 0-d parameter is one row of one element.           */
/* ------------------------------------------------------------------------ */

/* Per parameter: chunk rows c_i, row length r_i and offset in a rank's
 * buffer; *shard = S. */
void or_shard0_geometry(int32_t n, const int32_t* ndims, const int64_t* shapes,
                        int32_t world, int64_t* rows, int64_t* row_elems,
                        int64_t* offset, int64_t* shard)
{
    int64_t d = 0, o = 0;
    for (int32_t i = 0; i < n; ++i) {
        int64_t d0 = ndims[i] > 0 ? shapes[d] : 1;
        int64_t r = 1;
        for (int32_t k = 1; k < ndims[i]; ++k)
            r *= shapes[d + k];
        d += ndims[i];
        rows[i] = (d0 + world - 1) / world;
        row_elems[i] = r;
        offset[i] = o;
        o += rows[i] * r;
    }
    *shard = o;
}

/* Rows of a chunk of c rows that rank q really holds out of d0. */
static int64_t or_shard0_real_rows(int64_t d0, int64_t c, int32_t q)
{
    int64_t left = d0 - (int64_t)q * c;
    return left < 0 ? 0 : (left < c ? left : c);
}

static int64_t or_dim0(const int32_t* ndims, const int64_t* shapes, int32_t i)
{
    int64_t d = 0;
    for (int32_t j = 0; j < i; ++j)
        d += ndims[j];
    return ndims[i] > 0 ? shapes[d] : 1;
}

/* Rank `rank`'s buffer: for each parameter its real rows (row-major, bit for
 * bit) followed by zero rows up to c_i rows. */
void or_shard0_pack(int32_t n, const int32_t* ndims, const int64_t* shapes,
                    int32_t world, int32_t elem_size, int32_t rank,
                    const void* const* src, void* dst)
{
    int64_t c[n > 0 ? n : 1], r[n > 0 ? n : 1], off[n > 0 ? n : 1], S;
    or_shard0_geometry(n, ndims, shapes, world, c, r, off, &S);
    unsigned char* out = (unsigned char*)dst;
    for (int32_t i = 0; i < n; ++i) {
        int64_t d0 = or_dim0(ndims, shapes, i);
        int64_t real = or_shard0_real_rows(d0, c[i], rank) * r[i];
        const unsigned char* in = (const unsigned char*)src[i] + (int64_t)rank * c[i] * r[i] * elem_size;
        for (int64_t k = 0; k < real * elem_size; ++k)
            out[off[i] * elem_size + k] = in[k];
        for (int64_t k = real * elem_size; k < c[i] * r[i] * elem_size; ++k)
            out[off[i] * elem_size + k] = 0;
    }
}

/* The inverse after a gather: full = the world ranks' buffers one after the
 * other; parameter i's row j comes from rank j / c_i, row j % c_i of that
 * rank's chunk.  Padding rows are dropped. */
void or_shard0_unpack(int32_t n, const int32_t* ndims, const int64_t* shapes,
                      int32_t world, int32_t elem_size, const void* full,
                      void* const* dst)
{
    int64_t c[n > 0 ? n : 1], r[n > 0 ? n : 1], off[n > 0 ? n : 1], S;
    or_shard0_geometry(n, ndims, shapes, world, c, r, off, &S);
    const unsigned char* in = (const unsigned char*)full;
    for (int32_t i = 0; i < n; ++i) {
        int64_t d0 = or_dim0(ndims, shapes, i);
        unsigned char* out = (unsigned char*)dst[i];
        for (int64_t j = 0; j < d0; ++j) {
            int64_t q = j / c[i], jj = j % c[i];
            const unsigned char* row = in + (q * S + off[i] + jj * r[i]) * elem_size;
            for (int64_t k = 0; k < r[i] * elem_size; ++k)
                out[j * r[i] * elem_size + k] = row[k];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Resharding a flat buffer from N to N' ranks.  [DP] section             */
/* "Checkpoint：让各张卡保存自己的分片": a sharded checkpoint may be loaded  */
/* into a different number of ranks.  The flat buffer (T elements, then zero padding) is the same;  */
/* only the cut changes: new rank q' holds flat[q'S', (q'+1)S'), read from  */
/* the old shards (old rank q holds flat[qS, (q+1)S)), zeros past T.        */
/* new_rank = -1 writes every new rank's shard, one after the other.        */
/* ------------------------------------------------------------------------ */

void or_reshard(int64_t t, int32_t world_old, int32_t world_new, int32_t elem_size, int32_t new_rank,
                const void* const* old_shards, void* out)
{
    int64_t s_old = (t + world_old - 1) / world_old;
    int64_t s_new = (t + world_new - 1) / world_new;
    int32_t q0 = new_rank < 0 ? 0 : new_rank;
    int32_t q1 = new_rank < 0 ? world_new : new_rank + 1;
    unsigned char* o = (unsigned char*)out;
    int64_t k = 0;
    for (int32_t q = q0; q < q1; ++q) {
        for (int64_t j = 0; j < s_new; ++j, ++k) {
            int64_t e = (int64_t)q * s_new + j;
            if (e < t) {
                const unsigned char* src = (const unsigned char*)old_shards[e / s_old];
                memcpy(o + k * elem_size, src + (e % s_old) * elem_size, (size_t)elem_size);
            } else {
                memset(o + k * elem_size, 0, (size_t)elem_size);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32.  A bf16 value is the upper half of an fp32 bit pattern.   */
/* ------------------------------------------------------------------------ */

float or_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round to nearest, ties to even, on the 16 dropped bits.  NaN stays NaN
 * (quiet bit set, sign kept); values that round past the largest finite
 * bf16 become infinity through the carry into the exponent. */
uint16_t or_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)(upper | 0x0040u);
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

void or_f32_to_bf16_array(int64_t n, const float* x, uint16_t* y)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = or_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Reduce-scatter arithmetic for this rank's shard.                         */
/* [GUIDE] section 2, equation for g-bar: the synchronised gradient is the  */
/* mean, not the sum, of the N local gradients.  [DP] ZeRO-1/ZeRO-2         */
/* paragraphs: reduce-scatter with averaging leaves each rank only its own  */
/* reduced slice.  [DP] "Naive Data Parallelism": with n equal micro-       */
/* batches each loss is divided by n.  [FSDP] section 3.5: communication in */
/* low precision (bf16 here), high precision (fp32) for the optimizer.      */
/* grads[q] points at rank q's bf16 gradient restricted to this shard.      */
/* ------------------------------------------------------------------------ */

void or_reduce(int64_t shard, int32_t world, const uint16_t* const* grads,
               float scale, int32_t accumulate, float* acc)
{
    for (int64_t i = 0; i < shard; ++i) {
        float sum = or_bf16_to_f32(grads[0][i]);
        for (int32_t q = 1; q < world; ++q)
            sum = sum + or_bf16_to_f32(grads[q][i]);
        float y = sum * scale;
        if (accumulate)
            acc[i] = acc[i] + y;
        else
            acc[i] = y;
    }
}

/* Hybrid sharding with factor F ([FSDP] section 3.3 and the sharding-factor */
/* bullet: groups of F GPUs fully shard, the W/F groups replicate; [GUIDE]  */
/* HYBRID_SHARD: reduce-scatter inside the group, all-reduce across the     */
/* groups).  The unit is split into F slices; rank (group g, position p)    */
/* owns slice p, and its reduced gradient averages all W ranks' gradients   */
/* of that slice in two levels: each group's F gradients summed in rank     */
/* order, then the W/F group sums in group order, then one multiply by the  */
/* scale (1/(W n)).  grads[g*F + j] is rank j of group g.  F = W (one group) */
/* and F = 1 (one rank per group) are the flat rank order above.            */
void or_reduce_hybrid(int64_t shard, int32_t world, int32_t group, const uint16_t* const* grads,
                      float scale, int32_t accumulate, float* acc)
{
    int32_t n_groups = world / group;
    for (int64_t i = 0; i < shard; ++i) {
        float total = 0.0f;
        for (int32_t g = 0; g < n_groups; ++g) {
            float part = or_bf16_to_f32(grads[g * group][i]);
            for (int32_t j = 1; j < group; ++j)
                part = part + or_bf16_to_f32(grads[g * group + j][i]);
            total = g == 0 ? part : total + part;
        }
        float y = total * scale;
        if (accumulate)
            acc[i] = acc[i] + y;
        else
            acc[i] = y;
    }
}

/* Overflow check of the sharded gradient scaler ([FSDP] section 3.5): 1 if
 * any reduced gradient element is +-inf or NaN. */
int32_t or_found_inf(int64_t n, const float* acc)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(acc[i]))
            return 1;
    return 0;
}

/* Sum of squares of the reduced gradient, serially in fp64. */
double or_sq_norm(int64_t n, const float* acc)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s = s + (double)acc[i] * (double)acc[i];
    return s;
}

/* ------------------------------------------------------------------------ */
/* Local accumulation without communication.  [DP] "Naive Data             */
/* Parallelism", gradient-accumulation paragraph: the gradients of the     */
/* first micro-batches are accumulated locally (DDP's no_sync) and only the */
/* last micro-batch's backward synchronises; [FSDP] section 3.4: gradient   */
/* accumulation without communication trades memory for fewer exchanges.    */
/* Reading: a rank keeps an fp32 buffer over its whole unit; micro-batches  */
/* are added in order in fp32, starting from the first one's value; on the  */
/* last micro-batch the sum is rounded once to bf16 (the exchange is low     */
/* precision, [FSDP] section 3.5) and that row enters the reduce above with */
/* the same scale 1/(N n).                                                  */
/* ------------------------------------------------------------------------ */

void or_local_accumulate(int64_t n, const uint16_t* grad, int32_t accumulate, float* local)
{
    for (int64_t i = 0; i < n; ++i) {
        float g = or_bf16_to_f32(grad[i]);
        local[i] = accumulate ? local[i] + g : g;
    }
}

/* The last micro-batch: out = bf16(local + g), or bf16(g) when nothing was
 * accumulated (one micro-batch). */
void or_local_finish(int64_t n, const uint16_t* grad, int32_t accumulate, const float* local,
                     uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        float g = or_bf16_to_f32(grad[i]);
        out[i] = or_f32_to_bf16(accumulate ? local[i] + g : g);
    }
}

/* ------------------------------------------------------------------------ */
/* AdamW on the shard.  [DP] ZeRO-1 paragraph: AdamW is elementwise, so a   */
/* rank updates its slice from its averaged gradient and its own moments.   */
/* [DP] ZeRO figure legend and [GUIDE] section 7: the optimizer state is an */
/* fp32 master copy plus two fp32 moments (k = 12 bytes per parameter).     */
/* The pages name AdamW without writing it; this is decoupled weight decay  */
/* (Loshchilov & Hutter) with bias-corrected moments.                       */
/* skip != 0: the step is skipped (overflow found) and nothing changes.     */
/* ------------------------------------------------------------------------ */

/* coef multiplies every gradient element in fp64 before the update (the   */
/* unscale of a loss-scaled gradient and the clipping factor, below).       */
void or_adamw_coef(int64_t n, double lr, double beta1, double beta2, double eps,
                   double weight_decay, int64_t step, double coef, const float* grad,
                   float* master, float* exp_avg, float* exp_avg_sq, int32_t skip)
{
    if (skip)
        return;
    double bias1 = 1.0 - pow(beta1, (double)step);
    double bias2 = 1.0 - pow(beta2, (double)step);
    for (int64_t i = 0; i < n; ++i) {
        double g = (double)grad[i] * coef;
        double theta = master[i];
        double m = exp_avg[i];
        double v = exp_avg_sq[i];
        theta = theta * (1.0 - lr * weight_decay);
        m = beta1 * m + (1.0 - beta1) * g;
        v = beta2 * v + (1.0 - beta2) * g * g;
        double m_hat = m / bias1;
        double v_hat = v / bias2;
        theta = theta - lr * m_hat / (sqrt(v_hat) + eps);
        master[i] = (float)theta;
        exp_avg[i] = (float)m;
        exp_avg_sq[i] = (float)v;
    }
}

void or_adamw(int64_t n, double lr, double beta1, double beta2, double eps,
              double weight_decay, int64_t step, const float* grad,
              float* master, float* exp_avg, float* exp_avg_sq, int32_t skip)
{
    or_adamw_coef(n, lr, beta1, beta2, eps, weight_decay, step, 1.0, grad, master, exp_avg,
                  exp_avg_sq, skip);
}

/* ------------------------------------------------------------------------ */
/* Consumers of the overflow flag and of the gradient norm.  [FSDP] section */
/* 3.5: the sharded gradient scaler handles overflow of loss-scaled low-    */
/* precision gradients over sharded state; the pages give no policy, so the */
/* usual dynamic loss-scaling rule is taken: an overflow skips the step,    */
/* multiplies the scale by the backoff factor and restarts the count of     */
/* clean steps; every growth_interval clean steps in a row multiply it by   */
/* the growth factor.  The scale is an fp32 value.  Global-norm clipping is */
/* not on the pages; the usual rule is taken: with the unscaled norm        */
/* ||g|| = sqrt(sum of squares) / scale, gradients are multiplied by        */
/* min(1, max_norm / (||g|| + 1e-6)); max_norm <= 0 means no clipping.     */
/* ------------------------------------------------------------------------ */

/* The fp64 coefficient AdamW applies to the (still loss-scaled) gradient. */
double or_grad_coef(double sq_norm, float loss_scale, double max_norm)
{
    double inv = 1.0 / (double)loss_scale;
    if (max_norm <= 0.0)
        return inv;
    double norm = sqrt(sq_norm) * inv;
    double clip = max_norm / (norm + 1e-6);
    return clip < 1.0 ? inv * clip : inv;
}

void or_scaler_update(int32_t found_inf, float* scale, int32_t* clean_steps, float growth_factor,
                      float backoff_factor, int32_t growth_interval)
{
    if (found_inf) {
        *scale = *scale * backoff_factor;
        *clean_steps = 0;
        return;
    }
    *clean_steps = *clean_steps + 1;
    if (*clean_steps == growth_interval) {
        *scale = *scale * growth_factor;
        *clean_steps = 0;
    }
}

/* ------------------------------------------------------------------------ */
/* Unshard: the all-gather's data movement.  [DP] ZeRO-1 paragraph: after  */
/* the update every rank gathers the updated slices into the full model;   */
/* [DP] ZeRO-3 paragraph: the unit is gathered again before it is used.    */
/* full[q*S + j] = shards[q][j].                                            */
/* ------------------------------------------------------------------------ */

void or_unshard(int64_t shard, int32_t world, const uint16_t* const* shards,
                uint16_t* full)
{
    for (int32_t q = 0; q < world; ++q)
        for (int64_t j = 0; j < shard; ++j)
            full[(int64_t)q * shard + j] = shards[q][j];
}

/* ------------------------------------------------------------------------ */
/* Model-state bytes per GPU.  [DP] ZeRO figure, one formula per row;      */
/* [GUIDE] sections 6.1 and 7.  Parameters and gradients 2 bytes each,    */
/* optimizer state k bytes per parameter.                                   */
/* stage 0 (replicated): 2P + 2P + kP                                       */
/* stage 1: 2P + 2P + kP/N;  stage 2: 2P + (2P + kP)/N;                    */
/* stage 3: (2P + 2P + kP)/N.  Returns -1 for an unknown stage.             */
/* ------------------------------------------------------------------------ */

double or_state_bytes(double psi, int32_t world, double k, int32_t stage)
{
    double n = (double)world;
    switch (stage) {
    case 0: return 2.0 * psi + 2.0 * psi + k * psi;
    case 1: return 2.0 * psi + 2.0 * psi + k * psi / n;
    case 2: return 2.0 * psi + (2.0 * psi + k * psi) / n;
    case 3: return (2.0 * psi + 2.0 * psi + k * psi) / n;
    default: return -1.0;
    }
}
