// step_kernels.hip -- gfx950 kernels of the per-step path: reduce, AdamW with
// the bf16 cast, unshard, and the shard step (one-pass or two-phase).
//
// Each lane moves 8-element chunks: one 16-byte word per bf16 stream and
// two per fp32 stream, so every HBM access is a 128-bit (dwordx4) load or
// store and a wave touches 1 KiB (bf16) or 2 KiB (fp32) of contiguous
// memory per access.  Workgroups own dispatch-ordered tiles of
// kTileChunks chunks.  Elements past the last whole chunk are handled one
// by one by workgroup 0.  Nothing here is a contraction, so there is no
// MFMA; the kernels are bound by HBM.
//
// Compiled with -ffp-contract=off: every fp32 / fp64 operation below is one
// IEEE round-to-nearest-even operation, in the order written.

#include <atomic>

#include "fp_device.h"

namespace fpk {

// ---------------------------------------------------------------- reduce
// Ascending-rank fp32 sum of the ranks' bf16 gradients at chunk j0.  The
// loads of up to 8 ranks are issued before any add, so each lane has up to
// 128 bytes in flight.  "Infra: Data Parallel", ZeRO-1/ZeRO-2 paragraphs
// (reduce-scatter with averaging); "4.1 数据并行详解" section 2 (average of
// the local gradients).
template <class A>
__device__ __forceinline__ void sum_ranks8(const A& a, int64_t j0, float s[8]) {
    const int world = a.world;
    for (int q0 = 0; q0 < world; q0 += 8) {
        uint4 w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (q0 + k < world) w[k] = load16_any(a.grads[q0 + k] + j0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (q0 + k < world) {
                float f[8];
                bf16x8_to_f32(w[k], f);
                if (q0 + k == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] = f[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] = s[e] + f[e];
                }
            }
        }
    }
}

template <class A>
__device__ __forceinline__ float sum_ranks1(const A& a, int64_t j) {
    float s = bf16_lo(a.grads[0][j]);
    for (int q = 1; q < a.world; ++q) s = s + bf16_lo(a.grads[q][j]);
    return s;
}

__device__ __forceinline__ void load_f32x8(const float* p, float f[8]) {
    const float4 u = reinterpret_cast<const float4*>(p)[0];
    const float4 v = reinterpret_cast<const float4*>(p)[1];
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
    f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
}

__device__ __forceinline__ void store_f32x8(float* p, const float f[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// y = scale * (sum over ranks), then y = acc + y when accumulating.
template <class A>
__device__ __forceinline__ void reduce_chunk(const A& a, int64_t j0, bool accumulate, float y[8]) {
    sum_ranks8(a, j0, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * a.scale;
    if (accumulate) {
        float p[8];
        load_f32x8(a.acc + j0, p);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = p[e] + y[e];
    }
}

template <class A>
__device__ __forceinline__ float reduce_elem(const A& a, int64_t j, bool accumulate) {
    float y = sum_ranks1(a, j) * a.scale;
    if (accumulate) y = a.acc[j] + y;
    return y;
}

__device__ __forceinline__ void check_chunk(const float y[8], bool& bad, double& sq, bool want_sq) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bad |= !finite_f32(y[e]);
        if (want_sq) sq += (double)y[e] * (double)y[e];
    }
}

// ---------------------------------------------------------------- AdamW
// One element of decoupled-weight-decay AdamW with bias correction,
// evaluated in fp64 in the order of its definition; master, exp_avg and
// exp_avg_sq are each rounded once to fp32.  "Infra: Data Parallel", ZeRO-1
// paragraph (elementwise update of the rank's slice) and ZeRO figure legend
// (fp32 master and moments, k = 12).
__device__ __forceinline__ void adamw_elem(const AdamCoef& c, float g, float& th, float& m,
                                           float& v) {
    const double gd = (double)g;
    double theta = (double)th;
    double md = (double)m;
    double vd = (double)v;
    theta = theta * c.decay;
    md = c.beta1 * md + c.one_m_beta1 * gd;
    vd = c.beta2 * vd + c.one_m_beta2 * gd * gd;
    const double m_hat = md / c.bias1;
    const double v_hat = vd / c.bias2;
    theta = theta - c.lr * m_hat / (sqrt(v_hat) + c.eps);
    th = (float)theta;
    m = (float)md;
    v = (float)vd;
}

// AdamW on chunk j0 with gradient y, then the bf16 cast to out + j0.
template <class A>
__device__ __forceinline__ void update_chunk(const A& a, int64_t j0, const float y[8], bool skip,
                                             uint16_t* out) {
    float th[8];
    load_f32x8(a.master + j0, th);
    if (!skip) {
        float m[8], v[8];
        load_f32x8(a.exp_avg + j0, m);
        load_f32x8(a.exp_avg_sq + j0, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) adamw_elem(a.c, y[e], th[e], m[e], v[e]);
        store_f32x8(a.master + j0, th);
        store_f32x8(a.exp_avg + j0, m);
        store_f32x8(a.exp_avg_sq + j0, v);
    }
    if (out != nullptr) store16_any(out + j0, f32x8_to_bf16(th));
}

template <class A>
__device__ __forceinline__ void update_elem(const A& a, int64_t j, float y, bool skip, uint16_t* out) {
    float th = a.master[j];
    if (!skip) {
        float m = a.exp_avg[j], v = a.exp_avg_sq[j];
        adamw_elem(a.c, y, th, m, v);
        a.master[j] = th;
        a.exp_avg[j] = m;
        a.exp_avg_sq[j] = v;
    }
    if (out != nullptr) out[j] = (uint16_t)bf16x2(th, 0.0f);
}

// ---------------------------------------------------------------- unshard
// Shard q occupies full[qS, (q+1)S).  Its interior 16-byte words of `full`
// are copied with one aligned store each (the source word is realigned when
// needed); the at most 14 edge elements that share a word with a
// neighbouring shard are copied one by one.
struct ShardSpan {
    int64_t lo, a, b, hi;  // [lo, a) head, [a, b) whole words, [b, hi) tail
};

__device__ __forceinline__ ShardSpan shard_span(const uint16_t* full, int64_t S, int q) {
    // element index e is 16-byte aligned in `full` when e % 8 == phase
    const int64_t phase = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(full) & 15u)) & 15u) >> 1);
    ShardSpan s;
    s.lo = (int64_t)q * S;
    s.hi = s.lo + S;
    const int64_t up = s.lo + (((phase - s.lo) % 8) + 8) % 8;     // first aligned >= lo
    s.a = up < s.hi ? up : s.hi;
    const int64_t down = s.hi - (((s.hi - phase) % 8) + 8) % 8;   // last aligned <= hi
    s.b = down > s.a ? down : s.a;
    return s;
}

// Words w = w0 + u * kThreads (u < kUnroll) of shard q; loads first, then stores.
__device__ __forceinline__ void copy_words(const uint16_t* src, uint16_t* full, const ShardSpan& sp,
                                           int64_t w0) {
    const int64_t n_words = (sp.b - sp.a) >> 3;
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t w = w0 + (int64_t)u * kThreads;
        if (w < n_words) v[u] = load16_any(src + (sp.a + (w << 3) - sp.lo));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t w = w0 + (int64_t)u * kThreads;
        if (w < n_words) *reinterpret_cast<uint4*>(full + sp.a + (w << 3)) = v[u];
    }
}

__device__ __forceinline__ void unshard_edges(const uint16_t* src, uint16_t* full, int64_t S, int q,
                                              int t, int stride) {
    const ShardSpan sp = shard_span(full, S, q);
    const int64_t n_head = sp.a - sp.lo;
    const int64_t n_edge = n_head + (sp.hi - sp.b);
    for (int64_t k = t; k < n_edge; k += stride) {
        const int64_t e = k < n_head ? sp.lo + k : sp.b + (k - n_head);
        full[e] = src[e - sp.lo];
    }
}

// ---------------------------------------------------------------- grid barrier
// Split-phase barrier over a grid whose workgroups are all resident, that
// also ORs one bit (the overflow flag) over the grid.  Only thread 0 of a
// workgroup takes part.  Arrival adds 1 (plus the bit at position 16) to
// its group's counter; the group's last arrival resets that counter and
// adds its group's result to the top counter; the last group resets the top
// and writes the next generation, with the grid's bit in bit 31, into every
// group's copy of the generation word, which the group's members poll.  The
// bit travels only through read-modify-write results on the counters, so
// relaxed agent-scope atomics suffice: no fences, no cache write-back.
// Spreading the counters and the polled words over 32 cache lines keeps
// arrival and polling off a single address.  The wait is bounded: should it
// ever give up (possible only if the grid were not resident) it counts a
// timeout in the workspace instead of hanging.
constexpr unsigned kSpinLimit = 1u << 22;

__device__ __forceinline__ unsigned sync_load(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned sync_add(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct BarrierTicket {
    unsigned group;
    unsigned gen0;
};

__device__ __forceinline__ BarrierTicket grid_ticket(GridSync* s) {
    BarrierTicket t;
    t.group = blockIdx.x % kSyncGroups;
    t.gen0 = sync_load(&s->gen[t.group * kLineWords]);
    return t;
}

__device__ __forceinline__ void grid_arrive(GridSync* s, const BarrierTicket& t, unsigned bit) {
    const unsigned n = gridDim.x;
    const unsigned n_groups = n < (unsigned)kSyncGroups ? n : (unsigned)kSyncGroups;
    const unsigned members = n / kSyncGroups + (t.group < n % kSyncGroups ? 1u : 0u);
    const unsigned inc = 1u + (bit << 16);
    const unsigned old = sync_add(&s->group[t.group * kLineWords], inc);
    if ((old & 0xFFFFu) != members - 1) return;
    sync_store(&s->group[t.group * kLineWords], 0u);
    const unsigned group_bit = ((old + inc) >> 16) != 0 ? 1u : 0u;
    const unsigned tinc = 1u + (group_bit << 16);
    const unsigned told = sync_add(&s->top[0], tinc);
    if ((told & 0xFFFFu) != n_groups - 1) return;
    sync_store(&s->top[0], 0u);
    const unsigned grid_bit = ((told + tinc) >> 16) != 0 ? 1u : 0u;
    const unsigned next = ((t.gen0 + 1u) & 0x7FFFFFFFu) | (grid_bit << 31);
    for (unsigned k = 0; k < n_groups; ++k) sync_store(&s->gen[k * kLineWords], next);
}

// Returns the grid's OR of the arrival bits.
__device__ __forceinline__ unsigned grid_wait(GridSync* s, const BarrierTicket& t) {
    const unsigned* word = &s->gen[t.group * kLineWords];
    for (unsigned i = 0; i < kSpinLimit; ++i) {
        const unsigned v = sync_load(word);
        if ((v & 0x7FFFFFFFu) != (t.gen0 & 0x7FFFFFFFu)) return v >> 31;
        __builtin_amdgcn_s_sleep(2);
    }
    sync_add(&s->timeouts, 1u);
    return 0u;
}

// ---------------------------------------------------------------- norm
// Sum of the per-workgroup partials in a fixed order (one workgroup).
__device__ __forceinline__ void finalize_norm(const double* partials, int n, double* out) {
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += kThreads) s += partials[i];
    const double t = group_sum(s);
    if (threadIdx.x == 0) *out = t;
}

__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(const double* partials, int n,
                                                                 double* out) {
    finalize_norm(partials, n, out);
}

// ---------------------------------------------------------------- kernels

__device__ __forceinline__ int64_t lane_chunk(int64_t tile, int u) {
    return tile * kTileChunks + (int64_t)u * kThreads + threadIdx.x;
}

template <bool kAccumulate, bool kNorm>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const ReduceArgs a) {
    const int64_t n_chunks = a.shard >> 3;
    bool bad = false;
    double sq = 0.0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = lane_chunk(blockIdx.x, u);
        if (c < n_chunks) {
            float y[8];
            reduce_chunk(a, c << 3, kAccumulate, y);
            store_f32x8(a.acc + (c << 3), y);
            check_chunk(y, bad, sq, kNorm);
        }
    }
    const int64_t tail0 = n_chunks << 3;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        const float y = reduce_elem(a, j, kAccumulate);
        a.acc[j] = y;
        bad |= !finite_f32(y);
        if (kNorm) sq += (double)y * (double)y;
    }
    flag_if_any(bad, a.found_inf);
    if (kNorm) {
        const double t = group_sum(sq);
        if (threadIdx.x == 0) a.partials[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(kThreads) void adamw_kernel(const AdamArgs a) {
    if (a.sq_norm != nullptr && blockIdx.x == 0) finalize_norm(a.partials, a.n_partials, a.sq_norm);
    const bool skip = a.found_inf != nullptr && *a.found_inf != 0;
    const int64_t n_chunks = a.shard >> 3;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = lane_chunk(blockIdx.x, u);
        if (c < n_chunks) {
            float g[8];
            if (!skip) load_f32x8(a.grad + (c << 3), g);
            update_chunk(a, c << 3, g, skip, a.param_bf16);
        }
    }
    const int64_t tail0 = n_chunks << 3;
    if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        update_elem(a, j, skip ? 0.0f : a.grad[j], skip, a.param_bf16);
    }
}

__global__ __launch_bounds__(kThreads) void unshard_kernel(const UnshardArgs a) {
    const int q = blockIdx.y;
    const uint16_t* src = a.shards[q];
    if (src == nullptr) return;
    const ShardSpan sp = shard_span(a.full, a.shard, q);
    copy_words(src, a.full, sp, (int64_t)blockIdx.x * kTileChunks + threadIdx.x);
    if (blockIdx.x == 0) unshard_edges(src, a.full, a.shard, q, threadIdx.x, kThreads);
}

// First phase of the two-phase step (kFused = false: reduce into acc; the
// AdamW kernel follows once the overflow flag of the whole shard is known)
// or the whole no-skip step (kFused = true: reduce, AdamW and cast in one
// pass).  Workgroups [0, reduce_groups) take reduce tiles; the others take
// (shard, tile) pairs of the copy of the other ranks' shards into `full`.
template <bool kFused>
__global__ __launch_bounds__(kThreads) void step_phase1_kernel(const StepArgs a) {
    if ((int)blockIdx.x < a.reduce_groups) {
        const int64_t n_chunks = a.shard >> 3;
        uint16_t* own = a.full + (int64_t)a.rank * a.shard;
        const bool want_sq = a.partials != nullptr;
        const bool acc_in = a.accumulate != 0;
        bool bad = false;
        double sq = 0.0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t c = lane_chunk(blockIdx.x, u);
            if (c < n_chunks) {
                float y[8];
                reduce_chunk(a, c << 3, acc_in, y);
                check_chunk(y, bad, sq, want_sq);
                if (!kFused || a.keep_grad) store_f32x8(a.acc + (c << 3), y);
                if (kFused) update_chunk(a, c << 3, y, false, own);
            }
        }
        const int64_t tail0 = n_chunks << 3;
        if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
            const int64_t j = tail0 + threadIdx.x;
            const float y = reduce_elem(a, j, acc_in);
            bad |= !finite_f32(y);
            if (want_sq) sq += (double)y * (double)y;
            if (!kFused || a.keep_grad) a.acc[j] = y;
            if (kFused) update_elem(a, j, y, false, own);
        }
        flag_if_any(bad, a.found_inf);
        if (want_sq) {
            const double t = group_sum(sq);
            if (threadIdx.x == 0) a.partials[blockIdx.x] = t;
        }
    } else {
        const unsigned idx = blockIdx.x - (unsigned)a.reduce_groups;
        const unsigned qi = idx / (unsigned)a.copy_tiles;
        const unsigned tile = idx - qi * (unsigned)a.copy_tiles;
        const int q = (int)qi < a.rank ? (int)qi : (int)qi + 1;
        const uint16_t* src = a.shards[q];
        const ShardSpan sp = shard_span(a.full, a.shard, q);
        copy_words(src, a.full, sp, (int64_t)tile * kTileChunks + threadIdx.x);
        if (tile == 0) unshard_edges(src, a.full, a.shard, q, threadIdx.x, kThreads);
    }
}

// Copy of every other rank's shard, words lane_base + u*256 (+ span), with
// the loads of kQ shards in flight before their stores.
template <int kC>
__device__ __forceinline__ void copy_other_shards(const StepArgs& a, int64_t lane_base, int64_t span) {
    constexpr int kQ = 8 / kC;
    for (int q0 = 0; q0 < a.world; q0 += kQ) {
        ShardSpan sp[kQ];
        int64_t n_words[kQ];
        bool use[kQ];
#pragma unroll
        for (int k = 0; k < kQ; ++k) {
            const int q = q0 + k;
            use[k] = q < a.world && q != a.rank;
            if (use[k]) {
                sp[k] = shard_span(a.full, a.shard, q);
                n_words[k] = (sp[k].b - sp[k].a) >> 3;
            } else {
                n_words[k] = 0;
            }
        }
        for (int64_t w0 = lane_base;; w0 += span) {
            bool more = false;
            uint4 v[kQ][kC];
#pragma unroll
            for (int k = 0; k < kQ; ++k)
#pragma unroll
                for (int u = 0; u < kC; ++u) {
                    const int64_t w = w0 + (int64_t)u * kThreads;
                    if (w < n_words[k]) {
                        v[k][u] = load16_any(a.shards[q0 + k] + (sp[k].a + (w << 3) - sp[k].lo));
                        more = true;
                    }
                }
#pragma unroll
            for (int k = 0; k < kQ; ++k)
#pragma unroll
                for (int u = 0; u < kC; ++u) {
                    const int64_t w = w0 + (int64_t)u * kThreads;
                    if (w < n_words[k]) *reinterpret_cast<uint4*>(a.full + sp[k].a + (w << 3)) = v[k][u];
                }
            if (!more) break;
        }
    }
}

// One-pass exact-skip step over a resident grid.  Each lane loads, for its
// kC chunks, the ranks' gradient words and the fp32 master / moments (none
// of which depends on the overflow flag), reduces, and computes the AdamW
// update into registers.  The workgroup ORs its overflow bit (and the flag
// left by earlier micro-batches) into the grid barrier and arrives; it
// copies its share of the other ranks' shards while the barrier completes;
// the barrier returns the grid's flag, after which the lane only stores:
// the new state and its bf16 cast, or on overflow just the cast of the old
// master.  The reduced gradient never leaves the registers, so the step
// moves exactly the algorithmic bytes.
template <int kC>
__global__ __launch_bounds__(kThreads) void step_coop_kernel(const StepArgs a) {
    __shared__ unsigned s_skip;
    const int64_t n_chunks = a.shard >> 3;
    const bool want_sq = a.partials != nullptr;
    const bool acc_in = a.accumulate != 0;
    uint16_t* own = a.full + (int64_t)a.rank * a.shard;
    const int64_t base = (int64_t)blockIdx.x * kThreads * kC + threadIdx.x;
    BarrierTicket ticket = {0u, 0u};
    unsigned prior = 0u;
    if (threadIdx.x == 0) {
        ticket = grid_ticket(a.sync);
        prior = *a.found_inf != 0 ? 1u : 0u;   // written by earlier kernels
    }

    // reduce and speculative update, all in registers
    float th[kC][8], m[kC][8], v[kC][8];
    uint4 old_bf16[kC];
    bool bad = false;
    double sq = 0.0;
#pragma unroll
    for (int u = 0; u < kC; ++u) {
        const int64_t c = base + (int64_t)u * kThreads;
        if (c < n_chunks) {
            const int64_t j0 = c << 3;
            load_f32x8(a.master + j0, th[u]);
            load_f32x8(a.exp_avg + j0, m[u]);
            load_f32x8(a.exp_avg_sq + j0, v[u]);
            float y[8];
            reduce_chunk(a, j0, acc_in, y);
            check_chunk(y, bad, sq, want_sq);
            if (a.keep_grad) store_f32x8(a.acc + j0, y);
            old_bf16[u] = f32x8_to_bf16(th[u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) adamw_elem(a.c, y[e], th[u][e], m[u][e], v[u][e]);
        }
    }
    const int64_t tail0 = n_chunks << 3;
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
        adamw_elem(a.c, yt, tt, tm, tv);
    }
    const int group_bad = __syncthreads_or(bad);
    if (want_sq) {
        const double t = group_sum(sq);
        if (threadIdx.x == 0) a.partials[blockIdx.x] = t;   // summed by a follow-up kernel
    }
    if (threadIdx.x == 0) grid_arrive(a.sync, ticket, (group_bad || prior) ? 1u : 0u);

    // the other ranks' shards, independent of the flag
    copy_other_shards<kC>(a, base, (int64_t)gridDim.x * kThreads * kC);
    if (blockIdx.x == 0)
        for (int q = 0; q < a.world; ++q)
            if (q != a.rank) unshard_edges(a.shards[q], a.full, a.shard, q, threadIdx.x, kThreads);

    if (threadIdx.x == 0) s_skip = grid_wait(a.sync, ticket);
    __syncthreads();
    const bool skip = s_skip != 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.found_inf = skip ? 1 : 0;

    // commit: stores only
#pragma unroll
    for (int u = 0; u < kC; ++u) {
        const int64_t c = base + (int64_t)u * kThreads;
        if (c < n_chunks) {
            const int64_t j0 = c << 3;
            if (skip) {
                store16_any(own + j0, old_bf16[u]);
            } else {
                store_f32x8(a.master + j0, th[u]);
                store_f32x8(a.exp_avg + j0, m[u]);
                store_f32x8(a.exp_avg_sq + j0, v[u]);
                store16_any(own + j0, f32x8_to_bf16(th[u]));
            }
        }
    }
    if (has_tail) {
        const int64_t j = tail0 + threadIdx.x;
        if (skip) {
            own[j] = (uint16_t)bf16x2(told, 0.0f);
        } else {
            a.master[j] = tt;
            a.exp_avg[j] = tm;
            a.exp_avg_sq[j] = tv;
            own[j] = (uint16_t)bf16x2(tt, 0.0f);
        }
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_reduce(const ReduceArgs& a, int64_t grid, hipStream_t s) {
    const bool norm = a.partials != nullptr;
    if (a.accumulate) {
        if (norm) reduce_kernel<true, true><<<(unsigned)grid, kThreads, 0, s>>>(a);
        else reduce_kernel<true, false><<<(unsigned)grid, kThreads, 0, s>>>(a);
    } else {
        if (norm) reduce_kernel<false, true><<<(unsigned)grid, kThreads, 0, s>>>(a);
        else reduce_kernel<false, false><<<(unsigned)grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_norm_finalize(const double* partials, int n, double* out, hipStream_t s) {
    norm_finalize_kernel<<<1, kThreads, 0, s>>>(partials, n, out);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamArgs& a, int64_t grid, hipStream_t s) {
    adamw_kernel<<<(unsigned)grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_unshard(const UnshardArgs& a, int64_t grid_x, hipStream_t s) {
    unshard_kernel<<<dim3((unsigned)grid_x, a.world), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_step_phase1(const StepArgs& a, int64_t grid, bool fused_update, hipStream_t s) {
    if (fused_update) step_phase1_kernel<true><<<(unsigned)grid, kThreads, 0, s>>>(a);
    else step_phase1_kernel<false><<<(unsigned)grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

namespace {
// Co-resident workgroups per CU of each one-pass instantiation and the CU
// count, per device: fixed properties of the device and the code object,
// computed on first use and kept for the life of the process.
constexpr int kMaxDevices = 64;
struct CoopLimits {
    std::atomic<int> state{0};  // 0 unknown, 1 computing, 2 ready
    int cus = 0;
    int per_cu[2] = {0, 0};
};
CoopLimits g_limits[kMaxDevices];

const void* coop_fn(int i) {
    return i == 0 ? reinterpret_cast<const void*>(&step_coop_kernel<1>)
                  : reinterpret_cast<const void*>(&step_coop_kernel<kMaxCoopChunks>);
}

hipError_t coop_limits(int dev, const CoopLimits** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    CoopLimits& L = g_limits[dev];
    int expect = 0;
    if (L.state.load(std::memory_order_acquire) != 2) {
        if (L.state.compare_exchange_strong(expect, 1)) {
            hipError_t e = hipDeviceGetAttribute(&L.cus, hipDeviceAttributeMultiprocessorCount, dev);
            for (int i = 0; i < 2 && e == hipSuccess; ++i)
                e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&L.per_cu[i], coop_fn(i), kThreads, 0);
            if (e != hipSuccess) {
                L.state.store(0, std::memory_order_release);
                return e;
            }
            L.state.store(2, std::memory_order_release);
        } else {
            while (L.state.load(std::memory_order_acquire) != 2) {
                if (L.state.load(std::memory_order_acquire) == 0) return coop_limits(dev, out);
            }
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
    const int64_t n_chunks = shard >> 3;
    const int chunks[2] = {1, kMaxCoopChunks};
    for (int i = 0; i < 2; ++i) {
        const int64_t g = n_chunks > 0 ? ceil_div64(n_chunks, (int64_t)kThreads * chunks[i]) : 1;
        if (g <= (int64_t)L->per_cu[i] * L->cus) {
            *variant = i;
            *grid = (int)g;
            return hipSuccess;
        }
    }
    return hipSuccess;
}

hipError_t launch_step_coop(const StepArgs& a, int variant, int grid, hipStream_t s) {
    // A plain launch: the grid fits the device's resident capacity, so on a
    // GPU not running other work every workgroup is resident at once (a
    // cooperative launch would guarantee it at ~17 us extra per launch).
    if (variant == 0) step_coop_kernel<1><<<grid, kThreads, 0, s>>>(a);
    else step_coop_kernel<kMaxCoopChunks><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
