// step_ops.h -- device building blocks of the per-step kernels: quad
// streams, the fixed-order reduce, AdamW, the bf16 cast, the unshard copy,
// the grid barrier, and the per-tile bodies that the single-unit kernels
// (step_kernels.hip) and the multi-unit kernels (unit_kernels.hip) share.
//
// Element streams are processed in quads of 4 elements: one 16-byte access
// of an fp32 stream, one 8-byte access of a bf16 stream.  Lane t of a
// workgroup holds quads base + u * 256 + t (u < kU), so every load or store
// instruction of a wave covers one contiguous span (1 KiB of fp32, 512 bytes
// of bf16) and writes every byte of each cache line it touches.  That is
// what makes the stores fast: with each lane owning a 32-byte fp32 chunk
// written in two 16-byte halves, every instruction left its 128-byte lines
// half written, and with the non-temporal hint the halves reached HBM
// separately (measured on MI355X: 2.1 TB/s for pure fp32 stores, against
// 5.7 TB/s in the quad layout).  Every access carries the non-temporal hint
// (each stream is touched once per step).  Workgroups own dispatch-ordered
// tiles of 256 * kU quads.  Lanes past the last quad load the last quad
// again and store nothing, so the loads of every lane are unconditional and
// all in flight together; the at most 3 elements past the last quad are
// handled one by one by the unit's first tile.  Every kernel comes in an
// aligned form (bf16 quad streams 8-byte aligned, copy sources 16-byte
// aligned) and a general form: bf16 quads on any 2-byte boundary (the same
// instructions, served by the hardware's unaligned access) and copy sources
// realigned from aligned loads.  Nothing here is a
// contraction, so there is no MFMA; the kernels are bound by HBM.
//
// Compiled with -ffp-contract=off: every fp32 / fp64 operation below is one
// IEEE round-to-nearest-even operation, in the order written.
#pragma once

#include <type_traits>
#include <utility>

#include "fp_device.h"

namespace fpk {

// Optional per-workgroup phase timestamps for tuning builds (never defined
// in the library build): thread 0 records the 100 MHz real-time counter.
#ifdef FP_PHASE_TRACE
__device__ unsigned long long fp_phase_trace[1 << 16][6];
#define FP_PHASE_MARK(k)                                                               \
    do {                                                                               \
        if (threadIdx.x == 0 && blockIdx.x < (1u << 16))                               \
            fp_phase_trace[blockIdx.x][k] = __builtin_amdgcn_s_memrealtime();          \
    } while (0)
#else
#define FP_PHASE_MARK(k) \
    do {                 \
    } while (0)
#endif

// ---------------------------------------------------------------- streams

// The lane's kU quads in tile `tile` of a stream of nq > 0 quads: quads
// start + off[u], off[u] = u * 256 + t.  ok[u] tells whether quad u exists;
// a missing one is replaced by the last quad, which the caller loads but
// does not store.  Addresses are formed as a workgroup-uniform tile base
// plus a 32-bit lane offset, so each access needs one offset register per
// quad, shared by all streams, instead of a 64-bit address per stream.
template <int kU>
struct Quads {
    int64_t start;
    uint32_t off[kU];
    bool ok[kU];
};

template <int kU>
__device__ __forceinline__ Quads<kU> lane_quads(int64_t tile, int64_t nq) {
    Quads<kU> Q;
    Q.start = tile * (kThreads * kU);
    const int64_t last = nq - 1 - Q.start;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t x = (uint32_t)(u * kThreads) + threadIdx.x;
        Q.ok[u] = (int64_t)x <= last;
        Q.off[u] = Q.ok[u] ? x : (uint32_t)last;
    }
    return Q;
}

// Byte offsets are formed in 32 bits (a tile spans far less than 4 GiB), so
// that the compiler can use the scalar-base + 32-bit-offset address form.
__device__ __forceinline__ const char* at(const void* tile_base, uint32_t byte_off) {
    return static_cast<const char*>(tile_base) + byte_off;
}
__device__ __forceinline__ char* at(void* tile_base, uint32_t byte_off) {
    return static_cast<char*>(tile_base) + byte_off;
}

template <int kU>
__device__ __forceinline__ void ld_f32q(const float* p, const Quads<kU>& Q, int u, float f[4]) {
    const float* tb = p + (Q.start << 2);
    const uint4 v = ld16(at(tb, Q.off[u] * 16u));
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <int kU>
__device__ __forceinline__ void st_f32q(float* p, const Quads<kU>& Q, int u, const float f[4]) {
    float* tb = p + (Q.start << 2);
    st16(at(tb, Q.off[u] * 16u), make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                                        __float_as_uint(f[2]), __float_as_uint(f[3])));
}

// Quad u of a bf16 stream starting at `base`.
template <bool kAligned, int kU>
__device__ __forceinline__ uint2 ld_bf16q(const uint16_t* base, const Quads<kU>& Q, int u) {
    const uint16_t* tb = base + (Q.start << 2);
    if (kAligned) return ld8(at(tb, Q.off[u] * 8u));
    return ld8u(at(tb, Q.off[u] * 8u));
}

template <bool kAligned, int kU>
__device__ __forceinline__ void st_bf16q(uint16_t* base, const Quads<kU>& Q, int u, const uint2 v) {
    uint16_t* tb = base + (Q.start << 2);
    if (kAligned) st8(at(tb, Q.off[u] * 8u), v);
    else st8u(at(tb, Q.off[u] * 8u), v);
}

// 16-byte word `word` of a bf16 stream (the copies move whole words).
template <bool kAligned>
__device__ __forceinline__ uint4 ld_bf16_word(const uint16_t* base, int64_t word) {
    if (kAligned) return ld16(base + (word << 3));
    return ld16u(base + (word << 3));
}

// ---------------------------------------------------------------- reduce
// Ascending-rank fp32 sum of the ranks' bf16 gradients at the lane's kU
// quads, in groups of kG ranks: the loads of a group are all issued before
// its adds, so a group costs one memory round trip (kG = 16 for large
// groups of ranks, at the price of the registers that hold them).  "Infra:
// Data Parallel", ZeRO-1/ZeRO-2 paragraphs (reduce-scatter with averaging);
// "4.1 数据并行详解" section 2 (average of the local gradients).
//
// The gradient quads of ranks [q0, q0 + kG) below world.  From a table in
// device memory (a multi-unit plan's unit record, kTable), a whole group
// reads all its row pointers before its first gradient load, so that the
// group's loads leave back to back; read inside the per-rank condition,
// each pointer's scalar load was waited for before its rank's load was
// issued (measured on MI355X: the bucketed 611M model's fused multi-unit
// launch 436 -> 391 us).  Groups of 16 keep the per-rank form: sixteen
// held pointers raised their multi-unit kernels from 48 to 78 VGPRs (six
// workgroups per SIMD instead of eight) and slowed the two-phase
// multi-unit launch at 16 ranks 658 -> 766 us.  From kernel arguments the per-rank form stays too:
// there the hoisted form raised the one-pass kernel's registers (86 -> 108
// VGPRs, a smaller co-resident grid) and slowed the 64-rank fused launch.
template <bool kAligned, int kG, int kU, bool kTable, class P>
__device__ __forceinline__ void load_group(const P& grads, int q0, int world, const Quads<kU>& Q,
                                           uint2 w[kG][kU]) {
    if (kTable && kG <= 8 && q0 + kG <= world) {
        const uint16_t* p[kG];
#pragma unroll
        for (int k = 0; k < kG; ++k) p[k] = grads[q0 + k];
#pragma unroll
        for (int k = 0; k < kG; ++k) {
#pragma unroll
            for (int u = 0; u < kU; ++u) w[k][u] = ld_bf16q<kAligned>(p[k], Q, u);
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < kG; ++k) {
        if (q0 + k < world) {
#pragma unroll
            for (int u = 0; u < kU; ++u) w[k][u] = ld_bf16q<kAligned>(grads[q0 + k], Q, u);
        }
    }
}

// Whether a stream view's gradient row pointers sit in device memory (a
// pointer to a table) rather than in the kernel arguments (an array).
template <class A>
constexpr bool grads_in_table() {
    return std::is_pointer<std::remove_reference_t<decltype(std::declval<A>().grads)>>::value;
}

template <bool kAligned, int kG, int kU, class A>
__device__ __forceinline__ void sum_ranks(const A& a, const Quads<kU>& Q, float s[kU][4]) {
    const int world = a.world;
    for (int q0 = 0; q0 < world; q0 += kG) {
        uint2 w[kG][kU];
        load_group<kAligned, kG, kU, grads_in_table<A>()>(a.grads, q0, world, Q, w);
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            if (q0 + k < world) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    float f[4];
                    bf16x4_to_f32(w[k][u], f);
                    if (q0 + k == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[u][e] = f[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[u][e] = s[u][e] + f[e];
                    }
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

// y = scale * (sum over ranks), then y = acc + y when accumulating.  With
// kAccFirst the accumulator is loaded before the gradients, so that its
// load is in flight with theirs (at the cost of holding it across the sum);
// without it, after the sum.
template <bool kAligned, bool kAccFirst, int kG, int kU, class A>
__device__ __forceinline__ void reduce_quads(const A& a, const Quads<kU>& Q, bool accumulate,
                                             float y[kU][4]) {
    float p[kU][4];
    if (kAccFirst && accumulate) {
#pragma unroll
        for (int u = 0; u < kU; ++u) ld_f32q(a.acc, Q, u, p[u]);
    }
    sum_ranks<kAligned, kG, kU>(a, Q, y);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[u][e] = y[u][e] * a.scale;
    }
    if (accumulate) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (!kAccFirst) ld_f32q(a.acc, Q, u, p[u]);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[u][e] = p[u][e] + y[u][e];
        }
    }
}

template <class A>
__device__ __forceinline__ float reduce_elem(const A& a, int64_t j, bool accumulate) {
    float y = sum_ranks1(a, j) * a.scale;
    if (accumulate) y = a.acc[j] + y;
    return y;
}

__device__ __forceinline__ void check_quad(const float y[4], bool& bad, double& sq, bool want_sq) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bad |= !finite_f32(y[e]);
        if (want_sq) sq += (double)y[e] * (double)y[e];
    }
}

// ---------------------------------------------------------------- AdamW
// One element of decoupled-weight-decay AdamW with bias correction, in fp64
// from the fp32 state; master, exp_avg and exp_avg_sq are each rounded once
// to fp32.  The bias corrections are folded into two host-side coefficients,
//   theta - lr * (m / b1) / (sqrt(v / b2) + eps)
//     = theta - (lr / b1) * m / (sqrt(v) * (1 / sqrt(b2)) + eps),
// which leaves one fp64 division per element; in fp64 the two forms differ
// by a few units of 2^-53, far below the fp32 rounding that follows.
// "Infra: Data Parallel", ZeRO-1 paragraph (elementwise update of the
// rank's slice) and ZeRO figure legend (fp32 master and moments, k = 12).
__device__ __forceinline__ void adamw_elem(const AdamCoef& c, float g, float& th, float& m,
                                           float& v) {
    const double gd = (double)g;
    double theta = (double)th;
    double md = (double)m;
    double vd = (double)v;
    theta = theta * c.decay;
    md = c.beta1 * md + c.one_m_beta1 * gd;
    vd = c.beta2 * vd + c.one_m_beta2 * gd * gd;
    const double denom = sqrt(vd) * c.inv_sqrt_bias2 + c.eps;
    theta = theta - c.step_size * md / denom;
    th = (float)theta;
    m = (float)md;
    v = (float)vd;
}

// The coefficients for a gradient multiplied by k (the unscale and clip
// factor of the loss scaler): (1 - beta1) k and (1 - beta2) k^2 take the
// place of the moment weights, so the per-element arithmetic is unchanged.
// k is a device value read when the workgroup starts (null: k = 1).
__device__ __forceinline__ AdamCoef coef_for(const AdamCoef& c, const double* k) {
    AdamCoef r = c;
    if (k != nullptr) {
        const double x = *k;
        r.one_m_beta1 = c.one_m_beta1 * x;
        r.one_m_beta2 = c.one_m_beta2 * x * x;
    }
    return r;
}

// The fp32 master and moments of a lane's kU quads.  Callers issue these
// loads before anything they wait on (gradient quads, the overflow flag), so
// that a wave pays one memory round trip, not two.
template <int kU>
struct State {
    float th[kU][4], m[kU][4], v[kU][4];
};

template <int kU, class A>
__device__ __forceinline__ void load_state(const A& a, const Quads<kU>& Q, State<kU>& st) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        ld_f32q(a.master, Q, u, st.th[u]);
        ld_f32q(a.exp_avg, Q, u, st.m[u]);
        ld_f32q(a.exp_avg_sq, Q, u, st.v[u]);
    }
}

template <int kU>
__device__ __forceinline__ void adamw_quads(const AdamCoef& c, const float y[kU][4], State<kU>& st) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) adamw_elem(c, y[u][e], st.th[u][e], st.m[u][e], st.v[u][e]);
    }
}

// Stores of the lane's existing quads: the state (unless skip) and the bf16
// cast of the master to `out` (if not null).
template <bool kAligned, int kU, class A>
__device__ __forceinline__ void store_quads(const A& a, const Quads<kU>& Q, bool skip,
                                            const State<kU>& st, uint16_t* out) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        if (!Q.ok[u]) continue;
        if (!skip) {
            st_f32q(a.master, Q, u, st.th[u]);
            st_f32q(a.exp_avg, Q, u, st.m[u]);
            st_f32q(a.exp_avg_sq, Q, u, st.v[u]);
        }
        if (out != nullptr) st_bf16q<kAligned>(out, Q, u, f32x4_to_bf16(st.th[u]));
    }
}

// One element: the state read through `a`, stored through `o`.
template <class A, class O>
__device__ __forceinline__ void update_elem(const A& a, const O& o, const AdamCoef& c, int64_t j, float y,
                                            bool skip, uint16_t* out) {
    float th = a.master[j];
    if (!skip) {
        float m = a.exp_avg[j], v = a.exp_avg_sq[j];
        adamw_elem(c, y, th, m, v);
        o.master[j] = th;
        o.exp_avg[j] = m;
        o.exp_avg_sq[j] = v;
    }
    if (out != nullptr) out[j] = (uint16_t)bf16x2(th, 0.0f);
}

// The buffers a fused update stores the state to: the step's output buffers
// (the speculative step's separate ones, else its inputs); other views
// update in place.
struct StateOut {
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
};
template <class A>
__device__ __forceinline__ StateOut state_out(const A& a) {
    return {a.master, a.exp_avg, a.exp_avg_sq};
}
__device__ __forceinline__ StateOut state_out(const StepArgs& a) {
    return {a.master_out, a.exp_avg_out, a.exp_avg_sq_out};
}

// ---------------------------------------------------------------- unshard
// Shard q's whole words of `full` are copied with one aligned store each
// (the source realigned when needed); its at most 14 edge elements, which
// share a word with a neighbouring shard, are copied one by one.
// Copy tile `tile` of shard q's whole words: lane t moves words
// tile * 256 * kWords + u * 256 + t, u < kWords.  A full tile (the common
// case, decided per workgroup) loads without bounds checks so that all its
// loads are in flight together.  A misaligned source is read either with
// one unaligned 16-byte load per lane (kRealign = false) or as aligned words
// realigned across lanes (kRealign = true).
template <bool kAligned, int kWords, bool kRealign = true>
__device__ __forceinline__ void copy_tile(const uint16_t* src, uint16_t* full, const ShardSpan& sp,
                                          int64_t tile) {
    constexpr int64_t kTile = (int64_t)kThreads * kWords;
    const int64_t n_words = (sp.b - sp.a) >> 3;
    const uint16_t* from = src + (sp.a - sp.lo);
    uint16_t* to = full + sp.a;
    const int64_t w0 = tile * kTile + threadIdx.x;
    if ((tile + 1) * kTile <= n_words) {
        uint4 v[kWords];
        if (kAligned) {
#pragma unroll
            for (int u = 0; u < kWords; ++u) v[u] = ld16(from + ((w0 + u * kThreads) << 3));
        } else if (!kRealign) {
            // The step's copies of whole shards: measured on MI355X, the 10k-
            // tensor group's 63 misaligned shards 1766 -> 1747 us against the
            // realigned form.
#pragma unroll
            for (int u = 0; u < kWords; ++u) v[u] = ld16u(from + ((w0 + u * kThreads) << 3));
        } else {
            // Realignment takes the word after each lane's own from the next
            // lane (the lanes of a wave hold consecutive words); only the
            // wave's last lane loads that word itself.  Measured faster than
            // one unaligned 16-byte load per lane where many short pieces are
            // copied (the 10k-tensor group's dim-0 layout at 64 ranks: 1.94 /
            // 1.80 ms against 2.00 / 1.89 ms for pack / unpack).
            const Src16 s = src16(from);
            uint4 hi[kWords] = {};
#pragma unroll
            for (int u = 0; u < kWords; ++u) v[u] = ld16(s.abase + w0 + u * kThreads);
            if ((threadIdx.x & 63) == 63) {
#pragma unroll
                for (int u = 0; u < kWords; ++u) hi[u] = ld16(s.abase + w0 + u * kThreads + s.step);
            }
#pragma unroll
            for (int u = 0; u < kWords; ++u) v[u] = realign16(s, v[u], from_next_lane(v[u], hi[u]));
        }
#pragma unroll
        for (int u = 0; u < kWords; ++u) st16(to + ((w0 + u * kThreads) << 3), v[u]);
    } else {
#pragma unroll
        for (int u = 0; u < kWords; ++u) {
            const int64_t w = w0 + u * kThreads;
            if (w < n_words) st16(to + (w << 3), ld_bf16_word<kAligned>(from, w));
        }
    }
}

// The edge elements of span sp of `full` (those that share a 16-byte word
// with a neighbour), from src (the source of element sp.lo), one per lane.
__device__ __forceinline__ void span_edges(const uint16_t* src, uint16_t* full, const ShardSpan& sp,
                                           int t, int stride) {
    const int64_t n_head = sp.a - sp.lo;
    const int64_t n_edge = n_head + (sp.hi - sp.b);
    for (int64_t k = t; k < n_edge; k += stride) {
        const int64_t e = k < n_head ? sp.lo + k : sp.b + (k - n_head);
        full[e] = src != nullptr ? src[e - sp.lo] : (uint16_t)0;
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
// Split-phase barrier over workgroups [0, n) of a grid, all resident, that
// also ORs one bit (the overflow flag) over them.  Only thread 0 of a
// workgroup takes part.  Arrival adds 1 (plus the bit at position 16) to
// its group's counter; the group's last arrival resets that counter and
// adds its group's result to the top counter; the last group decides,
// resets the top counter and writes the next generation, with the decision
// in bits 30-31, into every group's copy of the generation word, which the
// group's members poll.  The bit travels only through read-modify-write
// results on the counters, so relaxed agent-scope atomics suffice: no
// fences, no cache write-back.  Spreading the counters and the polled words
// over 32 cache lines keeps arrival and polling off a single address.
//
// The wait is bounded.  A member that gives up (possible only if the
// members were not resident together) counts a timeout in the workspace and
// cancels the barrier: a compare-and-swap sets the cancel bit in the top
// counter while groups are still missing.  The last group's add returns
// that bit, so it publishes "cancelled"; if instead every group had already
// arrived, the member adopts the last group's decision.  Either way every
// member leaves with the same one of three decisions, and a cancelled
// barrier still completes (every member arrives before it waits), which
// leaves the counters reusable.
//
// Top counter: bits 0-15 groups arrived, 16-21 groups that saw the bit,
// 22 cancel requested, 23 / 24 overflow / cancelled decided by the
// generation that completed last, 28-29 the generation in progress (low two
// bits).  Generation word: bits 0-29 generation, 30 cancelled, 31 overflow.
constexpr unsigned kSpinLimit = 1u << 22;
constexpr unsigned kBarrierClean = 0u, kBarrierOverflow = 1u, kBarrierCancelled = 2u;
constexpr unsigned kGenMask = 0x3FFFFFFFu;
constexpr unsigned kTopCount = 0xFFFFu;
constexpr unsigned kTopCancel = 1u << 22;
constexpr unsigned kTopPrevOverflow = 1u << 23;
constexpr unsigned kTopPrevCancel = 1u << 24;
constexpr unsigned kTopTagShift = 28;

__device__ __forceinline__ unsigned sync_load(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned sync_add(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Compare-and-swap; on failure `expect` receives the current value.
__device__ __forceinline__ bool sync_cas(unsigned* p, unsigned& expect, unsigned v) {
    return __hip_atomic_compare_exchange_strong(p, &expect, v, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}

struct BarrierTicket {
    unsigned group;
    unsigned gen0;  // the generation in progress (bits 0-29)
};

__device__ __forceinline__ BarrierTicket grid_ticket(GridSync* s) {
    BarrierTicket t;
    t.group = blockIdx.x % kSyncGroups;
    t.gen0 = sync_load(&s->gen[t.group * kLineWords]) & kGenMask;
    return t;
}

__device__ __forceinline__ unsigned sync_groups(unsigned n) { return n < (unsigned)kSyncGroups ? n : (unsigned)kSyncGroups; }

__device__ __forceinline__ void grid_arrive(GridSync* s, const BarrierTicket& t, unsigned bit, unsigned n) {
    const unsigned n_groups = sync_groups(n);
    const unsigned members = n / kSyncGroups + (t.group < n % kSyncGroups ? 1u : 0u);
    const unsigned inc = 1u + (bit << 16);
    const unsigned old = sync_add(&s->group[t.group * kLineWords], inc);
    if ((old & 0xFFFFu) != members - 1) return;
    sync_store(&s->group[t.group * kLineWords], 0u);
    const unsigned group_bit = ((old + inc) >> 16) != 0 ? 1u : 0u;
    const unsigned tinc = 1u + (group_bit << 16);
    const unsigned told = sync_add(&s->top[0], tinc);
    if ((told & kTopCount) != n_groups - 1) return;
    const unsigned v = told + tinc;
    const unsigned overflow = ((v >> 16) & 0x3Fu) != 0 ? 1u : 0u;
    const unsigned cancelled = (v & kTopCancel) != 0 ? 1u : 0u;
    const unsigned next = (t.gen0 + 1u) & kGenMask;
    sync_store(&s->top[0], ((next & 3u) << kTopTagShift) | (overflow ? kTopPrevOverflow : 0u) |
                               (cancelled ? kTopPrevCancel : 0u));
    const unsigned word = next | (cancelled << 30) | (overflow << 31);
    for (unsigned k = 0; k < n_groups; ++k) sync_store(&s->gen[k * kLineWords], word);
}

// A member that gave up waiting: cancel the barrier unless every group has
// arrived, and return the decision all members share.  The top counter takes
// at most n_groups + 2 distinct values per generation, and every failed
// compare-and-swap returns a newer one, so the loop ends within its bound.
__device__ __forceinline__ unsigned grid_cancel(GridSync* s, const BarrierTicket& t, unsigned n) {
    const unsigned n_groups = sync_groups(n);
    unsigned v = sync_load(&s->top[0]);
    for (int k = 0; k < 4 * kSyncGroups; ++k) {
        if (((v >> kTopTagShift) & 3u) != (t.gen0 & 3u))  // completed and reset: the decision is kept
            return (v & kTopPrevCancel) ? kBarrierCancelled
                                        : ((v & kTopPrevOverflow) ? kBarrierOverflow : kBarrierClean);
        if (v & kTopCancel) return kBarrierCancelled;
        if ((v & kTopCount) >= n_groups)                   // decided by the last group, not yet reset
            return ((v >> 16) & 0x3Fu) != 0 ? kBarrierOverflow : kBarrierClean;
        if (sync_cas(&s->top[0], v, v | kTopCancel)) return kBarrierCancelled;
    }
    return kBarrierCancelled;
}

// The barrier's decision: kBarrierClean, kBarrierOverflow (some member
// arrived with the bit) or kBarrierCancelled (some member gave up).
__device__ __forceinline__ unsigned grid_wait(GridSync* s, const BarrierTicket& t, unsigned n,
                                              unsigned spin_limit) {
    const unsigned* word = &s->gen[t.group * kLineWords];
    for (unsigned i = 0; i < spin_limit; ++i) {
        const unsigned v = sync_load(word);
        if ((v & kGenMask) != t.gen0) return (v >> 30) & 1u ? kBarrierCancelled : (v >> 31);
        __builtin_amdgcn_s_sleep(2);
    }
    sync_add(&s->timeouts, 1u);
    return grid_cancel(s, t, n);
}

// ---------------------------------------------------------------- norm
// Sum of the per-workgroup partials in a fixed order (one workgroup).
__device__ __forceinline__ void finalize_norm(const double* partials, int n, double* out) {
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += kThreads) s += partials[i];
    const double t = group_sum(s);
    if (threadIdx.x == 0) *out = t;
}


// ---------------------------------------------------------------- tile bodies
// A "stream view" A gives a tile body one unit's pointers: grads (world row
// pointers), acc, master, exp_avg, exp_avg_sq (the unit's fp32 shard), shard
// (S), scale, world, c (AdamCoef); the copy role also uses shards, full,
// rank and copy_tiles.

// Reduce tile `tile` of one micro-batch into acc, with the overflow check
// (flag OR-ed into found_inf) and, with kNorm, the tile's sum of squares
// written to *partial by thread 0.
template <bool kAligned, bool kAccumulate, bool kNorm, int kG, class A>
__device__ __forceinline__ void reduce_tile(const A& a, int64_t tile, int32_t* found_inf,
                                            double* partial) {
    constexpr int kU = kQuadsPerLane;
    const int64_t nq = a.shard >> 2;
    bool bad = false;
    double sq = 0.0;
    if (nq > 0) {
        const Quads<kU> Q = lane_quads<kU>(tile, nq);
        float y[kU][4];
        reduce_quads<kAligned, true, kG, kU>(a, Q, kAccumulate, y);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (!Q.ok[u]) continue;
            st_f32q(a.acc, Q, u, y[u]);
            check_quad(y[u], bad, sq, kNorm);
        }
    }
    const int64_t tail0 = nq << 2;
    if (tile == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        const float y = reduce_elem(a, j, kAccumulate);
        a.acc[j] = y;
        bad |= !finite_f32(y);
        if (kNorm) sq += (double)y * (double)y;
    }
    flag_if_any(bad, found_inf);
    if (kNorm) {
        const double t = group_sum(sq);
        if (threadIdx.x == 0) *partial = t;
    }
}

// AdamW tile `tile` from the reduced gradient in `grad` (the unit's fp32
// shard), gated by *found_inf, with the bf16 cast of the master to `out`.
// The gradient and state loads do not wait for the overflow flag: they are
// issued first and the flag is read beside them (a skipped step, which is
// rare, loads 12 bytes per element it does not need).
template <bool kAligned, class A>
__device__ __forceinline__ void adamw_tile(const A& a, const float* grad, int64_t tile,
                                           const int32_t* found_inf, uint16_t* out) {
    constexpr int kU = kQuadsPerLane;
    const int64_t nq = a.shard >> 2;
    const AdamCoef c = coef_for(a.c, a.g_coef);
    if (nq > 0) {
        const Quads<kU> Q = lane_quads<kU>(tile, nq);
        float g[kU][4];
        State<kU> st;
#pragma unroll
        for (int u = 0; u < kU; ++u) ld_f32q(grad, Q, u, g[u]);
        load_state<kU>(a, Q, st);
        const bool skip = found_inf != nullptr && *found_inf != 0;
        if (!skip) adamw_quads<kU>(c, g, st);
        store_quads<kAligned, kU>(a, Q, skip, st, out);
    }
    const int64_t tail0 = nq << 2;
    if (tile == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        const bool skip = found_inf != nullptr && *found_inf != 0;
        update_elem(a, a, c, j, skip ? 0.0f : grad[j], skip, out);
    }
}

// Copy role of the step kernels: copy workgroup idx takes tile
// idx % copy_tiles of the idx / copy_tiles-th shard other than the own one.
template <bool kAligned, int kWords, class A>
__device__ __forceinline__ void copy_role(const A& a, unsigned idx) {
    const unsigned qi = idx / (unsigned)a.copy_tiles;
    const unsigned tile = idx - qi * (unsigned)a.copy_tiles;
    const int q = (int)qi < a.rank ? (int)qi : (int)qi + 1;
    const uint16_t* src = a.shards[q];
    const ShardSpan sp = shard_span(a.full, a.shard, q);
    copy_tile<kAligned, kWords, false>(src, a.full, sp, tile);
    if (tile == 0) unshard_edges(src, a.full, a.shard, q, threadIdx.x, kThreads);
}

// Reduce tile of the last micro-batch in a step: kFused = false writes the
// reduced gradient to acc for the AdamW kernel that follows once the
// overflow flag of the whole step is known; kFused = true also runs AdamW
// and the cast to `own` in the same pass (no gate), the new state stored to
// state_out(a).  keep_grad: with
// kFused, also leave the reduced gradient in acc.
template <bool kAligned, bool kFused, int kG, class A>
__device__ __forceinline__ void step_reduce_tile(const A& a, int64_t tile, bool accumulate,
                                                 bool keep_grad, uint16_t* own, int32_t* found_inf,
                                                 double* partial) {
    constexpr int kU = kQuadsPerLane;
    const int64_t nq = a.shard >> 2;
    const bool want_sq = partial != nullptr;
    const AdamCoef c = coef_for(a.c, kFused ? a.g_coef : nullptr);
    bool bad = false;
    double sq = 0.0;
    if (nq > 0) {
        const Quads<kU> Q = lane_quads<kU>(tile, nq);
        State<kU> st;
        if (kFused) load_state<kU>(a, Q, st);
        float y[kU][4];
        reduce_quads<kAligned, true, kG, kU>(a, Q, accumulate, y);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (!Q.ok[u]) continue;
            check_quad(y[u], bad, sq, want_sq);
            if (!kFused || keep_grad) st_f32q(a.acc, Q, u, y[u]);
        }
        if (kFused) {
            adamw_quads<kU>(c, y, st);
            store_quads<kAligned, kU>(state_out(a), Q, false, st, own);
        }
    }
    const int64_t tail0 = nq << 2;
    if (tile == 0 && (int64_t)threadIdx.x < a.shard - tail0) {
        const int64_t j = tail0 + threadIdx.x;
        const float y = reduce_elem(a, j, accumulate);
        bad |= !finite_f32(y);
        if (want_sq) sq += (double)y * (double)y;
        if (!kFused || keep_grad) a.acc[j] = y;
        if (kFused) update_elem(a, state_out(a), c, j, y, false, own);
    }
    flag_if_any(bad, found_inf);
    if (want_sq) {
        const double t = group_sum(sq);
        if (threadIdx.x == 0) *partial = t;
    }
}

}  // namespace fpk
