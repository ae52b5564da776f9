// abi.hip -- the extern "C" entry points of libflatparam.so: argument
// validation, FlatParameter plans, launch geometry and error reporting.
// Every check runs before anything is enqueued, so a rejected call leaves
// the device untouched.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "fp_extra.h"

using namespace fpk;

namespace {

thread_local char g_error[512] = "";

fp_status fail(fp_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return st;
}

fp_status device_fail(hipError_t e, const char* what) {
    return fail(FP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool is_aligned8(const void* p) { return aligned(p, 8); }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A dispatch packet carries the grid size as a 32-bit count of work-items,
// so one launch of 256-lane workgroups takes at most this many.
constexpr int64_t kMaxGroups = 0xFFFFFFFFLL / kThreads;

fp_status check_groups(int64_t groups, const char* what) {
    if (groups > kMaxGroups)
        return fail(FP_ERR_RANGE, "%s needs %lld workgroups, more than one launch holds (%lld)", what,
                    (long long)groups, (long long)kMaxGroups);
    return FP_OK;
}

// Workgroups of a tiled stream over S elements in 4-element quads.
int64_t stream_grid(int64_t shard) {
    const int64_t t = tiles_of(shard >> 2);
    return t > 0 ? t : 1;
}

double* partials_of(void* workspace) {
    return reinterpret_cast<double*>(static_cast<char*>(workspace) + kWorkspaceHeader);
}

fp_status check_hparams(const fp_adamw_hparams* hp, AdamCoef* c) {
    if (hp == nullptr) return fail(FP_ERR_INVALID, "hparams is NULL");
    if (hp->step < 1) return fail(FP_ERR_RANGE, "step must be >= 1 (got %lld)", (long long)hp->step);
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
        return fail(FP_ERR_RANGE, "betas must lie in [0, 1)");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) ||
        hp->eps < 0.0)
        return fail(FP_ERR_RANGE, "lr, eps and weight_decay must be finite, eps >= 0");
    c->decay = 1.0 - hp->lr * hp->weight_decay;
    c->beta1 = hp->beta1;
    c->one_m_beta1 = 1.0 - hp->beta1;
    c->beta2 = hp->beta2;
    c->one_m_beta2 = 1.0 - hp->beta2;
    const double bias1 = 1.0 - std::pow(hp->beta1, (double)hp->step);
    const double bias2 = 1.0 - std::pow(hp->beta2, (double)hp->step);
    c->step_size = hp->lr / bias1;
    c->inv_sqrt_bias2 = 1.0 / std::sqrt(bias2);
    c->eps = hp->eps;
    return FP_OK;
}

fp_status check_ptr_table(const uint16_t* const* t, int32_t world, int64_t shard, bool allow_null,
                          const char* name) {
    if (t == nullptr) return fail(FP_ERR_INVALID, "%s table is NULL", name);
    for (int32_t q = 0; q < world; ++q) {
        if (t[q] == nullptr) {
            if (allow_null || shard == 0) continue;
            return fail(FP_ERR_INVALID, "%s[%d] is NULL", name, q);
        }
        if (!aligned(t[q], 2)) return fail(FP_ERR_ALIGN, "%s[%d] is not 2-byte aligned", name, q);
    }
    return FP_OK;
}

fp_status check_f32(const void* p, int64_t shard, const char* name) {
    if (p == nullptr && shard > 0) return fail(FP_ERR_INVALID, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(FP_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return FP_OK;
}

fp_status check_world(int32_t world) {
    if (world < 1 || world > FP_MAX_WORLD)
        return fail(FP_ERR_RANGE, "world %d outside [1, %d]", world, FP_MAX_WORLD);
    return FP_OK;
}

}  // namespace

// ---------------------------------------------------------------------- segment lists
// The bit-copy operations (FlatParameter pack, the dim-0 layout, resharding)
// are lists of copy / zero-fill entries run by one launch of the segment
// kernel.  A plan keeps, per (operation, element size, rank) and device, the
// entry list and its per-workgroup index on the device, and a per-call table
// of the buffers' device pointers that entries name by index.

namespace {
// Device tables of one segment list on one device, and the staging of its
// per-call pointer table.
struct SegTable {
    int op = -1, es = 0, rank = 0;   // what the list is for
    int device = -1;
    int64_t groups = 0;
    int32_t n_ptrs = 0;
    SegDesc* segs = nullptr;
    int32_t* seg_of = nullptr;
    void** tab = nullptr;
    void** tab_staging = nullptr;
    hipEvent_t uploaded = nullptr;
    bool have_last = false;          // tab holds (or will hold) last_ptrs
    std::vector<void*> last_ptrs;
};

void free_seg_table(SegTable& t) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (t.device >= 0) (void)hipSetDevice(t.device);
    if (t.uploaded) (void)hipEventSynchronize(t.uploaded), (void)hipEventDestroy(t.uploaded);
    if (t.segs) (void)hipFree(t.segs);
    if (t.seg_of) (void)hipFree(t.seg_of);
    if (t.tab) (void)hipFree(t.tab);
    if (t.tab_staging) (void)hipHostFree(t.tab_staging);
    if (cur >= 0) (void)hipSetDevice(cur);
    t = SegTable();
}

constexpr int kOpPackRank = 0, kOpPackAll = 1, kOpUnpack = 2, kOpReshardRank = 3, kOpReshardAll = 4,
              kOpFlatPack = 5;

// The segment tables of one plan, keyed by (operation, element size, rank),
// and the pointer sets its calls last validated.
struct SegCache {
    std::mutex mu;
    std::vector<SegTable> tables;
    struct Validated {
        int op, es, rank;
        std::vector<void*> ptrs;
    };
    std::vector<Validated> validated;
    ~SegCache() {
        for (auto& t : tables) free_seg_table(t);
    }
};

// The device tables of (op, es, rank) on the current device, built on first
// use from the segment list that `build` returns.
template <class Build>
fp_status seg_table(SegCache& c, int op, int es, int rank, int32_t n_ptrs, Build build, SegTable** out) {
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return device_fail(e, "hipGetDevice");
    for (auto& t : c.tables)
        if (t.device == device && t.op == op && t.es == es && t.rank == rank) {
            *out = &t;
            return FP_OK;
        }
    std::vector<SegDesc> segs = build();
    std::vector<int32_t> seg_of;
    int64_t g = 0;
    for (size_t s = 0; s < segs.size(); ++s) {
        // copy entries under 2 MiB take two 16-byte words per lane: half the
        // workgroups where many short pieces make per-workgroup costs count
        // (measured: the 10k-tensor group's dim-0 layout at 64 ranks 12 %
        // faster); long entries keep one, the faster form for long copies
        segs[s].words = (segs[s].kind == kSegCopy && segs[s].len < ((int64_t)1 << 20)) ? 2 : 1;
        segs[s].tile0 = g;
        const int64_t n = segment_tiles(segs[s]);
        if (g + n > kMaxGroups) return check_groups(g + n, "the copy layout");
        for (int64_t k = 0; k < n; ++k) seg_of.push_back((int32_t)s);
        g += n;
    }
    SegTable t;
    t.op = op;
    t.es = es;
    t.rank = rank;
    t.device = device;
    t.groups = g;
    t.n_ptrs = n_ptrs;
    const size_t segs_b = (segs.empty() ? 1 : segs.size()) * sizeof(SegDesc);
    const size_t of_b = (seg_of.empty() ? 1 : seg_of.size()) * sizeof(int32_t);
    const size_t tab_b = (size_t)t.n_ptrs * sizeof(void*);
    if ((e = hipMalloc((void**)&t.segs, segs_b)) != hipSuccess ||
        (e = hipMalloc((void**)&t.seg_of, of_b)) != hipSuccess ||
        (e = hipMalloc((void**)&t.tab, tab_b)) != hipSuccess ||
        (e = hipHostMalloc((void**)&t.tab_staging, tab_b, hipHostMallocDefault)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&t.uploaded, hipEventDisableTiming)) != hipSuccess ||
        (!segs.empty() && (e = hipMemcpy(t.segs, segs.data(), segs.size() * sizeof(SegDesc),
                                         hipMemcpyHostToDevice)) != hipSuccess) ||
        (!seg_of.empty() && (e = hipMemcpy(t.seg_of, seg_of.data(), seg_of.size() * sizeof(int32_t),
                                           hipMemcpyHostToDevice)) != hipSuccess)) {
        free_seg_table(t);
        return device_fail(e, "allocating the layout's device tables");
    }
    c.tables.push_back(t);
    *out = &c.tables.back();
    return FP_OK;
}

// Uploads the pointer table (unless it holds these pointers already) and
// launches the segment copy of a table.
fp_status seg_run(SegTable* t, void* const* ptrs, hipStream_t s) {
    hipError_t e;
    const bool same = t->have_last && std::equal(ptrs, ptrs + t->n_ptrs, t->last_ptrs.begin());
    if (same) {
        // the table's last upload, wherever it was enqueued, comes first
        if ((e = hipStreamWaitEvent(s, t->uploaded, 0)) != hipSuccess) return device_fail(e, "hipStreamWaitEvent");
    } else {
        // the staging buffer may still feed the previous call's upload
        if ((e = hipEventSynchronize(t->uploaded)) != hipSuccess) return device_fail(e, "hipEventSynchronize");
        for (int32_t i = 0; i < t->n_ptrs; ++i) t->tab_staging[i] = ptrs[i];
        t->have_last = false;
        if ((e = hipMemcpyAsync(t->tab, t->tab_staging, (size_t)t->n_ptrs * sizeof(void*),
                                hipMemcpyHostToDevice, s)) != hipSuccess)
            return device_fail(e, "uploading the pointer table");
        if ((e = hipEventRecord(t->uploaded, s)) != hipSuccess) return device_fail(e, "hipEventRecord");
        t->last_ptrs.assign(ptrs, ptrs + t->n_ptrs);
        t->have_last = true;
    }
    if (t->groups == 0) return FP_OK;
    SegArgs a;
    a.segs = t->segs;
    a.seg_of = t->seg_of;
    a.dst_tab = t->tab;
    a.src_tab = t->tab;
    if ((e = launch_segments(a, t->groups, s)) != hipSuccess) return device_fail(e, "segment copy launch");
    return FP_OK;
}

// The pointer set a call of (op, es, rank) last passed validation with: a
// call with the same pointers skips the checks (they depend on nothing else).
bool seg_validated(SegCache& c, int op, int es, int rank, const std::vector<void*>& ptrs) {
    for (const auto& v : c.validated)
        if (v.op == op && v.es == es && v.rank == rank) return v.ptrs == ptrs;
    return false;
}
void seg_remember(SegCache& c, int op, int es, int rank, const std::vector<void*>& ptrs) {
    for (auto& v : c.validated)
        if (v.op == op && v.es == es && v.rank == rank) {
            v.ptrs = ptrs;
            return;
        }
    c.validated.push_back({op, es, rank, ptrs});
}

}  // namespace

// ---------------------------------------------------------------------- plan

struct fp_plan {
    int32_t n = 0;
    int32_t world = 1;
    std::vector<int32_t> ndims;
    std::vector<int64_t> dim_start;  // first dim of tensor i in `dims`
    std::vector<int64_t> dims;
    std::vector<int64_t> numel;
    std::vector<int64_t> offsets;    // n + 1
    int64_t total = 0, padded = 0, shard = 0;
    SegCache cache;                  // fp_pack's entry lists
};

namespace {
fp_status fp_plan_create_impl(int32_t n_tensors, const int32_t* ndims, const int64_t* shapes,
                                    int32_t world, fp_plan** out) {
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (n_tensors < 1) return fail(FP_ERR_RANGE, "n_tensors must be >= 1");
    if (ndims == nullptr) return fail(FP_ERR_INVALID, "ndims is NULL");
    if (world < 1 || world > (1 << 20)) return fail(FP_ERR_RANGE, "world %d outside [1, 2^20]", world);
    int64_t n_dims = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (ndims[i] < 0 || ndims[i] > FP_MAX_NDIM)
            return fail(FP_ERR_RANGE, "tensor %d: ndim %d outside [0, %d]", i, ndims[i], FP_MAX_NDIM);
        n_dims += ndims[i];
    }
    if (n_dims > 0 && shapes == nullptr) return fail(FP_ERR_INVALID, "shapes is NULL");
    fp_plan* p = new (std::nothrow) fp_plan();
    if (p == nullptr) return fail(FP_ERR_DEVICE, "out of host memory");
    p->n = n_tensors;
    p->world = world;
    p->ndims.assign(ndims, ndims + n_tensors);
    p->dims.assign(shapes, shapes + n_dims);
    p->offsets.push_back(0);
    const int64_t limit = (int64_t)1 << 62;
    int64_t d = 0, total = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        p->dim_start.push_back(d);
        int64_t ne = 1;
        for (int32_t k = 0; k < ndims[i]; ++k, ++d) {
            const int64_t s = shapes[d];
            if (s < 0) {
                delete p;
                return fail(FP_ERR_RANGE, "tensor %d: negative dimension", i);
            }
            if (s != 0 && ne > limit / s) {
                delete p;
                return fail(FP_ERR_RANGE, "tensor %d: too many elements", i);
            }
            ne *= s;
        }
        if (total > limit - ne) {
            delete p;
            return fail(FP_ERR_RANGE, "FlatParameter exceeds 2^62 elements");
        }
        total += ne;
        p->numel.push_back(ne);
        p->offsets.push_back(total);
    }
    p->total = total;
    p->padded = ceil_div(total, world) * world;
    p->shard = p->padded / world;
    *out = p;
    return FP_OK;
}
}  // namespace

extern "C" fp_status fp_plan_create(int32_t n_tensors, const int32_t* ndims, const int64_t* shapes,
                                    int32_t world, fp_plan** out) {
    try {
        return fp_plan_create_impl(n_tensors, ndims, shapes, world, out);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

extern "C" void fp_plan_destroy(fp_plan* plan) {
    delete plan;
}

extern "C" fp_status fp_plan_info(const fp_plan* plan, int64_t* numel, int64_t* padded, int64_t* shard) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (numel) *numel = plan->total;
    if (padded) *padded = plan->padded;
    if (shard) *shard = plan->shard;
    return FP_OK;
}

// ---------------------------------------------------------------------- views

extern "C" fp_status fp_unpack_views(const fp_plan* plan, int32_t rank, fp_view* out, int32_t cap,
                                     int32_t* n_out) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (rank < -1 || rank >= plan->world) return fail(FP_ERR_RANGE, "rank %d outside [-1, %d)", rank, plan->world);
    if (n_out) *n_out = plan->n;
    if (cap < plan->n) return fail(FP_ERR_RANGE, "cap %d < %d tensors", cap, plan->n);
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    const int64_t S = plan->shard;
    for (int32_t i = 0; i < plan->n; ++i) {
        fp_view v;
        std::memset(&v, 0, sizeof v);
        v.tensor = i;
        const int64_t o = plan->offsets[i], ne = plan->numel[i];
        if (rank < 0) {
            v.ndim = plan->ndims[i];
            v.buf_offset = o;
            v.numel = ne;
            for (int32_t k = 0; k < v.ndim; ++k) v.shape[k] = plan->dims[plan->dim_start[i] + k];
        } else {
            const int64_t lo = o > rank * S ? o : rank * S;
            const int64_t hi = (o + ne) < (rank + 1) * S ? (o + ne) : (rank + 1) * S;
            v.ndim = 1;
            if (hi > lo) {
                v.buf_offset = lo - rank * S;
                v.numel = hi - lo;
                v.tensor_offset = lo - o;
                v.shape[0] = hi - lo;
            }
        }
        out[i] = v;
    }
    return FP_OK;
}

// ---------------------------------------------------------------------- pack

namespace {
// FlatParameter construction as a segment list (2-byte units): tensor i is
// copied to flat[o_i, o_i + n_i) -- one copy entry, or for a tensor under
// kSegSmallPiece units one strided entry of a single piece, so that tiny
// tensors do not each cost a workgroup's worth of partial cache lines --
// and flat[T, P) is zero-filled.  Pointer table: [flat, tensors...].
std::vector<SegDesc> pack_segments(const fp_plan* p, int es) {
    const int64_t u = es / 2;
    std::vector<SegDesc> v;
    for (int32_t i = 0; i < p->n; ++i) {
        const int64_t len = p->numel[i] * u;
        if (len <= 0) continue;
        SegDesc d;
        std::memset(&d, 0, sizeof d);
        d.dst = 0;
        d.dst_off = p->offsets[i] * u;
        d.src = 1 + i;
        d.len = len;
        if (len < kSegSmallPiece) {
            d.kind = kSegStrided;
            d.piece = len;
            d.valid = len;
            d.dst_stride = len;
            d.src_stride = len;
        } else {
            d.kind = kSegCopy;
        }
        v.push_back(d);
    }
    if (p->padded > p->total) {
        SegDesc d;
        std::memset(&d, 0, sizeof d);
        d.kind = kSegCopy;
        d.dst = 0;
        d.dst_off = p->total * u;
        d.src = -1;
        d.len = (p->padded - p->total) * u;
        v.push_back(d);
    }
    return v;
}
}  // namespace

namespace {
fp_status fp_pack_impl(fp_plan* plan, int32_t elem_size, const void* const* src, void* flat,
                             void* stream) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (elem_size != 2 && elem_size != 4) return fail(FP_ERR_INVALID, "elem_size must be 2 or 4");
    if (src == nullptr) return fail(FP_ERR_INVALID, "src table is NULL");
    std::vector<void*> ptrs((size_t)plan->n + 1);
    ptrs[0] = flat;
    for (int32_t i = 0; i < plan->n; ++i) ptrs[1 + i] = const_cast<void*>(src[i]);
    std::lock_guard<std::mutex> lock(plan->cache.mu);
    if (!seg_validated(plan->cache, kOpFlatPack, elem_size, 0, ptrs)) {
        if (flat == nullptr && plan->padded > 0) return fail(FP_ERR_INVALID, "flat is NULL");
        if (!aligned(flat, 16)) return fail(FP_ERR_ALIGN, "flat is not 16-byte aligned");
        const int64_t flat_bytes = plan->padded * elem_size;
        for (int32_t i = 0; i < plan->n; ++i) {
            if (plan->numel[i] == 0) continue;
            if (src[i] == nullptr) return fail(FP_ERR_INVALID, "src[%d] is NULL", i);
            if (!aligned(src[i], (uintptr_t)elem_size)) return fail(FP_ERR_ALIGN, "src[%d] misaligned", i);
            if (overlap(src[i], plan->numel[i] * elem_size, flat, flat_bytes))
                return fail(FP_ERR_INVALID, "src[%d] overlaps flat", i);
        }
        seg_remember(plan->cache, kOpFlatPack, elem_size, 0, ptrs);
    }
    SegTable* t = nullptr;
    fp_status st = seg_table(plan->cache, kOpFlatPack, elem_size, 0, plan->n + 1,
                             [&] { return pack_segments(plan, elem_size); }, &t);
    if (st != FP_OK) return st;
    return seg_run(t, ptrs.data(), static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" fp_status fp_pack(fp_plan* plan, int32_t elem_size, const void* const* src, void* flat,
                             void* stream) {
    try {
        return fp_pack_impl(plan, elem_size, src, flat, stream);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

// ---------------------------------------------------------------------- reduce

extern "C" int64_t fp_workspace_bytes(int64_t shard) {
    if (shard < 0) shard = 0;
    return kWorkspaceHeader + 8 * partial_slots(shard);
}

namespace {
// Checks of the reduce's arguments and the filled kernel arguments.
fp_status reduce_args(int64_t shard, int32_t world, const uint16_t* const* grads, float scale, int32_t accumulate,
                      float* acc, int32_t* found_inf, double* sq_norm, void* workspace, ReduceArgs* a,
                      bool* aligned_grads) {
    fp_status st;
    if (shard < 0) return fail(FP_ERR_RANGE, "shard must be >= 0");
    if ((st = check_groups(stream_grid(shard), "the reduce")) != FP_OK) return st;
    if ((st = check_world(world)) != FP_OK) return st;
    if ((st = check_ptr_table(grads, world, shard, false, "grads")) != FP_OK) return st;
    if ((st = check_f32(acc, shard, "acc")) != FP_OK) return st;
    if (found_inf != nullptr && !aligned(found_inf, 4)) return fail(FP_ERR_ALIGN, "found_inf misaligned");
    if (sq_norm != nullptr) {
        if (!aligned(sq_norm, 8)) return fail(FP_ERR_ALIGN, "sq_norm misaligned");
        if (workspace == nullptr) return fail(FP_ERR_INVALID, "sq_norm needs a workspace");
        if (!aligned(workspace, 16)) return fail(FP_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    for (int32_t q = 0; q < world; ++q)
        if (overlap(grads[q], shard * 2, acc, shard * 4)) return fail(FP_ERR_INVALID, "grads[%d] overlaps acc", q);
    for (int32_t q = 0; q < world; ++q) a->grads[q] = grads[q];
    a->acc = acc;
    a->found_inf = found_inf;
    a->partials = sq_norm != nullptr ? partials_of(workspace) : nullptr;
    a->shard = shard;
    a->scale = scale;
    a->world = world;
    a->accumulate = accumulate ? 1 : 0;
    bool al = true;
    for (int32_t q = 0; q < world; ++q) al = al && is_aligned8(grads[q]);
    *aligned_grads = al;
    return FP_OK;
}
}  // namespace

extern "C" fp_status fp_reduce_shard(int64_t shard, int32_t world, const uint16_t* const* grads,
                                     float scale, int32_t accumulate, float* acc, int32_t* found_inf,
                                     double* sq_norm, void* workspace, void* stream) {
    ReduceArgs a;
    std::memset(&a, 0, sizeof a);
    bool al = false;
    fp_status st = reduce_args(shard, world, grads, scale, accumulate, acc, found_inf, sq_norm, workspace, &a, &al);
    if (st != FP_OK) return st;
    const int64_t grid = stream_grid(shard);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_reduce(a, grid, al, s);
    if (e != hipSuccess) return device_fail(e, "reduce launch");
    if (sq_norm != nullptr && (e = launch_norm_finalize(a.partials, (int)grid, sq_norm, s)) != hipSuccess)
        return device_fail(e, "norm launch");
    return FP_OK;
}

extern "C" fp_status fp_reduce_shard_hybrid(int64_t shard, int32_t world, int32_t group,
                                            const uint16_t* const* grads, float scale, int32_t accumulate,
                                            float* acc, int32_t* found_inf, double* sq_norm, void* workspace,
                                            void* stream) {
    if (group < 1 || group > world || (world > 0 && world % group != 0))
        return fail(FP_ERR_RANGE, "group %d must divide world %d", group, world);
    HybridArgs a;
    std::memset(&a, 0, sizeof a);
    bool al = false;
    fp_status st = reduce_args(shard, world, grads, scale, accumulate, acc, found_inf, sq_norm, workspace, &a, &al);
    if (st != FP_OK) return st;
    a.group = group;
    const int64_t grid = stream_grid(shard);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_reduce_hybrid(a, grid, al, s);
    if (e != hipSuccess) return device_fail(e, "hybrid reduce launch");
    if (sq_norm != nullptr && (e = launch_norm_finalize(a.partials, (int)grid, sq_norm, s)) != hipSuccess)
        return device_fail(e, "norm launch");
    return FP_OK;
}

extern "C" fp_status fp_adamw_shard(int64_t shard, const fp_adamw_hparams* hp, const float* grad,
                                    float* master, float* exp_avg, float* exp_avg_sq,
                                    const int32_t* found_inf, uint16_t* param_bf16, const double* grad_coef,
                                    void* stream) {
    fp_status st;
    if (shard < 0) return fail(FP_ERR_RANGE, "shard must be >= 0");
    if ((st = check_groups(stream_grid(shard), "AdamW")) != FP_OK) return st;
    AdamArgs a;
    std::memset(&a, 0, sizeof a);
    if ((st = check_hparams(hp, &a.c)) != FP_OK) return st;
    if ((st = check_f32(grad, shard, "grad")) != FP_OK || (st = check_f32(master, shard, "master")) != FP_OK ||
        (st = check_f32(exp_avg, shard, "exp_avg")) != FP_OK ||
        (st = check_f32(exp_avg_sq, shard, "exp_avg_sq")) != FP_OK)
        return st;
    const int64_t b = shard * 4;
    if (overlap(master, b, exp_avg, b) || overlap(master, b, exp_avg_sq, b) ||
        overlap(exp_avg, b, exp_avg_sq, b) || overlap(grad, b, master, b) || overlap(grad, b, exp_avg, b) ||
        overlap(grad, b, exp_avg_sq, b))
        return fail(FP_ERR_INVALID, "grad / master / exp_avg / exp_avg_sq overlap");
    if (param_bf16 != nullptr) {
        if (!aligned(param_bf16, 2)) return fail(FP_ERR_ALIGN, "param_bf16 misaligned");
        if (overlap(param_bf16, shard * 2, master, b) || overlap(param_bf16, shard * 2, exp_avg, b) ||
            overlap(param_bf16, shard * 2, exp_avg_sq, b) || overlap(param_bf16, shard * 2, grad, b))
            return fail(FP_ERR_INVALID, "param_bf16 overlaps the fp32 buffers");
    }
    if (found_inf != nullptr && !aligned(found_inf, 4)) return fail(FP_ERR_ALIGN, "found_inf misaligned");
    if (grad_coef != nullptr && !aligned(grad_coef, 8)) return fail(FP_ERR_ALIGN, "grad_coef misaligned");
    a.g_coef = grad_coef;
    a.grad = grad;
    a.master = master;
    a.exp_avg = exp_avg;
    a.exp_avg_sq = exp_avg_sq;
    a.param_bf16 = param_bf16;
    a.found_inf = found_inf;
    a.shard = shard;
    const bool aligned = param_bf16 == nullptr || is_aligned8(param_bf16);
    hipError_t e = launch_adamw(a, stream_grid(shard), aligned, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "adamw launch");
    return FP_OK;
}

// ---------------------------------------------------------------------- unshard

extern "C" fp_status fp_unshard(int64_t shard, int32_t world, const uint16_t* const* shards,
                                uint16_t* full, void* stream) {
    fp_status st;
    if (shard < 0) return fail(FP_ERR_RANGE, "shard must be >= 0");
    if ((st = check_groups(copy_tiles_per_shard(shard, kCopyWordsStream), "the unshard")) != FP_OK) return st;
    if ((st = check_world(world)) != FP_OK) return st;
    if ((st = check_ptr_table(shards, world, shard, true, "shards")) != FP_OK) return st;
    if (full == nullptr && shard > 0) return fail(FP_ERR_INVALID, "full is NULL");
    if (!aligned(full, 2)) return fail(FP_ERR_ALIGN, "full misaligned");
    for (int32_t q = 0; q < world; ++q)
        if (shards[q] != nullptr && overlap(shards[q], shard * 2, full, shard * world * 2))
            return fail(FP_ERR_INVALID, "shards[%d] overlaps full", q);
    if (shard == 0) return FP_OK;
    UnshardArgs a;
    std::memset(&a, 0, sizeof a);
    for (int32_t q = 0; q < world; ++q) a.shards[q] = shards[q];
    a.full = full;
    a.shard = shard;
    a.world = world;
    bool aligned = true;
    for (int32_t q = 0; q < world; ++q)
        if (shards[q] != nullptr) aligned = aligned && copy_source_aligned(shards[q], full, shard, q);
    hipError_t e = launch_unshard(a, copy_tiles_per_shard(shard, kCopyWordsStream), aligned, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "unshard launch");
    return FP_OK;
}

// ---------------------------------------------------------------------- step

namespace {

// Every check of fp_shard_step's arguments; the AdamW coefficients on success.
fp_status check_step(const fp_step_args& x, AdamCoef* c) {
    fp_status st;
    const int64_t S = x.shard;
    if (S < 0) return fail(FP_ERR_RANGE, "shard must be >= 0");
    if ((st = check_world(x.world)) != FP_OK) return st;
    if (x.rank < 0 || x.rank >= x.world) return fail(FP_ERR_RANGE, "rank %d outside [0, %d)", x.rank, x.world);
    // the first launch of the two-phase and no-skip paths: reduce tiles and
    // the other shards' copy tiles
    if ((st = check_groups(stream_grid(S) + (int64_t)(x.world - 1) * copy_tiles_per_shard(S, kCopyWordsStream),
                           "the step")) != FP_OK)
        return st;
    if (x.flags & ~(FP_STEP_NO_SKIP | FP_STEP_KEEP_GRAD | FP_STEP_NO_COOP))
        return fail(FP_ERR_INVALID, "unknown flags");
    if ((st = check_hparams(&x.hp, c)) != FP_OK) return st;
    if ((st = check_ptr_table(x.grads, x.world, S, false, "grads")) != FP_OK) return st;
    if ((st = check_ptr_table(x.shards, x.world, S, true, "shards")) != FP_OK) return st;
    for (int32_t q = 0; q < x.world; ++q)
        if (q != x.rank && x.shards[q] == nullptr && S > 0) return fail(FP_ERR_INVALID, "shards[%d] is NULL", q);
    if ((st = check_f32(x.acc, S, "acc")) != FP_OK || (st = check_f32(x.master, S, "master")) != FP_OK ||
        (st = check_f32(x.exp_avg, S, "exp_avg")) != FP_OK || (st = check_f32(x.exp_avg_sq, S, "exp_avg_sq")) != FP_OK)
        return st;
    if (x.full == nullptr && S > 0) return fail(FP_ERR_INVALID, "full is NULL");
    if (!aligned(x.full, 2)) return fail(FP_ERR_ALIGN, "full misaligned");
    if (x.found_inf == nullptr) return fail(FP_ERR_INVALID, "found_inf is NULL");
    if (!aligned(x.found_inf, 4)) return fail(FP_ERR_ALIGN, "found_inf misaligned");
    if (x.workspace != nullptr && !aligned(x.workspace, 16))
        return fail(FP_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (x.sq_norm != nullptr) {
        if (!aligned(x.sq_norm, 8)) return fail(FP_ERR_ALIGN, "sq_norm misaligned");
        if (x.workspace == nullptr) return fail(FP_ERR_INVALID, "sq_norm needs a workspace");
    }
    if (x.grad_coef != nullptr && !aligned(x.grad_coef, 8)) return fail(FP_ERR_ALIGN, "grad_coef misaligned");
    const int n_out = (x.master_out != nullptr) + (x.exp_avg_out != nullptr) + (x.exp_avg_sq_out != nullptr);
    if (n_out != 0 && n_out != 3)
        return fail(FP_ERR_INVALID, "master_out / exp_avg_out / exp_avg_sq_out: give all three or none");
    if (n_out == 3 && ((st = check_f32(x.master_out, S, "master_out")) != FP_OK ||
                       (st = check_f32(x.exp_avg_out, S, "exp_avg_out")) != FP_OK ||
                       (st = check_f32(x.exp_avg_sq_out, S, "exp_avg_sq_out")) != FP_OK))
        return st;
    const int64_t b4 = S * 4, b2 = S * 2, bf = S * x.world * 2;
    const void* f32s[7] = {x.acc, x.master, x.exp_avg, x.exp_avg_sq, x.master_out, x.exp_avg_out, x.exp_avg_sq_out};
    const int n_f32 = 4 + n_out;
    for (int i = 0; i < n_f32; ++i) {
        for (int j = i + 1; j < n_f32; ++j)
            if (overlap(f32s[i], b4, f32s[j], b4)) return fail(FP_ERR_INVALID, "fp32 buffers overlap");
        if (overlap(f32s[i], b4, x.full, bf)) return fail(FP_ERR_INVALID, "an fp32 buffer overlaps full");
    }
    for (int32_t q = 0; q < x.world; ++q) {
        if (overlap(x.grads[q], b2, x.full, bf)) return fail(FP_ERR_INVALID, "grads[%d] overlaps full", q);
        for (int i = 0; i < n_f32; ++i)
            if (overlap(x.grads[q], b2, f32s[i], b4)) return fail(FP_ERR_INVALID, "grads[%d] overlaps state", q);
        if (q != x.rank && overlap(x.shards[q], b2, x.full, bf))
            return fail(FP_ERR_INVALID, "shards[%d] overlaps full", q);
    }
    return FP_OK;
}

// The kernels a validated step launches: FP_PATH_*, and for the one-pass
// path its variant and grid.
fp_status step_path(const fp_step_args& x, int32_t* path, int* variant, int* grid) {
    *variant = -1;
    *grid = 0;
    if (x.flags & FP_STEP_NO_SKIP) {
        *path = x.shard >= kSplitElems ? FP_PATH_NO_SKIP_SPLIT : FP_PATH_NO_SKIP;
        return FP_OK;
    }
    const bool out_of_place = x.master_out != nullptr;
    // The one-pass kernel writes a kept gradient before its barrier, so it is
    // not used when acc is also an input (a cancelled barrier must leave acc
    // as it was).
    const bool acc_in_and_out = (x.flags & FP_STEP_KEEP_GRAD) && x.accumulate;
    if (x.workspace != nullptr && !(x.flags & FP_STEP_NO_COOP) && !acc_in_and_out) {
        const hipError_t e = plan_step_coop(x.shard, variant, grid);
        if (e != hipSuccess) return device_fail(e, "occupancy query");
    }
    if (*variant >= 0) {
        *path = out_of_place ? FP_PATH_SPECULATIVE_ONE_PASS : FP_PATH_ONE_PASS;
    } else if (out_of_place) {
        *path = x.shard >= kSplitElems ? FP_PATH_SPECULATIVE_SPLIT : FP_PATH_SPECULATIVE;
    } else {
        *path = FP_PATH_TWO_PHASE;
    }
    return FP_OK;
}

}  // namespace

extern "C" fp_status fp_step_path(const fp_step_args* args, int32_t* path) {
    if (args == nullptr || path == nullptr) return fail(FP_ERR_INVALID, "args or path is NULL");
    AdamCoef c;
    fp_status st = check_step(*args, &c);
    if (st != FP_OK) return st;
    int variant, grid;
    return step_path(*args, path, &variant, &grid);
}

namespace fpk {
fp_status report_error(fp_status status, const char* message) { return fail(status, "%s", message); }

fp_status shard_step_run(const fp_step_args* args, void* stream, bool give_up_test) {
    if (args == nullptr) return fail(FP_ERR_INVALID, "args is NULL");
    const fp_step_args& x = *args;
    const int64_t S = x.shard;
    StepArgs a;
    std::memset(&a, 0, sizeof a);
    fp_status st = check_step(x, &a.c);
    if (st != FP_OK) return st;
    int32_t path = 0;
    int variant = -1, grid = 0;
    if ((st = step_path(x, &path, &variant, &grid)) != FP_OK) return st;
    const bool one_pass = path == FP_PATH_ONE_PASS || path == FP_PATH_SPECULATIVE_ONE_PASS;
    if (give_up_test && !one_pass) return fail(FP_ERR_INVALID, "these arguments do not take the one-pass path");

    const bool speculative = path == FP_PATH_SPECULATIVE || path == FP_PATH_SPECULATIVE_SPLIT;
    // the fused launch(es) without a gate: no-skip, and speculative (gate after)
    const bool no_skip = path == FP_PATH_NO_SKIP || path == FP_PATH_NO_SKIP_SPLIT || speculative;
    const bool split = path == FP_PATH_NO_SKIP_SPLIT || path == FP_PATH_SPECULATIVE_SPLIT;
    const bool out_of_place = x.master_out != nullptr;
    for (int32_t q = 0; q < x.world; ++q) {
        a.grads[q] = x.grads[q];
        a.shards[q] = q == x.rank ? nullptr : x.shards[q];
    }
    a.acc = x.acc;
    a.master = x.master;
    a.exp_avg = x.exp_avg;
    a.exp_avg_sq = x.exp_avg_sq;
    a.full = x.full;
    a.found_inf = x.found_inf;
    a.partials = x.sq_norm != nullptr ? partials_of(x.workspace) : nullptr;
    a.sq_norm = x.sq_norm;
    a.g_coef = x.grad_coef;
    a.shard = S;
    a.scale = x.scale;
    a.world = x.world;
    a.rank = x.rank;
    a.accumulate = x.accumulate ? 1 : 0;
    a.keep_grad = (x.flags & FP_STEP_KEEP_GRAD) ? 1 : 0;
    a.sync = x.workspace != nullptr ? static_cast<GridSync*>(x.workspace) : nullptr;
    a.master_out = out_of_place ? x.master_out : x.master;
    a.exp_avg_out = out_of_place ? x.exp_avg_out : x.exp_avg;
    a.exp_avg_sq_out = out_of_place ? x.exp_avg_sq_out : x.exp_avg_sq;

    uint16_t* own = x.full + (int64_t)x.rank * S;
    bool aligned = is_aligned8(own), copy_aligned = true;
    for (int32_t q = 0; q < x.world; ++q) {
        aligned = aligned && is_aligned8(x.grads[q]);
        if (q != x.rank) copy_aligned = copy_aligned && copy_source_aligned(x.shards[q], x.full, S, q);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev[FP_STEP_EVENTS] = {nullptr, nullptr, nullptr};
    if (x.profile_events != nullptr)
        for (int i = 0; i < FP_STEP_EVENTS; ++i) ev[i] = static_cast<hipEvent_t>(x.profile_events[i]);
    hipError_t e;

    if (one_pass) {
        if (ev[0] && (e = hipEventRecord(ev[0], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
        if ((e = launch_step_coop(a, variant, grid, aligned, copy_aligned, s, give_up_test)) != hipSuccess)
            return device_fail(e, "one-pass step launch");
        if (ev[1] && (e = hipEventRecord(ev[1], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
        if (x.sq_norm != nullptr && (e = launch_norm_finalize(a.partials, grid, x.sq_norm, s)) != hipSuccess)
            return device_fail(e, "norm launch");
        if (ev[2] && (e = hipEventRecord(ev[2], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
        return FP_OK;
    }
    if (ev[0] && (e = hipEventRecord(ev[0], s)) != hipSuccess) return device_fail(e, "hipEventRecord");

    // Reduce (and, without the gate, update) tiles plus the copy of the other
    // ranks' shards as (shard, tile) pairs, in one launch.
    const int64_t reduce_groups = stream_grid(S);
    a.reduce_groups = (int32_t)reduce_groups;
    a.copy_tiles = (int32_t)copy_tiles_per_shard(S, kCopyWordsStream);
    const int64_t n_groups = reduce_groups + (int64_t)(x.world - 1) * a.copy_tiles;
    AdamArgs d;
    std::memset(&d, 0, sizeof d);
    d.grad = x.acc;
    d.master = x.master;
    d.exp_avg = x.exp_avg;
    d.exp_avg_sq = x.exp_avg_sq;
    d.param_bf16 = own;
    d.found_inf = x.found_inf;
    d.shard = S;
    d.c = a.c;
    d.g_coef = a.g_coef;
    d.partials = a.partials;
    d.sq_norm = x.sq_norm;
    d.n_partials = (int32_t)reduce_groups;
    if ((e = launch_step_phase1(a, split ? reduce_groups : n_groups, no_skip, split, aligned, copy_aligned, s)) !=
        hipSuccess)
        return device_fail(e, "step launch");
    if (ev[1] && (e = hipEventRecord(ev[1], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
    if (split) {
        // the copy of the other shards, at full occupancy
        UnshardArgs u;
        std::memset(&u, 0, sizeof u);
        for (int32_t q = 0; q < x.world; ++q) u.shards[q] = a.shards[q];
        u.full = a.full;
        u.shard = S;
        u.world = x.world;
        if ((e = launch_unshard(u, a.copy_tiles, copy_aligned, s)) != hipSuccess) return device_fail(e, "copy launch");
    }
    if (no_skip) {
        if (x.sq_norm != nullptr &&
            (e = launch_norm_finalize(a.partials, (int)reduce_groups, x.sq_norm, s)) != hipSuccess)
            return device_fail(e, "norm launch");
        if (speculative && S > 0) {
            // the skip rule, applied after the update: restore on overflow
            ResolveArgs r;
            std::memset(&r, 0, sizeof r);
            r.found_inf = x.found_inf;
            r.master = x.master;
            r.exp_avg = x.exp_avg;
            r.exp_avg_sq = x.exp_avg_sq;
            r.master_out = x.master_out;
            r.exp_avg_out = x.exp_avg_out;
            r.exp_avg_sq_out = x.exp_avg_sq_out;
            r.own = own;
            r.shard = S;
            if ((e = launch_step_resolve(r, s)) != hipSuccess) return device_fail(e, "resolve launch");
        }
    } else {
        if ((e = launch_adamw(d, stream_grid(S), is_aligned8(own), s)) != hipSuccess)
            return device_fail(e, "adamw launch");
    }
    if (ev[2] && (e = hipEventRecord(ev[2], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
    return FP_OK;
}
}  // namespace fpk

extern "C" fp_status fp_shard_step(const fp_step_args* args, void* stream) {
    return shard_step_run(args, stream, false);
}

extern "C" fp_status fp_step_test_give_up(const fp_step_args* args, void* stream) {
    return shard_step_run(args, stream, true);
}

// ---------------------------------------------------------------------- units

struct fp_units {
    int32_t n = 0, world = 1, rank = 0;
    int device = -1;
    bool has_unshard = false;
    bool aligned = true;        // gradient rows and own slices 8-byte aligned
    bool copy_aligned = true;   // copy sources 16-byte aligned
    int64_t partition = 0;
    int64_t reduce_groups = 0, copy_groups = 0;
    std::vector<int64_t> shard, offset;
    std::vector<const uint16_t*> grads, shards;  // host copies, for validation
    std::vector<uint16_t*> full;
    void* dev = nullptr;  // unit records [n], then the per-workgroup unit index [groups]
    int64_t record_bytes = 0;
    int32_t tile_run = 0, copy_run = 0;  // equal tile counts of all units but the last, or 0
};

namespace {
void free_units(fp_units* u) {
    if (u->dev != nullptr) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(u->device);
        (void)hipFree(u->dev);
        if (cur >= 0) (void)hipSetDevice(cur);
    }
    delete u;
}

int64_t units_workspace_bytes(const fp_units* u) { return kWorkspaceHeader + 8 * (u->reduce_groups + 1); }

fp_status check_units_state(const fp_units* u, const float* const* f32, const char* const* names, int n) {
    const int64_t b4 = u->partition * 4;
    for (int i = 0; i < n; ++i) {
        fp_status st = check_f32(f32[i], u->partition, names[i]);
        if (st != FP_OK) return st;
        for (int j = 0; j < i; ++j)
            if (overlap(f32[i], b4, f32[j], b4)) return fail(FP_ERR_INVALID, "%s overlaps %s", names[i], names[j]);
        for (int32_t k = 0; k < u->n; ++k) {
            const int64_t S = u->shard[k];
            for (int32_t q = 0; q < u->world; ++q)
                if (overlap(u->grads[(size_t)k * u->world + q], 2 * S, f32[i], b4))
                    return fail(FP_ERR_INVALID, "unit %d: grads[%d] overlaps %s", k, q, names[i]);
            if (u->has_unshard && overlap(u->full[k], 2 * S * u->world, f32[i], b4))
                return fail(FP_ERR_INVALID, "unit %d: full overlaps %s", k, names[i]);
        }
    }
    return FP_OK;
}

fp_status check_units_device(const fp_units* u) {
    int device = -1;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return device_fail(e, "hipGetDevice");
    if (device != u->device)
        return fail(FP_ERR_INVALID, "units plan was created on device %d, current is %d", u->device, device);
    return FP_OK;
}

void fill_units_args(const fp_units* u, UnitsArgs* a) {
    std::memset(a, 0, sizeof *a);
    a->records = static_cast<const char*>(u->dev);
    a->unit_of = reinterpret_cast<const int32_t*>(static_cast<const char*>(u->dev) +
                                                  u->record_bytes * u->n);
    a->record_bytes = u->record_bytes;
    a->tile_run = u->tile_run;
    a->copy_run = u->copy_run;
    a->reduce_groups = u->reduce_groups;
    a->n_units = u->n;
    a->world = u->world;
    a->rank = u->rank;
}
}  // namespace

namespace {
fp_status fp_units_create_impl(int32_t n_units, int32_t world, int32_t rank, const int64_t* shard,
                                     const uint16_t* const* grads, const uint16_t* const* shards,
                                     uint16_t* const* full, fp_units** out) {
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    *out = nullptr;
    fp_status st;
    if (n_units < 1) return fail(FP_ERR_RANGE, "n_units must be >= 1");
    if ((st = check_world(world)) != FP_OK) return st;
    if (rank < 0 || rank >= world) return fail(FP_ERR_RANGE, "rank %d outside [0, %d)", rank, world);
    if (shard == nullptr || grads == nullptr) return fail(FP_ERR_INVALID, "shard or grads table is NULL");
    if ((shards == nullptr) != (full == nullptr))
        return fail(FP_ERR_INVALID, "shards and full must both be given or both be NULL");
    const bool unshard = shards != nullptr;
    int64_t partition = 0, tiles = 0, copies = 0;
    for (int32_t k = 0; k < n_units; ++k) {
        const int64_t S = shard[k];
        if (S < 0 || S > ((int64_t)1 << 40)) return fail(FP_ERR_RANGE, "unit %d: shard %lld out of range", k, (long long)S);
        if ((st = check_ptr_table(grads + (size_t)k * world, world, S, false, "grads")) != FP_OK) return st;
        if (unshard) {
            if ((st = check_ptr_table(shards + (size_t)k * world, world, S, true, "shards")) != FP_OK) return st;
            if (full[k] == nullptr && S > 0) return fail(FP_ERR_INVALID, "unit %d: full is NULL", k);
            if (!aligned(full[k], 2)) return fail(FP_ERR_ALIGN, "unit %d: full misaligned", k);
            for (int32_t q = 0; q < world; ++q) {
                const uint16_t* src = shards[(size_t)k * world + q];
                if (q != rank && src == nullptr && S > 0) return fail(FP_ERR_INVALID, "unit %d: shards[%d] is NULL", k, q);
                if (q != rank && overlap(src, 2 * S, full[k], 2 * S * world))
                    return fail(FP_ERR_INVALID, "unit %d: shards[%d] overlaps full", k, q);
                if (overlap(grads[(size_t)k * world + q], 2 * S, full[k], 2 * S * world))
                    return fail(FP_ERR_INVALID, "unit %d: grads[%d] overlaps full", k, q);
            }
        }
        partition += (S + 3) & ~(int64_t)3;
        tiles += unit_tiles(S);
        if (unshard) copies += (int64_t)(world - 1) * copy_tiles_per_shard(S, kCopyWordsStream);
    }
    if ((st = check_groups(tiles + copies, "the units' step")) != FP_OK) return st;

    fp_units* u = new (std::nothrow) fp_units();
    if (u == nullptr) return fail(FP_ERR_DEVICE, "out of host memory");
    u->n = n_units;
    u->world = world;
    u->rank = rank;
    u->has_unshard = unshard;
    u->shard.assign(shard, shard + n_units);
    u->grads.assign(grads, grads + (size_t)n_units * world);
    if (unshard) {
        u->shards.assign(shards, shards + (size_t)n_units * world);
        u->full.assign(full, full + n_units);
    }
    u->reduce_groups = tiles;
    u->copy_groups = copies;
    u->partition = partition;

    // host image of the device tables: unit records, then the unit index of every workgroup
    const size_t n = (size_t)n_units, w = (size_t)world;
    u->record_bytes = unit_record_bytes(world);
    const size_t rec_b = n * (size_t)u->record_bytes;
    const size_t total_b = rec_b + (size_t)(tiles + copies) * sizeof(int32_t);
    std::vector<unsigned char> img(total_b, 0);
    int32_t* unit_of = reinterpret_cast<int32_t*>(img.data() + rec_b);
    hipError_t e = hipGetDevice(&u->device);
    if (e == hipSuccess) e = hipMalloc(&u->dev, total_b);
    if (e != hipSuccess) {
        u->dev = nullptr;
        free_units(u);
        return device_fail(e, "allocating the units tables");
    }
    int64_t off = 0, t0 = 0, c0 = 0;
    bool al = true, cal = true;
    for (size_t k = 0; k < n; ++k) {
        const int64_t S = shard[k];
        unsigned char* rec = img.data() + k * (size_t)u->record_bytes;
        UnitDesc d;
        std::memset(&d, 0, sizeof d);
        d.shard = S;
        d.offset = off;
        d.tile0 = t0;
        d.copy0 = c0;
        d.full = unshard ? full[k] : nullptr;
        d.copy_tiles = unshard ? (int32_t)copy_tiles_per_shard(S, kCopyWordsStream) : 0;
        std::memcpy(rec, &d, sizeof d);
        const uint16_t** gtab = reinterpret_cast<const uint16_t**>(rec + kUnitHeader);
        const uint16_t** stab = gtab + w;
        u->offset.push_back(off);
        const int64_t nt = unit_tiles(S), nc = unshard ? (int64_t)(world - 1) * d.copy_tiles : 0;
        for (int64_t i = 0; i < nt; ++i) unit_of[t0 + i] = (int32_t)k;
        for (int64_t i = 0; i < nc; ++i) unit_of[tiles + c0 + i] = (int32_t)k;
        off += (S + 3) & ~(int64_t)3;
        t0 += nt;
        c0 += nc;
        for (size_t q = 0; q < w; ++q) {
            gtab[q] = grads[k * w + q];
            al = al && is_aligned8(grads[k * w + q]);
            if (unshard) {
                stab[q] = (int32_t)q == rank ? nullptr : shards[k * w + q];
                if ((int32_t)q != rank) cal = cal && copy_source_aligned(shards[k * w + q], full[k], S, (int)q);
            }
        }
        if (unshard) al = al && is_aligned8(full[k] + (int64_t)rank * S);
    }
    u->aligned = al;
    u->copy_aligned = cal;
    // equal units (all but the last): the unit of a workgroup is a division
    {
        const int64_t t = unit_tiles(shard[0]);
        const int64_t c = unshard ? (int64_t)(world - 1) * copy_tiles_per_shard(shard[0], kCopyWordsStream) : 0;
        bool eq_t = true, eq_c = true;
        for (size_t k = 1; k + 1 < n; ++k) {
            eq_t = eq_t && unit_tiles(shard[k]) == t;
            eq_c = eq_c && (unshard ? (int64_t)(world - 1) * copy_tiles_per_shard(shard[k], kCopyWordsStream) : 0) == c;
        }
        u->tile_run = eq_t && t <= 0x7FFFFFFF ? (int32_t)t : 0;
        u->copy_run = eq_c && c > 0 && c <= 0x7FFFFFFF ? (int32_t)c : 0;
    }
    if ((e = hipMemcpy(u->dev, img.data(), total_b, hipMemcpyHostToDevice)) != hipSuccess) {
        free_units(u);
        return device_fail(e, "uploading the units tables");
    }
    *out = u;
    return FP_OK;
}
}  // namespace

extern "C" fp_status fp_units_create(int32_t n_units, int32_t world, int32_t rank, const int64_t* shard,
                                     const uint16_t* const* grads, const uint16_t* const* shards,
                                     uint16_t* const* full, fp_units** out) {
    try {
        return fp_units_create_impl(n_units, world, rank, shard, grads, shards, full, out);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

extern "C" void fp_units_destroy(fp_units* units) {
    if (units != nullptr) free_units(units);
}

extern "C" fp_status fp_units_info(const fp_units* units, int64_t* partition, int64_t* workspace_bytes) {
    if (units == nullptr) return fail(FP_ERR_INVALID, "units is NULL");
    if (partition) *partition = units->partition;
    if (workspace_bytes) *workspace_bytes = units_workspace_bytes(units);
    return FP_OK;
}

extern "C" fp_status fp_units_offsets(const fp_units* units, int64_t* offsets) {
    if (units == nullptr || offsets == nullptr) return fail(FP_ERR_INVALID, "units or offsets is NULL");
    for (int32_t k = 0; k < units->n; ++k) offsets[k] = units->offset[k];
    return FP_OK;
}

extern "C" fp_status fp_units_reduce(const fp_units* units, float scale, int32_t accumulate, float* acc,
                                     int32_t* found_inf, double* sq_norm, void* workspace, void* stream) {
    if (units == nullptr) return fail(FP_ERR_INVALID, "units is NULL");
    fp_status st;
    const float* f32[1] = {acc};
    const char* names[1] = {"acc"};
    if ((st = check_units_state(units, f32, names, 1)) != FP_OK) return st;
    if (found_inf != nullptr && !aligned(found_inf, 4)) return fail(FP_ERR_ALIGN, "found_inf misaligned");
    if (sq_norm != nullptr) {
        if (!aligned(sq_norm, 8)) return fail(FP_ERR_ALIGN, "sq_norm misaligned");
        if (workspace == nullptr) return fail(FP_ERR_INVALID, "sq_norm needs a workspace");
        if (!aligned(workspace, 16)) return fail(FP_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    if ((st = check_units_device(units)) != FP_OK) return st;
    UnitsArgs a;
    fill_units_args(units, &a);
    a.acc = acc;
    a.found_inf = found_inf;
    a.partials = sq_norm != nullptr ? partials_of(workspace) : nullptr;
    a.scale = scale;
    a.accumulate = accumulate ? 1 : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_units_reduce(a, units->aligned, units->partition >= kSplitElems, s);
    if (e != hipSuccess) return device_fail(e, "units reduce launch");
    if (sq_norm != nullptr && (e = launch_norm_finalize(a.partials, (int)units->reduce_groups, sq_norm, s)) != hipSuccess)
        return device_fail(e, "norm launch");
    return FP_OK;
}

namespace {
// Every check of fp_units_step's arguments; fills the launch arguments.
fp_status check_units_step(const fp_units* units, const fp_units_step_args& x, UnitsArgs* a) {
    if (!units->has_unshard) return fail(FP_ERR_INVALID, "units plan has no shards / full buffers");
    if (x.flags & ~(FP_STEP_NO_SKIP | FP_STEP_KEEP_GRAD)) return fail(FP_ERR_INVALID, "unknown flags");
    fill_units_args(units, a);
    fp_status st;
    if ((st = check_hparams(&x.hp, &a->c)) != FP_OK) return st;
    const int n_out = (x.master_out != nullptr) + (x.exp_avg_out != nullptr) + (x.exp_avg_sq_out != nullptr);
    if (n_out != 0 && n_out != 3)
        return fail(FP_ERR_INVALID, "master_out / exp_avg_out / exp_avg_sq_out: give all three or none");
    const float* f32[7] = {x.acc, x.master, x.exp_avg, x.exp_avg_sq, x.master_out, x.exp_avg_out, x.exp_avg_sq_out};
    const char* names[7] = {"acc", "master", "exp_avg", "exp_avg_sq", "master_out", "exp_avg_out", "exp_avg_sq_out"};
    if ((st = check_units_state(units, f32, names, 4 + n_out)) != FP_OK) return st;
    if (x.found_inf == nullptr) return fail(FP_ERR_INVALID, "found_inf is NULL");
    if (!aligned(x.found_inf, 4)) return fail(FP_ERR_ALIGN, "found_inf misaligned");
    if (x.sq_norm != nullptr) {
        if (!aligned(x.sq_norm, 8)) return fail(FP_ERR_ALIGN, "sq_norm misaligned");
        if (x.workspace == nullptr) return fail(FP_ERR_INVALID, "sq_norm needs a workspace");
        if (!aligned(x.workspace, 16)) return fail(FP_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    if (x.grad_coef != nullptr && !aligned(x.grad_coef, 8)) return fail(FP_ERR_ALIGN, "grad_coef misaligned");
    a->g_coef = x.grad_coef;
    a->master_out = x.master_out;
    a->exp_avg_out = x.exp_avg_out;
    a->exp_avg_sq_out = x.exp_avg_sq_out;
    a->acc = x.acc;
    a->master = x.master;
    a->exp_avg = x.exp_avg;
    a->exp_avg_sq = x.exp_avg_sq;
    a->found_inf = x.found_inf;
    a->partials = x.sq_norm != nullptr ? partials_of(x.workspace) : nullptr;
    a->scale = x.scale;
    a->accumulate = x.accumulate ? 1 : 0;
    a->keep_grad = (x.flags & FP_STEP_KEEP_GRAD) ? 1 : 0;
    return FP_OK;
}

// The launches of a validated multi-unit step: FP_PATH_TWO_PHASE, or the
// fused launch without a gate -- no-skip, or speculative (gate after) --
// whose copies go to a launch of their own for partitions of kSplitElems
// elements and more (measured at the bucketed 611M model: 1.58 ms per step
// with the copies in the fused launch, 1.55 ms split).
int32_t units_path(const fp_units* u, const fp_units_step_args& x) {
    const bool speculative = x.master_out != nullptr && !(x.flags & FP_STEP_NO_SKIP);
    if (!speculative && !(x.flags & FP_STEP_NO_SKIP)) return FP_PATH_TWO_PHASE;
    const bool split = u->partition >= kSplitElems && u->copy_groups > 0;
    if (speculative) return split ? FP_PATH_SPECULATIVE_SPLIT : FP_PATH_SPECULATIVE;
    return split ? FP_PATH_NO_SKIP_SPLIT : FP_PATH_NO_SKIP;
}
}  // namespace

extern "C" fp_status fp_units_step_path(const fp_units* units, const fp_units_step_args* args, int32_t* path) {
    if (units == nullptr || args == nullptr || path == nullptr)
        return fail(FP_ERR_INVALID, "units, args or path is NULL");
    UnitsArgs a;
    fp_status st = check_units_step(units, *args, &a);
    if (st != FP_OK) return st;
    *path = units_path(units, *args);
    return FP_OK;
}

extern "C" fp_status fp_units_step(const fp_units* units, const fp_units_step_args* args, void* stream) {
    if (units == nullptr || args == nullptr) return fail(FP_ERR_INVALID, "units or args is NULL");
    const fp_units_step_args& x = *args;
    UnitsArgs a;
    fp_status st = check_units_step(units, x, &a);
    if (st != FP_OK) return st;
    if ((st = check_units_device(units)) != FP_OK) return st;
    const int32_t path = units_path(units, x);
    const bool speculative = path == FP_PATH_SPECULATIVE || path == FP_PATH_SPECULATIVE_SPLIT;
    const bool split = path == FP_PATH_SPECULATIVE_SPLIT || path == FP_PATH_NO_SKIP_SPLIT;
    const bool no_skip = path != FP_PATH_TWO_PHASE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev[FP_STEP_EVENTS] = {nullptr, nullptr, nullptr};
    if (x.profile_events != nullptr)
        for (int i = 0; i < FP_STEP_EVENTS; ++i) ev[i] = static_cast<hipEvent_t>(x.profile_events[i]);
    hipError_t e;
    if (ev[0] && (e = hipEventRecord(ev[0], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
    // The split launch's reduce + AdamW workgroups keep full occupancy: at the
    // bucketed 611M model's 16 ranks (38.2M-element partition) the occupancy
    // cap that serves the single-unit step made them slower (MI355X: 612 us
    // capped at four workgroups per CU, 517 us at five, 445 us uncapped).
    if ((e = launch_units_phase1(a, split ? 0 : units->copy_groups, no_skip, false, units->aligned,
                                 units->copy_aligned, s)) != hipSuccess)
        return device_fail(e, "units step launch");
    if (ev[1] && (e = hipEventRecord(ev[1], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
    if (split && (e = launch_units_copy(a, units->copy_groups, units->copy_aligned, s)) != hipSuccess)
        return device_fail(e, "units copy launch");
    if (no_skip) {
        if (x.sq_norm != nullptr &&
            (e = launch_norm_finalize(a.partials, (int)units->reduce_groups, x.sq_norm, s)) != hipSuccess)
            return device_fail(e, "norm launch");
        // the skip rule, applied after the update: restore on overflow
        if (speculative && (e = launch_units_resolve(a, s)) != hipSuccess)
            return device_fail(e, "units resolve launch");
    } else {
        a.sq_norm = x.sq_norm;
        if ((e = launch_units_adamw(a, units->aligned, s)) != hipSuccess) return device_fail(e, "units adamw launch");
    }
    if (ev[2] && (e = hipEventRecord(ev[2], s)) != hipSuccess) return device_fail(e, "hipEventRecord");
    return FP_OK;
}

// ---------------------------------------------------------------------- dim-0 layout

struct fp_shard0_plan {
    int32_t n = 0, world = 1;
    std::vector<int32_t> ndims;
    std::vector<int64_t> dims, dim_start, d0, rows, row_elems, off, numel;
    int64_t shard = 0, total = 0;
    SegCache cache;
};

namespace {
int64_t real_rows(const fp_shard0_plan* p, int32_t i, int32_t q) {
    const int64_t left = p->d0[i] - (int64_t)q * p->rows[i];
    return left < 0 ? 0 : (left < p->rows[i] ? left : p->rows[i]);
}

// The segment list of an operation, in 2-byte units.  Pointer table: pack ->
// [dst, params...]; unpack -> [params..., full].  A parameter whose per-rank
// piece is below kSegSmallPiece units gets one strided entry for all its
// pieces; the others one copy entry per piece (and per padding fill).
std::vector<SegDesc> shard0_segments(const fp_shard0_plan* p, int op, int es, int rank) {
    const int64_t u = es / 2;
    const int64_t S = p->shard * u;
    std::vector<SegDesc> v;
    auto copy = [&](int32_t dst, int64_t dst_off, int32_t src, int64_t src_off, int64_t len) {
        if (len <= 0) return;
        SegDesc d;
        std::memset(&d, 0, sizeof d);
        d.kind = kSegCopy;
        d.dst = dst;
        d.dst_off = dst_off;
        d.src = src;
        d.src_off = src_off;
        d.len = len;
        v.push_back(d);
    };
    auto strided = [&](int32_t dst, int64_t dst_off, int64_t dst_stride, int32_t src, int64_t src_off,
                       int64_t src_stride, int64_t piece, int64_t len, int64_t valid) {
        if (len <= 0) return;
        SegDesc d;
        std::memset(&d, 0, sizeof d);
        d.kind = kSegStrided;
        d.dst = dst;
        d.dst_off = dst_off;
        d.dst_stride = dst_stride;
        d.src = src;
        d.src_off = src_off;
        d.src_stride = src_stride;
        d.piece = piece;
        d.len = len;
        d.valid = valid < 0 ? 0 : (valid < len ? valid : len);
        v.push_back(d);
    };
    auto piece = [&](int32_t i) { return p->rows[i] * p->row_elems[i] * u; };
    auto small = [&](int32_t i) { return piece(i) < kSegSmallPiece; };
    if (op == kOpUnpack) {
        for (int32_t i = 0; i < p->n; ++i) {
            if (small(i)) {
                strided(i, 0, piece(i), p->n, p->off[i] * u, S, piece(i), p->numel[i] * u, p->numel[i] * u);
                continue;
            }
            for (int32_t q = 0; q < p->world; ++q)
                copy(i, q * piece(i), p->n, q * S + p->off[i] * u, real_rows(p, i, q) * p->row_elems[i] * u);
        }
        return v;
    }
    const bool all = op == kOpPackAll;
    const int32_t q0 = all ? 0 : rank, q1 = all ? p->world : rank + 1;
    for (int32_t q = q0; q < q1; ++q) {
        const int64_t base = all ? q * S : 0;
        for (int32_t i = 0; i < p->n; ++i) {
            if (small(i)) continue;
            const int64_t real = real_rows(p, i, q) * p->row_elems[i] * u;
            copy(0, base + p->off[i] * u, 1 + i, q * piece(i), real);
            copy(0, base + p->off[i] * u + real, -1, 0, piece(i) - real);
        }
    }
    for (int32_t i = 0; i < p->n; ++i) {
        if (!small(i)) continue;
        if (all)
            strided(0, p->off[i] * u, S, 1 + i, 0, piece(i), piece(i), p->world * piece(i), p->numel[i] * u);
        else
            strided(0, p->off[i] * u, piece(i), 1 + i, rank * piece(i), piece(i), piece(i), piece(i),
                    p->numel[i] * u - rank * piece(i));
    }
    return v;
}

fp_status shard0_table(fp_shard0_plan* p, int op, int es, int rank, SegTable** out) {
    return seg_table(p->cache, op, es, rank, p->n + 1, [&] { return shard0_segments(p, op, es, rank); }, out);
}

}  // namespace

namespace {
fp_status fp_shard0_plan_create_impl(int32_t n_params, const int32_t* ndims, const int64_t* shapes,
                                           int32_t world, fp_shard0_plan** out) {
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (n_params < 1) return fail(FP_ERR_RANGE, "n_params must be >= 1");
    if (ndims == nullptr) return fail(FP_ERR_INVALID, "ndims is NULL");
    fp_status st;
    if ((st = check_world(world)) != FP_OK) return st;
    int64_t n_dims = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        if (ndims[i] < 0 || ndims[i] > FP_MAX_NDIM)
            return fail(FP_ERR_RANGE, "parameter %d: ndim %d outside [0, %d]", i, ndims[i], FP_MAX_NDIM);
        n_dims += ndims[i];
    }
    if (n_dims > 0 && shapes == nullptr) return fail(FP_ERR_INVALID, "shapes is NULL");
    fp_shard0_plan* p = new (std::nothrow) fp_shard0_plan();
    if (p == nullptr) return fail(FP_ERR_DEVICE, "out of host memory");
    p->n = n_params;
    p->world = world;
    p->ndims.assign(ndims, ndims + n_params);
    p->dims.assign(shapes, shapes + n_dims);
    const int64_t limit = (int64_t)1 << 40;
    int64_t d = 0, off = 0, total = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        p->dim_start.push_back(d);
        int64_t d0 = 1, r = 1;
        for (int32_t k = 0; k < ndims[i]; ++k, ++d) {
            const int64_t s = shapes[d];
            if (s < 0 || s > limit) {
                delete p;
                return fail(FP_ERR_RANGE, "parameter %d: dimension %lld out of range", i, (long long)s);
            }
            if (k == 0) d0 = s;
            else r *= s;
            if (r > limit) {
                delete p;
                return fail(FP_ERR_RANGE, "parameter %d: too many elements", i);
            }
        }
        const int64_t c = (d0 + world - 1) / world;
        if (r > 0 && d0 > limit / r) {          // numel, and so c * r, above 2^40
            delete p;
            return fail(FP_ERR_RANGE, "parameter %d: too many elements", i);
        }
        p->d0.push_back(d0);
        p->rows.push_back(c);
        p->row_elems.push_back(r);
        p->off.push_back(off);
        p->numel.push_back(d0 * r);
        off += c * r;
        total += d0 * r;
        if (off > limit) {
            delete p;
            return fail(FP_ERR_RANGE, "group buffer exceeds 2^40 elements");
        }
    }
    p->shard = off;
    p->total = total;
    *out = p;
    return FP_OK;
}
}  // namespace

extern "C" fp_status fp_shard0_plan_create(int32_t n_params, const int32_t* ndims, const int64_t* shapes,
                                           int32_t world, fp_shard0_plan** out) {
    try {
        return fp_shard0_plan_create_impl(n_params, ndims, shapes, world, out);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

extern "C" void fp_shard0_plan_destroy(fp_shard0_plan* plan) {
    delete plan;
}

extern "C" fp_status fp_shard0_plan_info(const fp_shard0_plan* plan, int64_t* shard, int64_t* numel) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (shard) *shard = plan->shard;
    if (numel) *numel = plan->total;
    return FP_OK;
}

extern "C" fp_status fp_shard0_views(const fp_shard0_plan* plan, int32_t rank, fp_view* out, int32_t cap,
                                     int32_t* n_out) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (rank < 0 || rank >= plan->world) return fail(FP_ERR_RANGE, "rank %d outside [0, %d)", rank, plan->world);
    if (n_out) *n_out = plan->n;
    if (cap < plan->n) return fail(FP_ERR_RANGE, "cap %d < %d parameters", cap, plan->n);
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    for (int32_t i = 0; i < plan->n; ++i) {
        fp_view v;
        std::memset(&v, 0, sizeof v);
        v.tensor = i;
        const int64_t real = real_rows(plan, i, rank);
        v.buf_offset = plan->off[i];
        v.numel = real * plan->row_elems[i];
        v.tensor_offset = (int64_t)rank * plan->rows[i] * plan->row_elems[i];
        if (v.numel == 0) v.tensor_offset = 0;
        v.ndim = plan->ndims[i] > 0 ? plan->ndims[i] : 1;
        v.shape[0] = real;
        for (int32_t k = 1; k < plan->ndims[i]; ++k) v.shape[k] = plan->dims[plan->dim_start[i] + k];
        out[i] = v;
    }
    return FP_OK;
}

namespace {
// Null, alignment and overlap checks of the parameters against `other`
// (dst or full); with `disjoint`, also of the parameters among themselves
// (sorted by address: O(n log n)).
fp_status shard0_check_params(const fp_shard0_plan* p, int32_t es, const void* const* params,
                              const void* other, int64_t other_elems, const char* other_name, bool disjoint) {
    std::vector<std::pair<uintptr_t, int32_t>> spans;
    for (int32_t i = 0; i < p->n; ++i) {
        if (p->numel[i] == 0) continue;
        if (params[i] == nullptr) return fail(FP_ERR_INVALID, "params[%d] is NULL", i);
        if (!aligned(params[i], (uintptr_t)es)) return fail(FP_ERR_ALIGN, "params[%d] misaligned", i);
        if (overlap(params[i], p->numel[i] * es, other, other_elems * es))
            return fail(FP_ERR_INVALID, "params[%d] overlaps %s", i, other_name);
        if (disjoint) spans.emplace_back(reinterpret_cast<uintptr_t>(params[i]), i);
    }
    std::sort(spans.begin(), spans.end());
    for (size_t k = 1; k < spans.size(); ++k) {
        const int32_t a = spans[k - 1].second, b = spans[k].second;
        if (overlap(params[a], p->numel[a] * es, params[b], p->numel[b] * es))
            return fail(FP_ERR_INVALID, "params[%d] overlaps params[%d]", b < a ? b : a, b < a ? a : b);
    }
    return FP_OK;
}
}  // namespace

namespace {
fp_status fp_shard0_pack_impl(fp_shard0_plan* plan, int32_t elem_size, int32_t rank,
                                    const void* const* params, void* dst, void* stream) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (elem_size != 2 && elem_size != 4) return fail(FP_ERR_INVALID, "elem_size must be 2 or 4");
    if (rank < -1 || rank >= plan->world) return fail(FP_ERR_RANGE, "rank %d outside [-1, %d)", rank, plan->world);
    if (params == nullptr) return fail(FP_ERR_INVALID, "params table is NULL");
    const int op = rank < 0 ? kOpPackAll : kOpPackRank;
    const int key_rank = rank < 0 ? 0 : rank;
    std::vector<void*> ptrs((size_t)plan->n + 1);
    ptrs[0] = dst;
    for (int32_t i = 0; i < plan->n; ++i) ptrs[1 + i] = const_cast<void*>(params[i]);
    std::lock_guard<std::mutex> lock(plan->cache.mu);
    if (!seg_validated(plan->cache, op, elem_size, key_rank, ptrs)) {
        const int64_t dst_elems = rank < 0 ? plan->shard * plan->world : plan->shard;
        if (dst == nullptr && dst_elems > 0) return fail(FP_ERR_INVALID, "dst is NULL");
        if (!aligned(dst, (uintptr_t)elem_size)) return fail(FP_ERR_ALIGN, "dst misaligned");
        fp_status st = shard0_check_params(plan, elem_size, params, dst, dst_elems, "dst", false);
        if (st != FP_OK) return st;
        seg_remember(plan->cache, op, elem_size, key_rank, ptrs);
    }
    SegTable* t = nullptr;
    fp_status st = shard0_table(plan, op, elem_size, key_rank, &t);
    if (st != FP_OK) return st;
    return seg_run(t, ptrs.data(), static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" fp_status fp_shard0_pack(fp_shard0_plan* plan, int32_t elem_size, int32_t rank,
                                    const void* const* params, void* dst, void* stream) {
    try {
        return fp_shard0_pack_impl(plan, elem_size, rank, params, dst, stream);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

namespace {
fp_status fp_shard0_unpack_impl(fp_shard0_plan* plan, int32_t elem_size, const void* full,
                                      void* const* params, void* stream) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (elem_size != 2 && elem_size != 4) return fail(FP_ERR_INVALID, "elem_size must be 2 or 4");
    if (params == nullptr) return fail(FP_ERR_INVALID, "params table is NULL");
    std::vector<void*> ptrs((size_t)plan->n + 1);
    for (int32_t i = 0; i < plan->n; ++i) ptrs[i] = params[i];
    ptrs[plan->n] = const_cast<void*>(full);
    std::lock_guard<std::mutex> lock(plan->cache.mu);
    if (!seg_validated(plan->cache, kOpUnpack, elem_size, 0, ptrs)) {
        const int64_t full_elems = plan->shard * plan->world;
        if (full == nullptr && full_elems > 0) return fail(FP_ERR_INVALID, "full is NULL");
        if (!aligned(full, (uintptr_t)elem_size)) return fail(FP_ERR_ALIGN, "full misaligned");
        fp_status st = shard0_check_params(plan, elem_size, params, full, full_elems, "full", true);
        if (st != FP_OK) return st;
        seg_remember(plan->cache, kOpUnpack, elem_size, 0, ptrs);
    }
    SegTable* t = nullptr;
    fp_status st = shard0_table(plan, kOpUnpack, elem_size, 0, &t);
    if (st != FP_OK) return st;
    return seg_run(t, ptrs.data(), static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" fp_status fp_shard0_unpack(fp_shard0_plan* plan, int32_t elem_size, const void* full,
                                      void* const* params, void* stream) {
    try {
        return fp_shard0_unpack_impl(plan, elem_size, full, params, stream);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

// ---------------------------------------------------------------------- reshard

struct fp_reshard_plan {
    int64_t numel = 0, s_old = 0, s_new = 0;
    int32_t world_old = 1, world_new = 1;
    SegCache cache;
};

namespace {
// Segments of new rank(s) [q0, q1): pieces of the old shards, zeros past T.
// Pointer table: [dst, old shards...].  Units of 2 bytes.
std::vector<SegDesc> reshard_segments(const fp_reshard_plan* p, int es, int new_rank) {
    const int64_t u = es / 2, T = p->numel, So = p->s_old, Sn = p->s_new;
    const bool all = new_rank < 0;
    const int32_t q0 = all ? 0 : new_rank, q1 = all ? p->world_new : new_rank + 1;
    std::vector<SegDesc> v;
    auto add = [&](int64_t dst_off, int32_t src, int64_t src_off, int64_t len) {
        if (len <= 0) return;
        SegDesc d;
        std::memset(&d, 0, sizeof d);
        d.kind = kSegCopy;
        d.dst = 0;
        d.dst_off = dst_off * u;
        d.src = src;
        d.src_off = src_off * u;
        d.len = len * u;
        v.push_back(d);
    };
    for (int32_t q = q0; q < q1; ++q) {
        const int64_t base = all ? (int64_t)q * Sn : 0, lo = (int64_t)q * Sn, hi_all = lo + Sn;
        const int64_t hi = hi_all < T ? hi_all : T;
        for (int64_t e = lo; e < hi;) {
            const int64_t o = e / So, end = (o + 1) * So < hi ? (o + 1) * So : hi;
            add(base + (e - lo), 1 + (int32_t)o, e - o * So, end - e);
            e = end;
        }
        const int64_t z = lo > T ? lo : T;
        add(base + (z - lo), -1, 0, hi_all - z);
    }
    return v;
}
}  // namespace

extern "C" fp_status fp_reshard_plan_create(int64_t numel, int32_t world_old, int32_t world_new,
                                            fp_reshard_plan** out) {
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (numel < 0 || numel > ((int64_t)1 << 40)) return fail(FP_ERR_RANGE, "numel outside [0, 2^40]");
    if (world_old < 1 || world_old > (1 << 20) || world_new < 1 || world_new > (1 << 20))
        return fail(FP_ERR_RANGE, "world sizes must be in [1, 2^20]");
    fp_reshard_plan* p = new (std::nothrow) fp_reshard_plan();
    if (p == nullptr) return fail(FP_ERR_DEVICE, "out of host memory");
    p->numel = numel;
    p->world_old = world_old;
    p->world_new = world_new;
    p->s_old = (numel + world_old - 1) / world_old;
    p->s_new = (numel + world_new - 1) / world_new;
    *out = p;
    return FP_OK;
}

extern "C" void fp_reshard_plan_destroy(fp_reshard_plan* plan) { delete plan; }

extern "C" fp_status fp_reshard_plan_info(const fp_reshard_plan* plan, int64_t* shard_old, int64_t* shard_new) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (shard_old) *shard_old = plan->s_old;
    if (shard_new) *shard_new = plan->s_new;
    return FP_OK;
}

namespace {
fp_status fp_reshard_impl(fp_reshard_plan* plan, int32_t elem_size, int32_t new_rank,
                                const void* const* old_shards, void* dst, void* stream) {
    if (plan == nullptr) return fail(FP_ERR_INVALID, "plan is NULL");
    if (elem_size != 2 && elem_size != 4) return fail(FP_ERR_INVALID, "elem_size must be 2 or 4");
    if (new_rank < -1 || new_rank >= plan->world_new)
        return fail(FP_ERR_RANGE, "new_rank %d outside [-1, %d)", new_rank, plan->world_new);
    if (old_shards == nullptr) return fail(FP_ERR_INVALID, "old_shards table is NULL");
    const int32_t N = plan->world_old;
    std::vector<void*> ptrs((size_t)N + 1);
    ptrs[0] = dst;
    for (int32_t q = 0; q < N; ++q) ptrs[1 + q] = const_cast<void*>(old_shards[q]);
    const int key = new_rank < 0 ? 0 : new_rank;
    const int op = new_rank < 0 ? kOpReshardAll : kOpReshardRank;
    std::lock_guard<std::mutex> lock(plan->cache.mu);
    if (!seg_validated(plan->cache, op, elem_size, key, ptrs)) {
        const int64_t dst_elems = plan->s_new * (new_rank < 0 ? plan->world_new : 1);
        if (dst == nullptr && dst_elems > 0) return fail(FP_ERR_INVALID, "dst is NULL");
        if (!aligned(dst, (uintptr_t)elem_size)) return fail(FP_ERR_ALIGN, "dst misaligned");
        for (int32_t q = 0; q < N; ++q) {
            if ((int64_t)q * plan->s_old >= plan->numel) continue;   // holds only padding: never read
            if (old_shards[q] == nullptr) return fail(FP_ERR_INVALID, "old_shards[%d] is NULL", q);
            if (!aligned(old_shards[q], (uintptr_t)elem_size)) return fail(FP_ERR_ALIGN, "old_shards[%d] misaligned", q);
            if (overlap(old_shards[q], plan->s_old * elem_size, dst, dst_elems * elem_size))
                return fail(FP_ERR_INVALID, "old_shards[%d] overlaps dst", q);
        }
        seg_remember(plan->cache, op, elem_size, key, ptrs);
    }
    SegTable* t = nullptr;
    fp_status st = seg_table(plan->cache, op, elem_size, key, N + 1,
                             [&] { return reshard_segments(plan, elem_size, new_rank); }, &t);
    if (st != FP_OK) return st;
    return seg_run(t, ptrs.data(), static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" fp_status fp_reshard(fp_reshard_plan* plan, int32_t elem_size, int32_t new_rank,
                                const void* const* old_shards, void* dst, void* stream) {
    try {
        return fp_reshard_impl(plan, elem_size, new_rank, old_shards, dst, stream);
    } catch (const std::bad_alloc&) {
        return fail(FP_ERR_DEVICE, "out of host memory");
    } catch (...) {
        return fail(FP_ERR_DEVICE, "unexpected host error");
    }
}

// ---------------------------------------------------------------------- no_sync, scaler

namespace {
fp_status local_call(int64_t n, const uint16_t* grad, int32_t accumulate, const float* local, uint16_t* out,
                     bool finish, void* stream) {
    if (n < 0) return fail(FP_ERR_RANGE, "n must be >= 0");
    if (n == 0) return FP_OK;
    fp_status st = check_groups(stream_grid(n), "the local accumulation");
    if (st != FP_OK) return st;
    if (grad == nullptr) return fail(FP_ERR_INVALID, "grad is NULL");
    if (!aligned(grad, 2)) return fail(FP_ERR_ALIGN, "grad misaligned");
    if (accumulate || !finish) {
        if ((st = check_f32(local, n, "local")) != FP_OK) return st;
        if (overlap(grad, n * 2, local, n * 4)) return fail(FP_ERR_INVALID, "grad overlaps local");
    }
    bool al = is_aligned8(grad);
    if (finish) {
        if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
        if (!aligned(out, 2)) return fail(FP_ERR_ALIGN, "out misaligned");
        if (overlap(out, n * 2, grad, n * 2)) return fail(FP_ERR_INVALID, "out overlaps grad");
        if (accumulate && overlap(out, n * 2, local, n * 4)) return fail(FP_ERR_INVALID, "out overlaps local");
        al = al && is_aligned8(out);
    }
    LocalArgs a;
    a.grad = grad;
    a.local = const_cast<float*>(local);
    a.out = out;
    a.n = n;
    hipError_t e = launch_local(a, finish, accumulate != 0, al, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "local accumulation launch");
    return FP_OK;
}
}  // namespace

extern "C" fp_status fp_local_accumulate(int64_t n, const uint16_t* grad, int32_t accumulate, float* local,
                                         void* stream) {
    return local_call(n, grad, accumulate, local, nullptr, false, stream);
}

extern "C" fp_status fp_local_finish(int64_t n, const uint16_t* grad, int32_t accumulate, const float* local,
                                     uint16_t* out, void* stream) {
    return local_call(n, grad, accumulate, local, out, true, stream);
}

extern "C" fp_status fp_grad_coef(const double* sq_norm, const float* loss_scale, double max_norm, double* coef,
                                  void* stream) {
    if (coef == nullptr) return fail(FP_ERR_INVALID, "coef is NULL");
    if (!aligned(coef, 8)) return fail(FP_ERR_ALIGN, "coef misaligned");
    if (!(max_norm == max_norm)) return fail(FP_ERR_INVALID, "max_norm is NaN");
    if (max_norm > 0.0) {
        if (sq_norm == nullptr) return fail(FP_ERR_INVALID, "clipping needs sq_norm");
        if (!aligned(sq_norm, 8)) return fail(FP_ERR_ALIGN, "sq_norm misaligned");
    }
    if (loss_scale != nullptr && !aligned(loss_scale, 4)) return fail(FP_ERR_ALIGN, "loss_scale misaligned");
    hipError_t e = launch_grad_coef(max_norm > 0.0 ? sq_norm : nullptr, loss_scale, max_norm, coef,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "grad coef launch");
    return FP_OK;
}

extern "C" fp_status fp_scaler_update(const int32_t* found_inf, float* scale, int32_t* clean_steps,
                                      float growth_factor, float backoff_factor, int32_t growth_interval,
                                      void* stream) {
    if (found_inf == nullptr || scale == nullptr || clean_steps == nullptr)
        return fail(FP_ERR_INVALID, "found_inf, scale and clean_steps are required");
    if (!aligned(found_inf, 4) || !aligned(scale, 4) || !aligned(clean_steps, 4))
        return fail(FP_ERR_ALIGN, "scaler values misaligned");
    if (growth_interval < 1) return fail(FP_ERR_RANGE, "growth_interval must be >= 1");
    if (!(growth_factor > 0.0f) || !(backoff_factor > 0.0f)) return fail(FP_ERR_RANGE, "factors must be > 0");
    hipError_t e = launch_scaler_update(found_inf, scale, clean_steps, growth_factor, backoff_factor,
                                        growth_interval, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(e, "scaler update launch");
    return FP_OK;
}

// ---------------------------------------------------------------------- helpers

extern "C" fp_status fp_state_bytes(double psi, int32_t world, double k, int32_t stage, double* out) {
    if (out == nullptr) return fail(FP_ERR_INVALID, "out is NULL");
    if (!(psi >= 0.0) || !(k >= 0.0) || world < 1) return fail(FP_ERR_INVALID, "psi, k >= 0 and world >= 1");
    const double n = world;
    switch (stage) {
        case 0: *out = (2.0 + 2.0 + k) * psi; break;
        case 1: *out = 4.0 * psi + k * psi / n; break;
        case 2: *out = 2.0 * psi + (2.0 + k) * psi / n; break;
        case 3: *out = (4.0 + k) * psi / n; break;
        default: return fail(FP_ERR_INVALID, "stage %d outside [0, 3]", stage);
    }
    return FP_OK;
}

extern "C" const char* fp_status_string(fp_status status) {
    switch (status) {
        case FP_OK: return "ok";
        case FP_ERR_INVALID: return "invalid argument";
        case FP_ERR_RANGE: return "argument out of range";
        case FP_ERR_ALIGN: return "misaligned pointer";
        case FP_ERR_DEVICE: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* fp_last_error(void) { return g_error; }
