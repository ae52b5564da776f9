// pack_kernels.hip -- FlatParameter construction on gfx950.
//
// "Infra: Data Parallel", section "FSDP1: pack first, then split" and its
// figure: a unit's tensors are flattened row-major and concatenated into one
// 1-D buffer, zero-padded here to a multiple of the world size.
//
// The kernel is tiled over the destination: workgroup b owns flat elements
// [b*8192, (b+1)*8192) and every lane writes whole aligned 16-byte words of
// it.  The host precomputes, per workgroup, the first tensor that overlaps
// its range; the workgroup stages the offsets and source pointers of the
// tensors it overlaps in LDS, and each lane finds the tensor of its word by
// binary search there.  A word inside one tensor is one or two aligned
// 16-byte loads and a byte funnel shift; a word that straddles tensors or the
// padding is assembled element by element.  The copy moves bits only (NaN
// payloads and -0 survive).

#include "fp_device.h"

namespace fpk {

template <int ES>
__global__ __launch_bounds__(kThreads) void pack_kernel(const PackArgs a) {
    constexpr int kEpw = 16 / ES;                       // elements per 16-byte word
    constexpr int kWords = kPackBlockElems / kEpw;      // words per workgroup
    __shared__ int64_t s_off[kPackLdsTensors + 1];
    __shared__ const void* s_src[kPackLdsTensors];

    const int64_t g0 = (int64_t)blockIdx.x * kPackBlockElems;
    const int t_first = a.group_first[blockIdx.x];
    int t_last = a.group_first[blockIdx.x + 1];
    if (t_last > a.n_tensors - 1) t_last = a.n_tensors - 1;
    const int count = t_first < a.n_tensors ? t_last - t_first + 1 : 0;
    const bool staged = count <= kPackLdsTensors;
    if (staged) {
        for (int k = threadIdx.x; k <= count; k += kThreads) s_off[k] = a.offsets[t_first + k];
        for (int k = threadIdx.x; k < count; k += kThreads) s_src[k] = a.src[t_first + k];
    }
    __syncthreads();

    auto off = [&](int k) -> int64_t { return staged ? s_off[k] : a.offsets[t_first + k]; };
    auto src = [&](int k) -> const unsigned char* {
        return static_cast<const unsigned char*>(staged ? s_src[k] : a.src[t_first + k]);
    };
    // local index k of the tensor holding element e (t_first's offset <= e < T)
    auto find = [&](int64_t e) -> int {
        int lo = 0, hi = count - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off(mid) <= e) lo = mid; else hi = mid - 1;
        }
        return lo;
    };

    unsigned char* flat = static_cast<unsigned char*>(a.flat);
    // kBatch words per lane at a time: every lane computes the source words
    // of its kBatch destination words, then all their loads are issued before
    // the first store.  A word inside one tensor (the common case) is one
    // aligned load, realigned with a byte funnel shift when the source is not
    // 16-byte aligned; its address is chosen arithmetically so that the loads
    // of every lane are unconditional (lanes without such a word load their
    // own destination word and discard it).  Words that straddle tensors or
    // the padding are assembled element by element afterwards.
    constexpr int kBatch = 4;
    for (int wb = threadIdx.x; wb < kWords; wb += kThreads * kBatch) {
        uint4 lo[kBatch], hi[kBatch];
        uint32_t mis[kBatch];
        int kind[kBatch];        // 0: none, 1: inside one tensor, 2: assembled
        int kt[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int w = wb + b * kThreads;
            const int64_t e0 = g0 + (int64_t)w * kEpw;
            const unsigned char* dst = flat + e0 * ES;
            const unsigned char* addr = dst;
            kind[b] = 0;
            kt[b] = -1;
            if (w < kWords && e0 < a.padded) {
                kind[b] = 2;
                if (e0 < a.total) {
                    const int k = find(e0);
                    kt[b] = k;
                    if (e0 + kEpw <= off(k + 1)) {
                        kind[b] = 1;
                        addr = src(k) + (e0 - off(k)) * ES;
                    }
                }
            }
            if (kind[b] != 1) addr = (w < kWords && e0 < a.padded) ? dst : flat;
            mis[b] = kind[b] == 1 ? (uint32_t)(reinterpret_cast<uintptr_t>(addr) & 15u) : 0u;
            lo[b] = ld16(addr - mis[b]);
            hi[b] = make_uint4(0u, 0u, 0u, 0u);
        }
        // A misaligned word needs the next aligned source word too.  The
        // lanes of a wave hold consecutive destination words, so when the next
        // lane's word lies in the same tensor its load is that word: it comes
        // over by a wave-shift DPP move.  Only the other lanes (the wave's
        // last lane, tensor ends) load it themselves.
        const uint32_t lane = threadIdx.x & 63u;
        bool own[kBatch];
        bool any_own = false;
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int next_kind = (int)from_next_lane((uint32_t)kind[b], 0u);
            const int next_kt = (int)from_next_lane((uint32_t)kt[b], 0xFFFFFFFFu);
            const bool shared = lane < 63u && kind[b] == 1 && next_kind == 1 && next_kt == kt[b];
            own[b] = mis[b] != 0 && !shared;
            any_own |= own[b];
        }
        if (__any(any_own)) {
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (own[b]) {
                    const int w = wb + b * kThreads;
                    const int64_t e0 = g0 + (int64_t)w * kEpw;
                    hi[b] = ld16(src(kt[b]) + (e0 - off(kt[b])) * ES - mis[b] + 16);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const uint4 next = from_next_lane(lo[b], lo[b]);
            if (!own[b]) hi[b] = next;
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (kind[b] == 0) continue;
            const int w = wb + b * kThreads;
            const int64_t e0 = g0 + (int64_t)w * kEpw;
            const int64_t e1 = e0 + kEpw;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (kind[b] == 1) {
                Src16 sh;
                sh.abase = nullptr;
                sh.ds = mis[b] >> 2;
                sh.bs = mis[b] & 3u;
                sh.step = 0;
                v = realign16(sh, lo[b], hi[b]);
            } else if (kt[b] >= 0) {
                int k = kt[b];
                uint32_t d[4] = {0u, 0u, 0u, 0u};
                for (int i = 0; i < kEpw; ++i) {
                    const int64_t e = e0 + i;
                    if (e >= a.total) break;
                    while (e >= off(k + 1)) ++k;     // skips empty tensors too
                    const unsigned char* p = src(k) + (e - off(k)) * ES;
                    if (ES == 4) d[i] = *reinterpret_cast<const uint32_t*>(p);
                    else d[i >> 1] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << ((i & 1) * 16);
                }
                v = make_uint4(d[0], d[1], d[2], d[3]);
            }
            if (e1 <= a.padded) {
                st16(flat + e0 * ES, v);
            } else {                                  // last, partial word of the buffer
                const uint32_t d[4] = {v.x, v.y, v.z, v.w};
                for (int i = 0; e0 + i < a.padded; ++i) {
                    if (ES == 4) reinterpret_cast<uint32_t*>(flat)[e0 + i] = d[i];
                    else reinterpret_cast<uint16_t*>(flat)[e0 + i] = (uint16_t)(d[i >> 1] >> ((i & 1) * 16));
                }
            }
        }
    }
}

hipError_t launch_pack(const PackArgs& a, int elem_size, int64_t n_groups, hipStream_t s) {
    if (elem_size == 4) pack_kernel<4><<<(unsigned)n_groups, kThreads, 0, s>>>(a);
    else pack_kernel<2><<<(unsigned)n_groups, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
