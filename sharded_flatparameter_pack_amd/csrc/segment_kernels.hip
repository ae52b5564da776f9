// segment_kernels.hip -- many copies (and zero fills) in one launch, for the
// per-parameter dim-0 layout: every rank's chunk of every parameter into the
// rank-major group buffer (with zero padding rows), and after the gather,
// every rank's chunk back into each parameter ("Infra: Data Parallel",
// FSDP2 sections and the FSDP1 / FSDP2 comparison figure: each parameter is
// cut along dim 0, keeps its global shape, and the group's parameters
// travel together).
//
// A workgroup reads its entry from the per-workgroup table.  A copy entry
// moves whole 16-byte words of its destination range with the same
// realigning copy as the unshard (one load per word, the following word from
// the next lane); the entry's first workgroup also moves the edge elements
// that share a word with a neighbouring entry.  A strided entry gathers the
// small pieces of one parameter, one 2-byte unit per lane: one workgroup
// then writes what would otherwise be many workgroups' partial cache lines.
// Units are 2 bytes, so fp32 and bf16 buffers use the same kernel.

#include "fp_extra.h"
#include "step_ops.h"

namespace fpk {

// A strided tile: lane t takes units e0 + j * 256 + t, j < 16.  All loads
// of a lane are issued before its first store, unconditionally (a unit past
// `valid` loads the entry's first source unit and stores 0), and the stores
// of a full tile are unconditional too: with branches around them every
// store would wait for all earlier memory operations of the lane.
__device__ __forceinline__ void strided_tile(const SegDesc& d, const uint16_t* src, uint16_t* dst,
                                             int64_t tile) {
    constexpr int kPer = (int)(kSegStridedTile / kThreads);
    const uint32_t e0 = (uint32_t)(tile * kSegStridedTile) + threadIdx.x;
    const uint32_t len = (uint32_t)d.len, piece = (uint32_t)d.piece, valid = (uint32_t)d.valid;
    uint16_t v[kPer];
    if (valid > 0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t e = e0 + (uint32_t)j * kThreads;
            const uint32_t q = e / piece;
            const bool ok = e < valid;
            const int64_t at = ok ? (int64_t)q * d.src_stride + (e - q * piece) : 0;
            v[j] = src[d.src_off + at];
            if (!ok) v[j] = 0;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) v[j] = 0;
    }
    const bool full = (int64_t)(tile + 1) * kSegStridedTile <= d.len;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint32_t e = e0 + (uint32_t)j * kThreads;
        const uint32_t q = e / piece;
        if (full || e < len) dst[d.dst_off + (int64_t)q * d.dst_stride + (e - q * piece)] = v[j];
    }
}

__global__ __launch_bounds__(kThreads) void segment_kernel(const SegArgs a) {
    const int s = a.seg_of[blockIdx.x];
    const SegDesc d = a.segs[s];      // a copy: the stores below cannot alias it
    const int64_t tile = (int64_t)blockIdx.x - d.tile0;
    uint16_t* dst = static_cast<uint16_t*>(a.dst_tab[d.dst]);
    if (d.kind == kSegStrided) {
        const uint16_t* src = d.valid > 0 ? static_cast<const uint16_t*>(a.src_tab[d.src]) : nullptr;
        strided_tile(d, src, dst, tile);
        return;
    }
    const ShardSpan sp = elem_span(dst, d.dst_off, d.len);
    if (d.src < 0) {
        const int64_t n_words = (sp.b - sp.a) >> 3;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u >= d.words) break;
            const int64_t w = (tile * d.words + u) * kThreads + threadIdx.x;
            if (w < n_words) st16(dst + sp.a + (w << 3), make_uint4(0u, 0u, 0u, 0u));
        }
        if (tile == 0) span_edges(nullptr, dst, sp, threadIdx.x, kThreads);
        return;
    }
    const uint16_t* src = static_cast<const uint16_t*>(a.src_tab[d.src]) + d.src_off;
    const bool aligned = ((reinterpret_cast<uintptr_t>(src + (sp.a - sp.lo))) & 15u) == 0;
    if (d.words == 2) {
        if (aligned) copy_tile<true, 2>(src, dst, sp, tile);
        else copy_tile<false, 2>(src, dst, sp, tile);
    } else {
        if (aligned) copy_tile<true, 1>(src, dst, sp, tile);
        else copy_tile<false, 1>(src, dst, sp, tile);
    }
    if (tile == 0) span_edges(src, dst, sp, threadIdx.x, kThreads);
}

hipError_t launch_segments(const SegArgs& a, int64_t n_groups, hipStream_t s) {
    segment_kernel<<<(unsigned)n_groups, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
