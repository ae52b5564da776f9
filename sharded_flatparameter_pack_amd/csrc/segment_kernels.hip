// segment_kernels.hip -- many contiguous copies (and zero fills) in one
// launch, for the per-parameter dim-0 layout: a rank's chunk of every
// parameter into the group buffer (with zero padding rows), and after the
// gather, every rank's chunk back into each parameter ("Infra: Data
// Parallel", FSDP2 section and figure: each parameter is cut along dim 0,
// keeps its global shape, and the group's parameters travel together).
//
// A workgroup reads its segment from the per-workgroup table, then moves
// whole 16-byte words of the destination range with the same realigning
// copy as the unshard (one load per word, the following word from the next
// lane); the segment's first workgroup also moves the edge elements that
// share a word with a neighbouring segment.  Units are 2 bytes, so fp32 and
// bf16 buffers use the same kernel.

#include "step_ops.h"

namespace fpk {

__global__ __launch_bounds__(kThreads) void segment_kernel(const SegArgs a) {
    const int s = a.seg_of[blockIdx.x];
    const SegDesc& d = a.segs[s];
    const int64_t tile = (int64_t)blockIdx.x - d.tile0;
    uint16_t* dst = static_cast<uint16_t*>(a.dst_tab[d.dst]);
    const ShardSpan sp = elem_span(dst, d.dst_off, d.len);
    if (d.src < 0) {
        const int64_t n_words = (sp.b - sp.a) >> 3;
#pragma unroll
        for (int u = 0; u < kSegWords; ++u) {
            const int64_t w = (tile * kSegWords + u) * kThreads + threadIdx.x;
            if (w < n_words) st16(dst + sp.a + (w << 3), make_uint4(0u, 0u, 0u, 0u));
        }
        if (tile == 0) span_edges(nullptr, dst, sp, threadIdx.x, kThreads);
        return;
    }
    const uint16_t* src = static_cast<const uint16_t*>(a.src_tab[d.src]) + d.src_off;
    const bool aligned = ((reinterpret_cast<uintptr_t>(src + (sp.a - sp.lo))) & 15u) == 0;
    if (aligned) copy_tile<true, kSegWords>(src, dst, sp, tile);
    else copy_tile<false, kSegWords>(src, dst, sp, tile);
    if (tile == 0) span_edges(src, dst, sp, threadIdx.x, kThreads);
}

hipError_t launch_segments(const SegArgs& a, int64_t n_groups, hipStream_t s) {
    segment_kernel<<<(unsigned)n_groups, kThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fpk
