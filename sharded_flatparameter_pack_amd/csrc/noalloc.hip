// noalloc.hip -- fp_shard_step_noalloc: the shard step for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  The step's scratch --
// the one-pass kernel's grid-barrier state and the per-workgroup partials of
// the gradient norm, which fp_shard_step takes from a caller-provided
// workspace -- lives in a file-scope device array of kScratchBytes instead.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Its device address is taken once per device with
// hipGetSymbolAddress (in host code the array's name is only a stand-in,
// never a device address) and the barrier state is cleared by a small fill
// kernel on the first call on a device.  Every call on a GPU shares that
// GPU's array: calls that overlap on one GPU race.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "fp_internal.h"

namespace fpk {
namespace {

constexpr int64_t kScratchBytes = (int64_t)2 << 20;  // barrier header + norm partials of 2^18 workgroups
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zeroes the barrier state at the start of the array (16-byte vector stores).
__global__ __launch_bounds__(kThreads) void scratch_clear_kernel(uint4* p, int n_words) {
    for (int i = threadIdx.x; i < n_words; i += kThreads) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct DeviceScratch {
    void* ptr = nullptr;   // the array's address on that device
    bool cleared = false;  // the clear has run outside graph capture
};
std::mutex g_mutex;
DeviceScratch g_scratch[kMaxScratchDevices];

fp_status scratch_address(int* device, void** out) {
    hipError_t e = hipGetDevice(device);
    if (e != hipSuccess) return report_error(FP_ERR_DEVICE, hipGetErrorString(e));
    if (*device < 0 || *device >= kMaxScratchDevices)
        return report_error(FP_ERR_DEVICE, "device index beyond the library's scratch table");
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceScratch& d = g_scratch[*device];
    if (d.ptr == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            char msg[160];
            snprintf(msg, sizeof msg, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
            return report_error(FP_ERR_DEVICE, msg);
        }
        d.ptr = p;
    }
    *out = d.ptr;
    return FP_OK;
}

// Enqueue the clear of the barrier state on `s` until one has run outside
// graph capture (a clear captured into a graph runs again at every replay,
// which leaves the state as valid as a completed call does).
fp_status clear_once(int device, void* ptr, hipStream_t s) {
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceScratch& d = g_scratch[device];
    if (d.cleared) return FP_OK;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &capture);
    if (e != hipSuccess) return report_error(FP_ERR_DEVICE, hipGetErrorString(e));
    scratch_clear_kernel<<<1, kThreads, 0, s>>>(static_cast<uint4*>(ptr), (int)(kWorkspaceHeader / 16));
    if ((e = hipGetLastError()) != hipSuccess) return report_error(FP_ERR_DEVICE, hipGetErrorString(e));
    if (capture == hipStreamCaptureStatusNone) d.cleared = true;
    return FP_OK;
}

}  // namespace
}  // namespace fpk

using namespace fpk;

extern "C" fp_status fp_shard_step_noalloc(const fp_step_args* args, void* stream) {
    if (args == nullptr) return report_error(FP_ERR_INVALID, "args is NULL");
    if (args->workspace != nullptr)
        return report_error(FP_ERR_INVALID, "workspace must be NULL: this entry point uses the library's scratch");
    if (args->sq_norm != nullptr && args->shard > 0 && fp_workspace_bytes(args->shard) > kScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof msg,
                 "the norm of a shard of %lld elements needs %lld bytes of scratch; the library holds %lld "
                 "(shards up to %lld elements with sq_norm)",
                 (long long)args->shard, (long long)fp_workspace_bytes(args->shard), (long long)kScratchBytes,
                 (long long)(((kScratchBytes - kWorkspaceHeader) / 8 - 1) * kTileQuads * 4 + 3));
        return report_error(FP_ERR_RANGE, msg);
    }
    int device = -1;
    void* ptr = nullptr;
    fp_status st = scratch_address(&device, &ptr);
    if (st != FP_OK) return st;
    fp_step_args a = *args;
    a.workspace = ptr;
    int32_t path = 0;
    if ((st = fp_step_path(&a, &path)) != FP_OK) return st;  // every argument check, nothing enqueued
    if ((st = clear_once(device, ptr, static_cast<hipStream_t>(stream))) != FP_OK) return st;
    return shard_step_run(&a, stream, false);
}
