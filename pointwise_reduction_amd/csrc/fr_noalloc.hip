// fr_noalloc.hip - fr_sumsq_full_noalloc: the split sum of squares with its
// chunk partials in a device array the library owns, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation). The kernels are those of fr_sumsq_full;
// only where the partials live differs.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy until the process ends. In host code its name is a
// host-side stand-in, not a device address, so it is never passed to a
// kernel or a copy: the address comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call there and kept.
// Calls on one GPU share the array: two calls that overlap in time on that
// GPU (different streams, no ordering between them) race on it. Nothing in
// it needs clearing between calls: every chunk partial is written before the
// finishing kernel reads it, in stream order.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fr.h"
#include "fr_internal.h"

namespace {

constexpr size_t kScratchBytes = FR_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch`.
int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FR_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return FR_E_DEVICE;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return FR_OK;
}

}  // namespace

extern "C" int fr_sumsq_full_noalloc(const void* x, int64_t n, void* out, int dtype, void* stream) {
    // the argument checks of fr_sumsq_full, before any HIP call
    if (n < 0 || n >= (int64_t(1) << 30)) return FR_E_SIZE;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (!out || (n > 0 && !x)) return FR_E_NULL;
    if ((uintptr_t)x % 4 || (uintptr_t)out % 4) return FR_E_ALIGN;
    if (fr_sumsq_full_workspace_bytes(n, dtype) > kScratchBytes) return FR_E_WORKSPACE;
    void* ws = nullptr;
    const int st = scratch_for_current_device(&ws);
    if (st != FR_OK) return st;
    // a plan (or tuning override) needing more than the array is refused
    // with FR_E_WORKSPACE inside fr_sumsq_full
    return fr_sumsq_full(x, n, out, ws, kScratchBytes, dtype, stream);
}
