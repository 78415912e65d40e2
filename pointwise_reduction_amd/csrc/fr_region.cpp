// fr_region.cpp - recorded regions: the launches of one region recorded once
// as a HIP graph and replayed with a single call ("Stax (4): GPU Codegen and
// Dynamic Shapes", 9.9).
//
// A region of n short kernels launched one by one costs about
// max(n * t_launch, sum t_k); replayed as a graph it costs about
// t_graph + sum t_k. Recording fixes the sequence of kernels, their grids
// and their arguments, device pointers included, so a replay is only valid
// when the call has the shapes and addresses it had at recording time (9.9,
// condition 2). The caller states those in a key; every call compares it.
// State machine, as 9.9 describes it:
//   empty     -> record (stream capture of the callback's launches), then
//                replay; a failed capture or instantiation -> fallback
//   recorded  -> key and device equal: replay; otherwise run the callback
//                directly (the recording is kept)
//   fallback  -> always run the callback directly
// Host code only; the region object lives in host memory.
#include <hip/hip_runtime.h>
#include <string.h>

#include <new>
#include <vector>

#include "fr.h"

struct fr_region {
    int state = FR_REGION_EMPTY;
    int device = -1;
    std::vector<unsigned char> key;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    uint64_t replays = 0;
    uint64_t direct = 0;
};

namespace {

void release(fr_region* r) {
    if (r->exec) (void)hipGraphExecDestroy(r->exec);
    if (r->graph) (void)hipGraphDestroy(r->graph);
    r->exec = nullptr;
    r->graph = nullptr;
}

int run_direct(fr_region* r, fr_region_fn fn, void* ctx, void* stream) {
    ++r->direct;
    return fn(ctx, stream);
}

int to_fallback(fr_region* r, fr_region_fn fn, void* ctx, void* stream) {
    (void)hipGetLastError();  // the failed capture's error is not the caller's
    release(r);
    r->state = FR_REGION_FALLBACK;
    return run_direct(r, fn, ctx, stream);
}

bool same_key(const fr_region* r, const void* key, uint64_t key_bytes) {
    return r->key.size() == key_bytes && (key_bytes == 0 || memcmp(r->key.data(), key, key_bytes) == 0);
}

}  // namespace

extern "C" {

int fr_region_create(fr_region** out) {
    if (!out) return FR_E_NULL;
    *out = new (std::nothrow) fr_region();
    return *out ? FR_OK : FR_E_ARG;
}

void fr_region_destroy(fr_region* r) {
    if (!r) return;
    release(r);
    delete r;
}

int fr_region_state(const fr_region* r) { return r ? r->state : FR_E_NULL; }

int fr_region_counts(const fr_region* r, uint64_t* replays, uint64_t* direct) {
    if (!r) return FR_E_NULL;
    if (replays) *replays = r->replays;
    if (direct) *direct = r->direct;
    return FR_OK;
}

int fr_region_run(fr_region* r, const void* key, uint64_t key_bytes, fr_region_fn fn, void* ctx, void* stream) {
    if (!r || !fn || (key_bytes > 0 && !key)) return FR_E_NULL;
    if (r->state == FR_REGION_FALLBACK) return run_direct(r, fn, ctx, stream);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return FR_E_DEVICE;
    }
    const hipStream_t s = (hipStream_t)stream;
    if (r->state == FR_REGION_RECORDED) {
        if (dev != r->device || !same_key(r, key, key_bytes)) return run_direct(r, fn, ctx, stream);
        if (hipGraphLaunch(r->exec, s) != hipSuccess) return to_fallback(r, fn, ctx, stream);
        ++r->replays;
        return FR_OK;
    }
    // empty: record. The legacy default stream cannot be captured.
    if (!stream) return to_fallback(r, fn, ctx, stream);
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return to_fallback(r, fn, ctx, stream);
    const int st = fn(ctx, stream);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (st != FR_OK || e != hipSuccess || !g) {
        // nothing was executed while capturing: run the region directly now
        if (g) (void)hipGraphDestroy(g);
        return to_fallback(r, fn, ctx, stream);
    }
    hipGraphExec_t x = nullptr;
    if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(g);
        return to_fallback(r, fn, ctx, stream);
    }
    r->graph = g;
    r->exec = x;
    r->device = dev;
    r->key.assign((const unsigned char*)key, (const unsigned char*)key + key_bytes);
    r->state = FR_REGION_RECORDED;
    if (hipGraphLaunch(x, s) != hipSuccess) return to_fallback(r, fn, ctx, stream);
    ++r->replays;
    return FR_OK;
}

}  // extern "C"
