// fr_stream.hip - streaming reference kernels: the practical ceiling of an
// HBM-bound step, measured with the same harness as the reduction kernels
// ("Stax (4): GPU Codegen and Dynamic Shapes", 9.1: a memory-bound kernel is
// judged by the bandwidth it reaches, and Little's law sets the bytes that
// must be in flight). Both move contiguous 16-byte vectors with the hints the
// reduction kernels use (non-temporal loads and stores), grid-stride over a
// fixed grid.
//   fr_stream_copy_k  y = x
//   fr_stream_read_k  per-workgroup XOR of every 32-bit word read, so that
//                     the loads are observable and the result checkable
//   fr_stream_write_k y = a repeated 32-bit word (stores only)
//   fr_empty_k        one workgroup that does nothing: launched back to back,
//                     the cost of a kernel boundary alone, the floor under
//                     every step that is one launch
#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

template <int T, int NV>
__global__ __launch_bounds__(T) void fr_stream_copy_k(const f32x4* __restrict__ x, f32x4* __restrict__ y,
                                                      int64_t nvec) {
    const int64_t step = (int64_t)gridDim.x * T * NV;
    for (int64_t b = (int64_t)blockIdx.x * T * NV + threadIdx.x; b < nvec; b += step) {
        f32x4 v[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k)
            v[k] = b + k * T < nvec ? __builtin_nontemporal_load(x + b + k * T) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NV; ++k)
            if (b + k * T < nvec) __builtin_nontemporal_store(v[k], y + b + k * T);
    }
}

template <int T, int NV>
__global__ __launch_bounds__(T) void fr_stream_read_k(const u32x4* __restrict__ x, int64_t nvec,
                                                      uint32_t* __restrict__ sink) {
    __shared__ int sl[T / kWave];
    const int64_t step = (int64_t)gridDim.x * T * NV;
    uint32_t acc = 0u;
    for (int64_t b = (int64_t)blockIdx.x * T * NV + threadIdx.x; b < nvec; b += step) {
        u32x4 v[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k)
            v[k] = b + k * T < nvec ? __builtin_nontemporal_load(x + b + k * T) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < NV; ++k) acc ^= (v[k].x ^ v[k].y) ^ (v[k].z ^ v[k].w);
    }
    struct OpXor {
        __device__ int operator()(int a, int b) const { return a ^ b; }
    };
    int r = group_reduce<kWave>((int)acc, OpXor());
    r = block_fold(r, sl, T / kWave, OpXor());
    if (threadIdx.x == 0) sink[blockIdx.x] = (uint32_t)r;
}

template <int T, int NV>
__global__ __launch_bounds__(T) void fr_stream_write_k(u32x4* __restrict__ y, int64_t nvec, uint32_t value) {
    const int64_t step = (int64_t)gridDim.x * T * NV;
    const u32x4 v = {value, value, value, value};
    for (int64_t b = (int64_t)blockIdx.x * T * NV + threadIdx.x; b < nvec; b += step) {
#pragma unroll
        for (int k = 0; k < NV; ++k)
            if (b + k * T < nvec) __builtin_nontemporal_store(v, y + b + k * T);
    }
}

__global__ __launch_bounds__(64) void fr_empty_k() {}

// One lane stores the device's constant wall clock (the counter the wait
// loops of the split kernels read) into out[slot] when the kernel runs: two
// of these around a sequence of launches on one stream time exactly that
// sequence on the device.
__global__ __launch_bounds__(64) void fr_clock_k(uint64_t* __restrict__ out, int slot) {
    if (threadIdx.x == 0) out[slot] = wall_clock64();
}

// Dependent loads: one lane follows a chain of indices, next = chain[i],
// for `steps` loads, each waiting for the one before; out[0] = wall-clock
// ticks taken, out[1] = the index reached (so the walk is observable and
// checkable). Indices are clamped to [0, n) before use, so every load stays
// inside the buffer whatever it holds. Non-temporal loads: the walk's lines
// are not kept for a later visit.
__global__ __launch_bounds__(64) void fr_chase_k(const uint32_t* __restrict__ chain, int64_t n, int64_t steps,
                                                 uint32_t start, uint64_t* __restrict__ out) {
    if (threadIdx.x != 0) return;
    uint32_t i = start < n ? start : 0u;
    const uint64_t t0 = wall_clock64();
    for (int64_t k = 0; k < steps; ++k) {
        const uint32_t nx = __builtin_nontemporal_load(chain + i);
        i = nx < (uint64_t)n ? nx : 0u;
    }
    const uint64_t t1 = wall_clock64();
    out[0] = t1 - t0;
    out[1] = i;
}

hipError_t launch_pointer_chase(const uint32_t* chain, int64_t n, int64_t steps, uint32_t start, uint64_t* out,
                                hipStream_t s) {
    hipLaunchKernelGGL(fr_chase_k, dim3(1), dim3(64), 0, s, chain, n, steps, start, out);
    return hipGetLastError();
}

hipError_t launch_device_clock(uint64_t* out, int slot, hipStream_t s) {
    hipLaunchKernelGGL(fr_clock_k, dim3(1), dim3(64), 0, s, out, slot);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void* x, void* y, int64_t nvec, hipStream_t s) {
    const int64_t grid = std::min<int64_t>(kStreamGrid, (nvec + 1023) / 1024);
    hipLaunchKernelGGL((fr_stream_copy_k<256, 4>), dim3((unsigned)grid), dim3(256), 0, s,
                       static_cast<const f32x4*>(x), static_cast<f32x4*>(y), nvec);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* x, int64_t nvec, uint32_t* sink, hipStream_t s) {
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(kStreamGrid, (nvec + 1023) / 1024));
    hipLaunchKernelGGL((fr_stream_read_k<256, 4>), dim3((unsigned)grid), dim3(256), 0, s,
                       static_cast<const u32x4*>(x), nvec, sink);
    return hipGetLastError();
}

hipError_t launch_stream_write(void* y, int64_t nvec, uint32_t value, hipStream_t s) {
    const int64_t grid = std::min<int64_t>(kStreamGrid, (nvec + 1023) / 1024);
    hipLaunchKernelGGL((fr_stream_write_k<256, 4>), dim3((unsigned)grid), dim3(256), 0, s, static_cast<u32x4*>(y),
                       nvec, value);
    return hipGetLastError();
}

hipError_t launch_empty(hipStream_t s) {
    hipLaunchKernelGGL(fr_empty_k, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

}  // namespace fr
