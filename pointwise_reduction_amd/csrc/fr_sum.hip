// fr_sum.hip - row sums with a fused pointwise prologue, in the three
// reduction forms of "Stax (4): GPU Codegen and Dynamic Shapes", 9.4:
//   persistent  fr_per_sum_f32    a lane group holds a whole row in registers
//   looped      fr_red_sum_f32    one workgroup streams a row in chunks
//   split       fr_split_sum_f32  chunks of few, long rows reduced by separate
//                                 workgroups into a workspace; the persistent
//                                 kernel then folds each row's partials
//                                 (Listing 9.4: a looped kernel writing partial
//                                 sums, a persistent kernel finishing them).
// Prologues: 2 * relu(a + b) (Listing 9.1, Example 1.1) and x * x (Listing
// 9.4, Example 6.2). Masked lanes contribute the identity 0 (9.2, part (4)).
#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

// kIdent sums the input as is (the finishing pass over partial sums).
constexpr int kIdent = 2;

// relu with NaN propagation: maximum(t, 0) per IEEE 754-2019 keeps a NaN and
// maps -0 to +0. The factor 2 of Example 1.1 is applied once to the row sum:
// scaling by 2 is exact in binary floating point, so 2 * sum(r) has the same
// bits as sum(2 * r) for every summation order (barring overflow).
template <int P>
__device__ __forceinline__ float prologue(float a, float b) {
    if constexpr (P == kReluAdd) return fmax_nan(a + b, 0.f);
    else if constexpr (P == kSquare) return a * a;
    else return a;
}

template <int P>
__device__ __forceinline__ float fold4(float s, f32x4 a, f32x4 b) {
    s += prologue<P>(a.x, b.x);
    s += prologue<P>(a.y, b.y);
    s += prologue<P>(a.z, b.z);
    s += prologue<P>(a.w, b.w);
    return s;
}

template <int P>
__device__ __forceinline__ f32x4 map4(f32x4 a, f32x4 b) {
    return f32x4{prologue<P>(a.x, b.x), prologue<P>(a.y, b.y), prologue<P>(a.z, b.z), prologue<P>(a.w, b.w)};
}

// ------------------------------------------------------------------ persistent
// SEG lanes per row, NV 16-byte vectors per lane: row capacity 4 * SEG * NV.
// A 256-thread workgroup serves 256 / SEG rows per step of a grid-stride
// loop over row groups. Lane l of a group owns elements (k * SEG + l) * 4 + c,
// so each load instruction of a group covers 64 * SEG contiguous bytes. M is
// the masking mode (kNone: dense rows that fill the capacity exactly).
template <int P, int SEG, int NV, int M>
__global__ __launch_bounds__(256) void fr_per_sum_f32(const float* __restrict__ a, const float* __restrict__ b,
                                                      float* __restrict__ out, int rows, int cols, int64_t a_rs,
                                                      int64_t b_rs, int64_t out_s, float post) {
    constexpr int RPB = 256 / SEG;
    const int g = threadIdx.x / SEG;
    const int l = threadIdx.x % SEG;
    const int ngroups = (rows + RPB - 1) / RPB;
    for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        const int r = grp * RPB + g;
        const bool live = r < rows;
        const int L = live ? cols : 0;
        // kNone: a row past the end re-reads the last row (in bounds) and
        // stores nothing, so the loads carry no branch
        const int rl = live ? r : (M == kNone ? rows - 1 : 0);
        const float* ar = a + (int64_t)rl * a_rs;
        const float* br = P == kReluAdd ? b + (int64_t)rl * b_rs : nullptr;
        f32x4 va[NV], vb[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int j0 = (k * SEG + l) * 4;
            if constexpr (M == kNone) {
                va[k] = ld4<true>(ar + j0);
                if constexpr (P == kReluAdd) vb[k] = ld4<true>(br + j0);
                else vb[k] = va[k];
            } else {
                va[k] = load4m<M, true>(ar, j0, L, 0.f);
                if constexpr (P == kReluAdd) vb[k] = load4m<M, true>(br, j0, L, 0.f);
                else vb[k] = va[k];
            }
        }
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) s = fold4<P>(s, va[k], vb[k]);
        s = group_reduce<SEG>(s, OpSum());
        if (live && l == 0) out[(int64_t)r * out_s] = s * post;
    }
}

// ------------------------------------------------------------------ looped
// One workgroup of T threads per row (grid-stride over rows). Each step loads
// U independent 16-byte vectors per lane (U * T * 64 bytes in flight per
// workgroup), accumulating into U x 4 per-lane partial sums in a fixed order.
// Steps wholly inside [start, end) run unmasked; only the last one is masked.
template <int P, int M, int T, int U>
__device__ __forceinline__ void sum_step(const float* __restrict__ ar, const float* __restrict__ br, int base,
                                         int end, f32x4* acc) {
    f32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j0 = base + (u * T + (int)threadIdx.x) * 4;
        va[u] = load4m<M, true>(ar, j0, end, 0.f);
        if constexpr (P == kReluAdd) vb[u] = load4m<M, true>(br, j0, end, 0.f);
        else vb[u] = va[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] += map4<P>(va[u], vb[u]);
}

template <int P, int T, int U, bool VEC>
__device__ __forceinline__ float lane_sum_range(const float* __restrict__ ar, const float* __restrict__ br,
                                                int start, int end) {
    constexpr int STEP = T * 4 * U;
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int full = start + (end - start) / STEP * STEP;
    int base = start;
    for (; base < full; base += STEP) sum_step<P, body_mask<VEC>(), T, U>(ar, br, base, end, acc);
    if (base < end) sum_step<P, tail_mask<VEC>(), T, U>(ar, br, base, end, acc);
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) s += (acc[u].x + acc[u].y) + (acc[u].z + acc[u].w);
    return s;
}

template <int P, int T, int U, bool VEC>
__global__ __launch_bounds__(T) void fr_red_sum_f32(const float* __restrict__ a, const float* __restrict__ b,
                                                    float* __restrict__ out, int rows, int cols, int64_t a_rs,
                                                    int64_t b_rs, int64_t out_s, float post) {
    __shared__ float slots[T / kWave];
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const float* ar = a + (int64_t)r * a_rs;
        const float* br = P == kReluAdd ? b + (int64_t)r * b_rs : nullptr;
        float s = lane_sum_range<P, T, U, VEC>(ar, br, 0, cols);
        s = group_reduce<kWave>(s, OpSum());
        s = block_fold(s, slots, T / kWave, OpSum());
        if (threadIdx.x == 0) out[(int64_t)r * out_s] = s * post;
        __syncthreads();  // slots are rewritten by the next row
    }
}

// ------------------------------------------------------------------ split
// Workgroup w reduces chunk c = w % S of row r = w / S, i.e. elements
// [c * chunk, min(cols, (c + 1) * chunk)), and writes the raw partial sum to
// ws[r * S + c]. chunk is a multiple of 4 * T * U, so every chunk starts on a
// 16-byte boundary of its row and all its steps but the row's last are full.
template <int P, int T, int U, bool VEC>
__global__ __launch_bounds__(T) void fr_split_sum_f32(const float* __restrict__ a, const float* __restrict__ b,
                                                      float* __restrict__ ws, int rows, int cols, int64_t a_rs,
                                                      int64_t b_rs, int chunk, int S) {
    __shared__ float slots[T / kWave];
    const int64_t w = blockIdx.x;
    const int r = (int)(w / S);
    const int c = (int)(w % S);
    if (r >= rows) return;
    const int start = c * chunk;
    const int end = min(cols, start + chunk);
    const float* ar = a + (int64_t)r * a_rs;
    const float* br = P == kReluAdd ? b + (int64_t)r * b_rs : nullptr;
    float s = lane_sum_range<P, T, U, VEC>(ar, br, start, end);
    s = group_reduce<kWave>(s, OpSum());
    s = block_fold(s, slots, T / kWave, OpSum());
    if (threadIdx.x == 0) ws[w] = s;
}

// ------------------------------------------------------------------ launchers
namespace {

using PerFn = void (*)(const float*, const float*, float*, int, int, int64_t, int64_t, int64_t, float);
using SplitFn = void (*)(const float*, const float*, float*, int, int, int64_t, int64_t, int, int);

template <int P, int M>
PerFn pick_per_m(int seg, int nv) {
    switch (seg) {
        case 8: return nv == 1 ? fr_per_sum_f32<P, 8, 1, M> : nullptr;
        case 16: return nv == 1 ? fr_per_sum_f32<P, 16, 1, M> : nullptr;
        case 32: return nv == 1 ? fr_per_sum_f32<P, 32, 1, M> : nullptr;
        case 64:
            switch (nv) {
                case 1: return fr_per_sum_f32<P, 64, 1, M>;
                case 2: return fr_per_sum_f32<P, 64, 2, M>;
                case 4: return fr_per_sum_f32<P, 64, 4, M>;
                case 8: return fr_per_sum_f32<P, 64, 8, M>;
            }
    }
    return nullptr;
}

template <int P>
PerFn pick_per(int mask, int seg, int nv) {
    switch (mask) {
        case kNone: return pick_per_m<P, kNone>(seg, nv);
        case kVec: return pick_per_m<P, kVec>(seg, nv);
        case kElem: return pick_per_m<P, kElem>(seg, nv);
        default: return pick_per_m<P, kScalar>(seg, nv);
    }
}

// Mask mode of a persistent launch over dense rows of `cols` elements.
int per_mask(bool vec, int cols, int seg, int nv) {
    if (!vec) return kScalar;
    if (cols == 4 * seg * nv) return kNone;
    return cols % 4 == 0 ? kVec : kElem;
}

template <int P, bool VEC>
PerFn pick_red(int threads, int u) {
    if (threads == 256 && u == 4) return fr_red_sum_f32<P, 256, 4, VEC>;
    if (threads == 512 && u == 2) return fr_red_sum_f32<P, 512, 2, VEC>;
    if (threads == 256 && u == 8) return fr_red_sum_f32<P, 256, 8, VEC>;
    return nullptr;
}

template <int P, bool VEC>
SplitFn pick_split(int threads, int u) {
    if (threads == 256 && u == 4) return fr_split_sum_f32<P, 256, 4, VEC>;
    if (threads == 256 && u == 8) return fr_split_sum_f32<P, 256, 8, VEC>;
    if (threads == 512 && u == 2) return fr_split_sum_f32<P, 512, 2, VEC>;
    return nullptr;
}

template <int P>
hipError_t launch_sum_p(const fr_plan& p, const SumArgs& a, hipStream_t s) {
    const float post = P == kReluAdd ? 2.f : 1.f;
    if (p.form == FR_FORM_PER) {
        if (p.seg < 8 || p.rows_per_wg != 256 / p.seg) return hipErrorInvalidDeviceFunction;  // one row per group
        PerFn f = pick_per<P>(per_mask(p.vec16 != 0, a.cols, p.seg, p.vec), p.seg, p.vec);
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(256), 0, s, a.a, a.b, a.out, a.rows, a.cols, a.a_rs,
                           a.b_rs, a.out_s, post);
        return hipGetLastError();
    }
    if (p.form == FR_FORM_RED) {
        PerFn f = p.vec16 ? pick_red<P, true>(p.threads, p.vec) : pick_red<P, false>(p.threads, p.vec);
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.a, a.b, a.out, a.rows, a.cols,
                           a.a_rs, a.b_rs, a.out_s, post);
        return hipGetLastError();
    }
    if (p.form == FR_FORM_SPLIT) {
        SplitFn f = p.vec16 ? pick_split<P, true>(p.threads, p.vec) : pick_split<P, false>(p.threads, p.vec);
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.a, a.b, a.ws, a.rows, a.cols,
                           a.a_rs, a.b_rs, p.chunk, p.splits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // Finishing pass: a persistent reduction over each row's S partials.
        const int S = p.splits;
        const int seg = S <= 32 ? 8 : (S <= 64 ? 16 : (S <= 128 ? 32 : 64));
        int nv = (S + 4 * seg - 1) / (4 * seg);
        nv = nv <= 1 ? 1 : (nv <= 2 ? 2 : (nv <= 4 ? 4 : 8));
        PerFn fin = pick_per<kIdent>(per_mask(S % 4 == 0, S, seg, nv), seg, nv);
        if (!fin) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(fin, dim3((unsigned)p.grid2), dim3(256), 0, s, a.ws, nullptr, a.out, a.rows, S,
                           (int64_t)S, (int64_t)0, a.out_s, post);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sum(const fr_plan& p, const SumArgs& a, hipStream_t s) {
    return a.prologue == kReluAdd ? launch_sum_p<kReluAdd>(p, a, s) : launch_sum_p<kSquare>(p, a, s);
}

}  // namespace fr
