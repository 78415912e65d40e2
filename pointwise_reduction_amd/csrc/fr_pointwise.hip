// fr_pointwise.hip - pointwise kernels: no reduction dimension, one or more
// elementwise dimensions ("Stax (4): GPU Codegen and Dynamic Shapes", 9.3).
//
//   fr_add_2d_f32   out = a + b over a 2-D index space in which each operand
//                   is contiguous either along the output's rows or along
//                   its columns (Listing 9.2: Example 6.1, x.t() + y). A
//                   workgroup owns a TI x TJ output tile. Operands that are
//                   contiguous along the output's rows are read along them
//                   directly; a transposed operand is read along its own
//                   contiguous direction into LDS and read back across it,
//                   so that every global access coalesces (the 2-D tiling
//                   of 9.3, with the exchange done in LDS).
//   fr_gelu_bwd     dx = dy * (Phi(h) + h phi(h)) (Listing 9.3, the GELU
//                   backward of Example 5.1): dy is one broadcast value (the
//                   upstream gradient of a scalar loss) or one per element;
//                   fp32 or bf16 storage, fp32 arithmetic.
#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

// ------------------------------------------------------------------ add 2-D
// Thread layouts of a TI x TJ tile over 256 threads, 4 consecutive elements
// per thread and pass:
//   along the output's rows (the output, row-major operands): TJ / 4 threads
//   per tile row, 1024 / TJ tile rows per pass;
//   along the output's columns (transposed operands): TI / 4 threads per
//   tile column, 1024 / TI tile columns per pass.
// A transposed operand's tile sits in LDS as [TJ][TI + 1] floats; the odd
// pitch spreads the column reads of one wave over the banks.
template <int TI, int TJ>
struct Tile {
    static constexpr int kPasses = TI * TJ / 1024;
    static constexpr int kRowThreads = TJ / 4, kRowsPerPass = 1024 / TJ;
    static constexpr int kColThreads = TI / 4, kColsPerPass = 1024 / TI;
    static constexpr int kPitch = TI + 1;
    static_assert(TI % 4 == 0 && TJ % 4 == 0 && (TI * TJ) % 1024 == 0 && TI <= 1024 && TJ <= 1024, "tile");
};

// Loads of one operand for one pass. T (transposed): the column layout,
// else the row layout. FULL: the tile lies inside the matrix and every
// access may be a 16-byte vector; otherwise element loads with bounds
// checks, 0 outside.
template <int TI, int TJ, bool T, bool FULL>
__device__ __forceinline__ f32x4 add2d_load(const float* p, int64_t rs, int64_t cs, int64_t i0, int64_t j0, int q,
                                            int64_t rows, int64_t cols) {
    using G = Tile<TI, TJ>;
    const int t = threadIdx.x;
    if constexpr (T) {
        const int64_t i = i0 + (t % G::kColThreads) * 4;
        const int64_t j = j0 + t / G::kColThreads + q * G::kColsPerPass;
        if constexpr (FULL) return ld4<true>(p + j * cs + i);
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (i + c < rows && j < cols) ? ld1<true>(p + (i + c) * rs + j * cs) : 0.f;
        return v;
    } else {
        const int64_t i = i0 + t / G::kRowThreads + q * G::kRowsPerPass;
        const int64_t j = j0 + (t % G::kRowThreads) * 4;
        if constexpr (FULL) return ld4<true>(p + i * rs + j);
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (i < rows && j + c < cols) ? ld1<true>(p + i * rs + (j + c) * cs) : 0.f;
        return v;
    }
}

// Column-layout registers -> LDS tile [TJ][TI + 1].
template <int TI, int TJ>
__device__ __forceinline__ void add2d_stage(float* s, f32x4 v, int q) {
    using G = Tile<TI, TJ>;
    const int t = threadIdx.x;
    const int i = (t % G::kColThreads) * 4, j = t / G::kColThreads + q * G::kColsPerPass;
#pragma unroll
    for (int c = 0; c < 4; ++c) s[j * G::kPitch + i + c] = v[c];
}

// LDS tile -> the row layout of pass q.
template <int TI, int TJ>
__device__ __forceinline__ f32x4 add2d_unstage(const float* s, int q) {
    using G = Tile<TI, TJ>;
    const int t = threadIdx.x;
    const int i = t / G::kRowThreads + q * G::kRowsPerPass, j = (t % G::kRowThreads) * 4;
    f32x4 v;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = s[(j + c) * G::kPitch + i];
    return v;
}

template <int TI, int TJ, bool TA, bool TB, bool FULL>
__device__ __forceinline__ void add2d_tile(const float* __restrict__ a, const float* __restrict__ b,
                                           float* __restrict__ out, int64_t rows, int64_t cols, int64_t a_rs,
                                           int64_t a_cs, int64_t b_rs, int64_t b_cs, int64_t out_rs, int64_t i0,
                                           int64_t j0, float* sa, float* sb) {
    using G = Tile<TI, TJ>;
    f32x4 va[G::kPasses], vb[G::kPasses];
    // every load of the tile is issued before the first is used
#pragma unroll
    for (int q = 0; q < G::kPasses; ++q) {
        va[q] = add2d_load<TI, TJ, TA, FULL>(a, a_rs, a_cs, i0, j0, q, rows, cols);
        vb[q] = add2d_load<TI, TJ, TB, FULL>(b, b_rs, b_cs, i0, j0, q, rows, cols);
    }
    if constexpr (TA || TB) {
#pragma unroll
        for (int q = 0; q < G::kPasses; ++q) {
            if constexpr (TA) add2d_stage<TI, TJ>(sa, va[q], q);
            if constexpr (TB) add2d_stage<TI, TJ>(sb, vb[q], q);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < G::kPasses; ++q) {
            if constexpr (TA) va[q] = add2d_unstage<TI, TJ>(sa, q);
            if constexpr (TB) vb[q] = add2d_unstage<TI, TJ>(sb, q);
        }
    }
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < G::kPasses; ++q) {
        const f32x4 r = va[q] + vb[q];
        const int64_t i = i0 + t / G::kRowThreads + q * G::kRowsPerPass;
        const int64_t j = j0 + (t % G::kRowThreads) * 4;
        if constexpr (FULL) {
            st4<true>(out + i * out_rs + j, r);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (i < rows && j + c < cols) st1<true>(out + i * out_rs + j + c, r[c]);
        }
    }
    // the next tile of this workgroup overwrites the LDS tiles
    if constexpr (TA || TB) __syncthreads();
}

// Grid-stride over tiles in row-major tile order. vec: every base and the
// stride along which an operand is read allow 16-byte vectors; then tiles
// inside the matrix use them and edge tiles use element accesses.
template <int TI, int TJ, bool TA, bool TB>
__global__ __launch_bounds__(256) void fr_add_2d_f32(const float* __restrict__ a, const float* __restrict__ b,
                                                     float* __restrict__ out, int64_t rows, int64_t cols,
                                                     int64_t a_rs, int64_t a_cs, int64_t b_rs, int64_t b_cs,
                                                     int64_t out_rs, int64_t tiles_j, int64_t tiles, int vec) {
    using G = Tile<TI, TJ>;
    constexpr int kTileFloats = TJ * G::kPitch;
    __shared__ float lds[(TA ? kTileFloats : 0) + (TB ? kTileFloats : 0) + 1];
    float* sa = lds;
    float* sb = lds + (TA ? kTileFloats : 0);
    // tiles in bands of two tile rows, column by column within a band:
    // consecutive workgroups read a transposed operand's adjacent segments
    // (rows i0 and i0 + TI of one column run) while the row-major operands
    // still move along their rows (row order alone: 140.0 us at 8192 x 8192;
    // bands of 2: 137.5; of 4: 137.8; column order: 198)
    const int64_t tiles_i = tiles / tiles_j;
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        constexpr int BD = 2;
        const int64_t band = tile / (BD * tiles_j), in = tile % (BD * tiles_j);
        const int64_t bh = (band + 1) * BD <= tiles_i ? BD : tiles_i - band * BD;  // tile rows in this band
        const int64_t i0 = (band * BD + in % bh) * TI, j0 = (in / bh) * TJ;
        if (vec && i0 + TI <= rows && j0 + TJ <= cols)
            add2d_tile<TI, TJ, TA, TB, true>(a, b, out, rows, cols, a_rs, a_cs, b_rs, b_cs, out_rs, i0, j0, sa, sb);
        else
            add2d_tile<TI, TJ, TA, TB, false>(a, b, out, rows, cols, a_rs, a_cs, b_rs, b_cs, out_rs, i0, j0, sa, sb);
    }
}

using Add2dFn = void (*)(const float*, const float*, float*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                         int64_t, int64_t, int64_t, int);

template <int TI, int TJ>
Add2dFn pick_add2d_tile(bool ta, bool tb) {
    if (ta) return tb ? fr_add_2d_f32<TI, TJ, true, true> : fr_add_2d_f32<TI, TJ, true, false>;
    return tb ? fr_add_2d_f32<TI, TJ, false, true> : fr_add_2d_f32<TI, TJ, false, false>;
}

Add2dFn pick_add2d(int ti, int tj, bool ta, bool tb) {
    if (ti == 64 && tj == 64) return pick_add2d_tile<64, 64>(ta, tb);
    if (ti == 32 && tj == 128) return pick_add2d_tile<32, 128>(ta, tb);
    if (ti == 128 && tj == 32) return pick_add2d_tile<128, 32>(ta, tb);
    if (ti == 64 && tj == 128) return pick_add2d_tile<64, 128>(ta, tb);
    if (ti == 128 && tj == 64) return pick_add2d_tile<128, 64>(ta, tb);
    if (ti == 32 && tj == 32) return pick_add2d_tile<32, 32>(ta, tb);
    return nullptr;
}

hipError_t launch_add_2d(const fr_plan& p, const Add2dArgs& a, hipStream_t s) {
    Add2dFn f = pick_add2d(p.rows_per_wg, p.chunk, a.a_t, a.b_t);
    if (!f) return hipErrorInvalidDeviceFunction;
    const int64_t tiles_j = (a.cols + p.chunk - 1) / p.chunk;
    const int64_t tiles = (a.rows + p.rows_per_wg - 1) / p.rows_per_wg * tiles_j;
    hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(256), 0, s, a.a, a.b, a.out, a.rows, a.cols, a.a_rs, a.a_cs,
                       a.b_rs, a.b_cs, a.out_rs, tiles_j, tiles, p.vec16);
    return hipGetLastError();
}

// ------------------------------------------------------------ GELU backward
// GELU'(h) = Phi(h) + h phi(h), Phi(h) = (1 + erf(h / sqrt 2)) / 2 and
// phi(h) = exp(-h^2 / 2) / sqrt(2 pi), evaluated as the pages' kernel
// orders it; erff and expf are the device library's (OCML) functions.
constexpr float kInvSqrt2 = 0.70710678118654752f;
constexpr float kInvSqrt2Pi = 0.39894228040143268f;

__device__ __forceinline__ float gelu_grad(float h) {
    const float cdf = 0.5f * (1.0f + erff(h * kInvSqrt2));
    const float pdf = kInvSqrt2Pi * expf(-0.5f * (h * h));
    return cdf + h * pdf;
}

// Storage types: 16-byte vectors of 4 fp32 or 8 bf16.
struct F32s {
    using V = f32x4;
    static constexpr int kPer = 4;
    __device__ static float get(const float* p, int64_t i) { return ld1<true>(p + i); }
    __device__ static void put(float* p, int64_t i, float v) { st1<true>(p + i, v); }
    __device__ static V load(const float* p, int64_t v) { return ld4<true>(p + v * 4); }
    __device__ static void store(float* p, int64_t v, V x) { st4<true>(p + v * 4, x); }
    __device__ static float lane(const V& x, int e) { return x[e]; }
    template <typename F>
    __device__ static V map(const V& x, F f) {
        return V{f(x[0], 0), f(x[1], 1), f(x[2], 2), f(x[3], 3)};
    }
};
struct Bf16s {
    using V = u32x4;
    static constexpr int kPer = 8;
    __device__ static float get(const uint16_t* p, int64_t i) {
        return __builtin_bit_cast(float, (uint32_t)__builtin_nontemporal_load(p + i) << 16);
    }
    __device__ static void put(uint16_t* p, int64_t i, float v) {
        __builtin_nontemporal_store((uint16_t)(pack_bf16(v, 0.f) & 0xFFFFu), p + i);
    }
    __device__ static V load(const uint16_t* p, int64_t v) { return ld4u<true>(p + v * 8); }
    __device__ static void store(uint16_t* p, int64_t v, V x) { st4u<true>(p + v * 8, x); }
    __device__ static float lane(const V& x, int e) { return (e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1]); }
    template <typename F>
    __device__ static V map(const V& x, F f) {
        V r;
#pragma unroll
        for (int w = 0; w < 4; ++w) r[w] = pack_bf16(f(bf16_lo(x[w]), 2 * w), f(bf16_hi(x[w]), 2 * w + 1));
        return r;
    }
};

// VEC: 16-byte vectors (h, dx and a per-element dy 16-byte aligned), NV per
// thread per step, grid-stride; the last n mod kPer elements are done one by
// one. Otherwise every element is accessed alone. BCAST: dy[0] for all.
template <typename S, typename T, int NV, bool BCAST, bool VEC>
__global__ __launch_bounds__(256) void fr_gelu_bwd(const T* __restrict__ dy, const T* __restrict__ h,
                                                   T* __restrict__ dx, int64_t n) {
    const float g0 = BCAST ? S::get(dy, 0) : 0.f;
    const int64_t t = threadIdx.x;
    if constexpr (VEC) {
        const int64_t nvec = n / S::kPer;
        const int64_t step = (int64_t)gridDim.x * 256 * NV;
        for (int64_t v0 = (int64_t)blockIdx.x * 256 * NV + t; v0 < nvec; v0 += step) {
            typename S::V hv[NV], gv[NV];
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int64_t v = v0 + k * 256;
                if (v < nvec) {
                    hv[k] = S::load(h, v);
                    if constexpr (!BCAST) gv[k] = S::load(dy, v);
                }
            }
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int64_t v = v0 + k * 256;
                if (v < nvec) {
                    const typename S::V& gk = gv[k];
                    typename S::V r = S::map(hv[k], [&](float x, int e) {
                        return (BCAST ? g0 : S::lane(gk, e)) * gelu_grad(x);
                    });
                    S::store(dx, v, r);
                }
            }
        }
        if (blockIdx.x == gridDim.x - 1)
            for (int64_t i = nvec * S::kPer + t; i < n; i += 256)
                S::put(dx, i, (BCAST ? g0 : S::get(dy, i)) * gelu_grad(S::get(h, i)));
    } else {
        const int64_t step = (int64_t)gridDim.x * 256;
        for (int64_t i = (int64_t)blockIdx.x * 256 + t; i < n; i += step)
            S::put(dx, i, (BCAST ? g0 : S::get(dy, i)) * gelu_grad(S::get(h, i)));
    }
}

template <typename S, typename T, bool BCAST>
void* pick_gelu_nv(int nv, bool vec) {
    if (!vec) return (void*)fr_gelu_bwd<S, T, 1, BCAST, false>;
    switch (nv) {
        case 1: return (void*)fr_gelu_bwd<S, T, 1, BCAST, true>;
        case 2: return (void*)fr_gelu_bwd<S, T, 2, BCAST, true>;
        case 4: return (void*)fr_gelu_bwd<S, T, 4, BCAST, true>;
    }
    return nullptr;
}

hipError_t launch_gelu_bwd(const fr_plan& p, const GeluBwdArgs& a, hipStream_t s) {
    const bool vec = p.vec16 != 0;
    if (a.bf16) {
        using Fn = void (*)(const uint16_t*, const uint16_t*, uint16_t*, int64_t);
        Fn f = (Fn)(a.bcast ? pick_gelu_nv<Bf16s, uint16_t, true>(p.vec, vec)
                            : pick_gelu_nv<Bf16s, uint16_t, false>(p.vec, vec));
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(256), 0, s, (const uint16_t*)a.dy, (const uint16_t*)a.h,
                           (uint16_t*)a.dx, a.n);
    } else {
        using Fn = void (*)(const float*, const float*, float*, int64_t);
        Fn f = (Fn)(a.bcast ? pick_gelu_nv<F32s, float, true>(p.vec, vec)
                            : pick_gelu_nv<F32s, float, false>(p.vec, vec));
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(256), 0, s, (const float*)a.dy, (const float*)a.h,
                           (float*)a.dx, a.n);
    }
    return hipGetLastError();
}

}  // namespace fr
