// fr_layernorm.hip - LayerNorm over bf16 rows with fp32 arithmetic: the mean
// and the variance are two fused reductions over the row, followed by the
// normalize / affine / round-to-bf16 epilogue ("Stax (4): GPU Codegen and
// Dynamic Shapes", 10.4 names variance reductions that also output the mean;
// 9.8: half precision is computed in fp32).
//   persistent  fr_per_layernorm_bf16  one workgroup holds the whole row in
//                                      registers (8 bf16 per 16-byte vector,
//                                      NV vectors per lane): exact two-pass
//                                      mean and variance over registers, one
//                                      read and one write of the row
//   looped      fr_red_layernorm_bf16  one workgroup streams the row: per-lane
//                                      Welford statistics, merged per 8-value
//                                      vector and across lanes and waves with
//                                      Chan's pairwise update; a second pass
//                                      re-reads the row and writes y
#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

// Load the 8 bf16 at j0..j0+7 of a row of length L as packed words; element
// j >= L is never touched and reads as +0. Mask modes as for fp32 rows:
// kNone (every vector inside the row), kVec (16-byte aligned rows whose
// length is a multiple of 8: a vector is wholly inside or outside), kScalar
// (element accesses).
template <int M, bool NT>
__device__ __forceinline__ u32x4 load8m(const uint16_t* row, int j0, int L) {
    if constexpr (M == kNone) return ld4u<NT>(row + j0);
    else if constexpr (M == kVec) return j0 < L ? ld4u<NT>(row + j0) : u32x4{0u, 0u, 0u, 0u};
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 8; ++c)
        if (j0 + c < L) w[c >> 1] |= (uint32_t)row[j0 + c] << ((c & 1) * 16);
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <int M, bool NT>
__device__ __forceinline__ void store8m(uint16_t* row, int j0, int L, u32x4 v) {
    if constexpr (M == kNone) {
        st4u<NT>(row + j0, v);
        return;
    } else if constexpr (M == kVec) {
        if (j0 < L) st4u<NT>(row + j0, v);
        return;
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 8; ++c)
        if (j0 + c < L) row[j0 + c] = (uint16_t)(w[c >> 1] >> ((c & 1) * 16));
}

__device__ __forceinline__ uint32_t word(u32x4 v, int i) { return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w)); }

// y = (x - mu) * rstd * gamma + beta for the 8 values of one vector, packed
// back to bf16 with round-to-nearest-even. When x == mu the product is an
// exact 0 and y is exactly beta.
__device__ __forceinline__ u32x4 affine8(u32x4 xv, u32x4 gv, u32x4 bv, float mu, float rstd) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t xw = word(xv, i), gw = word(gv, i), bw = word(bv, i);
        const float lo = (bf16_lo(xw) - mu) * rstd * bf16_lo(gw) + bf16_lo(bw);
        const float hi = (bf16_hi(xw) - mu) * rstd * bf16_hi(gw) + bf16_hi(bw);
        o[i] = pack_bf16(lo, hi);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

template <int M>
__device__ __forceinline__ u32x4 normalize8(u32x4 xv, int j0, int L, const uint16_t* __restrict__ gamma,
                                            const uint16_t* __restrict__ beta, float mu, float rstd) {
    u32x4 gv = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // 1.0 in bf16
    u32x4 bv = {0u, 0u, 0u, 0u};
    if (gamma) gv = load8m<M, false>(gamma, j0, L);
    if (beta) bv = load8m<M, false>(beta, j0, L);
    return affine8(xv, gv, bv, mu, rstd);
}

// ------------------------------------------------------------------ persistent
// One workgroup of T threads per row, NV vectors of 8 bf16 per lane (row
// capacity 8 * T * NV); M is the masking mode (kNone when the row fills the
// capacity exactly). OCC > 1 would ask the compiler for at least OCC waves
// per SIMD; the compiled variants use 1 (no request).
//
// Rows that fill the capacity exactly (kNone) use buffer instructions: the
// row base lives in a scalar buffer resource and each lane keeps one offset
// register (the vector index goes into the scalar offset), where 64-bit
// addresses would take two registers per vector and per operand (x, gamma,
// beta, y). Every access is inside the row, so the resource's range check
// never applies (a missing gamma or beta gets an empty range and reads
// zeros; without gamma the launcher picks the UNIT_GAMMA instance). The register values are hidden from the compiler between passes so
// that it converts bf16 -> fp32 in each pass instead of keeping 64 fp32
// copies alive, and gamma / beta are loaded in two halves. The row stays in
// 32 packed registers per lane; the 512 x 8 kernel fits 7 waves per SIMD.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufferRsrcWord3);
}
__device__ __forceinline__ void hide(u32x4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
constexpr int kAuxNT = 2;  // buffer instruction cache policy: non-temporal

// y = affine of the row held in v, through buffer resources; gamma and beta
// are loaded in two halves so that only half of them is live at a time.
template <int T, int NV, bool UNIT_GAMMA>
__device__ __forceinline__ void affine_row(const u32x4* v, __amdgpu_buffer_rsrc_t ry, __amdgpu_buffer_rsrc_t rg,
                                           __amdgpu_buffer_rsrc_t rb, int voff, float mu, float rstd) {
    constexpr int H = NV > 1 ? NV / 2 : 1;
#pragma unroll
    for (int h = 0; h < NV / H; ++h) {
        u32x4 gv[H], bv[H];
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const int off = (h * H + k) * T * 16;
            if constexpr (UNIT_GAMMA) gv[k] = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // 1.0
            else gv[k] = __builtin_amdgcn_raw_buffer_load_b128(rg, voff, off, 0);
            bv[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, off, 0);
        }
#pragma unroll
        for (int k = 0; k < H; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(affine8(v[h * H + k], gv[k], bv[k], mu, rstd), ry, voff,
                                                   (h * H + k) * T * 16, kAuxNT);
        asm volatile("" ::: "memory");  // the next half's loads stay after these stores
    }
}

template <int T, int NV, int M, int OCC, bool UNIT_GAMMA = false>
__global__ __launch_bounds__(T, OCC) void fr_per_layernorm_bf16(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                                const uint16_t* __restrict__ beta, uint16_t* y,
                                                                int rows, int cols, int64_t x_rs, int64_t y_rs,
                                                                float eps) {
    __shared__ float sl_s[T / kWave];
    __shared__ float sl_q[T / kWave];
    const int tid = threadIdx.x;
    const float n = (float)cols;
    constexpr bool BUF = M == kNone;
    const uint32_t bytes = (uint32_t)cols * 2u;
    const int voff = tid * 16;
    // a missing gamma / beta gets an empty range: its loads read zeros
    const __amdgpu_buffer_rsrc_t rg = row_rsrc(gamma, gamma ? bytes : 0u);
    const __amdgpu_buffer_rsrc_t rb = row_rsrc(beta, beta ? bytes : 0u);
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const uint16_t* xr = x + (int64_t)r * x_rs;
        u32x4 v[NV];
        if constexpr (BUF) {
            const __amdgpu_buffer_rsrc_t rx = row_rsrc(xr, bytes);
#pragma unroll
            for (int k = 0; k < NV; ++k) v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, k * T * 16, kAuxNT);
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k) v[k] = load8m<M, true>(xr, (k * T + tid) * 8, cols);
        }
        // pass 1 over registers: the sum (masked elements read as +0)
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) s += bf16_lo(word(v[k], i)) + bf16_hi(word(v[k], i));
        if constexpr (BUF) {
#pragma unroll
            for (int k = 0; k < NV; ++k) hide(v[k]);
        }
        s = group_reduce<kWave>(s, OpSum());
        s = block_fold(s, sl_s, T / kWave, OpSum());
        const float mu = s / n;  // correctly rounded: a constant row gives mu == x exactly
        // pass 2 over registers: sum of squared deviations of valid elements
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int j0 = (k * T + tid) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float dl = (M == kNone || j0 + 2 * i < cols) ? bf16_lo(word(v[k], i)) - mu : 0.f;
                const float dh = (M == kNone || j0 + 2 * i + 1 < cols) ? bf16_hi(word(v[k], i)) - mu : 0.f;
                q += dl * dl + dh * dh;
            }
        }
        if constexpr (BUF) {
#pragma unroll
            for (int k = 0; k < NV; ++k) hide(v[k]);
        }
        q = group_reduce<kWave>(q, OpSum());
        q = block_fold(q, sl_q, T / kWave, OpSum());
        const float rstd = 1.0f / sqrtf(q / n + eps);
        uint16_t* yr = y + (int64_t)r * y_rs;
        if constexpr (BUF) {
            const __amdgpu_buffer_rsrc_t ry = row_rsrc(yr, bytes);
            affine_row<T, NV, UNIT_GAMMA>(v, ry, rg, rb, voff, mu, rstd);
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int j0 = (k * T + tid) * 8;
                if (j0 < cols) store8m<M, true>(yr, j0, cols, normalize8<M>(v[k], j0, cols, gamma, beta, mu, rstd));
            }
        }
        __syncthreads();  // slots are rewritten by the next row
    }
}

// ------------------------------------------------------------------ looped (Welford)
// Statistics of the (up to) 8 valid values of one vector: count, mean and
// sum of squared deviations, computed exactly in two steps over registers.
__device__ __forceinline__ Stat stat8(u32x4 v, int j0, int L) {
    const int cnt = L - j0 >= 8 ? 8 : (L - j0 > 0 ? L - j0 : 0);
    if (cnt == 0) return Stat{0.f, 0.f, 0.f};
    float val[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        val[2 * i] = bf16_lo(word(v, i));
        val[2 * i + 1] = bf16_hi(word(v, i));
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) s += val[c];  // masked values are +0
    const float n = (float)cnt;
    const float mean = cnt == 8 ? s * 0.125f : s / n;
    float m2 = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float d = c < cnt ? val[c] - mean : 0.f;
        m2 += d * d;
    }
    return Stat{n, mean, m2};
}

template <int M, int T, int U>
__device__ __forceinline__ Stat welford_step(const uint16_t* xr, int base, int cols, Stat st) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load8m<M, false>(xr, base + (u * T + (int)threadIdx.x) * 8, cols);
#pragma unroll
    for (int u = 0; u < U; ++u) st = stat_combine(st, stat8(v[u], base + (u * T + (int)threadIdx.x) * 8, cols));
    return st;
}

template <int M, int T, int U>
__device__ __forceinline__ void normalize_step(const uint16_t* xr, uint16_t* yr, int base, int cols,
                                               const uint16_t* __restrict__ gamma,
                                               const uint16_t* __restrict__ beta, float mu, float rstd) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load8m<M, true>(xr, base + (u * T + (int)threadIdx.x) * 8, cols);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j0 = base + (u * T + (int)threadIdx.x) * 8;
        if (M == kNone || j0 < cols)
            store8m<M, true>(yr, j0, cols, normalize8<M>(v[u], j0, cols, gamma, beta, mu, rstd));
    }
}

// Steps wholly inside the row run unmasked; only the last step is masked.
template <int T, int U, bool VEC>
__global__ __launch_bounds__(T) void fr_red_layernorm_bf16(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                           const uint16_t* __restrict__ beta, uint16_t* y, int rows,
                                                           int cols, int64_t x_rs, int64_t y_rs, float eps) {
    constexpr int STEP = T * 8 * U;
    constexpr int BODY = VEC ? kNone : kScalar;
    constexpr int TAIL = VEC ? kVec : kScalar;
    __shared__ Stat sl[T / kWave];
    const int full = cols - cols % STEP;
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const uint16_t* xr = x + (int64_t)r * x_rs;
        Stat st{0.f, 0.f, 0.f};
        int base = 0;
        for (; base < full; base += STEP) st = welford_step<BODY, T, U>(xr, base, cols, st);
        if (base < cols) st = welford_step<TAIL, T, U>(xr, base, cols, st);
        st = group_reduce<kWave>(st, OpStat());
        st = block_fold(st, sl, T / kWave, OpStat());
        const float mu = st.mu;
        const float rstd = 1.0f / sqrtf(st.m2 / (float)cols + eps);
        uint16_t* yr = y + (int64_t)r * y_rs;
        for (base = 0; base < full; base += STEP) normalize_step<BODY, T, U>(xr, yr, base, cols, gamma, beta, mu, rstd);
        if (base < cols) normalize_step<TAIL, T, U>(xr, yr, base, cols, gamma, beta, mu, rstd);
        __syncthreads();  // slots are rewritten by the next row
    }
}

// ------------------------------------------------------------------ launchers
namespace {

using LnFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int64_t, int64_t,
                      float);

// Persistent configurations: 16-byte vector kernels hold up to 8 vectors
// (64 bf16) per lane, or 4 with 1024 threads, without spilling; element-wise
// kernels (unaligned rows) up to 4. Asking for more waves per SIMD than the
// compiler's own choice (occ > 1) makes these kernels spill, so no such
// variant is compiled.
template <int M, bool UG>
LnFn pick_per_m(int threads, int nv) {
    constexpr bool VEC = M != kScalar;
    if (threads == 64) {
        switch (nv) {
            case 1: return fr_per_layernorm_bf16<64, 1, M, 1, UG>;
            case 2: return fr_per_layernorm_bf16<64, 2, M, 1, UG>;
            case 4: return fr_per_layernorm_bf16<64, 4, M, 1, UG>;
        }
        if constexpr (VEC)
            if (nv == 8) return fr_per_layernorm_bf16<64, 8, M, 1, UG>;
        return nullptr;
    }
    if (nv == (VEC ? 8 : 4)) {
        switch (threads) {
            case 128: return fr_per_layernorm_bf16<128, VEC ? 8 : 4, M, 1, UG>;
            case 256: return fr_per_layernorm_bf16<256, VEC ? 8 : 4, M, 1, UG>;
            case 512: return fr_per_layernorm_bf16<512, VEC ? 8 : 4, M, 1, UG>;
        }
    }
    if constexpr (VEC)
        if (threads == 1024 && nv == 4) return fr_per_layernorm_bf16<1024, 4, M, 1, UG>;
    return nullptr;
}

// unit_gamma (no gamma given) selects separate instances only where the
// buffer path (kNone) reads gamma; the other paths test the pointer.
LnFn pick_per(int mask, int threads, int nv, int occ, bool unit_gamma) {
    if (occ > 1) return nullptr;
    switch (mask) {
        case kNone:
            return unit_gamma ? pick_per_m<kNone, true>(threads, nv) : pick_per_m<kNone, false>(threads, nv);
        case kVec: return pick_per_m<kVec, false>(threads, nv);
        default: return pick_per_m<kScalar, false>(threads, nv);
    }
}

template <bool VEC>
LnFn pick_red(int threads, int u) {
    if (threads == 256 && u == 4) return fr_red_layernorm_bf16<256, 4, VEC>;
    if (threads == 512 && u == 2) return fr_red_layernorm_bf16<512, 2, VEC>;
    if (threads == 1024 && u == 2) return fr_red_layernorm_bf16<1024, 2, VEC>;
    return nullptr;
}

}  // namespace

hipError_t launch_layernorm(const fr_plan& p, const LayerNormArgs& a, hipStream_t s) {
    const bool vec = p.vec16 != 0;
    LnFn f = nullptr;
    if (p.form == FR_FORM_PER) {
        const int mask = !vec ? kScalar : (a.cols == 8 * p.threads * p.vec ? kNone : kVec);
        f = pick_per(mask, p.threads, p.vec, p.occupancy, a.gamma == nullptr);
    }
    else if (p.form == FR_FORM_RED)
        f = vec ? pick_red<true>(p.threads, p.vec) : pick_red<false>(p.threads, p.vec);
    if (!f) return hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.gamma, a.beta, a.y, a.rows, a.cols,
                       a.x_rs, a.y_rs, a.eps);
    return hipGetLastError();
}

}  // namespace fr
