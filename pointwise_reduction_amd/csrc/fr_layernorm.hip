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
//               fr_pipe_layernorm_bf16 the same per row, one workgroup per CU
//                                      taking several rows with three in
//                                      flight (loads overlap the folds and
//                                      stores of earlier rows)
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
// register (a load's vector index goes into its scalar offset), where 64-bit
// addresses would take two registers per vector and per operand (x, gamma,
// beta, y). Every access is inside the row, so the resource's range check
// never applies (a missing gamma or beta gets an empty range and reads
// zeros; without gamma the launcher picks the UNIT_GAMMA instance). The register values are hidden from the compiler between passes so
// that it converts bf16 -> fp32 in each pass instead of keeping 64 fp32
// copies alive, and gamma / beta are loaded in two halves. The row stays in
// 32 packed registers per lane; the 512 x 8 kernel fits 7 waves per SIMD.
__device__ __forceinline__ void hide(u32x4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

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
            if constexpr (UNIT_GAMMA) {
                // 1.0, hidden from the compiler so that it multiplies as with
                // a loaded gamma (the pipelined kernel gives the same bits)
                gv[k] = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
                hide(gv[k]);
            } else {
                gv[k] = __builtin_amdgcn_raw_buffer_load_b128(rg, voff, off, 0);
            }
            bv[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, off, 0);
        }
#pragma unroll
        for (int k = 0; k < H; ++k)
            store16<kAuxNT>(affine8(v[h * H + k], gv[k], bv[k], mu, rstd), ry, voff + (h * H + k) * T * 16);
        asm volatile("" ::: "memory");  // the next half's loads stay after these stores
    }
}

// The statistics a training step's backward pass reads (both nullable).
__device__ __forceinline__ void save_stats(float* mean_out, float* rstd_out, int r, float mu, float rstd) {
    if (threadIdx.x == 0) {
        if (mean_out) mean_out[r] = mu;
        if (rstd_out) rstd_out[r] = rstd;
    }
}

template <int T, int NV, int M, int OCC, bool UNIT_GAMMA = false>
__global__ __launch_bounds__(T, OCC) void fr_per_layernorm_bf16(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                                const uint16_t* __restrict__ beta, uint16_t* y,
                                                                int rows, int cols, int64_t x_rs, int64_t y_rs,
                                                                float eps, float* __restrict__ mean_out,
                                                                float* __restrict__ rstd_out) {
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
        float s = sum_bf16<NV>(v);
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
        save_stats(mean_out, rstd_out, r, mu, rstd);
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

// ------------------------------------------------------------------ persistent, pipelined rows
// One workgroup per CU takes NR rows (r = blockIdx.x + i * gridDim.x) and
// keeps R of them in flight in registers: while one row's statistics, affine
// epilogue and stores run, the next R - 1 rows are loading, and a row's
// registers are reloaded with row i + R as soon as its stores are issued.
// When every workgroup holds its rows whole for the full read-fold-write
// chain (the kernel above), the whole device reads, then folds, then writes
// in step; here the HBM queue always holds some workgroup's next rows.
//
// gamma and beta are read once per workgroup into LDS (2 x 64 KiB at 32768
// columns, so one workgroup per CU), through the registers of the last two
// row sets: their loads are issued first, the first R - 2 rows' loads behind
// them, so waiting for gamma / beta waits for nothing else (vector loads
// complete in issue order); then the last two rows' loads go out. The row
// loop is unrolled over all NR rows, so that every wait counts exactly the
// loads still needed (a loop back edge would make the compiler wait for all).
// Rows past `rows` (the last workgroups when rows % gridDim.x != 0) load and
// store through empty buffer ranges: no memory is touched. Each row's
// arithmetic is the kernel above's with the same lane order (T threads, NV
// vectors per lane), so both give the same bits. Requires cols == 8 * T * NV
// and 16-byte aligned rows, gamma and beta.
template <int T, int NV, int R, int NR, bool STATS>
__global__ __launch_bounds__(T, 1) void fr_pipe_layernorm_bf16(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                              const uint16_t* __restrict__ beta, uint16_t* y, int rows,
                                                              int cols, int64_t x_rs, int64_t y_rs, float eps,
                                                              float* __restrict__ mean_out,
                                                              float* __restrict__ rstd_out) {
    static_assert(R >= 3 && R <= NR, "gamma and beta are staged through two row sets; one more row loads ahead");
    __shared__ u32x4 sg[NV * T];
    __shared__ u32x4 sb[NV * T];
    __shared__ float sl_s[T / kWave];
    __shared__ float sl_q[T / kWave];
    const int tid = threadIdx.x;
    const uint32_t bytes = (uint32_t)cols * 2u;
    const int voff = tid * 16;
    const float n = (float)cols;
    const int G = gridDim.x;
    auto load_row = [&](u32x4* v, int r) {
        const bool ok = r < rows;
        const __amdgpu_buffer_rsrc_t rx = row_rsrc(ok ? x + (int64_t)r * x_rs : x, ok ? bytes : 0u);
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, k * T * 16, kAuxNT);
    };
    u32x4 v[R][NV];
    {
        // a missing gamma reads as 1, a missing beta as 0 (empty range)
        const __amdgpu_buffer_rsrc_t rg = row_rsrc(gamma, gamma ? bytes : 0u);
        const __amdgpu_buffer_rsrc_t rb = row_rsrc(beta, beta ? bytes : 0u);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            v[R - 2][k] = __builtin_amdgcn_raw_buffer_load_b128(rg, voff, k * T * 16, 0);
            v[R - 1][k] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, k * T * 16, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < R - 2; ++i) load_row(v[i], blockIdx.x + i * G);
    const u32x4 one = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        sg[k * T + tid] = gamma ? v[R - 2][k] : one;
        sb[k * T + tid] = v[R - 1][k];
    }
#pragma unroll
    for (int i = R - 2; i < R; ++i) load_row(v[i], blockIdx.x + i * G);
    // (the first fold's barrier orders these LDS writes before any read)
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int c = i % R;
        const int r = blockIdx.x + i * G;
        float s = sum_bf16<NV>(v[c]);
#pragma unroll
        for (int k = 0; k < NV; ++k) hide(v[c][k]);
        s = group_reduce<kWave>(s, OpSum());
        s = block_fold(s, sl_s, T / kWave, OpSum());
        const float mu = s / n;
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float dl = bf16_lo(word(v[c][k], j)) - mu, dh = bf16_hi(word(v[c][k], j)) - mu;
                q += dl * dl + dh * dh;
            }
#pragma unroll
        for (int k = 0; k < NV; ++k) hide(v[c][k]);
        q = group_reduce<kWave>(q, OpSum());
        q = block_fold(q, sl_q, T / kWave, OpSum());
        const float rstd = 1.0f / sqrtf(q / n + eps);
        const bool ok = r < rows;
        if constexpr (STATS) {
            // the row statistics (each nullable): thread 0 inside a 4-byte
            // range, no branch (the instances without them run 1% faster)
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(uint32_t, mu), row_rsrc(mean_out ? mean_out + (ok ? r : 0) : mean_out,
                                                           mean_out && ok ? 4u : 0u), tid == 0 ? 0 : 4, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(uint32_t, rstd), row_rsrc(rstd_out ? rstd_out + (ok ? r : 0) : rstd_out,
                                                             rstd_out && ok ? 4u : 0u), tid == 0 ? 0 : 4, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t ry = row_rsrc(ok ? y + (int64_t)r * y_rs : y, ok ? bytes : 0u);
#pragma unroll
        for (int k = 0; k < NV; ++k)
            store16<kAuxNT>(affine8(v[c][k], sg[k * T + tid], sb[k * T + tid], mu, rstd), ry, voff + k * T * 16);
        // the two folds' slots are safe to rewrite: every thread has read
        // this row's sum slots before the variance barrier, and the variance
        // slots before the next row's sum barrier
        if (i + R < NR) load_row(v[c], r + R * G);
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
                                                           int cols, int64_t x_rs, int64_t y_rs, float eps,
                                                           float* __restrict__ mean_out,
                                                           float* __restrict__ rstd_out) {
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
        save_stats(mean_out, rstd_out, r, mu, rstd);
        uint16_t* yr = y + (int64_t)r * y_rs;
        for (base = 0; base < full; base += STEP) normalize_step<BODY, T, U>(xr, yr, base, cols, gamma, beta, mu, rstd);
        if (base < cols) normalize_step<TAIL, T, U>(xr, yr, base, cols, gamma, beta, mu, rstd);
        __syncthreads();  // slots are rewritten by the next row
    }
}

// ------------------------------------------------------------------ backward
// The derivative of the forward definition, from the statistics the forward
// pass saved: with xh = (x - mu) rstd and g = dy gamma,
//   dx = rstd (g - mean(g) - xh mean(g xh)),
//   dgamma = sum over rows of dy xh,  dbeta = sum over rows of dy.
// Persistent: one workgroup of T threads holds a row of x and of dy in
// registers (NV vectors of 8 bf16 per lane and array), forms the two row
// sums in a first pass over the registers and writes dx in a second. Each
// lane keeps the same columns for every row its workgroup handles, so with
// DG the second pass also accumulates that workgroup's dgamma and dbeta
// contributions (there, where x-hat and dy are unpacked anyway; in the first
// pass the compiler kept both unpacked copies alive) and the workgroup writes
// them as one partial row of ws[2][G][ldw] at the end; fr_layernorm_bwd_fin
// sums the G partials of each column in a fixed order. Masked elements read
// x = dy = 0 and contribute nothing (g = 0 and dy = 0). With 4 vectors per lane the dbeta partials
// live in LDS instead (each lane reads and writes only its own 8 x NV
// slots, so no barrier is involved): up to 128 KB for a 32768-column row,
// which keeps the register count under the 128 that 16 waves of a
// 1024-thread workgroup may use.
__device__ __forceinline__ float lane8(u32x4 v, int e) { return (e & 1) ? bf16_hi(word(v, e >> 1)) : bf16_lo(word(v, e >> 1)); }

template <int T, int NV, int M, bool DG>
__global__ __launch_bounds__(T) void fr_per_layernorm_bwd_bf16(const uint16_t* x, const uint16_t* dy,
                                                               const uint16_t* __restrict__ gamma,
                                                               const float* __restrict__ mean,
                                                               const float* __restrict__ rstd, uint16_t* dx,
                                                               float* __restrict__ ws, int rows, int cols,
                                                               int64_t x_rs, int64_t dy_rs, int64_t dx_rs,
                                                               int64_t ldw) {
    constexpr bool BL = DG && NV == 4;  // dbeta partials in LDS
    // 16-byte aligned rows use buffer instructions: the row base sits in a
    // scalar resource and a lane needs no 64-bit addresses. Whole rows
    // (kNone) put the vector's offset in the scalar offset; with kVec the
    // whole offset is in the lane's offset register, which the resource's
    // range check covers: vectors past the row read zeros and are not stored.
    constexpr bool BUF = M == kNone || M == kVec;
    auto bvo = [](int k) { return M == kNone ? (int)threadIdx.x * 16 : (k * T + (int)threadIdx.x) * 16; };
    auto bso = [](int k) { return M == kNone ? k * T * 16 : 0; };
    __shared__ float sl_a[T / kWave];
    __shared__ float sl_b[T / kWave];
    __shared__ f32x4 lb[BL ? T * NV * 2 : 1];
    const int tid = threadIdx.x;
    const float n = (float)cols;
    u32x4 gv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k)
        gv[k] = gamma ? load8m<M, false>(gamma, (k * T + tid) * 8, cols)
                      : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // 1.0
    float ag[DG ? NV : 1][8], ab[DG && !BL ? NV : 1][8];
    if constexpr (DG) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ag[k][e] = 0.f;
            if constexpr (BL) {
                lb[(k * T + tid) * 2] = f32x4{0.f, 0.f, 0.f, 0.f};
                lb[(k * T + tid) * 2 + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ab[k][e] = 0.f;
            }
        }
    }
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const uint16_t* xr = x + (int64_t)r * x_rs;
        const uint16_t* dr = dy + (int64_t)r * dy_rs;
        u32x4 xv[NV], dv[NV];
        if constexpr (BUF) {
            const __amdgpu_buffer_rsrc_t rx = row_rsrc(xr, (uint32_t)cols * 2u);
            const __amdgpu_buffer_rsrc_t rd = row_rsrc(dr, (uint32_t)cols * 2u);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                xv[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, bvo(k), bso(k), kAuxNT);
                dv[k] = __builtin_amdgcn_raw_buffer_load_b128(rd, bvo(k), bso(k), kAuxNT);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                xv[k] = load8m<M, true>(xr, (k * T + tid) * 8, cols);
                dv[k] = load8m<M, true>(dr, (k * T + tid) * 8, cols);
            }
        }
        const float mu = mean[r], rs = rstd[r];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xh = (lane8(xv[k], e) - mu) * rs;
                const float g = lane8(dv[k], e) * lane8(gv[k], e);
                s1 += g;
                s2 += g * xh;
            }
        // the second pass unpacks x, dy and gamma again rather than keeping
        // 3 x 8 fp32 copies per vector alive across the row sums
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            hide(xv[k]);
            hide(dv[k]);
            hide(gv[k]);
        }
        s1 = group_reduce<kWave>(s1, OpSum());
        s2 = group_reduce<kWave>(s2, OpSum());
        s1 = block_fold(s1, sl_a, T / kWave, OpSum());
        s2 = block_fold(s2, sl_b, T / kWave, OpSum());
        const float m1 = s1 / n, m2 = s2 / n;
        // second pass: dx, and this row's dgamma / dbeta contributions
        uint16_t* outr = dx + (int64_t)r * dx_rs;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int j0 = (k * T + tid) * 8;
            f32x4 b0, b1;
            if constexpr (BL) {
                b0 = lb[(k * T + tid) * 2];
                b1 = lb[(k * T + tid) * 2 + 1];
            }
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int e = 2 * i + h;
                    const float d = lane8(dv[k], e);
                    const float xh = (lane8(xv[k], e) - mu) * rs;
                    const float g = d * lane8(gv[k], e);
                    v[h] = rs * ((g - m1) - xh * m2);
                    if constexpr (DG) {
                        ag[k][e] += d * xh;
                        if constexpr (BL) {
                            if (e < 4) b0[e] += d;
                            else b1[e - 4] += d;
                        } else {
                            ab[k][e] += d;
                        }
                    }
                }
                o[i] = pack_bf16(v[0], v[1]);
            }
            if constexpr (BL) {
                lb[(k * T + tid) * 2] = b0;
                lb[(k * T + tid) * 2 + 1] = b1;
            }
            if constexpr (BUF)
                store16<kAuxNT>(u32x4{o[0], o[1], o[2], o[3]}, row_rsrc(outr, (uint32_t)cols * 2u), bvo(k) + bso(k));
            else if (j0 < cols)
                store8m<M, true>(outr, j0, cols, u32x4{o[0], o[1], o[2], o[3]});
        }
        __syncthreads();  // slots are rewritten by the next row
    }
    if constexpr (DG) {
        float* pg = ws + (int64_t)blockIdx.x * ldw;
        float* pb = ws + ((int64_t)gridDim.x + blockIdx.x) * ldw;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int j0 = (k * T + tid) * 8;
            f32x4 b0, b1;
            if constexpr (BL) {
                b0 = lb[(k * T + tid) * 2];
                b1 = lb[(k * T + tid) * 2 + 1];
            } else {
                b0 = f32x4{ab[k][0], ab[k][1], ab[k][2], ab[k][3]};
                b1 = f32x4{ab[k][4], ab[k][5], ab[k][6], ab[k][7]};
            }
            if (M == kNone || j0 + 8 <= cols) {
                // ldw and ws are multiples of 8 floats / 16-byte aligned
                st4<false>(pg + j0, f32x4{ag[k][0], ag[k][1], ag[k][2], ag[k][3]});
                st4<false>(pg + j0 + 4, f32x4{ag[k][4], ag[k][5], ag[k][6], ag[k][7]});
                st4<false>(pb + j0, b0);
                st4<false>(pb + j0 + 4, b1);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (j0 + e < cols) {
                        pg[j0 + e] = ag[k][e];
                        pb[j0 + e] = e < 4 ? b0[e] : b1[e - 4];
                    }
            }
        }
    }
}

// ---- rows split across a team of P workgroups of 1024 threads. Member p of
// team k holds columns [p W, p W + W) of rows k, k + K, k + 2K, ... (K
// teams), one vector of 8 bf16 per lane and array. Each member forms the two
// row sums over its part and publishes them in the workspace; every member
// adds the P parts in part order, so all of them use the same bits. The
// dgamma / dbeta partials are then per team (K partial rows, not one per
// workgroup), which cuts the partial traffic by the team size.
// A member works in steps of R rows and keeps NB = DL + 1 steps in
// registers. Step s issues the loads of step s + DL, forms and publishes the
// sums of step s + DL - 1 (one workgroup fold for all R rows) and finishes
// step s, whose partner sums were published DL - 1 steps earlier and whose
// slot words were loaded one step ahead: loads and exchange are in flight
// while other rows are worked on.
// A partner sum still missing after wait_ticks is computed from x and dy by
// the waiting member with the partner's lane mapping and reduction tree,
// which gives the partner's bits (so dx must not alias x or dy here; the
// launcher never picks this form then). Every wait ends, and the result does
// not depend on which members are resident. Slots: 16 bytes per (row, part),
// words (tag | a) and (tag | b), tagged with the call's epoch (fr_device.h):
// nothing is cleared between calls. The last workgroup advances the epoch at
// its end. A workspace that fr_ln_team_init has not prepared (no mark), or
// whose epoch has run out, trusts no slot: every partner's sums are then
// computed from x and dy, which gives the same bits, only slower.
constexpr int kLnTeamT = 1024;
constexpr int kLnTeamW = kLnTeamT / kWave;
constexpr uint64_t kLnWsMagic = 0x464C4E424B574D4Bull;

// Workspace initialization: zeros everywhere (no slot carries a tag), epoch
// 0, the mark.
__global__ __launch_bounds__(256) void fr_ln_team_init(uint32_t* __restrict__ ws, int64_t nwords) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nwords)
        ws[i] = i == kHdrMagic ? (uint32_t)kLnWsMagic : (i == kHdrMagic + 1 ? (uint32_t)(kLnWsMagic >> 32) : 0u);
}

// this lane's contribution to the two sums of one part of a row
__device__ __forceinline__ void ln_lane_sums(u32x4 xv, u32x4 dv, u32x4 gv, float mu, float rs, float& a, float& b) {
    a = 0.f;
    b = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float xh = (lane8(xv, e) - mu) * rs;
        const float g = lane8(dv, e) * lane8(gv, e);
        a += g;
        b += g * xh;
    }
}

// N values reduced over the workgroup: wave butterflies, then the waves in
// order through f[kLnTeamW][N]; every thread returns the N totals
template <int N>
__device__ __forceinline__ void ln_fold(float (&v)[N], float (*f)[N]) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = group_reduce<kWave>(v[k], OpSum());
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (lane == 0)
#pragma unroll
        for (int k = 0; k < N; ++k) f[w][k] = v[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        float r = f[0][k];
#pragma unroll
        for (int u = 1; u < kLnTeamW; ++u) r += f[u][k];
        v[k] = r;
    }
}

template <int P, int R, int DL, bool DG>
__global__ __launch_bounds__(kLnTeamT) void fr_team_layernorm_bwd_bf16(
    const uint16_t* x, const uint16_t* dy, const uint16_t* __restrict__ gamma, const float* __restrict__ mean,
    const float* __restrict__ rstd, uint16_t* dx, float* __restrict__ part, uint32_t* hdr, uint64_t* slots, int rows,
    int cols, int W, int64_t x_rs, int64_t dy_rs, int64_t dx_rs, int64_t ldw, int64_t wait_ticks) {
    constexpr int NB = DL + 1;
    static_assert(P * R <= kWave, "one polling lane per (part, row)");
    // workgroup folds: step s uses set s & 1 (two folds run back to back with
    // only their own barrier between them at the pipeline's start); a
    // recomputed partner sum uses sfb. Each value is reduced on its own, so
    // a sum folded alone has the bits it has when folded with others.
    __shared__ float sf[2][kLnTeamW][2 * R];
    __shared__ float sfb[kLnTeamW][2];
    // the member's own sums of each step in flight, by register buffer
    __shared__ float own[NB][2 * R];
    // exchange results by step parity: a step's writes are separated from
    // the reads two steps earlier by the barrier of the step between
    __shared__ float ex[2][P][2 * R];
    __shared__ uint32_t s_miss[2];
    const int tid = threadIdx.x;
    // this call's tag, the same in every thread (0: no slot is trusted, none
    // is written); thread 0 acknowledges it in the workgroup's flag
    uint32_t* flags = hdr + kLnTeamHeaderFlags;
    const uint64_t magic = __hip_atomic_load(reinterpret_cast<const uint64_t*>(hdr + kHdrMagic), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t epoch = __hip_atomic_load(hdr + kHdrEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tag =
        __builtin_amdgcn_readfirstlane(magic == kLnWsMagic && epoch < kMaxEpoch ? epoch + 1 : 0u);
    if (tid == 0 && tag != 0u) __hip_atomic_store(&flags[blockIdx.x], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int K = gridDim.x / P;
    // a team's members on one XCD (workgroup b runs on XCD b mod 8): when
    // the grid allows, members are the XCD's consecutive workgroups
    const bool xcd = gridDim.x % (8 * P) == 0;
    const int slot = blockIdx.x / 8;
    const int team = xcd ? (slot / P) * 8 + (int)(blockIdx.x % 8) : blockIdx.x / P;
    const int p = xcd ? slot % P : blockIdx.x % P;
    const int c0 = p * W;
    const uint32_t pbytes = (uint32_t)min(W, cols - c0) * 2u;
    const int voff = tid * 16;
    const int n = team < rows ? (rows - 1 - team) / K + 1 : 0;  // rows of this team
    const int ns = (n + R - 1) / R;                               // steps
    const float fn = (float)cols;
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    auto gamma_of = [&](int q) __attribute__((always_inline)) {
        return gamma ? __builtin_amdgcn_raw_buffer_load_b128(
                           row_rsrc(gamma + q * W, (uint32_t)min(W, cols - q * W) * 2u), voff, 0, 0)
                     : ones;
    };
    const u32x4 gv = gamma_of(p);
    u32x4 xb[NB][R], db[NB][R];
    float mub[NB][R], rsb[NB][R];
    float ag[8], ab[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[e] = ab[e] = 0.f;

    // Every step issues the same memory instructions whether or not its rows
    // exist (a row past the team's end loads and stores through an empty
    // range: zeros, no memory access), and no memory instruction of the
    // common path sits under a branch, so the compiler's waits for older
    // loads count the newer ones exactly instead of waiting for all of them
    // (the rare paths drain the counter before they rejoin).
    auto load = [&](int st, int bi) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const int i = st * R + t;
            const bool live = i < n;
            const int r = team + (live ? i : 0) * K;  // n >= 1: row `team` exists
            const uint32_t nb = live ? pbytes : 0u;
            xb[bi][t] =
                __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(x + (int64_t)r * x_rs + c0, nb), voff, 0, kAuxNT);
            db[bi][t] =
                __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(dy + (int64_t)r * dy_rs + c0, nb), voff, 0, kAuxNT);
            mub[bi][t] = live ? mean[r] : 0.f;
            rsb[bi][t] = live ? rstd[r] : 0.f;
        }
    };
    auto sums = [&](int st, int bi) __attribute__((always_inline)) {
        float v[2 * R];
#pragma unroll
        for (int t = 0; t < R; ++t) ln_lane_sums(xb[bi][t], db[bi][t], gv, mub[bi][t], rsb[bi][t], v[2 * t], v[2 * t + 1]);
        // finish unpacks the rows again rather than keeping fp32 copies of
        // them alive across the steps between
#pragma unroll
        for (int t = 0; t < R; ++t) {
            hide(xb[bi][t]);
            hide(db[bi][t]);
        }
        ln_fold<2 * R>(v, sf[st & 1]);
#pragma unroll
        for (int t = 0; t < R; ++t) {
            if (tid == 0) {
                own[bi][2 * t] = v[2 * t];
                own[bi][2 * t + 1] = v[2 * t + 1];
            }
            // one store instruction for every lane, no branch: the slot's
            // range admits lanes 0 and 1 (its two words); the others, and
            // every lane for a row past the team's end, fall outside it and
            // write nothing. sc1: visible to the other compute dies.
            const int i = st * R + t;
            const int r = team + i * K;
            const uint64_t word = slot_word(tag, tid & 1 ? v[2 * t + 1] : v[2 * t]);
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{(uint32_t)word, (uint32_t)(word >> 32)},
                __builtin_amdgcn_make_buffer_rsrc(slots + 2 * ((int64_t)(i < n ? r : 0) * P + p), 0,
                                                  i < n && tag != 0u ? 16 : 0, kBufferRsrcWord3),
                min(tid, 2) * 8, 0, kAuxSc1);
        }
    };
    // wave 0, lane l = q + P t < P R: the slot of part q of row t of the
    // step. Partners' words are loaded one step ahead.
    const int lq = tid % P, lt = tid / P;
    // One load instruction for every lane of every wave, no branch: lane
    // q + P t < P R reads slot (row t of the step, part q); the others point
    // past the slots' range and read zeros without a memory access. The
    // words are looked at only in the next finish.
    const int slot_bytes = rows * P * 16;  // < 2^31 (the planner's bound)
    const __amdgpu_buffer_rsrc_t rslots = __builtin_amdgcn_make_buffer_rsrc(slots, 0, slot_bytes, kBufferRsrcWord3);
    uint64_t pw0 = ~0ull, pw1 = ~0ull;
    auto poll_ahead = [&](int st) __attribute__((always_inline)) {
        const int i = st * R + lt;
        const bool use = tid < P * R && i < n;
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            rslots, use ? ((team + i * K) * P + lq) * 16 : slot_bytes, 0, kAuxSc1);
        pw0 = ((uint64_t)w.y << 32) | w.x;
        pw1 = ((uint64_t)w.w << 32) | w.z;
    };
    auto finish = [&](int st, int bi) __attribute__((always_inline)) {
        float(*e)[2 * R] = ex[st & 1];
        if (tid < kWave) {
            const int i = st * R + lt;
            uint64_t w0 = pw0, w1 = pw1;
            // own part and rows past the team's end need no slot; with no
            // wait (wait_ticks < 0), or no tag, every partner's sums are
            // recomputed
            const bool need = tid < P * R && i < n && lq != p;
            const bool trust = wait_ticks >= 0 && tag != 0u;
            bool ok = !need || (trust && published(w0, tag) && published(w1, tag));
            const uint64_t* ws = slots + 2 * ((int64_t)(team + i * K) * P + lq);
            if (!__all(ok) && trust) {  // else read no partner's slot (all are recomputed)
                const uint64_t t0 = wall_clock64();
                for (;;) {
                    if ((int64_t)(wall_clock64() - t0) >= wait_ticks) break;
                    __builtin_amdgcn_s_sleep(2);
                    if (!ok) {
                        if (!published(w0, tag))
                            w0 = __hip_atomic_load(&ws[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (!published(w1, tag))
                            w1 = __hip_atomic_load(&ws[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = published(w0, tag) && published(w1, tag);
                    }
                    if (__all(ok)) break;
                }
            }
            const uint64_t miss = __ballot(!ok);
            if (tid < P * R && lq != p && i < n && ok) {
                e[lq][2 * lt] = __builtin_bit_cast(float, (uint32_t)w0);
                e[lq][2 * lt + 1] = __builtin_bit_cast(float, (uint32_t)w1);
            }
            if (tid == 0) s_miss[st & 1] = (uint32_t)miss;
        }
        __syncthreads();
        const uint32_t miss = s_miss[st & 1];
#pragma unroll
        for (int l = 0; l < P * R; ++l) {
            if (!(miss >> l & 1u)) continue;  // rare: a partner has not published in time
            const int q = l % P, t = l / P;
            const int r = team + (st * R + t) * K;
            const uint32_t qb = (uint32_t)min(W, cols - q * W) * 2u;
            const u32x4 xq =
                __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(x + (int64_t)r * x_rs + q * W, qb), voff, 0, 0);
            const u32x4 dq =
                __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(dy + (int64_t)r * dy_rs + q * W, qb), voff, 0, 0);
            float v[2];
            ln_lane_sums(xq, dq, gamma_of(q), mub[bi][t], rsb[bi][t], v[0], v[1]);
            ln_fold<2>(v, sfb);
            if (tid == 0) {
                e[q][2 * t] = v[0];
                e[q][2 * t + 1] = v[1];
                __hip_atomic_fetch_add(&hdr[kHdrRecomputed], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
            // a row past the team's end (last step) holds zeros: it adds
            // nothing to the column sums and its store has an empty range
            const int i = st * R + t;
            const bool live = i < n;
            const int r = team + (live ? i : 0) * K;
            // part order; the member's own sums from its own slots
            float a = p == 0 ? own[bi][2 * t] : e[0][2 * t], b = p == 0 ? own[bi][2 * t + 1] : e[0][2 * t + 1];
#pragma unroll
            for (int q = 1; q < P; ++q) {
                a += q == p ? own[bi][2 * t] : e[q][2 * t];
                b += q == p ? own[bi][2 * t + 1] : e[q][2 * t + 1];
            }
            const float m1 = a / fn, m2 = b / fn, mu = mub[bi][t], rs = rsb[bi][t];
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float vv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int el = 2 * k + h;
                    const float d = lane8(db[bi][t], el);
                    const float xh = (lane8(xb[bi][t], el) - mu) * rs;
                    const float g = d * lane8(gv, el);
                    vv[h] = rs * ((g - m1) - xh * m2);
                    if constexpr (DG) {
                        ag[el] += d * xh;
                        ab[el] += d;
                    }
                }
                o[k] = pack_bf16(vv[0], vv[1]);
            }
            store16<kAuxNT>(u32x4{o[0], o[1], o[2], o[3]}, row_rsrc(dx + (int64_t)r * dx_rs + c0, live ? pbytes : 0u),
                            voff);
        }
        poll_ahead(st + 1);
    };

#pragma unroll
    for (int u = 0; u < DL; ++u) load(u, u);
#pragma unroll
    for (int u = 0; u < DL - 1; ++u) sums(u, u);
    poll_ahead(0);
    for (int s0 = 0; s0 < ns; s0 += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int st = s0 + u;
            if (st >= ns) break;
            load(st + DL, (u + DL) % NB);
            sums(st + DL - 1, (u + DL - 1) % NB);
            finish(st, u);
        }
    }
    if constexpr (DG) {
        if (tid * 8 < (int)(pbytes / 2)) {
            float* pg = part + (int64_t)team * ldw + c0 + tid * 8;
            float* pbp = part + ((int64_t)K + team) * ldw + c0 + tid * 8;
            st4<false>(pg, f32x4{ag[0], ag[1], ag[2], ag[3]});
            st4<false>(pg + 4, f32x4{ag[4], ag[5], ag[6], ag[7]});
            st4<false>(pbp, f32x4{ab[0], ab[1], ab[2], ab[3]});
            st4<false>(pbp + 4, f32x4{ab[4], ab[5], ab[6], ab[7]});
        }
    }
    if (blockIdx.x == gridDim.x - 1 && tag != 0u) epoch_advance<kLnTeamT>(hdr, flags, tag, epoch);
}

// dgamma[j] = sum_g ws[0][g][j], dbeta[j] = sum_g ws[1][g][j]: 256 threads as
// Q column quads x S slices; slice s sums partials g = s, s + S, ... in
// order, then slice 0 adds the slices in order. Every run gives the same bits.
// With hdr (the persistent form's call), thread 0 of workgroup 0 also
// clears the workspace's initialization mark: the partial rows went to the
// bytes that the split form's slots use, so no slot may be trusted until
// the workspace is initialized again.
template <int Q, int S>
__global__ __launch_bounds__(Q * S) void fr_layernorm_bwd_fin(const float* __restrict__ ws, float* __restrict__ dgamma,
                                                              float* __restrict__ dbeta, int G, int cols,
                                                              int64_t ldw, uint32_t* __restrict__ hdr) {
    if (hdr && blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[kHdrMagic] = 0u;
        hdr[kHdrMagic + 1] = 0u;
    }
    __shared__ f32x4 sg[S][Q];
    __shared__ f32x4 sb[S][Q];
    const int q = threadIdx.x % Q, sl = threadIdx.x / Q;
    const int j = (blockIdx.x * Q + q) * 4;
    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, ab = {0.f, 0.f, 0.f, 0.f};
    if (j < cols) {
#pragma unroll 8
        for (int g = sl; g < G; g += S) {
            ag += ld4<true>(ws + (int64_t)g * ldw + j);
            ab += ld4<true>(ws + ((int64_t)G + g) * ldw + j);
        }
    }
    sg[sl][q] = ag;
    sb[sl][q] = ab;
    __syncthreads();
    if (sl == 0 && j < cols) {
#pragma unroll
        for (int t = 1; t < S; ++t) {
            ag += sg[t][q];
            ab += sb[t][q];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (j + c < cols) {
                if (dgamma) dgamma[j + c] = ag[c];
                if (dbeta) dbeta[j + c] = ab[c];
            }
    }
}

// ------------------------------------------------------------------ launchers
namespace {

using LnFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int64_t, int64_t,
                      float, float*, float*);

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

// Pipelined rows: 512 threads x 8 vectors (32768 columns), 3 rows in flight.
// Measured at 2048 x 32768 on MI355X: 3 rows in flight 44.9 us, 2 rows
// 46.9 us, 4 rows 47.2 us; 1024 threads x 4 vectors with 3 or 4 rows 46.8 /
// 47.2 us; 256 threads x 16 vectors with 2 rows 49.8 us (the kernel above:
// 48.8 us on the same box).
constexpr int kLnPipeR = 3;
template <bool STATS>
LnFn pick_pipe_s(int nr) {
    constexpr int R = kLnPipeR;
    switch (nr) {
        case 3: return fr_pipe_layernorm_bf16<512, 8, R, 3, STATS>;
        case 4: return fr_pipe_layernorm_bf16<512, 8, R, 4, STATS>;
        case 5: return fr_pipe_layernorm_bf16<512, 8, R, 5, STATS>;
        case 6: return fr_pipe_layernorm_bf16<512, 8, R, 6, STATS>;
        case 7: return fr_pipe_layernorm_bf16<512, 8, R, 7, STATS>;
        case 8: return fr_pipe_layernorm_bf16<512, 8, R, 8, STATS>;
    }
    return nullptr;
}
LnFn pick_pipe(int threads, int nv, int nr, bool stats) {
    if (threads != 512 || nv != 8) return nullptr;
    return stats ? pick_pipe_s<true>(nr) : pick_pipe_s<false>(nr);
}

template <bool VEC>
LnFn pick_red(int threads, int u) {
    if (threads == 256 && u == 4) return fr_red_layernorm_bf16<256, 4, VEC>;
    if (threads == 512 && u == 2) return fr_red_layernorm_bf16<512, 2, VEC>;
    if (threads == 1024 && u == 2) return fr_red_layernorm_bf16<1024, 2, VEC>;
    return nullptr;
}

using LnBwdFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*, uint16_t*,
                         float*, int, int, int64_t, int64_t, int64_t, int64_t);

template <int M, bool DG>
LnBwdFn pick_bwd_m(int threads, int nv) {
    // element accesses with 4 vectors per lane and column partials need more
    // than the 128 registers a 1024-thread workgroup allows: not compiled
    if constexpr (M != kScalar || !DG)
        if (threads == 1024 && nv == 4) return fr_per_layernorm_bwd_bf16<1024, 4, M, DG>;
    switch (threads * 16 + nv) {
        case 128 * 16 + 1: return fr_per_layernorm_bwd_bf16<128, 1, M, DG>;
        case 256 * 16 + 1: return fr_per_layernorm_bwd_bf16<256, 1, M, DG>;
        case 256 * 16 + 2: return fr_per_layernorm_bwd_bf16<256, 2, M, DG>;
        case 256 * 16 + 4: return fr_per_layernorm_bwd_bf16<256, 4, M, DG>;
        case 512 * 16 + 1: return fr_per_layernorm_bwd_bf16<512, 1, M, DG>;
        case 512 * 16 + 2: return fr_per_layernorm_bwd_bf16<512, 2, M, DG>;
        case 512 * 16 + 4: return fr_per_layernorm_bwd_bf16<512, 4, M, DG>;
        case 1024 * 16 + 1: return fr_per_layernorm_bwd_bf16<1024, 1, M, DG>;
        case 1024 * 16 + 2: return fr_per_layernorm_bwd_bf16<1024, 2, M, DG>;
    }
    return nullptr;
}

template <bool DG>
LnBwdFn pick_bwd(int mask, int threads, int nv) {
    switch (mask) {
        case kNone: return pick_bwd_m<kNone, DG>(threads, nv);
        case kVec: return pick_bwd_m<kVec, DG>(threads, nv);
        default: return pick_bwd_m<kScalar, DG>(threads, nv);
    }
}

}  // namespace

namespace {
using LnTeamFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*, uint16_t*,
                         float*, uint32_t*, uint64_t*, int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t);

// Split-row pipeline: DL = 3 rows loaded ahead, R = 1 row per step
// (measured at 2048 x 32768: DL 2 / 3 / 4 gave 87.4 / 85.9 / 89.1 us; R = 2
// spills). The finishing kernel for the team partials: 32 column quads x
// 8 slices (5 us for 64 partial rows; 8 x 32 took 8.4 us).
constexpr int kLnTeamDL = 3, kLnTeamR = 1, kLnTeamFinQ = 32;
template <bool DG>
LnTeamFn pick_team(int parts) {
    constexpr int DL = kLnTeamDL, R = kLnTeamR;
    switch (parts) {
        case 2: return fr_team_layernorm_bwd_bf16<2, R, DL, DG>;
        case 3: return fr_team_layernorm_bwd_bf16<3, R, DL, DG>;
        case 4: return fr_team_layernorm_bwd_bf16<4, R, DL, DG>;
    }
    return nullptr;
}
}  // namespace

hipError_t launch_layernorm_bwd(const fr_plan& p, const LayerNormBwdArgs& a, hipStream_t s) {
    const bool vec = p.vec16 != 0;
    const bool dg = a.dgamma || a.dbeta;
    constexpr int Q = 8, S = 32;
    const int64_t ldw = ln_bwd_ldw(a.cols);
    const int64_t grid2 = (a.cols + 4 * Q - 1) / (4 * Q);
    if (p.form == FR_FORM_SPLIT) {
        // the team kernel (its slots are epoch-tagged: no clearing), then
        // the column sums
        const int parts = p.splits;
        LnTeamFn f = dg ? pick_team<true>(parts) : pick_team<false>(parts);
        if (!f || !vec || a.rows < 1 || p.grid % parts || p.grid > kLnTeamMaxGrid)
            return hipErrorInvalidDeviceFunction;
        char* base = reinterpret_cast<char*>(a.ws);
        uint32_t* hdr = reinterpret_cast<uint32_t*>(base);
        u32x4* slots = reinterpret_cast<u32x4*>(base + kLnTeamHeader);
        float* part = reinterpret_cast<float*>(base + kLnTeamHeader + ln_team_slots_bytes(a.rows, parts));
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(kLnTeamT), 0, s, a.x, a.dy, a.gamma, a.mean, a.rstd, a.dx,
                           part, hdr, reinterpret_cast<uint64_t*>(slots), a.rows, a.cols, p.chunk, a.x_rs, a.dy_rs,
                           a.dx_rs, ldw, a.wait_ticks);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !dg) return e;
        constexpr int TQ = kLnTeamFinQ, TS = 256 / TQ;
        hipLaunchKernelGGL((fr_layernorm_bwd_fin<TQ, TS>), dim3((unsigned)((a.cols + 4 * TQ - 1) / (4 * TQ))),
                           dim3(256), 0, s, part, a.dgamma, a.dbeta, (int)(p.grid / parts), a.cols, ldw, nullptr);
        return hipGetLastError();
    }
    const int mask = !vec ? kScalar : (a.cols == 8 * p.threads * p.vec ? kNone : kVec);
    LnBwdFn f = p.form == FR_FORM_PER ? (dg ? pick_bwd<true>(mask, p.threads, p.vec)
                                             : pick_bwd<false>(mask, p.threads, p.vec))
                                      : nullptr;
    if (!f) return hipErrorInvalidDeviceFunction;
    // the partial rows start after the split form's header, which the
    // finishing kernel marks uninitialized (the split form's slots may now
    // hold partial-row bytes); with no rows nothing is written there
    const bool rows_part = dg && a.rows > 0;
    float* part = rows_part ? a.ws + kLnTeamHeader / 4 : nullptr;
    if (a.rows > 0) {
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.dy, a.gamma, a.mean, a.rstd,
                           a.dx, part, a.rows, a.cols, a.x_rs, a.dy_rs, a.dx_rs, ldw);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!dg) return hipSuccess;
    hipLaunchKernelGGL((fr_layernorm_bwd_fin<Q, S>), dim3((unsigned)grid2), dim3(Q * S), 0, s, part, a.dgamma,
                       a.dbeta, (int)p.grid, a.cols, ldw, rows_part ? reinterpret_cast<uint32_t*>(a.ws) : nullptr);
    return hipGetLastError();
}

hipError_t launch_layernorm_bwd_ws_init(void* ws, uint64_t ws_bytes, hipStream_t s) {
    const int64_t nwords = (int64_t)(ws_bytes / 4);
    hipLaunchKernelGGL(fr_ln_team_init, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(ws), nwords);
    return hipGetLastError();
}

hipError_t launch_layernorm(const fr_plan& p, const LayerNormArgs& a, hipStream_t s) {
    const bool vec = p.vec16 != 0;
    LnFn f = nullptr;
    if (p.form == FR_FORM_PER && p.rows_per_wg > 1) {
        // pipelined rows: 16-byte accesses over rows that fill the capacity
        if (vec && a.cols == 8 * p.threads * p.vec)
            f = pick_pipe(p.threads, p.vec, p.rows_per_wg, a.mean != nullptr || a.rstd != nullptr);
    } else if (p.form == FR_FORM_PER) {
        const int mask = !vec ? kScalar : (a.cols == 8 * p.threads * p.vec ? kNone : kVec);
        f = pick_per(mask, p.threads, p.vec, p.occupancy, a.gamma == nullptr);
    }
    else if (p.form == FR_FORM_RED)
        f = vec ? pick_red<true>(p.threads, p.vec) : pick_red<false>(p.threads, p.vec);
    if (!f) return hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.gamma, a.beta, a.y, a.rows, a.cols,
                       a.x_rs, a.y_rs, a.eps, a.mean, a.rstd);
    return hipGetLastError();
}

}  // namespace fr
