// fr_softmax.hip - row softmax with fused max / sum-of-exponentials
// reductions ("Stax (4): GPU Codegen and Dynamic Shapes", 9.5), optional
// ragged runtime row lengths (10.3: bounds are runtime values, masks stay)
// and optional argmax.
//   persistent  fr_per_softmax_f32      the row lives in a lane group's
//                                       registers: max, exp, sum, scale; one
//                                       read and one write per element
//                                       (Listing 9.5; two passes over
//                                       registers, as 9.5 notes for short rows)
//   looped      fr_red_softmax_f32      one workgroup streams the row with
//                                       the online (m, d) rescaling (9.5, the
//                                       merge; hello-gpu Chapter 12, 12.3),
//                                       then a normalizing pass
//   split       fr_split_softmax_part + fr_split_softmax_fin
//                                       chunks of long rows on separate
//                                       workgroups; per-chunk (m, d, argmax)
//                                       partials merged in chunk order
//                                       (Proposition 9.1: any segmentation)
// Masked lanes take the identity of each reduction: -inf for the max, 0 for
// the sum (9.5, Listing 9.5), never 0 for the max.
#include <limits.h>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

__device__ __forceinline__ int row_len(const int32_t* __restrict__ lengths, int r, int cols) {
    if (!lengths) return cols;
    int L = lengths[r];
    return L < 0 ? 0 : (L > cols ? cols : L);
}

// Element c of a 4-vector.
__device__ __forceinline__ float comp(f32x4 v, int c) { return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w)); }

// Does x match the row maximum m (a NaN maximum matches the first NaN)?
__device__ __forceinline__ bool is_max(float x, float m) { return x == m || (m != m && x != x); }

__device__ __forceinline__ float max4(float m, f32x4 v) { return fmax_nan(fmax_nan(m, fmax_nan(v.x, v.y)), fmax_nan(v.z, v.w)); }

// e^(v - m) for the elements j0..j0+3 below L, 0 elsewhere.
__device__ __forceinline__ f32x4 exp4_masked(f32x4 v, float m, int j0, int L) {
    return f32x4{j0 + 0 < L ? exp_fast(v.x - m) : 0.f, j0 + 1 < L ? exp_fast(v.y - m) : 0.f,
                 j0 + 2 < L ? exp_fast(v.z - m) : 0.f, j0 + 3 < L ? exp_fast(v.w - m) : 0.f};
}

__device__ __forceinline__ f32x4 exp4(f32x4 v, float m) {
    return f32x4{exp_fast(v.x - m), exp_fast(v.y - m), exp_fast(v.z - m), exp_fast(v.w - m)};
}

// ------------------------------------------------------------------ persistent
// SEG lanes per row and NV 16-byte vectors per lane (row capacity 4*SEG*NV);
// each lane group takes RPW adjacent rows and issues all their loads before
// any arithmetic, so RPW * NV loads per lane are in flight at once. A
// 256-thread workgroup serves 256 / SEG * RPW rows per step of a grid-stride
// loop over row groups. M is the masking mode (kNone: dense rows that fill
// the capacity exactly).
template <int SEG, int NV, int M, int RPW>
__global__ __launch_bounds__(256) void fr_per_softmax_f32(const float* x, float* y, int rows, int cols,
                                                          int64_t x_rs, int64_t y_rs,
                                                          const int32_t* __restrict__ lengths,
                                                          int32_t* __restrict__ argmax) {
    constexpr int RPB = 256 / SEG * RPW;
    const int g = threadIdx.x / SEG;
    const int l = threadIdx.x % SEG;
    const int ngroups = (rows + RPB - 1) / RPB;
    for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        f32x4 v[RPW][NV];
        int L[RPW];
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            const int r = grp * RPB + g * RPW + q;
            const bool live = r < rows;
            // kNone (dense rows, no lengths): a row past the end re-reads the
            // last row, which is in bounds, and stores nothing - so the loads
            // carry no branch
            const int rl = live ? r : (M == kNone ? rows - 1 : 0);
            if constexpr (M == kNone) L[q] = live ? cols : 0;
            else L[q] = live ? row_len(lengths, r, cols) : 0;
            const float* xr = x + (int64_t)rl * x_rs;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int j0 = (k * SEG + l) * 4;
                if constexpr (M == kNone) v[q][k] = ld4<true>(xr + j0);
                else v[q][k] = load4m<M, true>(xr, j0, L[q], -INFINITY);
            }
        }
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            const int r = grp * RPB + g * RPW + q;
            const bool live = r < rows;
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < NV; ++k) m = max4(m, v[q][k]);
            m = group_reduce<SEG>(m, OpMax());
            if (argmax) {
                int cand = INT_MAX;
#pragma unroll
                for (int k = NV - 1; k >= 0; --k)
#pragma unroll
                    for (int c = 3; c >= 0; --c) {
                        const int j = (k * SEG + l) * 4 + c;
                        if (j < L[q] && is_max(comp(v[q][k], c), m)) cand = j;
                    }
                cand = group_reduce<SEG>(cand, OpMinI());
                if (live && l == 0) argmax[r] = L[q] > 0 ? cand : -1;
            }
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                v[q][k] = M == kNone ? exp4(v[q][k], m) : exp4_masked(v[q][k], m, (k * SEG + l) * 4, L[q]);
                s += (v[q][k].x + v[q][k].y) + (v[q][k].z + v[q][k].w);
            }
            s = group_reduce<SEG>(s, OpSum());
            const float inv = 1.0f / s;  // one correctly rounded division per row
            float* yr = y + (int64_t)(live ? r : 0) * y_rs;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int j0 = (k * SEG + l) * 4;
                if constexpr (M == kNone) {
                    if (live) st4<true>(yr + j0, v[q][k] * inv);
                } else {
                    store4m<M, true>(yr, j0, L[q], v[q][k] * inv);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ looped (online)
// One workgroup of T threads per row. Pass 1 keeps a per-lane (m, d) state:
// for each step of U vectors it takes the step maximum m', rescales the old
// sum by e^(m - m') and adds the new terms e^(x - m') - the online update of
// hello-gpu Chapter 12, 12.3, one rescale per step rather than per element.
// The lane states are merged with the (m, d) monoid. Pass 2 re-reads the row,
// writes e^(x - M) / D and finds the first index of the maximum. Steps wholly
// inside the row run unmasked; only the last step of a row is masked.
template <int M, int T, int U>
__device__ __forceinline__ MD online_step(const float* xr, int base, int L, MD st) {
    const int tid = threadIdx.x;
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load4m<M, false>(xr, base + (u * T + tid) * 4, L, -INFINITY);
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) cm = max4(cm, v[u]);
    const float mx = fmax_nan(st.m, cm);
    float add = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const f32x4 e = M == kNone ? exp4(v[u], mx) : exp4_masked(v[u], mx, base + (u * T + tid) * 4, L);
            add += (e.x + e.y) + (e.z + e.w);
        }
    }
    const float scale = st.m == -INFINITY ? 0.f : exp_fast(st.m - mx);
    return MD{mx, st.d * scale + add};
}

template <int M, int T, int U>
__device__ __forceinline__ int normalize_step(const float* xr, float* yr, int base, int L, float mx, float inv,
                                              bool want_argmax, int cand) {
    const int tid = threadIdx.x;
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load4m<M, true>(xr, base + (u * T + tid) * 4, L, -INFINITY);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j0 = base + (u * T + tid) * 4;
        if (want_argmax && cand == INT_MAX) {
            for (int c = 0; c < 4; ++c)
                if (j0 + c < L && cand == INT_MAX && is_max(comp(v[u], c), mx)) cand = j0 + c;
        }
        store4m<M, true>(yr, j0, L, exp4(v[u], mx) * inv);
    }
    return cand;
}

template <int T, int U, bool VEC>
__global__ __launch_bounds__(T) void fr_red_softmax_f32(const float* x, float* y, int rows, int cols,
                                                        int64_t x_rs, int64_t y_rs,
                                                        const int32_t* __restrict__ lengths,
                                                        int32_t* __restrict__ argmax) {
    constexpr int STEP = T * 4 * U;
    __shared__ MD sl_md[T / kWave];
    __shared__ int sl_i[T / kWave];
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const int L = row_len(lengths, r, cols);
        const int full = L - L % STEP;
        const float* xr = x + (int64_t)r * x_rs;
        MD st{-INFINITY, 0.f};
        int base = 0;
        for (; base < full; base += STEP) st = online_step<body_mask<VEC>(), T, U>(xr, base, L, st);
        if (base < L) st = online_step<tail_mask<VEC>(), T, U>(xr, base, L, st);
        st = group_reduce<kWave>(st, OpMD());
        st = block_fold(st, sl_md, T / kWave, OpMD());
        const float inv = 1.0f / st.d;
        float* yr = y + (int64_t)r * y_rs;
        const bool want = argmax != nullptr;
        int cand = INT_MAX;
        for (base = 0; base < full; base += STEP)
            cand = normalize_step<body_mask<VEC>(), T, U>(xr, yr, base, L, st.m, inv, want, cand);
        if (base < L) cand = normalize_step<tail_mask<VEC>(), T, U>(xr, yr, base, L, st.m, inv, want, cand);
        if (want) {
            cand = group_reduce<kWave>(cand, OpMinI());
            cand = block_fold(cand, sl_i, T / kWave, OpMinI());
            if (threadIdx.x == 0) argmax[r] = L > 0 ? cand : -1;
        }
        __syncthreads();  // slots are rewritten by the next row
    }
}

// ------------------------------------------------------------------ split
// Chunk c of row r (workgroup r * S + c) covers [c * C, min(len_r, (c+1) * C))
// with C = 4 * T * NV. Part 1 keeps the chunk in registers and writes its
// partial (m, d, first index of m). Part 2 merges the row's partials in chunk
// order, writes the argmax (chunk 0) and the normalized chunk. A chunk wholly
// inside its row is loaded without masks.
template <int M, int T, int NV>
__device__ __forceinline__ void part_body(const float* xr, int start, int end, SoftmaxPartial* out, float* sl_m,
                                          float* sl_d, int* sl_i) {
    const int tid = threadIdx.x;
    f32x4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load4m<M, false>(xr, start + (k * T + tid) * 4, end, -INFINITY);
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NV; ++k) m = max4(m, v[k]);
    m = group_reduce<kWave>(m, OpMax());
    m = block_fold(m, sl_m, T / kWave, OpMax());
    int cand = INT_MAX;
    float s = 0.f;
#pragma unroll
    for (int k = NV - 1; k >= 0; --k)
#pragma unroll
        for (int c = 3; c >= 0; --c) {
            const int j = start + (k * T + tid) * 4 + c;
            if (j < end && is_max(comp(v[k], c), m)) cand = j;
        }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const f32x4 e = M == kNone ? exp4(v[k], m) : exp4_masked(v[k], m, start + (k * T + tid) * 4, end);
        s += (e.x + e.y) + (e.z + e.w);
    }
    cand = group_reduce<kWave>(cand, OpMinI());
    cand = block_fold(cand, sl_i, T / kWave, OpMinI());
    s = group_reduce<kWave>(s, OpSum());
    s = block_fold(s, sl_d, T / kWave, OpSum());
    if (tid == 0) *out = SoftmaxPartial{m, s, cand, 0};
}

template <int T, int NV, bool VEC>
__global__ __launch_bounds__(T) void fr_split_softmax_part(const float* __restrict__ x, int rows, int cols,
                                                           int64_t x_rs, const int32_t* __restrict__ lengths,
                                                           SoftmaxPartial* __restrict__ ws, int S) {
    constexpr int C = 4 * T * NV;
    __shared__ float sl_m[T / kWave];
    __shared__ float sl_d[T / kWave];
    __shared__ int sl_i[T / kWave];
    const int64_t w = blockIdx.x;
    const int r = (int)(w / S);
    const int c = (int)(w % S);
    if (r >= rows) return;
    const int L = row_len(lengths, r, cols);
    const int start = c * C;
    if (start >= L) return;
    const int end = min(L, start + C);
    const float* xr = x + (int64_t)r * x_rs;
    if (end - start == C) part_body<body_mask<VEC>(), T, NV>(xr, start, end, ws + w, sl_m, sl_d, sl_i);
    else part_body<tail_mask<VEC>(), T, NV>(xr, start, end, ws + w, sl_m, sl_d, sl_i);
}

template <int M, int T, int NV>
__device__ __forceinline__ void fin_body(const float* xr, float* yr, int start, int end, float mx, float inv) {
    const int tid = threadIdx.x;
    f32x4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load4m<M, true>(xr, start + (k * T + tid) * 4, end, -INFINITY);
#pragma unroll
    for (int k = 0; k < NV; ++k) store4m<M, true>(yr, start + (k * T + tid) * 4, end, exp4(v[k], mx) * inv);
}

template <int T, int NV, bool VEC>
__global__ __launch_bounds__(T) void fr_split_softmax_fin(const float* x, float* y, int rows, int cols,
                                                          int64_t x_rs, int64_t y_rs,
                                                          const int32_t* __restrict__ lengths,
                                                          int32_t* __restrict__ argmax,
                                                          const SoftmaxPartial* __restrict__ ws, int S) {
    constexpr int C = 4 * T * NV;
    const int64_t w = blockIdx.x;
    const int r = (int)(w / S);
    const int c = (int)(w % S);
    if (r >= rows) return;
    const int L = row_len(lengths, r, cols);
    const int start = c * C;
    if (start >= L) {
        if (c == 0 && argmax && threadIdx.x == 0) argmax[r] = -1;
        return;
    }
    const int end = min(L, start + C);
    const int nc = (L + C - 1) / C;
    MD st{-INFINITY, 0.f};
    MI best{-INFINITY, INT_MAX};
    const SoftmaxPartial* pr = ws + (int64_t)r * S;
    for (int k = 0; k < nc; ++k) {
        const SoftmaxPartial p = pr[k];
        st = md_combine(st, MD{p.m, p.d});
        best = mi_combine(best, MI{p.m, p.idx});
    }
    if (c == 0 && argmax && threadIdx.x == 0) argmax[r] = best.i;
    const float inv = 1.0f / st.d;
    const float* xr = x + (int64_t)r * x_rs;
    float* yr = y + (int64_t)r * y_rs;
    if (end - start == C) fin_body<body_mask<VEC>(), T, NV>(xr, yr, start, end, st.m, inv);
    else fin_body<tail_mask<VEC>(), T, NV>(xr, yr, start, end, st.m, inv);
}

// ------------------------------------------------------------------ split, single pass
// The two-kernel split above reads every chunk twice. Here each chunk is read
// once and kept in registers: workgroups claim chunks through an atomic
// ticket in row-major order, publish the chunk's partial (m, d, first index
// of m), wait until every chunk of the row has published, merge the row's
// partials in chunk order and normalize the registers they still hold.
//
// Progress: a claimed ticket always belongs to a running workgroup, and a
// workgroup publishes before it waits, so only the workgroups on the last
// partly-claimed row can wait on unclaimed chunks; with more resident
// workgroups than chunks per row (S <= 64 here) another workgroup claims
// them. The wait is bounded all the same: past the spin limit the workgroup
// stops waiting, poisons its chunk with NaN and raises the error word of the
// workspace header, so every wave always exits.
//
// Visibility across XCDs: partial fields are stored and loaded with
// agent-scope atomics, the row counter is incremented with release
// semantics and read back with an acquire fence.
constexpr int kFusedMaxSplits = 64;
constexpr int kSpinLimit = 1 << 20;

struct FusedWs {
    uint32_t* hdr;         // [0] ticket, [1] error
    uint32_t* row_cnt;     // rows counters of published chunks
    SoftmaxPartial* part;  // rows x S partials
};

__host__ __device__ inline FusedWs fused_layout(void* ws, int rows) {
    char* b = static_cast<char*>(ws);
    FusedWs f;
    f.hdr = reinterpret_cast<uint32_t*>(b);
    f.row_cnt = reinterpret_cast<uint32_t*>(b + 64);
    f.part = reinterpret_cast<SoftmaxPartial*>(b + 64 + ((int64_t)rows * 4 + 15) / 16 * 16);
    return f;
}

__global__ __launch_bounds__(256) void fr_split_softmax_prep(uint32_t* hdr, uint32_t* row_cnt, int rows) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < 16) hdr[i] = 0u;
    if (i < rows) row_cnt[i] = 0u;
}

template <int M, int T, int NV>
__device__ __forceinline__ void fused_load(const float* xr, int start, int end, f32x4* v) {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load4m<M, true>(xr, start + (k * T + (int)threadIdx.x) * 4, end, -INFINITY);
}

template <int M, int T, int NV>
__device__ __forceinline__ void fused_store(float* yr, int start, int end, const f32x4* v, float mx, float inv) {
#pragma unroll
    for (int k = 0; k < NV; ++k) store4m<M, true>(yr, start + (k * T + (int)threadIdx.x) * 4, end, exp4(v[k], mx) * inv);
}

template <int T, int NV, bool VEC>
__global__ __launch_bounds__(T) void fr_split_softmax_fused(const float* x, float* y, int rows, int cols,
                                                            int64_t x_rs, int64_t y_rs,
                                                            const int32_t* __restrict__ lengths,
                                                            int32_t* __restrict__ argmax, void* ws, int S) {
    constexpr int C = 4 * T * NV;
    __shared__ float sl_m[T / kWave];
    __shared__ float sl_d[T / kWave];
    __shared__ int sl_i[T / kWave];
    __shared__ uint32_t s_ticket;
    __shared__ float s_max, s_inv;
    __shared__ int s_timeout;
    const FusedWs f = fused_layout(ws, rows);
    const int tid = threadIdx.x;
    const uint32_t total = (uint32_t)rows * (uint32_t)S;
    for (;;) {
        if (tid == 0) s_ticket = __hip_atomic_fetch_add(&f.hdr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t t = s_ticket;
        __syncthreads();  // every thread has read the ticket before it is rewritten
        if (t >= total) break;
        const int r = (int)(t / (uint32_t)S);
        const int c = (int)(t % (uint32_t)S);
        const int L = row_len(lengths, r, cols);
        const int nc = (L + C - 1) / C;
        if (c >= nc) {
            if (c == 0 && argmax && tid == 0) argmax[r] = -1;
            continue;
        }
        const int start = c * C;
        const int end = min(L, start + C);
        const bool full = end - start == C;
        const float* xr = x + (int64_t)r * x_rs;
        f32x4 v[NV];
        if (full) fused_load<body_mask<VEC>(), T, NV>(xr, start, end, v);
        else fused_load<tail_mask<VEC>(), T, NV>(xr, start, end, v);
        // chunk statistics
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < NV; ++k) m = max4(m, v[k]);
        m = group_reduce<kWave>(m, OpMax());
        m = block_fold(m, sl_m, T / kWave, OpMax());
        int cand = INT_MAX;
        float sum = 0.f;
#pragma unroll
        for (int k = NV - 1; k >= 0; --k)
#pragma unroll
            for (int cc = 3; cc >= 0; --cc) {
                const int j = start + (k * T + tid) * 4 + cc;
                if (j < end && is_max(comp(v[k], cc), m)) cand = j;
            }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const f32x4 e = exp4_masked(v[k], m, start + (k * T + tid) * 4, end);
            sum += (e.x + e.y) + (e.z + e.w);
        }
        cand = group_reduce<kWave>(cand, OpMinI());
        cand = block_fold(cand, sl_i, T / kWave, OpMinI());
        sum = group_reduce<kWave>(sum, OpSum());
        sum = block_fold(sum, sl_d, T / kWave, OpSum());
        // publish, then wait for the rest of the row
        if (tid == 0) {
            SoftmaxPartial* p = f.part + t;
            __hip_atomic_store(&p->m, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&p->d, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&p->idx, cand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&f.row_cnt[r], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            int spins = 0;
            while (__hip_atomic_load(&f.row_cnt[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)nc &&
                   spins < kSpinLimit) {
                __builtin_amdgcn_s_sleep(2);
                ++spins;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_timeout = spins < kSpinLimit ? 0 : 1;
            if (spins >= kSpinLimit) __hip_atomic_store(&f.hdr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const bool timed_out = s_timeout != 0;
        // merge the row's partials in chunk order (wave 0), broadcast through LDS
        if (tid < kWave) {
            MD st{-INFINITY, 0.f};
            MI best{-INFINITY, INT_MAX};
            const SoftmaxPartial* pr = f.part + (int64_t)r * S;
            for (int k = tid; k < nc; k += kWave) {
                const float pm = __hip_atomic_load(&pr[k].m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const float pd = __hip_atomic_load(&pr[k].d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int pi = __hip_atomic_load(&pr[k].idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                st = md_combine(st, MD{pm, pd});
                best = mi_combine(best, MI{pm, pi});
            }
            st = group_reduce<kWave>(st, OpMD());
            best = group_reduce<kWave>(best, OpMI());
            if (tid == 0) {
                s_max = timed_out ? NAN : st.m;
                s_inv = 1.0f / st.d;
                if (c == 0 && argmax) argmax[r] = timed_out ? -1 : best.i;
            }
        }
        __syncthreads();
        const float mx = s_max, inv = s_inv;
        float* yr = y + (int64_t)r * y_rs;
        if (full) fused_store<body_mask<VEC>(), T, NV>(yr, start, end, v, mx, inv);
        else fused_store<tail_mask<VEC>(), T, NV>(yr, start, end, v, mx, inv);
        __syncthreads();  // LDS slots and broadcasts are rewritten by the next chunk
    }
}

// ------------------------------------------------------------------ launchers
namespace {

using SmFn = void (*)(const float*, float*, int, int, int64_t, int64_t, const int32_t*, int32_t*);
using PartFn = void (*)(const float*, int, int, int64_t, const int32_t*, SoftmaxPartial*, int);
using FinFn = void (*)(const float*, float*, int, int, int64_t, int64_t, const int32_t*, int32_t*,
                       const SoftmaxPartial*, int);

template <int M>
SmFn pick_per_m(int seg, int nv, int rpw) {
    if (rpw == 2) {
        if (seg != 64) return nullptr;
        switch (nv) {
            case 1: return fr_per_softmax_f32<64, 1, M, 2>;
            case 2: return fr_per_softmax_f32<64, 2, M, 2>;
            case 4: return fr_per_softmax_f32<64, 4, M, 2>;
        }
        return nullptr;
    }
    if (rpw != 1) return nullptr;
    switch (seg) {
        case 8: return fr_per_softmax_f32<8, 1, M, 1>;
        case 16: return fr_per_softmax_f32<16, 1, M, 1>;
        case 32: return fr_per_softmax_f32<32, 1, M, 1>;
        case 64:
            switch (nv) {
                case 1: return fr_per_softmax_f32<64, 1, M, 1>;
                case 2: return fr_per_softmax_f32<64, 2, M, 1>;
                case 4: return fr_per_softmax_f32<64, 4, M, 1>;
                case 8: return fr_per_softmax_f32<64, 8, M, 1>;
            }
    }
    return nullptr;
}

SmFn pick_per(int mask, int seg, int nv, int rpw) {
    switch (mask) {
        case kNone: return pick_per_m<kNone>(seg, nv, rpw);
        case kVec: return pick_per_m<kVec>(seg, nv, rpw);
        case kElem: return pick_per_m<kElem>(seg, nv, rpw);
        default: return pick_per_m<kScalar>(seg, nv, rpw);
    }
}

template <bool VEC>
SmFn pick_red(int threads, int u) {
    if (threads == 256 && u == 4) return fr_red_softmax_f32<256, 4, VEC>;
    if (threads == 512 && u == 2) return fr_red_softmax_f32<512, 2, VEC>;
    if (threads == 1024 && u == 2) return fr_red_softmax_f32<1024, 2, VEC>;
    if (threads == 1024 && u == 1) return fr_red_softmax_f32<1024, 1, VEC>;
    return nullptr;
}

using FusedFn = void (*)(const float*, float*, int, int, int64_t, int64_t, const int32_t*, int32_t*, void*, int);

template <bool VEC>
FusedFn pick_fused(int threads, int nv) {
    if (threads == 256 && nv == 8) return fr_split_softmax_fused<256, 8, VEC>;
    if (threads == 256 && nv == 4) return fr_split_softmax_fused<256, 4, VEC>;
    if (threads == 512 && nv == 4) return fr_split_softmax_fused<512, 4, VEC>;
    return nullptr;
}

template <bool VEC>
void pick_split(int threads, int nv, PartFn* part, FinFn* fin) {
    *part = nullptr;
    *fin = nullptr;
    if (threads == 256 && nv == 8) {
        *part = fr_split_softmax_part<256, 8, VEC>;
        *fin = fr_split_softmax_fin<256, 8, VEC>;
    } else if (threads == 256 && nv == 4) {
        *part = fr_split_softmax_part<256, 4, VEC>;
        *fin = fr_split_softmax_fin<256, 4, VEC>;
    } else if (threads == 512 && nv == 4) {
        *part = fr_split_softmax_part<512, 4, VEC>;
        *fin = fr_split_softmax_fin<512, 4, VEC>;
    }
}

}  // namespace

hipError_t launch_softmax(const fr_plan& p, const SoftmaxArgs& a, hipStream_t s) {
    const bool vec = p.vec16 != 0;
    if (p.form == FR_FORM_PER) {
        const int rpw = p.rows_per_wg / (256 / p.seg);
        // dense rows that fill the capacity exactly run without masks
        const int mask = !vec ? kScalar
                              : (a.lengths ? kElem
                                           : (a.cols == 4 * p.seg * p.vec ? kNone : (a.cols % 4 == 0 ? kVec : kElem)));
        SmFn f = pick_per(mask, p.seg, p.vec, rpw);
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(256), 0, s, a.x, a.y, a.rows, a.cols, a.x_rs, a.y_rs,
                           a.lengths, a.argmax);
        return hipGetLastError();
    }
    if (p.form == FR_FORM_RED) {
        SmFn f = vec ? pick_red<true>(p.threads, p.vec) : pick_red<false>(p.threads, p.vec);
        if (!f) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.y, a.rows, a.cols, a.x_rs,
                           a.y_rs, a.lengths, a.argmax);
        return hipGetLastError();
    }
    if (p.form == FR_FORM_SPLIT && p.passes == 1) {
        if (p.splits > kFusedMaxSplits) return hipErrorInvalidDeviceFunction;
        FusedFn fused = vec ? pick_fused<true>(p.threads, p.vec) : pick_fused<false>(p.threads, p.vec);
        if (!fused) return hipErrorInvalidDeviceFunction;
        const FusedWs f = fused_layout(a.ws, a.rows);
        hipLaunchKernelGGL(fr_split_softmax_prep, dim3((unsigned)((a.rows + 16 + 255) / 256)), dim3(256), 0, s, f.hdr,
                           f.row_cnt, a.rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fused, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.y, a.rows, a.cols, a.x_rs,
                           a.y_rs, a.lengths, a.argmax, a.ws, p.splits);
        return hipGetLastError();
    }
    if (p.form == FR_FORM_SPLIT) {
        PartFn part;
        FinFn fin;
        if (vec) pick_split<true>(p.threads, p.vec, &part, &fin);
        else pick_split<false>(p.threads, p.vec, &part, &fin);
        if (!part || !fin) return hipErrorInvalidDeviceFunction;
        SoftmaxPartial* ws = static_cast<SoftmaxPartial*>(a.ws);
        hipLaunchKernelGGL(part, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.rows, a.cols, a.x_rs,
                           a.lengths, ws, p.splits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fin, dim3((unsigned)p.grid2), dim3(p.threads), 0, s, a.x, a.y, a.rows, a.cols, a.x_rs,
                           a.y_rs, a.lengths, a.argmax, (const SoftmaxPartial*)ws, p.splits);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace fr
