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
        // The RPW rows go through each phase together, so their reduction
        // chains overlap: maxima, then argmax, then sums, then stores.
        float m[RPW], inv[RPW];
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            m[q] = -INFINITY;
#pragma unroll
            for (int k = 0; k < NV; ++k) m[q] = max4(m[q], v[q][k]);
        }
#pragma unroll
        for (int q = 0; q < RPW; ++q) m[q] = group_reduce<SEG>(m[q], OpMax());
        if (argmax) {
#pragma unroll
            for (int q = 0; q < RPW; ++q) {
                const int r = grp * RPB + g * RPW + q;
                int cand = INT_MAX;
#pragma unroll
                for (int k = NV - 1; k >= 0; --k)
#pragma unroll
                    for (int c = 3; c >= 0; --c) {
                        const int j = (k * SEG + l) * 4 + c;
                        if (j < L[q] && is_max(comp(v[q][k], c), m[q])) cand = j;
                    }
                cand = group_reduce<SEG>(cand, OpMinI());
                if (r < rows && l == 0) argmax[r] = L[q] > 0 ? cand : -1;
            }
        }
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            float s;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                v[q][k] = M == kNone ? exp4(v[q][k], m[q]) : exp4_masked(v[q][k], m[q], (k * SEG + l) * 4, L[q]);
                const float t = (v[q][k].x + v[q][k].y) + (v[q][k].z + v[q][k].w);
                s = k == 0 ? t : s + t;  // the terms are >= +0, so no -0 to keep
            }
            inv[q] = s;
        }
#pragma unroll
        for (int q = 0; q < RPW; ++q) inv[q] = 1.0f / group_reduce<SEG>(inv[q], OpSum());  // one division per row
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            const int r = grp * RPB + g * RPW + q;
            const bool live = r < rows;
            float* yr = y + (int64_t)(live ? r : 0) * y_rs;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int j0 = (k * SEG + l) * 4;
                if constexpr (M == kNone) {
                    if (live) st4<true>(yr + j0, v[q][k] * inv[q]);
                } else {
                    store4m<M, true>(yr, j0, L[q], v[q][k] * inv[q]);
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

// Workspace slot words (the split forms): a 32-bit tag above a 32-bit value
// (slot_word, published and the header layout in fr_device.h).
constexpr uint32_t kTwoKernelTag = 0x80000000u;  // never an epoch tag
constexpr uint64_t kWsMagic = 0x46525753664D4158ull;
__device__ __forceinline__ float slot_value(uint64_t w) { return __builtin_bit_cast(float, (uint32_t)w); }

// ------------------------------------------------------------------ split
// Chunk c of a row covers [c * C, min(len, (c+1) * C)) with C = 4 * T * NV.
// Its partial state is (m, d, i): the chunk maximum, the sum of e^(x - m)
// over the chunk and the first index of m ("Stax (4)", 9.5, Proposition 9.1:
// the (m, d) states of any segmentation of the row merge into the row's).
// A chunk wholly inside its row is loaded without masks.

// Partial of a chunk held in registers (all threads return it).
template <int M, int T, int NV>
__device__ __forceinline__ SoftmaxPartial chunk_partial(const f32x4* v, int start, int end, float* sl_m, float* sl_d,
                                                        int* sl_i) {
    const int tid = threadIdx.x;
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
    return SoftmaxPartial{m, s, cand, 0};
}

// The same partial with the chunk read from memory one vector at a time, so
// that it needs no second register copy of a chunk. Every thread performs
// the operations of chunk_partial in the same order on the same values, so
// the bits are those of chunk_partial.
template <int M, int T, int NV>
__device__ SoftmaxPartial chunk_partial_streamed(const float* xr, int start, int end, float* sl_m, float* sl_d,
                                                 int* sl_i) {
    const int tid = threadIdx.x;
    float m = -INFINITY;
#pragma unroll 1
    for (int k = 0; k < NV; ++k) m = max4(m, load4m<M, false>(xr, start + (k * T + tid) * 4, end, -INFINITY));
    m = group_reduce<kWave>(m, OpMax());
    m = block_fold(m, sl_m, T / kWave, OpMax());
    int cand = INT_MAX;
    float s = 0.f;
#pragma unroll 1
    for (int k = NV - 1; k >= 0; --k) {
        const f32x4 v = load4m<M, false>(xr, start + (k * T + tid) * 4, end, -INFINITY);
#pragma unroll
        for (int c = 3; c >= 0; --c) {
            const int j = start + (k * T + tid) * 4 + c;
            if (j < end && is_max(comp(v, c), m)) cand = j;
        }
    }
#pragma unroll 1
    for (int k = 0; k < NV; ++k) {
        const f32x4 v = load4m<M, false>(xr, start + (k * T + tid) * 4, end, -INFINITY);
        const f32x4 e = M == kNone ? exp4(v, m) : exp4_masked(v, m, start + (k * T + tid) * 4, end);
        s += (e.x + e.y) + (e.z + e.w);
    }
    cand = group_reduce<kWave>(cand, OpMinI());
    cand = block_fold(cand, sl_i, T / kWave, OpMinI());
    s = group_reduce<kWave>(s, OpSum());
    s = block_fold(s, sl_d, T / kWave, OpSum());
    return SoftmaxPartial{m, s, cand, 0};
}

template <int M, int T, int NV, bool NT>
__device__ __forceinline__ void load_chunk(const float* xr, int start, int end, f32x4* v) {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load4m<M, NT>(xr, start + (k * T + (int)threadIdx.x) * 4, end, -INFINITY);
}

template <int M, int T, int NV>
__device__ __forceinline__ void store_chunk(float* yr, int start, int end, const f32x4* v, float mx, float inv) {
#pragma unroll
    for (int k = 0; k < NV; ++k) store4m<M, true>(yr, start + (k * T + (int)threadIdx.x) * 4, end, exp4(v[k], mx) * inv);
}

// ---- two kernels: workgroup r * S + c takes chunk c of row r. Part 1 writes
// the chunk's (m, d) as two slot words tagged kTwoKernelTag (a tag the
// single pass never accepts, so the two forms can share a workspace); part 2
// merges the row's partials in chunk order and writes the normalized chunk;
// the workgroup of the first chunk holding the row maximum writes the argmax
// (the first index of the maximum in that chunk). Part 1 reads x with
// ordinary loads so that part 2 can find it in the device caches.
template <int T, int NV, bool VEC>
__global__ __launch_bounds__(T) void fr_split_softmax_part(const float* __restrict__ x, int rows, int cols,
                                                           int64_t x_rs, const int32_t* __restrict__ lengths,
                                                           uint64_t* __restrict__ slots, int S) {
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
    f32x4 v[NV];
    SoftmaxPartial p;
    if (end - start == C) {
        load_chunk<body_mask<VEC>(), T, NV, false>(xr, start, end, v);
        p = chunk_partial<body_mask<VEC>(), T, NV>(v, start, end, sl_m, sl_d, sl_i);
    } else {
        load_chunk<tail_mask<VEC>(), T, NV, false>(xr, start, end, v);
        p = chunk_partial<tail_mask<VEC>(), T, NV>(v, start, end, sl_m, sl_d, sl_i);
    }
    if (threadIdx.x == 0) {
        slots[2 * w] = slot_word(kTwoKernelTag, p.m);
        slots[2 * w + 1] = slot_word(kTwoKernelTag, p.d);
    }
}

template <int M, int T, int NV>
__device__ __forceinline__ void fin_body(const float* xr, float* yr, int start, int end, float mx, float inv,
                                         int32_t* argmax_r, int* sl_i) {
    f32x4 v[NV];
    load_chunk<M, T, NV, true>(xr, start, end, v);
    if (argmax_r) {  // this chunk holds the row maximum first: its first index of it
        int cand = INT_MAX;
#pragma unroll
        for (int k = NV - 1; k >= 0; --k)
#pragma unroll
            for (int c = 3; c >= 0; --c) {
                const int j = start + (k * T + (int)threadIdx.x) * 4 + c;
                if (j < end && is_max(comp(v[k], c), mx)) cand = j;
            }
        cand = group_reduce<kWave>(cand, OpMinI());
        cand = block_fold(cand, sl_i, T / kWave, OpMinI());
        if (threadIdx.x == 0) *argmax_r = cand;
    }
    store_chunk<M, T, NV>(yr, start, end, v, mx, inv);
}

template <int T, int NV, bool VEC>
__global__ __launch_bounds__(T) void fr_split_softmax_fin(const float* x, float* y, int rows, int cols,
                                                          int64_t x_rs, int64_t y_rs,
                                                          const int32_t* __restrict__ lengths,
                                                          int32_t* __restrict__ argmax,
                                                          const uint64_t* __restrict__ slots, int S) {
    constexpr int C = 4 * T * NV;
    __shared__ int sl_i[T / kWave];
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
    const uint64_t* pr = slots + 2 * (int64_t)r * S;
    for (int k = 0; k < nc; ++k) {
        const float pm = slot_value(pr[2 * k]);
        st = md_combine(st, MD{pm, slot_value(pr[2 * k + 1])});
        best = mi_combine(best, MI{pm, k});  // the first chunk holding the row maximum
    }
    const float inv = 1.0f / st.d;
    const float* xr = x + (int64_t)r * x_rs;
    float* yr = y + (int64_t)r * y_rs;
    int32_t* am = (argmax && c == best.i) ? argmax + r : nullptr;
    if (end - start == C) fin_body<body_mask<VEC>(), T, NV>(xr, yr, start, end, st.m, inv, am, sl_i);
    else fin_body<tail_mask<VEC>(), T, NV>(xr, yr, start, end, st.m, inv, am, sl_i);
}

// ---- one kernel: every chunk is read once and stays in registers while the
// row's partials are exchanged through the workspace.
//  - Each workgroup derives the list of non-empty chunks from the row
//    lengths (chunk counts and their exclusive prefix sum, kept in LDS), and
//    workgroup w takes list entries w, w + G, w + 2G, ... (G = grid size):
//    no workgroup is spent on the empty tail of a ragged row, and the chunks
//    of one row are worked on at the same time by neighbouring workgroups.
//  - A chunk's partial is published in its slot as two 64-bit words, (tag,
//    m) and (tag, d). The tag is the call's epoch: the workspace header
//    holds a counter E that every workgroup reads at its start (tag = E + 1)
//    and then acknowledges by storing the tag in its own flag word (the
//    store depends on the value read). The last workgroup (the one with the
//    fewest entries), at its end, waits until every flag holds the tag -
//    every workgroup has read E - and stores E + 1 for the next call. No two
//    workgroups update one word.
//    A word whose tag is not this call's (an earlier call's, the zeros of an
//    initialized workspace, or the reserved tag of the two-kernel form) is
//    not yet written. Each word is written with one 64-bit store and read
//    with one 64-bit load, the instructions of 64-bit atomic accesses, so a
//    reader that sees the tag sees the value beside it and no fence is
//    needed. Nothing has to be cleared between calls.
//  - The header also holds a magic number that only the initialization
//    writes. Without it (a workspace never initialized), or once the epoch
//    has reached its last value, no slot is trusted: every partner partial
//    is computed from x, which gives the same bits, only slower.
//  - A workgroup waits, up to a wall-clock limit, for the other slots of its
//    row (a negative limit: it reads none of them). A partial still missing
//    at the limit it computes itself from x
//    with chunk_partial_streamed, which gives the owner's bits. Nothing
//    depends on other workgroups being resident, so every launch finishes
//    and the result does not depend on scheduling. Each partial computed this
//    way is added to a count in the workspace header.
//  - The row's partials are merged in a fixed order (64-lane butterflies over
//    groups of 64 chunks, groups in order), so every chunk of a row is
//    normalized with the same (m, d) bits. The merge also yields the first
//    chunk whose maximum is the row's; that chunk's workgroup writes the
//    argmax, the first index of the maximum within its own chunk.
// Workspace initialization: zeros everywhere, epoch 0, the magic number.
__global__ __launch_bounds__(256) void fr_split_softmax_init(uint32_t* __restrict__ ws, int64_t nwords) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nwords)
        ws[i] = i == kHdrMagic ? (uint32_t)kWsMagic : (i == kHdrMagic + 1 ? (uint32_t)(kWsMagic >> 32) : 0u);
}

// Pipelined form of the one-kernel split (16-byte aligned rows): entry
// t + G is loaded while entry t is reduced, exchanged and stored, so each
// workgroup keeps a chunk of loads in flight through the wait for its row's
// other partials. Every memory instruction of the common path is issued by
// every lane, without a branch: a lane past its chunk, or an entry past the
// list, lies outside its buffer resource's range, reads zeros and writes
// nothing. The compiler's waits for older loads then count the newer ones
// instead of draining them; only the wait loop and the recomputation (the
// rare paths) drain. A workgroup looks at its partners' slots once right
// after publishing its own partial, before the next chunk's loads, and waits
// only if some were not yet there.
// This call's tag (0: no slot is trusted), taken by thread 0 from the
// header words it loaded at the start and acknowledged in the workgroup's
// flag (the stored value depends on the epoch read). The other threads read
// it from LDS after the next barrier, so the header's latency is hidden
// behind the first chunk's loads.
__device__ __forceinline__ void take_tag(u32x2 magic_w, uint32_t epoch, uint32_t* flags, uint32_t* s_tag,
                                         uint32_t* s_epoch) {
    const uint64_t magic = (uint64_t)magic_w.y << 32 | magic_w.x;
    const uint32_t t = (magic == kWsMagic && epoch < kMaxEpoch) ? epoch + 1 : 0u;
    if (t != 0u) __hip_atomic_store(&flags[blockIdx.x], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_tag = t;
    *s_epoch = epoch;
}

struct OneEntry {
    int r, c, nc, base, start, n;
};
// Entries per workgroup whose rows are found while the list is built.
constexpr int kEntryTable = 8;

// chunk_partial for a chunk of n elements in registers (lanes past n hold
// -inf) with chunk-relative indices and the thread id passed in: the same
// operations in the same order, so the same bits (the index is relative).
template <int T, int NV>
__device__ __forceinline__ SoftmaxPartial pipe_partial(const f32x4* v, int n, int lt, float* sl_m, float* sl_d,
                                                       int* sl_i) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NV; ++k) m = max4(m, v[k]);
    m = group_reduce<kWave>(m, OpMax());
    m = block_fold(m, sl_m, T / kWave, OpMax());
    int cand = INT_MAX;
    float s = 0.f;
    const int l4 = lt * 4;
#pragma unroll
    for (int k = NV - 1; k >= 0; --k)
#pragma unroll
        for (int c = 3; c >= 0; --c)
            if (l4 + c < n - k * T * 4 && is_max(comp(v[k], c), m)) cand = k * T * 4 + l4 + c;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int rem = n - k * T * 4;
        const f32x4 e = {l4 + 0 < rem ? exp_fast(v[k].x - m) : 0.f, l4 + 1 < rem ? exp_fast(v[k].y - m) : 0.f,
                         l4 + 2 < rem ? exp_fast(v[k].z - m) : 0.f, l4 + 3 < rem ? exp_fast(v[k].w - m) : 0.f};
        s += (e.x + e.y) + (e.z + e.w);
    }
    cand = group_reduce<kWave>(cand, OpMinI());
    cand = block_fold(cand, sl_i, T / kWave, OpMinI());
    s = group_reduce<kWave>(s, OpSum());
    s = block_fold(s, sl_d, T / kWave, OpSum());
    return SoftmaxPartial{m, s, cand, 0};
}

template <int T, int NV>
__device__ __forceinline__ void one_pass_pipelined(const float* x, float* y, int64_t x_rs, int64_t y_rs,
                                                   const int* s_base, const int* s_len, const int* s_erow,
                                                   int rows, int total,
                                                   int32_t* argmax, uint32_t* hdr, uint64_t* slots, float* sl_m,
                                                   float* sl_d, int* sl_i, uint64_t* s_missing, float* s_mx,
                                                   int* s_kstar, u32x2 magic_w, uint32_t epoch, uint32_t* flags,
                                                   uint32_t* s_tag, uint32_t* s_epoch, int64_t wait_ticks) {
    constexpr int C = 4 * T * NV;
    const int tid = threadIdx.x;
    const int G = gridDim.x;
    // the list lives in LDS; its values are the same for every lane, and
    // reading them as such keeps the search and the buffer resources scalar
    auto uni = [](int v) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(v); };
    // entry t = blockIdx.x + k G of the list: its row from the table built
    // with the list (k < kEntryTable), else by binary search
    auto entry = [&](int t, int k) __attribute__((always_inline)) {
        OneEntry e;
        if (t >= total) {  // past the list: an empty range, nothing read or written
            e.r = 0, e.base = 0, e.nc = 1, e.c = 0, e.start = 0, e.n = 0;
            return e;
        }
        int lo = k < kEntryTable ? uni(s_erow[k]) : 0;
        e.base = uni(s_base[lo]);
        e.nc = uni(s_base[lo + 1]) - e.base;
        if (k >= kEntryTable || t < e.base || t >= e.base + e.nc) {
            lo = 0;
            int hi = rows;  // s_base[lo] <= t < s_base[hi]; rows without chunks never qualify
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (uni(s_base[mid]) <= t) lo = mid;
                else hi = mid;
            }
            e.base = uni(s_base[lo]);
            e.nc = uni(s_base[lo + 1]) - e.base;
        }
        e.r = lo;
        e.c = t - e.base;
        e.start = e.c * C;
        e.n = min(uni(s_len[lo]) - e.start, C);
        return e;
    };
    // lane offset in a register, vector offset k * T * 16 as a constant
    auto issue = [&](f32x4(&v)[NV], const OneEntry& e, int lt) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + (int64_t)e.r * x_rs + e.start, (uint32_t)e.n * 4u);
#pragma unroll
        for (int k = 0; k < NV; ++k)
            v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, lt * 16, k * T * 16, kAuxNT));
    };
    auto step = [&](const OneEntry& ec, f32x4(&cur)[NV], const OneEntry& en, f32x4(&nxt)[NV])
                    __attribute__((always_inline)) {
        // the thread id, opaque to the compiler here, so that the per-element
        // index arithmetic is redone in each step instead of being hoisted
        // out of the loop into 40 live registers
        int lt = tid;
        asm volatile("" : "+v"(lt));
        const int l4 = lt * 4;
        // lanes past the chunk read zeros: give them the maximum's identity
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int rem = ec.n - k * T * 4;
            cur[k].x = l4 + 0 < rem ? cur[k].x : -INFINITY;
            cur[k].y = l4 + 1 < rem ? cur[k].y : -INFINITY;
            cur[k].z = l4 + 2 < rem ? cur[k].z : -INFINITY;
            cur[k].w = l4 + 3 < rem ? cur[k].w : -INFINITY;
        }
        SoftmaxPartial own = pipe_partial<T, NV>(cur, ec.n, lt, sl_m, sl_d, sl_i);
        if (own.idx != INT_MAX) own.idx += ec.start;
        const uint32_t tag = uni((int)*s_tag);  // written before the partial's barriers
        const uint64_t own0 = slot_word(tag, own.m), own1 = slot_word(tag, own.d);
        // the row's slots, 16 bytes per chunk; a row of one chunk exchanges
        // nothing, and without a tag nothing is published (an empty range)
        uint64_t* rs = slots + 2 * (int64_t)ec.base;
        const int row_slot_bytes = (tag != 0u && ec.nc > 1) ? ec.nc * 16 : 0;
        const __amdgpu_buffer_rsrc_t rslots = row_rsrc(rs, (uint32_t)row_slot_bytes);
        // publish: threads 0 and 1 write the slot's two words, every other
        // lane falls outside the range; sc1: seen by the other dies
        const uint64_t word = tid & 1 ? own1 : own0;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{(uint32_t)word, (uint32_t)(word >> 32)}, rslots,
                                              tid < 2 ? ec.c * 16 + tid * 8 : row_slot_bytes, 0, kAuxSc1);
        // first look at the partners: lane k of wave 0 reads chunk k's two
        // words, each with one 64-bit load
        const bool look = tid < kWave && tid < ec.nc && tid != ec.c;
        const int look_off = look ? tid * 16 : row_slot_bytes;
        const u32x2 pw0 = __builtin_amdgcn_raw_buffer_load_b64(rslots, look_off, 0, kAuxSc1);
        const u32x2 pw1 = __builtin_amdgcn_raw_buffer_load_b64(rslots, look_off + 8, 0, kAuxSc1);
        issue(nxt, en, lt);

        const float* xr = x + (int64_t)ec.r * x_rs;
        const int L = uni(s_len[ec.r]);
        // a row of one chunk: its partial is the row's (the merge below would
        // return it unchanged, up to the d of a row whose y is all NaN)
        MD st = ec.nc == 1 ? MD{own.m, own.d} : MD{-INFINITY, 0.f};
        MI best = ec.nc == 1 ? MI{own.m, 0} : MI{-INFINITY, INT_MAX};
        for (int g0 = 0; g0 < (ec.nc == 1 ? 0 : ec.nc); g0 += kWave) {
            const int k = g0 + (tid & (kWave - 1));
            uint64_t w0 = g0 == 0 ? ((uint64_t)pw0.y << 32 | pw0.x) : 0ull;
            uint64_t w1 = g0 == 0 ? ((uint64_t)pw1.y << 32 | pw1.x) : 0ull;
            if (k == ec.c) {
                w0 = own0;
                w1 = own1;
            }
            if (tid < kWave) {
                // with no wait (wait_ticks < 0), or no tag, every partner's
                // partial is recomputed
                const bool trust = wait_ticks >= 0 && tag != 0u;
                bool ok = k >= ec.nc || k == ec.c || (trust && published(w0, tag) && published(w1, tag));
                if (!__all(ok) && trust) {
                    const uint64_t t0 = wall_clock64();
                    for (;;) {
                        if (!ok) {
                            if (!published(w0, tag))
                                w0 = __hip_atomic_load(&rs[2 * k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (!published(w1, tag))
                                w1 = __hip_atomic_load(&rs[2 * k + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            ok = published(w0, tag) && published(w1, tag);
                        }
                        if (__all(ok)) break;
                        if ((int64_t)(wall_clock64() - t0) >= wait_ticks) break;
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                const uint64_t miss = __ballot(!ok);
                if (tid == 0) *s_missing = miss;
            }
            __syncthreads();
            uint64_t miss = *s_missing;
            while (miss) {  // rare: the owner has not published in time
                const int j = __builtin_ctzll(miss);
                miss &= miss - 1;
                const int ks = (g0 + j) * C;
                const int ke = min(L, ks + C);
                const SoftmaxPartial p = chunk_partial_streamed<kElem, T, NV>(xr, ks, ke, sl_m, sl_d, sl_i);
                if (tid == j) {
                    w0 = slot_word(tag, p.m);
                    w1 = slot_word(tag, p.d);
                }
                if (tid == 0)
                    __hip_atomic_fetch_add(&hdr[kHdrRecomputed], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0);
            }
            if (tid < kWave) {
                MD a{-INFINITY, 0.f};
                MI b{-INFINITY, INT_MAX};
                if (k < ec.nc) {
                    const float pm = slot_value(w0);
                    a = MD{pm, slot_value(w1)};
                    b = MI{pm, k};  // the first chunk holding the row maximum
                }
                // up to 16 chunks sit in one DPP row: 4 butterfly steps, not 6
                if (ec.nc <= 16) {
                    st = md_combine(st, group_reduce<16>(a, OpMD()));
                    best = mi_combine(best, group_reduce<16>(b, OpMI()));
                } else {
                    st = md_combine(st, group_reduce<kWave>(a, OpMD()));
                    best = mi_combine(best, group_reduce<kWave>(b, OpMI()));
                }
            }
            __syncthreads();  // s_missing and the fold slots are rewritten next
        }
        if (tid == 0) {
            s_mx[0] = st.m;
            s_mx[1] = 1.0f / st.d;
            *s_kstar = best.i;
        }
        __syncthreads();
        const float mx = s_mx[0], inv = s_mx[1];
        // the row's argmax is the first index of the maximum in the first
        // chunk that holds it: that chunk's workgroup writes it (thread 0 in range)
        const bool am = argmax != nullptr && ec.c == uni(*s_kstar);
        __builtin_amdgcn_raw_buffer_store_b32(
            (uint32_t)own.idx, row_rsrc(reinterpret_cast<char*>(argmax) + (am ? 4 * (int64_t)ec.r : 0), am ? 4u : 0u),
            tid == 0 ? 0 : 4, 0, 0);
        const __amdgpu_buffer_rsrc_t ry = row_rsrc(y + (int64_t)ec.r * y_rs + ec.start, (uint32_t)ec.n * 4u);
#pragma unroll
        for (int k = 0; k < NV; ++k)
            store16<kAuxNT>(__builtin_bit_cast(u32x4, exp4(cur[k], mx) * inv), ry, lt * 16 + k * T * 16);
    };

    f32x4 va[NV], vb[NV];
    OneEntry ea = entry(blockIdx.x, 0);
    issue(va, ea, tid);
    if (tid == 0) take_tag(magic_w, epoch, flags, s_tag, s_epoch);
    for (int t = blockIdx.x, k = 0; t < total; t += 2 * G, k += 2) {
        const OneEntry eb = entry(t + G, k + 1);
        step(ea, va, eb, vb);
        if (t + G >= total) break;
        ea = entry(t + 2 * G, k + 2);
        step(eb, vb, ea, va);
    }
}

// Element-wise form of the one-kernel split (rows not 16-byte aligned): one
// chunk in registers at a time, read with masked loads.
template <int T, int NV>
__device__ __forceinline__ void one_pass_elementwise(const float* x, float* y, int64_t x_rs, int64_t y_rs,
                                                     const int* s_base, const int* s_len, int rows, int total,
                                                     int32_t* argmax, uint32_t* hdr, uint64_t* slots, float* sl_m,
                                                     float* sl_d, int* sl_i, uint64_t* s_missing, float* s_mx,
                                                     int* s_kstar, u32x2 magic_w, uint32_t epoch,
                                                     uint32_t* flags, uint32_t* s_tag, uint32_t* s_epoch,
                                                     int64_t wait_ticks) {
    constexpr bool VEC = false;
    constexpr int C = 4 * T * NV;
    const int tid = threadIdx.x;
    if (tid == 0) take_tag(magic_w, epoch, flags, s_tag, s_epoch);
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        int lo = 0, hi = rows;  // s_base[lo] <= t < s_base[hi]; rows without chunks never qualify
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_base[mid] <= t) lo = mid;
            else hi = mid;
        }
        const int r = lo;
        const int base = s_base[r];
        const int nc = s_base[r + 1] - base;
        const int c = t - base;
        const int L = s_len[r];
        const int start = c * C;
        const int end = min(L, start + C);
        const bool full = end - start == C;
        const float* xr = x + (int64_t)r * x_rs;
        f32x4 v[NV];
        SoftmaxPartial own;
        if (full) {
            load_chunk<body_mask<VEC>(), T, NV, true>(xr, start, end, v);
            own = chunk_partial<body_mask<VEC>(), T, NV>(v, start, end, sl_m, sl_d, sl_i);
        } else {
            load_chunk<tail_mask<VEC>(), T, NV, true>(xr, start, end, v);
            own = chunk_partial<tail_mask<VEC>(), T, NV>(v, start, end, sl_m, sl_d, sl_i);
        }
        const uint32_t tag = __builtin_amdgcn_readfirstlane(*s_tag);  // written before the partial's barriers
        uint64_t* rs = slots + 2 * (int64_t)base;
        // a row of one chunk exchanges nothing; without a tag nothing is published
        if (tid == 0 && tag != 0u && nc > 1) {
            __hip_atomic_store(&rs[2 * c], slot_word(tag, own.m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&rs[2 * c + 1], slot_word(tag, own.d), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // merge the row's partials, 64 at a time: wave 0 gathers (lane j: chunk g0 + j)
        MD st{-INFINITY, 0.f};
        MI best{-INFINITY, INT_MAX};
        for (int g0 = 0; g0 < nc; g0 += kWave) {
            const int k = g0 + (tid & (kWave - 1));
            uint64_t w0 = 0ull, w1 = 0ull;
            if (tid < kWave) {
                bool ok = k >= nc;
                if (k == c) {
                    w0 = slot_word(tag, own.m);
                    w1 = slot_word(tag, own.d);
                    ok = true;
                }
                const uint64_t t0 = wall_clock64();
                // wait_ticks < 0, or no tag: read no other partial (all are recomputed)
                for (; wait_ticks >= 0 && tag != 0u;) {
                    if (!ok) {
                        if (!published(w0, tag))
                            w0 = __hip_atomic_load(&rs[2 * k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (!published(w1, tag))
                            w1 = __hip_atomic_load(&rs[2 * k + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = published(w0, tag) && published(w1, tag);
                    }
                    if (__all(ok)) break;
                    if ((int64_t)(wall_clock64() - t0) >= wait_ticks) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                const uint64_t miss = __ballot(!ok);
                if (tid == 0) *s_missing = miss;
            }
            __syncthreads();
            uint64_t miss = *s_missing;
            while (miss) {  // rare: the owner has not published in time
                const int j = __builtin_ctzll(miss);
                miss &= miss - 1;
                const int ks = (g0 + j) * C;
                const int ke = min(L, ks + C);
                const SoftmaxPartial p =
                    ke - ks == C ? chunk_partial_streamed<body_mask<VEC>(), T, NV>(xr, ks, ke, sl_m, sl_d, sl_i)
                                 : chunk_partial_streamed<tail_mask<VEC>(), T, NV>(xr, ks, ke, sl_m, sl_d, sl_i);
                if (tid == j) {
                    w0 = slot_word(tag, p.m);
                    w1 = slot_word(tag, p.d);
                }
                if (tid == 0)
                    __hip_atomic_fetch_add(&hdr[kHdrRecomputed], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (tid < kWave) {
                MD a{-INFINITY, 0.f};
                MI b{-INFINITY, INT_MAX};
                if (k < nc) {
                    const float pm = slot_value(w0);
                    a = MD{pm, slot_value(w1)};
                    b = MI{pm, k};  // the first chunk holding the row maximum
                }
                st = md_combine(st, group_reduce<kWave>(a, OpMD()));
                best = mi_combine(best, group_reduce<kWave>(b, OpMI()));
            }
            __syncthreads();  // s_missing and the fold slots are rewritten next
        }
        if (tid == 0) {
            s_mx[0] = st.m;
            s_mx[1] = 1.0f / st.d;
            // the first index of the maximum, from the first chunk holding it
            if (c == best.i && argmax) argmax[r] = own.idx;
        }
        __syncthreads();
        const float mx = s_mx[0], inv = s_mx[1];
        float* yr = y + (int64_t)r * y_rs;
        if (full) store_chunk<body_mask<VEC>(), T, NV>(yr, start, end, v, mx, inv);
        else store_chunk<tail_mask<VEC>(), T, NV>(yr, start, end, v, mx, inv);
    }
}

template <int T, int NV, bool VEC>
__global__ __launch_bounds__(T) void fr_split_softmax_one(const float* x, float* y, int rows, int cols, int64_t x_rs,
                                                          int64_t y_rs, const int32_t* __restrict__ lengths,
                                                          int32_t* __restrict__ argmax, void* ws,
                                                          int64_t wait_ticks) {
    constexpr int C = 4 * T * NV;
    __shared__ int s_base[kOnePassMaxRows + 1];  // first list entry of each row; [rows] = list length
    __shared__ int s_len[kOnePassMaxRows];
    __shared__ int s_scan[T / kWave];
    __shared__ int s_erow[kEntryTable];  // row of entry blockIdx.x + k G
    __shared__ float sl_m[T / kWave];
    __shared__ float sl_d[T / kWave];
    __shared__ int sl_i[T / kWave];
    __shared__ uint64_t s_missing;
    __shared__ float s_mx[2];
    __shared__ int s_kstar;
    __shared__ uint32_t s_tag, s_epoch;
    uint32_t* hdr = static_cast<uint32_t*>(ws);
    uint32_t* flags = hdr + kSplitWsHeader / 4;
    uint64_t* slots = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kSplitWsSlots);
    const int tid = threadIdx.x;

    // The row lengths (out-of-range offsets read 0), then the initialization
    // mark and the epoch (loads with sc1, as the agent-scope atomic loads
    // they stand for; only thread 0's offsets lie in range): every load is
    // issued, without a branch, before any value is used, so the list build
    // waits for one memory latency, not one per load, and the lengths do not
    // wait for the header.
    constexpr int RPT = kOnePassMaxRows / T;
    const __amdgpu_buffer_rsrc_t rlen = row_rsrc(lengths, lengths ? (uint32_t)rows * 4u : 0u);
    int lv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) lv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rlen, (tid + i * T) * 4, 0, 0);
    const __amdgpu_buffer_rsrc_t rhdr = row_rsrc(hdr, (uint32_t)kSplitWsHeader);
    const u32x2 magic_w =
        __builtin_amdgcn_raw_buffer_load_b64(rhdr, tid == 0 ? kHdrMagic * 4 : kSplitWsHeader, 0, kAuxSc1);
    const uint32_t epoch =
        __builtin_amdgcn_raw_buffer_load_b32(rhdr, tid == 0 ? kHdrEpoch * 4 : kSplitWsHeader, 0, kAuxSc1);
    // no lengths: the loads read 0 and every row gets cols elements. Entries
    // past the rows are written too (never read), so that no store, and no
    // load, sits under a branch
    const int len0 = lengths ? 0 : cols;
#pragma unroll
    for (int i = 0; i < RPT; ++i) s_len[tid + i * T] = min(max(lv[i] + len0, 0), cols);
    __syncthreads();
    // thread tid counts the chunks of rows [r0, r1)
    const int per = (rows + T - 1) / T;
    const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
    int local = 0;
    for (int r = r0; r < r1; ++r) local += (s_len[r] + C - 1) / C;
    // exclusive prefix sum of the counts: an inclusive scan inside each
    // 16-lane DPP row (shifts by 1, 2, 4, 8), the row totals before this
    // row from lanes 15, 31 and 47, then the wave totals before this wave
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    int incl = local;
    incl += __builtin_amdgcn_update_dpp(0, incl, kDppRowShr1, 0xF, 0xF, false);
    incl += __builtin_amdgcn_update_dpp(0, incl, kDppRowShr2, 0xF, 0xF, false);
    incl += __builtin_amdgcn_update_dpp(0, incl, kDppRowShr4, 0xF, 0xF, false);
    incl += __builtin_amdgcn_update_dpp(0, incl, kDppRowShr8, 0xF, 0xF, false);
    {
        const int row16 = lane >> 4;
        const int a = __builtin_amdgcn_readlane(incl, 15), b = __builtin_amdgcn_readlane(incl, 31),
                  c = __builtin_amdgcn_readlane(incl, 47);
        incl += (row16 >= 1 ? a : 0) + (row16 >= 2 ? b : 0) + (row16 >= 3 ? c : 0);
    }
    if (lane == kWave - 1) s_scan[wv] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wv; ++w) run += s_scan[w];
    // the first list entry of each row, and the rows of this workgroup's
    // entries blockIdx.x + k G for k < kEntryTable
    for (int r = r0; r < r1; ++r) {
        const int cnt = (s_len[r] + C - 1) / C;
        s_base[r] = run;
#pragma unroll
        for (int k = 0; k < kEntryTable; ++k) {
            const int64_t t = (int64_t)blockIdx.x + (int64_t)k * gridDim.x;
            if (t >= run && t < run + cnt) s_erow[k] = r;
        }
        run += cnt;
    }
    if (tid == T - 1) s_base[rows] = run;
    __syncthreads();
    const int total = s_base[rows];
    if (blockIdx.x == 0 && argmax)
        for (int r = tid; r < rows; r += T)
            if (s_len[r] == 0) argmax[r] = -1;

    if constexpr (VEC) {
        one_pass_pipelined<T, NV>(x, y, x_rs, y_rs, s_base, s_len, s_erow, rows, total, argmax, hdr, slots, sl_m,
                                  sl_d, sl_i, &s_missing, s_mx, &s_kstar, magic_w, epoch, flags, &s_tag, &s_epoch,
                                  wait_ticks);
    } else {
        one_pass_elementwise<T, NV>(x, y, x_rs, y_rs, s_base, s_len, rows, total, argmax, hdr, slots, sl_m, sl_d,
                                    sl_i, &s_missing, s_mx, &s_kstar, magic_w, epoch, flags, &s_tag, &s_epoch,
                                    wait_ticks);
    }
    __syncthreads();  // a workgroup without entries passed no barrier since thread 0 wrote the tag
    const uint32_t tag = __builtin_amdgcn_readfirstlane(s_tag);
    if (blockIdx.x == gridDim.x - 1 && tag != 0u) epoch_advance<T>(hdr, flags, tag, s_epoch);
}

// ------------------------------------------------------------------ backward
// dx = y (dy - s), s = sum_k dy_k y_k: one row reduction (the dot product of
// the upstream gradient with the forward output) and a pointwise epilogue.
// Masked lanes read y = dy = 0 (the identity of the dot product); elements
// past a row's length are neither read nor written.
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return (a.x * b.x + a.y * b.y) + (a.z * b.z + a.w * b.w); }

// Persistent: SEG lanes per row, NV vectors of y and NV of dy per lane, RPW
// rows per lane group through each phase together (as the forward kernel).
template <int SEG, int NV, int M, int RPW>
__global__ __launch_bounds__(256) void fr_per_softmax_bwd_f32(const float* y, const float* dy, float* dx, int rows,
                                                              int cols, int64_t y_rs, int64_t dy_rs, int64_t dx_rs,
                                                              const int32_t* __restrict__ lengths) {
    constexpr int RPB = 256 / SEG * RPW;
    const int g = threadIdx.x / SEG;
    const int l = threadIdx.x % SEG;
    const int ngroups = (rows + RPB - 1) / RPB;
    for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        f32x4 a[RPW][NV], b[RPW][NV];
        int L[RPW];
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            const int r = grp * RPB + g * RPW + q;
            const bool live = r < rows;
            // kNone: a row past the end re-reads the last row (in bounds) and stores nothing
            const int rl = live ? r : (M == kNone ? rows - 1 : 0);
            if constexpr (M == kNone) L[q] = live ? cols : 0;
            else L[q] = live ? row_len(lengths, r, cols) : 0;
            const float* yr = y + (int64_t)rl * y_rs;
            const float* gr = dy + (int64_t)rl * dy_rs;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int j0 = (k * SEG + l) * 4;
                if constexpr (M == kNone) {
                    a[q][k] = ld4<true>(yr + j0);
                    b[q][k] = ld4<true>(gr + j0);
                } else {
                    a[q][k] = load4m<M, true>(yr, j0, L[q], 0.f);
                    b[q][k] = load4m<M, true>(gr, j0, L[q], 0.f);
                }
            }
        }
        float sdot[RPW];
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            sdot[q] = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) sdot[q] += dot4(a[q][k], b[q][k]);
        }
#pragma unroll
        for (int q = 0; q < RPW; ++q) sdot[q] = group_reduce<SEG>(sdot[q], OpSum());
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            const int r = grp * RPB + g * RPW + q;
            const bool live = r < rows;
            float* xr = dx + (int64_t)(live ? r : 0) * dx_rs;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int j0 = (k * SEG + l) * 4;
                const f32x4 d = a[q][k] * (b[q][k] - sdot[q]);
                if constexpr (M == kNone) {
                    if (live) st4<true>(xr + j0, d);
                } else {
                    store4m<M, true>(xr, j0, L[q], d);
                }
            }
        }
    }
}

// Looped: one workgroup of T threads per row, U vectors per lane per step.
// Pass 1 accumulates the dot product per lane in step order; pass 2 reads
// the row again and writes dx. Steps wholly inside the row run unmasked.
template <int M, int T, int U>
__device__ __forceinline__ float bwd_dot_step(const float* yr, const float* gr, int base, int L, float s) {
    f32x4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        a[u] = load4m<M, false>(yr, base + (u * T + (int)threadIdx.x) * 4, L, 0.f);
        b[u] = load4m<M, false>(gr, base + (u * T + (int)threadIdx.x) * 4, L, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) s += dot4(a[u], b[u]);
    return s;
}

template <int M, int T, int U>
__device__ __forceinline__ void bwd_out_step(const float* yr, const float* gr, float* xr, int base, int L, float s) {
    f32x4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        a[u] = load4m<M, true>(yr, base + (u * T + (int)threadIdx.x) * 4, L, 0.f);
        b[u] = load4m<M, true>(gr, base + (u * T + (int)threadIdx.x) * 4, L, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) store4m<M, true>(xr, base + (u * T + (int)threadIdx.x) * 4, L, a[u] * (b[u] - s));
}

template <int T, int U, bool VEC>
__global__ __launch_bounds__(T) void fr_red_softmax_bwd_f32(const float* y, const float* dy, float* dx, int rows,
                                                            int cols, int64_t y_rs, int64_t dy_rs, int64_t dx_rs,
                                                            const int32_t* __restrict__ lengths) {
    constexpr int STEP = T * 4 * U;
    __shared__ float sl[T / kWave];
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const int L = row_len(lengths, r, cols);
        const int full = L - L % STEP;
        const float* yr = y + (int64_t)r * y_rs;
        const float* gr = dy + (int64_t)r * dy_rs;
        float s = 0.f;
        int base = 0;
        for (; base < full; base += STEP) s = bwd_dot_step<body_mask<VEC>(), T, U>(yr, gr, base, L, s);
        if (base < L) s = bwd_dot_step<tail_mask<VEC>(), T, U>(yr, gr, base, L, s);
        s = group_reduce<kWave>(s, OpSum());
        s = block_fold(s, sl, T / kWave, OpSum());
        float* xr = dx + (int64_t)r * dx_rs;
        for (base = 0; base < full; base += STEP) bwd_out_step<body_mask<VEC>(), T, U>(yr, gr, xr, base, L, s);
        if (base < L) bwd_out_step<tail_mask<VEC>(), T, U>(yr, gr, xr, base, L, s);
        __syncthreads();  // the slots are rewritten by the next row
    }
}

// ------------------------------------------------------------------ launchers
namespace {

using SmFn = void (*)(const float*, float*, int, int, int64_t, int64_t, const int32_t*, int32_t*);
using PartFn = void (*)(const float*, int, int, int64_t, const int32_t*, uint64_t*, int);
using FinFn = void (*)(const float*, float*, int, int, int64_t, int64_t, const int32_t*, int32_t*,
                       const uint64_t*, int);

template <int M>
SmFn pick_per_m(int seg, int nv, int rpw) {
    if (rpw == 4) {
        if (seg != 64) return nullptr;
        switch (nv) {
            case 1: return fr_per_softmax_f32<64, 1, M, 4>;
            case 2: return fr_per_softmax_f32<64, 2, M, 4>;
            case 4: return fr_per_softmax_f32<64, 4, M, 4>;
        }
        return nullptr;
    }
    if (rpw == 2) {
        if (seg == 32) return nv == 8 ? fr_per_softmax_f32<32, 8, M, 2> : nullptr;
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
        case 8: return nv == 1 ? fr_per_softmax_f32<8, 1, M, 1> : nullptr;
        case 16: return nv == 1 ? fr_per_softmax_f32<16, 1, M, 1> : nullptr;
        case 32:
            switch (nv) {
                case 1: return fr_per_softmax_f32<32, 1, M, 1>;
                case 2: return fr_per_softmax_f32<32, 2, M, 1>;
                case 4: return fr_per_softmax_f32<32, 4, M, 1>;
                case 8: return fr_per_softmax_f32<32, 8, M, 1>;
            }
            return nullptr;
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

using OneFn = void (*)(const float*, float*, int, int, int64_t, int64_t, const int32_t*, int32_t*, void*, int64_t);

template <bool VEC>
OneFn pick_one(int threads, int nv) {
    if (threads == 256 && nv == 8) return fr_split_softmax_one<256, 8, VEC>;
    if (threads == 256 && nv == 4) return fr_split_softmax_one<256, 4, VEC>;
    if (threads == 512 && nv == 4) return fr_split_softmax_one<512, 4, VEC>;
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

namespace {
using BwdFn = void (*)(const float*, const float*, float*, int, int, int64_t, int64_t, int64_t, const int32_t*);

template <int M>
BwdFn pick_bwd_per_m(int seg, int nv, int rpw) {
    if (rpw == 2) {
        if (seg != 64) return nullptr;
        switch (nv) {
            case 1: return fr_per_softmax_bwd_f32<64, 1, M, 2>;
            case 2: return fr_per_softmax_bwd_f32<64, 2, M, 2>;
            case 4: return fr_per_softmax_bwd_f32<64, 4, M, 2>;
        }
        return nullptr;
    }
    if (rpw != 1) return nullptr;
    switch (seg) {
        case 8: return nv == 1 ? fr_per_softmax_bwd_f32<8, 1, M, 1> : nullptr;
        case 16: return nv == 1 ? fr_per_softmax_bwd_f32<16, 1, M, 1> : nullptr;
        case 32: return nv == 1 ? fr_per_softmax_bwd_f32<32, 1, M, 1> : nullptr;
        case 64:
            switch (nv) {
                case 1: return fr_per_softmax_bwd_f32<64, 1, M, 1>;
                case 2: return fr_per_softmax_bwd_f32<64, 2, M, 1>;
                case 4: return fr_per_softmax_bwd_f32<64, 4, M, 1>;
                case 8: return fr_per_softmax_bwd_f32<64, 8, M, 1>;
            }
    }
    return nullptr;
}

template <bool VEC>
BwdFn pick_bwd_red(int threads, int u) {
    if (threads == 256 && u == 4) return fr_red_softmax_bwd_f32<256, 4, VEC>;
    if (threads == 512 && u == 2) return fr_red_softmax_bwd_f32<512, 2, VEC>;
    return nullptr;
}
}  // namespace

hipError_t launch_softmax_bwd(const fr_plan& p, const SoftmaxBwdArgs& a, hipStream_t s) {
    const bool vec = p.vec16 != 0;
    BwdFn f = nullptr;
    if (p.form == FR_FORM_PER) {
        const int rpw = p.rows_per_wg / (256 / p.seg);
        const int mask = !vec ? kScalar
                              : (a.lengths ? kElem
                                           : (a.cols == 4 * p.seg * p.vec ? kNone : (a.cols % 4 == 0 ? kVec : kElem)));
        switch (mask) {
            case kNone: f = pick_bwd_per_m<kNone>(p.seg, p.vec, rpw); break;
            case kVec: f = pick_bwd_per_m<kVec>(p.seg, p.vec, rpw); break;
            case kElem: f = pick_bwd_per_m<kElem>(p.seg, p.vec, rpw); break;
            default: f = pick_bwd_per_m<kScalar>(p.seg, p.vec, rpw); break;
        }
    } else if (p.form == FR_FORM_RED) {
        f = vec ? pick_bwd_red<true>(p.threads, p.vec) : pick_bwd_red<false>(p.threads, p.vec);
    }
    if (!f) return hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(f, dim3((unsigned)p.grid), dim3(p.form == FR_FORM_PER ? 256 : p.threads), 0, s, a.y, a.dy,
                       a.dx, a.rows, a.cols, a.y_rs, a.dy_rs, a.dx_rs, a.lengths);
    return hipGetLastError();
}

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
        if (a.rows > kOnePassMaxRows) return hipErrorInvalidDeviceFunction;
        OneFn one = vec ? pick_one<true>(p.threads, p.vec) : pick_one<false>(p.threads, p.vec);
        if (!one) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(one, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.y, a.rows, a.cols, a.x_rs,
                           a.y_rs, a.lengths, a.argmax, a.ws, a.wait_ticks);
        return hipGetLastError();
    }
    if (p.form == FR_FORM_SPLIT) {
        PartFn part;
        FinFn fin;
        if (vec) pick_split<true>(p.threads, p.vec, &part, &fin);
        else pick_split<false>(p.threads, p.vec, &part, &fin);
        if (!part || !fin) return hipErrorInvalidDeviceFunction;
        uint64_t* ws = reinterpret_cast<uint64_t*>(static_cast<char*>(a.ws) + kSplitWsSlots);
        hipLaunchKernelGGL(part, dim3((unsigned)p.grid), dim3(p.threads), 0, s, a.x, a.rows, a.cols, a.x_rs,
                           a.lengths, ws, p.splits);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fin, dim3((unsigned)p.grid2), dim3(p.threads), 0, s, a.x, a.y, a.rows, a.cols, a.x_rs,
                           a.y_rs, a.lengths, a.argmax, (const uint64_t*)ws, p.splits);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

hipError_t launch_softmax_ws_init(void* ws, uint64_t ws_bytes, hipStream_t s) {
    const int64_t nwords = (int64_t)(ws_bytes / 4);
    hipLaunchKernelGGL(fr_split_softmax_init, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(ws), nwords);
    return hipGetLastError();
}

}  // namespace fr
