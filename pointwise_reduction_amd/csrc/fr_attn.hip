// fr_attn.hip - decode attention split over the keys ("Stax (4): GPU Codegen
// and Dynamic Shapes", 9.10: attention is a row softmax between two
// contractions; the triple (m, l, a) = (max_j s_j, sum_j e^{s_j - m},
// sum_j e^{s_j - m} v_j) of a key segment merges with (+) like the (m, d)
// pair of 9.5, so the keys of one query row can be split across workgroups,
// which is what the decode template does; hello-gpu, Chapter 12, 12.1 and
// 12.3 for the one-row definition and the rescale).
//
// One query row per (batch b, query head h); the G = Hq / Hkv query heads of
// one key-value head share its keys and values, so a workgroup serves all G
// of them and every key and value byte is read once.
//
//   fr_attn_part     workgroup (chunk c, key-value head, batch): the keys
//                    [c * kAttnChunk, ...) of that head. Scores s = scale q.k
//                    for the G rows (bf16: 16x16 tiles of the matrix cores,
//                    query rows padded to 16; fp32: lane groups of VPR lanes
//                    hold one key row each and sum their partial dots), the
//                    chunk maximum and sum of e^{s - m}, then a = sum p v on
//                    the vector units (p stays fp32). Writes the chunk's
//                    (m, l, a[D]) for each of the G rows.
//   fr_attn_combine  workgroup per (b, h): merges the chunk triples with (+) (the
//                    largest maximum first, then weighted sums in chunk
//                    order), writes o = a / l and lse = m + log l.
//
// Memory-bound: each key and value row is read once. The score contraction
// runs on the matrix cores for bf16, which takes it off the vector units;
// the value contraction stays on the vector units because its left operand
// (the probabilities) would lose precision as bf16.
#include <limits.h>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

constexpr int kAttnValueBatch = 16;  // value vectors in flight per lane
constexpr int kAttnKeyTiles = 2;     // bf16: 16-key tiles whose loads are in flight together

// Element access for fp32 and bf16 (uint16 bits) rows, 16 bytes at a time.
template <typename DT>
struct Elems;
template <>
struct Elems<float> {
    static constexpr int kPerVec = 4;
    __device__ __forceinline__ static void unpack(f32x4 raw, float* out) {
        out[0] = raw.x;
        out[1] = raw.y;
        out[2] = raw.z;
        out[3] = raw.w;
    }
    // q . k over the 4 elements of one vector
    __device__ __forceinline__ static float dot(f32x4 a, f32x4 b) {
        return ((a.x * b.x + a.y * b.y) + a.z * b.z) + a.w * b.w;
    }
};
template <>
struct Elems<uint16_t> {
    static constexpr int kPerVec = 8;
    __device__ __forceinline__ static void unpack(f32x4 raw, float* out) {
        const u32x4 w = __builtin_bit_cast(u32x4, raw);
        out[0] = bf16_lo(w.x);
        out[1] = bf16_hi(w.x);
        out[2] = bf16_lo(w.y);
        out[3] = bf16_hi(w.y);
        out[4] = bf16_lo(w.z);
        out[5] = bf16_hi(w.z);
        out[6] = bf16_lo(w.w);
        out[7] = bf16_hi(w.w);
    }
};

__device__ __forceinline__ f32x4 ld16(const void* p) { return *static_cast<const f32x4*>(p); }

// Sum over aligned groups of W lanes (W a power of two <= 64), every lane
// of a group ending with the group's sum: DPP below 16 lanes, ds_bpermute
// above. Fixed order.
template <int W>
__device__ __forceinline__ float lane_group_sum(float v) {
    return group_reduce<W>(v, OpSum());
}

// Sum over the lanes that hold the same vector index in the KPW lane groups
// of a wave (lanes l, l ^ VPR, l ^ 2 VPR, ...): xor butterflies through
// ds_bpermute in a fixed order. The operator is a commutative add, so every
// lane of an orbit ends with the same bits.
template <int VPR>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
    for (int st = VPR; st < kWave; st <<= 1) v += shfl_xor(v, st);
    return v;
}

template <int D, int G, typename DT>
__global__ __launch_bounds__(256) void fr_attn_part(const DT* __restrict__ q, const DT* __restrict__ k,
                                                    const DT* __restrict__ v, const int32_t* __restrict__ lengths,
                                                    float* __restrict__ ws, int Hq, int Hkv, int S, int nchunks,
                                                    float scale) {
    using E = Elems<DT>;
    constexpr int EPV = E::kPerVec;                // elements per 16-byte vector
    constexpr int VPR = D / EPV;                   // vectors per key row = lanes per key
    constexpr int KPW = kWave / VPR;               // keys per wave instruction
    constexpr int KPS = 4 * KPW;                   // keys per workgroup step (4 waves)
    constexpr int NSTEP = kAttnChunk / KPS;        // steps per chunk
    constexpr int BATCH = NSTEP < 8 ? NSTEP : 8;   // key vectors loaded per lane before use (fp32)
    constexpr int VB = NSTEP < kAttnValueBatch ? NSTEP : kAttnValueBatch;  // value vectors likewise
    static_assert(kAttnChunk % KPS == 0 && NSTEP % BATCH == 0 && NSTEP % VB == 0, "chunk geometry");
    constexpr int SLOT = D + 4;                    // floats per (row, chunk) triple: m, l, pad, pad, a[D]
    __shared__ float s_p[G][kAttnChunk];           // scores, then e^{s - m}
    __shared__ float s_red[2][G][4];               // cross-wave folds of the maxima and sums
    __shared__ float s_acc[4][G][D];               // per-wave partial a

    const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int grp = lane / VPR, vl = lane % VPR;
    int L = lengths ? lengths[b] : S;
    L = L < 0 ? 0 : (L > S ? S : L);
    const int c0 = c * kAttnChunk;
    if (c0 >= L) return;  // the combine reads only chunks below len_b
    const int64_t kv_base = ((int64_t)b * Hkv + hk) * S;
    const int h0 = hk * G;
    // the head's keys and values below len_b as buffer resources: a key past
    // it reads zeros through the range check, so no load sits under a
    // branch (the compiler's waits then count the loads in flight exactly)
    const uint32_t kvb = (uint32_t)L * D * (uint32_t)sizeof(DT);  // < 2^31 (checked by the entry point)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<DT*>(k + kv_base * D), 0, (int)kvb, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<DT*>(v + kv_base * D), 0, (int)kvb, kBufferRsrcWord3);
    auto kv_load = [&](__amdgpu_buffer_rsrc_t r, int j, int e) __attribute__((always_inline)) {
        // element e of key j; j >= len_b (or j past the chunk) reads zeros
        return __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(((uint32_t)j * D + e) * sizeof(DT)), 0,
                                                         2 /* non-temporal */));
    };

    if constexpr (EPV == 8) {
        // bf16: the scores of 16 keys x 16 query rows (rows >= G are zero)
        // are one 16x16 tile of v_mfma_f32_16x16x32_bf16 per 32 dims: lane l
        // holds query row l % 16 and key l % 16 at dims 8 (l / 16) .. +7 of
        // each 32-dim slice, and receives the scores of key l % 16 for rows
        // 4 (l / 16) .. +3. Wave w scores the keys 64 w .. 64 w + 63 of the chunk.
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        constexpr int NS = D / 32;  // 32-dim slices
        constexpr int TPW = kAttnChunk / (4 * 16);  // key tiles per wave
        const int n = lane & 15, kq = lane >> 4;
        f32x4 qa[NS];
#pragma unroll
        for (int sl = 0; sl < NS; ++sl)
            qa[sl] = n < G ? ld16(q + ((int64_t)b * Hq + h0 + n) * D + sl * 32 + kq * 8) : f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr int KT = TPW < kAttnKeyTiles ? TPW : kAttnKeyTiles;
#pragma unroll
        for (int t0 = 0; t0 < TPW; t0 += KT) {
            f32x4 kb[KT][NS];
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int j = c0 + w * 64 + (t0 + t) * 16 + n;
#pragma unroll
                for (int sl = 0; sl < NS; ++sl)
                    kb[t][sl] = kv_load(rk, j, sl * 32 + kq * 8);
            }
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sl = 0; sl < NS; ++sl)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[sl]),
                                                                  __builtin_bit_cast(bf16x8, kb[t][sl]), acc, 0, 0, 0);
                const int jj = w * 64 + (t0 + t) * 16 + n;  // key index within the chunk
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int g = kq * 4 + i;
                    if (g < G) s_p[g][jj] = c0 + jj < L ? acc[i] * scale : -INFINITY;
                }
            }
        }
    } else {
    // fp32: lane groups of VPR lanes hold one key row; partial dot products
    // are summed across the group
    f32x4 qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qs[g] = ld16(q + ((int64_t)b * Hq + h0 + g) * D + vl * EPV);

    // scores: step i, wave w, lane group grp hold key c0 + i * KPS + w * KPW + grp
#pragma unroll
    for (int i0 = 0; i0 < NSTEP; i0 += BATCH) {
        f32x4 kv[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int j = c0 + (i0 + u) * KPS + w * KPW + grp;
            kv[u] = kv_load(rk, j, vl * EPV);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int jj = (i0 + u) * KPS + w * KPW + grp;  // key index within the chunk
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float d = lane_group_sum<VPR>(E::dot(qs[g], kv[u]));
                if (vl == 0) s_p[g][jj] = c0 + jj < L ? d * scale : -INFINITY;
            }
        }
    }
    }
    // the first batch of values goes out now, so that its latency overlaps
    // the chunk softmax below
    f32x4 vpre[VB];
#pragma unroll
    for (int u = 0; u < VB; ++u) {
        const int j = c0 + u * KPS + w * KPW + grp;
        // past len_b: zeros (the tail is never read, and p = 0 there)
        vpre[u] = kv_load(rv, j, vl * EPV);
    }
    __syncthreads();

    // chunk maximum and sum of e^{s - m}: thread t owns key t of the chunk
    static_assert(kAttnChunk == 256, "one key per thread below");
    float m[G], lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = group_reduce<kWave>(s_p[g][tid], OpMax());
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) s_red[0][g][w] = m[g];
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
        m[g] = fmax_nan(fmax_nan(s_red[0][g][0], s_red[0][g][1]), fmax_nan(s_red[0][g][2], s_red[0][g][3]));
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float p = exp_fast(s_p[g][tid] - m[g]);  // masked keys: e^{-inf} = 0
        s_p[g][tid] = p;
        lsum[g] = group_reduce<kWave>(p, OpSum());
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) s_red[1][g][w] = lsum[g];
    }
    __syncthreads();  // e^{s - m} and the sums are visible

    // a = sum_j p_j v_j: lane (grp, vl) accumulates its vector slice of the
    // keys it loads, then lanes with the same slice are summed
    float acc[G][EPV];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[g][e] = 0.f;
#pragma unroll
    for (int i0 = 0; i0 < NSTEP; i0 += VB) {
        f32x4 vv[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int j = c0 + (i0 + u) * KPS + w * KPW + grp;
            vv[u] = i0 == 0 ? vpre[u] : kv_load(rv, j, vl * EPV);
        }
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int jj = (i0 + u) * KPS + w * KPW + grp;
            float ve[EPV];
            E::unpack(vv[u], ve);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = s_p[g][jj];
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[g][e] += p * ve[e];
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[g][e] = across_groups_sum<VPR>(acc[g][e]);
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPV; ++e) s_acc[w][g][vl * EPV + e] = acc[g][e];
    }
    __syncthreads();
    // write the G triples of this chunk: (m, l, 0, 0, a[D])
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        float* slot = ws + (((int64_t)b * Hq + h0 + g) * nchunks + c) * SLOT;
        slot[4 + d] = (s_acc[0][g][d] + s_acc[1][g][d]) + (s_acc[2][g][d] + s_acc[3][g][d]);
        if (d == 0) {
            slot[0] = m[g];
            slot[1] = (s_red[1][g][0] + s_red[1][g][1]) + (s_red[1][g][2] + s_red[1][g][3]);
        }
    }
}

__device__ __forceinline__ void store_out(float* o, int d, float x) { o[d] = x; }
__device__ __forceinline__ void store_out(uint16_t* o, int d, float x) {
    o[d] = (uint16_t)(pack_bf16(x, 0.f) & 0xFFFFu);
}

// Workgroup of four waves per (b, h); lane l owns dims l, l + 64, ... The
// chunk triples of the row are merged as one (+) over all of them: mu = the
// largest chunk maximum, weights f_c = e^{m_c - mu} (0 for a state whose
// maximum is -inf, the identity), l = sum_c f_c l_c and a = sum_c f_c a_c.
// Wave w sums the chunks of the w-th quarter of each group of 64 in chunk
// order; the four quarter sums are added in wave order. Every thread derives
// mu and l itself (the same reads, the same order), so all agree.
template <int D, typename DT>
__global__ __launch_bounds__(256) void fr_attn_combine(const float* __restrict__ ws,
                                                       const int32_t* __restrict__ lengths, DT* __restrict__ o,
                                                       float* __restrict__ lse, int Hq, int S, int nchunks) {
    constexpr int SLOT = D + 4;
    constexpr int PER = D / kWave;
    __shared__ float s_f[kWave];
    __shared__ float s_a[4][D];
    const int row = blockIdx.x;  // b * Hq + h
    const int b = row / Hq;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    int L = lengths ? lengths[b] : S;
    L = L < 0 ? 0 : (L > S ? S : L);
    const int nc = (L + kAttnChunk - 1) / kAttnChunk;
    DT* orow = o + (int64_t)row * D;
    if (nc == 0) {
        if (w == 0) {
#pragma unroll
            for (int e = 0; e < PER; ++e) store_out(orow, lane + e * kWave, 0.f);
            if (lse && lane == 0) lse[row] = -INFINITY;
        }
        return;
    }
    const float* base = ws + (int64_t)row * nchunks * SLOT;
    float mu = -INFINITY;
    float ll = 0.f;
    float a[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) a[e] = 0.f;
    if (nc <= kWave) {
        // one group of chunks: every read is issued before any arithmetic
        // (same operations in the same order as the general loop below)
        constexpr int QMAX = kWave / 4;
        const int q0 = (nc * w) / 4, q1 = (nc * (w + 1)) / 4;
        float mc = -INFINITY, lc = 0.f;
        if (lane < nc) {
            mc = base[(int64_t)lane * SLOT];
            lc = base[(int64_t)lane * SLOT + 1];
        }
        float av[QMAX][PER];
#pragma unroll
        for (int j = 0; j < QMAX; ++j)
#pragma unroll
            for (int e = 0; e < PER; ++e)
                av[j][e] = q0 + j < q1 ? base[(int64_t)(q0 + j) * SLOT + 4 + lane + e * kWave] : 0.f;
        mu = group_reduce<kWave>(mc, OpMax());
        const float f = lane < nc && mc != -INFINITY ? exp_fast(mc - mu) : 0.f;
        ll = group_reduce<kWave>(f * lc, OpSum());
#pragma unroll
        for (int j = 0; j < QMAX; ++j) {
            const float fj = __shfl(f, q0 + j, kWave);
            if (q0 + j < q1) {
#pragma unroll
                for (int e = 0; e < PER; ++e) a[e] += fj * av[j][e];
            }
        }
    } else {
    for (int g0 = 0; g0 < nc; g0 += kWave) {
        const int c = g0 + lane;
        mu = fmax_nan(mu, group_reduce<kWave>(c < nc ? base[(int64_t)c * SLOT] : -INFINITY, OpMax()));
    }
    for (int g0 = 0; g0 < nc; g0 += kWave) {
        const int c = g0 + lane;
        float f = 0.f, lc = 0.f;
        if (c < nc) {
            const float mc = base[(int64_t)c * SLOT];
            lc = base[(int64_t)c * SLOT + 1];
            f = mc == -INFINITY ? 0.f : exp_fast(mc - mu);
        }
        ll += group_reduce<kWave>(f * lc, OpSum());
        if (w == 0) s_f[lane] = f;
        __syncthreads();
        const int n = nc - g0 < kWave ? nc - g0 : kWave;
        const int q0 = (n * w) / 4, q1 = (n * (w + 1)) / 4;  // this wave's quarter of the group
#pragma unroll 4
        for (int j = q0; j < q1; ++j) {
            const float fj = s_f[j];
            const float* slot = base + (int64_t)(g0 + j) * SLOT + 4;
#pragma unroll
            for (int e = 0; e < PER; ++e) a[e] += fj * slot[lane + e * kWave];
        }
        __syncthreads();  // s_f is rewritten by the next group
    }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) s_a[w][lane + e * kWave] = a[e];
    __syncthreads();
    if (w == 0) {
        const float inv = 1.0f / ll;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int d = lane + e * kWave;
            store_out(orow, d, ((s_a[0][d] + s_a[1][d]) + (s_a[2][d] + s_a[3][d])) * inv);
        }
        if (lse && lane == 0) lse[row] = mu + logf(ll);
    }
}

namespace {

template <typename DT>
auto pick_part(int D, int G) -> void (*)(const DT*, const DT*, const DT*, const int32_t*, float*, int, int, int, int,
                                         float) {
    if (D == 128) {
        switch (G) {
            case 1: return fr_attn_part<128, 1, DT>;
            case 2: return fr_attn_part<128, 2, DT>;
            case 4: return fr_attn_part<128, 4, DT>;
            case 8: return fr_attn_part<128, 8, DT>;
        }
    } else if (D == 64) {
        switch (G) {
            case 1: return fr_attn_part<64, 1, DT>;
            case 2: return fr_attn_part<64, 2, DT>;
            case 4: return fr_attn_part<64, 4, DT>;
            case 8: return fr_attn_part<64, 8, DT>;
        }
    }
    return nullptr;
}

template <typename DT>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
    auto part = pick_part<DT>(a.dim, a.heads_q / a.heads_kv);
    if (!part) return hipErrorInvalidDeviceFunction;
    const int nchunks = (int)attn_chunks(a.seq);
    if (nchunks > 0) {  // no keys: the combine alone writes o = 0, lse = -inf
        hipLaunchKernelGGL(part, dim3((unsigned)nchunks, (unsigned)a.heads_kv, (unsigned)a.batch), dim3(256), 0, s,
                           static_cast<const DT*>(a.q), static_cast<const DT*>(a.k), static_cast<const DT*>(a.v),
                           a.lengths, a.ws, a.heads_q, a.heads_kv, a.seq, nchunks, a.scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    auto comb = a.dim == 128 ? fr_attn_combine<128, DT> : fr_attn_combine<64, DT>;
    hipLaunchKernelGGL(comb, dim3((unsigned)(a.batch * a.heads_q)), dim3(256), 0, s, a.ws, a.lengths,
                       static_cast<DT*>(a.o), a.lse, a.heads_q, a.seq, nchunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
    return a.bf16 ? launch_attn_t<uint16_t>(a, s) : launch_attn_t<float>(a, s);
}

}  // namespace fr
