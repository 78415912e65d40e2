// fr_attn_block.hip - tiled single-pass attention over blocks of query rows
// ("Stax (4): GPU Codegen and Dynamic Shapes", 9.10: Theorem 9.2's tiled
// algorithm, Figure 9.2; the (m, l, a) triple updated online; LSE = m +
// log l kept for the backward pass; the causal mask of Listing 9.7).
//
// One workgroup of 8 waves owns a block of 256 query rows of one head (each
// wave 32 rows) and scans the keys and values in blocks of 64. Both products
// run on the matrix cores (v_mfma_f32_16x16x32_bf16, lane l: A row l % 16,
// B column l % 16, k = 8 (l / 16) .. +7; D rows 4 (l / 16) .. +3, column
// l % 16):
//   S^T = K Q^T   A = a K tile (key rows, read from LDS), B = the wave's Q
//                 rows (read from LDS). D holds, for lane l's query (column
//                 l % 16), the keys 4 (l / 16) .. +3 of each 16-key tile.
//   O  += P V     A = P, as two bf16 parts (its rounding and the rounding
//                 of the remainder, two products), so that P enters at about
//                 fp32 accuracy. A lane's D registers of two consecutive key tiles
//                 hold exactly 8 keys of its own query: they are its A
//                 fragment, with the k positions of the 32-key step mapped
//                 to keys 4 (l / 16) + i and 16 + 4 (l / 16) + i. B = V with
//                 the same key mapping, read from the row-major V tile in LDS
//                 with gfx950's transposing read (ds_read_b64_tr_b16: within
//                 each 16-lane group, lane j's element e comes from the
//                 8-byte piece that lane 4 e + j / 4 addresses, component
//                 j % 4; two reads per fragment).
// Computing S transposed is what lets P stay in the registers that received
// it: no exchange between lanes before the second product. The online
// softmax works in base 2 (the scale carries log2 e); a row's maximum and
// sum need one butterfly over the 4 lane groups; the rescale factor of a row
// reaches the O rows 4 (l / 16) + i with one shuffle each.
// LDS holds the block's Q rows and two K and two V blocks (147 KB at 128
// dimensions: one workgroup, 8 waves, per CU). K runs one block ahead of V,
// so a step forms the next block's S^T while it turns this block's S^T into
// P and accumulates P V, stages the blocks in flight (loaded into registers
// by buffer loads one step earlier) into the buffers the previous step
// finished with, and needs one barrier. With the causal mask, blocks wholly
// above the diagonal are skipped, and each XCD takes its heads' query blocks
// heaviest first.
#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v* lds_s4p;

constexpr int kBM = kAttnBlockRows;  // query rows per workgroup
constexpr int kBN = 64;              // keys per block
constexpr int kWaves = kBM / 32;     // 32 query rows per wave
constexpr int kThreads = kWaves * 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, each with its own L2
// Causal order: an XCD takes its heads two at a time, each pair's query
// blocks heaviest first. Longest-first over the pair keeps the CUs busy to
// the end, and two heads' K and V (4 MB at 4096 x 128) mostly stay in the
// XCD's L2. At 4096 x 128 causal: one head at a time 374 us, pairs 309,
// four 302-320, all eight 309-331.
constexpr int kHeadGroup = 2;
constexpr float kLazy = 8.0f;  // P <= 2^8 between rescales (base-2 exponent)
// LDS row padding (bf16 elements) of the K, V and Q tiles: rows 288 bytes
// apart (D = 128) keep every fragment read free of bank conflicts. An
// earlier layout (V staged transposed, consecutive lanes on different
// dimension octets) spent 68% of the LDS-active cycles in bank conflicts.
constexpr int kKPad = 16;

__device__ __forceinline__ f32x4 mfma(f32x4 a, f32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ f32x4 ld16g(const uint16_t* p) { return *reinterpret_cast<const f32x4*>(p); }

// Two fp32 values p0, p1 as two packed bf16 pairs: their roundings to
// nearest even (hw) and the roundings of what those leave over (lw). The
// remainders p - bf16(p) are exact in fp32, so hi + lo differs from p only
// by the rounding of the remainder, at most 2^-9 of it: 2^-18 p. The
// matrix cores take both pairs, so P V carries P to about fp32 accuracy
// instead of the 2^-9 of one bf16 rounding.
__device__ __forceinline__ void split2(float p0, float p1, float& hw, float& lw) {
    const uint32_t h = pack_bf16(p0, p1);
    const float r0 = p0 - __builtin_bit_cast(float, h << 16);
    const float r1 = p1 - __builtin_bit_cast(float, h & 0xFFFF0000u);
    hw = __builtin_bit_cast(float, h);
    lw = __builtin_bit_cast(float, pack_bf16(r0, r1));
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fr_attn_block_bf16(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 uint16_t* __restrict__ o, float* __restrict__ lse,
                                                                 int Hq, int Hkv, int Nq, int Nk, float scale_log2) {
    constexpr int NS = D / 32;        // 32-dim steps of S^T
    constexpr int NT = D / 16;        // 16-dim tiles of O
    constexpr int KCH = kBN * D / 8;  // 16-byte chunks of a K (or V) block
    constexpr int KPT = KCH / kThreads;
    constexpr int KLD = D + kKPad;
    static_assert(KCH % kThreads == 0, "block shape");
    // K and V blocks, two of each (K runs one block ahead of V), and the
    // workgroup's Q rows (147 KB in all for D = 128: one workgroup per CU)
    __shared__ __align__(16) uint16_t sk[2][kBN * KLD];
    __shared__ __align__(16) uint16_t sv[2][kBN * KLD];
    __shared__ __align__(16) uint16_t sq[kBM * KLD];

    // XCD-aware order: the dispatcher sends workgroup L to XCD L % 8, so
    // logical tile L % 8 * (G / 8) + L / 8 gives each XCD a contiguous run of
    // tiles, i.e. whole heads, whose K and V then stay in that XCD's L2
    // (causal: each XCD's heads are taken heaviest query block first across
    // all of them, longest-first list scheduling over the XCD's CUs)
    const int nqb = (Nq + kBM - 1) / kBM;
    const int G = (int)gridDim.x;
    const int L = (int)blockIdx.x;
    int qi0, hb;  // query block (0 = the heaviest when causal), head x batch
    if (G % kXcds == 0) {
        const int x = L % kXcds, i = L / kXcds, R = G / kXcds;
        if (CAUSAL && R % nqb == 0) {
            const int hpx = R / nqb;  // whole heads per XCD
            // groups of kHeadGroup heads, each group's query blocks heaviest
            // first across its heads
            const int hg = hpx % kHeadGroup == 0 ? kHeadGroup : hpx;
            const int gi = i / (hg * nqb), r = i % (hg * nqb);
            qi0 = r / hg;
            hb = x * hpx + gi * hg + r % hg;
        } else {
            const int tile = x * R + i;
            qi0 = tile % nqb;
            hb = tile / nqb;
        }
    } else {
        qi0 = L % nqb;
        hb = L / nqb;
    }
    const int qb = CAUSAL ? nqb - 1 - qi0 : qi0;
    const int h = hb % Hq, b = hb / Hq;
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int64_t qrow0 = ((int64_t)b * Hq + h) * Nq;
    const int64_t kv0 = ((int64_t)b * Hkv + hk) * Nk;
    const int qbase = qb * kBM + w * 32;  // the wave's first query row

    // the workgroup's Q rows in LDS; B fragments are read from there per key
    // block (in registers they would leave too few for the pipeline)
#pragma unroll
    for (int r = 0; r < kBM * D / 8 / kThreads; ++r) {
        const int c = tid + kThreads * r, row = c / (D / 8), oc = c % (D / 8);
        const int qi = qb * kBM + row;
        *reinterpret_cast<f32x4*>(&sq[row * KLD + 8 * oc]) =
            qi < Nq ? ld16g(q + (qrow0 + qi) * D + 8 * oc) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int nkb = (Nk + kBN - 1) / kBN;
    if (CAUSAL) {
        const int last = qb * kBM + kBM - 1;  // the block's last query sees keys <= last
        const int need = last / kBN + 1;
        nkb = need < nkb ? need : nkb;
    }

    // K block jk and V block jv, in registers until staged. Buffer loads
    // over the head's keys: rows past the end read zeros without a memory
    // access (the range check), and so does a block past the last (its
    // offsets point past the range). No branch around a load, so the
    // compiler's waits count the loads in flight exactly.
    const uint32_t kvbytes = (uint32_t)Nk * D * 2;  // < 2^31 (checked by the entry point)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + kv0 * D), 0, (int)kvbytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v + kv0 * D), 0, (int)kvbytes, kBufferRsrcWord3);
    f32x4 kr[KPT], vr[KPT];
    auto fetch = [&](int jk, int jv) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int c = tid + kThreads * r, jr = c / (D / 8), oc = c % (D / 8);
            const uint32_t o1 = jk < nkb ? (uint32_t)((jk * kBN + jr) * D + 8 * oc) * 2u : kvbytes;
            const uint32_t o2 = jv < nkb ? (uint32_t)((jv * kBN + jr) * D + 8 * oc) * 2u : kvbytes;
            kr[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)o1, 0, 0));
            vr[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)o2, 0, 0));
        }
    };
    auto stage_k = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int c = tid + kThreads * r, j = c / (D / 8), oc = c % (D / 8);
            *reinterpret_cast<f32x4*>(&sk[buf][j * KLD + 8 * oc]) = kr[r];
        }
    };
    auto stage_v = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int c = tid + kThreads * r, j = c / (D / 8), oc = c % (D / 8);
            *reinterpret_cast<f32x4*>(&sv[buf][j * KLD + 8 * oc]) = vr[r];
        }
    };

    f32x4 acc[2][NT];
#pragma unroll
    for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[bq][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    // S^T of the K block in sk[buf]: 4 key tiles x 2 query tiles
    auto s_block = [&](int buf, f32x4 (&st)[4][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int bq = 0; bq < 2; ++bq) st[t][bq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&sk[buf][(16 * t + n) * KLD + 32 * s + 8 * g]);
#pragma unroll
                for (int bq = 0; bq < 2; ++bq) {
                    const f32x4 qv =
                        *reinterpret_cast<const f32x4*>(&sq[(w * 32 + 16 * bq + n) * KLD + 32 * s + 8 * g]);
                    st[t][bq] = mfma(a, qv, st[t][bq]);
                }
            }
    };
    // online softmax per query (lane's column), base 2, against a
    // reference: m holds a per-row reference maximum (scaled), the exponents
    // are exp2(fma(s, c, -m)) and l and the O rows are relative to it. The
    // reference moves (and O, l are rescaled) only when some row of the wave
    // sees a block maximum more than kLazy above its reference, so P stays
    // <= 2^kLazy and o = a / l is unchanged; after the first blocks the
    // rescale is rarely needed. Blocks wholly inside the keys (and, causal,
    // wholly at or below every query of the wave) need no mask. The first
    // half (mask, maxima, rescale) ends in branches; the second half (the
    // exponentials and sums) is branch-free, and the next block's S^T
    // products are issued beside it.
    auto softmax_max = [&](int jb, f32x4 (&st)[4][2]) __attribute__((always_inline)) {
        const bool full = (jb + 1) * kBN <= Nk && (!CAUSAL || (jb + 1) * kBN - 1 <= qbase);
        if (!full) [[unlikely]] {
#pragma unroll
            for (int bq = 0; bq < 2; ++bq) {
                const int qi = qbase + 16 * bq + n;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = jb * kBN + 16 * t + 4 * g + i;
                        if (!(j < Nk && (!CAUSAL || j <= qi))) st[t][bq][i] = -INFINITY;
                    }
            }
        }
        float mxs[2];
        bool need = false;
#pragma unroll
        for (int bq = 0; bq < 2; ++bq) {
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][bq][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            mxs[bq] = mx * scale_log2;
            need |= mxs[bq] > m[bq] + kLazy;
        }
        if (__any(need)) {
#pragma unroll
            for (int bq = 0; bq < 2; ++bq) {
                const float nm = fmaxf(m[bq], mxs[bq]);
                const float alpha = nm == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[bq] - nm);
                l[bq] *= alpha;
                m[bq] = nm;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[bq][t][i] *= a;
                }
            }
        }
    };
    auto softmax_exp = [&](f32x4 (&st)[4][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int bq = 0; bq < 2; ++bq) {
            const float mu = m[bq] == -INFINITY ? 0.f : m[bq];  // nothing seen yet: everything stays 0
            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(st[t][bq][i], scale_log2, -mu));
                    st[t][bq][i] = p;
                    sum += p;
                }
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            l[bq] += sum;
        }
    };
    // O += P V from the V block in sv[buf], two 32-key steps
    auto pv_block = [&](int buf, const f32x4 (&st)[4][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f32x4 pa[2], pl[2];  // P as bf16 pairs, and the remainders
#pragma unroll
            for (int bq = 0; bq < 2; ++bq) {
                const f32x4 lo = st[2 * kk][bq], hi = st[2 * kk + 1][bq];
                float h0, h1, h2, h3, l0, l1, l2, l3;
                split2(lo[0], lo[1], h0, l0);
                split2(lo[2], lo[3], h1, l1);
                split2(hi[0], hi[1], h2, l2);
                split2(hi[2], hi[3], h3, l3);
                pa[bq] = f32x4{h0, h1, h2, h3};
                pl[bq] = f32x4{l0, l1, l2, l3};
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                // transposing reads of the row-major V tile: lane p of lane
                // group g points at key 32 kk + 4 g + p / 4 (+ 16), dims
                // 16 t + 4 (p % 4) .. +3; lane n then receives dim 16 t + n
                // of the 4 keys
                const uint16_t* row = &sv[buf][(32 * kk + 4 * g + (n >> 2)) * KLD + 16 * t + 4 * (n & 3)];
                const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)row);
                const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(row + 16 * KLD));
                const f32x4 bv = __builtin_bit_cast(
                    f32x4, (short __attribute__((ext_vector_type(8)))){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1],
                                                                        v1[2], v1[3]});
#pragma unroll
                for (int bq = 0; bq < 2; ++bq) acc[bq][t] = mfma(pl[bq], bv, mfma(pa[bq], bv, acc[bq][t]));
            }
        }
    };

    // Pipeline over key blocks. At the top of step jb: S^T of block jb is in
    // registers, sk[(jb + 1) & 1] holds K of block jb + 1, sv[jb & 1] holds V
    // of block jb, and the registers receive K of block jb + 2 and V of
    // block jb + 1. Step jb turns S^T(jb) into P while the matrix cores form
    // S^T(jb + 1), accumulates P V(jb), stages the blocks in flight into the
    // buffers that step jb - 1 finished with, and issues the next loads. One
    // barrier per step.
    f32x4 sa[4][2], sb[4][2];
    if (nkb > 0) {
        fetch(0, 0);
        stage_k(0);
        stage_v(0);
        fetch(1, 1);
        __syncthreads();
        s_block(0, sa);  // block 0 is never past a wave's last query
        if (1 < nkb) stage_k(1);
        fetch(2, 1);  // V of block 1 was loaded above and is not staged yet: the same values again
        __syncthreads();
    }
    auto step = [&](int jb, f32x4 (&cur)[4][2], f32x4 (&nxt)[4][2]) __attribute__((always_inline)) {
        softmax_max(jb, cur);
        if (jb + 1 < nkb) s_block((jb + 1) & 1, nxt);
        softmax_exp(cur);
        pv_block(jb & 1, cur);
        if (jb + 2 < nkb) stage_k(jb & 1);
        if (jb + 1 < nkb) stage_v((jb + 1) & 1);
        fetch(jb + 3, jb + 2);
        __syncthreads();
    };
    for (int jb = 0; jb < nkb; jb += 2) {
        step(jb, sa, sb);
        if (jb + 1 < nkb) step(jb + 1, sb, sa);
    }

    // o = a / l (rows 4 g + i of each query tile); lse = (m + log2 l) ln 2.
    // The lane's position is taken afresh (mbcnt) rather than kept alive
    // across the scan, where every register is in use.
    {
    const int lane2 = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int n = lane2 & 15, g = lane2 >> 4;
#pragma unroll
    for (int bq = 0; bq < 2; ++bq) {
        const int qi = qbase + 16 * bq + n;
        if (g == 0 && qi < Nq)
            lse[qrow0 + qi] = l[bq] > 0.f ? (m[bq] + __log2f(l[bq])) * 0.69314718055994531f : -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(l[bq], 4 * g + i, 64);
            const float inv = li > 0.f ? 1.0f / li : 0.f;
            const int qr = qbase + 16 * bq + 4 * g + i;
            if (qr < Nq) {
                uint16_t* orow = o + (qrow0 + qr) * D;
#pragma unroll
                for (int t = 0; t < NT; ++t) orow[16 * t + n] = (uint16_t)(pack_bf16(acc[bq][t][i] * inv, 0.f) & 0xFFFFu);
            }
        }
    }
    }
}

hipError_t launch_attn_block(const AttnBlockArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)(a.seq_q + kBM - 1) / kBM * a.heads_q * a.batch));
    const float sl2 = a.scale * 1.4426950408889634f;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, (const uint16_t*)a.q, (const uint16_t*)a.k,
                           (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.heads_q, a.heads_kv, a.seq_q, a.seq_kv, sl2);
    };
    if (a.dim == 128) a.causal ? go(fr_attn_block_bf16<128, true>) : go(fr_attn_block_bf16<128, false>);
    else a.causal ? go(fr_attn_block_bf16<64, true>) : go(fr_attn_block_bf16<64, false>);
    return hipGetLastError();
}

}  // namespace fr
