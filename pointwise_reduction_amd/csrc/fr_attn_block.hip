// fr_attn_block.hip - tiled single-pass attention over blocks of query rows
// ("Stax (4): GPU Codegen and Dynamic Shapes", 9.10: Theorem 9.2's tiled
// algorithm, Figure 9.2; the (m, l, a) triple updated online; LSE = m +
// log l kept for the backward pass; the causal mask of Listing 9.7).
//
// One workgroup of 4 waves owns a block of 128 query rows of one head (each
// wave 32 rows) and scans the keys and values in blocks of 64. Both products
// run on the matrix cores (v_mfma_f32_16x16x32_bf16, lane l: A row l % 16,
// B column l % 16, k = 8 (l / 16) .. +7; D rows 4 (l / 16) .. +3, column
// l % 16):
//   S^T = K Q^T   A = a K tile (key rows, read from LDS), B = the wave's Q
//                 rows (registers, loaded once). D holds, for lane l's query
//                 (column l % 16), the keys 4 (l / 16) .. +3 of each 16-key
//                 tile.
//   O  += P V     A = P. A lane's D registers of two consecutive key tiles
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
// K and V are staged row-major in LDS with 16-byte writes; the next key /
// value block is loaded into registers while the current one is computed. The block's Q rows sit in LDS rather than in
// registers, which holds the kernel to 256 registers: two workgroups share a
// CU and one's softmax overlaps the other's matrix products. With the causal
// mask, blocks wholly above the diagonal are skipped and the heaviest query
// blocks of a head are launched first.
#include "fr_device.h"
#include "fr_internal.h"

namespace fr {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v* lds_s4p;

constexpr int kBM = kAttnBlockRows;  // query rows per workgroup
constexpr int kBN = 64;              // keys per block
constexpr int kWaves = 4;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, each with its own L2
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

// two fp32 -> packed bf16 (round to nearest even)
__device__ __forceinline__ float pk(float lo, float hi) { return __builtin_bit_cast(float, pack_bf16(lo, hi)); }

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fr_attn_block_bf16(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, int Hq, int Hkv, int Nq, int Nk,
                                                          float scale_log2) {
    constexpr int NS = D / 32;        // 32-dim steps of S^T
    constexpr int NT = D / 16;        // 16-dim tiles of O
    constexpr int KCH = kBN * D / 8;  // 16-byte chunks of a K block
    constexpr int KPT = KCH / 256;    // per thread
    constexpr int VPT = KPT;
    constexpr int KLD = D + kKPad;
    static_assert(KCH % 256 == 0, "block shape");
    __shared__ __align__(16) uint16_t sk[kBN * KLD];
    __shared__ __align__(16) uint16_t sv[kBN * KLD];  // V row-major, like K
    __shared__ __align__(16) uint16_t sq[kBM * KLD];

    // XCD-aware order: the dispatcher sends workgroup L to XCD L % 8, so
    // logical tile L % 8 * (G / 8) + L / 8 gives each XCD a contiguous run of
    // tiles, i.e. whole heads, whose K and V then stay in that XCD's L2
    const int nqb = (Nq + kBM - 1) / kBM;
    const int G = (int)gridDim.x;
    const int L = (int)blockIdx.x;
    const int tile = (G % kXcds == 0) ? (L % kXcds) * (G / kXcds) + L / kXcds : L;
    const int qi0 = tile % nqb;
    const int qb = CAUSAL ? nqb - 1 - qi0 : qi0;  // heaviest first within a head
    const int h = (tile / nqb) % Hq, b = tile / (nqb * Hq);
    const int hk = h / (Hq / Hkv);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int64_t qrow0 = ((int64_t)b * Hq + h) * Nq;
    const int64_t kv0 = ((int64_t)b * Hkv + hk) * Nk;
    const int qbase = qb * kBM + w * 32;  // the wave's first query row

    // the block's Q rows in LDS; B fragments are read from there per key block
#pragma unroll
    for (int r = 0; r < kBM * D / 8 / 256; ++r) {
        const int c = tid + 256 * r, row = c / (D / 8), oc = c % (D / 8);
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

    // the next block's K chunks and V units, in registers
    f32x4 kr[KPT], vr[VPT];
    // loads of the next block; only a block that crosses the end of the keys
    // checks each row (the branch is the same for the whole workgroup)
    auto fetch = [&](int jb) {
        if ((jb + 1) * kBN <= Nk) {
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                const int c = tid + 256 * r, j = jb * kBN + c / (D / 8), oc = c % (D / 8);
                kr[r] = ld16g(k + (kv0 + j) * D + 8 * oc);
                vr[r] = ld16g(v + (kv0 + j) * D + 8 * oc);
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int c = tid + 256 * r, j = jb * kBN + c / (D / 8), oc = c % (D / 8);
            kr[r] = j < Nk ? ld16g(k + (kv0 + j) * D + 8 * oc) : f32x4{0.f, 0.f, 0.f, 0.f};
            vr[r] = j < Nk ? ld16g(v + (kv0 + j) * D + 8 * oc) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int c = tid + 256 * r, j = c / (D / 8), oc = c % (D / 8);
            *reinterpret_cast<f32x4*>(&sk[j * KLD + 8 * oc]) = kr[r];
            *reinterpret_cast<f32x4*>(&sv[j * KLD + 8 * oc]) = vr[r];
        }
    };

    f32x4 acc[2][NT];
#pragma unroll
    for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[bq][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    if (nkb > 0) fetch(0);
    for (int jb = 0; jb < nkb; ++jb) {
        stage();
        __syncthreads();
        if (jb + 1 < nkb) fetch(jb + 1);  // in flight while this block is computed

        // S^T for 4 key tiles x 2 query tiles
        f32x4 st[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int bq = 0; bq < 2; ++bq) st[t][bq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&sk[(16 * t + n) * KLD + 32 * s + 8 * g]);
#pragma unroll
                for (int bq = 0; bq < 2; ++bq) {
                    const f32x4 qv = *reinterpret_cast<const f32x4*>(&sq[(w * 32 + 16 * bq + n) * KLD + 32 * s + 8 * g]);
                    st[t][bq] = mfma(a, qv, st[t][bq]);
                }
            }

        // online softmax per query (lane's column), base 2, against a
        // reference: m holds a per-row reference maximum (scaled), the
        // exponents are exp2(fma(s, c, -m)) and l and the O rows are relative
        // to it. The reference moves (and O, l are rescaled) only when some
        // row of the wave sees a block maximum more than kLazy above its
        // reference, so P stays <= 2^kLazy and o = a / l is unchanged; after
        // the first blocks the rescale is rarely needed. Blocks wholly inside
        // the keys (and, causal, wholly at or below every query of the wave)
        // need no mask.
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
        // O += P V, two 32-key steps
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f32x4 pa[2];
#pragma unroll
            for (int bq = 0; bq < 2; ++bq) {
                const f32x4 lo = st[2 * kk][bq], hi = st[2 * kk + 1][bq];
                pa[bq] = f32x4{pk(lo[0], lo[1]), pk(lo[2], lo[3]), pk(hi[0], hi[1]), pk(hi[2], hi[3])};
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                // transposing reads of the row-major V tile: lane p of lane
                // group g points at key 32 kk + 4 g + p / 4 (+ 16), dims
                // 16 t + 4 (p % 4) .. +3; lane n then receives dim 16 t + n
                // of the 4 keys
                const uint16_t* row = &sv[(32 * kk + 4 * g + (n >> 2)) * KLD + 16 * t + 4 * (n & 3)];
                const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)row);
                const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(row + 16 * KLD));
                const f32x4 bv = __builtin_bit_cast(
                    f32x4, (short __attribute__((ext_vector_type(8)))){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1],
                                                                        v1[2], v1[3]});
#pragma unroll
                for (int bq = 0; bq < 2; ++bq) acc[bq][t] = mfma(pa[bq], bv, acc[bq][t]);
            }
        }
        __syncthreads();  // the next block overwrites the LDS tiles
    }

    // o = a / l (rows 4 g + i of each query tile); lse = (m + log2 l) ln 2
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

hipError_t launch_attn_block(const AttnBlockArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)(a.seq_q + kBM - 1) / kBM * a.heads_q * a.batch));
    const float sl2 = a.scale * 1.4426950408889634f;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const uint16_t*)a.q, (const uint16_t*)a.k,
                           (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.heads_q, a.heads_kv, a.seq_q, a.seq_kv, sl2);
    };
    if (a.dim == 128) a.causal ? go(fr_attn_block_bf16<128, true>) : go(fr_attn_block_bf16<128, false>);
    else a.causal ? go(fr_attn_block_bf16<64, true>) : go(fr_attn_block_bf16<64, false>);
    return hipGetLastError();
}

}  // namespace fr
