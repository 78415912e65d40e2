// fr_device.h - wave64 building blocks for the fused row-reduction kernels
// on gfx950 (CDNA4): lane-group butterflies on DPP, cross-wave combines
// through LDS, masked 16-byte loads and stores, bf16 packing.
//
// Reductions here are deterministic: every butterfly step and every
// cross-wave fold runs in a fixed order, and every combine operator is
// written so that op(a, b) and op(b, a) give the same bits. All lanes of a
// group therefore end with the identical result, and repeated runs give the
// same bits ("Stax (4): GPU Codegen and Dynamic Shapes", 9.5: the merge is
// associative and commutative, so the order is ours to fix).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fr {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ DPP moves
// dpp_ctrl encodings (GCN/CDNA DPP): quad_perm [1,0,3,2] = 0xB1 (lane ^ 1),
// quad_perm [2,3,0,1] = 0x4E (lane ^ 2), row_half_mirror = 0x141 (lane i of
// 8 reads 7 - i), row_mirror = 0x140 (lane i of 16 reads 15 - i).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
// row_shr:n = 0x110 + n: lane i of a 16-lane row reads lane i - n of the
// same row; lanes with no such source keep the old value
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor(int v, int m) { return __shfl_xor(v, m, kWave); }

// Value of the partner lane at butterfly step STEP (1, 2, 4, 8). After the
// steps up to k every lane of an aligned 2k-lane group holds the group
// result: xor 1 and xor 2 inside quads, then the half-row and row mirrors,
// whose partner always lies in the other (already reduced) half of the
// group. Steps 16 and 32 cross DPP rows: group_reduce takes them with the
// permlane swaps below.
template <int STEP, typename T>
__device__ __forceinline__ T partner(T v) {
    static_assert(STEP == 1 || STEP == 2 || STEP == 4 || STEP == 8, "DPP butterfly step");
    if constexpr (STEP == 1) return dpp<kDppXor1>(v);
    else if constexpr (STEP == 2) return dpp<kDppXor2>(v);
    else if constexpr (STEP == 4) return dpp<kDppHalfMirror>(v);
    else return dpp<kDppMirror>(v);
}

// ------------------------------------------------------------------ operators
// NaN-propagating maximum (v_maximum3_f32 on gfx950).
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmax_nan(a, b); }
};
struct OpMinI {
    __device__ __forceinline__ int operator()(int a, int b) const { return a < b ? a : b; }
};

// The two halves of each aligned group of 2 * STEP lanes (STEP 16 or 32),
// as seen from every lane of the group: lo is the value of lane i & ~STEP,
// hi that of lane i | STEP. gfx950's v_permlane16_swap / v_permlane32_swap
// with both operands the same register: the first result keeps the lower
// rows and receives the lower rows' values in the upper ones, the second
// the reverse. VALU moves, no LDS traffic.
template <int STEP>
__device__ __forceinline__ void halves(uint32_t v, uint32_t& lo, uint32_t& hi) {
    static_assert(STEP == 16 || STEP == 32, "cross-row step");
    if constexpr (STEP == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        lo = p[0];
        hi = p[1];
    } else {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        lo = p[0];
        hi = p[1];
    }
}
template <int STEP>
__device__ __forceinline__ void halves(float v, float& lo, float& hi) {
    uint32_t l, h;
    halves<STEP>(__builtin_bit_cast(uint32_t, v), l, h);
    lo = __builtin_bit_cast(float, l);
    hi = __builtin_bit_cast(float, h);
}
template <int STEP>
__device__ __forceinline__ void halves(int v, int& lo, int& hi) {
    uint32_t l, h;
    halves<STEP>((uint32_t)v, l, h);
    lo = (int)l;
    hi = (int)h;
}

// Reduce over aligned groups of SEG lanes (SEG a power of two, <= 64). The
// steps inside a 16-lane row are DPP butterflies; the steps across rows
// combine the group's lower and upper halves in that order, so every lane
// computes the same op(lo, hi).
template <int SEG, typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, Op op) {
    if constexpr (SEG >= 2) v = op(v, partner<1>(v));
    if constexpr (SEG >= 4) v = op(v, partner<2>(v));
    if constexpr (SEG >= 8) v = op(v, partner<4>(v));
    if constexpr (SEG >= 16) v = op(v, partner<8>(v));
    if constexpr (SEG >= 32) {
        T lo, hi;
        halves<16>(v, lo, hi);
        v = op(lo, hi);
    }
    if constexpr (SEG >= 64) {
        T lo, hi;
        halves<32>(v, lo, hi);
        v = op(lo, hi);
    }
    return v;
}

// ------------------------------------------------------------------ (m, d) monoid
// (m1, d1) (+) (m2, d2) = (M, d1 e^(m1-M) + d2 e^(m2-M)), M = max(m1, m2);
// identity (-inf, 0) ("Stax (4)", 9.5). Exponentials use e^t = 2^(t log2 e)
// on the hardware exp2. A side whose m is -inf contributes 0; the sum is
// symmetric in its two terms, so op(a, b) and op(b, a) agree bit for bit.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_fast(float t) { return __builtin_amdgcn_exp2f(t * kLog2e); }

struct MD {
    float m, d;
};
__device__ __forceinline__ MD md_combine(MD a, MD b) {
    float M = fmax_nan(a.m, b.m);
    float ta = a.m == -INFINITY ? 0.f : a.d * exp_fast(a.m - M);
    float tb = b.m == -INFINITY ? 0.f : b.d * exp_fast(b.m - M);
    return MD{M, ta + tb};
}

// (max, first index of the max) with NaN counted as the largest value and the
// lower index winning ties. Symmetric by construction.
struct MI {
    float m;
    int i;
};
__device__ __forceinline__ MI mi_combine(MI a, MI b) {
    bool an = a.m != a.m, bn = b.m != b.m;
    if (an || bn) {
        if (an && bn) return MI{a.m, a.i < b.i ? a.i : b.i};
        return an ? a : b;
    }
    if (a.m > b.m) return a;
    if (b.m > a.m) return b;
    return MI{a.m, a.i < b.i ? a.i : b.i};
}

// ------------------------------------------------------------------ Chan merge
// Mean/M2 statistics (count n, mean mu, sum of squared deviations M2), merged
// with the pairwise update of Chan, Golub & LeVeque (1979), written
// symmetrically: mu = (na mu_a + nb mu_b) / n, M2 = M2a + M2b + delta^2 na nb / n.
struct Stat {
    float n, mu, m2;
};
__device__ __forceinline__ Stat stat_combine(Stat a, Stat b) {
    if (a.n == 0.f) return b;
    if (b.n == 0.f) return a;
    float n = a.n + b.n;
    float delta = b.mu - a.mu;
    // divide (not multiply by 1/n) so that equal means merge to exactly that mean
    float mu = (a.n * a.mu + b.n * b.mu) / n;
    float m2 = (a.m2 + b.m2) + delta * delta * (a.n * b.n) / n;
    return Stat{n, mu, m2};
}

// Group reductions of the composite states: each field rides the same DPP step.
template <int STEP>
__device__ __forceinline__ MD partner(MD v) {
    return MD{partner<STEP>(v.m), partner<STEP>(v.d)};
}
template <int STEP>
__device__ __forceinline__ MI partner(MI v) {
    return MI{partner<STEP>(v.m), partner<STEP>(v.i)};
}
template <int STEP>
__device__ __forceinline__ Stat partner(Stat v) {
    return Stat{partner<STEP>(v.n), partner<STEP>(v.mu), partner<STEP>(v.m2)};
}
template <int STEP>
__device__ __forceinline__ void halves(MD v, MD& lo, MD& hi) {
    halves<STEP>(v.m, lo.m, hi.m);
    halves<STEP>(v.d, lo.d, hi.d);
}
template <int STEP>
__device__ __forceinline__ void halves(MI v, MI& lo, MI& hi) {
    halves<STEP>(v.m, lo.m, hi.m);
    halves<STEP>(v.i, lo.i, hi.i);
}
template <int STEP>
__device__ __forceinline__ void halves(Stat v, Stat& lo, Stat& hi) {
    halves<STEP>(v.n, lo.n, hi.n);
    halves<STEP>(v.mu, lo.mu, hi.mu);
    halves<STEP>(v.m2, lo.m2, hi.m2);
}

struct OpMD {
    __device__ __forceinline__ MD operator()(MD a, MD b) const { return md_combine(a, b); }
};
struct OpMI {
    __device__ __forceinline__ MI operator()(MI a, MI b) const { return mi_combine(a, b); }
};
struct OpStat {
    __device__ __forceinline__ Stat operator()(Stat a, Stat b) const { return stat_combine(a, b); }
};

// ------------------------------------------------------------------ workgroup fold
// All-reduce a wave-uniform value across the NW waves of a workgroup. Lane 0
// of each wave writes its slot, one barrier, then every thread folds the
// slots in wave order, so all threads hold the same bits. `slots` must be
// private to this call (a later reuse needs a barrier first).
template <typename T, typename Op>
__device__ __forceinline__ T block_fold(T v, T* slots, int nw, Op op) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (lane == 0) slots[wave] = v;
    __syncthreads();
    T r = slots[0];
    for (int w = 1; w < nw; ++w) r = op(r, slots[w]);
    return r;
}

// ------------------------------------------------------------------ epoch-tagged workspaces
// Split kernels that exchange partials between workgroups through a
// workspace publish each value as one 64-bit word: a 32-bit tag above the
// 32-bit value. The tag is the call's epoch + 1, read from the workspace
// header at the start of the call; a word whose tag differs (an earlier
// call's, or the zeros of an initialized workspace) is not yet written, so
// nothing has to be cleared between calls. Header words (uint32): 0 a
// cumulative count of partials a workgroup computed itself instead of
// reading them, 2 the epoch, 4-5 an initialization mark (a different value
// per workspace kind), one flag per workgroup after that.
constexpr uint32_t kMaxEpoch = 0x7FFFFFFFu;  // tags run 1 .. kMaxEpoch
constexpr int kHdrRecomputed = 0, kHdrEpoch = 2, kHdrMagic = 4;

__device__ __forceinline__ uint64_t slot_word(uint32_t tag, float v) {
    return ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bool published(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// End of a call, in one workgroup (all its threads): once every
// workgroup's flag holds this call's tag, every workgroup has read the
// epoch, which is then advanced for the next call. Workgroups never wait for
// this one, so one that has not started yet does so as others finish.
template <int T>
__device__ void epoch_advance(uint32_t* hdr, const uint32_t* flags, uint32_t tag, uint32_t epoch) {
    const int tid = threadIdx.x;
    for (;;) {
        bool ok = true;
        for (int b = tid; b < (int)gridDim.x; b += T)
            ok &= __hip_atomic_load(&flags[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
        if (__syncthreads_and(ok)) break;
        __builtin_amdgcn_s_sleep(8);
    }
    if (tid == 0) __hip_atomic_store(&hdr[kHdrEpoch], epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ memory
// Streaming loads/stores: the data is touched once, so they carry the
// non-temporal hint (the role of evict_first in "Stax (4)", 9.2).
template <bool NT>
__device__ __forceinline__ f32x4 ld4(const float* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    else return *reinterpret_cast<const f32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ float ld1(const float* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st4(float* p, f32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void st1(float* p, float v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}
template <bool NT>
__device__ __forceinline__ u32x4 ld4u(const uint16_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void st4u(uint16_t* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}

// Masking modes of a row access. A masked element is never touched and reads
// as `fill` (the identity of the reduction that follows); stores skip it.
//   kNone    every vector is inside the row: straight-line 16-byte accesses
//   kVec     row length and base allow 16-byte vectors and the length is a
//            multiple of 4: a vector is wholly inside or wholly outside
//   kElem    16-byte aligned rows of any length: whole vectors load as one,
//            the one vector that straddles the end element by element
//   kScalar  rows not 16-byte aligned: element accesses only
// Keeping kNone / kVec free of element branches lets the compiler issue all
// loads of a lane back to back and wait for them one vector at a time.
enum Mask : int { kNone = 0, kVec = 1, kElem = 2, kScalar = 3 };

template <int M, bool NT>
__device__ __forceinline__ f32x4 load4m(const float* row, int j0, int L, float fill) {
    if constexpr (M == kNone) {
        return ld4<NT>(row + j0);
    } else if constexpr (M == kVec) {
        return j0 < L ? ld4<NT>(row + j0) : f32x4{fill, fill, fill, fill};
    } else {
        if (M == kElem && j0 + 3 < L) return ld4<NT>(row + j0);
        f32x4 v = {fill, fill, fill, fill};
        if (j0 + 0 < L) v.x = ld1<NT>(row + j0 + 0);
        if (j0 + 1 < L) v.y = ld1<NT>(row + j0 + 1);
        if (j0 + 2 < L) v.z = ld1<NT>(row + j0 + 2);
        if (j0 + 3 < L) v.w = ld1<NT>(row + j0 + 3);
        return v;
    }
}

template <int M, bool NT>
__device__ __forceinline__ void store4m(float* row, int j0, int L, f32x4 v) {
    if constexpr (M == kNone) {
        st4<NT>(row + j0, v);
    } else if constexpr (M == kVec) {
        if (j0 < L) st4<NT>(row + j0, v);
    } else {
        if (M == kElem && j0 + 3 < L) {
            st4<NT>(row + j0, v);
            return;
        }
        if (j0 + 0 < L) st1<NT>(row + j0 + 0, v.x);
        if (j0 + 1 < L) st1<NT>(row + j0 + 1, v.y);
        if (j0 + 2 < L) st1<NT>(row + j0 + 2, v.z);
        if (j0 + 3 < L) st1<NT>(row + j0 + 3, v.w);
    }
}

// Mask mode for the tail step of a loop whose full steps run unmasked.
template <bool VEC>
constexpr int tail_mask() { return VEC ? kElem : kScalar; }
template <bool VEC>
constexpr int body_mask() { return VEC ? kNone : kScalar; }

// Word 3 of a raw buffer resource on gfx9-family devices (gfx950): 32-bit
// data format, no swizzle; with stride 0 the record count is a byte range
// and accesses past it read zero and drop stores.
constexpr int kBufferRsrcWord3 = 0x00020000;

// A raw buffer resource over `bytes` bytes from p (at most 2^31 - 1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufferRsrcWord3);
}
constexpr int kAuxNT = 2;    // buffer instruction cache policy: non-temporal
constexpr int kAuxSc1 = 16;  // buffer instruction cache policy: sc1 (coherent across the compute dies)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A 16-byte buffer store at byte offset `off` of the resource, with the
// scalar offset held at the constant 0. A store of more than 8 bytes reads
// its data registers over several cycles after it issues; a VALU write to
// those registers right behind it must wait one cycle. The compiler inserts
// that wait only when the scalar offset is not a register. With an SGPR
// scalar offset it let the next instruction overwrite the first data
// register, and on MI355X the upper lanes (from lane 12 on) then stored the
// new value. Every wide buffer store goes through here.
template <int AUX>
__device__ __forceinline__ void store16(u32x4 v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
// Sum of the 8 * NV bf16 values in v: each packed pair enters one of four
// fp32 accumulators through v_dot2_f32_bf16 against (1, 1), the four are
// added pairwise at the end. One instruction per pair instead of two unpacks
// and two adds. Products with 1 are exact, so a sum of equal values that fits
// the fp32 significand is exact.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// The packed pair of one word, taken by value: clang compiles a bit_cast of a
// vector element lvalue (v.y) to a load of the vector's first element.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

template <int NV>
__device__ __forceinline__ float sum_bf16(const u32x4* v) {
    const bf16x2 one = as_bf16x2(0x3F803F80u);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[k].x), one, acc[0], false);
        acc[1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[k].y), one, acc[1], false);
        acc[2] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[k].z), one, acc[2], false);
        acc[3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v[k].w), one, acc[3], false);
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

}  // namespace fr
