/*
 * synth.c - seeded synthetic inputs for the fused row-reduction kernels.
 *
 * This module only draws numbers. It holds none of the arithmetic of the
 * reductions themselves: both the fp64 CPU oracle and the GPU path consume
 * what it writes, and neither side links against the other.
 *
 * Generator: a counter-based SplitMix64. Value i of stream s under seed k is
 *     mix64(key(k, s) + (i + 1) * 0x9E3779B97F4A7C15)
 * where mix64 is the SplitMix64 output function (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to
 * a Weyl sequence, and key(k, s) mixes the seed and the stream number. Being counter based, any element can be drawn without
 * drawing the ones before it, so a row of a large matrix is reproducible on
 * its own.
 *
 * Distributions:
 *   uniform  : lo + (hi - lo) * (u >> 40) * 2^-24            (24-bit grid)
 *   normal   : Box-Muller in fp64 on two 53-bit uniforms, then cast
 *   bf16     : fp32 -> bf16 round-to-nearest-even, NaN kept quiet
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Key of (seed, stream): streams are independent sequences under one seed. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(seed * GOLDEN + 0x632BE59BD9B4E019ULL) ^ mix64((stream + 1) * 0xD1B54A32D192ED03ULL);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double u53(uint64_t u) { return ((double)(u >> 11) + 0.5) * 0x1.0p-53; } /* (0,1) */

static inline double std_normal(uint64_t key, uint64_t i) {
    double u1 = u53(draw(key, 2 * i));
    double u2 = u53(draw(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

uint64_t syn_u64(uint64_t seed, uint64_t stream, uint64_t i) { return draw(stream_key(seed, stream), i); }

/* Values i0 .. i0+n-1 of a stream into out[0 .. n): a counter-based draw, so
 * any slice can be produced on its own (callers split large arrays across
 * threads; the values do not depend on the split). */
void syn_uniform_f32_at(float* out, int64_t n, uint64_t seed, uint64_t stream, int64_t i0, double lo, double hi) {
    uint64_t key = stream_key(seed, stream);
    for (int64_t i = 0; i < n; ++i) {
        double u = (double)(draw(key, (uint64_t)(i0 + i)) >> 40) * 0x1.0p-24;
        out[i] = (float)(lo + (hi - lo) * u);
    }
}

void syn_normal_f32_at(float* out, int64_t n, uint64_t seed, uint64_t stream, int64_t i0, double mean, double std) {
    uint64_t key = stream_key(seed, stream);
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * std_normal(key, (uint64_t)(i0 + i)));
}

void syn_uniform_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, double lo, double hi) {
    syn_uniform_f32_at(out, n, seed, stream, 0, lo, hi);
}

void syn_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, double mean, double std) {
    syn_normal_f32_at(out, n, seed, stream, 0, mean, std);
}

/*
 * Row-softmax stress input: N(0,1)*scale, and each entry independently
 * replaced with probability p_spike by +spike or -spike (fair sign).
 * Rows are `cols` long at a row stride of `rs` elements; only the first
 * `cols` of each row are written.
 */
void syn_spiky_normal_rows_range(float* out, int64_t r0, int64_t r1, int64_t cols, int64_t rs, uint64_t seed,
                                 double scale, double p_spike, double spike) {
    uint64_t kn = stream_key(seed, 0), ks = stream_key(seed, 1);
    uint64_t thresh = (uint64_t)(p_spike * 18446744073709551616.0);
    if (p_spike >= 1.0) thresh = UINT64_MAX;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint64_t i = (uint64_t)(r * cols + c);
            uint64_t s = draw(ks, i);
            double v = scale * std_normal(kn, i);
            if (p_spike > 0.0 && s < thresh) v = ((draw(ks, i ^ 0x8000000000000000ULL) & 1) ? spike : -spike);
            out[r * rs + c] = (float)v;
        }
}

void syn_spiky_normal_rows(float* out, int64_t rows, int64_t cols, int64_t rs, uint64_t seed,
                           double scale, double p_spike, double spike) {
    syn_spiky_normal_rows_range(out, 0, rows, cols, rs, seed, scale, p_spike, spike);
}

/* Each row length is drawn uniformly from `choices[0..nchoices)`. */
void syn_lengths(int32_t* len, int64_t rows, uint64_t seed, const int32_t* choices, int32_t nchoices) {
    uint64_t key = stream_key(seed, 7);
    for (int64_t r = 0; r < rows; ++r) len[r] = choices[draw(key, (uint64_t)r) % (uint64_t)nchoices];
}

/* Ragged rows: N(mean, std) over j < len[r]; the padded tail j >= len[r] is set to `tail`. */
void syn_ragged_normal_rows_range(float* out, int64_t r0, int64_t r1, int64_t rs, const int32_t* len,
                                  uint64_t seed, double mean, double std, float tail) {
    uint64_t key = stream_key(seed, 0);
    for (int64_t r = r0; r < r1; ++r) {
        int64_t L = len[r];
        for (int64_t c = 0; c < rs; ++c)
            out[r * rs + c] = c < L ? (float)(mean + std * std_normal(key, (uint64_t)(r * rs + c))) : tail;
    }
}

void syn_ragged_normal_rows(float* out, int64_t rows, int64_t rs, const int32_t* len, uint64_t seed,
                            double mean, double std, float tail) {
    syn_ragged_normal_rows_range(out, 0, rows, rs, len, seed, mean, std, tail);
}

/*
 * Pick `count` cells (row, col) at seeded positions, all in distinct rows.
 * The caller decides what to write there (the NaN-injection variants).
 */
int32_t syn_pick_cells(int64_t rows, int64_t cols, uint64_t seed, uint64_t stream, int32_t count,
                       int32_t* rows_out, int32_t* cols_out) {
    uint64_t key = stream_key(seed, 100 + stream);
    int32_t placed = 0;
    for (uint64_t t = 0; placed < count && placed < rows && t < 1000000; ++t) {
        int64_t r = (int64_t)(draw(key, 2 * t) % (uint64_t)rows);
        int64_t c = (int64_t)(draw(key, 2 * t + 1) % (uint64_t)cols);
        int dup = 0;
        for (int32_t k = 0; k < placed; ++k) dup |= rows_out[k] == r;
        if (dup) continue;
        rows_out[placed] = (int32_t)r;
        cols_out[placed] = (int32_t)c;
        ++placed;
    }
    return placed;
}

/* fp32 -> bf16 round-to-nearest-even on the bit pattern; NaN stays a quiet NaN. */
void syn_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &in[i], 4);
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
            out[i] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        uint32_t lsb = (u >> 16) & 1u;
        out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
    }
}

void syn_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)in[i] << 16;
        memcpy(&out[i], &u, 4);
    }
}
