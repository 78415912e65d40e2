/*
 * oracle.c - plain, slow, fp64 CPU reference for the fused pointwise-prologue
 * + row-reduction operations.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can check the GPU library against the plain
 * definitions. It shares no code, header, table or helper with the GPU
 * library; the only thing both sides see is the seeded input generator.
 *
 * Every function below is the plain definition written out with sequential
 * loops and fp64 accumulation. No blocking, fusion or reordering is done
 * beyond what the cited definition states. Sources (web pages):
 *   [Stax4]  "Stax (4): GPU Codegen and Dynamic Shapes" (TensorPlay blog),
 *            section 9.2 (Listing 9.1, Example 1.1), 9.3 (Listing 9.2, the
 *            transposed add of Example 6.1; Listing 9.3, the GELU backward
 *            of Example 5.1), 9.4 (Listing 9.4,
 *            Example 6.2), 9.5 (softmax definition, Listing 9.5, the (m, d)
 *            merge and Proposition 9.1), 10.2 (Example 10.1).
 *   [HG12]   "hello-gpu, Chapter 12: Fusion", section 12.1 (attention of one
 *            query row, worked example) and 12.3 (online m, l, a update).
 *   [Stax4]  also 9.10 (attention S = QK^T / sqrt(d), row softmax, O = PV; the
 *            (m, l, a) triple, its merge, and LSE = m + log l; the decode
 *            template that splits the keys).
 *   [L8]     "CMU 15-779 Lecture 8: ML Compilers Part 1, Tile-based DSLs",
 *            section 3 (fused softmax) and Exercise 1 (row L2 norm).
 * Backward passes (softmax, LayerNorm) are not defined on the pages; they
 * are the derivatives of the forward definitions above, as stated at each.
 * Readings of points the pages leave open are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */

double orc_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * Round an fp64 value once to bf16 (1 sign, 8 exponent, 7 fraction bits),
 * round-to-nearest, ties to even. Done on the value, not on bit patterns:
 * the quantum of a bf16 number with unbiased exponent E is 2^(E-7), with E
 * clamped below at -126 (subnormals). NaN -> quiet NaN 0x7FC0 (sign kept).
 */
uint16_t orc_double_to_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;         /* a = g * 2^E, g in [1, 2) */
    if (E < -126) E = -126;
    double q = ldexp(a, 7 - E);     /* a in units of the quantum, exact */
    double r = nearbyint(q);        /* default rounding mode: ties to even */
    double res = ldexp(r, E - 7);
    const double maxbf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (res > maxbf) return (uint16_t)(sign | 0x7F80u);
    float f = (float)res;           /* exact: every bf16 value is an fp32 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------- Example 1.1 (C1) */

/*
 * out[i] = sum_r 2 * relu(a[i,r] + b[i,r])      [Stax4] 9.2, Listing 9.1;
 *                                               10.2, Example 10.1.
 * The add is an fp32 add (the kernel adds two fp32 loads); relu propagates
 * NaN (maximum with NaN propagation, [Stax4] 9.2 part (3)); the sum is fp64.
 * Reading: relu(-0) = +0 and +/-inf follow IEEE; neither changes a sum whose
 * identity is +0. out64 (nullable) receives the fp64 value before rounding.
 */
void orc_sum_relu_add(const float* a, const float* b, int64_t rows, int64_t cols, int64_t a_rs, int64_t b_rs,
                      float* out, double* out64) {
    for (int64_t i = 0; i < rows; ++i) {
        double acc = 0.0;
        for (int64_t r = 0; r < cols; ++r) {
            float t = (float)((double)a[i * a_rs + r] + (double)b[i * b_rs + r]); /* fp32 add */
            double rt = isnan(t) ? (double)t : (t > 0.0f ? (double)t : 0.0);
            acc += 2.0 * rt;
        }
        out[i] = (float)acc;
        if (out64) out64[i] = acc;
    }
}

/* --------------------------------------------------- softmax (C2, C5) */

/*
 * Softmax of one row held in fp64, the definition of [Stax4] 9.5:
 *   m = max_k x_k,  y_j = e^(x_j - m) / sum_k e^(x_k - m).
 * Two passes (max, then sum of exponentials), exp from the C library in
 * fp64. Reading: a NaN anywhere makes m NaN and so the whole row NaN.
 * Returns the argmax: the smallest j with x_j == m (first occurrence;
 * reading, the pages are silent on ties); with a NaN, the first NaN.
 */
static int64_t softmax_row_f64(const double* x, int64_t n, double* y) {
    if (n <= 0) return -1;
    double m = x[0];
    int64_t am = 0;
    for (int64_t j = 1; j < n; ++j) {
        if (isnan(m)) break;
        if (isnan(x[j]) || x[j] > m) {
            m = x[j];
            am = j;
        }
    }
    double d = 0.0;
    for (int64_t j = 0; j < n; ++j) d += exp(x[j] - m);
    for (int64_t j = 0; j < n; ++j) y[j] = exp(x[j] - m) / d;
    return am;
}

void orc_softmax_f64(const double* x, int64_t n, double* y) { (void)softmax_row_f64(x, n, y); }

/*
 * Row softmax over fp32 rows, optionally ragged: row r covers j < len_r
 * where len_r = lengths[r] clamped to [0, cols] (lengths NULL: len_r = cols).
 * Only j < len_r is read or written; the padded tail of x is never read and
 * the tail of y is left untouched ([Stax4] 10.3: loop bounds are runtime
 * values, so the masks stay).
 *   y   (nullable): fp32 result, rounded once from fp64.
 *   y64 (nullable): fp64 result, row stride y_rs.
 *   argmax (nullable): first index of the row maximum; -1 for an empty row.
 * `scratch` must hold 2 * cols doubles.
 */
void orc_softmax_rows(const float* x, int64_t rows, int64_t cols, int64_t x_rs, const int32_t* lengths, float* y,
                      double* y64, int64_t y_rs, int32_t* argmax, double* scratch) {
    double* xin = scratch;
    double* yout = scratch + cols;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t L = cols;
        if (lengths) {
            L = lengths[r];
            if (L < 0) L = 0;
            if (L > cols) L = cols;
        }
        for (int64_t j = 0; j < L; ++j) xin[j] = (double)x[r * x_rs + j];
        int64_t am = softmax_row_f64(xin, L, yout);
        for (int64_t j = 0; j < L; ++j) {
            if (y) y[r * y_rs + j] = (float)yout[j];
            if (y64) y64[r * y_rs + j] = yout[j];
        }
        if (argmax) argmax[r] = (int32_t)am;
    }
}

/* ------------------------------------------ the (m, d) monoid, online update */

/*
 * (m1, d1) (+) (m2, d2) = (M, d1 e^(m1 - M) + d2 e^(m2 - M)), M = max(m1, m2)
 * [Stax4] 9.5. The identity is (-inf, 0); (-inf,0) (+) (-inf,0) = (-inf,0).
 */
void orc_md_combine(double m1, double d1, double m2, double d2, double* m, double* d) {
    double M = m1 > m2 ? m1 : m2;
    if (isinf(M) && M < 0) {
        *m = M;
        *d = 0.0;
        return;
    }
    *m = M;
    *d = d1 * exp(m1 - M) + d2 * exp(m2 - M);
}

/* Fold a sequence with (+), left to right, each element x as (x, 1). */
void orc_md_fold(const double* x, int64_t n, double* m, double* d) {
    double cm = -INFINITY, cd = 0.0;
    for (int64_t j = 0; j < n; ++j) orc_md_combine(cm, cd, x[j], 1.0, &cm, &cd);
    *m = cm;
    *d = cd;
}

/*
 * One query row of attention by the online update of [HG12] 12.3: state
 * (m, l, a) starts at (-inf, 0, 0); for each score s_j with value row V_j:
 *   m' = max(m, s_j), alpha = e^(m - m'), beta = e^(s_j - m'),
 *   l' = alpha l + beta,  a' = alpha a + beta V_j;  output o = a / l.
 * V is n x dv row-major. Outputs the final m, l, a[dv] and o[dv].
 */
void orc_online_attention_row(const double* s, const double* V, int64_t n, int64_t dv, double* m_out, double* l_out,
                              double* a, double* o) {
    double m = -INFINITY, l = 0.0;
    for (int64_t k = 0; k < dv; ++k) a[k] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double mp = s[j] > m ? s[j] : m;
        double alpha = exp(m - mp); /* m = -inf on the first step gives 0 */
        double beta = exp(s[j] - mp);
        l = alpha * l + beta;
        for (int64_t k = 0; k < dv; ++k) a[k] = alpha * a[k] + beta * V[j * dv + k];
        m = mp;
    }
    *m_out = m;
    *l_out = l;
    for (int64_t k = 0; k < dv; ++k) o[k] = a[k] / l;
}

/* ------------------------------------------------------ softmax backward */

/*
 * Gradient of the row softmax ([Stax4] 9.5 defines y = softmax(x); the
 * gradient is not on the pages and is taken from the calculus of that
 * definition): with L depending on y and dy = dL/dy,
 *   dx_j = y_j (dy_j - sum_k dy_k y_k).
 * Written out in fp64 over fp32 rows; row r covers j < len_r (lengths
 * clamped to [0, cols], NULL: cols) and nothing beyond is read or written.
 *   dx64 (row stride cols): the result; untouched past len_r.
 *   mag  (nullable, row stride cols): |y_j dy_j| + y_j sum_k |dy_k y_k|,
 *        the size of the terms of dx_j.
 */
void orc_softmax_backward_rows(const float* y, const float* dy, int64_t rows, int64_t cols, int64_t y_rs,
                               int64_t dy_rs, const int32_t* lengths, double* dx64, double* mag) {
    for (int64_t r = 0; r < rows; ++r) {
        int64_t L = lengths ? lengths[r] : cols;
        if (L < 0) L = 0;
        if (L > cols) L = cols;
        const float* yr = y + r * y_rs;
        const float* gr = dy + r * dy_rs;
        double s = 0.0, sa = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            s += (double)gr[j] * (double)yr[j];
            sa += fabs((double)gr[j] * (double)yr[j]);
        }
        for (int64_t j = 0; j < L; ++j) {
            dx64[r * cols + j] = (double)yr[j] * ((double)gr[j] - s);
            if (mag) mag[r * cols + j] = fabs((double)yr[j] * (double)gr[j]) + fabs((double)yr[j]) * sa;
        }
    }
}

/* ------------------------------------------------------ attention decode */

/*
 * One query row per (batch b, query head h) against the keys and values of
 * its key-value head ([Stax4] 9.10: S = Q K^T / sqrt(d), P = softmax(S) by
 * rows, O = P V; [HG12] 12.1: s_j = q . k_j / sqrt(D), p_j = e^{s_j} /
 * sum_k e^{s_k}, o = sum_j p_j v_j). Written out as the definition: scores,
 * their maximum, the exponentials, their sum, the weighted sum of values,
 * one division; all in fp64.
 * Readings where the pages are silent:
 *  - several query heads may share one key-value head: head h reads head
 *    h / (Hq / Hkv) (Hq a multiple of Hkv; the pages have one head);
 *  - scale multiplies q . k (the pages' 1 / sqrt(d));
 *  - lengths (nullable, [B]) limits batch b to its first len_b keys,
 *    clamped to [0, S]; an empty key set gives o = 0 and lse = -inf;
 *  - a NaN among the scores makes the maximum NaN, so o and lse are NaN.
 * Layouts (row-major, contiguous): q, o64, mag [B, Hq, D]; k, v [B, Hkv, S,
 * D]; lse, smag [B, Hq].
 *   lse  = m + log(l) ([Stax4] 9.10), the log of the sum of e^{s_j}.
 *   mag  (nullable): sum_j p_j |v_jd|, the size of the terms of o.
 *   smag (nullable): max_j sum_d |scale q_d k_jd|, the size of the terms of
 *                    the scores.
 */
void orc_attn_decode(const double* q, const double* k, const double* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t S,
                     int64_t D, const int32_t* lengths, double scale, double* s_scratch, double* o64, double* lse,
                     double* mag, double* smag) {
    const int64_t G = Hq / Hkv;
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = lengths ? lengths[b] : S;
        if (L < 0) L = 0;
        if (L > S) L = S;
        for (int64_t h = 0; h < Hq; ++h) {
            const double* qr = q + (b * Hq + h) * D;
            const double* kh = k + (b * Hkv + h / G) * S * D;
            const double* vh = v + (b * Hkv + h / G) * S * D;
            double* orow = o64 + (b * Hq + h) * D;
            double* mrow = mag ? mag + (b * Hq + h) * D : 0;
            double sm = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                orow[d] = 0.0;
                if (mrow) mrow[d] = 0.0;
            }
            if (L == 0) {
                lse[b * Hq + h] = -INFINITY;
                if (smag) smag[b * Hq + h] = 0.0;
                continue;
            }
            double m = -INFINITY;
            int nan = 0;
            for (int64_t j = 0; j < L; ++j) {
                double s = 0.0, t = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    s += qr[d] * kh[j * D + d];
                    t += fabs(scale * qr[d] * kh[j * D + d]);
                }
                s *= scale;
                s_scratch[j] = s;
                if (isnan(s)) nan = 1;
                if (s > m) m = s;
                if (t > sm) sm = t;
            }
            if (nan) m = NAN;
            double l = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                const double p = exp(s_scratch[j] - m);
                s_scratch[j] = p;
                l += p;
            }
            for (int64_t j = 0; j < L; ++j)
                for (int64_t d = 0; d < D; ++d) {
                    orow[d] += s_scratch[j] * vh[j * D + d];
                    if (mrow) mrow[d] += s_scratch[j] * fabs(vh[j * D + d]);
                }
            for (int64_t d = 0; d < D; ++d) {
                orow[d] /= l;
                if (mrow) mrow[d] /= l;
            }
            lse[b * Hq + h] = m + log(l);
            if (smag) smag[b * Hq + h] = sm;
        }
    }
}

/*
 * The merge of two partial states of one query row over disjoint key sets
 * ([Stax4] 9.10): with mu = max(m1, m2),
 *   (m1, l1, a1) (+) (m2, l2, a2) = (mu, l1 e^{m1-mu} + l2 e^{m2-mu},
 *                                    a1 e^{m1-mu} + a2 e^{m2-mu}).
 * The identity is (-inf, 0, 0): its factor e^{-inf - mu} is 0.
 */
void orc_attn_merge(double m1, double l1, const double* a1, double m2, double l2, const double* a2, int64_t D,
                    double* m, double* l, double* a) {
    const double mu = m1 > m2 ? m1 : m2;
    const double f1 = m1 == -INFINITY ? 0.0 : exp(m1 - mu);
    const double f2 = m2 == -INFINITY ? 0.0 : exp(m2 - mu);
    *m = mu;
    *l = l1 * f1 + l2 * f2;
    for (int64_t d = 0; d < D; ++d) a[d] = a1[d] * f1 + a2[d] * f2;
}

/* ------------------------------------------------------ attention, many query rows */

/*
 * Attention of a block of query rows ([Stax4] 9.10: S = Q K^T scaled,
 * P = softmax(S) by rows, O = P V, LSE = m + log l kept for the backward
 * pass; the causal mask of Listing 9.7 lets query i see key j when i >= j).
 * Each query row is the plain definition, as in orc_attn_decode: scores
 * over the keys it may see, their maximum, exponentials, sum, weighted sum
 * of values, one division; fp64 throughout.
 * Readings: heads as in orc_attn_decode (query head h reads key-value head
 * h / (Hq / Hkv)); the causal rule compares the query's and the key's
 * positions from the start of the sequence (so with Nq < Nk the last keys
 * are seen by no query); a row that sees no key gives o = 0, lse = -inf.
 * Layouts (row-major, contiguous): q, o64, mag [B, Hq, Nq, D]; k, v [B, Hkv,
 * Nk, D]; lse, smag [B, Hq, Nq]. mag: sum_j p_j |v_jd|; smag: max_j sum_d
 * |scale q_d k_jd| (the sizes of the terms, for tolerances).
 */
void orc_attn_fwd(const double* q, const double* k, const double* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                  int64_t Nk, int64_t D, int causal, double scale, double* s_scratch, double* o64, double* lse,
                  double* mag, double* smag) {
    const int64_t G = Hq / Hkv;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h) {
            const double* kh = k + (b * Hkv + h / G) * Nk * D;
            const double* vh = v + (b * Hkv + h / G) * Nk * D;
            for (int64_t i = 0; i < Nq; ++i) {
                const int64_t row = (b * Hq + h) * Nq + i;
                const double* qr = q + row * D;
                double* orow = o64 + row * D;
                double* mrow = mag ? mag + row * D : 0;
                const int64_t L = causal ? (i + 1 < Nk ? i + 1 : Nk) : Nk;
                for (int64_t d = 0; d < D; ++d) {
                    orow[d] = 0.0;
                    if (mrow) mrow[d] = 0.0;
                }
                double m = -INFINITY, sm = 0.0;
                int nan = 0;
                for (int64_t j = 0; j < L; ++j) {
                    double s = 0.0, t = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        s += qr[d] * kh[j * D + d];
                        t += fabs(scale * qr[d] * kh[j * D + d]);
                    }
                    s *= scale;
                    s_scratch[j] = s;
                    if (isnan(s)) nan = 1;
                    if (s > m) m = s;
                    if (t > sm) sm = t;
                }
                if (smag) smag[row] = sm;
                if (L == 0) {
                    lse[row] = -INFINITY;
                    continue;
                }
                if (nan) m = NAN;
                double l = 0.0;
                for (int64_t j = 0; j < L; ++j) {
                    const double e = exp(s_scratch[j] - m);
                    s_scratch[j] = e;
                    l += e;
                }
                for (int64_t j = 0; j < L; ++j)
                    for (int64_t d = 0; d < D; ++d) {
                        orow[d] += s_scratch[j] * vh[j * D + d];
                        if (mrow) mrow[d] += s_scratch[j] * fabs(vh[j * D + d]);
                    }
                for (int64_t d = 0; d < D; ++d) {
                    orow[d] /= l;
                    if (mrow) mrow[d] /= l;
                }
                lse[row] = m + log(l);
            }
        }
}

/* ------------------------------------------------------ LayerNorm (C3) */

/*
 * y = (x - mu) / sqrt(var + eps) * gamma + beta over each row, on bf16 data.
 * The pages do not define LayerNorm. They name variance reductions that also
 * output the mean ([Stax4] 10.4) and state that half-precision arithmetic is
 * carried out in float32 ([Stax4] 9.8, tensor cores and mixed precision;
 * Listing 9.5 upcasts its load). Readings: mu = sum(x)/N;
 * var = sum((x - mu)^2)/N (biased, the
 * two-pass definition, not Welford); eps inside the square root; gamma and
 * beta per column (NULL: 1 and 0). All arithmetic in fp64, one rounding to
 * bf16 at the end (round to nearest even).
 *   y   (nullable): bf16 result bits.
 *   y64 (nullable): fp64 result before rounding.
 *   mag (nullable): |(x - mu) * rstd * gamma| + |beta|, the size of the
 *                   terms that make y (used for the near-zero tolerance).
 * Output arrays use row stride y_rs.
 */
void orc_layernorm_rows(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows, int64_t cols,
                        int64_t x_rs, double eps, uint16_t* y, double* y64, double* mag, int64_t y_rs) {
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * x_rs;
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += orc_bf16_to_double(xr[j]);
        double mu = s / (double)cols;
        double q = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double t = orc_bf16_to_double(xr[j]) - mu;
            q += t * t;
        }
        double var = q / (double)cols;
        double rstd = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < cols; ++j) {
            double g = gamma ? orc_bf16_to_double(gamma[j]) : 1.0;
            double b = beta ? orc_bf16_to_double(beta[j]) : 0.0;
            double t = (orc_bf16_to_double(xr[j]) - mu) * rstd * g;
            double v = t + b;
            if (y) y[r * y_rs + j] = orc_double_to_bf16(v);
            if (y64) y64[r * y_rs + j] = v;
            if (mag) mag[r * y_rs + j] = fabs(t) + fabs(b);
        }
    }
}

/*
 * The row statistics of the LayerNorm above, as the forward pass of a
 * training step saves them: mu = sum(x)/N and rstd = 1 / sqrt(var + eps) with
 * the biased two-pass variance, in fp64 over the bf16 row.
 */
void orc_layernorm_stats(const uint16_t* x, int64_t rows, int64_t cols, int64_t x_rs, double eps, double* mean,
                         double* rstd) {
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * x_rs;
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += orc_bf16_to_double(xr[j]);
        const double mu = s / (double)cols;
        double q = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            const double d = orc_bf16_to_double(xr[j]) - mu;
            q += d * d;
        }
        mean[r] = mu;
        rstd[r] = 1.0 / sqrt(q / (double)cols + eps);
    }
}

/*
 * LayerNorm backward. The pages define no LayerNorm gradient; this is the
 * derivative of the forward definition above, in which mu and rstd are
 * functions of the row. With xh_j = (x_j - mu) rstd, g_j = dy_j gamma_j and
 * C = cols:
 *   dx_j     = rstd (g_j - (1/C) sum_k g_k - xh_j (1/C) sum_k g_k xh_k)
 *   dgamma_j = sum_i dy_ij xh_ij,      dbeta_j = sum_i dy_ij.
 * mu and rstd are inputs: the values the forward pass saved (read, not
 * recomputed, by the backward pass). fp64 over bf16 x, dy, gamma (NULL: 1).
 *   dx64   [rows, cols], row stride cols.
 *   dxmag  (nullable): rstd (|g_j| + (1/C) sum|g_k| + |xh_j| (1/C) sum|g_k xh_k|),
 *          the size of the terms of dx_j.
 *   dgamma64, dbeta64 [cols] (nullable); gmag, bmag (nullable): sum_i |dy_ij xh_ij|
 *          and sum_i |dy_ij|, the sizes of their terms.
 */
void orc_layernorm_backward_rows(const uint16_t* x, const uint16_t* dy, const uint16_t* gamma, const double* mean,
                                 const double* rstd, int64_t rows, int64_t cols, int64_t x_rs, int64_t dy_rs,
                                 double* dx64, double* dxmag, double* dgamma64, double* dbeta64, double* gmag,
                                 double* bmag) {
    for (int64_t j = 0; j < cols; ++j) {
        if (dgamma64) dgamma64[j] = 0.0;
        if (dbeta64) dbeta64[j] = 0.0;
        if (gmag) gmag[j] = 0.0;
        if (bmag) bmag[j] = 0.0;
    }
    const double C = (double)cols;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * x_rs;
        const uint16_t* gr = dy + r * dy_rs;
        const double mu = mean[r], rs = rstd[r];
        double sg = 0.0, sgx = 0.0, ag = 0.0, agx = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            const double xh = (orc_bf16_to_double(xr[j]) - mu) * rs;
            const double d = orc_bf16_to_double(gr[j]);
            const double g = d * (gamma ? orc_bf16_to_double(gamma[j]) : 1.0);
            sg += g;
            sgx += g * xh;
            ag += fabs(g);
            agx += fabs(g * xh);
            if (dgamma64) dgamma64[j] += d * xh;
            if (dbeta64) dbeta64[j] += d;
            if (gmag) gmag[j] += fabs(d * xh);
            if (bmag) bmag[j] += fabs(d);
        }
        for (int64_t j = 0; j < cols; ++j) {
            const double xh = (orc_bf16_to_double(xr[j]) - mu) * rs;
            const double g = orc_bf16_to_double(gr[j]) * (gamma ? orc_bf16_to_double(gamma[j]) : 1.0);
            dx64[r * cols + j] = rs * (g - sg / C - xh * (sgx / C));
            if (dxmag) dxmag[r * cols + j] = rs * (fabs(g) + ag / C + fabs(xh) * (agx / C));
        }
    }
}

/* --------------------------------------------------------- sum of squares (C4) */

/*
 * sum_i x_i^2 ([Stax4] 9.4, Listing 9.4: the x * x prologue of Example 6.2;
 * [L8] Exercise 1: the row L2 norm is the square root of this sum).
 * Squares are exact in fp64 (24 x 24 bits); the sum is sequential fp64.
 */
double orc_sumsq(const float* x, int64_t n) {
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i) acc += (double)x[i] * (double)x[i];
    return acc;
}

void orc_sumsq_rows(const float* x, int64_t rows, int64_t cols, int64_t x_rs, double* out) {
    for (int64_t r = 0; r < rows; ++r) out[r] = orc_sumsq(x + r * x_rs, cols);
}

/* fp64 values -> bf16 bit patterns, each rounded once to nearest even. */
void orc_round_bf16(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_bf16(v[i]);
}

/* ------------------------------------------------------------- pointwise */

/*
 * Elementwise add of two 2-D operands with independent strides ([Stax4]
 * 9.3, Listing 9.2: Example 6.1, x.t() + y, where the first operand is
 * contiguous along the output's rows and the second along its columns):
 *   out[i * out_rs + j] = a[i * a_rs + j * a_cs] + b[i * b_rs + j * b_cs]
 * for i < rows, j < cols. Each sum is formed in fp64 and rounded once to
 * fp32. For two fp32 operands that equals the correctly rounded fp32 sum:
 * fp64 carries more than twice the fp32 significand plus two bits, so the
 * second rounding cannot change the first.
 */
void orc_add_2d(const float* a, int64_t a_rs, int64_t a_cs, const float* b, int64_t b_rs, int64_t b_cs, float* out,
                int64_t out_rs, int64_t rows, int64_t cols) {
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            out[i * out_rs + j] = (float)((double)a[i * a_rs + j * a_cs] + (double)b[i * b_rs + j * b_cs]);
}

/*
 * GELU backward ([Stax4] 9.3, Listing 9.3, the backward pointwise kernel of
 * Example 5.1): with h the saved pre-activation and GELU(h) = h Phi(h),
 *   GELU'(h) = Phi(h) + h phi(h),   dx = dy * GELU'(h),
 * Phi the standard normal distribution function and phi its density. dy is
 * one element broadcast to every output when dy_stride is 0 (the pages'
 * case: the loss is a scalar), else element i reads dy[i * dy_stride].
 * In fp64: Phi(h) = erfc(-h / sqrt 2) / 2, the same function as
 * (1 + erf(h / sqrt 2)) / 2 without its cancellation for negative h;
 * phi(h) = exp(-h^2 / 2) / sqrt(2 pi).
 *   mag (nullable): |dy| (Phi(h) + |h| phi(h)), the size of the terms of dx.
 */
void orc_gelu_backward(const double* dy, int64_t dy_stride, const double* h, int64_t n, double* dx64, double* mag) {
    const double inv_sqrt2 = 0.70710678118654752440;
    const double inv_sqrt2pi = 0.39894228040143267794;
    for (int64_t i = 0; i < n; ++i) {
        const double hi = h[i];
        const double g = dy[i * dy_stride];
        const double cdf = 0.5 * erfc(-hi * inv_sqrt2);
        const double pdf = inv_sqrt2pi * exp(-0.5 * hi * hi);
        dx64[i] = g * (cdf + hi * pdf);
        if (mag) mag[i] = fabs(g) * (cdf + fabs(hi) * pdf);
    }
}
