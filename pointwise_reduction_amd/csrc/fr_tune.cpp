// fr_tune.cpp - black-box search over launch configurations ("Stax (4): GPU
// Codegen and Dynamic Shapes", 9.6).
//
// A configuration space is a product of finite value sets, one per tunable
// parameter (Definition 9.2); the cost t(c) is a caller-supplied callback
// (a measured time, or +infinity for a configuration that cannot run). Two
// searches:
//   coordinate descent (Algorithm 9.2): from c, try for each parameter the
//     values twice and half the current one (when they belong to the
//     parameter's set); accept c' when t(c') < (1 - eps) t(c); repeat until
//     a full round accepts nothing. With a deterministic t this ends after
//     at most log(t(c0) / t_min) / -log(1 - eps) acceptances, at a point no
//     single-parameter doubling or halving improves by more than eps
//     (Proposition 9.2).
//   random search (Proposition 9.3): N independent uniform draws from the
//     space; the best of them lies in the fastest q-fraction with
//     probability at least 1 - (1 - q)^N, so N >= ln(1/delta) / q suffices.
// Every evaluation is memoised: a configuration is measured at most once
// per search. Host code only: no HIP call.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <vector>

#include "fr.h"

namespace {

struct Search {
    const int32_t* const* values;
    const int32_t* counts;
    int p;
    fr_tune_cost_fn cost;
    void* ctx;
    std::map<std::vector<int32_t>, double> seen;
    int64_t evals = 0;

    // t(c) for a vector of value indices; memoised
    double eval(const std::vector<int32_t>& idx) {
        auto it = seen.find(idx);
        if (it != seen.end()) return it->second;
        std::vector<int32_t> cfg(p);
        for (int i = 0; i < p; ++i) cfg[i] = values[i][idx[i]];
        double t = cost(ctx, cfg.data(), p);
        if (!(t >= 0.0)) t = INFINITY;  // NaN or negative: cannot run
        ++evals;
        seen.emplace(idx, t);
        return t;
    }

    // index of `v` in parameter i's set, or -1
    int find(int i, int64_t v) const {
        for (int k = 0; k < counts[i]; ++k)
            if (values[i][k] == v) return k;
        return -1;
    }
};

int check_space(const int32_t* const* values, const int32_t* counts, int p) {
    if (!values || !counts || p < 1 || p > FR_TUNE_MAX_PARAMS) return FR_E_ARG;
    for (int i = 0; i < p; ++i)
        if (!values[i] || counts[i] < 1) return FR_E_ARG;
    return FR_OK;
}

// splitmix64: a counter-based generator (Steele, Lea and Flood, 2014)
uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

}  // namespace

extern "C" {

int fr_tune_random_draws(double q, double delta) {
    if (!(q > 0.0 && q <= 1.0) || !(delta > 0.0 && delta < 1.0)) return FR_E_ARG;
    return (int)ceil(log(1.0 / delta) / q - 1e-12);
}

double fr_tune_threshold(double eta_max) {
    if (!(eta_max >= 0.0) || !(eta_max < 1.0)) return -1.0;
    // eps must exceed 2 eta / (1 + eta) for every accepted step to be a real
    // improvement under relative noise |eta| <= eta_max (the remark after
    // Proposition 9.2); take the smallest value above it and at least 1e-3
    const double bound = 2.0 * eta_max / (1.0 + eta_max);
    const double eps = bound * (1.0 + 1e-6) + 1e-12;
    return eps < 1e-3 ? 1e-3 : eps;
}

int fr_tune_coordinate_descent(const int32_t* const* values, const int32_t* counts, int p, int32_t* config,
                               double eps, fr_tune_cost_fn cost, void* ctx, fr_tune_result* out) {
    int st = check_space(values, counts, p);
    if (st != FR_OK) return st;
    if (!config || !cost) return FR_E_NULL;
    if (!(eps > 0.0 && eps < 1.0)) return FR_E_ARG;
    Search s{values, counts, p, cost, ctx, {}, 0};
    std::vector<int32_t> c(p);
    for (int i = 0; i < p; ++i) {
        const int k = s.find(i, config[i]);
        if (k < 0) return FR_E_ARG;  // the start must lie in the space
        c[i] = k;
    }
    double tc = s.eval(c);
    if (!(tc < INFINITY)) return FR_E_ARG;  // Proposition 9.2 needs t(c0) < infinity
    int64_t accepted = 0, rounds = 0;
    bool improved = true;
    while (improved) {
        improved = false;
        ++rounds;
        for (int i = 0; i < p; ++i) {
            const int64_t v = values[i][c[i]];
            const int64_t cand[2] = {v * 2, (v % 2 == 0) ? v / 2 : INT64_MIN};
            for (int j = 0; j < 2; ++j) {
                const int k = cand[j] == INT64_MIN ? -1 : s.find(i, cand[j]);
                if (k < 0) continue;  // c' not in the space
                std::vector<int32_t> n = c;
                n[i] = k;
                const double tn = s.eval(n);
                if (tn < (1.0 - eps) * tc) {
                    c = n;
                    tc = tn;
                    ++accepted;
                    improved = true;
                }
            }
        }
    }
    for (int i = 0; i < p; ++i) config[i] = values[i][c[i]];
    if (out) {
        out->cost = tc;
        out->evaluations = s.evals;
        out->accepted = accepted;
        out->rounds = rounds;
    }
    return FR_OK;
}

int fr_tune_random_search(const int32_t* const* values, const int32_t* counts, int p, int draws, uint64_t seed,
                          fr_tune_cost_fn cost, void* ctx, int32_t* best, fr_tune_result* out) {
    int st = check_space(values, counts, p);
    if (st != FR_OK) return st;
    if (!best || !cost) return FR_E_NULL;
    if (draws < 1) return FR_E_ARG;
    Search s{values, counts, p, cost, ctx, {}, 0};
    std::vector<int32_t> c(p), bestc;
    double tb = INFINITY;
    uint64_t ctr = seed;
    for (int d = 0; d < draws; ++d) {
        for (int i = 0; i < p; ++i) {
            // uniform index by rejection: no modulo bias
            const uint64_t n = (uint64_t)counts[i];
            const uint64_t lim = UINT64_MAX - UINT64_MAX % n;
            uint64_t r;
            do r = splitmix64(ctr++);
            while (r >= lim);
            c[i] = (int32_t)(r % n);
        }
        const double t = s.eval(c);
        if (t < tb) {
            tb = t;
            bestc = c;
        }
    }
    if (bestc.empty()) return FR_E_ARG;  // every draw was infinite
    for (int i = 0; i < p; ++i) best[i] = values[i][bestc[i]];
    if (out) {
        out->cost = tb;
        out->evaluations = s.evals;
        out->accepted = 0;
        out->rounds = draws;
    }
    return FR_OK;
}

}  // extern "C"
