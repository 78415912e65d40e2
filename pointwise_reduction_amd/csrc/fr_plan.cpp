// fr_plan.cpp - reduction-form selection and launch configuration.
//
// Host-only code (no HIP call), so the choice can be inspected and tested
// without a GPU. The structure follows "Stax (4): GPU Codegen and Dynamic
// Shapes": 9.4 picks the form from the reduction length (persistent when the
// row fits, looped when it does not, split when there are too few outputs to
// fill the device); 9.6 makes block sizes and warp counts launch parameters
// whose grid follows from them, chosen by measuring candidates (Algorithm
// 9.1, run offline here: the constants below are the measured winners on
// MI355X, and fr_tune_override lets a tuner time any other candidate); 10.3
// decides against the upper bound of a runtime length (here `cols`, the row
// capacity of a ragged input).
//
// The MI355X thresholds differ from the pages' Triton/H100 rule (persistent
// up to 1024 elements): a 64-lane wave holding 8 x 16-byte vectors per lane
// keeps 2048 fp32 values in 32 VGPRs, and a 512-thread workgroup holds a
// 32K-element bf16 row in registers (32 VGPRs of packed bf16 per lane).
#include <stdint.h>

#include <algorithm>

#include "fr_internal.h"

namespace fr {

namespace {

constexpr int64_t kMaxGrid = 1 << 20;      // grid-stride loops cover the rest
constexpr int kPerMaxF32 = 2048;           // 64 lanes x 8 vectors x 4 floats
constexpr int kSumSplitRows = 512;         // fewer rows than 2 per CU: split
constexpr int kSoftmaxSplitRows = 1024;    // fewer rows than 4 per CU: split
constexpr int kSplitTargetWgs = 2048;      // 8 workgroups per CU on 256 CUs
constexpr int kSumSplitThreads = 256, kSumSplitU = 4;            // 4096 floats per step
constexpr int kSoftmaxSplitThreads = 256, kSoftmaxSplitNV = 8;   // 8192-float chunks
// Two rows per wave pay off while the grid would otherwise launch more than
// ~2 waves per SIMD of one-row waves (measured: 4096 x 1024 fp32 runs 15%
// faster, 16384 x 1024 3% slower).
constexpr int64_t kTwoRowsPerWaveMaxRows = 8192;

// LayerNorm backward: rows up to 1024 threads x 4 vectors x 8 bf16; the
// grid (and the number of dgamma / dbeta partial rows) is at most 256
// workgroups of 1024 threads, or as many threads in smaller workgroups.
constexpr int kLnBwdMaxCols = 1024 * 4 * 8;
constexpr int kLnBwdWgs1024 = 256;

// LayerNorm forward, pipelined rows: a workgroup takes kLnPipeMinRows to
// kLnPipeMaxRows rows (3 in flight). Taken automatically from 3 rows per CU
// on: 2048 x 32768 bf16 on MI355X ran 44.9 us against 48.8 us with one row
// per workgroup.
constexpr int kLnPipeMinRows = 3, kLnPipeMaxRows = 8;
constexpr int64_t kLnPipeMinRowsPerCu = 3;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
int pow2_ceil(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

void clear(fr_plan* p, int op) {
    *p = fr_plan{};
    p->op = op;
    p->splits = 1;
    p->rows_per_wg = 1;
}

// Launch knobs before the grid and workspace follow from the shape.
struct Knobs {
    int form = 0;
    int threads = 256;
    int seg = 64;
    int vec = 1;
    int rpw = 1;     // rows per lane group (persistent fp32); rows per workgroup (pipelined LayerNorm)
    int chunk = 0;   // elements per split chunk (sum split)
    int occ = 0;     // minimum waves per SIMD (persistent LayerNorm)
    int passes = 0;  // split softmax: 1 single read with in-kernel exchange, 2 two kernels, 0 automatic
    int wait_us = 0; // single-pass split softmax: wait for a row's partials (0 default, < 0 none)
    int num_cus = 0; // device compute units (sizes persistent grids only; results do not depend on it)
};

// Single-pass split softmax: resident waves per SIMD (the compiler's
// occupancy for the 256-thread, 8-vector kernel, which holds two chunks in
// registers; the grid is sized so that every workgroup is resident at once)
// and the default wait before a workgroup computes a missing partial itself.
constexpr int kOnePassWavesPerSimd = 4;
constexpr int kOnePassWaitUs = 200;
// Split-row LayerNorm backward: the default wait for a partner's row sums,
// and the fewest rows for which the automatic choice takes that form.
constexpr int kLnTeamWaitUs = 200;
constexpr int64_t kLnTeamMinRows = 256;

// Persistent fp32 geometry: the smallest lane group (8..64 lanes) whose
// 16-byte vectors cover the row with at most 8 vectors per lane.
Knobs per_f32_knobs(int64_t rows, int64_t cols, bool two_rows_ok) {
    Knobs k;
    k.form = FR_FORM_PER;
    const int q = (int)cdiv(cols, 4);
    k.seg = q <= 8 ? 8 : (q <= 16 ? 16 : (q <= 32 ? 32 : 64));
    int nv = (int)cdiv(q, k.seg);
    k.vec = nv <= 1 ? 1 : pow2_ceil(nv);
    k.rpw = (two_rows_ok && k.seg == 64 && k.vec <= 4 && rows <= kTwoRowsPerWaveMaxRows) ? 2 : 1;
    return k;
}

// A full reduction (one row) splits into kFullSplitTargetWgs chunks: the
// configuration search measured 2^28 fp32 at 151.5 us with 2^19-element
// chunks (512) against 154.6 us with 2^17 (2048).
constexpr int kFullSplitTargetWgs = 512;

int64_t sum_split_count(int64_t rows, int64_t cols, int64_t step) {
    const int64_t target = rows == 1 ? kFullSplitTargetWgs : kSplitTargetWgs;
    int64_t s = min64(cdiv(target, rows), cdiv(cols, step));
    return s < 1 ? 1 : s;
}

// Turn knobs into a complete plan for this shape: grid, splits, workspace.
// Returns FR_E_ARG when the knobs cannot serve the shape.
int finalize_plan(int op, int64_t rows, int64_t cols, const Knobs& k, fr_plan* p) {
    p->form = k.form;
    p->threads = k.threads;
    p->vec = k.vec;
    p->occupancy = k.occ;
    if (k.threads < 64 || k.threads > 1024 || k.threads % 64 || k.vec < 1 || k.vec > 16) return FR_E_ARG;
    const bool f32 = op != FR_OP_LAYERNORM && op != FR_OP_LAYERNORM_BWD;
    if (k.form == FR_FORM_PER) {
        if (op == FR_OP_LAYERNORM_BWD) {
            if (cols > (int64_t)k.threads * 8 * k.vec) return FR_E_ARG;
            // one partial row of dgamma / dbeta per workgroup: enough
            // workgroups to fill the device, and at least 16 rows per
            // workgroup where the rows allow it, so the partials stay small
            // next to the rows themselves
            p->grid = min64(min64(rows, std::max<int64_t>(kLnBwdWgs1024, rows / 16)),
                            (int64_t)kLnBwdWgs1024 * 1024 / k.threads);
            // the partial rows after the split form's header (see
            // launch_layernorm_bwd)
            p->ws_bytes = p->grid > 0 ? (uint64_t)(kLnTeamHeader + 2 * p->grid * ln_bwd_ldw(cols) * 4) : 0;
            return FR_OK;
        }
        if (f32) {
            if (k.threads != 256 || !is_pow2(k.seg) || k.seg < 8 || k.seg > 64 || !is_pow2(k.rpw) || k.rpw > 4)
                return FR_E_ARG;
            if (cols > (int64_t)4 * k.seg * k.vec) return FR_E_ARG;
            p->seg = k.seg;
            p->rows_per_wg = 256 / k.seg * k.rpw;
            p->grid = min64(cdiv(rows, p->rows_per_wg), kMaxGrid);
        } else {
            if (cols > (int64_t)k.threads * 8 * k.vec) return FR_E_ARG;
            if (k.rpw > 1) {
                // pipelined rows: 16-byte rows that fill the capacity exactly
                if (k.threads != 512 || k.vec != 8 || k.rpw < kLnPipeMinRows || k.rpw > kLnPipeMaxRows ||
                    cols != (int64_t)k.threads * 8 * k.vec || !p->vec16)
                    return FR_E_ARG;
                p->rows_per_wg = k.rpw;
                p->grid = cdiv(rows, k.rpw);
                if (p->grid > kMaxGrid) return FR_E_ARG;
            } else {
                p->grid = min64(rows, kMaxGrid);
            }
        }
        return FR_OK;
    }
    if (k.form == FR_FORM_RED) {
        p->grid = min64(rows, kMaxGrid);
        return FR_OK;
    }
    if (k.form == FR_FORM_SPLIT && op == FR_OP_LAYERNORM_BWD) {
        // a team of P workgroups per row, one 16-byte vector per lane and
        // member; as many teams as fill the device, at most one per row
        if (rows < 1 || cols <= kLnTeamPartCols || cols > 4 * kLnTeamPartCols) return FR_E_ARG;
        const int64_t parts = cdiv(cols, kLnTeamPartCols);
        if (rows * parts * 16 >= (int64_t(1) << 31)) return FR_E_ARG;  // slot offsets are 32-bit
        const int64_t teams = min64(rows, std::max<int64_t>(1, kLnBwdWgs1024 / parts));
        p->threads = 1024;
        p->vec = 1;
        p->splits = (int)parts;
        p->chunk = (int)(cdiv(cdiv(cols, parts), 8) * 8);
        p->grid = teams * parts;
        p->ws_bytes = (uint64_t)(kLnTeamHeader + ln_team_slots_bytes(rows, parts) + 2 * teams * ln_bwd_ldw(cols) * 4);
        p->wait_us = k.wait_us == 0 ? kLnTeamWaitUs : k.wait_us;
        return FR_OK;
    }
    if (k.form == FR_FORM_SPLIT) {
        if (!f32 || rows < 1 || cols < 1) return FR_E_ARG;
        if (op == FR_OP_SOFTMAX) {
            const int64_t chunk = (int64_t)k.threads * 4 * k.vec;
            const int64_t s = cdiv(cols, chunk);
            // One kernel by default where the row lengths fit in LDS: measured
            // on MI355X (512 ragged rows of up to 131071), it takes 0.78x the
            // time of the two-kernel form, which reads x twice.
            const bool one_ok = rows <= kOnePassMaxRows && rows * s < (int64_t(1) << 31);
            const int passes = k.passes == 0 ? (one_ok ? 1 : 2) : k.passes;
            if (passes != 1 && passes != 2) return FR_E_ARG;
            if (passes == 1 && !one_ok) return FR_E_ARG;
            p->splits = (int)s;
            p->chunk = (int)chunk;
            p->passes = passes;
            p->ws_bytes = (uint64_t)(kSplitWsSlots + rows * s * (int64_t)sizeof(SoftmaxPartial));
            if (passes == 1) {
                const int64_t per_cu = std::max(1, kOnePassWavesPerSimd * 4 / (k.threads / 64));
                p->grid = min64(min64(rows * s, (int64_t)(k.num_cus > 0 ? k.num_cus : 256) * per_cu),
                                kOnePassMaxGrid);
                p->grid2 = 0;
                p->wait_us = k.wait_us == 0 ? kOnePassWaitUs : k.wait_us;
            } else {
                p->grid = rows * s;
                p->grid2 = rows * s;
            }
        } else {
            const int64_t step = (int64_t)k.threads * 4 * k.vec;
            int64_t chunk = k.chunk;
            if (chunk <= 0) chunk = cdiv(cdiv(cols, sum_split_count(rows, cols, step)), step) * step;
            if (chunk % step) return FR_E_ARG;
            const int64_t s = cdiv(cols, chunk);
            if (s > kPerMaxF32) return FR_E_ARG;  // the finishing pass is one persistent row
            p->splits = (int)s;
            p->chunk = (int)chunk;
            p->grid = rows * s;
            const int seg = s <= 32 ? 8 : (s <= 64 ? 16 : (s <= 128 ? 32 : 64));
            p->grid2 = cdiv(rows, 256 / seg);
            p->ws_bytes = (uint64_t)(rows * s * 4);
        }
        if (p->grid * p->threads >= (int64_t(1) << 32)) return FR_E_ARG;
        return FR_OK;
    }
    return FR_E_ARG;
}

}  // namespace

uint64_t sum_split_ws(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    fr_plan p;
    clear(&p, FR_OP_SUMSQ);
    Knobs k;
    k.form = FR_FORM_SPLIT;
    k.threads = kSumSplitThreads;
    k.vec = kSumSplitU;
    return finalize_plan(FR_OP_SUMSQ, rows, cols, k, &p) == FR_OK ? p.ws_bytes : 0;
}

uint64_t softmax_split_ws(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    fr_plan p;
    clear(&p, FR_OP_SOFTMAX);
    Knobs k;
    k.form = FR_FORM_SPLIT;
    k.threads = kSoftmaxSplitThreads;
    k.vec = kSoftmaxSplitNV;
    return finalize_plan(FR_OP_SOFTMAX, rows, cols, k, &p) == FR_OK ? p.ws_bytes : 0;
}

int make_plan(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int has_lengths, uint64_t ws_bytes,
              int aligned16, int forced, const fr_plan* override_plan, fr_plan* p) {
    (void)has_lengths;
    // thresholds are fixed per library build so that workspace sizes and
    // results do not depend on the device; num_cus only sizes persistent grids
    if (!p) return FR_E_NULL;
    if (rows < 0 || cols < 0 || rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 30)) return FR_E_SIZE;
    if (forced < FR_FORM_AUTO || forced > FR_FORM_SPLIT) return FR_E_ARG;
    clear(p, op);
    p->vec16 = aligned16 ? 1 : 0;
    Knobs k;
    switch (op) {
        case FR_OP_SUM_RELU_ADD:
        case FR_OP_SUMSQ: {
            if (dtype != FR_F32) return FR_E_DTYPE;
            const bool per_ok = cols <= kPerMaxF32;
            const bool split_ok = cols > 0 && rows > 0 && ws_bytes >= sum_split_ws(rows, cols);
            int form = forced;
            if (form == FR_FORM_AUTO)
                form = per_ok ? FR_FORM_PER : (split_ok && rows < kSumSplitRows ? FR_FORM_SPLIT : FR_FORM_RED);
            if (form == FR_FORM_PER) {
                if (!per_ok) return FR_E_ARG;
                k = per_f32_knobs(rows, cols, false);
            } else if (form == FR_FORM_RED) {
                k.form = FR_FORM_RED;
                k.threads = 256;
                k.vec = 4;
            } else {
                if (!split_ok) return FR_E_ARG;
                k.form = FR_FORM_SPLIT;
                k.threads = kSumSplitThreads;
                k.vec = kSumSplitU;
            }
            break;
        }
        case FR_OP_SOFTMAX: {
            if (dtype != FR_F32) return FR_E_DTYPE;
            const bool per_ok = cols <= kPerMaxF32;
            const bool split_ok = cols > 0 && rows > 0 && ws_bytes >= softmax_split_ws(rows, cols);
            int form = forced;
            if (form == FR_FORM_AUTO)
                form = per_ok ? FR_FORM_PER
                              : (split_ok && rows < kSoftmaxSplitRows ? FR_FORM_SPLIT : FR_FORM_RED);
            if (form == FR_FORM_PER) {
                if (!per_ok) return FR_E_ARG;
                k = per_f32_knobs(rows, cols, true);
            } else if (form == FR_FORM_RED) {
                k.form = FR_FORM_RED;
                k.threads = cols > 16384 ? 512 : 256;
                k.vec = cols > 16384 ? 2 : 4;
            } else {
                if (!split_ok) return FR_E_ARG;
                k.form = FR_FORM_SPLIT;
                k.threads = kSoftmaxSplitThreads;
                k.vec = kSoftmaxSplitNV;
            }
            break;
        }
        case FR_OP_SOFTMAX_BWD: {
            // persistent rows up to kPerMaxF32 (y and dy both in registers),
            // looped beyond; there is no split form
            if (dtype != FR_F32) return FR_E_DTYPE;
            const bool per_ok = cols <= kPerMaxF32;
            const int form = forced == FR_FORM_AUTO ? (per_ok ? FR_FORM_PER : FR_FORM_RED) : forced;
            if (form == FR_FORM_PER) {
                if (!per_ok) return FR_E_ARG;
                // one row per wave: with three arrays in flight two rows per
                // wave measured slower (9.96 against 9.62 us at 4096 x 1024)
                k = per_f32_knobs(rows, cols, false);
            } else if (form == FR_FORM_RED) {
                k.form = FR_FORM_RED;
                k.threads = cols > 16384 ? 512 : 256;
                k.vec = cols > 16384 ? 2 : 4;
            } else {
                return FR_E_ARG;
            }
            break;
        }
        case FR_OP_LAYERNORM: {
            if (dtype != FR_BF16) return FR_E_DTYPE;
            if (cols < 1) return FR_E_SIZE;
            // a workgroup of up to 512 threads holds the row: 8 vectors of
            // 8 bf16 per lane with 16-byte accesses, 4 with element accesses
            const int nv_max = aligned16 ? 8 : 4;
            const bool per_ok = cols <= (int64_t)512 * 8 * nv_max;
            int form = forced == FR_FORM_AUTO ? (per_ok ? FR_FORM_PER : FR_FORM_RED) : forced;
            if (form == FR_FORM_PER) {
                if (!per_ok) return FR_E_ARG;
                const int q = (int)cdiv(cols, 8);  // 8-element vectors per row
                int t = pow2_ceil((int)cdiv(q, nv_max));
                int nv = nv_max;
                if (t < 64) {
                    t = 64;
                    nv = pow2_ceil((int)cdiv(q, 64));
                }
                k.form = FR_FORM_PER;
                k.threads = t;
                k.vec = nv;
                // rows that fill 512 threads x 8 vectors exactly, at least
                // kLnPipeMinRowsPerCu per CU: one pipelined workgroup per CU
                // takes up to 8 of them (same bits as one row per workgroup)
                const int64_t cus = num_cus > 0 ? num_cus : 256;
                if (aligned16 && t == 512 && nv == 8 && cols == (int64_t)512 * 8 * 8 &&
                    rows >= kLnPipeMinRowsPerCu * cus)
                    k.rpw = (int)std::min<int64_t>(kLnPipeMaxRows, cdiv(rows, cus));
            } else if (form == FR_FORM_RED) {
                k.form = FR_FORM_RED;
                k.threads = 512;
                k.vec = 2;
            } else {
                return FR_E_ARG;  // rows of LayerNorm are never split
            }
            break;
        }
        case FR_OP_LAYERNORM_BWD: {
            // persistent: a workgroup holds the rows of x and dy, and each
            // lane the dgamma / dbeta partials of its columns, in registers
            // (at most 4 vectors of 8 bf16 per lane and array). Split: rows
            // longer than one member's part, shared by a team of workgroups,
            // when the accesses are 16-byte and the workspace holds the
            // exchange slots (automatic from kLnTeamMinRows rows on).
            if (dtype != FR_BF16) return FR_E_DTYPE;
            if (cols < 1 || cols > kLnBwdMaxCols) return FR_E_SIZE;
            if (forced == FR_FORM_SPLIT || forced == FR_FORM_AUTO) {
                Knobs t;
                t.form = FR_FORM_SPLIT;
                fr_plan tp;
                clear(&tp, op);
                const bool fits = aligned16 && finalize_plan(op, rows, cols, t, &tp) == FR_OK && ws_bytes >= tp.ws_bytes;
                if (forced == FR_FORM_SPLIT || (fits && rows >= kLnTeamMinRows)) {
                    if (!aligned16 || rows < 1) return FR_E_ARG;
                    k = t;
                    break;
                }
            }
            if (forced != FR_FORM_AUTO && forced != FR_FORM_PER) return FR_E_ARG;
            const int q = (int)cdiv(cols, 8);
            const int t = std::min(1024, std::max(128, pow2_ceil(q)));
            k.form = FR_FORM_PER;
            k.threads = t;
            k.vec = pow2_ceil((int)cdiv(q, t));
            break;
        }
        default:
            return FR_E_ARG;
    }
    if (override_plan) {
        // a tuner's candidate: form and launch knobs from the override,
        // grid / splits / workspace recomputed for this shape
        k.form = override_plan->form;
        k.threads = override_plan->threads;
        k.seg = override_plan->seg;
        k.vec = override_plan->vec;
        if (op == FR_OP_LAYERNORM)
            k.rpw = override_plan->form == FR_FORM_PER && override_plan->rows_per_wg > 1 ? override_plan->rows_per_wg : 1;
        else
            k.rpw = (override_plan->seg > 0 && override_plan->form == FR_FORM_PER)
                        ? override_plan->rows_per_wg / (256 / override_plan->seg)
                        : 1;
        k.chunk = override_plan->chunk;
        k.occ = override_plan->occupancy;
        k.passes = override_plan->passes;
        k.wait_us = override_plan->wait_us;
    }
    k.num_cus = num_cus;
    const int st = finalize_plan(op, rows, cols, k, p);
    if (st != FR_OK) return st;
    if (p->form == FR_FORM_SPLIT && ws_bytes < p->ws_bytes)
        return (override_plan || op == FR_OP_LAYERNORM_BWD) ? FR_E_WORKSPACE : FR_E_ARG;
    return FR_OK;
}

// Pointwise kernels ("Stax (4)", 9.3). The 2-D add covers its output with
// rows_per_wg x chunk tiles, 64 x 128 by default (32 KB of LDS per
// transposed operand; measured at 8192 x 8192 with one transposed operand:
// 140 us against 159 us for 64 x 64 and 143 us for 32 x 128). GELU backward
// streams 16-byte vectors, `vec` per lane per step (2: 346 us at 2^28 fp32,
// 350 us with 4, 394 us with 1), one step per thread. An override's grid > 0
// caps the grid (grid-stride loops cover the rest; capped grids measured
// slower for both kernels).
constexpr int kAddTileRows = 64, kAddTileCols = 128;
constexpr int kGeluNV = 2;

int make_pointwise_plan(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int aligned16, int forced,
                        const fr_plan* ov, fr_plan* p) {
    (void)num_cus;
    if (!p) return FR_E_NULL;
    if (forced != FR_FORM_AUTO && forced != FR_FORM_POINTWISE) return FR_E_ARG;
    clear(p, op);
    p->form = FR_FORM_POINTWISE;
    p->threads = 256;
    p->vec16 = aligned16 ? 1 : 0;
    p->vec = 1;
    if (ov && ov->threads != 256) return FR_E_ARG;
    const int64_t cap = (ov && ov->grid > 0) ? min64(ov->grid, kMaxGrid) : kMaxGrid;
    if (op == FR_OP_ADD_2D) {
        if (rows < 0 || cols < 0 || rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 30)) return FR_E_SIZE;
        if (dtype != FR_F32) return FR_E_DTYPE;
        const int ti = ov ? ov->rows_per_wg : kAddTileRows;
        const int tj = ov ? ov->chunk : kAddTileCols;
        if (ti < 4 || tj < 4 || ti % 4 || tj % 4 || (ti * tj) % 1024 || ti > 1024 || tj > 1024) return FR_E_ARG;
        p->rows_per_wg = ti;
        p->chunk = tj;
        p->grid = min64(cdiv(rows, ti) * cdiv(cols, tj), cap);
        return FR_OK;
    }
    if (op == FR_OP_GELU_BWD) {
        if (rows < 0 || cols < 0 || (rows > 0 && cols > (int64_t(1) << 40) / rows)) return FR_E_SIZE;
        const int64_t n = rows * cols;
        if (n >= (int64_t(1) << 40)) return FR_E_SIZE;
        if (dtype != FR_F32 && dtype != FR_BF16) return FR_E_DTYPE;
        const int nv = ov ? ov->vec : kGeluNV;
        if (nv != 1 && nv != 2 && nv != 4) return FR_E_ARG;
        p->vec = nv;
        const int64_t per = dtype == FR_F32 ? 4 : 8;
        const int64_t units = aligned16 ? cdiv(n / per, (int64_t)256 * nv) : cdiv(n, 256);
        p->grid = n == 0 ? 0 : std::max<int64_t>(1, min64(units, cap));
        return FR_OK;
    }
    return FR_E_ARG;
}

}  // namespace fr

