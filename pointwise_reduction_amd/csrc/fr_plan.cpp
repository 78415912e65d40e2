// fr_plan.cpp - reduction-form selection and launch configuration.
//
// Host-only code (no HIP call), so the choice can be inspected and tested
// without a GPU. The structure follows "Stax (4): GPU Codegen and Dynamic
// Shapes": 9.4 picks the form from the reduction length (persistent when the
// row fits, looped when it does not, split when there are too few outputs to
// fill the device); 9.6 makes block sizes and warp counts launch parameters
// whose grid follows from them; 10.3 decides against the upper bound of a
// runtime length (here `cols`, the row capacity of a ragged input).
//
// The MI355X thresholds differ from the pages' Triton/H100 rule (persistent
// up to 1024 elements): a 64-lane wave holding 8 x 16-byte vectors per lane
// keeps 2048 fp32 values in 32 VGPRs, and a 512-thread workgroup holds a
// 32K-element bf16 row in registers (32 VGPRs of packed bf16 per lane).
#include <stdint.h>

#include "fr_internal.h"

namespace fr {

namespace {

constexpr int64_t kMaxGrid = 1 << 20;    // grid-stride loops cover the rest
constexpr int kPerMaxF32 = 2048;         // 64 lanes x 8 vectors x 4 floats
constexpr int kSumSplitRows = 512;       // fewer rows than 2 per CU: split
constexpr int kSoftmaxSplitRows = 1024;  // fewer rows than 4 per CU: split
constexpr int kSplitTargetWgs = 2048;    // 8 workgroups per CU on 256 CUs
constexpr int kSumSplitThreads = 256, kSumSplitU = 4;     // 4096 floats per step
constexpr int kSoftmaxSplitThreads = 256, kSoftmaxSplitNV = 8;  // 8192-float chunks

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
int pow2_ceil(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

void clear(fr_plan* p, int op) {
    *p = fr_plan{};
    p->op = op;
    p->splits = 1;
    p->rows_per_wg = 1;
}

// Persistent geometry for fp32 rows of `cols` <= 2048 elements: the smallest
// lane group (8..64 lanes) whose 16-byte vectors cover the row with at most
// 8 vectors per lane.
void per_f32(fr_plan* p, int64_t rows, int64_t cols) {
    const int q = (int)cdiv(cols, 4);
    const int seg = q <= 8 ? 8 : (q <= 16 ? 16 : (q <= 32 ? 32 : 64));
    int nv = (int)cdiv(q, seg);
    nv = nv <= 1 ? 1 : pow2_ceil(nv);
    p->form = FR_FORM_PER;
    p->threads = 256;
    p->seg = seg;
    p->vec = nv;
    p->rows_per_wg = 256 / seg;
    p->grid = min64(cdiv(rows, p->rows_per_wg), kMaxGrid);
}

void sum_split(fr_plan* p, int64_t rows, int64_t cols) {
    const int64_t step = (int64_t)kSumSplitThreads * 4 * kSumSplitU;
    int64_t s = min64(cdiv(kSplitTargetWgs, rows), cdiv(cols, step));
    if (s < 1) s = 1;
    const int64_t chunk = cdiv(cdiv(cols, s), step) * step;
    s = cdiv(cols, chunk);
    p->form = FR_FORM_SPLIT;
    p->threads = kSumSplitThreads;
    p->vec = kSumSplitU;
    p->splits = (int)s;
    p->chunk = (int)chunk;
    p->grid = rows * s;
    // finishing pass: a persistent reduction over rows of s partials
    const int seg = s <= 32 ? 8 : (s <= 64 ? 16 : (s <= 128 ? 32 : 64));
    p->grid2 = cdiv(rows, 256 / seg);
    p->ws_bytes = (uint64_t)(rows * s * 4);
}

void softmax_split(fr_plan* p, int64_t rows, int64_t cols) {
    const int64_t chunk = (int64_t)kSoftmaxSplitThreads * 4 * kSoftmaxSplitNV;
    const int64_t s = cdiv(cols, chunk);
    p->form = FR_FORM_SPLIT;
    p->threads = kSoftmaxSplitThreads;
    p->vec = kSoftmaxSplitNV;
    p->splits = (int)s;
    p->chunk = (int)chunk;
    p->grid = rows * s;
    p->grid2 = rows * s;
    p->ws_bytes = (uint64_t)(rows * s * (int64_t)sizeof(SoftmaxPartial));
}

}  // namespace

uint64_t sum_split_ws(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    fr_plan p;
    clear(&p, FR_OP_SUMSQ);
    sum_split(&p, rows, cols);
    return p.ws_bytes;
}

uint64_t softmax_split_ws(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    fr_plan p;
    clear(&p, FR_OP_SOFTMAX);
    softmax_split(&p, rows, cols);
    return p.ws_bytes;
}

int make_plan(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int has_lengths, uint64_t ws_bytes,
              int aligned16, int forced, fr_plan* p) {
    (void)has_lengths;
    (void)num_cus;  // the thresholds are fixed per library build so that
                    // workspace sizes and results do not depend on the device
    if (!p) return FR_E_NULL;
    if (rows < 0 || cols < 0 || rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 30)) return FR_E_SIZE;
    if (forced < FR_FORM_AUTO || forced > FR_FORM_SPLIT) return FR_E_ARG;
    clear(p, op);
    p->vec16 = aligned16 ? 1 : 0;
    switch (op) {
        case FR_OP_SUM_RELU_ADD:
        case FR_OP_SUMSQ: {
            if (dtype != FR_F32) return FR_E_DTYPE;
            const bool per_ok = cols <= kPerMaxF32;
            const uint64_t need = sum_split_ws(rows, cols);
            const bool split_ok = cols > 0 && rows > 0 && ws_bytes >= need;
            int form = forced;
            if (form == FR_FORM_AUTO)
                form = per_ok ? FR_FORM_PER
                              : (split_ok && rows < kSumSplitRows ? FR_FORM_SPLIT : FR_FORM_RED);
            if (form == FR_FORM_PER) {
                if (!per_ok) return FR_E_ARG;
                per_f32(p, rows, cols);
            } else if (form == FR_FORM_RED) {
                p->form = FR_FORM_RED;
                p->threads = 256;
                p->vec = 4;
                p->grid = min64(rows, kMaxGrid);
            } else {
                if (!split_ok) return FR_E_ARG;
                sum_split(p, rows, cols);
                if (p->grid * p->threads >= (int64_t(1) << 32)) return FR_E_ARG;
            }
            return FR_OK;
        }
        case FR_OP_SOFTMAX: {
            if (dtype != FR_F32) return FR_E_DTYPE;
            const bool per_ok = cols <= kPerMaxF32;
            const uint64_t need = softmax_split_ws(rows, cols);
            const bool split_ok = cols > 0 && rows > 0 && ws_bytes >= need;
            int form = forced;
            if (form == FR_FORM_AUTO)
                form = per_ok ? FR_FORM_PER
                              : (split_ok && rows < kSoftmaxSplitRows ? FR_FORM_SPLIT : FR_FORM_RED);
            if (form == FR_FORM_PER) {
                if (!per_ok) return FR_E_ARG;
                per_f32(p, rows, cols);
            } else if (form == FR_FORM_RED) {
                p->form = FR_FORM_RED;
                p->threads = cols > 16384 ? 512 : 256;
                p->vec = cols > 16384 ? 2 : 4;
                p->grid = min64(rows, kMaxGrid);
            } else {
                if (!split_ok) return FR_E_ARG;
                softmax_split(p, rows, cols);
                if (p->grid * p->threads >= (int64_t(1) << 32)) return FR_E_ARG;
            }
            return FR_OK;
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
                p->form = FR_FORM_PER;
                p->threads = t;
                p->vec = nv;
            } else if (form == FR_FORM_RED) {
                p->form = FR_FORM_RED;
                p->threads = 512;
                p->vec = 2;
            } else {
                return FR_E_ARG;  // rows of LayerNorm are never split
            }
            p->grid = min64(rows, kMaxGrid);
            return FR_OK;
        }
    }
    return FR_E_ARG;
}

}  // namespace fr
