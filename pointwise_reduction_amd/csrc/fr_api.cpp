// fr_api.cpp - the C ABI of libfr: argument checks, plan, launch.
//
// Mirrors the wrapper of "Stax (4): GPU Codegen and Dynamic Shapes", 9.7
// (Listing 9.6): sizes and strides are checked before anything runs, the
// kernels of one call are enqueued on the caller's stream in program order
// with no synchronization, and scratch memory comes from the caller. Every
// argument error is reported before the first HIP call. An unsupported
// device or dtype is an error, never a silent fallback (9.10 makes the same
// choice for an unavailable attention backend).
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>

#include "fr.h"
#include "fr_internal.h"

namespace fr {
uint64_t sum_split_ws(int64_t rows, int64_t cols);
uint64_t softmax_split_ws(int64_t rows, int64_t cols);
}  // namespace fr

using namespace fr;

namespace {

int g_forced_form = FR_FORM_AUTO;

// Tuning overrides, one per operation (index = FR_OP_*).
constexpr int kOps = 9;
fr_plan g_override[kOps];
bool g_has_override[kOps] = {};

// Recorded selections ("Stax (4)", 9.6, Algorithm 9.1, lines 1 and 7): the
// configuration a tuner measured best for one (operation, shape, dtype).
struct RecordKey {
    int op;
    int64_t rows, cols;
    int dtype;
    bool operator<(const RecordKey& o) const {
        if (op != o.op) return op < o.op;
        if (rows != o.rows) return rows < o.rows;
        if (cols != o.cols) return cols < o.cols;
        return dtype < o.dtype;
    }
};
std::map<RecordKey, fr_plan> g_records;
std::mutex g_records_mu;
thread_local fr_plan t_record;  // the record in use by this thread's current call

// A process-wide override (tuning) wins; then a recorded selection for this
// exact shape; else the planner's defaults.
const fr_plan* override_for(int op, int64_t rows, int64_t cols, int dtype) {
    if (op > 0 && op < kOps && g_has_override[op]) return &g_override[op];
    std::lock_guard<std::mutex> lk(g_records_mu);
    if (g_records.empty()) return nullptr;
    auto it = g_records.find(RecordKey{op, rows, cols, dtype});
    if (it == g_records.end()) return nullptr;
    t_record = it->second;
    return &t_record;
}

constexpr int kMaxDevices = 64;
struct DeviceInfo {
    int state = 0;  // 0 unknown, 1 usable gfx950, -1 unusable
    int num_cus = 0;
    int clock_khz = 0;  // constant wall clock read by wall_clock64()
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Current device: usable gfx950? Queried once per device, then cached.
int device_check(int* num_cus, int* clock_khz = nullptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FR_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceInfo& d = g_dev[dev];
    if (d.state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            d.state = -1;
        } else {
            d.state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
            d.num_cus = prop.multiProcessorCount;
            int khz = 0;
            if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
                khz = 100000;  // the documented 100 MHz constant clock
            d.clock_khz = khz;
        }
    }
    if (d.state != 1) return FR_E_DEVICE;
    *num_cus = d.num_cus;
    if (clock_khz) *clock_khz = d.clock_khz;
    return FR_OK;
}

bool aligned(const void* p, uintptr_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; }

// Checks common to every row-major [rows, cols] operand.
// A [rows, 0] operand is never dereferenced and may be NULL.
int check_matrix(const void* p, int64_t rows, int64_t cols, int64_t rs, int64_t cs, size_t elem) {
    if (!p) return cols == 0 ? FR_OK : FR_E_NULL;
    if (cs != 1) return FR_E_STRIDE;
    if (rs < 0 || (rows > 1 && rs < cols)) return FR_E_STRIDE;
    if (!aligned(p, elem)) return FR_E_ALIGN;
    return FR_OK;
}

// Do two row-major operands share any byte? Each spans from its base to the
// end of its last row.
bool spans_overlap(const void* p, int64_t p_rs, const void* q, int64_t q_rs, int64_t rows, int64_t cols,
                   size_t elem) {
    if (!p || !q || rows == 0 || cols == 0) return false;
    const uintptr_t a0 = (uintptr_t)p, b0 = (uintptr_t)q;
    const uintptr_t a1 = a0 + (uintptr_t)(((rows - 1) * p_rs + cols) * (int64_t)elem);
    const uintptr_t b1 = b0 + (uintptr_t)(((rows - 1) * q_rs + cols) * (int64_t)elem);
    return a0 < b1 && b0 < a1;
}

bool vec_ok(const void* p, int64_t rs, int64_t elems_per_vec) {
    return p == nullptr || (((uintptr_t)p % 16) == 0 && rs % elems_per_vec == 0);
}

// rows < 2^31; cols < 2^30 keeps every in-row offset, including the padding
// of the last loop step, inside a 32-bit int.
constexpr int64_t kMaxRows = int64_t(1) << 31;
constexpr int64_t kMaxCols = int64_t(1) << 30;

int check_sizes(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return FR_E_SIZE;
    if (rows >= kMaxRows || cols >= kMaxCols) return FR_E_SIZE;
    return FR_OK;
}

// A plan whose kernel was not compiled (only reachable through a tuning
// override) is an argument error; any other failure is a launch error.
int finish_launch(hipError_t e) {
    if (e == hipSuccess) return FR_OK;
    return e == hipErrorInvalidDeviceFunction ? FR_E_ARG : FR_E_LAUNCH;
}

int run_sum(int prologue, const void* a, const void* b, void* out, int64_t rows, int64_t cols, int64_t a_rs,
            int64_t b_rs, int64_t out_s, void* ws, uint64_t ws_bytes, void* stream) {
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    const int v16 = vec_ok(a, a_rs, 4) && vec_ok(b, b_rs, 4);
    fr_plan plan;
    const int op = prologue == kReluAdd ? FR_OP_SUM_RELU_ADD : FR_OP_SUMSQ;
    st = make_plan(op, rows, cols, FR_F32, num_cus, 0, ws ? ws_bytes : 0, v16, g_forced_form,
                   override_for(op, rows, cols, FR_F32), &plan);
    if (st != FR_OK) return st;
    SumArgs args{prologue, (const float*)a, (const float*)b, (float*)out, (int)rows, (int)cols, a_rs, b_rs, out_s,
                 (float*)ws};
    (void)hipGetLastError();  // clear a stale error so the launch status is ours
    return finish_launch(launch_sum(plan, args, (hipStream_t)stream));
}

// Layout of one operand of the 2-D add: 0 row-major, 1 column-major (a
// transposed view), -1 neither.
int add2d_layout(int64_t rows, int64_t cols, int64_t rs, int64_t cs) {
    if (rs < 0 || cs < 0) return -1;
    if (cs == 1 && (rows == 1 || rs >= cols)) return 0;
    if (rs == 1 && (cols == 1 || cs >= rows)) return 1;
    return -1;
}

}  // namespace

extern "C" {

const char* fr_status_string(int status) {
    switch (status) {
        case FR_OK: return "FR_OK: success";
        case FR_E_NULL: return "FR_E_NULL: a required pointer is NULL";
        case FR_E_SIZE: return "FR_E_SIZE: a size is negative or too large";
        case FR_E_STRIDE: return "FR_E_STRIDE: column stride must be 1 and row stride >= cols";
        case FR_E_DTYPE: return "FR_E_DTYPE: dtype not supported by this entry point";
        case FR_E_ALIGN: return "FR_E_ALIGN: pointer not aligned to its element (workspace: 16 bytes)";
        case FR_E_WORKSPACE: return "FR_E_WORKSPACE: workspace missing or too small";
        case FR_E_ARG: return "FR_E_ARG: invalid argument";
        case FR_E_DEVICE: return "FR_E_DEVICE: no usable gfx950 device";
        case FR_E_LAUNCH: return "FR_E_LAUNCH: kernel launch failed";
    }
    return "unknown status";
}

int fr_version(void) { return 100; }

int fr_force_form(int form) {
    const int prev = g_forced_form;
    if (form >= FR_FORM_AUTO && form <= FR_FORM_POINTWISE) g_forced_form = form;
    return prev;
}

int fr_plan_query(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int has_lengths, uint64_t ws_bytes,
                  int aligned16, fr_plan* plan) {
    if (!plan) return FR_E_NULL;
    if (op == FR_OP_ADD_2D || op == FR_OP_GELU_BWD)
        return make_pointwise_plan(op, rows, cols, dtype, num_cus, aligned16, g_forced_form,
                                   override_for(op, rows, cols, dtype), plan);
    return make_plan(op, rows, cols, dtype, num_cus, has_lengths, ws_bytes, aligned16, g_forced_form,
                     override_for(op, rows, cols, dtype), plan);
}

int fr_tune_override(int op, const fr_plan* plan) {
    if (op <= 0 || op >= kOps) return FR_E_ARG;
    if (plan) {
        g_override[op] = *plan;
        g_has_override[op] = true;
    } else {
        g_has_override[op] = false;
    }
    return FR_OK;
}

int fr_tune_record(int op, int64_t rows, int64_t cols, int dtype, const fr_plan* plan) {
    if (op <= 0 || op >= kOps) return FR_E_ARG;
    if (rows < 0 || cols < 0) return FR_E_SIZE;
    std::lock_guard<std::mutex> lk(g_records_mu);
    const RecordKey key{op, rows, cols, dtype};
    if (plan) g_records[key] = *plan;
    else g_records.erase(key);
    return FR_OK;
}

int fr_tune_lookup(int op, int64_t rows, int64_t cols, int dtype, fr_plan* plan) {
    if (!plan) return FR_E_NULL;
    std::lock_guard<std::mutex> lk(g_records_mu);
    auto it = g_records.find(RecordKey{op, rows, cols, dtype});
    if (it == g_records.end()) return FR_E_ARG;
    *plan = it->second;
    return FR_OK;
}

void fr_tune_clear(void) {
    std::lock_guard<std::mutex> lk(g_records_mu);
    g_records.clear();
}

uint64_t fr_sum_workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    if (dtype != FR_F32 || check_sizes(rows, cols) != FR_OK) return 0;
    return sum_split_ws(rows, cols);
}

int fr_sum_relu_add(const void* a, const void* b, void* out, int64_t rows, int64_t cols, int64_t a_rs,
                    int64_t a_cs, int64_t b_rs, int64_t b_cs, int64_t out_s, void* ws, uint64_t ws_bytes,
                    int dtype, void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (rows == 0) return FR_OK;
    if ((st = check_matrix(a, rows, cols, a_rs, a_cs, 4)) != FR_OK) return st;
    if ((st = check_matrix(b, rows, cols, b_rs, b_cs, 4)) != FR_OK) return st;
    if (!out) return FR_E_NULL;
    if (out_s < 1) return FR_E_STRIDE;
    if (!aligned(out, 4)) return FR_E_ALIGN;
    if (ws && !aligned(ws, 16)) return FR_E_ALIGN;
    return run_sum(kReluAdd, a, b, out, rows, cols, a_rs, b_rs, out_s, ws, ws_bytes, stream);
}

int fr_sumsq_rows(const void* x, void* out, int64_t rows, int64_t cols, int64_t x_rs, int64_t x_cs, void* ws,
                  uint64_t ws_bytes, int dtype, void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (rows == 0) return FR_OK;
    if ((st = check_matrix(x, rows, cols, x_rs, x_cs, 4)) != FR_OK) return st;
    if (!out) return FR_E_NULL;
    if (!aligned(out, 4)) return FR_E_ALIGN;
    if (ws && !aligned(ws, 16)) return FR_E_ALIGN;
    return run_sum(kSquare, x, nullptr, out, rows, cols, x_rs, 0, 1, ws, ws_bytes, stream);
}

uint64_t fr_sumsq_full_workspace_bytes(int64_t n, int dtype) {
    if (dtype != FR_F32 || n <= 2048 || n >= kMaxCols) return 0;
    return sum_split_ws(1, n);
}

int fr_sumsq_full(const void* x, int64_t n, void* out, void* ws, uint64_t ws_bytes, int dtype, void* stream) {
    if (n < 0 || n >= kMaxCols) return FR_E_SIZE;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (!out) return FR_E_NULL;
    if (n > 0 && !x) return FR_E_NULL;
    if (!aligned(x, 4) || !aligned(out, 4)) return FR_E_ALIGN;
    const uint64_t need = fr_sumsq_full_workspace_bytes(n, dtype);
    if (need > 0) {
        if (!ws || ws_bytes < need) return FR_E_WORKSPACE;
        if (!aligned(ws, 16)) return FR_E_ALIGN;
    }
    int num_cus = 0;
    int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    const int v16 = vec_ok(x, 0, 4);
    fr_plan plan;
    // A full reduction has a single output: split whenever the vector does
    // not fit one persistent row (the form is not left to the row heuristics).
    const int form = need > 0 ? FR_FORM_SPLIT : FR_FORM_PER;
    st = make_plan(FR_OP_SUMSQ, 1, n, FR_F32, num_cus, 0, need > 0 ? ws_bytes : 0, v16, form,
                   override_for(FR_OP_SUMSQ, 1, n, FR_F32), &plan);
    if (st != FR_OK) return st;
    SumArgs args{kSquare, (const float*)x, nullptr, (float*)out, 1, (int)n, n, 0, 1, (float*)ws};
    (void)hipGetLastError();
    return finish_launch(launch_sum(plan, args, (hipStream_t)stream));
}

uint64_t fr_softmax_rows_workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    if (dtype != FR_F32 || check_sizes(rows, cols) != FR_OK) return 0;
    return softmax_split_ws(rows, cols);
}

int fr_softmax_rows_workspace_init(void* ws, uint64_t ws_bytes, void* stream) {
    if (!ws) return FR_E_NULL;
    if (!aligned(ws, 16)) return FR_E_ALIGN;
    if (ws_bytes < (uint64_t)kSplitWsHeader) return FR_E_WORKSPACE;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_softmax_ws_init(ws, ws_bytes, (hipStream_t)stream));
}

int fr_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t x_rs, int64_t x_cs, int64_t y_rs,
                    int64_t y_cs, const int32_t* lengths, int32_t* argmax, void* ws, uint64_t ws_bytes, int dtype,
                    void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (rows == 0) return FR_OK;
    if (cols == 0 && !argmax) return FR_OK;  // nothing to read or write
    if ((st = check_matrix(x, rows, cols, x_rs, x_cs, 4)) != FR_OK) return st;
    if ((st = check_matrix(y, rows, cols, y_rs, y_cs, 4)) != FR_OK) return st;
    if (x == y && x_rs != y_rs) return FR_E_STRIDE;
    if (!aligned(lengths, 4) || !aligned(argmax, 4)) return FR_E_ALIGN;
    if (ws) {
        if (!aligned(ws, 16)) return FR_E_ALIGN;
        if (cols > 0 && ws_bytes < softmax_split_ws(rows, cols)) return FR_E_WORKSPACE;
    }
    int num_cus = 0, clock_khz = 0;
    st = device_check(&num_cus, &clock_khz);
    if (st != FR_OK) return st;
    const int v16 = vec_ok(x, x_rs, 4) && vec_ok(y, y_rs, 4);
    const fr_plan* ov = override_for(FR_OP_SOFTMAX, rows, cols, FR_F32);
    fr_plan plan;
    st = make_plan(FR_OP_SOFTMAX, rows, cols, FR_F32, num_cus, lengths != nullptr, ws ? ws_bytes : 0, v16,
                   g_forced_form, ov, &plan);
    if (st != FR_OK) return st;
    // The single-pass split recomputes a late partner's chunk partial from
    // x, and by then that partner may have overwritten its chunk with y. When
    // x and y share memory the split takes two kernels instead (every element
    // is read before it is written, by the same thread); a tuning override
    // that asks for the single pass is an argument error.
    if (plan.form == FR_FORM_SPLIT && plan.passes == 1 && spans_overlap(x, x_rs, y, y_rs, rows, cols, 4)) {
        if (g_has_override[FR_OP_SOFTMAX] && ov && ov->passes == 1) return FR_E_ARG;
        fr_plan two = ov ? *ov : plan;
        two.passes = 2;
        st = make_plan(FR_OP_SOFTMAX, rows, cols, FR_F32, num_cus, lengths != nullptr, ws ? ws_bytes : 0, v16,
                       g_forced_form, &two, &plan);
        if (st != FR_OK) return st;
    }
    const int64_t wait_ticks = plan.wait_us > 0 ? (int64_t)plan.wait_us * clock_khz / 1000 : (plan.wait_us < 0 ? -1 : 0);
    SoftmaxArgs args{(const float*)x, (float*)y, (int)rows, (int)cols, x_rs, y_rs, lengths, argmax, ws, wait_ticks};
    (void)hipGetLastError();
    return finish_launch(launch_softmax(plan, args, (hipStream_t)stream));
}

int fr_layernorm_rows(const void* x, const void* gamma, const void* beta, void* y, int64_t rows, int64_t cols,
                      int64_t x_rs, int64_t x_cs, int64_t y_rs, int64_t y_cs, float eps, int dtype, void* stream) {
    return fr_layernorm_rows_stats(x, gamma, beta, y, nullptr, nullptr, rows, cols, x_rs, x_cs, y_rs, y_cs, eps,
                                   dtype, stream);
}

int fr_layernorm_rows_stats(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                            int64_t rows, int64_t cols, int64_t x_rs, int64_t x_cs, int64_t y_rs, int64_t y_cs,
                            float eps, int dtype, void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_BF16) return FR_E_DTYPE;
    if (cols < 1) return FR_E_SIZE;
    if (!(eps >= 0.0f) || isinf(eps)) return FR_E_ARG;
    if (rows == 0) return FR_OK;
    if ((st = check_matrix(x, rows, cols, x_rs, x_cs, 2)) != FR_OK) return st;
    if ((st = check_matrix(y, rows, cols, y_rs, y_cs, 2)) != FR_OK) return st;
    if (x == y && x_rs != y_rs) return FR_E_STRIDE;
    if (!aligned(gamma, 2) || !aligned(beta, 2) || !aligned(mean, 4) || !aligned(rstd, 4)) return FR_E_ALIGN;
    int num_cus = 0;
    st = device_check(&num_cus);
    if (st != FR_OK) return st;
    const int v16 = cols % 8 == 0 && vec_ok(x, x_rs, 8) && vec_ok(y, y_rs, 8) && vec_ok(gamma, 0, 8) &&
                    vec_ok(beta, 0, 8);
    fr_plan plan;
    st = make_plan(FR_OP_LAYERNORM, rows, cols, FR_BF16, num_cus, 0, 0, v16, g_forced_form,
                   override_for(FR_OP_LAYERNORM, rows, cols, FR_BF16), &plan);
    if (st != FR_OK) return st;
    LayerNormArgs args{(const uint16_t*)x, (const uint16_t*)gamma, (const uint16_t*)beta, (uint16_t*)y,
                       (int)rows, (int)cols, x_rs, y_rs, eps, mean, rstd};
    (void)hipGetLastError();
    return finish_launch(launch_layernorm(plan, args, (hipStream_t)stream));
}

uint64_t fr_layernorm_rows_backward_workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    if (dtype != FR_BF16 || check_sizes(rows, cols) != FR_OK || rows == 0 || cols == 0) return 0;
    // enough for every form the call may take (split rows with 16-byte
    // accesses, persistent rows otherwise or when dx aliases an input); it
    // does not depend on alignment or the device
    const fr_plan* ov = override_for(FR_OP_LAYERNORM_BWD, rows, cols, FR_BF16);
    uint64_t need = 0;
    for (int form : {FR_FORM_AUTO, FR_FORM_PER, FR_FORM_SPLIT}) {
        fr_plan plan;
        if (make_plan(FR_OP_LAYERNORM_BWD, rows, cols, FR_BF16, 256, 0, UINT64_MAX, 1, form, ov, &plan) == FR_OK &&
            plan.ws_bytes > need)
            need = plan.ws_bytes;
    }
    return need;
}

int fr_layernorm_rows_backward_workspace_init(void* ws, uint64_t ws_bytes, void* stream) {
    if (!ws) return FR_E_NULL;
    if (!aligned(ws, 16)) return FR_E_ALIGN;
    if (ws_bytes < 64) return FR_E_WORKSPACE;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_layernorm_bwd_ws_init(ws, ws_bytes, (hipStream_t)stream));
}

int fr_layernorm_rows_backward(const void* x, const void* dy, const void* gamma, const float* mean,
                               const float* rstd, void* dx, float* dgamma, float* dbeta, int64_t rows, int64_t cols,
                               int64_t x_rs, int64_t x_cs, int64_t dy_rs, int64_t dy_cs, int64_t dx_rs,
                               int64_t dx_cs, void* ws, uint64_t ws_bytes, int dtype, void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_BF16) return FR_E_DTYPE;
    if (cols < 1) return FR_E_SIZE;
    if (rows == 0 && !dgamma && !dbeta) return FR_OK;
    // no rows with dgamma / dbeta: only the column sums run (empty sums: 0)
    if (rows > 0) {
        if ((st = check_matrix(x, rows, cols, x_rs, x_cs, 2)) != FR_OK) return st;
        if ((st = check_matrix(dy, rows, cols, dy_rs, dy_cs, 2)) != FR_OK) return st;
        if ((st = check_matrix(dx, rows, cols, dx_rs, dx_cs, 2)) != FR_OK) return st;
        if ((dx == x && dx_rs != x_rs) || (dx == dy && dx_rs != dy_rs)) return FR_E_STRIDE;
        if (!mean || !rstd) return FR_E_NULL;
    }
    if (!aligned(gamma, 2) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(dgamma, 4) || !aligned(dbeta, 4) ||
        !aligned(ws, 16))
        return FR_E_ALIGN;
    const int v16 = cols % 8 == 0 && vec_ok(x, x_rs, 8) && vec_ok(dy, dy_rs, 8) && vec_ok(dx, dx_rs, 8) &&
                    vec_ok(gamma, 0, 8);
    // split rows read a partner's part of x and dy when its sums are late:
    // never while dx overwrites them
    const bool alias = rows > 0 && (dx == x || dx == dy);
    int forced = g_forced_form;
    if (alias && forced == FR_FORM_AUTO) forced = FR_FORM_PER;
    fr_plan plan;
    st = make_plan(FR_OP_LAYERNORM_BWD, rows, cols, FR_BF16, 256, 0, ws ? ws_bytes : 0, v16, forced,
                   override_for(FR_OP_LAYERNORM_BWD, rows, cols, FR_BF16), &plan);
    if (st != FR_OK) return st;
    if (alias && plan.form == FR_FORM_SPLIT) return FR_E_ARG;
    const bool dg = dgamma || dbeta;
    if ((dg || plan.form == FR_FORM_SPLIT) && plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes))
        return FR_E_WORKSPACE;
    // rows beyond 16384 columns with dgamma / dbeta need 16-byte accesses
    if (dg && !v16 && plan.threads * plan.vec > 1024 * 2) return FR_E_ALIGN;
    int num_cus = 0, clock_khz = 0;
    st = device_check(&num_cus, &clock_khz);
    if (st != FR_OK) return st;
    const int64_t wait_ticks = plan.wait_us > 0 ? (int64_t)plan.wait_us * clock_khz / 1000 : (plan.wait_us < 0 ? -1 : 0);
    LayerNormBwdArgs args{(const uint16_t*)x, (const uint16_t*)dy, (const uint16_t*)gamma, mean, rstd,
                          (uint16_t*)dx, dgamma, dbeta, (float*)ws, (int)rows, (int)cols, x_rs, dy_rs, dx_rs,
                          wait_ticks};
    (void)hipGetLastError();
    return finish_launch(launch_layernorm_bwd(plan, args, (hipStream_t)stream));
}

int fr_softmax_rows_backward(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols, int64_t y_rs,
                             int64_t y_cs, int64_t dy_rs, int64_t dy_cs, int64_t dx_rs, int64_t dx_cs,
                             const int32_t* lengths, int dtype, void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (rows == 0 || cols == 0) return FR_OK;  // nothing to read or write
    if ((st = check_matrix(y, rows, cols, y_rs, y_cs, 4)) != FR_OK) return st;
    if ((st = check_matrix(dy, rows, cols, dy_rs, dy_cs, 4)) != FR_OK) return st;
    if ((st = check_matrix(dx, rows, cols, dx_rs, dx_cs, 4)) != FR_OK) return st;
    if ((dx == y && dx_rs != y_rs) || (dx == dy && dx_rs != dy_rs)) return FR_E_STRIDE;
    if (!aligned(lengths, 4)) return FR_E_ALIGN;
    int num_cus = 0;
    st = device_check(&num_cus);
    if (st != FR_OK) return st;
    const int v16 = vec_ok(y, y_rs, 4) && vec_ok(dy, dy_rs, 4) && vec_ok(dx, dx_rs, 4);
    fr_plan plan;
    st = make_plan(FR_OP_SOFTMAX_BWD, rows, cols, FR_F32, num_cus, lengths != nullptr, 0, v16, g_forced_form,
                   override_for(FR_OP_SOFTMAX_BWD, rows, cols, FR_F32), &plan);
    if (st != FR_OK) return st;
    SoftmaxBwdArgs args{(const float*)y, (const float*)dy, (float*)dx, (int)rows, (int)cols, y_rs, dy_rs, dx_rs,
                        lengths};
    (void)hipGetLastError();
    return finish_launch(launch_softmax_bwd(plan, args, (hipStream_t)stream));
}

uint64_t fr_attn_decode_workspace_bytes(int64_t batch, int64_t heads_q, int64_t seq, int64_t dim) {
    if (batch < 0 || heads_q < 0 || seq < 0 || seq >= kMaxCols || (dim != 64 && dim != 128)) return 0;
    return attn_ws_bytes(batch, heads_q, seq, dim);
}

int fr_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch, int64_t heads_q,
                   int64_t heads_kv, int64_t seq, int64_t dim, const int32_t* lengths, float scale, void* ws,
                   uint64_t ws_bytes, int dtype, void* stream) {
    if (dtype != FR_F32 && dtype != FR_BF16) return FR_E_DTYPE;
    if (batch < 0 || heads_q < 0 || heads_kv < 0 || seq < 0) return FR_E_SIZE;
    if (dim != 64 && dim != 128) return FR_E_SIZE;
    if (batch > 65535 || heads_kv > 65535 || seq >= kMaxCols || batch * heads_q >= kMaxRows) return FR_E_SIZE;
    if (seq * dim * (dtype == FR_BF16 ? 2 : 4) >= (int64_t(1) << 31)) return FR_E_SIZE;  // 32-bit offsets per head
    if (batch == 0 || heads_q == 0) return FR_OK;
    if (heads_kv == 0 || heads_q % heads_kv) return FR_E_ARG;
    const int64_t G = heads_q / heads_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return FR_E_ARG;
    if (!isfinite(scale)) return FR_E_ARG;
    if (!q || !o || (seq > 0 && (!k || !v))) return FR_E_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(lengths, 4) || !aligned(ws, 16))
        return FR_E_ALIGN;
    const uint64_t need = attn_ws_bytes(batch, heads_q, seq, dim);
    if (need > 0 && (!ws || ws_bytes < need)) return FR_E_WORKSPACE;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    AttnArgs args{q, k, v, o, lse, (int)batch, (int)heads_q, (int)heads_kv, (int)seq, (int)dim, lengths, scale,
                  static_cast<float*>(ws), dtype == FR_BF16};
    (void)hipGetLastError();
    return finish_launch(launch_attn_decode(args, (hipStream_t)stream));
}

int fr_attn_block(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch, int64_t heads_q,
                  int64_t heads_kv, int64_t seq_q, int64_t seq_kv, int64_t dim, int causal, float scale, int dtype,
                  void* stream) {
    if (dtype != FR_BF16) return FR_E_DTYPE;
    if (batch < 0 || heads_q < 0 || heads_kv < 0 || seq_q < 0 || seq_kv < 0) return FR_E_SIZE;
    if (dim != 64 && dim != 128) return FR_E_SIZE;
    if (batch > 65535 || heads_q > 65535 || seq_q >= kMaxCols || seq_kv >= kMaxCols) return FR_E_SIZE;
    if (seq_kv * dim * 2 >= (int64_t(1) << 31)) return FR_E_SIZE;  // one head's keys: 32-bit byte offsets
    if (batch == 0 || heads_q == 0 || seq_q == 0) return FR_OK;
    // one workgroup per (block of kAttnBlockRows query rows, head, batch): a 1-D grid
    if ((seq_q + kAttnBlockRows - 1) / kAttnBlockRows * heads_q * batch >= (int64_t(1) << 31)) return FR_E_SIZE;
    if (heads_kv == 0 || heads_q % heads_kv) return FR_E_ARG;
    if (!isfinite(scale) || !(scale > 0.0f)) return FR_E_ARG;
    if (!q || !o || !lse || (seq_kv > 0 && (!k || !v))) return FR_E_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FR_E_ALIGN;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    AttnBlockArgs args{q, k, v, o, lse, (int)batch, (int)heads_q, (int)heads_kv, (int)seq_q, (int)seq_kv, (int)dim,
                       causal != 0, scale};
    (void)hipGetLastError();
    return finish_launch(launch_attn_block(args, (hipStream_t)stream));
}

int fr_stream_copy(const void* x, void* y, int64_t nbytes, void* stream) {
    if (nbytes < 0 || nbytes % 16) return FR_E_SIZE;
    if (nbytes == 0) return FR_OK;
    if (!x || !y) return FR_E_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return FR_E_ALIGN;
    const uintptr_t a = (uintptr_t)x, b = (uintptr_t)y;
    if (a < b + (uintptr_t)nbytes && b < a + (uintptr_t)nbytes) return FR_E_ARG;  // overlap
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_stream_copy(x, y, nbytes / 16, (hipStream_t)stream));
}

int fr_stream_read(const void* x, int64_t nbytes, uint32_t* sink, void* stream) {
    static_assert(FR_STREAM_SINK_WORDS == kStreamGrid, "one sink word per workgroup");
    if (nbytes < 0 || nbytes % 16) return FR_E_SIZE;
    if (!sink || (nbytes > 0 && !x)) return FR_E_NULL;
    if (!aligned(x, 16) || !aligned(sink, 4)) return FR_E_ALIGN;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_stream_read(x, nbytes / 16, sink, (hipStream_t)stream));
}

int fr_stream_write(void* y, int64_t nbytes, uint32_t value, void* stream) {
    if (nbytes < 0 || nbytes % 16) return FR_E_SIZE;
    if (nbytes == 0) return FR_OK;
    if (!y) return FR_E_NULL;
    if (!aligned(y, 16)) return FR_E_ALIGN;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_stream_write(y, nbytes / 16, value, (hipStream_t)stream));
}

int fr_stream_empty(void* stream) {
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_empty((hipStream_t)stream));
}

int fr_device_clock(uint64_t* out, int slot, void* stream) {
    if (!out) return FR_E_NULL;
    if (slot < 0) return FR_E_ARG;
    if (!aligned(out, 8)) return FR_E_ALIGN;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_device_clock(out, slot, (hipStream_t)stream));
}

int fr_pointer_chase(const uint32_t* chain, int64_t n, int64_t steps, uint32_t start, uint64_t* out, void* stream) {
    if (!chain || !out) return FR_E_NULL;
    if (n < 1 || n > (int64_t(1) << 32) || steps < 0) return FR_E_SIZE;
    if (!aligned(chain, 4) || !aligned(out, 8)) return FR_E_ALIGN;
    int num_cus = 0;
    const int st = device_check(&num_cus);
    if (st != FR_OK) return st;
    (void)hipGetLastError();
    return finish_launch(launch_pointer_chase(chain, n, steps, start, out, (hipStream_t)stream));
}

int fr_device_clock_khz(int* khz) {
    if (!khz) return FR_E_NULL;
    int num_cus = 0, clock_khz = 0;
    const int st = device_check(&num_cus, &clock_khz);
    if (st != FR_OK) return st;
    *khz = clock_khz;
    return FR_OK;
}

int fr_add_2d(const void* a, int64_t a_rs, int64_t a_cs, const void* b, int64_t b_rs, int64_t b_cs, void* out,
              int64_t out_rs, int64_t rows, int64_t cols, int dtype, void* stream) {
    int st = check_sizes(rows, cols);
    if (st != FR_OK) return st;
    if (dtype != FR_F32) return FR_E_DTYPE;
    if (rows == 0 || cols == 0) return FR_OK;
    if (!a || !b || !out) return FR_E_NULL;
    const int la = add2d_layout(rows, cols, a_rs, a_cs), lb = add2d_layout(rows, cols, b_rs, b_cs);
    if (la < 0 || lb < 0 || out_rs < 0 || (rows > 1 && out_rs < cols)) return FR_E_STRIDE;
    if (!aligned(a, 4) || !aligned(b, 4) || !aligned(out, 4)) return FR_E_ALIGN;
    // in place only over an operand of the output's own layout
    if ((out == a && (la != 0 || a_rs != out_rs)) || (out == b && (lb != 0 || b_rs != out_rs))) return FR_E_ARG;
    int num_cus = 0;
    st = device_check(&num_cus);
    if (st != FR_OK) return st;
    // 16-byte vectors along each operand's contiguous direction
    const int v16 = aligned(a, 16) && aligned(b, 16) && aligned(out, 16) && (la ? a_cs : a_rs) % 4 == 0 &&
                    (lb ? b_cs : b_rs) % 4 == 0 && out_rs % 4 == 0;
    fr_plan plan;
    st = make_pointwise_plan(FR_OP_ADD_2D, rows, cols, FR_F32, num_cus, v16, g_forced_form,
                             override_for(FR_OP_ADD_2D, rows, cols, FR_F32), &plan);
    if (st != FR_OK) return st;
    Add2dArgs args{(const float*)a, (const float*)b, (float*)out, rows, cols, a_rs, a_cs, b_rs, b_cs, out_rs,
                   la == 1, lb == 1};
    (void)hipGetLastError();
    return finish_launch(launch_add_2d(plan, args, (hipStream_t)stream));
}

int fr_gelu_backward(const void* dy, int64_t dy_stride, const void* h, void* dx, int64_t n, int dtype,
                     void* stream) {
    if (dtype != FR_F32 && dtype != FR_BF16) return FR_E_DTYPE;
    if (n < 0 || n >= (int64_t(1) << 40)) return FR_E_SIZE;
    if (dy_stride != 0 && dy_stride != 1) return FR_E_STRIDE;
    if (n == 0) return FR_OK;
    if (!dy || !h || !dx) return FR_E_NULL;
    const size_t es = dtype == FR_F32 ? 4 : 2;
    if (!aligned(dy, es) || !aligned(h, es) || !aligned(dx, es)) return FR_E_ALIGN;
    int num_cus = 0;
    const int st0 = device_check(&num_cus);
    if (st0 != FR_OK) return st0;
    const int v16 = aligned(h, 16) && aligned(dx, 16) && (dy_stride == 0 || aligned(dy, 16));
    fr_plan plan;
    const int st = make_pointwise_plan(FR_OP_GELU_BWD, 1, n, dtype, num_cus, v16, g_forced_form,
                                       override_for(FR_OP_GELU_BWD, 1, n, dtype), &plan);
    if (st != FR_OK) return st;
    GeluBwdArgs args{dy, h, dx, n, dy_stride == 0, dtype == FR_BF16};
    (void)hipGetLastError();
    return finish_launch(launch_gelu_bwd(plan, args, (hipStream_t)stream));
}

}  // extern "C"
