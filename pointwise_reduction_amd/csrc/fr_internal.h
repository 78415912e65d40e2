// fr_internal.h - what the host entry points hand to the kernel launchers.
// Arguments are validated and a plan is chosen before any of these runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fr.h"

namespace fr {

enum Prologue : int { kReluAdd = 0, kSquare = 1 };

// Row sums with a pointwise prologue: out[i] = post * sum_j f(a[i,j], b[i,j]).
struct SumArgs {
    int prologue;      // kReluAdd (2 * relu(a + b)) or kSquare (a * a)
    const float* a;
    const float* b;    // kReluAdd only
    float* out;
    int rows, cols;
    int64_t a_rs, b_rs, out_s;
    float* ws;         // split form: rows x splits partial sums
};

struct SoftmaxArgs {
    const float* x;
    float* y;
    int rows, cols;
    int64_t x_rs, y_rs;
    const int32_t* lengths;  // nullable
    int32_t* argmax;         // nullable
    void* ws;                // split form: header + rows x splits partial states
    int64_t wait_ticks;      // single-pass split: wall-clock ticks a workgroup waits for a row's partials
};

struct SoftmaxBwdArgs {
    const float* y;
    const float* dy;
    float* dx;
    int rows, cols;
    int64_t y_rs, dy_rs, dx_rs;
    const int32_t* lengths;  // nullable
};

struct LayerNormArgs {
    const uint16_t* x;
    const uint16_t* gamma;  // nullable
    const uint16_t* beta;   // nullable
    uint16_t* y;
    int rows, cols;
    int64_t x_rs, y_rs;
    float eps;
    float* mean;  // nullable: per-row mean, as the backward pass reads it
    float* rstd;  // nullable: per-row 1 / sqrt(var + eps)
};

// Partial state of one chunk of a split softmax row: the (m, d) pair of the
// chunk and the first index of its maximum.
// Workspace of the split softmax: a header of kSplitWsHeader bytes (the
// single pass's call epoch, initialization mark and a count of the partials
// it computed for another workgroup), one 32-bit flag per workgroup of the
// single pass (kOnePassMaxGrid of them), then one 16-byte slot per chunk
// from kSplitWsSlots on: two 64-bit words (tag, m) and (tag, d).
constexpr int kSplitWsHeader = 64;
constexpr int kOnePassMaxGrid = 4096;
constexpr int kSplitWsSlots = kSplitWsHeader + 4 * kOnePassMaxGrid;
// The single pass keeps per-row chunk counts in LDS: at most this many rows.
constexpr int kOnePassMaxRows = 2048;

struct alignas(16) SoftmaxPartial {
    float m, d;
    int32_t idx, pad;
};

hipError_t launch_sum(const fr_plan& p, const SumArgs& a, hipStream_t s);
hipError_t launch_softmax(const fr_plan& p, const SoftmaxArgs& a, hipStream_t s);
hipError_t launch_softmax_ws_init(void* ws, uint64_t ws_bytes, hipStream_t s);
hipError_t launch_layernorm(const fr_plan& p, const LayerNormArgs& a, hipStream_t s);
// LayerNorm backward from saved statistics; ws holds the dgamma / dbeta
// partials [2][grid][ln_bwd_ldw(cols)] fp32 when either is requested.
struct LayerNormBwdArgs {
    const uint16_t* x;
    const uint16_t* dy;
    const uint16_t* gamma;  // nullable: 1
    const float* mean;
    const float* rstd;
    uint16_t* dx;
    float* dgamma;  // nullable
    float* dbeta;   // nullable
    float* ws;
    int rows, cols;
    int64_t x_rs, dy_rs, dx_rs;
    int64_t wait_ticks;  // split rows: wall-clock ticks a member waits for its partners' sums (< 0: none)
};
inline int64_t ln_bwd_ldw(int64_t cols) { return (cols + 7) / 8 * 8; }
// Split-row LayerNorm backward (a team of workgroups per row): workspace =
// a kLnTeamHeader-byte header (word 0: partner sums recomputed after the
// wait, cumulative; word 2: the call epoch; words 4-5: the initialization
// mark; from word kLnTeamHeaderFlags one flag per workgroup, at most
// kLnTeamMaxGrid), 16 bytes per (row, part) exchange slot, padded to 256
// bytes, then the dgamma / dbeta partials [2][teams][ln_bwd_ldw(cols)] fp32.
constexpr int kLnTeamMaxGrid = 256;
constexpr int kLnTeamHeaderFlags = 16;
constexpr int kLnTeamHeader = 4 * kLnTeamHeaderFlags + 4 * kLnTeamMaxGrid;
constexpr int kLnTeamPartCols = 8192;  // columns per member: one 16-byte vector per lane of 1024
inline int64_t ln_team_slots_bytes(int64_t rows, int64_t parts) { return (rows * parts * 16 + 255) / 256 * 256; }
hipError_t launch_layernorm_bwd(const fr_plan& p, const LayerNormBwdArgs& a, hipStream_t s);
hipError_t launch_layernorm_bwd_ws_init(void* ws, uint64_t ws_bytes, hipStream_t s);
hipError_t launch_softmax_bwd(const fr_plan& p, const SoftmaxBwdArgs& a, hipStream_t s);
// Pointwise: 2-D add (a_t / b_t: the operand is column-major, a transposed
// view with unit row stride) and GELU backward.
struct Add2dArgs {
    const float* a;
    const float* b;
    float* out;
    int64_t rows, cols;
    int64_t a_rs, a_cs, b_rs, b_cs, out_rs;
    bool a_t, b_t;
};
struct GeluBwdArgs {
    const void* dy;
    const void* h;
    void* dx;
    int64_t n;
    bool bcast;  // dy[0] for every element
    bool bf16;
};
hipError_t launch_add_2d(const fr_plan& p, const Add2dArgs& a, hipStream_t s);
hipError_t launch_gelu_bwd(const fr_plan& p, const GeluBwdArgs& a, hipStream_t s);

// Decode attention: keys are split into chunks of kAttnChunk per workgroup;
// the workspace holds one (m, l, pad, pad, a[dim]) fp32 slot per (batch,
// query head, chunk).
constexpr int kAttnChunk = 256;
inline int64_t attn_chunks(int64_t seq) { return (seq + kAttnChunk - 1) / kAttnChunk; }
inline uint64_t attn_ws_bytes(int64_t batch, int64_t heads_q, int64_t seq, int64_t dim) {
    return (uint64_t)(batch * heads_q * attn_chunks(seq) * (dim + 4) * 4);
}
struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;              // nullable
    int batch, heads_q, heads_kv, seq, dim;
    const int32_t* lengths;  // nullable
    float scale;
    float* ws;
    bool bf16;
};
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s);
// Tiled attention over blocks of kAttnBlockRows query rows (bf16).
constexpr int kAttnBlockRows = 256;
struct AttnBlockArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int batch, heads_q, heads_kv, seq_q, seq_kv, dim;
    bool causal;
    float scale;
};
hipError_t launch_attn_block(const AttnBlockArgs& a, hipStream_t s);

// Streaming reference kernels: at most kStreamGrid workgroups of 256 threads,
// 4 vectors of 16 bytes per thread per step.
constexpr int kStreamGrid = 1024;
hipError_t launch_stream_copy(const void* x, void* y, int64_t nvec, hipStream_t s);
hipError_t launch_stream_read(const void* x, int64_t nvec, uint32_t* sink, hipStream_t s);
hipError_t launch_stream_write(void* y, int64_t nvec, uint32_t value, hipStream_t s);
hipError_t launch_empty(hipStream_t s);
hipError_t launch_device_clock(uint64_t* out, int slot, hipStream_t s);
hipError_t launch_pointer_chase(const uint32_t* chain, int64_t n, int64_t steps, uint32_t start, uint64_t* out,
                                hipStream_t s);

// Planner (host only, no HIP calls).
int make_plan(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int has_lengths, uint64_t ws_bytes,
              int aligned16, int forced_form, const fr_plan* override_plan, fr_plan* plan);
// Pointwise operations: FR_OP_ADD_2D over rows x cols, FR_OP_GELU_BWD over
// n = rows * cols elements.
int make_pointwise_plan(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int aligned16, int forced_form,
                        const fr_plan* override_plan, fr_plan* plan);

}  // namespace fr
