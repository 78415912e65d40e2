/*
 * fr.h - C ABI of libfr, fused pointwise-prologue + row-reduction kernels
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are the non-template reduction nodes of a tensor compiler,
 * as described in "Stax (4): GPU Codegen and Dynamic Shapes" (TensorPlay
 * blog), section 9.4 (three reduction forms), 9.5 (multi-reduction fusion and
 * the online (m, d) merge), 9.7 (the wrapper that checks sizes and strides,
 * hands workspaces to the kernels and launches them in stream order), and
 * 10.3 (sizes are runtime values, so masks stay).
 *
 * Conventions shared by every entry point:
 *  - Memory. Every data pointer is a device pointer (HBM) owned by the
 *    caller. The library never allocates or frees memory; where a split
 *    reduction needs scratch, the caller passes a workspace sized by the
 *    matching *_workspace_bytes query.
 *  - Layout. Row-major: element (i, j) of a matrix lives at
 *    base + i * row_stride + j * col_stride, strides counted in elements.
 *    The column stride must be 1 and the row stride >= cols; other strides
 *    are an error (FR_E_STRIDE), not a slow path.
 *  - Streams. `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream). Work is enqueued asynchronously; the library never
 *    synchronizes. Kernels of one call run in stream order.
 *  - Errors. Invalid arguments return a negative status before any HIP call
 *    and launch nothing. FR_E_DEVICE means the current device is not gfx950
 *    or could not be queried; FR_E_LAUNCH means a kernel launch failed.
 *  - Sizes. rows and cols are counted in elements; 0 <= rows < 2^31 and
 *    0 <= cols < 2^30 (in-row offsets are 32-bit, row offsets 64-bit);
 *    larger sizes return FR_E_SIZE.
 *  - Determinism. For a given device model, library build and arguments,
 *    results are bit-identical from run to run (fixed partitions, fixed
 *    reduction trees, no floating-point atomics).
 *  - Aliasing. y may equal x (in place, same row stride); any other overlap
 *    between inputs and outputs is undefined.
 */
#ifndef FR_H
#define FR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
#define FR_OK 0
#define FR_E_NULL (-1)      /* a required pointer is NULL */
#define FR_E_SIZE (-2)      /* a size is negative or too large */
#define FR_E_STRIDE (-3)    /* column stride != 1, or row stride < cols */
#define FR_E_DTYPE (-4)     /* dtype not supported by this entry point */
#define FR_E_ALIGN (-5)     /* pointer not aligned to its element (or workspace to 16 B) */
#define FR_E_WORKSPACE (-6) /* workspace required but missing, or too small */
#define FR_E_ARG (-7)       /* another argument is invalid (eps, form, plan) */
#define FR_E_DEVICE (-8)    /* no usable gfx950 device */
#define FR_E_LAUNCH (-9)    /* a kernel launch failed */

/* ------------------------------------------------------------ element types */
#define FR_F32 0  /* IEEE binary32 */
#define FR_BF16 1 /* bfloat16 (upper half of a binary32), stored as uint16 */

/* ------------------------------------------------------------ reduction forms
 * "Stax (4)", 9.4: persistent (the whole row in registers, one pass), looped
 * (the row streamed in chunks with a register accumulator), split (too few
 * outputs: per-chunk partials in a workspace, then a finishing pass). */
#define FR_FORM_AUTO 0
#define FR_FORM_PER 1
#define FR_FORM_RED 2
#define FR_FORM_SPLIT 3
/* Pointwise operations have no reduction dimension and one form. */
#define FR_FORM_POINTWISE 4

/* ------------------------------------------------------------ operations */
#define FR_OP_SUM_RELU_ADD 1
#define FR_OP_SOFTMAX 2
#define FR_OP_LAYERNORM 3
#define FR_OP_SUMSQ 4
#define FR_OP_SOFTMAX_BWD 5
#define FR_OP_ADD_2D 6
#define FR_OP_GELU_BWD 7
#define FR_OP_LAYERNORM_BWD 8

/* Launch plan chosen for one call: the reduction form and its launch
 * configuration ("Stax (4)", 9.6: block sizes and warp counts are launch
 * parameters; the grid follows from them). */
typedef struct fr_plan {
    int32_t op;           /* FR_OP_* */
    int32_t form;         /* FR_FORM_PER / _RED / _SPLIT */
    int32_t threads;      /* threads per workgroup (multiple of 64) */
    int32_t seg;          /* lanes that share one row (persistent form) */
    int32_t vec;          /* 16-byte vectors per lane: per pass (PER, SPLIT chunk) or per loop step (RED) */
    int32_t rows_per_wg;  /* rows handled by one workgroup */
    int32_t splits;       /* chunks per row (SPLIT; LayerNorm backward: workgroups per row), else 1 */
    int32_t chunk;        /* elements per chunk (SPLIT; LayerNorm backward: columns per workgroup), else 0 */
    int32_t vec16;        /* 1: 16-byte vector accesses; 0: element accesses */
    int32_t occupancy;    /* minimum waves per SIMD requested from the compiler (0: none) */
    int32_t passes;       /* reads of the input (split softmax: 1 = chunks kept in registers while the
                             row's partials are exchanged in one kernel, 2 = partial + finishing kernels) */
    int32_t wait_us;      /* single-pass split softmax and split LayerNorm backward: microseconds a
                             workgroup waits for the other partials of its row before computing the
                             missing ones itself from the inputs (same bits); in an override 0 means
                             the default, and < 0 makes every workgroup compute all partials of its
                             row itself (a test of that path) */
    int64_t grid;         /* workgroups of the main kernel */
    int64_t grid2;        /* workgroups of the finishing kernel (0: none) */
    uint64_t ws_bytes;    /* workspace bytes this plan uses */
} fr_plan;

/* Human-readable name of a status code (static string). */
const char* fr_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fr_version(void);

/* Compute the plan a call with these arguments would use, without touching
 * the GPU (no HIP call). num_cus is the compute-unit count of the target
 * device (256 on MI355X). has_lengths: ragged softmax. ws_bytes: workspace
 * the caller would pass (0 = none). aligned16: all row bases and strides
 * allow 16-byte accesses. Honours fr_force_form. Returns FR_OK or an error
 * status for arguments the entry point itself would reject. */
int fr_plan_query(int op, int64_t rows, int64_t cols, int dtype, int num_cus, int has_lengths,
                  uint64_t ws_bytes, int aligned16, fr_plan* plan);

/* Test and tuning hook: force a reduction form for every later call in this
 * process (FR_FORM_AUTO restores the automatic choice). A call whose shape or
 * workspace cannot use the forced form returns FR_E_ARG. Not thread-safe;
 * returns the previous setting. */
int fr_force_form(int form);

/* Tuning hook ("Stax (4)", 9.6, Algorithm 9.1: time candidate launch
 * configurations and keep the fastest). Every later call of operation `op`
 * uses the form and launch knobs of `plan` (form, threads, seg, vec,
 * rows_per_wg, chunk, occupancy, passes, wait_us); grid, splits and workspace size are
 * recomputed for each call's shape. A candidate that cannot serve a shape,
 * or has no compiled kernel, makes that call return FR_E_ARG; a split
 * candidate needing more workspace than given returns FR_E_WORKSPACE.
 * plan = NULL clears the override. Not thread-safe. */
int fr_tune_override(int op, const fr_plan* plan);

/* Recorded selections ("Stax (4)", 9.6, Algorithm 9.1: measure once, keep
 * the winner): later calls of `op` with exactly these rows, cols and dtype
 * use the knobs of `plan` (as fr_tune_override does, but for this shape
 * only; a process-wide override still wins). For FR_OP_SUMSQ full
 * reductions and FR_OP_GELU_BWD, rows = 1 and cols = n. plan = NULL removes
 * the record. A record that cannot serve a call makes it return FR_E_ARG, or
 * FR_E_WORKSPACE if its split needs more workspace than the call passes (the
 * tuner only records configurations measured with the workspace the query
 * functions report). fr_tune_lookup returns FR_E_ARG when there is no
 * record. Thread-safe. */
int fr_tune_record(int op, int64_t rows, int64_t cols, int dtype, const fr_plan* plan);
int fr_tune_lookup(int op, int64_t rows, int64_t cols, int dtype, fr_plan* plan);
void fr_tune_clear(void);

/* ------------------------------------------------------------ Example 1.1
 * out[i] = sum_j 2 * relu(a[i,j] + b[i,j])   ("Stax (4)", 9.2, Listing 9.1,
 * the kernel of Example 1.1; 10.2, Example 10.1 with a runtime row count).
 * The add is an fp32 add; relu propagates NaN (a NaN anywhere in a row makes
 * out[i] NaN). a, b: fp32 [rows, cols] with row strides a_rs, b_rs and column
 * strides a_cs, b_cs (must be 1); out: fp32 [rows] with element stride
 * out_s >= 1. cols = 0 writes 0 (the empty sum). ws/ws_bytes: optional
 * workspace (NULL/0 allowed) enabling the split form for few, long rows; size
 * it with fr_sum_workspace_bytes. dtype must be FR_F32. */
int fr_sum_relu_add(const void* a, const void* b, void* out, int64_t rows, int64_t cols, int64_t a_rs,
                    int64_t a_cs, int64_t b_rs, int64_t b_cs, int64_t out_s, void* ws, uint64_t ws_bytes,
                    int dtype, void* stream);

/* Workspace bytes that make the split form available to fr_sum_relu_add and
 * fr_sumsq_rows for this shape (0 for an empty shape). With it the library
 * splits rows only where there are too few rows to fill the device. */
uint64_t fr_sum_workspace_bytes(int64_t rows, int64_t cols, int dtype);

/* ------------------------------------------------------------ row softmax
 * y[i,j] = e^(x[i,j] - m_i) / sum_k e^(x[i,k] - m_i), m_i = max_k x[i,k]
 * ("Stax (4)", 9.5, the softmax definition and Listing 9.5), fused into one
 * kernel per form: the max and the sum of exponentials are two reductions
 * with different identities (-inf and 0), and long rows merge them with the
 * online (m, d) rescaling (9.5, the monoid and Proposition 9.1; hello-gpu,
 * Chapter 12, 12.3).
 *  x, y:     fp32 [rows, cols]; strides as in the conventions (y may be x).
 *  lengths:  optional int32[rows] device array. Row i then covers
 *            j < len_i = clamp(lengths[i], 0, cols) only: elements at
 *            j >= len_i are neither read in x nor written in y. NULL: every
 *            row has length cols.
 *  argmax:   optional int32[rows] device output: the smallest j < len_i with
 *            x[i,j] equal to the row maximum (a NaN counts as the maximum),
 *            -1 for an empty row.
 *  ws:       optional workspace (16-byte aligned) of at least
 *            fr_softmax_rows_workspace_bytes(rows, cols, dtype) bytes. With
 *            it, rows too long for registers may be split across
 *            workgroups; without it they are streamed by one workgroup each.
 *            Initialize it once with fr_softmax_rows_workspace_init before
 *            its first use (and again after it has held anything else);
 *            every call leaves it initialized for the next, with no clearing
 *            between calls. An uninitialized workspace gives the same
 *            results, but the single-pass split then computes every partner
 *            partial itself (slower). Word 0 (uint32) counts, since the
 *            initialization, the chunk partials the single-pass split
 *            computed a second time because their owner had not published
 *            them within plan.wait_us (a diagnostic: the results are the
 *            same either way). Calls that overlap in time on one workspace
 *            race on it; give concurrent streams their own.
 *  In place: when y shares memory with x, a split takes its two-kernel form
 *  (the single pass may read a partner's chunk of x after that partner has
 *  written y there); a tuning override that forces the single pass on such
 *  a call returns FR_E_ARG.
 * A NaN in a row makes that row's outputs NaN. dtype must be FR_F32. */
uint64_t fr_softmax_rows_workspace_bytes(int64_t rows, int64_t cols, int dtype);
/* Initialize a split-softmax workspace of ws_bytes bytes (enqueued on stream;
 * a fill kernel, no host synchronization, capturable in a graph): the slots
 * are marked empty and the single pass's call counter starts over. Once
 * initialized, a workspace stays usable for any shape it is large enough
 * for. FR_E_NULL / FR_E_ALIGN (16 bytes) / FR_E_WORKSPACE (< 64 bytes). The
 * single pass counts calls per workspace with a 31-bit counter: after
 * 2^31 - 1 calls it stops trusting the slots (same results, slower) until
 * the workspace is initialized again. */
int fr_softmax_rows_workspace_init(void* ws, uint64_t ws_bytes, void* stream);
int fr_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t x_rs, int64_t x_cs, int64_t y_rs,
                    int64_t y_cs, const int32_t* lengths, int32_t* argmax, void* ws, uint64_t ws_bytes, int dtype,
                    void* stream);

/* ------------------------------------------------------------ row softmax, backward
 * dx[i,j] = y[i,j] * (dy[i,j] - sum_k dy[i,k] y[i,k]): the gradient of the
 * row softmax of "Stax (4)", 9.5 with respect to its input, given its output
 * y and the upstream gradient dy (the derivative of that definition; the
 * pages define the forward pass). One fused row reduction (the dot product
 * of dy and y) followed by the pointwise epilogue, in the persistent or the
 * looped form.
 *  y, dy, dx: fp32 [rows, cols]; strides as in the conventions; dx may be
 *             y or dy (same row stride).
 *  lengths:   optional int32[rows] as in fr_softmax_rows: row i covers
 *             j < len_i only; nothing beyond is read or written.
 * dtype must be FR_F32. */
int fr_softmax_rows_backward(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols, int64_t y_rs,
                             int64_t y_cs, int64_t dy_rs, int64_t dy_cs, int64_t dx_rs, int64_t dx_cs,
                             const int32_t* lengths, int dtype, void* stream);

/* ------------------------------------------------------------ pointwise: 2-D add
 * out[i,j] = a[i*a_rs + j*a_cs] + b[i*b_rs + j*b_cs] for i < rows, j < cols
 * ("Stax (4)", 9.3, Listing 9.2: Example 6.1, x.t() + y, where one operand is
 * contiguous along the output's columns and the other along its rows). Each
 * operand is either row-major (a_cs = 1, a_rs >= cols) or column-major, i.e.
 * a transposed view (a_rs = 1, a_cs >= rows); any other layout returns
 * FR_E_STRIDE. The output is row-major (unit inner stride, out_rs >= cols).
 * Each element is the correctly rounded fp32 sum. The kernel tiles the output
 * in two dimensions (fr_plan: rows_per_wg x chunk elements per workgroup) and
 * passes transposed operands through LDS, so every access coalesces.
 *  a, b, out: fp32 device pointers, 4-byte aligned; 16-byte alignment of the
 *             bases and strides enables 16-byte accesses.
 *  out may be a or b only with the same (row-major) layout; other overlaps
 *  are undefined. rows < 2^31, cols < 2^30. dtype must be FR_F32. */
int fr_add_2d(const void* a, int64_t a_rs, int64_t a_cs, const void* b, int64_t b_rs, int64_t b_cs, void* out,
              int64_t out_rs, int64_t rows, int64_t cols, int dtype, void* stream);

/* ------------------------------------------------------------ pointwise: GELU backward
 * dx[i] = dy * GELU'(h[i]), GELU'(h) = Phi(h) + h phi(h), with Phi(h) =
 * (1 + erf(h / sqrt 2)) / 2 and phi(h) = exp(-h^2 / 2) / sqrt(2 pi)
 * ("Stax (4)", 9.3, Listing 9.3: the backward pointwise kernel of Example 5.1;
 * h is the pre-activation the forward pass saved).
 *  dy:        dy_stride 0: one element broadcast to every output (the
 *             upstream gradient of a scalar loss, as on the pages);
 *             dy_stride 1: one element per output. Other strides return
 *             FR_E_STRIDE.
 *  h, dx:     n contiguous elements; dx may be h or dy (elementwise, in
 *             place). n < 2^40.
 *  dtype:     FR_F32, or FR_BF16 for all three arrays (arithmetic in fp32,
 *             dx rounded to nearest even).
 * h = +-inf gives NaN (inf * 0 in h phi(h)), as the formula evaluates; NaN
 * propagates. */
int fr_gelu_backward(const void* dy, int64_t dy_stride, const void* h, void* dx, int64_t n, int dtype,
                     void* stream);

/* ------------------------------------------------------------ LayerNorm
 * y[i,j] = (x[i,j] - mu_i) * rstd_i * gamma[j] + beta[j],
 * mu_i = mean_j x[i,j], rstd_i = 1 / sqrt(var_i + eps), var_i the biased
 * (divide by cols) variance of row i. Mean and variance are fused reductions
 * over the row ("Stax (4)", 10.4 names variance reductions that also output
 * the mean; 9.8 states that half-precision arithmetic is done in fp32).
 *  x, y:        bf16 [rows, cols] (uint16 storage), fp32 arithmetic, y
 *               rounded to nearest even.
 *  gamma, beta: optional bf16 [cols] (NULL: 1 and 0).
 *  eps:         finite and >= 0 (else FR_E_ARG).
 * cols must be >= 1 (FR_E_SIZE otherwise). dtype must be FR_BF16. */
int fr_layernorm_rows(const void* x, const void* gamma, const void* beta, void* y, int64_t rows, int64_t cols,
                      int64_t x_rs, int64_t x_cs, int64_t y_rs, int64_t y_cs, float eps, int dtype, void* stream);

/* The same LayerNorm, also writing the row statistics a training step's
 * backward pass reads: mean[i] = mu_i and rstd[i] = 1 / sqrt(var_i + eps),
 * fp32 [rows] device arrays, 4-byte aligned, each nullable. */
int fr_layernorm_rows_stats(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                            int64_t rows, int64_t cols, int64_t x_rs, int64_t x_cs, int64_t y_rs, int64_t y_cs,
                            float eps, int dtype, void* stream);

/* ------------------------------------------------------------ LayerNorm, backward
 * The gradient of the LayerNorm above (the pages define the forward pass;
 * this is the derivative of that definition), from the statistics the
 * forward pass saved. With xh = (x[i,j] - mean[i]) * rstd[i] and
 * g = dy[i,j] * gamma[j]:
 *   dx[i,j]   = rstd[i] * (g - (1/cols) sum_k g_k - xh * (1/cols) sum_k g_k xh_k)
 *   dgamma[j] = sum_i dy[i,j] * xh,        dbeta[j] = sum_i dy[i,j].
 * Persistent form: one workgroup holds a row of x and dy in registers: two
 * fused row sums, then dx. Split form (rows of more than 8192 columns with
 * 16-byte accesses, at least 256 rows, a workspace given, dx not aliasing x
 * or dy): a team of up to 4 workgroups shares each row, each holding a part
 * of it; the parts' row sums are exchanged through the workspace and added
 * in part order, so every member uses the same bits. The dgamma / dbeta
 * sums over rows are accumulated per workgroup (persistent) or per team
 * (split) in registers, written as partial rows to the workspace and summed
 * in a fixed order by a second kernel (deterministic; no atomics).
 *  x, dy, dx:     bf16 [rows, cols], strides as in the conventions; dx may be
 *                 x or dy (same row stride). dx is rounded to nearest even.
 *  gamma:         bf16 [cols] or NULL (1).
 *  mean, rstd:    fp32 [rows], as fr_layernorm_rows_stats writes them.
 *  dgamma, dbeta: fp32 [cols] or NULL. When either is given, ws must hold
 *                 fr_layernorm_rows_backward_workspace_bytes(rows, cols)
 *                 bytes (16-byte aligned; FR_E_WORKSPACE otherwise); else ws
 *                 may be NULL (then the persistent form runs). That size
 *                 serves every form. The workspace's contents are the
 *                 library's during the call; calls that share one workspace
 *                 must not overlap. The split form exchanges the row sums
 *                 through slots tagged with a call epoch kept in the
 *                 workspace, so nothing is cleared between calls: initialize
 *                 the workspace once with
 *                 fr_layernorm_rows_backward_workspace_init before its first
 *                 use, and keep it for this entry point. A workspace never
 *                 initialized gives the same results, but every member
 *                 computes its partners' sums itself (slower). A call that
 *                 takes the persistent form with dgamma or dbeta writes its
 *                 partial rows over those slots and clears the
 *                 initialization: initialize again before the next split
 *                 call, or give the two forms separate workspaces.
 * 1 <= cols <= 32768 (FR_E_SIZE otherwise). With dgamma or dbeta and more
 * than 16384 columns, x, dy, dx and gamma must allow 16-byte accesses (bases
 * and row strides multiples of 8 elements, cols a multiple of 8; FR_E_ALIGN
 * otherwise). dtype must be FR_BF16. */
uint64_t fr_layernorm_rows_backward_workspace_bytes(int64_t rows, int64_t cols, int dtype);
/* Initialize a LayerNorm-backward workspace of ws_bytes bytes (enqueued on
 * stream; ws 16-byte aligned, FR_E_ALIGN otherwise; at least 64 bytes,
 * FR_E_WORKSPACE otherwise): zeros, call epoch 0 and the initialization
 * mark. Once per workspace; every later call leaves it initialized. */
int fr_layernorm_rows_backward_workspace_init(void* ws, uint64_t ws_bytes, void* stream);
int fr_layernorm_rows_backward(const void* x, const void* dy, const void* gamma, const float* mean,
                               const float* rstd, void* dx, float* dgamma, float* dbeta, int64_t rows, int64_t cols,
                               int64_t x_rs, int64_t x_cs, int64_t dy_rs, int64_t dy_cs, int64_t dx_rs,
                               int64_t dx_cs, void* ws, uint64_t ws_bytes, int dtype, void* stream);

/* ------------------------------------------------------------ sum of squares
 * fr_sumsq_rows: out[i] = sum_j x[i,j]^2 (fp32 squares, fp32 accumulation;
 * "Stax (4)", 9.4, Listing 9.4, the x * x prologue of Example 6.2, whose
 * [64, 16384] rows are split into partial sums plus a finishing pass). out:
 * fp32 [rows], contiguous. ws optional as for fr_sum_relu_add.
 * fr_sumsq_full: *out = sum_i x[i]^2 over a contiguous fp32 vector of n
 * elements, as per-workgroup partials in the workspace plus one finishing
 * workgroup, in a fixed order: repeated runs are bit-identical. A workspace
 * of fr_sumsq_full_workspace_bytes(n, dtype) bytes is required whenever that
 * query returns a non-zero size. n = 0 writes 0; n < 2^30. dtype must be
 * FR_F32. */
int fr_sumsq_rows(const void* x, void* out, int64_t rows, int64_t cols, int64_t x_rs, int64_t x_cs, void* ws,
                  uint64_t ws_bytes, int dtype, void* stream);
uint64_t fr_sumsq_full_workspace_bytes(int64_t n, int dtype);
int fr_sumsq_full(const void* x, int64_t n, void* out, void* ws, uint64_t ws_bytes, int dtype, void* stream);

/* ------------------------------------------------------------ decode attention
 * One query row per (batch b, query head h), keys and values of key-value
 * head g = h / (heads_q / heads_kv):
 *   s_j = scale * q[b,h,:] . k[b,g,j,:]                       (j < len_b)
 *   o[b,h,:] = sum_j e^{s_j - m} v[b,g,j,:] / sum_j e^{s_j - m},  m = max_j s_j
 *   lse[b,h] = m + log sum_j e^{s_j - m}
 * ("Stax (4)", 9.10: attention as a row softmax between two contractions;
 * the (m, l, a) triple and its merge let the keys be split across
 * workgroups, as the decode template does; hello-gpu, Chapter 12, 12.1).
 * The keys of a row are cut into chunks of 256; each chunk's triple goes to
 * the workspace and a second kernel merges them in chunk order, so results
 * are bit-identical run to run.
 *  q, o:    [batch, heads_q, dim], contiguous; k, v: [batch, heads_kv, seq,
 *           dim], contiguous; all of dtype FR_F32 or FR_BF16 (fp32
 *           arithmetic; a bf16 o is rounded to nearest even). 16-byte aligned.
 *  lengths: optional int32 [batch] device array, clamped to [0, seq] (NULL:
 *           seq). Keys and values at j >= len_b are never read.
 *  lse:     optional fp32 [batch, heads_q] device output.
 *  scale:   finite (the pages use 1 / sqrt(dim)).
 *  ws:      16-byte aligned workspace of at least
 *           fr_attn_decode_workspace_bytes(batch, heads_q, seq, dim) bytes
 *           (FR_E_WORKSPACE if smaller).
 * An empty key set gives o = 0 and lse = -inf; a NaN score makes the row's
 * o and lse NaN. dim must be 64 or 128 (FR_E_SIZE); heads_q must be 1, 2, 4
 * or 8 times heads_kv (FR_E_ARG); batch and heads_kv at most 65535, seq
 * below 2^30 (FR_E_SIZE). */
uint64_t fr_attn_decode_workspace_bytes(int64_t batch, int64_t heads_q, int64_t seq, int64_t dim);
int fr_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch, int64_t heads_q,
                   int64_t heads_kv, int64_t seq, int64_t dim, const int32_t* lengths, float scale, void* ws,
                   uint64_t ws_bytes, int dtype, void* stream);

/* ------------------------------------------------------------ attention over blocks of query rows
 * O = softmax(scale * Q K^T [+ causal mask]) V and LSE = m + log l per query
 * row, the tiled single-pass algorithm of "Stax (4)", 9.10 (Theorem 9.2,
 * Figure 9.2): one workgroup keeps a block of 256 query rows on chip and
 * scans K and V in blocks of 64 keys with the online (m, l, a) update; S
 * and P never reach memory. Both products run on the matrix cores in bf16
 * with fp32 accumulation; P enters the second product as bf16.
 *  q, o:   bf16 [batch, heads_q, seq_q, dim]; k, v: bf16 [batch, heads_kv,
 *          seq_kv, dim]; contiguous, 16-byte aligned. Query head h reads
 *          key-value head h / (heads_q / heads_kv).
 *  lse:    fp32 [batch, heads_q, seq_q] (natural log), 4-byte aligned.
 *  causal: query i sees key j only when i >= j (Listing 9.7's mask_mod);
 *          key blocks wholly above the diagonal are skipped.
 *  scale:  finite and > 0 (commonly 1 / sqrt(dim)); the row maxima are
 *          taken on the unscaled scores.
 * dim 64 or 128; heads_q a multiple of heads_kv; batch and heads_q <=
 * 65535; seq lengths < 2^30 and seq_kv * dim * 2 < 2^31 (one head's keys
 * addressed with 32-bit offsets). A row that sees no key (seq_kv = 0) gives
 * o = 0 and lse = -inf. dtype must be FR_BF16. */
int fr_attn_block(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch, int64_t heads_q,
                  int64_t heads_kv, int64_t seq_q, int64_t seq_kv, int64_t dim, int causal, float scale, int dtype,
                  void* stream);

/* ------------------------------------------------------------ streaming references
 * The practical ceiling of an HBM-bound step ("Stax (4)", 9.1: memory-bound
 * kernels are judged by the bandwidth they reach): the plainest kernels that
 * move the same bytes with the same access hints, timed by the same harness.
 * fr_stream_copy: y = x, nbytes bytes; x and y 16-byte aligned and not
 *   overlapping, nbytes a multiple of 16 (FR_E_ALIGN / FR_E_SIZE otherwise).
 * fr_stream_read: reads nbytes of x (same rules) and writes to sink[w], for
 *   each of its workgroups w, the XOR of all 32-bit words that workgroup
 *   read; the XOR of sink[0 .. FR_STREAM_SINK_WORDS) is then the XOR of all
 *   words of x (unused entries are not written: clear them first). sink:
 *   device array of FR_STREAM_SINK_WORDS uint32.
 * fr_stream_write: every 32-bit word of y (nbytes bytes, same rules as x
 *   above) = value; stores only, the write half of a step's traffic.
 * fr_stream_empty: enqueues a kernel of one workgroup that does nothing.
 *   Launched back to back, it times one kernel boundary (the end of one
 *   kernel to the start of the next), which every step that is one launch
 *   pays whatever bytes it moves. Errors: FR_E_DEVICE / FR_E_LAUNCH only. */
#define FR_STREAM_SINK_WORDS 1024
int fr_stream_copy(const void* x, void* y, int64_t nbytes, void* stream);
int fr_stream_read(const void* x, int64_t nbytes, uint32_t* sink, void* stream);
int fr_stream_write(void* y, int64_t nbytes, uint32_t value, void* stream);
int fr_stream_empty(void* stream);

/* ------------------------------------------------------------ sum of squares, no allocation
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): fr_sumsq_full with
 * the split's chunk partials in a device array the library owns, of
 * FR_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends), instead of
 * a caller workspace. Same kernels, so the same bits as fr_sumsq_full. x, n,
 * out, dtype and stream as there. It allocates nothing and calls no
 * allocating routine; its first call on a device looks up that device's
 * copy of the array. Every valid n fits the array (the split has at most
 * 2048 partials); a plan needing more returns FR_E_WORKSPACE. Calls on one
 * GPU share the array: calls that overlap in time on the same GPU race. */
#define FR_NOALLOC_SCRATCH_BYTES 8192
int fr_sumsq_full_noalloc(const void* x, int64_t n, void* out, int dtype, void* stream);

/* ------------------------------------------------------------ device clock marks
 * fr_device_clock enqueues a one-lane kernel that stores the device's
 * constant wall-clock counter into out[slot] (out: device array of uint64,
 * 8-byte aligned, at least slot + 1 entries; the caller owns it). Two marks
 * around a sequence of launches on one stream give the device time of exactly
 * that sequence, stream order making each mark wait for the work before it;
 * it is how a benchmark times K steps apart from the host's submission of
 * them ("Stax (4)", 9.6: device timing carries about 1% noise, so timings
 * are repeated). fr_device_clock_khz gives the counter's rate in kHz for the
 * current device. FR_E_NULL / FR_E_ARG / FR_E_ALIGN on bad arguments,
 * FR_E_DEVICE if the device is not gfx950. */
int fr_device_clock(uint64_t* out, int slot, void* stream);
int fr_device_clock_khz(int* khz);

/* ------------------------------------------------------------ memory latency
 * The latency lambda of Little's law ("Stax (4)", 9.1: bytes in flight =
 * latency x bandwidth), measured by dependent loads: one lane follows
 * chain[] from index `start` for `steps` loads, each load's address taken
 * from the previous load's value. chain: device array of n uint32 (n <=
 * 2^32), caller-owned; each index read is clamped to [0, n) before use, so
 * the walk never leaves the array whatever it holds. out: device uint64[2]:
 * out[0] = the walk's duration in the ticks of fr_device_clock (rate from
 * fr_device_clock_khz), out[1] = the index reached. A random cycle whose
 * entries lie one cache line or more apart over a span larger than the
 * device caches gives the idle HBM latency; a small span, the cache's.
 * FR_E_NULL / FR_E_SIZE / FR_E_ALIGN on bad arguments. */
int fr_pointer_chase(const uint32_t* chain, int64_t n, int64_t steps, uint32_t start, uint64_t* out, void* stream);

/* ------------------------------------------------------------ configuration search
 * "Stax (4)", 9.6: choosing a launch configuration is black-box optimisation
 * over a configuration space Pi = A_1 x ... x A_p of finite integer value
 * sets (Definition 9.2), with a measured cost t (+infinity, or any negative
 * or NaN value, for a configuration that cannot run). Host code only.
 *  values[i][0 .. counts[i]) is A_i; p <= FR_TUNE_MAX_PARAMS.
 *  cost(ctx, config, p) returns t for one configuration (config[i] a value
 *  of A_i). Each configuration is evaluated at most once per search.
 * fr_tune_coordinate_descent (Algorithm 9.2): starting from `config` (which
 * must lie in Pi with finite cost), for each parameter try twice and half
 * its value when in A_i, accept when t(c') < (1 - eps) t(c), repeat until a
 * round accepts nothing; writes the final configuration to `config`.
 * Returns FR_E_ARG for a bad space, start or eps (0 < eps < 1).
 * fr_tune_random_search (Proposition 9.3): `draws` independent uniform
 * configurations (splitmix64 stream from `seed`); the fastest is written to
 * `best`. FR_E_ARG if every draw is infinite.
 * fr_tune_random_draws(q, delta): the N = ceil(ln(1/delta) / q) draws after
 * which the best lies in the fastest q-fraction with probability >= 1 - delta.
 * fr_tune_threshold(eta_max): an eps above 2 eta / (1 + eta) (and >= 1e-3),
 * so that under relative timing noise |eta| <= eta_max every accepted step
 * of the descent is a real improvement (the remark after Proposition 9.2);
 * -1 for eta_max outside [0, 1). */
#define FR_TUNE_MAX_PARAMS 16
typedef double (*fr_tune_cost_fn)(void* ctx, const int32_t* config, int p);
typedef struct fr_tune_result {
    double cost;          /* t of the configuration returned */
    int64_t evaluations;  /* distinct configurations evaluated */
    int64_t accepted;     /* accepted moves (coordinate descent) */
    int64_t rounds;       /* rounds of the outer loop, or draws */
} fr_tune_result;
int fr_tune_coordinate_descent(const int32_t* const* values, const int32_t* counts, int p, int32_t* config,
                               double eps, fr_tune_cost_fn cost, void* ctx, fr_tune_result* out);
int fr_tune_random_search(const int32_t* const* values, const int32_t* counts, int p, int draws, uint64_t seed,
                          fr_tune_cost_fn cost, void* ctx, int32_t* best, fr_tune_result* out);
int fr_tune_random_draws(double q, double delta);
double fr_tune_threshold(double eta_max);

/* ------------------------------------------------------------ recorded regions
 * "Stax (4)", 9.9: a region of n short kernels launched one by one costs
 * about max(n * t_launch, sum t_k); recorded once as a graph and replayed
 * with one call it costs about t_graph + sum t_k. A region records the
 * launches that a callback enqueues on a stream (HIP stream capture) and
 * replays them while the call is the same:
 *  - fn(ctx, stream) enqueues the region's work on `stream` (fr_* calls with
 *    caller-owned buffers; no host synchronization, no allocation, no value
 *    read back to the host) and returns FR_OK or an error status. For one
 *    key it must enqueue the same kernels with the same grids (9.9,
 *    condition 1).
 *  - key / key_bytes: caller-chosen bytes naming everything a replay fixes,
 *    i.e. the shapes and the device pointers of the call (condition 2). They
 *    are compared on every call.
 *  - First call: records (the recording itself executes nothing), then
 *    replays once. Later calls with the same key, on the device of the
 *    recording: one graph launch. A different key or device: fn runs
 *    directly and the recording is kept. If recording, instantiating or
 *    replaying fails (for example on the legacy default stream, which cannot
 *    be captured), the region enters the fallback state and fn runs directly
 *    from then on.
 * A replay writes to the recorded output addresses; results that must
 * outlive the next call are the caller's to copy. The region object is host
 * memory owned by the caller (create / destroy). Not thread-safe. */
#define FR_REGION_EMPTY 0
#define FR_REGION_RECORDED 1
#define FR_REGION_FALLBACK 2
typedef struct fr_region fr_region;
typedef int (*fr_region_fn)(void* ctx, void* stream);
int fr_region_create(fr_region** out);
void fr_region_destroy(fr_region* r);
/* Returns FR_OK after a replay, else what fn returned. */
int fr_region_run(fr_region* r, const void* key, uint64_t key_bytes, fr_region_fn fn, void* ctx, void* stream);
/* FR_REGION_* state, or FR_E_NULL. */
int fr_region_state(const fr_region* r);
/* Graph launches and direct runs so far (either pointer may be NULL). */
int fr_region_counts(const fr_region* r, uint64_t* replays, uint64_t* direct);

#ifdef __cplusplus
}
#endif

#endif /* FR_H */
