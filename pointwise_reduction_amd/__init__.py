"""pointwise_reduction_amd - fused pointwise-prologue + row-reduction kernels
for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libfr.so`` (C ABI in ``include/fr.h``). The
functions below carry the names of the C entry points and only marshal
arguments: every step of every operation runs in the HIP kernels of libfr.
PyTorch is used for device memory and streams only; tensors are passed as
raw device pointers with their sizes and strides.

There is no CPU fallback: if the library is missing, importing this package
raises, and on a machine without a gfx950 GPU every compute call returns
FR_E_DEVICE (raised as FrError).
"""
import ctypes
import math
import os

try:  # load torch first so that libfr binds to the same HIP runtime as torch
    import torch  # noqa: F401
except ImportError:  # the C ABI is usable without torch
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
# FR_LIB names another build of the same library (the sanitizer run of the
# CPU tests loads a build whose host code is instrumented)
LIB_PATH = os.environ.get("FR_LIB") or os.path.join(_HERE, "libfr.so")

FR_OK = 0
FR_E_NULL, FR_E_SIZE, FR_E_STRIDE, FR_E_DTYPE, FR_E_ALIGN = -1, -2, -3, -4, -5
FR_E_WORKSPACE, FR_E_ARG, FR_E_DEVICE, FR_E_LAUNCH = -6, -7, -8, -9
FR_F32, FR_BF16 = 0, 1
FR_FORM_AUTO, FR_FORM_PER, FR_FORM_RED, FR_FORM_SPLIT, FR_FORM_POINTWISE = 0, 1, 2, 3, 4
FR_OP_SUM_RELU_ADD, FR_OP_SOFTMAX, FR_OP_LAYERNORM, FR_OP_SUMSQ, FR_OP_SOFTMAX_BWD = 1, 2, 3, 4, 5
FR_OP_ADD_2D, FR_OP_GELU_BWD, FR_OP_LAYERNORM_BWD = 6, 7, 8
FORM_NAMES = {FR_FORM_PER: "per", FR_FORM_RED: "red", FR_FORM_SPLIT: "split", FR_FORM_POINTWISE: "pointwise"}

# Every symbol include/fr.h declares.
EXPORTS = (
    "fr_status_string", "fr_version", "fr_plan_query", "fr_force_form", "fr_tune_override",
    "fr_sum_relu_add", "fr_sum_workspace_bytes",
    "fr_softmax_rows_workspace_bytes", "fr_softmax_rows_workspace_init", "fr_softmax_rows",
    "fr_softmax_rows_backward",
    "fr_layernorm_rows", "fr_layernorm_rows_stats", "fr_layernorm_rows_backward_workspace_bytes",
    "fr_layernorm_rows_backward_workspace_init",
    "fr_layernorm_rows_backward",
    "fr_sumsq_rows", "fr_sumsq_full_workspace_bytes", "fr_sumsq_full", "fr_sumsq_full_noalloc",
    "fr_stream_copy", "fr_stream_read", "fr_stream_write", "fr_stream_empty", "fr_device_clock", "fr_device_clock_khz", "fr_pointer_chase",
    "fr_attn_decode_workspace_bytes", "fr_attn_decode",
    "fr_add_2d", "fr_gelu_backward", "fr_attn_block",
    "fr_region_create", "fr_region_destroy", "fr_region_run", "fr_region_state", "fr_region_counts",
    "fr_tune_coordinate_descent", "fr_tune_random_search", "fr_tune_random_draws", "fr_tune_threshold",
    "fr_tune_record", "fr_tune_lookup", "fr_tune_clear",
)


class FrError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class fr_plan(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32), ("form", ctypes.c_int32), ("threads", ctypes.c_int32),
        ("seg", ctypes.c_int32), ("vec", ctypes.c_int32), ("rows_per_wg", ctypes.c_int32),
        ("splits", ctypes.c_int32), ("chunk", ctypes.c_int32), ("vec16", ctypes.c_int32),
        ("occupancy", ctypes.c_int32), ("passes", ctypes.c_int32), ("wait_us", ctypes.c_int32),
        ("grid", ctypes.c_int64), ("grid2", ctypes.c_int64),
        ("ws_bytes", ctypes.c_uint64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python pointwise_reduction_amd/build.py (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    I64, I32, U64, P = ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p
    sig = {
        "fr_status_string": (ctypes.c_char_p, [I32]),
        "fr_version": (I32, []),
        "fr_plan_query": (I32, [I32, I64, I64, I32, I32, I32, U64, I32, ctypes.POINTER(fr_plan)]),
        "fr_force_form": (I32, [I32]),
        "fr_tune_override": (I32, [I32, ctypes.POINTER(fr_plan)]),
        "fr_sum_relu_add": (I32, [P, P, P, I64, I64, I64, I64, I64, I64, I64, P, U64, I32, P]),
        "fr_sum_workspace_bytes": (U64, [I64, I64, I32]),
        "fr_softmax_rows_workspace_bytes": (U64, [I64, I64, I32]),
        "fr_softmax_rows_workspace_init": (I32, [P, U64, P]),
        "fr_softmax_rows": (I32, [P, P, I64, I64, I64, I64, I64, I64, P, P, P, U64, I32, P]),
        "fr_softmax_rows_backward": (I32, [P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, P, I32, P]),
        "fr_layernorm_rows": (I32, [P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_float, I32, P]),
        "fr_sumsq_rows": (I32, [P, P, I64, I64, I64, I64, P, U64, I32, P]),
        "fr_sumsq_full_workspace_bytes": (U64, [I64, I32]),
        "fr_sumsq_full": (I32, [P, I64, P, P, U64, I32, P]),
        "fr_sumsq_full_noalloc": (I32, [P, I64, P, I32, P]),
        "fr_attn_decode_workspace_bytes": (U64, [I64, I64, I64, I64]),
        "fr_attn_decode": (I32, [P, P, P, P, P, I64, I64, I64, I64, I64, P, ctypes.c_float, P, U64, I32, P]),
        "fr_stream_copy": (I32, [P, P, I64, P]),
        "fr_attn_block": (I32, [P, P, P, P, P, I64, I64, I64, I64, I64, I64, I32, ctypes.c_float, I32, P]),
        "fr_stream_read": (I32, [P, I64, P, P]),
        "fr_stream_write": (I32, [P, I64, ctypes.c_uint32, P]),
        "fr_stream_empty": (I32, [P]),
        "fr_device_clock": (I32, [P, I32, P]),
        "fr_device_clock_khz": (I32, [P]),
        "fr_pointer_chase": (I32, [P, I64, I64, ctypes.c_uint32, P, P]),
        "fr_add_2d": (I32, [P, I64, I64, P, I64, I64, P, I64, I64, I64, I32, P]),
        "fr_layernorm_rows_stats": (I32, [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_float, I32, P]),
        "fr_layernorm_rows_backward_workspace_bytes": (U64, [I64, I64, I32]),
        "fr_layernorm_rows_backward_workspace_init": (I32, [P, U64, P]),
        "fr_layernorm_rows_backward": (I32, [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, P, U64,
                                             I32, P]),
        "fr_gelu_backward": (I32, [P, I64, P, P, I64, I32, P]),
        "fr_tune_coordinate_descent": (I32, [P, P, I32, P, ctypes.c_double, P, P, P]),
        "fr_tune_random_search": (I32, [P, P, I32, I32, U64, P, P, P, P]),
        "fr_tune_random_draws": (I32, [ctypes.c_double, ctypes.c_double]),
        "fr_tune_record": (I32, [I32, I64, I64, I32, ctypes.POINTER(fr_plan)]),
        "fr_tune_lookup": (I32, [I32, I64, I64, I32, ctypes.POINTER(fr_plan)]),
        "fr_tune_clear": (None, []),
        "fr_tune_threshold": (ctypes.c_double, [ctypes.c_double]),
        "fr_region_create": (I32, [ctypes.POINTER(P)]),
        "fr_region_destroy": (None, [P]),
        "fr_region_run": (I32, [P, P, U64, P, P, P]),
        "fr_region_state": (I32, [P]),
        "fr_region_counts": (I32, [P, ctypes.POINTER(U64), ctypes.POINTER(U64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_string(status):
    return lib.fr_status_string(int(status)).decode()


def _check(status, where):
    if status != FR_OK:
        raise FrError(status, where)


# ------------------------------------------------------------------ marshalling helpers


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream) if torch is not None else None
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return FR_F32
    if t.dtype == torch.bfloat16:
        return FR_BF16
    return -1


def _mat(t):
    """(rows, cols, row_stride, col_stride) of a 2-D tensor view."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    return t.shape[0], t.shape[1], t.stride(0), t.stride(1)


# ------------------------------------------------------------------ entry points


def fr_plan_query(op, rows, cols, dtype=FR_F32, num_cus=256, has_lengths=False, ws_bytes=0, aligned16=True):
    plan = fr_plan()
    _check(lib.fr_plan_query(op, rows, cols, dtype, num_cus, int(has_lengths), ws_bytes, int(aligned16),
                             ctypes.byref(plan)), "fr_plan_query")
    return plan


def fr_force_form(form):
    return lib.fr_force_form(form)


def fr_tune_override(op, plan=None, **knobs):
    """Use a candidate launch configuration for every later call of `op`
    (tuning). Pass an fr_plan or keyword knobs (form, threads, seg, vec,
    rows_per_wg, chunk, occupancy); plan=None and no knobs clears it."""
    if plan is None and knobs:
        plan = fr_plan()
        for k, v in knobs.items():
            setattr(plan, k, v)
    _check(lib.fr_tune_override(op, None if plan is None else ctypes.byref(plan)), "fr_tune_override")


def fr_sum_workspace_bytes(rows, cols, dtype=FR_F32):
    return int(lib.fr_sum_workspace_bytes(rows, cols, dtype))


def fr_softmax_rows_workspace_bytes(rows, cols, dtype=FR_F32):
    return int(lib.fr_softmax_rows_workspace_bytes(rows, cols, dtype))


def fr_softmax_rows_workspace_init(ws, stream=None):
    """Initialize a split-softmax workspace tensor (once, before its first
    use); every fr_softmax_rows call leaves it initialized."""
    if not ws.is_contiguous():
        raise ValueError("expected a contiguous workspace")
    _check(lib.fr_softmax_rows_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "fr_softmax_rows_workspace_init")
    return ws


def fr_sumsq_full_workspace_bytes(n, dtype=FR_F32):
    return int(lib.fr_sumsq_full_workspace_bytes(n, dtype))


def fr_sum_relu_add(a, b, out, ws=None, stream=None):
    """out[i] = sum_j 2*relu(a[i,j] + b[i,j]) (fp32). out: 1-D, len rows."""
    rows, cols, a_rs, a_cs = _mat(a)
    rb, cb, b_rs, b_cs = _mat(b)
    if (rb, cb) != (rows, cols) or out.shape[0] != rows:
        raise ValueError("shape mismatch")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.fr_sum_relu_add(_ptr(a), _ptr(b), _ptr(out), rows, cols, a_rs, a_cs, b_rs, b_cs, out.stride(0),
                               _ptr(ws), ws_bytes, _dtype_code(a), _stream(stream)), "fr_sum_relu_add")
    return out


def fr_softmax_rows(x, y, lengths=None, argmax=None, ws=None, stream=None):
    rows, cols, x_rs, x_cs = _mat(x)
    ry, cy, y_rs, y_cs = _mat(y)
    if (ry, cy) != (rows, cols):
        raise ValueError("shape mismatch")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.fr_softmax_rows(_ptr(x), _ptr(y), rows, cols, x_rs, x_cs, y_rs, y_cs, _ptr(lengths), _ptr(argmax),
                               _ptr(ws), ws_bytes, _dtype_code(x), _stream(stream)), "fr_softmax_rows")
    return y


def fr_softmax_rows_backward(y, dy, dx, lengths=None, stream=None):
    """dx = y * (dy - sum(dy * y)) per row (fp32 [rows, cols] views)."""
    rows, cols, y_rs, y_cs = _mat(y)
    r2, c2, dy_rs, dy_cs = _mat(dy)
    r3, c3, dx_rs, dx_cs = _mat(dx)
    if (r2, c2) != (rows, cols) or (r3, c3) != (rows, cols):
        raise ValueError("shape mismatch")
    _check(lib.fr_softmax_rows_backward(_ptr(y), _ptr(dy), _ptr(dx), rows, cols, y_rs, y_cs, dy_rs, dy_cs, dx_rs, dx_cs,
                                        _ptr(lengths), _dtype_code(y), _stream(stream)), "fr_softmax_rows_backward")
    return dx


def fr_layernorm_rows(x, y, gamma=None, beta=None, eps=1e-5, stream=None):
    rows, cols, x_rs, x_cs = _mat(x)
    ry, cy, y_rs, y_cs = _mat(y)
    if (ry, cy) != (rows, cols):
        raise ValueError("shape mismatch")
    _check(lib.fr_layernorm_rows(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, cols, x_rs, x_cs, y_rs, y_cs,
                                 float(eps), _dtype_code(x), _stream(stream)), "fr_layernorm_rows")
    return y


def fr_layernorm_rows_stats(x, y, mean=None, rstd=None, gamma=None, beta=None, eps=1e-5, stream=None):
    """LayerNorm that also writes the per-row mean and rstd (fp32 [rows])."""
    rows, cols, x_rs, x_cs = _mat(x)
    ry, cy, y_rs, y_cs = _mat(y)
    if (ry, cy) != (rows, cols):
        raise ValueError("shape mismatch")
    _check(lib.fr_layernorm_rows_stats(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), rows, cols,
                                       x_rs, x_cs, y_rs, y_cs, float(eps), _dtype_code(x), _stream(stream)),
           "fr_layernorm_rows_stats")
    return y


def fr_layernorm_rows_backward_workspace_bytes(rows, cols, dtype=FR_BF16):
    return lib.fr_layernorm_rows_backward_workspace_bytes(rows, cols, dtype)


def fr_layernorm_rows_backward_workspace_init(ws, stream=None):
    """Initialize a LayerNorm-backward workspace tensor (once, before its
    first use); every fr_layernorm_rows_backward call leaves it initialized."""
    if not ws.is_contiguous():
        raise ValueError("expected a contiguous workspace")
    _check(lib.fr_layernorm_rows_backward_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "fr_layernorm_rows_backward_workspace_init")
    return ws


def fr_layernorm_rows_backward(x, dy, mean, rstd, dx, gamma=None, dgamma=None, dbeta=None, ws=None, stream=None):
    """dx (bf16), and optionally dgamma / dbeta (fp32 [cols]), from the saved
    mean and rstd. A workspace is allocated and initialized when dgamma or
    dbeta is requested and ws is None."""
    rows, cols, x_rs, x_cs = _mat(x)
    r2, c2, dy_rs, dy_cs = _mat(dy)
    r3, c3, dx_rs, dx_cs = _mat(dx)
    if (r2, c2) != (rows, cols) or (r3, c3) != (rows, cols):
        raise ValueError("shape mismatch")
    if ws is None and (dgamma is not None or dbeta is not None):
        nbytes = fr_layernorm_rows_backward_workspace_bytes(rows, cols)
        ws = torch.empty(max(nbytes, 64) // 4, dtype=torch.float32, device=x.device)
        fr_layernorm_rows_backward_workspace_init(ws, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.fr_layernorm_rows_backward(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx),
                                          _ptr(dgamma), _ptr(dbeta), rows, cols, x_rs, x_cs, dy_rs, dy_cs, dx_rs,
                                          dx_cs, _ptr(ws), ws_bytes, _dtype_code(x), _stream(stream)),
           "fr_layernorm_rows_backward")
    return dx


def fr_sumsq_rows(x, out, ws=None, stream=None):
    rows, cols, x_rs, x_cs = _mat(x)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.fr_sumsq_rows(_ptr(x), _ptr(out), rows, cols, x_rs, x_cs, _ptr(ws), ws_bytes, _dtype_code(x),
                             _stream(stream)), "fr_sumsq_rows")
    return out


def fr_sumsq_full(x, out, ws=None, stream=None):
    if x.dim() != 1 or (x.numel() > 1 and x.stride(0) != 1):
        raise ValueError("expected a contiguous 1-D tensor")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.fr_sumsq_full(_ptr(x), x.numel(), _ptr(out), _ptr(ws), ws_bytes, _dtype_code(x), _stream(stream)),
           "fr_sumsq_full")
    return out


FR_NOALLOC_SCRATCH_BYTES = 8192


def fr_sumsq_full_noalloc(x, out, stream=None):
    """fr_sumsq_full with its partials in the library's own device array (no
    workspace, nothing allocated)."""
    if x.dim() != 1 or (x.numel() > 1 and x.stride(0) != 1):
        raise ValueError("expected a contiguous 1-D tensor")
    _check(lib.fr_sumsq_full_noalloc(_ptr(x), x.numel(), _ptr(out), _dtype_code(x), _stream(stream)),
           "fr_sumsq_full_noalloc")
    return out


FR_STREAM_SINK_WORDS = 1024


def fr_stream_copy(x, y, stream=None):
    """y = x for contiguous tensors of the same byte size (a multiple of 16):
    the streaming reference copy."""
    nbytes = x.numel() * x.element_size()
    if not (x.is_contiguous() and y.is_contiguous()) or y.numel() * y.element_size() != nbytes:
        raise ValueError("expected contiguous tensors of the same byte size")
    _check(lib.fr_stream_copy(_ptr(x), _ptr(y), nbytes, _stream(stream)), "fr_stream_copy")
    return y


def fr_stream_read(x, sink, stream=None):
    """Read every byte of contiguous x; sink (FR_STREAM_SINK_WORDS int32 or
    uint32) receives per-workgroup XORs of the 32-bit words read."""
    if not x.is_contiguous() or sink.numel() * sink.element_size() < 4 * FR_STREAM_SINK_WORDS:
        raise ValueError("expected a contiguous input and a sink of FR_STREAM_SINK_WORDS words")
    _check(lib.fr_stream_read(_ptr(x), x.numel() * x.element_size(), _ptr(sink), _stream(stream)),
           "fr_stream_read")
    return sink


def fr_stream_write(y, value, stream=None):
    """Every 32-bit word of contiguous y (a multiple of 16 bytes) = value
    (an unsigned 32-bit pattern): the streaming reference write."""
    if not y.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    _check(lib.fr_stream_write(_ptr(y), y.numel() * y.element_size(), value & 0xFFFFFFFF, _stream(stream)),
           "fr_stream_write")
    return y


def fr_stream_empty(stream=None):
    """Enqueue a kernel that does nothing: back to back, one kernel boundary."""
    _check(lib.fr_stream_empty(_stream(stream)), "fr_stream_empty")


def fr_device_clock(out, slot, stream=None):
    """Enqueue a store of the device's constant wall clock into out[slot]
    (out: int64 device tensor)."""
    if out.dtype != torch.int64 or not out.is_contiguous() or not 0 <= slot < out.numel():
        raise ValueError("expected a contiguous int64 tensor with more than `slot` entries")
    _check(lib.fr_device_clock(_ptr(out), slot, _stream(stream)), "fr_device_clock")
    return out


def fr_device_clock_khz():
    """Rate of the counter fr_device_clock stores, in kHz."""
    khz = ctypes.c_int32()
    _check(lib.fr_device_clock_khz(ctypes.byref(khz)), "fr_device_clock_khz")
    return khz.value


def fr_pointer_chase(chain, steps, start, out, stream=None):
    """Follow chain (contiguous int32/uint32 device tensor of indices) from
    `start` for `steps` dependent loads; out (int64 device tensor, 2 entries)
    receives the ticks taken and the index reached."""
    if chain.dtype not in (torch.int32,) or not chain.is_contiguous():
        raise ValueError("expected a contiguous int32 chain")
    if out.dtype != torch.int64 or not out.is_contiguous() or out.numel() < 2:
        raise ValueError("expected an int64 tensor of 2 entries")
    _check(lib.fr_pointer_chase(_ptr(chain), chain.numel(), steps, start, _ptr(out), _stream(stream)),
           "fr_pointer_chase")
    return out


def fr_attn_decode_workspace_bytes(batch, heads_q, seq, dim):
    return int(lib.fr_attn_decode_workspace_bytes(batch, heads_q, seq, dim))


def fr_attn_decode(q, k, v, o, lse=None, lengths=None, scale=None, ws=None, stream=None):
    """Decode attention: q, o [B, Hq, D]; k, v [B, Hkv, S, D] (contiguous,
    float32 or bfloat16); lse optional fp32 [B, Hq]; lengths optional int32
    [B]. scale defaults to 1/sqrt(D). A workspace of the queried size is
    allocated with torch when none is given."""
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("expected q, o [B, Hq, D] and k, v [B, Hkv, S, D]")
    B, Hq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if not all(t.is_contiguous() for t in (q, k, v, o)):
        raise ValueError("expected contiguous tensors")
    Hkv, S = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = fr_attn_decode_workspace_bytes(B, Hq, S, D)
    if ws is None and need > 0:
        ws = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.fr_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, S, D, _ptr(lengths),
                              float(scale), _ptr(ws), ws_bytes, _dtype_code(q), _stream(stream)), "fr_attn_decode")
    return o


def fr_attn_block(q, k, v, o, lse, causal=False, scale=None, stream=None):
    """Tiled attention: q, o [B, Hq, Nq, D]; k, v [B, Hkv, Nk, D] bf16
    contiguous; lse fp32 [B, Hq, Nq]. scale defaults to 1 / sqrt(D)."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("q, o: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D]")
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("shape mismatch")
    for t in (q, k, v, o, lse):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(lib.fr_attn_block(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                             float(scale), _dtype_code(q), _stream(stream)), "fr_attn_block")
    return o


def fr_add_2d(a, b, out, stream=None):
    """out = a + b for fp32 2-D views of one shape; a or b may be a
    transposed view (x.t()). out must be row-major."""
    rows, cols, a_rs, a_cs = _mat(a)
    rb, cb, b_rs, b_cs = _mat(b)
    ro, co, out_rs, out_cs = _mat(out)
    if (rb, cb) != (rows, cols) or (ro, co) != (rows, cols):
        raise ValueError("shape mismatch")
    if out_cs != 1 and rows * cols > 0 and cols > 1:
        raise ValueError("out must have unit inner stride")
    if _dtype_code(b) != _dtype_code(a) or _dtype_code(out) != _dtype_code(a):
        raise ValueError("dtype mismatch")
    _check(lib.fr_add_2d(_ptr(a), a_rs, a_cs, _ptr(b), b_rs, b_cs, _ptr(out), out_rs, rows, cols, _dtype_code(a),
                         _stream(stream)), "fr_add_2d")
    return out


def fr_gelu_backward(dy, h, dx, stream=None):
    """dx = dy * (Phi(h) + h phi(h)); dy holds one element (broadcast) or as
    many as h. h, dx contiguous, fp32 or bf16 (all three alike)."""
    n = h.numel()
    if dx.numel() != n or not h.is_contiguous() or not dx.is_contiguous() or not dy.is_contiguous():
        raise ValueError("h, dx and dy must be contiguous and dx shaped like h")
    if dy.numel() not in (1, n):
        raise ValueError("dy must hold one element or one per element of h")
    if _dtype_code(dy) != _dtype_code(h) or _dtype_code(dx) != _dtype_code(h):
        raise ValueError("dtype mismatch")
    stride = 0 if dy.numel() == 1 and n != 1 else 1
    _check(lib.fr_gelu_backward(_ptr(dy), stride, _ptr(h), _ptr(dx), n, _dtype_code(h), _stream(stream)),
           "fr_gelu_backward")
    return dx


# ------------------------------------------------------------------ recorded regions

FR_REGION_EMPTY, FR_REGION_RECORDED, FR_REGION_FALLBACK = 0, 1, 2
_REGION_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p)


class Region:
    """A recorded region ("Stax (4)", 9.9): the launches fn(stream) enqueues
    are recorded once as a HIP graph and replayed while `key` (the shapes and
    device pointers of the call, as integers) stays the same; otherwise fn
    runs directly. fn receives the stream as an integer handle and passes it
    to the fr_* calls it makes; it must use preallocated buffers only."""

    def __init__(self):
        p = ctypes.c_void_p()
        _check(lib.fr_region_create(ctypes.byref(p)), "fr_region_create")
        self._r = p

    def __del__(self):
        r, self._r = getattr(self, "_r", None), None
        if r is not None and lib is not None:
            lib.fr_region_destroy(r)

    def run(self, key, fn, stream=None):
        kb = b"".join(int(k).to_bytes(8, "little", signed=True) for k in key)
        err = []

        def cb(_ctx, s):
            try:
                fn(0 if s is None else s)
                return FR_OK
            except FrError as e:
                err.append(e)
                return e.status
            except Exception as e:  # noqa: BLE001  (reported after the C call returns)
                err.append(e)
                return FR_E_ARG

        c = _REGION_FN(cb)
        st = lib.fr_region_run(self._r, kb, len(kb), c, None, _stream(stream))
        if err:
            raise err[-1]
        _check(st, "fr_region_run")

    @property
    def state(self):
        return lib.fr_region_state(self._r)

    def counts(self):
        rep, direct = ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib.fr_region_counts(self._r, ctypes.byref(rep), ctypes.byref(direct)), "fr_region_counts")
        return rep.value, direct.value


# ------------------------------------------------------------------ configuration search

_TUNE_COST = ctypes.CFUNCTYPE(ctypes.c_double, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int)


class fr_tune_result(ctypes.Structure):
    _fields_ = [("cost", ctypes.c_double), ("evaluations", ctypes.c_int64), ("accepted", ctypes.c_int64),
                ("rounds", ctypes.c_int64)]


def _space(space):
    """space: list of value lists -> (values**, counts*, keepalive)."""
    arrs = [(ctypes.c_int32 * len(v))(*v) for v in space]
    ptrs = (ctypes.POINTER(ctypes.c_int32) * len(space))(*[ctypes.cast(a, ctypes.POINTER(ctypes.c_int32))
                                                             for a in arrs])
    counts = (ctypes.c_int32 * len(space))(*[len(v) for v in space])
    return ptrs, counts, arrs


def _cost_cb(cost):
    err = []

    def cb(_ctx, cfg, p):
        try:
            t = float(cost(tuple(cfg[i] for i in range(p))))
            return t if math.isfinite(t) else math.inf
        except Exception as e:  # noqa: BLE001  (re-raised after the C call)
            err.append(e)
            return math.inf
    return _TUNE_COST(cb), err


def fr_tune_coordinate_descent(space, start, eps, cost):
    """Algorithm 9.2 over `space` (a list of value lists) from `start`; cost
    maps a configuration tuple to a time (math.inf if it cannot run).
    Returns (configuration, fr_tune_result)."""
    ptrs, counts, keep = _space(space)
    cfg = (ctypes.c_int32 * len(space))(*start)
    cb, err = _cost_cb(cost)
    res = fr_tune_result()
    st = lib.fr_tune_coordinate_descent(ptrs, counts, len(space), cfg, float(eps), cb, None, ctypes.byref(res))
    if err:
        raise err[-1]
    _check(st, "fr_tune_coordinate_descent")
    return tuple(cfg), res


def fr_tune_random_search(space, draws, seed, cost):
    """Proposition 9.3's random search: the best of `draws` uniform draws."""
    ptrs, counts, keep = _space(space)
    best = (ctypes.c_int32 * len(space))()
    cb, err = _cost_cb(cost)
    res = fr_tune_result()
    st = lib.fr_tune_random_search(ptrs, counts, len(space), int(draws), int(seed), cb, None, best,
                                   ctypes.byref(res))
    if err:
        raise err[-1]
    _check(st, "fr_tune_random_search")
    return tuple(best), res


def fr_tune_random_draws(q, delta):
    n = lib.fr_tune_random_draws(float(q), float(delta))
    _check(min(n, 0), "fr_tune_random_draws")
    return n


def fr_tune_record(op, rows, cols, dtype=FR_F32, plan=None, **knobs):
    """Record the configuration for calls of `op` at exactly (rows, cols,
    dtype); plan=None and no knobs removes the record."""
    if plan is None and knobs:
        plan = fr_plan()
        for k, v in knobs.items():
            setattr(plan, k, v)
    _check(lib.fr_tune_record(op, rows, cols, dtype, None if plan is None else ctypes.byref(plan)),
           "fr_tune_record")


def fr_tune_lookup(op, rows, cols, dtype=FR_F32):
    """The recorded configuration for this shape, or None."""
    plan = fr_plan()
    st = lib.fr_tune_lookup(op, rows, cols, dtype, ctypes.byref(plan))
    return plan if st == FR_OK else None


def fr_tune_clear():
    lib.fr_tune_clear()


def fr_tune_threshold(eta_max):
    return lib.fr_tune_threshold(float(eta_max))
