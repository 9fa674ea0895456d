"""Thin Python binding of libhdq (C ABI in include/hdq.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the path runs in libhdq's HIP kernels.  The names
follow the C entry points: select_precision, quantize, linear.  Importing
this module loads libhdq.so and raises if it is missing (build it with
__graft_entry__.build() or `python bit_quantized_video_amd/build.py`); there
is no CPU fallback.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhdq.so")

# status codes
OK, ERR_INVALID, ERR_SHAPE, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE, ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 2 << 20      # HDQ_NOALLOC_SCRATCH_BYTES
# formats
FMT_INT8_ROW, FMT_INT4_ROW, FMT_NVFP4, FMT_NVFP4_MX, FMT_NVFP4_P2 = 0, 1, 2, 3, 4
# precisions
PREC_NVFP4, PREC_INT8, PREC_BF16 = 0, 1, 2
# output dtypes
DTYPE_F32, DTYPE_BF16, DTYPE_I32 = 0, 1, 2
# workspace ops
OP_SELECT, OP_QUANTIZE, OP_LINEAR, OP_SELECT_Q8, OP_DQ_QUANTIZE, OP_DQ_LINEAR = 0, 1, 2, 3, 4, 5

EXPORTS = ("hdq_select_precision", "hdq_delta_sums", "hdq_select_precision_sums",
           "hdq_select_quantize_int8", "hdq_select_quantize_int8_noalloc", "hdq_linear_dispatch", "hdq_linear_dispatch_delta",
           "hdq_tdc_decide", "hdq_quantize", "hdq_dq_cubes", "hdq_dq_quantize", "hdq_dq_decode_weights",
           "hdq_dq_linear", "hdq_dq_linear_workspace_bytes",
           "hdq_linear", "hdq_workspace_bytes",
           "hdq_status_string", "hdq_version")

_c = ctypes
_p = _c.c_void_p


class QTensorDesc(_c.Structure):
    """hdq_qtensor."""
    _fields_ = [("fmt", _c.c_int32), ("had_block", _c.c_int32), ("rows", _c.c_int64),
                ("cols", _c.c_int64), ("codes", _p), ("row_scale", _p), ("blk_scale", _p),
                ("tensor_scale", _p), ("dec", _p)]


class DeltaSlice(_c.Structure):
    """hdq_delta_slice."""
    _fields_ = [("prev_in", _p), ("prev_out", _p), ("numel", _c.c_int64), ("chunk_begin", _c.c_int64),
                ("chunk_end", _c.c_int64), ("partials", _p)]


DELTA_CHUNK = 65536       # HDQ_DELTA_CHUNK
DELTA_MAX_SLICES = 4      # HDQ_DELTA_MAX_SLICES


def delta_chunks(numel):
    """Chunks (and partial pairs) of a module's difference statistic."""
    return (numel + DELTA_CHUNK - 1) // DELTA_CHUNK


class DqGridDesc(_c.Structure):
    """hdq_dq_grid."""
    _fields_ = [("frames", _c.c_int64), ("height", _c.c_int64), ("width", _c.c_int64),
                ("cube_f", _c.c_int32), ("cube_h", _c.c_int32), ("cube_w", _c.c_int32)]


class WeightsDesc(_c.Structure):
    """hdq_weights."""
    _fields_ = [("N", _c.c_int64), ("K", _c.c_int64), ("w_bf16", _p), ("w_int4", QTensorDesc),
                ("w_fp4", QTensorDesc)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libhdq.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    L = _c.CDLL(LIB_PATH)
    L.hdq_select_precision.restype = _c.c_int
    L.hdq_select_precision.argtypes = [_p, _p, _c.c_int64, _p, _c.c_int64, _c.c_int64, _c.c_int32,
                                       _c.c_float, _c.c_float, _p, _p, _p, _c.c_size_t, _p]
    L.hdq_delta_sums.restype = _c.c_int
    L.hdq_delta_sums.argtypes = [_p, _p, _c.c_int64, _p, _p, _c.c_size_t, _p]
    L.hdq_select_precision_sums.restype = _c.c_int
    L.hdq_select_precision_sums.argtypes = [_p, _c.c_int64, _p, _c.c_int64, _c.c_int64, _c.c_int32,
                                            _c.c_float, _c.c_float, _p, _p, _p, _c.c_size_t, _p]
    L.hdq_select_quantize_int8.restype = _c.c_int
    L.hdq_select_quantize_int8.argtypes = [_p, _c.c_int64, _p, _c.c_int64, _c.c_int64, _c.c_int32,
                                           _c.c_float, _c.c_float, _p, _p, _c.POINTER(QTensorDesc), _p,
                                           _c.c_size_t, _p]
    L.hdq_select_quantize_int8_noalloc.restype = _c.c_int
    L.hdq_select_quantize_int8_noalloc.argtypes = [_p, _c.c_int64, _p, _c.c_int64, _c.c_int64, _c.c_int32,
                                                   _c.c_float, _c.c_float, _p, _p, _c.POINTER(QTensorDesc), _p]
    L.hdq_linear_dispatch.restype = _c.c_int
    L.hdq_linear_dispatch.argtypes = [_p, _p, _c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc),
                                      _c.c_int64, _c.c_int64, _c.POINTER(WeightsDesc), _p, _c.c_int32, _p]
    L.hdq_linear_dispatch_delta.restype = _c.c_int
    L.hdq_linear_dispatch_delta.argtypes = [_p, _p, _c.POINTER(QTensorDesc), _c.POINTER(QTensorDesc),
                                            _c.c_int64, _c.c_int64, _c.POINTER(WeightsDesc), _p,
                                            _c.c_int32, _c.POINTER(DeltaSlice), _c.c_int32, _p, _p]
    L.hdq_tdc_decide.restype = _c.c_int
    L.hdq_tdc_decide.argtypes = [_p, _p, _p, _p, _p, _p, _c.c_int64, _c.c_float, _c.c_float, _p]
    L.hdq_quantize.restype = _c.c_int
    L.hdq_quantize.argtypes = [_p, _c.c_int64, _c.c_int64, _c.c_int32, _c.c_int32, _p, _p,
                               _c.POINTER(QTensorDesc), _p, _c.c_size_t, _p]
    L.hdq_linear.restype = _c.c_int
    L.hdq_linear.argtypes = [_c.c_int32, _p, _p, _c.POINTER(QTensorDesc), _p, _c.c_int64,
                             _c.c_int64, _c.POINTER(WeightsDesc), _p, _c.c_int32, _p,
                             _c.c_size_t, _p]
    L.hdq_dq_cubes.restype = _c.c_int64
    L.hdq_dq_cubes.argtypes = [_c.POINTER(DqGridDesc)]
    L.hdq_dq_quantize.restype = _c.c_int
    L.hdq_dq_quantize.argtypes = [_p, _c.c_int64, _c.POINTER(DqGridDesc), _c.c_int32, _p, _p, _p,
                                  _c.POINTER(QTensorDesc), _p, _c.c_size_t, _p]
    L.hdq_dq_decode_weights.restype = _c.c_int
    L.hdq_dq_decode_weights.argtypes = [_c.POINTER(QTensorDesc), _p, _p]
    L.hdq_dq_linear.restype = _c.c_int
    L.hdq_dq_linear.argtypes = [_c.POINTER(DqGridDesc), _p, _p, _p, _c.POINTER(QTensorDesc),
                                _c.POINTER(QTensorDesc), _p, _p, _c.c_int32, _p, _c.c_size_t, _p]
    L.hdq_dq_linear_workspace_bytes.restype = _c.c_size_t
    L.hdq_dq_linear_workspace_bytes.argtypes = [_c.POINTER(DqGridDesc), _c.c_int64, _c.c_int64, _c.c_int32]
    L.hdq_workspace_bytes.restype = _c.c_size_t
    L.hdq_workspace_bytes.argtypes = [_c.c_int32, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int32]
    L.hdq_status_string.restype = _c.c_char_p
    L.hdq_status_string.argtypes = [_c.c_int]
    L.hdq_version.restype = _c.c_int
    L.hdq_version.argtypes = []
    return L


lib = _load()


class HdqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {lib.hdq_status_string(status).decode()} ({status})")


def _check(fn, status):
    if status != OK:
        raise HdqError(fn, status)


def _ptr(t):
    return None if t is None else _p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _p(s.cuda_stream)


def _bf16(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    return t


def linear_dispatch(decision, x, xq8, xq4, w, y=None, y_dtype=DTYPE_BF16, stream=None):
    """hdq_linear_dispatch: the GEMM of the device decision's precision in
    one launch (INT8 from xq8, NVFP4 from xq4, bf16 from x)."""
    x = _bf16(x, "x")
    M, K = x.shape
    if y is None:
        dt = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}[y_dtype]
        y = torch.empty(M, w.N, dtype=dt, device=x.device)
    wd, d8, d4 = w.desc(), xq8.desc(), xq4.desc()
    st = lib.hdq_linear_dispatch(_ptr(decision), _ptr(x), _c.byref(d8), _c.byref(d4), M, K,
                                 _c.byref(wd), _ptr(y), y_dtype, _stream(stream))
    _check("hdq_linear_dispatch", st)
    return y


def linear_dispatch_delta(decision, x, xq8, xq4, w, slices, queue, y=None, y_dtype=DTYPE_BF16,
                          stream=None):
    """hdq_linear_dispatch_delta: linear_dispatch's GEMM, plus the chunk
    partials of difference statistics on extra workgroups of the launch.
    slices: up to DELTA_MAX_SLICES tuples (prev_in, prev_out, chunk_begin,
    chunk_end, partials), partials float64 [delta_chunks(numel), 2];
    queue: int32 [2] on the device, zero before the first call (each call
    leaves it zero)."""
    x = _bf16(x, "x")
    M, K = x.shape
    if y is None:
        dt = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}[y_dtype]
        y = torch.empty(M, w.N, dtype=dt, device=x.device)
    arr = (DeltaSlice * max(1, len(slices)))()
    for i, (pi, po, c0, c1, parts) in enumerate(slices):
        _bf16(pi, "prev_in")
        _bf16(po, "prev_out")
        if pi.numel() != po.numel():
            raise ValueError("prev_in and prev_out differ in size")
        if parts.dtype != torch.float64 or parts.numel() < 2 * delta_chunks(pi.numel()):
            raise ValueError("partials: float64 [delta_chunks(numel), 2] expected")
        arr[i] = DeltaSlice(_ptr(pi), _ptr(po), pi.numel(), c0, c1, _ptr(parts))
    if queue.dtype != torch.int32 or queue.numel() < 2:
        raise ValueError("queue: int32 [2] expected")
    wd, d8, d4 = w.desc(), xq8.desc(), xq4.desc()
    st = lib.hdq_linear_dispatch_delta(_ptr(decision), _ptr(x), _c.byref(d8), _c.byref(d4), M, K,
                                       _c.byref(wd), _ptr(y), y_dtype, arr, len(slices), _ptr(queue),
                                       _stream(stream))
    _check("hdq_linear_dispatch_delta", st)
    return y


def workspace_bytes(op, M, K, N=0, fmt=-1):
    return int(lib.hdq_workspace_bytes(op, M, K, N, fmt))


def _workspace(ws, nbytes, device):
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() < nbytes:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


class QuantizedTensor:
    """A quantized tensor: torch buffers plus the hdq_qtensor descriptor.
    decoded (NVFP4 formats): also a bf16 [rows, cols] buffer for the codes'
    exact values, which hdq_quantize fills and the plain-NVFP4 GEMM reads."""

    def __init__(self, fmt, rows, cols, had_block, device, decoded=False):
        self.fmt, self.rows, self.cols, self.had_block = fmt, rows, cols, had_block
        self.row_scale = self.blk_scale = self.tensor_scale = self.dec = None
        if fmt == FMT_INT8_ROW:
            self.codes = torch.empty(rows, cols, dtype=torch.int8, device=device)
        else:
            self.codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device=device)
        if fmt in (FMT_INT8_ROW, FMT_INT4_ROW):
            self.row_scale = torch.empty(rows, dtype=torch.float32, device=device)
        else:
            self.blk_scale = torch.empty(rows, cols // 16, dtype=torch.uint8, device=device)
            self.tensor_scale = torch.empty(1, dtype=torch.float32, device=device)
            if decoded:
                self.dec = torch.empty(rows, cols, dtype=torch.bfloat16, device=device)

    def desc(self):
        return QTensorDesc(self.fmt, self.had_block, self.rows, self.cols, _ptr(self.codes),
                           _ptr(self.row_scale), _ptr(self.blk_scale), _ptr(self.tensor_scale),
                           _ptr(self.dec))


def select_precision(prev_in, prev_out, cur_in, had_block=0, delta_thresh=0.1, ratio_thresh=50.0,
                     decision=None, stats=None, ws=None, stream=None):
    """hdq_select_precision.  prev_in/prev_out None = no history.  Returns the
    device tensors (decision int32[1], stats float32[5])."""
    cur_in = _bf16(cur_in, "cur_in")
    rows, cols = cur_in.shape
    dev = cur_in.device
    if (prev_in is None) != (prev_out is None):
        raise ValueError("prev_in and prev_out must both be given or both be None")
    n_prev = 0
    if prev_in is not None:
        _bf16(prev_in, "prev_in")
        _bf16(prev_out, "prev_out")
        if prev_in.numel() != prev_out.numel():
            raise ValueError("prev_in and prev_out differ in size")
        n_prev = prev_in.numel()
    decision = torch.empty(1, dtype=torch.int32, device=dev) if decision is None else decision
    stats = torch.empty(5, dtype=torch.float32, device=dev) if stats is None else stats
    ws = _workspace(ws, workspace_bytes(OP_SELECT, rows, cols, n_prev), dev)
    st = lib.hdq_select_precision(_ptr(prev_in), _ptr(prev_out), n_prev, _ptr(cur_in), rows, cols,
                                  had_block, delta_thresh, ratio_thresh, _ptr(decision),
                                  _ptr(stats), _ptr(ws), ws.numel(), _stream(stream))
    _check("hdq_select_precision", st)
    return decision, stats


def delta_sums(prev_in, prev_out, sums=None, ws=None, stream=None):
    """hdq_delta_sums: device double[2] {sum|prev_out - prev_in|, sum|prev_in|}."""
    _bf16(prev_in, "prev_in")
    _bf16(prev_out, "prev_out")
    if prev_in.numel() != prev_out.numel():
        raise ValueError("prev_in and prev_out differ in size")
    n = prev_in.numel()
    dev = prev_in.device
    sums = torch.empty(2, dtype=torch.float64, device=dev) if sums is None else sums
    ws = _workspace(ws, workspace_bytes(OP_SELECT, 1, n, n), dev)
    st = lib.hdq_delta_sums(_ptr(prev_in), _ptr(prev_out), n, _ptr(sums), _ptr(ws), ws.numel(),
                            _stream(stream))
    _check("hdq_delta_sums", st)
    return sums


def tdc_decide(sums, state, c, acc, skip=None, tau_skip=0.05, tau_acc=0.15, stream=None, offsets=None):
    """hdq_tdc_decide over n modules: sums float64 [n, 2] (or, with offsets
    int64 [n + 1], pairs [P, 2] of which module i's are rows offsets[i] ..
    offsets[i + 1] - 1), state int32 [n], c and acc float32 [n] (updated in
    place); returns skip int32 [n]."""
    n = state.numel()
    pairs = (n, 2) if offsets is None else (sums.shape[0], 2)
    checks = [(sums, torch.float64, pairs), (state, torch.int32, (n,)),
              (c, torch.float32, (n,)), (acc, torch.float32, (n,))]
    if offsets is not None:
        checks.append((offsets, torch.int64, (n + 1,)))
    for t, dt, shape in checks:
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"tdc_decide: expected {dt} {shape} contiguous, got {t.dtype} {tuple(t.shape)}")
    skip = torch.empty(n, dtype=torch.int32, device=state.device) if skip is None else skip
    st = lib.hdq_tdc_decide(_ptr(sums), _ptr(offsets), _ptr(state), _ptr(c), _ptr(acc), _ptr(skip), n,
                            float(tau_skip), float(tau_acc), _stream(stream))
    _check("hdq_tdc_decide", st)
    return skip


def _delta_parts(delta_sums):
    """(pointer, pairs) of a difference-sums argument: None, or float64 with
    an even number of elements -- one pair from delta_sums(), or the chunk
    partials of linear_dispatch_delta()."""
    if delta_sums is None:
        return None, 0
    if delta_sums.dtype != torch.float64 or not delta_sums.is_contiguous() or delta_sums.numel() % 2 or \
            delta_sums.numel() == 0:
        raise ValueError("delta sums: expected contiguous float64 pairs")
    return _ptr(delta_sums), delta_sums.numel() // 2


def select_precision_sums(delta_sums, cur_in, had_block=0, delta_thresh=0.1, ratio_thresh=50.0,
                          decision=None, stats=None, ws=None, stream=None):
    """hdq_select_precision_sums: the selection with the difference sums of
    delta_sums() (None = no history).  Returns (decision, stats)."""
    cur_in = _bf16(cur_in, "cur_in")
    rows, cols = cur_in.shape
    dev = cur_in.device
    decision = torch.empty(1, dtype=torch.int32, device=dev) if decision is None else decision
    stats = torch.empty(5, dtype=torch.float32, device=dev) if stats is None else stats
    ws = _workspace(ws, workspace_bytes(OP_SELECT, rows, cols, 0), dev)
    dp, parts = _delta_parts(delta_sums)
    st = lib.hdq_select_precision_sums(dp, parts, _ptr(cur_in), rows, cols, had_block,
                                       delta_thresh, ratio_thresh, _ptr(decision), _ptr(stats),
                                       _ptr(ws), ws.numel(), _stream(stream))
    _check("hdq_select_precision_sums", st)
    return decision, stats


def select_quantize_int8(delta_sums, cur_in, had_block, delta_thresh=0.1, ratio_thresh=50.0,
                         decision=None, stats=None, out=None, ws=None, stream=None):
    """hdq_select_quantize_int8: the selection (difference sums from
    delta_sums(), None = no history) fused with the INT8 per-token
    quantization of cur_in.  Returns (decision, stats, QuantizedTensor)."""
    cur_in = _bf16(cur_in, "cur_in")
    rows, cols = cur_in.shape
    dev = cur_in.device
    decision = torch.empty(1, dtype=torch.int32, device=dev) if decision is None else decision
    stats = torch.empty(5, dtype=torch.float32, device=dev) if stats is None else stats
    out = QuantizedTensor(FMT_INT8_ROW, rows, cols, had_block, dev) if out is None else out
    ws = _workspace(ws, workspace_bytes(OP_SELECT_Q8, rows, cols, 0), dev)
    d = out.desc()
    dp, parts = _delta_parts(delta_sums)
    st = lib.hdq_select_quantize_int8(dp, parts, _ptr(cur_in), rows, cols, had_block,
                                      delta_thresh, ratio_thresh, _ptr(decision), _ptr(stats),
                                      _c.byref(d), _ptr(ws), ws.numel(), _stream(stream))
    _check("hdq_select_quantize_int8", st)
    out.fmt, out.had_block, out.rows, out.cols = d.fmt, d.had_block, d.rows, d.cols
    return decision, stats, out


def select_quantize_int8_noalloc(delta_sums, cur_in, had_block, decision, stats, out, delta_thresh=0.1,
                                 ratio_thresh=50.0, stream=None):
    """hdq_select_quantize_int8_noalloc: select_quantize_int8 with the
    library's fixed per-GPU scratch instead of a workspace; the caller passes
    every output (decision int32[1], stats float32[5], an INT8 QuantizedTensor),
    so the call allocates nothing."""
    cur_in = _bf16(cur_in, "cur_in")
    rows, cols = cur_in.shape
    d = out.desc()
    dp, parts = _delta_parts(delta_sums)
    st = lib.hdq_select_quantize_int8_noalloc(dp, parts, _ptr(cur_in), rows, cols, had_block,
                                              delta_thresh, ratio_thresh, _ptr(decision), _ptr(stats),
                                              _c.byref(d), _stream(stream))
    _check("hdq_select_quantize_int8_noalloc", st)
    out.fmt, out.had_block, out.rows, out.cols = d.fmt, d.had_block, d.rows, d.cols
    return decision, stats, out


def quantize(x, had_block, fmt, tensor_amax=None, out=None, ws=None, stream=None, decision=None,
             decoded=False):
    """hdq_quantize: rotate + quantize a bf16 [rows, cols] tensor (only when
    the device decision matches the format's precision, if one is given).
    decoded: a new output also gets the NVFP4 codes' exact bf16 values."""
    x = _bf16(x, "x")
    rows, cols = x.shape
    out = QuantizedTensor(fmt, rows, cols, had_block, x.device, decoded) if out is None else out
    d = out.desc()
    nbytes = workspace_bytes(OP_QUANTIZE, rows, cols, 0, fmt) if tensor_amax is None else 0
    ws = _workspace(ws, nbytes, x.device)
    st = lib.hdq_quantize(_ptr(x), rows, cols, had_block, fmt, _ptr(tensor_amax), _ptr(decision),
                          _c.byref(d),
                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check("hdq_quantize", st)
    return out


# ---- DeltaQuant cube-delta quantization --------------------------------------

def dq_cubes(grid):
    """Cubes of grid = (frames, height, width, (cube_f, cube_h, cube_w))."""
    n = lib.hdq_dq_cubes(_c.byref(_dq_grid(grid)))
    if n < 0:
        raise ValueError(f"bad DeltaQuant grid {grid}")
    return n


def _dq_grid(grid):
    F, H, W, (cf, ch, cw) = grid
    return DqGridDesc(F, H, W, cf, ch, cw)


def dq_core_needs_bf16(fmt, cubes, K, N=None):
    """Whether hdq_dq_linear's core GEMM runs on the bf16 core values and
    decoded weights: unless the weights' block scales are powers of two (MX
    or per-16 format), K % 128 == 0, and the core codes and (N given) the
    FP4 weight codes fit 32-bit offsets -- the library's own rule."""
    fits = cubes * K < 2 ** 31 and (N is None or N * K // 2 < 2 ** 31)
    return not (fmt in (FMT_NVFP4_MX, FMT_NVFP4_P2) and K % 128 == 0 and fits)


class DqActivations:
    """hdq_dq_quantize's outputs: core codes [cubes, K], core scales [cubes],
    the differences' NVFP4 tensor and, when asked for (by default when the
    core GEMM needs them, see dq_core_needs_bf16), the core code values as
    bf16 [cubes, K]."""

    def __init__(self, grid, K, fmt, device, core_bf16=None):
        self.grid, self.K = grid, K
        n, M = dq_cubes(grid), grid[0] * grid[1] * grid[2]
        self.core = torch.empty(n, K, dtype=torch.uint8, device=device)
        self.core_scale = torch.empty(n, dtype=torch.float32, device=device)
        want = dq_core_needs_bf16(fmt, n, K) if core_bf16 is None else core_bf16
        self.core_bf16 = torch.empty(n, K, dtype=torch.bfloat16, device=device) if want else None
        self.delta = QuantizedTensor(fmt, M, K, 1, device)


def dq_quantize(x, grid, fmt, out=None, ws=None, stream=None, core_bf16=None):
    """hdq_dq_quantize: cube cores in FP8 and the differences in NVFP4."""
    x = _bf16(x, "x")
    M, K = x.shape
    out = DqActivations(grid, K, fmt, x.device, core_bf16) if out is None else out
    ws = _workspace(ws, workspace_bytes(OP_DQ_QUANTIZE, M, K), x.device)
    d = out.delta.desc()
    st = lib.hdq_dq_quantize(_ptr(x), K, _c.byref(_dq_grid(grid)), fmt, _ptr(out.core), _ptr(out.core_scale),
                             _ptr(out.core_bf16), _c.byref(d), _ptr(ws), ws.numel(), _stream(stream))
    _check("hdq_dq_quantize", st)
    return out


def dq_decode_weights(w_fp4, stream=None):
    """hdq_dq_decode_weights: bf16 [N, K] of E2M1 x block scale."""
    out = torch.empty(w_fp4.rows, w_fp4.cols, dtype=torch.bfloat16, device=w_fp4.codes.device)
    d = w_fp4.desc()
    _check("hdq_dq_decode_weights", lib.hdq_dq_decode_weights(_c.byref(d), _ptr(out), _stream(stream)))
    return out


def dq_linear_workspace_bytes(grid, K, N, fmt):
    """hdq_dq_linear_workspace_bytes: the scratch hdq_dq_linear needs on its route."""
    return lib.hdq_dq_linear_workspace_bytes(_c.byref(_dq_grid(grid)), K, N, fmt)


def dq_linear(a, w_fp4, w_dec=None, y=None, y_dtype=DTYPE_BF16, ws=None, stream=None):
    """hdq_dq_linear: y = differences x W^T + cube cores x W^T.  w_dec and
    the activations' bf16 core values are needed only when the core GEMM runs
    in bf16 (dq_core_needs_bf16 with N: plain NVFP4, K % 128 != 0, or codes
    past 32-bit offsets); the library returns HDQ_ERR_INVALID without them."""
    M, N = a.delta.rows, w_fp4.rows
    if y is None:
        dt = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}[y_dtype]
        y = torch.empty(M, N, dtype=dt, device=a.core.device)
    ws = _workspace(ws, dq_linear_workspace_bytes(a.grid, a.delta.cols, N, a.delta.fmt), a.core.device)
    dd, wd = a.delta.desc(), w_fp4.desc()
    st = lib.hdq_dq_linear(_c.byref(_dq_grid(a.grid)), _ptr(a.core), _ptr(a.core_bf16), _ptr(a.core_scale), _c.byref(dd),
                           _c.byref(wd), _ptr(w_dec), _ptr(y), y_dtype, _ptr(ws), ws.numel(), _stream(stream))
    _check("hdq_dq_linear", st)
    return y


class LinearWeights:
    """A linear layer's weights in every form a precision may need:
    bf16 (unrotated, for the full-precision fallback), INT4 per output
    channel, and NVFP4 (or its MX-compatible variant).  fp4_decoded: the
    NVFP4 weights also as their exact bf16 values (N x K x 2 bytes), which
    the plain-NVFP4 GEMM reads when the activations carry theirs too."""

    def __init__(self, w_bf16, had_block, fp4_fmt=FMT_NVFP4, keep_bf16=True, stream=None, fp4_decoded=False):
        w_bf16 = _bf16(w_bf16, "w")
        self.N, self.K = w_bf16.shape
        self.had_block = had_block
        self.w_bf16 = w_bf16 if keep_bf16 else None
        self.w_int4 = quantize(w_bf16, had_block, FMT_INT4_ROW, stream=stream)
        self.w_fp4 = (quantize(w_bf16, had_block, fp4_fmt, stream=stream, decoded=fp4_decoded)
                      if fp4_fmt is not None else None)

    def desc(self):
        empty = QTensorDesc(-1, 0, 0, 0, None, None, None, None, None)
        return WeightsDesc(self.N, self.K, _ptr(self.w_bf16), self.w_int4.desc(),
                           self.w_fp4.desc() if self.w_fp4 is not None else empty)


def linear(precision, x, w, decision=None, xq=None, x_amax=None, y=None, y_dtype=DTYPE_BF16,
           ws=None, stream=None):
    """hdq_linear: Y[M, N] = quantized X[M, K] @ W^T.  precision -1 reads the
    decision tensor on the device; a fixed precision with a decision tensor
    runs only when the device decision equals it."""
    if x is not None:
        x = _bf16(x, "x")
        M, K = x.shape
        dev = x.device
    else:
        M, K = xq.rows, xq.cols
        dev = xq.codes.device
    if y is None:
        dt = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16, DTYPE_I32: torch.int32}[y_dtype]
        y = torch.empty(M, w.N, dtype=dt, device=dev)
    wd = w.desc()
    fp4_fmt = w.w_fp4.fmt if w.w_fp4 is not None else -1
    nbytes = 0 if xq is not None else workspace_bytes(OP_LINEAR, M, K, w.N, fp4_fmt)
    ws = _workspace(ws, nbytes, dev)
    xqd = xq.desc() if xq is not None else None
    st = lib.hdq_linear(precision, _ptr(decision), _ptr(x), _c.byref(xqd) if xqd is not None else None,
                        _ptr(x_amax), M, K, _c.byref(wd), _ptr(y), y_dtype, _ptr(ws),
                        0 if ws is None else ws.numel(), _stream(stream))
    _check("hdq_linear", st)
    return y
