"""Python view of the CPU oracle (hdq_oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import
this module.  It never imports the GPU package and the GPU package never
imports it.  Arrays are numpy: bf16 tensors travel as uint16 bit patterns.
The C source cites, per function, the passage of the pages it follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_p = ctypes.c_void_p

# decision codes returned by decide()
NVFP4, INT8, BF16 = 0, 1, 2


def lib():
    """Load liboracle.so, compiling it first if it is missing or stale."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        sig = {
            "orc_bf16_to_f32": (_f32, [ctypes.c_uint16]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [_f32]),
            "orc_f32_to_bf16_array": (None, [_p, _i64, _p]),
            "orc_hadamard_sign": (_int, [_int, _int]),
            "orc_hadamard_scale": (_f32, [_int]),
            "orc_rotate_dense_f64": (None, [_p, _i64, _i64, _int, _p]),
            "orc_rotate_f32": (None, [_p, _i64, _i64, _int, _p]),
            "orc_rotated_amax": (_f32, [_p, _i64, _i64, _int]),
            "orc_e2m1_decode": (_f32, [ctypes.c_uint8]),
            "orc_e2m1_encode": (ctypes.c_uint8, [_f32]),
            "orc_e4m3_decode": (_f32, [ctypes.c_uint8]),
            "orc_e4m3_encode": (ctypes.c_uint8, [_f32]),
            "orc_quant_int_rotated": (None, [_p, _i64, _i64, _int, _p, _p]),
            "orc_quant_int": (None, [_p, _i64, _i64, _int, _int, _p, _p]),
            "orc_pack_int4": (None, [_p, _i64, _i64, _p]),
            "orc_unpack_int4": (None, [_p, _i64, _i64, _p]),
            "orc_quant_nvfp4_rotated": (None, [_p, _i64, _i64, _f32, _int, _p, _p, _p]),
            "orc_quant_nvfp4": (None, [_p, _i64, _i64, _int, _f32, _int, _p, _p, _p]),
            "orc_dequant_nvfp4": (None, [_p, _p, _f32, _i64, _i64, _p]),
            "orc_gemm_int": (None, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p]),
            "orc_gemm_nvfp4": (None, [_p, _p, _f32, _p, _p, _f32, _i64, _i64, _i64, _p]),
            "orc_gemm_bf16": (None, [_p, _p, _i64, _i64, _i64, _p]),
            "orc_stats": (None, [_p, _p, _i64, _p, _i64, _i64, _int, _p]),
            "orc_decide": (_int, [_int, _f64, _f64, _f64, _f64]),
            "orc_tdc_decide": (None, [_p, _p, _p, _p, _p, _i64, _f32, _f32]),
            "orc_num_threads": (_int, []),
            "orc_set_num_threads": (None, [_int]),
            "orc_dq_cube_of": (None, [_i64, _i64, _i64, _int, _int, _int, _p]),
            "orc_e4m3s_decode": (_f32, [ctypes.c_uint8]),
            "orc_dq_core": (None, [_p, _i64, _i64, _i64, _i64, _int, _int, _int, _p, _p]),
            "orc_dq_delta": (None, [_p, _i64, _i64, _i64, _i64, _int, _int, _int, _p, _p, _p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _c(a, dtype):
    """Contiguous array of the given dtype (no copy when already so)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(_p) if a is not None else None


def num_threads():
    return lib().orc_num_threads()


def set_num_threads(n):
    """Threads of the GEMM loops from now on (results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- bf16

def bf16_to_f32(x16):
    x16 = _c(x16, np.uint16)
    return (x16.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


# ------------------------------------------------------------ Hadamard

def hadamard_sign(i, j):
    return lib().orc_hadamard_sign(i, j)


def hadamard_matrix(b):
    return np.array([[hadamard_sign(i, j) for j in range(b)] for i in range(b)], np.int64)


def hadamard_scale(b):
    return np.float32(lib().orc_hadamard_scale(b))


def rotate_dense_f64(x, b):
    x = _c(x, np.float64)
    rows, cols = x.shape
    y = np.empty_like(x)
    lib().orc_rotate_dense_f64(_ptr(x), rows, cols, b, _ptr(y))
    return y


def rotate_f32(x16, b):
    x16 = _c(x16, np.uint16)
    rows, cols = x16.shape
    y = np.empty((rows, cols), np.float32)
    lib().orc_rotate_f32(_ptr(x16), rows, cols, b, _ptr(y))
    return y


def rotated_amax(x16, b):
    x16 = _c(x16, np.uint16)
    rows, cols = x16.shape
    return np.float32(lib().orc_rotated_amax(_ptr(x16), rows, cols, b))


# -------------------------------------------------------------- codecs

def e2m1_decode(codes):
    codes = np.asarray(codes, np.uint8)
    L = lib()
    return np.array([L.orc_e2m1_decode(int(c)) for c in codes.ravel()],
                    np.float32).reshape(codes.shape)


def e2m1_encode(v):
    v = np.asarray(v, np.float32)
    L = lib()
    return np.array([L.orc_e2m1_encode(float(t)) for t in v.ravel()],
                    np.uint8).reshape(v.shape)


def e4m3_decode(codes):
    codes = np.asarray(codes, np.uint8)
    L = lib()
    return np.array([L.orc_e4m3_decode(int(c)) for c in codes.ravel()],
                    np.float32).reshape(codes.shape)


def e4m3_encode(t):
    t = np.asarray(t, np.float32)
    L = lib()
    return np.array([L.orc_e4m3_encode(float(v)) for v in t.ravel()],
                    np.uint8).reshape(t.shape)


# ---------------------------------------------------------- quantizers

def quant_int_rotated(y, qmax):
    y = _c(y, np.float32)
    rows, cols = y.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    lib().orc_quant_int_rotated(_ptr(y), rows, cols, qmax, _ptr(q), _ptr(s))
    return q, s


def quant_int(x16, b, qmax):
    """Rotate then quantize rows symmetrically (qmax 127: INT8, 7: INT4).
    Returns (codes int8 [rows, cols], scales float32 [rows])."""
    x16 = _c(x16, np.uint16)
    rows, cols = x16.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    lib().orc_quant_int(_ptr(x16), rows, cols, b, qmax, _ptr(q), _ptr(s))
    return q, s


def pack_int4(q):
    q = _c(q, np.int8)
    rows, cols = q.shape
    p = np.empty((rows, cols // 2), np.uint8)
    lib().orc_pack_int4(_ptr(q), rows, cols, _ptr(p))
    return p


def unpack_int4(p, cols):
    p = _c(p, np.uint8)
    rows = p.shape[0]
    q = np.empty((rows, cols), np.int8)
    lib().orc_unpack_int4(_ptr(p), rows, cols, _ptr(q))
    return q


def quant_nvfp4_rotated(y, amax, mx=0):
    y = _c(y, np.float32)
    rows, cols = y.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    st = np.zeros(1, np.float32)
    lib().orc_quant_nvfp4_rotated(_ptr(y), rows, cols, float(amax), int(mx),
                                  _ptr(codes), _ptr(scales), _ptr(st))
    return codes, scales, np.float32(st[0])


def quant_nvfp4(x16, b, amax=None, mx=0):
    """Rotate then quantize to NVFP4.  mx: 0 plain, 1 (or True) the
    MX-compatible recipe (a power-of-two scale shared by each pair of
    16-blocks), 2 power-of-two scales per 16-block.
    amax=None takes the rotated amax of the rows given.  Returns
    (codes uint8 [rows, cols/2], E4M3 scales uint8 [rows, cols/16], s_t)."""
    x16 = _c(x16, np.uint16)
    rows, cols = x16.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    st = np.zeros(1, np.float32)
    a = -1.0 if amax is None else float(amax)
    lib().orc_quant_nvfp4(_ptr(x16), rows, cols, b, a, int(mx), _ptr(codes),
                          _ptr(scales), _ptr(st))
    return codes, scales, np.float32(st[0])


def dequant_nvfp4(codes, scales, s_t, cols):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = codes.shape[0]
    out = np.empty((rows, cols), np.float32)
    lib().orc_dequant_nvfp4(_ptr(codes), _ptr(scales), float(s_t), rows, cols, _ptr(out))
    return out


# --------------------------------------------------------------- GEMMs

def gemm_int(qa, sa, qw, sw):
    """Integer linear on unpacked codes: returns (y float32 [M,N], acc int64)."""
    qa = _c(qa, np.int8)
    qw = _c(qw, np.int8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.empty((M, N), np.int64)
    y = np.empty((M, N), np.float32)
    lib().orc_gemm_int(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, _ptr(acc), _ptr(y))
    return y, acc


def gemm_nvfp4(ac, ae, ast, wc, we, wst, K):
    ac, ae, wc, we = (_c(a, np.uint8) for a in (ac, ae, wc, we))
    M, N = ac.shape[0], wc.shape[0]
    y = np.empty((M, N), np.float64)
    lib().orc_gemm_nvfp4(_ptr(ac), _ptr(ae), float(ast), _ptr(wc), _ptr(we), float(wst),
                         M, N, K, _ptr(y))
    return y


def gemm_bf16(x16, w16):
    x16 = _c(x16, np.uint16)
    w16 = _c(w16, np.uint16)
    M, K = x16.shape
    N = w16.shape[0]
    y = np.empty((M, N), np.float64)
    lib().orc_gemm_bf16(_ptr(x16), _ptr(w16), M, N, K, _ptr(y))
    return y


# ----------------------------------------------------------- DeltaQuant
# Cube-delta quantization of video tokens (the DeltaQuant abstract on the
# paper-radar CVPR 2026 listing); the readings are stated in hdq_oracle.c.

def dq_cubes(F, H, W, cube):
    cf, ch, cw = cube
    return -(-F // cf) * -(-H // ch) * -(-W // cw)


def dq_cube_of(F, H, W, cube):
    out = np.empty(F * H * W, np.int32)
    lib().orc_dq_cube_of(F, H, W, *cube, _ptr(out))
    return out


def e4m3s_decode(codes):
    """Signed E4M3 bytes to float32."""
    L = lib()
    table = np.array([L.orc_e4m3s_decode(c) for c in range(256)], np.float32)
    return table[np.asarray(codes, np.uint8)]


def dq_core(x16, F, H, W, cube):
    """Core tokens: (signed E4M3 codes uint8 [cubes, K], scales float32 [cubes])."""
    x16 = _c(x16, np.uint16)
    K = x16.shape[1]
    assert x16.shape[0] == F * H * W
    n = dq_cubes(F, H, W, cube)
    codes = np.empty((n, K), np.uint8)
    scale = np.empty(n, np.float32)
    lib().orc_dq_core(_ptr(x16), F, H, W, K, *cube, _ptr(codes), _ptr(scale))
    return codes, scale


def dq_delta(x16, F, H, W, cube, codes, scale):
    """Each token minus its cube's stored core, float32 [F H W, K]."""
    x16 = _c(x16, np.uint16)
    codes = _c(codes, np.uint8)
    scale = _c(scale, np.float32)
    K = x16.shape[1]
    d = np.empty((F * H * W, K), np.float32)
    lib().orc_dq_delta(_ptr(x16), F, H, W, K, *cube, _ptr(codes), _ptr(scale), _ptr(d))
    return d


def dq_quantize(x16, F, H, W, cube, mx=0):
    """The whole activation side: core codes and scales, the differences, and
    their NVFP4 codes, block scales and tensor scale (amax of |difference|).
    Non-finite values (the abstract does not speak of them; this reading):
    when any difference is not finite -- which a NaN or infinite token
    element, or a cube sum or a difference that overflows float32, always
    causes -- the tensor scale is NaN, the flag that the codes (left zero
    here) mean nothing."""
    codes, scale = dq_core(x16, F, H, W, cube)
    d = dq_delta(x16, F, H, W, cube, codes, scale)
    if not np.isfinite(d).all():
        M, K = d.shape
        return dict(core=codes, core_scale=scale, delta=d, delta_amax=np.float32(np.nan),
                    codes=np.zeros((M, K // 2), np.uint8), blk=np.zeros((M, K // 16), np.uint8),
                    s_t=np.float32(np.nan))
    amax = np.float32(np.abs(d).max()) if d.size else np.float32(0)
    dc, de, st = quant_nvfp4_rotated(d, amax, mx)
    return dict(core=codes, core_scale=scale, delta=d, delta_amax=amax, codes=dc, blk=de, s_t=st)


def dq_linear(q, wc, we, wst, K, F, H, W, cube, rows=None):
    """y = (difference codes) x W^T + (its cube's FP8 core) x W^T for every
    token (or the tokens `rows`), float64, W the NVFP4 weights (codes, block
    scales, tensor scale)."""
    rows = np.arange(F * H * W) if rows is None else np.asarray(rows)
    yd = gemm_nvfp4(q["codes"][rows], q["blk"][rows], q["s_t"], wc, we, wst, K)
    wdec = dequant_nvfp4(wc, we, 1.0, K).astype(np.float64)       # e2m1 x block scale, exact
    core = e4m3s_decode(q["core"]).astype(np.float64) * q["core_scale"].astype(np.float64)[:, None]
    yc = (core @ wdec.T) * float(wst)
    return yd + yc[dq_cube_of(F, H, W, cube)[rows]]


# ------------------------------------------------------------ selection

def stats(prev_in16, prev_out16, cur16, b):
    """Returns [delta, ratio, max|x|, mean|x|, rotated amax] (float64)."""
    cur16 = _c(cur16, np.uint16)
    rows, cols = cur16.shape
    out = np.zeros(5, np.float64)
    if prev_in16 is None or prev_out16 is None:
        pi = po = None
        n = 0
    else:
        pi = _c(prev_in16, np.uint16)
        po = _c(prev_out16, np.uint16)
        n = pi.size
    lib().orc_stats(_ptr(pi), _ptr(po), n, _ptr(cur16), rows, cols, b, _ptr(out))
    return out


def decide(has_history, delta, ratio, delta_thresh=0.1, ratio_thresh=50.0):
    return lib().orc_decide(int(bool(has_history)), float(delta), float(ratio),
                            float(np.float32(delta_thresh)), float(np.float32(ratio_thresh)))


# ---------------------------------------------- temporal delta cache

def tdc_decide(sums, state, c, acc, tau_skip=0.05, tau_acc=0.15):
    """One step of the TDC skip rule over n modules (see orc_tdc_decide).
    sums float64 [n, 2], state int32 [n] (0 skipped, 1 computed first, 2
    computed with a previous output), c and acc float32 [n] (updated in
    place).  Returns skip int32 [n] for the next step."""
    sums = _c(sums, np.float64)
    state = _c(state, np.int32)
    assert c.dtype == np.float32 and acc.dtype == np.float32 and c.flags.c_contiguous
    n = state.size
    skip = np.zeros(n, np.int32)
    lib().orc_tdc_decide(_ptr(sums), _ptr(state), _ptr(c), _ptr(acc), _ptr(skip), n,
                         float(np.float32(tau_skip)), float(np.float32(tau_acc)))
    return skip

