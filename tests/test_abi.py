"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/hdq.h declares, and rejects bad arguments on the host before any
launch (so these calls never touch a GPU).  Also checks that the product
path never reaches the oracle."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hdq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hdq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def hdq():
    from bit_quantized_video_amd import hdq as H
    return H


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("hdq_select_precision", "hdq_delta_sums", "hdq_select_precision_sums",
               "hdq_select_quantize_int8", "hdq_select_quantize_int8_noalloc", "hdq_quantize", "hdq_tdc_decide",
               "hdq_linear", "hdq_linear_dispatch", "hdq_workspace_bytes",
               "hdq_status_string", "hdq_version", "hdq_dq_cubes", "hdq_dq_quantize",
               "hdq_dq_decode_weights", "hdq_dq_linear"):
        assert fn in names


def test_binding_structs_match_the_header(hdq, tmp_path):
    """Every struct the binding passes has the header's members, in order, at
    the offsets a C compiler gives them (gcc on the header itself)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    structs = {"hdq_qtensor": hdq.QTensorDesc, "hdq_weights": hdq.WeightsDesc,
               "hdq_delta_slice": hdq.DeltaSlice, "hdq_dq_grid": hdq.DqGridDesc}
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "hdq.h"', "int main(void) {"]
    for cname, cls in structs.items():
        body = re.search(r"typedef struct " + cname + r" \{(.*?)\} " + cname + ";", text, re.S).group(1)
        members = []
        for decl in body.split(";"):
            decl = decl.strip()
            if decl:
                head, *rest = decl.split(",")
                members.append(head.split()[-1].lstrip("*"))
                members += [r.strip().lstrip("*") for r in rest]
        assert members == [f[0] for f in cls._fields_], cname
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for m in members:
            lines.append(f'printf("{cname}.{m} %zu\\n", offsetof({cname}, {m}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for m, _ in cls._fields_:
            assert int(got[f"{cname}.{m}"]) == getattr(cls, m).offset, (cname, m)


def test_library_exports_every_declared_symbol(hdq):
    lib = ctypes.CDLL(hdq.LIB_PATH)
    for fn in declared_functions():
        assert hasattr(lib, fn), fn
    assert set(hdq.EXPORTS) == set(declared_functions())


def test_status_strings_and_version(hdq):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert hdq.lib.hdq_status_string(st)
    assert hdq.lib.hdq_status_string(99) == b"unknown status"
    assert hdq.lib.hdq_version() >= 10000


def test_workspace_sizes(hdq):
    M, K = 17776, 3072
    sel = hdq.workspace_bytes(hdq.OP_SELECT, M, K, M * K)
    assert sel >= 1024 * 6 * 8
    assert hdq.workspace_bytes(hdq.OP_QUANTIZE, M, K, 0, hdq.FMT_INT8_ROW) == 0
    assert hdq.workspace_bytes(hdq.OP_QUANTIZE, M, K, 0, hdq.FMT_NVFP4) > 0
    int8 = hdq.workspace_bytes(hdq.OP_LINEAR, M, K, 9216, -1)
    both = hdq.workspace_bytes(hdq.OP_LINEAR, M, K, 9216, hdq.FMT_NVFP4)
    assert int8 >= M * K + 4 * M
    assert both >= int8 + M * K // 2 + M * K // 16
    assert hdq.workspace_bytes(hdq.OP_LINEAR, 0, K, 1, -1) == 0
    assert hdq.workspace_bytes(7, M, K, 1, -1) == 0


def test_validation_happens_before_any_launch(hdq):
    L = hdq.lib
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation
    # select: null cur / decision, one-sided history, bad block, missing workspace
    assert L.hdq_select_precision(None, None, 0, None, 4, 64, 0, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_INVALID
    assert L.hdq_select_precision(fake, None, 8, fake, 4, 64, 0, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_INVALID
    assert L.hdq_select_precision(None, None, 0, fake, 4, 64, 48, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_select_precision(None, None, 0, fake, 4, 60, 16, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_select_precision(None, None, 0, fake, 0, 64, 0, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_select_precision(None, None, 0, fake, 4, 64, 0, 0.1, 50.0, fake, fake, None, 0, None) == hdq.ERR_WORKSPACE
    # the two-part selection: null tensors, bad sizes, missing workspace
    assert L.hdq_delta_sums(None, fake, 64, fake, fake, 1 << 20, None) == hdq.ERR_INVALID
    assert L.hdq_delta_sums(fake, fake, 64, None, fake, 1 << 20, None) == hdq.ERR_INVALID
    assert L.hdq_delta_sums(fake, fake, 0, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_delta_sums(fake, fake, 64, fake, None, 0, None) == hdq.ERR_WORKSPACE
    assert L.hdq_select_precision_sums(fake, 1, None, 4, 64, 0, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_INVALID
    assert L.hdq_select_precision_sums(None, 0, fake, 4, 64, 0, 0.1, 50.0, None, fake, fake, 1 << 20, None) == hdq.ERR_INVALID
    assert L.hdq_select_precision_sums(None, 0, fake, 4, 60, 16, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_select_precision_sums(None, 0, fake, 0, 64, 0, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_select_precision_sums(fake, 0, fake, 4, 64, 0, 0.1, 50.0, fake, fake, fake, 1 << 20, None) == hdq.ERR_SHAPE
    assert L.hdq_select_precision_sums(fake, 1, fake, 4, 64, 0, 0.1, 50.0, fake, fake, None, 0, None) == hdq.ERR_WORKSPACE
    # selection fused with INT8 quantization: no rotation, bad shapes, missing buffers or workspace
    q8 = hdq.QTensorDesc(0, 0, 0, 0, fake, fake, None, None)
    sq = lambda hb=16, cols=64, rows=4, q=q8, ws=fake, wsb=1 << 20, ds=None, parts=0: L.hdq_select_quantize_int8(
        ds, parts, fake, rows, cols, hb, 0.1, 50.0, fake, fake, ctypes.byref(q) if q is not None else None, ws,
        wsb, None)
    assert sq(q=None) == hdq.ERR_INVALID
    assert sq(q=hdq.QTensorDesc(0, 0, 0, 0, None, fake, None, None)) == hdq.ERR_INVALID
    assert sq(hb=0) == hdq.ERR_SHAPE
    assert sq(hb=12) == hdq.ERR_SHAPE
    assert sq(rows=0) == hdq.ERR_SHAPE
    assert sq(ws=None, wsb=0) == hdq.ERR_WORKSPACE
    assert sq(rows=100000, wsb=1 << 20) == hdq.ERR_WORKSPACE      # one partial per row does not fit
    assert sq(ds=fake, parts=0) == hdq.ERR_SHAPE                  # difference sums need >= 1 pair
    assert L.hdq_workspace_bytes(hdq.OP_SELECT_Q8, 17776, 3072, 0, 0) >= 17776 * 48
    # the allocation-free variant: the same checks, then the fixed scratch's limit (before any HIP call)
    nq = lambda hb=16, cols=64, rows=4, q=q8, dec=fake: L.hdq_select_quantize_int8_noalloc(
        None, 0, fake, rows, cols, hb, 0.1, 50.0, dec, fake, ctypes.byref(q) if q is not None else None, None)
    assert nq(q=None) == hdq.ERR_INVALID
    assert nq(dec=None) == hdq.ERR_INVALID
    assert nq(hb=0) == hdq.ERR_SHAPE
    assert nq(cols=60) == hdq.ERR_SHAPE
    max_rows = hdq.NOALLOC_SCRATCH_BYTES // 48
    assert nq(rows=max_rows + 1) == hdq.ERR_TOO_LARGE
    assert nq(rows=17776 * 4, cols=12288) == hdq.ERR_TOO_LARGE
    assert L.hdq_workspace_bytes(hdq.OP_SELECT_Q8, max_rows, 64, 0, 0) <= hdq.NOALLOC_SCRATCH_BYTES
    # quantize: bad fmt, bad shapes, missing buffers, missing workspace for the amax pre-pass
    q = hdq.QTensorDesc(0, 0, 0, 0, fake, fake, fake, fake)
    assert L.hdq_quantize(fake, 4, 64, 16, 9, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_INVALID
    assert L.hdq_quantize(fake, 4, 64, 12, 0, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_SHAPE
    assert L.hdq_quantize(fake, 4, 64, 256, 0, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_SHAPE
    assert L.hdq_quantize(fake, 4, 72, 16, 0, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_SHAPE
    assert L.hdq_quantize(fake, 4, 48, 16, hdq.FMT_NVFP4_MX, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_SHAPE
    assert L.hdq_quantize(fake, 4, 72, 8, hdq.FMT_NVFP4_P2, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_SHAPE
    assert L.hdq_quantize(fake, 4, 64, 16, hdq.FMT_NVFP4_P2 + 1, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_INVALID
    assert L.hdq_quantize(fake, 4, 64, 16, hdq.FMT_NVFP4, None, None, ctypes.byref(q), None, 0, None) == hdq.ERR_WORKSPACE
    q0 = hdq.QTensorDesc(0, 0, 0, 0, None, fake, fake, fake)
    assert L.hdq_quantize(fake, 4, 64, 16, 0, None, None, ctypes.byref(q0), None, 0, None) == hdq.ERR_INVALID
    # a decision gate makes no sense for weight (INT4) quantization
    assert L.hdq_quantize(fake, 4, 64, 16, hdq.FMT_INT4_ROW, None, fake, ctypes.byref(q), None, 0, None) == hdq.ERR_UNSUPPORTED
    # linear: descriptor mismatches
    w4 = hdq.QTensorDesc(hdq.FMT_INT4_ROW, 16, 32, 64, fake, fake, None, None)
    wf = hdq.QTensorDesc(hdq.FMT_NVFP4, 16, 32, 64, fake, None, fake, fake)
    w = hdq.WeightsDesc(32, 64, fake, w4, wf)
    ok = lambda prec, **kw: L.hdq_linear(prec, kw.get("dec"), kw.get("x", fake), kw.get("xq"), None,
                                         kw.get("M", 8), kw.get("K", 64), ctypes.byref(kw.get("w", w)),
                                         fake, kw.get("dt", 1), kw.get("ws", None), kw.get("wsb", 0), None)
    assert ok(5) == hdq.ERR_INVALID
    assert ok(-1) == hdq.ERR_INVALID                       # needs a decision pointer
    assert ok(1, K=32) == hdq.ERR_SHAPE                    # w.K != K
    assert ok(1, dt=2, x=fake) == hdq.ERR_WORKSPACE        # int8 needs room for the codes
    assert ok(0, dt=2) == hdq.ERR_UNSUPPORTED              # int32 output only on the INT8 path
    assert ok(2, x=None) == hdq.ERR_INVALID                # bf16 needs x
    assert ok(2, xq=ctypes.byref(hdq.QTensorDesc(hdq.FMT_INT8_ROW, 16, 8, 64, fake, fake, None, None))) == hdq.ERR_UNSUPPORTED
    bad4 = hdq.WeightsDesc(32, 64, fake, hdq.QTensorDesc(hdq.FMT_INT8_ROW, 16, 32, 64, fake, fake, None, None), wf)
    assert ok(1, w=bad4) == hdq.ERR_UNSUPPORTED
    badfp = hdq.WeightsDesc(32, 64, fake, w4, hdq.QTensorDesc(hdq.FMT_NVFP4, 16, 31, 64, fake, None, fake, fake))
    assert ok(0, w=badfp) == hdq.ERR_SHAPE
    xq = hdq.QTensorDesc(hdq.FMT_INT8_ROW, 32, 8, 64, fake, fake, None, None)
    assert ok(1, xq=ctypes.byref(xq)) == hdq.ERR_SHAPE     # block differs from the weights'
    # TDC rule: null pointers, bad module count
    assert L.hdq_tdc_decide(None, None, fake, fake, fake, fake, 4, 0.05, 0.15, None) == hdq.ERR_INVALID
    assert L.hdq_tdc_decide(fake, fake, fake, fake, fake, None, 4, 0.05, 0.15, None) == hdq.ERR_INVALID
    assert L.hdq_tdc_decide(fake, None, fake, fake, fake, fake, 0, 0.05, 0.15, None) == hdq.ERR_SHAPE
    assert L.hdq_tdc_decide(fake, fake, fake, fake, fake, fake, 1 << 31, 0.05, 0.15, None) == hdq.ERR_SHAPE
    # one-launch linear: every operand the decision may pick must be present and consistent
    x8 = hdq.QTensorDesc(hdq.FMT_INT8_ROW, 16, 8, 64, fake, fake, None, None)
    x4 = hdq.QTensorDesc(hdq.FMT_NVFP4, 16, 8, 64, fake, None, fake, fake)
    dsp = lambda **kw: L.hdq_linear_dispatch(
        kw.get("dec", fake), kw.get("x", fake), ctypes.byref(kw.get("x8", x8)), ctypes.byref(kw.get("x4", x4)),
        kw.get("M", 8), kw.get("K", 64), ctypes.byref(kw.get("w", w)), fake, kw.get("dt", 1), None)
    assert dsp(dec=None) == hdq.ERR_INVALID                 # the decision is read on the device
    assert dsp(x=None) == hdq.ERR_INVALID                   # the bf16 choice needs x
    assert dsp(dt=2) == hdq.ERR_UNSUPPORTED                 # int32 output has no one-launch form
    assert dsp(M=0) == hdq.ERR_SHAPE
    assert dsp(K=32) == hdq.ERR_SHAPE                       # w.K != K
    assert dsp(x8=hdq.QTensorDesc(hdq.FMT_INT8_ROW, 16, 7, 64, fake, fake, None, None)) == hdq.ERR_SHAPE
    assert dsp(x8=hdq.QTensorDesc(hdq.FMT_INT8_ROW, 32, 8, 64, fake, fake, None, None)) == hdq.ERR_SHAPE
    assert dsp(x4=hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 16, 8, 64, fake, None, fake, fake)) == hdq.ERR_UNSUPPORTED
    assert dsp(w=bad4) == hdq.ERR_UNSUPPORTED
    assert dsp(w=hdq.WeightsDesc(32, 64, None, w4, wf)) == hdq.ERR_INVALID
    # the one-launch linear with difference chunks: slice count, tensors, chunk ranges, shapes
    x4mx = hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 16, 8, 256, fake, None, fake, fake)
    w256 = hdq.WeightsDesc(32, 256, fake, hdq.QTensorDesc(hdq.FMT_INT4_ROW, 16, 32, 256, fake, fake, None, None),
                           hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 16, 32, 256, fake, None, fake, fake))
    x8k = hdq.QTensorDesc(hdq.FMT_INT8_ROW, 16, 8, 256, fake, fake, None, None)
    big = ctypes.c_void_p(0x100000)   # 16-byte aligned stand-ins, never dereferenced

    def dd(sl=None, n=1, queue=fake, K=256, w=w256):
        sl = sl if sl is not None else hdq.DeltaSlice(big, big, 1 << 17, 0, 2, big)
        arr = (hdq.DeltaSlice * 1)(sl)
        return L.hdq_linear_dispatch_delta(fake, fake, ctypes.byref(x8k), ctypes.byref(x4mx), 8, K,
                                           ctypes.byref(w), fake, 1, arr, n, queue, None)
    assert dd(n=-1) == hdq.ERR_SHAPE
    assert dd(n=hdq.DELTA_MAX_SLICES + 1) == hdq.ERR_SHAPE
    assert dd(queue=None) == hdq.ERR_INVALID
    assert dd(sl=hdq.DeltaSlice(None, big, 1 << 17, 0, 2, big)) == hdq.ERR_INVALID
    assert dd(sl=hdq.DeltaSlice(big, big, 1 << 17, 0, 2, None)) == hdq.ERR_INVALID
    assert dd(sl=hdq.DeltaSlice(big, big, 100, 0, 1, big)) == hdq.ERR_SHAPE        # numel % 8
    assert dd(sl=hdq.DeltaSlice(big, big, 1 << 17, 0, 3, big)) == hdq.ERR_SHAPE    # past the last chunk
    assert dd(sl=hdq.DeltaSlice(big, big, 1 << 17, 2, 1, big)) == hdq.ERR_SHAPE    # begin > end
    assert dd(sl=hdq.DeltaSlice(ctypes.c_void_p(0x100008), big, 1 << 17, 0, 2, big)) == hdq.ERR_SHAPE  # alignment
    w64 = hdq.WeightsDesc(32, 64, fake, w4, hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 16, 32, 64, fake, None, fake, fake))
    assert dd(K=64, w=w64) == hdq.ERR_SHAPE                 # only the one-launch kernel's shapes


def test_deltaquant_validation(hdq):
    """DeltaQuant entry points: grid, format, shape and workspace checks (no
    kernel runs: every call fails before a launch)."""
    L = hdq.lib
    fake = ctypes.c_void_p(0x1000)
    g = hdq.DqGridDesc(3, 5, 7, 2, 2, 2)
    assert L.hdq_dq_cubes(ctypes.byref(g)) == 2 * 3 * 4
    assert L.hdq_dq_cubes(ctypes.byref(hdq.DqGridDesc(3, 5, 7, 0, 2, 2))) == -1
    assert L.hdq_dq_cubes(None) == -1
    assert L.hdq_dq_cubes(ctypes.byref(hdq.DqGridDesc(13, 30, 45, 8, 8, 8))) == -1   # > 256 tokens per cube
    M, K = 105, 64
    delta = hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, M, K, fake, None, fake, fake)
    q = lambda x=fake, K=K, g=g, fmt=hdq.FMT_NVFP4_MX, d=delta, ws=fake, wsb=256: L.hdq_dq_quantize(
        x, K, ctypes.byref(g), fmt, fake, fake, None, ctypes.byref(d), ws, wsb, None)
    assert q(x=None) == hdq.ERR_INVALID
    assert q(fmt=hdq.FMT_INT8_ROW) == hdq.ERR_UNSUPPORTED
    assert q(K=48) == hdq.ERR_SHAPE
    assert q(g=hdq.DqGridDesc(3, 5, 0, 2, 2, 2)) == hdq.ERR_SHAPE
    assert q(d=hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 16, M, K, fake, None, fake, fake)) == hdq.ERR_SHAPE
    assert q(d=hdq.QTensorDesc(hdq.FMT_NVFP4, 1, M, K, fake, None, fake, fake)) == hdq.ERR_SHAPE
    assert q(d=hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, M, K, fake, None, None, fake)) == hdq.ERR_INVALID
    assert q(wsb=255) == hdq.ERR_WORKSPACE
    assert L.hdq_workspace_bytes(hdq.OP_DQ_QUANTIZE, M, K, 0, 0) == 256
    N, C = 40, 24
    need = L.hdq_workspace_bytes(hdq.OP_DQ_LINEAR, M, C, N, 0)
    assert need >= (M * N + C * N) * 4
    w = hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, N, K, fake, None, fake, fake)
    lin = lambda d=delta, w=w, dt=1, ws=fake, wsb=need, cc=fake, cb=fake, wd=fake: L.hdq_dq_linear(
        ctypes.byref(g), cc, cb, fake, ctypes.byref(d), ctypes.byref(w), wd, fake, dt, ws, wsb, None)
    assert lin(dt=2) == hdq.ERR_UNSUPPORTED
    assert lin(w=hdq.QTensorDesc(hdq.FMT_NVFP4, 1, N, K, fake, None, fake, fake)) == hdq.ERR_UNSUPPORTED
    assert lin(w=hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, 42, K, fake, None, fake, fake)) == hdq.ERR_SHAPE
    assert lin(w=hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 2, N, K, fake, None, fake, fake)) == hdq.ERR_SHAPE
    assert lin(d=hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, M + 1, K, fake, None, fake, fake)) == hdq.ERR_SHAPE
    assert lin(wsb=need - 1) == hdq.ERR_WORKSPACE
    # the route's exact scratch: the fused core-add route (MX or P2, K % 256 == 0) needs only the
    # core GEMM's fp32 [cubes, N]; the combine route also the difference GEMM's fp32 [tokens, N]
    big = hdq.DqGridDesc(13, 30, 45, 2, 2, 2)
    toks, cubes = 13 * 30 * 45, L.hdq_dq_cubes(ctypes.byref(big))
    fused = L.hdq_dq_linear_workspace_bytes(ctypes.byref(big), 3072, 12288, hdq.FMT_NVFP4_MX)
    assert fused == L.hdq_dq_linear_workspace_bytes(ctypes.byref(big), 3072, 12288, hdq.FMT_NVFP4_P2)
    assert cubes * 12288 * 4 <= fused < cubes * 12288 * 4 + 256
    combine = L.hdq_dq_linear_workspace_bytes(ctypes.byref(big), 3072, 12288, hdq.FMT_NVFP4)
    assert combine >= fused + toks * 12288 * 4
    assert L.hdq_dq_linear_workspace_bytes(ctypes.byref(big), 3072 + 32, 12288, hdq.FMT_NVFP4_MX) >= combine
    assert L.hdq_dq_linear_workspace_bytes(ctypes.byref(big), 3072, 12288, hdq.FMT_INT8_ROW) == 0
    assert L.hdq_workspace_bytes(hdq.OP_DQ_LINEAR, toks, cubes, 12288, 0) >= combine
    # K 256 (MX): the fused route; its exact need is accepted by the checks, one byte less is not
    K2 = 256
    d2 = hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, M, K2, fake, None, fake, fake)
    w2 = hdq.QTensorDesc(hdq.FMT_NVFP4_MX, 1, N, K2, fake, None, fake, fake)
    need2 = L.hdq_dq_linear_workspace_bytes(ctypes.byref(g), K2, N, hdq.FMT_NVFP4_MX)
    assert need2 < need
    assert lin(d=d2, w=w2, wsb=need2 - 1) == hdq.ERR_WORKSPACE
    # which buffers each core-GEMM route needs: K 256 with MX runs on the FP8 codes (the bf16 values
    # and decoded weights may be NULL, the codes may not); K 64, or plain NVFP4, on the bf16 values
    assert lin(d=d2, w=w2, wsb=need2 - 1, cb=None, wd=None) == hdq.ERR_WORKSPACE   # accepted, then stopped
    assert lin(d=d2, w=w2, cc=None) == hdq.ERR_INVALID
    assert lin(cb=None) == hdq.ERR_INVALID
    assert lin(wd=None) == hdq.ERR_INVALID
    assert lin(cc=None, wsb=need - 1) == hdq.ERR_WORKSPACE                          # codes unused at K 64
    # more rejections before any launch: cubes over 256 tokens, K over 32768, a bad grid
    big_cube = hdq.DqGridDesc(13, 30, 45, 8, 8, 8)
    assert L.hdq_dq_quantize(fake, K, ctypes.byref(big_cube), hdq.FMT_NVFP4_MX, fake, fake, None,
                             ctypes.byref(delta), fake, 256, None) == hdq.ERR_SHAPE
    assert L.hdq_dq_linear(ctypes.byref(big_cube), fake, fake, fake, ctypes.byref(delta), ctypes.byref(w), fake, fake, 1,
                           fake, need, None) == hdq.ERR_SHAPE
    assert q(K=32768 + 32) == hdq.ERR_SHAPE
    assert L.hdq_dq_linear_workspace_bytes(ctypes.byref(big_cube), K, N, hdq.FMT_NVFP4_MX) == 0
    assert L.hdq_dq_decode_weights(None, fake, None) == hdq.ERR_INVALID


def test_product_path_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "bit_quantized_video_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="replace").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|liboracle|\borc_[a-z]", text, re.M), f
