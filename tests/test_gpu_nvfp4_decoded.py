"""Plain NVFP4 with decoded operands (hdq_qtensor.dec), through the C ABI.

The exact NVFP4 product runs on bf16 MFMAs.  When the operands carry their
codes' exact bf16 values (E2M1 value x E4M3 block scale, which bf16 holds
exactly) -- both, or the activations only -- the GEMM reads those instead of
decoding the codes while it stages them.  It issues the same MFMAs on the same values in the same order,
so the outputs must equal the codes path bit for bit; the codes path itself
is checked against the oracle in test_gpu_parity.py.

  * decoded values: bit-exact against the format definitions (the OCP E2M1
    table in tests/golden and torch's E4M3 decode), and untouched when the
    device decision gates the quantization off;
  * hdq_linear, hdq_linear_dispatch and hdq_linear_dispatch_delta: output
    bits equal with and without the decoded operands.
"""
import os
import sys

import numpy as np
import pytest
import torch

from bit_quantized_video_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from bit_quantized_video_amd import hdq  # noqa: E402  (loads libhdq.so; fails loudly if missing)

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).to(DEV).view(torch.bfloat16)


def e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if len(line) == 2:
                vals[int(line[0], 16)] = float(line[1])
    # the sign bit (code bit 3) negates, zero included
    return np.array([np.copysign(vals[c & 7], -1.0 if c & 8 else 1.0) for c in range(16)], np.float32)


def expected_decoded(q):
    """bf16 bits of E2M1(code) x E4M3(block scale), from the stored bytes."""
    codes = q.codes.cpu().numpy()
    lo, hi = codes & 15, codes >> 4
    nib = np.empty((q.rows, q.cols), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = lo, hi
    scales = torch.from_numpy(q.blk_scale.cpu().numpy()).view(torch.float8_e4m3fn).float().numpy()
    vals = e2m1_table()[nib] * np.repeat(scales, 16, axis=1)
    bits = vals.astype(np.float32).view(np.uint32)
    assert not np.any(bits & 0xFFFF), "E2M1 x E4M3 must be exact in bf16"
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,K", [(300, 512), (37, 96), (129, 3072)])
@pytest.mark.parametrize("fmt", [hdq.FMT_NVFP4, hdq.FMT_NVFP4_MX])
def test_quantize_writes_exact_decoded_values(M, K, fmt):
    say(f"decoded values fmt={fmt} M={M} K={K}")
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(150, M + K))
    q = hdq.quantize(to_dev(x16), 32, fmt, decoded=True)
    torch.cuda.synchronize()
    got = q.dec.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, expected_decoded(q))


def test_decoded_values_gated_off():
    M, K = 64, 256
    x = to_dev(synth.lognormal_tokens(M, K, synth.rng_for(151, 0)))
    q = hdq.QuantizedTensor(hdq.FMT_NVFP4, M, K, 32, DEV, decoded=True)
    q.dec.view(torch.int16).fill_(0x1234)
    d = torch.full((1,), hdq.PREC_INT8, dtype=torch.int32, device=DEV)
    hdq.quantize(x, 32, hdq.FMT_NVFP4, out=q, decision=d)
    torch.cuda.synchronize()
    assert bool((q.dec.view(torch.int16) == 0x1234).all())
    d.fill_(hdq.PREC_NVFP4)
    hdq.quantize(x, 32, hdq.FMT_NVFP4, out=q, decision=d)
    torch.cuda.synchronize()
    assert np.array_equal(q.dec.view(torch.int16).cpu().numpy().view(np.uint16), expected_decoded(q))


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def operands(M, N, K, seed):
    hb = 32
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(152, seed))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(153, seed))
    xd, wd = to_dev(x16), to_dev(w16)
    W = hdq.LinearWeights(wd, hb, fp4_fmt=hdq.FMT_NVFP4)
    Wd = hdq.LinearWeights(wd, hb, fp4_fmt=hdq.FMT_NVFP4, fp4_decoded=True)
    xq = hdq.quantize(xd, hb, hdq.FMT_NVFP4)
    xqd = hdq.quantize(xd, hb, hdq.FMT_NVFP4, decoded=True)
    return xd, W, Wd, xq, xqd


@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (257, 129, 1024), (64, 640, 3072), (37, 19, 96),
                                   (1000, 600, 192)])
@pytest.mark.parametrize("y_dtype", [hdq.DTYPE_F32, hdq.DTYPE_BF16])
def test_linear_decoded_operands_same_bits(M, N, K, y_dtype):
    say(f"linear decoded M={M} N={N} K={K} y={y_dtype}")
    xd, W, Wd, xq, xqd = operands(M, N, K, M + N + K)
    y0 = hdq.linear(hdq.PREC_NVFP4, None, W, xq=xq, y_dtype=y_dtype)
    y1 = hdq.linear(hdq.PREC_NVFP4, None, Wd, xq=xqd, y_dtype=y_dtype)
    y2 = hdq.linear(hdq.PREC_NVFP4, None, Wd, xq=xq, y_dtype=y_dtype)    # weights only: codes path
    y3 = hdq.linear(hdq.PREC_NVFP4, None, W, xq=xqd, y_dtype=y_dtype)    # activations only: W decoded here
    torch.cuda.synchronize()
    assert torch.equal(bits(y1), bits(y0))
    assert torch.equal(bits(y2), bits(y0))
    assert torch.equal(bits(y3), bits(y0))


@pytest.mark.parametrize("M,N,K,y_dtype", [(300, 384, 512, hdq.DTYPE_BF16), (1000, 600, 1024, hdq.DTYPE_F32),
                                           (37, 19, 96, hdq.DTYPE_BF16), (17776, 3072, 3072, hdq.DTYPE_BF16)])
def test_dispatch_decoded_operands_same_bits(M, N, K, y_dtype):
    """The one-launch GEMM (or, for shapes it does not take, the gated ones)
    with decoded plain-NVFP4 operands: the same bits for every decision."""
    say(f"dispatch decoded M={M} N={N} K={K} y={y_dtype}")
    xd, W, Wd, xq, xqd = operands(M, N, K, 7 * M + N)
    xq8 = hdq.quantize(xd, 32, hdq.FMT_INT8_ROW)
    d = torch.empty(1, dtype=torch.int32, device=DEV)
    for prec in (hdq.PREC_NVFP4, hdq.PREC_INT8, hdq.PREC_BF16):
        d.fill_(prec)
        y0 = hdq.linear_dispatch(d, xd, xq8, xq, W, y_dtype=y_dtype)
        y1 = hdq.linear_dispatch(d, xd, xq8, xqd, Wd, y_dtype=y_dtype)
        y2 = hdq.linear_dispatch(d, xd, xq8, xqd, W, y_dtype=y_dtype)
        torch.cuda.synchronize()
        assert torch.equal(bits(y1), bits(y0)), prec
        assert torch.equal(bits(y2), bits(y0)), prec


def test_dispatch_delta_decoded_operands_same_bits():
    M, N, K = 700, 512, 1024
    xd, W, Wd, xq, xqd = operands(M, N, K, 11)
    xq8 = hdq.quantize(xd, 32, hdq.FMT_INT8_ROW)
    d = torch.full((1,), hdq.PREC_NVFP4, dtype=torch.int32, device=DEV)
    rng = synth.rng_for(154, 0)
    a = to_dev(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    b = to_dev(synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    nch = hdq.delta_chunks(M * K)
    queue = torch.zeros(2, dtype=torch.int32, device=DEV)
    parts = torch.zeros((nch, 2), dtype=torch.float64, device=DEV)
    y0 = hdq.linear_dispatch(d, xd, xq8, xq, W)
    y1 = hdq.linear_dispatch_delta(d, xd, xq8, xqd, Wd, [(a, b, 0, nch, parts)], queue)
    torch.cuda.synchronize()
    assert torch.equal(bits(y1), bits(y0))
    parts2 = torch.zeros_like(parts)
    y2 = hdq.linear_dispatch_delta(d, xd, xq8, xqd, W, [(a, b, 0, nch, parts2)], queue)
    torch.cuda.synchronize()
    assert torch.equal(bits(y2), bits(y0))
    assert torch.equal(parts2, parts)
    ref = hdq.delta_sums(a, b)
    torch.cuda.synchronize()
    got = parts.sum(dim=0).cpu().numpy()
    assert np.allclose(got, ref.cpu().numpy(), rtol=1e-12, atol=0.0)
