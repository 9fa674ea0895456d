"""GPU <-> oracle parity through the C ABI (libhdq via its Python binding).

Bars (per the method's numerics):
  * quantized codes and scales: bit-exact (a +-1 LSB at a rounding tie is
    tolerated on <= 1e-5 of the elements; none is expected, both sides round
    the same float32 values);
  * integer GEMM on identical codes: bit-exact int32;
  * INT8 linear outputs: bit-exact (same float32 epilogue order), and in any
    case relative Frobenius error <= 1e-3 against the oracle's output rounded
    to the output dtype;
  * NVFP4 / bf16 linear outputs: relative Frobenius <= 1e-3 against the
    oracle's double result rounded to the output dtype (only the float32
    accumulation order differs);
  * decisions equal unless the oracle's statistic is within 1e-5 (relative)
    of a threshold.
Sizes span several tiles and ragged tails; full CogVideoX-shaped configs are
checked on sampled rows/columns the oracle computes one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_video_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from bit_quantized_video_amd import hdq  # noqa: E402  (loads libhdq.so; fails loudly if missing)

DEV = torch.device("cuda:0")
REL_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_to_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_from_bf16_np(x16):
    return synth.bf16_bits_to_f32(x16)


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (den if den > 0 else 1.0)


def abs_products_nvfp4(ac, ae, ast, wc, we, wst, K):
    """S[m, n] = sum_k |a_k w_k| over the decoded NVFP4 operands (double)."""
    a = np.abs(O.dequant_nvfp4(ac, ae, ast, K).astype(np.float64))
    w = np.abs(O.dequant_nvfp4(wc, we, wst, K).astype(np.float64))
    return a @ w.T


def abs_products_bf16(x16, w16):
    """S[m, n] = sum_k |x_k w_k| over the bf16 operands (double)."""
    return np.abs(f32_from_bf16_np(x16).astype(np.float64)) @ np.abs(f32_from_bf16_np(w16).astype(np.float64)).T


def assert_elementwise(got, ref64, S, K, bf16_out, what=""):
    """Per-element bar beside the Frobenius one, so that a wrong tile whose
    error is small next to the whole output's norm still fails.  got is the
    GPU output, ref64 the oracle's unrounded double result, S = sum_k |a_k w_k|.
    The GPU's only freedom is the float32 accumulation order over K: c u S
    with c = max(4, 2 sqrt(K / 16)) (u = 2^-24; the probabilistic rounding-error
    bound of a sum of K / 16 accumulated MFMA partials, with margin), plus
    4 u |ref| for the epilogue's scale multiplies, plus half a bf16 ulp of the
    stored value for bf16 output."""
    got = np.asarray(got, np.float64)
    ref64 = np.asarray(ref64, np.float64)
    c = max(4.0, 2.0 * math.sqrt(K / 16.0))
    tol = c * 2.0 ** -24 * S + 4 * 2.0 ** -24 * np.abs(ref64) + 1e-35
    if bf16_out:
        tol = tol + 2.0 ** -8 * 1.01 * np.abs(got)
    err = np.abs(got - ref64)
    worst = float((err / tol).max()) if err.size else 0.0
    n_bad = int((err > tol).sum())
    assert n_bad == 0, f"{what}: {n_bad} of {err.size} outputs beyond the per-element bound (worst {worst:.2f}x)"
    return worst


def round_like(ref64, y_dtype):
    if y_dtype == hdq.DTYPE_BF16:
        return f32_from_bf16_np(O.f32_to_bf16(ref64.astype(np.float32))).astype(np.float64)
    return ref64.astype(np.float32).astype(np.float64)


def y_np(y):
    if y.dtype == torch.bfloat16:
        return f32_from_bf16_np(bf16_to_np(y)).astype(np.float64)
    return y.cpu().numpy().astype(np.float64)


def sample_rows(M, head=64, tail=48):
    if M <= head + tail:
        return np.arange(M)
    return np.concatenate([np.arange(head), np.arange(M - tail, M)])


def assert_codes_equal(got, ref, what):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, what
    diff = got != ref
    n = int(diff.sum())
    if n:
        frac = n / got.size
        # tolerated: <= 1e-5 of the elements off by one LSB
        d = np.abs(got.astype(np.int64) - ref.astype(np.int64))[diff]
        assert frac <= 1e-5 and d.max() <= 1, f"{what}: {n} mismatches ({frac:.2e}), max diff {d.max()}"


def nvfp4_codes_equal(got, ref, what):
    """Packed E2M1 bytes equal, with +0 and -0 codes taken as equal."""
    g = np.stack([got & 0xF, got >> 4], -1)
    r = np.stack([ref & 0xF, ref >> 4], -1)
    g = np.where((g & 7) == 0, 0, g)
    r = np.where((r & 7) == 0, 0, r)
    assert_codes_equal(g, r, what)


# ------------------------------------------------------------ quantizers

INT_CASES = [(1, 64, 16), (37, 128, 32), (130, 1024, 64), (300, 1920, 128), (9, 3072, 128),
             (5, 12288, 128), (3, 20480, 128), (17, 64, 2), (17, 64, 4), (17, 64, 8)]


@pytest.mark.parametrize("M,K,hb", INT_CASES)
@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_quantize_int_rows_bitexact(M, K, hb, fmt):
    say(f"quantize {fmt} M={M} K={K} hb={hb}")
    x16 = synth.gaussian_outliers(M, K, 0.01, 25.0, synth.rng_for(100, M * 7 + K))
    qmax = 127 if fmt == "int8" else 7
    f = hdq.FMT_INT8_ROW if fmt == "int8" else hdq.FMT_INT4_ROW
    q = hdq.quantize(to_dev(x16), hb, f)
    torch.cuda.synchronize()
    rq, rs = O.quant_int(x16, hb, qmax)
    assert np.array_equal(q.row_scale.cpu().numpy(), rs), "row scales"
    if fmt == "int8":
        assert_codes_equal(q.codes.cpu().numpy(), rq, "int8 codes")
    else:
        assert_codes_equal(q.codes.cpu().numpy(), O.pack_int4(rq), "int4 bytes")


def test_quantize_int_zero_and_tiny_rows():
    x = np.zeros((4, 256), np.float32)
    x[1, 7] = 2.0 ** -110            # below the zero-row threshold
    x[2, :] = 3.0
    x[3, 5] = -1e-20
    x16 = synth.to_bf16_bits(x)
    q = hdq.quantize(to_dev(x16), 64, hdq.FMT_INT8_ROW)
    rq, rs = O.quant_int(x16, 64, 127)
    assert np.array_equal(q.row_scale.cpu().numpy(), rs)
    assert np.array_equal(q.codes.cpu().numpy(), rq)


# (2800 x 12288 at block 128: more 32-element groups than the grid's threads,
# so the grid-stride loop runs a second, partial round)
NV_CASES = [(1, 64, 16), (37, 128, 32), (130, 1024, 64), (301, 3072, 128), (5, 12288, 128), (2800, 12288, 128)]


# NVFP4 recipes: the oracle's mx argument for each format
FP4_FMTS = {hdq.FMT_NVFP4: 0, hdq.FMT_NVFP4_MX: 1, hdq.FMT_NVFP4_P2: 2}


@pytest.mark.parametrize("M,K,hb", NV_CASES)
@pytest.mark.parametrize("fmt", list(FP4_FMTS))
@pytest.mark.parametrize("amax_given", [False, True])
def test_quantize_nvfp4_bitexact(M, K, hb, fmt, amax_given):
    mx = FP4_FMTS[fmt]
    say(f"quantize nvfp4 fmt={fmt} M={M} K={K} hb={hb} amax_given={amax_given}")
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(101, M * 7 + K))
    amax = O.rotated_amax(x16, hb)
    am = torch.tensor([amax], dtype=torch.float32, device=DEV) if amax_given else None
    q = hdq.quantize(to_dev(x16), hb, fmt, tensor_amax=am)
    torch.cuda.synchronize()
    rc, re_, rst = O.quant_nvfp4(x16, hb, mx=mx)
    assert q.tensor_scale.item() == rst
    assert_codes_equal(q.blk_scale.cpu().numpy(), re_, "E4M3 scales")
    nvfp4_codes_equal(q.codes.cpu().numpy(), rc, "E2M1 codes")


@pytest.mark.parametrize("hb", [64, 128])
@pytest.mark.parametrize("fmt", list(FP4_FMTS))
def test_quantize_nvfp4_zero_tensor(hb, fmt):
    x16 = np.zeros((8, 256), np.uint16)
    q = hdq.quantize(to_dev(x16), hb, fmt)
    assert q.tensor_scale.item() == 0.0
    assert not q.codes.any().item() and not q.blk_scale.any().item()


# -------------------------------------------------------- statistics

def stats_case(prev_in, prev_out, cur, hb):
    d, s = hdq.select_precision(None if prev_in is None else to_dev(prev_in),
                                None if prev_out is None else to_dev(prev_out), to_dev(cur), hb)
    torch.cuda.synchronize()
    ref = O.stats(prev_in, prev_out, cur, hb)
    return int(d.item()), s.cpu().numpy().astype(np.float64), ref


def decision_ok(got, ref_stats, has_hist, dth=0.1, rth=50.0):
    want = O.decide(has_hist, ref_stats[0], ref_stats[1], dth, rth)
    if got == want:
        return True
    near = lambda v, t: math.isfinite(v) and abs(v - t) <= 1e-5 * t
    return near(ref_stats[0], dth) or near(ref_stats[1], rth)


@pytest.mark.parametrize("M,K,s", [(64, 1024, 0.05), (333, 3072, 0.2), (17, 12288, 0.1), (1000, 128, 0.0999)])
def test_stats_match_oracle(M, K, s):
    say(f"stats M={M} K={K} s={s}")
    rng = synth.rng_for(102, M)
    x = rng.standard_normal((M, K)).astype(np.float32)
    cur = synth.to_bf16_bits(x)
    prev_in = synth.to_bf16_bits(x)
    prev_out = synth.to_bf16_bits(x + rng.standard_normal((M, K)).astype(np.float32) * np.float32(s))
    dec, st, ref = stats_case(prev_in, prev_out, cur, 128)
    assert abs(st[0] - ref[0]) <= 2e-6 * ref[0] + 1e-30
    assert abs(st[1] - ref[1]) <= 2e-6 * ref[1]
    assert st[2] == np.float32(ref[2])
    assert abs(st[3] - ref[3]) <= 2e-6 * ref[3]
    assert st[4] == np.float32(ref[4])          # rotated amax: exact (same float32 rotation)
    assert decision_ok(dec, ref, True)


@pytest.mark.parametrize("M,K,hb,s", [(333, 3072, 128, 0.2), (64, 1024, 0, 0.05), (17, 12288, 128, 0.1),
                                      (1000, 128, 64, 0.0999), (17776, 3072, 128, 0.08)])
def test_two_part_selection_matches_one_pass(M, K, hb, s):
    """hdq_delta_sums + hdq_select_precision_sums write the same bits as
    hdq_select_precision; the sums themselves match the oracle's."""
    say(f"two-part selection M={M} K={K} hb={hb}")
    rng = synth.rng_for(112, M)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x16 = synth.to_bf16_bits(x)
    po16 = synth.to_bf16_bits(x + rng.standard_normal((M, K)).astype(np.float32) * np.float32(s))
    xd, pid, pod = to_dev(x16), to_dev(x16.copy()), to_dev(po16)
    bits = lambda t: t.view(torch.int32).cpu().numpy()
    d1, s1 = hdq.select_precision(pid, pod, xd, hb)
    sums = hdq.delta_sums(pid, pod)
    d2, s2 = hdq.select_precision_sums(sums, xd, hb)
    d3, s3 = hdq.select_precision(None, None, xd, hb)
    d4, s4 = hdq.select_precision_sums(None, xd, hb)
    torch.cuda.synchronize()
    assert np.array_equal(bits(s1), bits(s2)) and int(d1.item()) == int(d2.item())
    assert np.array_equal(bits(s3), bits(s4)) and int(d3.item()) == int(d4.item())
    ref = O.stats(x16, po16, x16, hb)
    got = sums.cpu().numpy()
    assert abs(got[0] / got[1] - ref[0]) <= 2e-6 * ref[0]


# (K 3072 and 12288 at block 128 fill a workgroup's chunks exactly, the
# kernel without bounds checks; K 1920 at block 128 leaves chunks past the row)
@pytest.mark.parametrize("M,K,hb,s,hist", [(333, 3072, 128, 0.2, True), (64, 1024, 64, 0.05, True),
                                            (9, 12288, 128, 0.1, True), (5, 20480, 128, 0.03, True),
                                            (17776, 3072, 128, 0.08, True), (100, 512, 32, 0.0, False),
                                            (200, 1920, 128, 0.1, True)])
def test_select_fused_with_int8_quantization(M, K, hb, s, hist):
    """hdq_select_quantize_int8 = hdq_select_precision_sums + INT8 hdq_quantize:
    codes and row scales bit for bit, the decision and delta, max and rotated
    amax exactly, mean |x| and the ratio up to the double sum order."""
    say(f"select+int8 M={M} K={K} hb={hb}")
    rng = synth.rng_for(113, M + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x16 = synth.to_bf16_bits(x)
    po16 = synth.to_bf16_bits(x + rng.standard_normal((M, K)).astype(np.float32) * np.float32(s))
    xd, pid, pod = to_dev(x16), to_dev(x16.copy()), to_dev(po16)
    sums = hdq.delta_sums(pid, pod) if hist else None
    d1, s1 = hdq.select_precision_sums(sums, xd, hb)
    q1 = hdq.quantize(xd, hb, hdq.FMT_INT8_ROW)
    d2, s2, q2 = hdq.select_quantize_int8(sums, xd, hb)
    torch.cuda.synchronize()
    assert int(d1.item()) == int(d2.item())
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.row_scale, q2.row_scale)
    a, b = s1.cpu().numpy().astype(np.float64), s2.cpu().numpy().astype(np.float64)
    for i in (0, 2, 4):
        assert (math.isnan(a[i]) and math.isnan(b[i])) or a[i] == b[i], i
    for i in (1, 3):
        assert abs(a[i] - b[i]) <= 1e-6 * abs(a[i]), i
    # and the oracle: codes and the statistics
    ref = O.stats(x16 if hist else None, po16 if hist else None, x16, hb)
    qa, sa = O.quant_int(x16[:64], hb, 127)
    assert_codes_equal(q2.codes.cpu().numpy()[:64], qa, "codes")
    assert abs(b[1] - ref[1]) <= 2e-6 * ref[1] and b[4] == np.float32(ref[4])


def test_stats_hand_cases():
    ones = np.ones((4, 64), np.float32)
    b = synth.to_bf16_bits
    # no history -> INT8
    dec, st, ref = stats_case(None, None, b(ones), 64)
    assert dec == hdq.PREC_INT8 and math.isnan(st[0]) and st[1] == 1.0 and st[4] == 8.0
    # in == out -> NVFP4; out = 2 in -> INT8
    assert stats_case(b(ones), b(ones), b(ones), 0)[0] == hdq.PREC_NVFP4
    assert stats_case(b(ones), b(2 * ones), b(ones), 0)[0] == hdq.PREC_INT8
    # ratio exactly 50 (64 * 225 / 288) stays quantized, 226 goes to BF16
    x = np.ones((1, 64), np.float32)
    x[0, 9] = 225.0
    dec, st, _ = stats_case(b(ones), b(ones), b(x), 0)
    assert st[1] == 50.0 and dec == hdq.PREC_NVFP4
    x[0, 9] = 226.0
    assert stats_case(b(ones), b(ones), b(x), 0)[0] == hdq.PREC_BF16
    # non-finite input -> BF16; all-zero input -> ratio 0
    x[0, 9] = np.inf
    dec, st, _ = stats_case(b(ones), b(ones), b(x), 16)
    assert dec == hdq.PREC_BF16 and math.isnan(st[1])
    x[0, 9] = np.nan
    assert stats_case(None, None, b(x), 0)[0] == hdq.PREC_BF16
    z = np.zeros((2, 64), np.uint16)
    dec, st, _ = stats_case(z, z, z, 0)
    assert st[0] == 0.0 and st[1] == 0.0 and dec == hdq.PREC_NVFP4
    # a previous-step numel that is not a multiple of 8, and a cur without rotation
    pi = b(np.full((1, 13), 2.0, np.float32))
    po = b(np.full((1, 13), 2.5, np.float32))
    dec, st, ref = stats_case(pi, po, b(np.ones((3, 7), np.float32)), 0)
    assert st[0] == 0.25 and dec == hdq.PREC_INT8


def test_delta_exactly_at_threshold_goes_int8():
    """A difference exactly at the threshold takes the large-difference side
    (INT8), a threshold one float32 step above it gives NVFP4: in = 8,
    out = 9 gives delta = 1/8 exactly.  One-pass, two-part and fused
    selection, and the oracle's rule, agree."""
    b = synth.to_bf16_bits
    pi, po = to_dev(b(np.full((4, 64), 8.0, np.float32))), to_dev(b(np.full((4, 64), 9.0, np.float32)))
    cur16 = synth.gaussian(4, 64, 1.0, synth.rng_for(117, 0))
    cur = to_dev(cur16)
    above = float(np.nextafter(np.float32(0.125), np.float32(1)))
    for th, want in ((0.125, hdq.PREC_INT8), (above, hdq.PREC_NVFP4)):
        d1, s1 = hdq.select_precision(pi, po, cur, 64, delta_thresh=th)
        sums = hdq.delta_sums(pi, po)
        d2, s2 = hdq.select_precision_sums(sums, cur, 64, delta_thresh=th)
        d3, s3, _ = hdq.select_quantize_int8(sums, cur, 64, delta_thresh=th)
        torch.cuda.synchronize()
        assert float(s1[0].item()) == 0.125 and float(s2[0].item()) == 0.125 and float(s3[0].item()) == 0.125
        assert float(s1[1].item()) <= 50.0
        assert int(d1.item()) == int(d2.item()) == int(d3.item()) == want, th
        ref = O.stats(b(np.full((4, 64), 8.0, np.float32)), b(np.full((4, 64), 9.0, np.float32)), cur16, 64)
        assert ref[0] == 0.125 and O.decide(True, ref[0], ref[1], th, 50.0) == want


# ------------------------------------------------------------ GEMMs

def int_operands(M, N, K, hb, seed):
    x16 = synth.gaussian_outliers(M, K, 0.01, 20.0, synth.rng_for(103, seed))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(104, seed))
    return x16, w16


GEMM_CASES = [(1, 1, 32), (37, 19, 64), (300, 200, 96), (257, 129, 1920), (512, 384, 1024), (64, 5760, 128)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
def test_int_gemm_i32_bitexact(M, N, K):
    say(f"int gemm i32 M={M} N={N} K={K}")
    hb = 32
    x16, w16 = int_operands(M, N, K, hb, M * 31 + N)
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=None)
    xq = hdq.quantize(to_dev(x16), hb, hdq.FMT_INT8_ROW)
    y = hdq.linear(hdq.PREC_INT8, None, W, xq=xq, y_dtype=hdq.DTYPE_I32)
    torch.cuda.synchronize()
    qa, sa = O.quant_int(x16, hb, 127)
    qw, sw = O.quant_int(w16, hb, 7)
    _, acc = O.gemm_int(qa, sa, qw, sw)
    assert np.array_equal(y.cpu().numpy().astype(np.int64), acc)


# More 256 x 256 tiles (17 x 16 = 272) than persistent workgroups (at most
# one per CU), so some workgroups run a second tile right after the last
# K-stage of their first; K covers every count of K-stages modulo the LDS
# stage rotation.  Sampled rows reach every tile row.
MT_M, MT_N = 17 * 256, 16 * 256
MT_ROWS = np.r_[np.arange(0, MT_M, 17), MT_M - 1]


@pytest.mark.parametrize("K", [128, 256, 384, 512])
def test_int_gemm_multi_tile_workgroups(K):
    say(f"int gemm i32 multi-tile M={MT_M} N={MT_N} K={K}")
    hb = 32
    x16, w16 = int_operands(MT_M, MT_N, K, hb, K)
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=None)
    xq = hdq.quantize(to_dev(x16), hb, hdq.FMT_INT8_ROW)
    y = hdq.linear(hdq.PREC_INT8, None, W, xq=xq, y_dtype=hdq.DTYPE_I32)
    torch.cuda.synchronize()
    qa, sa = O.quant_int(x16[MT_ROWS], hb, 127)
    qw, sw = O.quant_int(w16, hb, 7)
    _, acc = O.gemm_int(qa, sa, qw, sw)
    assert np.array_equal(y.cpu().numpy()[MT_ROWS].astype(np.int64), acc)


@pytest.mark.parametrize("K", [64, 128, 192])
def test_bf16_gemm_multi_tile_workgroups(K):
    say(f"bf16 gemm f32 multi-tile M={MT_M} N={MT_N} K={K}")
    x16 = synth.gaussian_outliers(MT_M, K, 0.01, 20.0, synth.rng_for(108, K))
    w16 = synth.gaussian(MT_N, K, 0.02, synth.rng_for(109, K))
    W = hdq.LinearWeights(to_dev(w16), 32, fp4_fmt=None)
    y = hdq.linear(hdq.PREC_BF16, to_dev(x16), W, y_dtype=hdq.DTYPE_F32)
    torch.cuda.synchronize()
    ref64 = O.gemm_bf16(x16[MT_ROWS], w16)
    ref = round_like(ref64, hdq.DTYPE_F32)
    assert rel_fro(y_np(y)[MT_ROWS], ref) <= REL_TOL
    assert_elementwise(y_np(y)[MT_ROWS], ref64, abs_products_bf16(x16[MT_ROWS], w16), K, False, "bf16 multi-tile")


@pytest.mark.parametrize("fmt,K", [(hdq.FMT_NVFP4_MX, K) for K in (256, 512, 768)] +
                         [(hdq.FMT_NVFP4_P2, K) for K in (256, 768)])
def test_fp4_gemm_multi_tile_workgroups(fmt, K):
    say(f"fp4 gemm f32 multi-tile fmt={fmt} M={MT_M} N={MT_N} K={K}")
    hb = 32
    x16 = synth.lognormal_tokens(MT_M, K, synth.rng_for(105, K))
    w16 = synth.gaussian(MT_N, K, 0.02, synth.rng_for(106, K))
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=fmt)
    y = hdq.linear(hdq.PREC_NVFP4, to_dev(x16), W, y_dtype=hdq.DTYPE_F32)
    torch.cuda.synchronize()
    mx = FP4_FMTS[fmt]
    ac, ae, ast = O.quant_nvfp4(x16[MT_ROWS], hb, amax=O.rotated_amax(x16, hb), mx=mx)
    wc, we, wst = O.quant_nvfp4(w16, hb, mx=mx)
    ref64 = O.gemm_nvfp4(ac, ae, ast, wc, we, wst, K)
    ref = round_like(ref64, hdq.DTYPE_F32)
    assert rel_fro(y_np(y)[MT_ROWS], ref) <= REL_TOL
    assert_elementwise(y_np(y)[MT_ROWS], ref64, abs_products_nvfp4(ac, ae, ast, wc, we, wst, K), K, False,
                       "fp4 multi-tile")


@pytest.mark.parametrize("fmt", [hdq.FMT_NVFP4, hdq.FMT_NVFP4_MX, hdq.FMT_NVFP4_P2])
def test_fp4_gemm_subnormal_block_scales(fmt):
    # Rows scaled by powers of two and one zero row.  MX / per-16 powers of
    # two (rows x 2^-13 ... 2^-18): the blocks' power-of-two E4M3 scales are
    # the subnormal codes 2^-7, 2^-8 and 2^-9 (also the clamp, and the zero
    # row's), which the FP4 kernels turn into E8M0 exponents.  Plain NVFP4
    # (rows x 2^-14 ... 2^-19): t = a_blk / (6 s_t) walks from the smallest
    # normal E4M3 through the subnormal codes k 2^-9 to blocks flushed to 0,
    # through hdq_quantize and the exact bf16-MFMA kernel.
    M, N, K, hb = 300, 272, 512, 32
    rows = np.arange(M)
    first = 13 if fmt == hdq.FMT_NVFP4 else 12
    scale = np.where(rows % 8 == 0, 1.0, 2.0 ** -(first + rows % 8)).astype(np.float32)
    scale[7] = 0.0
    x = synth.bf16_bits_to_f32(synth.gaussian(M, K, 1.0, synth.rng_for(110, fmt)))
    x16 = synth.to_bf16_bits(x * scale[:, None])       # exact: powers of two
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(111, fmt))
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=fmt)
    xq = hdq.quantize(to_dev(x16), hb, fmt)
    y = hdq.linear(hdq.PREC_NVFP4, None, W, xq=xq, y_dtype=hdq.DTYPE_F32)
    torch.cuda.synchronize()
    mx = FP4_FMTS[fmt]
    ac, ae, ast = O.quant_nvfp4(x16, hb, mx=mx)
    if fmt == hdq.FMT_NVFP4:
        sub = (ae > 0) & (ae < 0x08)
        assert len(np.unique(ae[sub])) >= 4          # several subnormal scale codes occur
        assert (ae[(rows % 8 == 5) | (rows % 8 == 6)] == 0).any()   # and flushed blocks in nonzero rows
    else:
        assert np.isin([1, 2, 4], ae).all()          # the subnormal scales occur
    assert np.array_equal(xq.blk_scale.cpu().numpy().reshape(ae.shape), ae)
    assert xq.tensor_scale.item() == ast
    nvfp4_codes_equal(xq.codes.cpu().numpy(), ac, "E2M1 codes")
    wc, we, wst = O.quant_nvfp4(w16, hb, mx=mx)
    ref64 = O.gemm_nvfp4(ac, ae, ast, wc, we, wst, K)
    ref = round_like(ref64, hdq.DTYPE_F32)
    got = y_np(y)
    for r in range(8):       # every row class separately: the tiny rows carry tiny outputs
        sel = rows % 8 == r
        assert rel_fro(got[sel], ref[sel]) <= REL_TOL, r
    assert_elementwise(got, ref64, abs_products_nvfp4(ac, ae, ast, wc, we, wst, K), K, False, "subnormal scales")


@pytest.mark.parametrize("M,N,K", GEMM_CASES[1:])
@pytest.mark.parametrize("y_dtype", [hdq.DTYPE_F32, hdq.DTYPE_BF16])
def test_linear_int8_matches_oracle(M, N, K, y_dtype):
    say(f"linear int8 M={M} N={N} K={K} y={y_dtype}")
    hb = 64 if K % 64 == 0 else 32
    x16, w16 = int_operands(M, N, K, hb, M * 17 + N)
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=None)
    y = hdq.linear(hdq.PREC_INT8, to_dev(x16), W, y_dtype=y_dtype)
    torch.cuda.synchronize()
    qa, sa = O.quant_int(x16, hb, 127)
    qw, sw = O.quant_int(w16, hb, 7)
    ref, _ = O.gemm_int(qa, sa, qw, sw)
    ref = round_like(ref.astype(np.float64), y_dtype)
    got = y_np(y)
    assert rel_fro(got, ref) <= REL_TOL
    assert np.array_equal(got, ref)      # same float32 epilogue order: exact


@pytest.mark.parametrize("M,N,K", [(37, 19, 64), (300, 200, 96), (257, 129, 1024), (64, 640, 3072),
                                   (600, 520, 768)])
@pytest.mark.parametrize("fmt", list(FP4_FMTS))
@pytest.mark.parametrize("y_dtype", [hdq.DTYPE_F32, hdq.DTYPE_BF16])
def test_linear_nvfp4_matches_oracle(M, N, K, fmt, y_dtype):
    mx = FP4_FMTS[fmt]
    say(f"linear nvfp4 fmt={fmt} M={M} N={N} K={K} y={y_dtype}")
    hb = 32
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(105, M + N))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(106, M + N))
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=fmt)
    y = hdq.linear(hdq.PREC_NVFP4, to_dev(x16), W, y_dtype=y_dtype)
    torch.cuda.synchronize()
    ac, ae, ast = O.quant_nvfp4(x16, hb, mx=mx)
    wc, we, wst = O.quant_nvfp4(w16, hb, mx=mx)
    ref64 = O.gemm_nvfp4(ac, ae, ast, wc, we, wst, K)
    ref = round_like(ref64, y_dtype)
    assert rel_fro(y_np(y), ref) <= REL_TOL
    assert_elementwise(y_np(y), ref64, abs_products_nvfp4(ac, ae, ast, wc, we, wst, K), K,
                       y_dtype == hdq.DTYPE_BF16, "linear nvfp4")


@pytest.mark.parametrize("fmt", [hdq.FMT_NVFP4_MX, hdq.FMT_NVFP4_P2])
def test_nvfp4_exact_kernel_accepts_mx_bytes(fmt):
    # MX-compatible and per-16 power-of-two bytes are valid NVFP4: the exact
    # (bf16-MFMA) kernel on them must agree with the block-scaled FP4 kernel
    M, N, K, hb = 200, 160, 512, 64
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(107, 1))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(107, 2))
    Wmx = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=fmt)
    xq = hdq.quantize(to_dev(x16), hb, fmt)
    y_mx = hdq.linear(hdq.PREC_NVFP4, None, Wmx, xq=xq, y_dtype=hdq.DTYPE_F32)
    Wmx.w_fp4.fmt = hdq.FMT_NVFP4
    xq.fmt = hdq.FMT_NVFP4
    y_v1 = hdq.linear(hdq.PREC_NVFP4, None, Wmx, xq=xq, y_dtype=hdq.DTYPE_F32)
    torch.cuda.synchronize()
    assert rel_fro(y_mx.cpu().numpy(), y_v1.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("M,N,K", [(37, 19, 64), (300, 200, 96), (257, 129, 1024), (64, 640, 3072)])
@pytest.mark.parametrize("y_dtype", [hdq.DTYPE_F32, hdq.DTYPE_BF16])
def test_linear_bf16_matches_oracle(M, N, K, y_dtype):
    say(f"linear bf16 M={M} N={N} K={K}")
    x16 = synth.gaussian_outliers(M, K, 0.01, 20.0, synth.rng_for(108, M))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(109, M))
    W = hdq.LinearWeights(to_dev(w16), 32, fp4_fmt=None)
    y = hdq.linear(hdq.PREC_BF16, to_dev(x16), W, y_dtype=y_dtype)
    torch.cuda.synchronize()
    ref64 = O.gemm_bf16(x16, w16)
    ref = round_like(ref64, y_dtype)
    assert rel_fro(y_np(y), ref) <= REL_TOL
    assert_elementwise(y_np(y), ref64, abs_products_bf16(x16, w16), K, y_dtype == hdq.DTYPE_BF16, "linear bf16")


# ---------------------------------------- device-predicated dispatch

@pytest.mark.parametrize("case", ["nvfp4", "int8", "bf16", "nohist"])
def test_device_predicated_linear_matches_fixed(case):
    say(f"predicated {case}")
    M, N, K, hb = 300, 256, 512, 128
    rng = synth.rng_for(110, 0)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if case == "bf16":
        x[:, 3] *= 400.0                      # outlier ratio far above 50
    x16 = synth.to_bf16_bits(x)
    s = {"nvfp4": 0.02, "int8": 0.2, "bf16": 0.02, "nohist": 0.0}[case]
    po16 = synth.to_bf16_bits(x + rng.standard_normal((M, K)).astype(np.float32) * np.float32(s))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(110, 1))
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=hdq.FMT_NVFP4)
    xd = to_dev(x16)
    hist = case != "nohist"
    dec, st = hdq.select_precision(to_dev(x16) if hist else None, to_dev(po16) if hist else None, xd, hb)
    y_dyn = hdq.linear(-1, xd, W, decision=dec, x_amax=st[4:5], y_dtype=hdq.DTYPE_BF16)
    torch.cuda.synchronize()
    want = {"nvfp4": hdq.PREC_NVFP4, "int8": hdq.PREC_INT8, "bf16": hdq.PREC_BF16, "nohist": hdq.PREC_INT8}[case]
    assert int(dec.item()) == want
    y_fix = hdq.linear(want, xd, W, y_dtype=hdq.DTYPE_BF16)
    torch.cuda.synchronize()
    assert torch.equal(y_dyn.view(torch.int16), y_fix.view(torch.int16))


@pytest.mark.parametrize("M,N,K,y_dtype", [(m, n, k, yd) for (m, n, k) in [(300, 384, 512), (1000, 600, 1024), (37, 19, 96)]
                                             for yd in (hdq.DTYPE_BF16, hdq.DTYPE_F32)]
                         + [(17776, 3072, 3072, hdq.DTYPE_BF16)])   # full size: bf16 output only
@pytest.mark.parametrize("fmt", ["nvfp4", "nvfp4_mx", "nvfp4_p2"])
def test_linear_dispatch_matches_fixed_precision(M, N, K, fmt, y_dtype):
    """hdq_linear_dispatch runs the decided precision's GEMM (one launch, or
    three gated ones for shapes the single kernel does not take) with the
    same bits as hdq_linear at that precision."""
    say(f"linear dispatch M={M} N={N} K={K} {fmt} y={y_dtype}")
    hb = 32
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(114, M + N))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(114, K))
    f = {"nvfp4": hdq.FMT_NVFP4, "nvfp4_mx": hdq.FMT_NVFP4_MX, "nvfp4_p2": hdq.FMT_NVFP4_P2}[fmt]
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=f)
    xd = to_dev(x16)
    xq8 = hdq.quantize(xd, hb, hdq.FMT_INT8_ROW)
    xq4 = hdq.quantize(xd, hb, f)
    dec = torch.empty(1, dtype=torch.int32, device=DEV)
    for prec in (hdq.PREC_INT8, hdq.PREC_NVFP4, hdq.PREC_BF16):
        dec.fill_(prec)
        y = hdq.linear_dispatch(dec, xd, xq8, xq4, W, y_dtype=y_dtype)
        if prec == hdq.PREC_BF16:
            ref = hdq.linear(prec, xd, W, y_dtype=y_dtype)
        else:
            ref = hdq.linear(prec, None, W, xq=xq8 if prec == hdq.PREC_INT8 else xq4, y_dtype=y_dtype)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32)), prec


def _delta_pair(M, K, s, seed):
    rng = synth.rng_for(115, seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    return synth.to_bf16_bits(x), synth.to_bf16_bits(x + rng.standard_normal((M, K)).astype(np.float32) * np.float32(s))


def test_linear_dispatch_delta_chunks_across_launches():
    """hdq_linear_dispatch_delta: the GEMM output is hdq_linear_dispatch's bit
    for bit; the difference statistic of two modules, their chunks spread
    over three launches (one of them empty), matches hdq_delta_sums and the
    oracle, drives the fused selection as the one-pair sums do, and the queue
    is left zero."""
    M, N, K, hb = 600, 520, 512, 32
    say(f"linear dispatch + delta chunks M={M} N={N} K={K}")
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(116, 0))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(116, 1))
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=hdq.FMT_NVFP4_MX)
    xd = to_dev(x16)
    xq8 = hdq.quantize(xd, hb, hdq.FMT_INT8_ROW)
    xq4 = hdq.quantize(xd, hb, hdq.FMT_NVFP4_MX)
    # module A: 300 x 1000 (5 chunks, the last partial); module B: 1024 x 2048 (32 chunks)
    a_in, a_out = _delta_pair(300, 1000, 0.2, 1)
    b_in, b_out = _delta_pair(1024, 2048, 0.07, 2)
    ai, ao, bi, bo = (to_dev(t) for t in (a_in, a_out, b_in, b_out))
    na, nb = hdq.delta_chunks(ai.numel()), hdq.delta_chunks(bi.numel())
    assert (na, nb) == (5, 32)
    pa = torch.full((na, 2), float("nan"), dtype=torch.float64, device=DEV)
    pb = torch.full((nb, 2), float("nan"), dtype=torch.float64, device=DEV)
    queue = torch.zeros(2, dtype=torch.int32, device=DEV)
    dec = torch.empty(1, dtype=torch.int32, device=DEV)
    plan = [(hdq.PREC_INT8, [(ai, ao, 0, na), (bi, bo, 0, 10)]),
            (hdq.PREC_NVFP4, []),
            (hdq.PREC_BF16, [(bi, bo, 10, 31), (bi, bo, 31, 32)])]
    for prec, sl in plan:
        dec.fill_(prec)
        y = hdq.linear_dispatch_delta(dec, xd, xq8, xq4, W, [s + (pa if s[0] is ai else pb,) for s in sl], queue)
        ref = hdq.linear_dispatch(dec, xd, xq8, xq4, W)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), prec
        assert queue.cpu().tolist() == [0, 0]
    for parts, pi, po, t_in, t_out in ((pa, ai, ao, a_in, a_out), (pb, bi, bo, b_in, b_out)):
        got = parts.cpu().numpy()
        assert np.isfinite(got).all()                       # every chunk ran once
        one = hdq.delta_sums(pi, po).cpu().numpy()
        tot = got.sum(axis=0)
        assert np.allclose(tot, one, rtol=1e-12, atol=0)
        ref = O.stats(t_in, t_out, t_in, 0)[0]     # no rotation: module A's 1000 columns
        assert abs(tot[0] / tot[1] - ref) <= 2e-6 * ref
    # the chunk partials as the selection's difference input: the same
    # decision and statistics as with the one-pair sums, delta to rounding
    cur16 = x16
    cd = to_dev(cur16)
    d1, s1, _ = hdq.select_quantize_int8(hdq.delta_sums(bi, bo), cd, hb)
    d2, s2, _ = hdq.select_quantize_int8(pb, cd, hb)
    torch.cuda.synchronize()
    assert int(d1.item()) == int(d2.item())
    s1, s2 = s1.cpu().numpy(), s2.cpu().numpy()
    assert np.array_equal(s1[1:], s2[1:]) and abs(s1[0] - s2[0]) <= 1e-6 * s1[0]
    d3, s3 = hdq.select_precision_sums(pb, cd, hb)
    torch.cuda.synchronize()
    assert int(d3.item()) == int(d1.item()) and abs(float(s3[0]) - s1[0]) <= 1e-6 * s1[0]


def test_linear_dispatch_delta_full_size_schedule_shape():
    """The schedule's largest difference (FFN-down input, 17776 x 12288: 3333
    chunks) beside a full-size GEMM, in two launches; sums as hdq_delta_sums."""
    M, N, K, hb = 17776, 3072, 3072, 128
    say("linear dispatch + delta, full size")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    x = synth.device_gaussian((M, K), 1.0, gen, DEV)
    w = synth.device_gaussian((N, K), 0.02, gen, DEV)
    pi = synth.device_gaussian((M, 12288), 1.0, gen, DEV)
    po = (pi.float() + 0.1 * synth.device_gaussian((M, 12288), 1.0, gen, DEV).float()).to(torch.bfloat16)
    W = hdq.LinearWeights(w, hb, fp4_fmt=hdq.FMT_NVFP4_MX)
    xq8 = hdq.quantize(x, hb, hdq.FMT_INT8_ROW)
    xq4 = hdq.quantize(x, hb, hdq.FMT_NVFP4_MX)
    n = hdq.delta_chunks(pi.numel())
    parts = torch.full((n, 2), float("nan"), dtype=torch.float64, device=DEV)
    queue = torch.zeros(2, dtype=torch.int32, device=DEV)
    dec = torch.full((1,), hdq.PREC_INT8, dtype=torch.int32, device=DEV)
    y1 = hdq.linear_dispatch_delta(dec, x, xq8, xq4, W, [(pi, po, 0, 1000, parts)], queue)
    ref = hdq.linear_dispatch(dec, x, xq8, xq4, W)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), ref.view(torch.int16))
    dec.fill_(hdq.PREC_NVFP4)
    y2 = hdq.linear_dispatch_delta(dec, x, xq8, xq4, W, [(pi, po, 1000, n, parts)], queue)
    ref = hdq.linear_dispatch(dec, x, xq8, xq4, W)
    one = hdq.delta_sums(pi, po)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), ref.view(torch.int16))
    got = parts.cpu().numpy()
    assert np.isfinite(got).all() and queue.cpu().tolist() == [0, 0]
    assert np.allclose(got.sum(axis=0), one.cpu().numpy(), rtol=1e-12, atol=0)


def test_repeat_runs_are_bitwise_identical():
    M, N, K, hb = 513, 384, 1024, 128
    x16 = synth.lognormal_tokens(M, K, synth.rng_for(111, 0))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(111, 1))
    xd = to_dev(x16)
    for fmt in FP4_FMTS:
        W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=fmt)
        for prec in (hdq.PREC_INT8, hdq.PREC_NVFP4, hdq.PREC_BF16):
            a = hdq.linear(prec, xd, W, y_dtype=hdq.DTYPE_F32)
            b = hdq.linear(prec, xd, W, y_dtype=hdq.DTYPE_F32)
            torch.cuda.synchronize()
            assert torch.equal(a, b), (fmt, prec)
    d1, s1 = hdq.select_precision(xd, xd, xd, hb)
    d2, s2 = hdq.select_precision(xd, xd, xd, hb)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(d1, d2)


# ----------------------------- full-size configs, sampled outputs

def run_config(cfg, path, n_cols=384):
    c = synth.CONFIGS[cfg]
    M, K, N, hb = c["M"], c["K"], c["N"], c["had_block"]
    say(f"config {cfg} {path}: generating M={M} K={K} N={N}")
    x16 = synth.config_activations(cfg)
    w16 = synth.config_weights(cfg)
    y_dtype = hdq.DTYPE_F32 if c["out"] == "f32" else hdq.DTYPE_BF16
    fmt = {"int8": None, "nvfp4": hdq.FMT_NVFP4, "nvfp4_mx": hdq.FMT_NVFP4_MX,
           "nvfp4_p2": hdq.FMT_NVFP4_P2}[path]
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=fmt)
    xd = to_dev(x16)
    prec = hdq.PREC_INT8 if path == "int8" else hdq.PREC_NVFP4
    say(f"config {cfg} {path}: GPU linear")
    y = hdq.linear(prec, xd, W, y_dtype=y_dtype)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    cols = np.unique(np.concatenate([np.arange(min(n_cols // 2, N)),
                                     np.linspace(0, N - 1, n_cols // 2).astype(np.int64)]))
    say(f"config {cfg} {path}: oracle on {len(rows)} rows x {len(cols)} cols")
    xs = np.ascontiguousarray(x16[rows])
    ws = np.ascontiguousarray(w16[cols])
    if path == "int8":
        qa, sa = O.quant_int(xs, hb, 127)
        qw, sw = O.quant_int(ws, hb, 7)
        ref, _ = O.gemm_int(qa, sa, qw, sw)
        ref = ref.astype(np.float64)
        # the sampled rows' codes must also equal the GPU's
        gq = hdq.quantize(xd, hb, hdq.FMT_INT8_ROW)
        torch.cuda.synchronize()
        assert np.array_equal(gq.row_scale.cpu().numpy()[rows], sa)
        assert_codes_equal(gq.codes.cpu().numpy()[rows], qa, "codes")
    else:
        mx = FP4_FMTS[fmt]
        amax = O.rotated_amax(x16, hb)          # tensor amax over all rows
        wamax = O.rotated_amax(w16, hb)
        ac, ae, ast = O.quant_nvfp4(xs, hb, amax=amax, mx=mx)
        wc, we, wst = O.quant_nvfp4(ws, hb, amax=wamax, mx=mx)
        ref = O.gemm_nvfp4(ac, ae, ast, wc, we, wst, K)
        S = abs_products_nvfp4(ac, ae, ast, wc, we, wst, K)
    ref64 = ref
    ref = round_like(ref, y_dtype)
    got = y_np(y)[np.ix_(rows, cols)]
    err = rel_fro(got, ref)
    say(f"config {cfg} {path}: rel fro {err:.3e}")
    assert err <= REL_TOL
    if path == "int8":
        assert np.array_equal(got, ref)
    else:
        worst = assert_elementwise(got, ref64, S, K, y_dtype == hdq.DTYPE_BF16, f"config {cfg} {path}")
        say(f"config {cfg} {path}: worst error / per-element bound {worst:.3f}")


@pytest.mark.parametrize("cfg,path", [(1, "int8"), (1, "nvfp4"), (1, "nvfp4_mx"), (1, "nvfp4_p2"),
                                      (2, "int8"), (3, "nvfp4"), (3, "nvfp4_mx"), (3, "nvfp4_p2"),
                                      (4, "int8")])
def test_config_full_size_sampled(cfg, path):
    run_config(cfg, path)


def test_config1_full_oracle():
    # the 1024^3 case is small enough for the oracle on every output
    c = synth.CONFIGS[1]
    x16, w16 = synth.config_activations(1), synth.config_weights(1)
    hb = c["had_block"]
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=hdq.FMT_NVFP4)
    y = hdq.linear(hdq.PREC_NVFP4, to_dev(x16), W, y_dtype=hdq.DTYPE_F32)
    torch.cuda.synchronize()
    ac, ae, ast = O.quant_nvfp4(x16, hb)
    wc, we, wst = O.quant_nvfp4(w16, hb)
    ref64 = O.gemm_nvfp4(ac, ae, ast, wc, we, wst, 1024)
    ref = ref64.astype(np.float32)
    assert rel_fro(y.cpu().numpy(), ref) <= REL_TOL
    assert_elementwise(y_np(y), ref64, abs_products_nvfp4(ac, ae, ast, wc, we, wst, 1024), 1024, False, "config 1")


# ------------------------------ the mixed-precision schedule, full size

def schedule_call(prev_in, prev_out, x, W, hb, fmt4):
    """One layer call as the schedule enqueues it: selection, then both
    quantizers and all three GEMMs behind the device-side decision."""
    M, K = x.shape
    dec, st = hdq.select_precision(prev_in, prev_out, x, hb, 0.1, 50.0)
    xq8 = hdq.quantize(x, hb, hdq.FMT_INT8_ROW, decision=dec)
    xq4 = hdq.quantize(x, hb, fmt4, tensor_amax=st[4:5], decision=dec)
    y = torch.zeros(M, W.N, dtype=torch.bfloat16, device=DEV)
    hdq.linear(hdq.PREC_INT8, None, W, decision=dec, xq=xq8, y=y)
    hdq.linear(hdq.PREC_NVFP4, None, W, decision=dec, xq=xq4, y=y)
    hdq.linear(hdq.PREC_BF16, x, W, decision=dec, y=y)
    torch.cuda.synchronize()
    return int(dec.item()), st.cpu().numpy().astype(np.float64), y


@pytest.mark.parametrize("layer", range(len(synth.SCHEDULE_LAYERS)))
def test_schedule_layer_calls_match_oracle(layer):
    """CogVideoX-5B block layers at M = 17776 tokens: a low-noise step
    (NVFP4), a high-noise step (INT8) and, on the first layer, an input with
    outlier channels (bf16 fallback).  Inputs come from the seeded device
    generator; the oracle reads byte copies of what the GPU consumed."""
    name, K, N = synth.SCHEDULE_LAYERS[layer]
    M, hb = synth.M_COGVIDEOX, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1000 + layer)
    x = synth.device_gaussian((M, K), 1.0, gen, DEV)
    w = synth.device_gaussian((N, K), 0.02, gen, DEV)
    W = hdq.LinearWeights(w, hb, fp4_fmt=hdq.FMT_NVFP4_MX)
    w16 = bf16_to_np(w)
    rows = sample_rows(M, 24, 24)
    cols = np.unique(np.concatenate([np.arange(32), np.linspace(0, N - 1, 64).astype(np.int64)]))
    ws = np.ascontiguousarray(w16[cols])
    qw, sw = O.quant_int(ws, hb, 7)
    wc, we, wst = O.quant_nvfp4(ws, hb, amax=O.rotated_amax(w16, hb), mx=True)
    cases = [("low noise", 0.03, None), ("high noise", 0.25, None)]
    if layer == 0:
        cases.append(("outlier channels", 0.03, 400.0))
    for what, s, outlier in cases:
        xi = x
        if outlier is not None:
            xi = x.clone()
            xi[:, 7] *= outlier
        prev_out = synth.device_noisy_copy(xi, s, gen)
        dec, st, y = schedule_call(xi.clone(), prev_out, xi, W, hb, hdq.FMT_NVFP4_MX)
        x16, po16 = bf16_to_np(xi), bf16_to_np(prev_out)
        ref = O.stats(x16, po16, x16, hb)
        say(f"schedule {name} {what}: decision {dec}, delta {st[0]:.4f}, ratio {st[1]:.2f}")
        assert abs(st[0] - ref[0]) <= 2e-6 * ref[0]
        assert abs(st[1] - ref[1]) <= 2e-6 * ref[1]
        assert st[4] == np.float32(ref[4])
        assert decision_ok(dec, ref, True)
        want = {"low noise": hdq.PREC_NVFP4, "high noise": hdq.PREC_INT8,
                "outlier channels": hdq.PREC_BF16}[what]
        assert dec == want
        xs = np.ascontiguousarray(x16[rows])
        S = None
        if dec == hdq.PREC_INT8:
            qa, sa = O.quant_int(xs, hb, 127)
            r, _ = O.gemm_int(qa, sa, qw, sw)
            r = r.astype(np.float64)
        elif dec == hdq.PREC_NVFP4:
            ac, ae, ast = O.quant_nvfp4(xs, hb, amax=np.float32(ref[4]), mx=True)
            r = O.gemm_nvfp4(ac, ae, ast, wc, we, wst, K)
            S = abs_products_nvfp4(ac, ae, ast, wc, we, wst, K)
        else:
            r = O.gemm_bf16(xs, ws)
            S = abs_products_bf16(xs, ws)
        r64 = r
        r = round_like(r, hdq.DTYPE_BF16)
        got = y_np(y)[np.ix_(rows, cols)]
        err = rel_fro(got, r)
        say(f"schedule {name} {what}: rel fro {err:.3e}")
        assert err <= REL_TOL
        if dec == hdq.PREC_INT8:
            assert np.array_equal(got, r)
        else:
            assert_elementwise(got, r64, S, K, True, f"schedule {name} {what}")


# ------------------------------------------------- temporal delta cache

def test_tdc_decide_matches_oracle():
    say("tdc decide random states")
    rng = np.random.default_rng(120)
    n = 5000
    state = rng.integers(0, 3, n).astype(np.int32)
    base = rng.uniform(0.0, 10.0, n)
    base[rng.random(n) < 0.05] = 0.0
    diff = base * rng.uniform(0.0, 0.12, n)
    diff[rng.random(n) < 0.05] = 0.0
    diff[(base == 0) & (rng.random(n) < 0.5)] = 1.0
    sums = np.stack([diff, base], axis=1)
    c = rng.uniform(0.0, 0.1, n).astype(np.float32)
    c[rng.random(n) < 0.1] = np.nan
    acc = rng.uniform(0.0, 0.15, n).astype(np.float32)
    gc, gacc = torch.from_numpy(c.copy()).to(DEV), torch.from_numpy(acc.copy()).to(DEV)
    skip = hdq.tdc_decide(torch.from_numpy(sums).to(DEV), torch.from_numpy(state).to(DEV), gc, gacc)
    torch.cuda.synchronize()
    ref = O.tdc_decide(sums, state, c, acc)
    assert np.array_equal(skip.cpu().numpy(), ref)
    assert np.array_equal(gc.cpu().numpy().view(np.uint32), c.view(np.uint32))
    assert np.array_equal(gacc.cpu().numpy().view(np.uint32), acc.view(np.uint32))
    assert 0.1 < ref.mean() < 0.9


def test_tdc_decide_with_partial_sums_matches_oracle():
    """hdq_tdc_decide with change sums given as pairs per module (offsets): the
    pairs are dyadic, so every summation order gives the totals exactly, and
    the rule must match the oracle's on those totals bit for bit."""
    say("tdc decide, partial sums")
    rng = np.random.default_rng(121)
    n = 700
    state = rng.integers(0, 3, n).astype(np.int32)
    counts = rng.integers(0, 40, n)
    counts[state == 2] = np.maximum(counts[state == 2], 1)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    base_p = rng.integers(0, 2000, off[-1]).astype(np.float64) * 2.0 ** -10
    diff_p = np.floor(base_p * rng.uniform(0.0, 0.12, off[-1]) * 1024.0) * 2.0 ** -10
    parts = np.stack([diff_p, base_p], axis=1)
    tot = np.stack([np.add.reduceat(parts[:, 0], off[:-1]) if off[-1] else np.zeros(n),
                    np.add.reduceat(parts[:, 1], off[:-1]) if off[-1] else np.zeros(n)], axis=1)
    tot[counts == 0] = 0.0                   # reduceat repeats the next value for empty ranges
    c = rng.uniform(0.0, 0.1, n).astype(np.float32)
    c[rng.random(n) < 0.1] = np.nan
    acc = rng.uniform(0.0, 0.15, n).astype(np.float32)
    gc, gacc = torch.from_numpy(c.copy()).to(DEV), torch.from_numpy(acc.copy()).to(DEV)
    skip = hdq.tdc_decide(torch.from_numpy(parts).to(DEV), torch.from_numpy(state).to(DEV), gc, gacc,
                          offsets=torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    ref = O.tdc_decide(tot, state, c, acc)
    assert np.array_equal(skip.cpu().numpy(), ref)
    assert np.array_equal(gc.cpu().numpy().view(np.uint32), c.view(np.uint32))
    assert np.array_equal(gacc.cpu().numpy().view(np.uint32), acc.view(np.uint32))
    assert 0.1 < ref.mean() < 0.9


def test_tdc_trajectory_matches_oracle():
    """Three linear modules over a trajectory whose input changes shrink step
    by step: computed modules run the INT8 linear, the change statistic of
    each new output against the earlier one comes from hdq_delta_sums, and
    the GPU rule's skip pattern, c and acc equal the oracle rule's on the
    same sums; the sums themselves equal the oracle's relative L1 change."""
    say("tdc trajectory")
    M, K, N, hb, T = 300, 256, 192, 64, 14
    mods = []
    for m in range(3):
        rng = synth.rng_for(121, m)
        x0 = rng.standard_normal((M, K)).astype(np.float32)
        d = rng.standard_normal((M, K)).astype(np.float32)
        w16 = synth.gaussian(N, K, 0.02, synth.rng_for(122, m))
        mods.append(dict(x0=x0, d=d, W=hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=None), y=None))
    n = len(mods)
    gc = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    gacc = torch.zeros(n, dtype=torch.float32, device=DEV)
    c = np.full(n, np.nan, np.float32)
    acc = np.zeros(n, np.float32)
    skip = np.zeros(n, np.int32)
    a = 0.0
    skips = 0
    for t in range(T):
        a += 0.3 * 0.6 ** t                      # the input moves less every step
        sums = np.zeros((n, 2), np.float64)
        gsums = torch.zeros((n, 2), dtype=torch.float64, device=DEV)
        state = np.zeros(n, np.int32)
        for i, md in enumerate(mods):
            if skip[i]:
                skips += 1
                continue
            x16 = synth.to_bf16_bits(md["x0"] + np.float32(a) * md["d"])
            y = hdq.linear(hdq.PREC_INT8, to_dev(x16), md["W"], y_dtype=hdq.DTYPE_BF16)
            if md["y"] is None:
                state[i] = 1
            else:
                state[i] = 2
                hdq.delta_sums(md["y"], y, sums=gsums[i])
                torch.cuda.synchronize()
                y_old = md["y"].view(torch.int16).cpu().numpy().view(np.uint16)
                y_new = y.view(torch.int16).cpu().numpy().view(np.uint16)
                o = O.stats(y_old, y_new, y_new, 0)[0]
                g = gsums[i].cpu().numpy()
                assert abs(g[0] / g[1] - o) <= 1e-12 * max(o, 1e-30), (t, i)
                sums[i] = g
            md["y"] = y
        gskip = hdq.tdc_decide(gsums, torch.from_numpy(state).to(DEV), gc, gacc)
        skip = O.tdc_decide(sums, state, c, acc)
        torch.cuda.synchronize()
        assert np.array_equal(gskip.cpu().numpy(), skip), t
        assert np.array_equal(gc.cpu().numpy().view(np.uint32), c.view(np.uint32)), t
        assert np.array_equal(gacc.cpu().numpy().view(np.uint32), acc.view(np.uint32)), t
    assert skips > 0            # the smoothing trajectory does reuse the cache
