"""GPU <-> oracle parity of the DeltaQuant cube-delta path (DeltaQuant abstract,
paper-radar CVPR 2026 listing) through the C ABI: core codes, core scales,
difference codes, block and tensor scales bit-exact (both sides round the
same float32 values in the same order); decoded weights exact; the linear
output within relative Frobenius 1e-3 of the oracle's double result (full
size: on sampled rows)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_video_amd import synth

import dq_cases

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
from bit_quantized_video_amd import hdq  # noqa: E402  (loads libhdq.so; fails loudly if missing)

DEV = torch.device("cuda:0")
MX = {hdq.FMT_NVFP4: 0, hdq.FMT_NVFP4_MX: 1, hdq.FMT_NVFP4_P2: 2}
FMTS = {"nvfp4": hdq.FMT_NVFP4, "mx": hdq.FMT_NVFP4_MX, "p2": hdq.FMT_NVFP4_P2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).to(DEV).view(torch.bfloat16)


def u8(t):
    return t.cpu().numpy().view(np.uint8)


def check_quantize(x16, F, H, W, cube, fmt):
    a = hdq.dq_quantize(to_dev(x16), (F, H, W, cube), fmt, core_bf16=True)
    q = O.dq_quantize(x16, F, H, W, cube, MX[fmt])
    torch.cuda.synchronize()
    assert np.array_equal(u8(a.core), q["core"])
    assert np.array_equal(a.core_scale.cpu().numpy().view(np.uint32), q["core_scale"].view(np.uint32))
    core_vals = O.e4m3s_decode(q["core"])
    assert np.array_equal(a.core_bf16.float().cpu().numpy(), core_vals)
    assert float(a.delta.tensor_scale.item()) == float(q["s_t"])
    assert np.array_equal(u8(a.delta.blk_scale), q["blk"])
    assert np.array_equal(u8(a.delta.codes), q["codes"])
    return a, q


@pytest.mark.parametrize("grid,cube,K,fmt", [
    ((3, 5, 7), (2, 2, 2), 64, "nvfp4"), ((3, 5, 7), (2, 2, 2), 64, "mx"), ((3, 5, 7), (1, 1, 1), 96, "p2"),
    ((4, 6, 10), (2, 3, 4), 256, "mx"), ((2, 3, 3), (2, 3, 3), 32, "nvfp4"), ((5, 4, 9), (4, 4, 4), 512, "mx"),
    # cubes of <= 8 tokens take the register-resident core pass: one chunk
    # column per thread up to K 8192 (1024 threads), four up to 16384; past
    # that, and for larger cubes, the two-read pass
    ((3, 3, 5), (2, 2, 2), 8192, "mx"), ((2, 3, 3), (2, 2, 2), 12288, "p2"), ((2, 2, 3), (2, 2, 2), 16416, "nvfp4"),
    ((3, 5, 6), (1, 2, 2), 3072, "mx")])
def test_dq_quantize_bit_exact(grid, cube, K, fmt):
    F, H, W = grid
    say(f"dq quantize grid={grid} cube={cube} K={K} {fmt}")
    x16 = synth.smooth_video_tokens(F, H, W, K, synth.rng_for(130, K + F))
    check_quantize(x16, F, H, W, cube, FMTS[fmt])


def test_dq_quantize_constant_cubes_give_zero_differences():
    """Tokens equal to an on-grid core: zero differences, zero tensor scale,
    all-zero codes and block scales (the degenerate case of the method)."""
    F, H, W, K, cube = 2, 4, 4, 64, (2, 2, 2)
    row = np.array([1.0, -1.5, 2.0, -3.0, 4.0, 6.0, -8.0, 14.0] * (K // 8), np.float32)
    x16 = synth.to_bf16_bits(np.tile(row, (F * H * W, 1)))
    a, q = check_quantize(x16, F, H, W, cube, hdq.FMT_NVFP4_MX)
    assert q["s_t"] == 0.0 and not u8(a.delta.codes).any()


def test_dq_quantize_full_size_video_grid():
    """The CogVideoX-5B latent video grid (13 x 30 x 45 = 17550 tokens), K 3072,
    2 x 2 x 2 cubes (ragged in frames and columns): every byte as the oracle."""
    F, H, W, K = 13, 30, 45, 3072
    say("dq quantize full size")
    x16 = synth.smooth_video_tokens(F, H, W, K, synth.rng_for(131, 0))
    check_quantize(x16, F, H, W, (2, 2, 2), hdq.FMT_NVFP4_MX)


@pytest.mark.parametrize("cube", [(2, 2, 2), (2, 2, 4)])
@pytest.mark.parametrize("fmt", ["mx", "nvfp4"])
def test_dq_nonfinite_flag_and_extreme_values(cube, fmt):
    """Non-finite tokens: wherever the oracle flags a non-finite difference
    (a NaN or infinite element, a cube sum or a difference past float32's
    range) the GPU's tensor scale is NaN too; the finite extreme case (a cube
    summing to the largest bf16, a bf16 subnormal) matches the oracle byte for
    byte.  Cubes of 8 tokens take the register-resident pass, of 16 the
    two-read pass."""
    F, H, W, K, cases = dq_cases.nonfinite_cases()
    for name, (x, _) in cases.items():
        say(f"dq non-finite case {name!r} cube={cube} {fmt}")
        x16 = synth.to_bf16_bits(x)
        q = O.dq_quantize(x16, F, H, W, cube, MX[FMTS[fmt]])
        if np.isnan(q["s_t"]):
            a = hdq.dq_quantize(to_dev(x16), (F, H, W, cube), FMTS[fmt])
            torch.cuda.synchronize()
            assert np.isnan(float(a.delta.tensor_scale.item())), name
        else:
            check_quantize(x16, F, H, W, cube, FMTS[fmt])


@pytest.mark.parametrize("fmt", ["nvfp4", "mx", "p2"])
def test_dq_decode_weights_exact(fmt):
    N, K = 96, 256
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(132, 0))
    wq = hdq.quantize(to_dev(w16), 1, FMTS[fmt])
    dec = hdq.dq_decode_weights(wq)
    c, e, st = O.quant_nvfp4(w16, 1, mx=MX[FMTS[fmt]])
    torch.cuda.synchronize()
    assert np.array_equal(u8(wq.codes), c) and np.array_equal(u8(wq.blk_scale), e)
    assert np.array_equal(dec.float().cpu().numpy(), O.dequant_nvfp4(c, e, 1.0, K))


def core_fp8_mfma_bound(core, wabs, fmt):
    """Error bound of the core GEMM on the FP8 x FP4 scaled MFMA, [cubes, N].
    That instruction does not sum its 64 products at float32 precision: on
    gfx950 the error of one instruction measured at most 2^-10.1 of its
    largest |product| (random and one-signed codes over the whole E4M3 range,
    65536 outputs per pattern), consistent with products aligned to the
    largest one's exponent and kept to at least 14 fraction bits, which bounds
    64 products by 2^-8 max|p|.  Per 64-k step: 2^-8 max_k |core_k w_k|, twice
    for the per-16 format's two passes."""
    C, K = core.shape
    out = np.zeros((C, wabs.shape[0]))
    for k0 in range(0, K, 64):
        pm = np.max(core[:, None, k0:k0 + 64] * wabs[None, :, k0:k0 + 64], axis=2)
        out += pm
    return (2.0 if fmt == hdq.FMT_NVFP4_P2 else 1.0) * 2.0 ** -8 * out


def linear_case(F, H, W, K, N, cube, fmt, rows=None, y_dtype=hdq.DTYPE_BF16, seed=0):
    """The GPU linear against the oracle's double result computed from the
    oracle's own codes (rows: the tokens compared; all when None).  Returns the
    relative Frobenius error; asserts the GPU's codes on those rows are the
    oracle's and the per-element bound: float32 accumulation over K (c u S,
    c = max(4, 2 sqrt(K / 16)), S = sum_k |d_k w_k| + sum_k |core_k w_k|), the
    epilogue's roundings (4 u |ref|) and half a bf16 ulp for bf16 output."""
    x16 = synth.smooth_video_tokens(F, H, W, K, synth.rng_for(133, seed))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(134, seed))
    a = hdq.dq_quantize(to_dev(x16), (F, H, W, cube), fmt)
    wq = hdq.quantize(to_dev(w16), 1, fmt)
    y = hdq.dq_linear(a, wq, hdq.dq_decode_weights(wq), y_dtype=y_dtype)
    torch.cuda.synchronize()
    rows = np.arange(F * H * W) if rows is None else np.asarray(rows)
    q = O.dq_quantize(x16, F, H, W, cube, MX[fmt])
    assert np.array_equal(u8(a.delta.codes)[rows], q["codes"][rows])
    assert np.array_equal(u8(a.delta.blk_scale)[rows], q["blk"][rows])
    assert np.array_equal(u8(a.core), q["core"]) and float(a.delta.tensor_scale.item()) == float(q["s_t"])
    wc, we, wst = O.quant_nvfp4(w16, 1, mx=MX[fmt])
    ref64 = O.dq_linear(q, wc, we, wst, K, F, H, W, cube, rows=rows)
    got = y.float().cpu().numpy()[rows].astype(np.float64)
    ref = ref64
    if y_dtype == hdq.DTYPE_BF16:      # the oracle's result rounded to the output dtype
        ref = synth.bf16_bits_to_f32(O.f32_to_bf16(ref64.astype(np.float32))).astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    # per-element bound
    wabs = np.abs(O.dequant_nvfp4(wc, we, wst, K).astype(np.float64))
    dabs = np.abs(O.dequant_nvfp4(q["codes"][rows], q["blk"][rows], q["s_t"], K).astype(np.float64))
    core = np.abs(O.e4m3s_decode(q["core"]).astype(np.float64) * q["core_scale"].astype(np.float64)[:, None])
    cube_of = O.dq_cube_of(F, H, W, cube)[rows]
    S = dabs @ wabs.T + (core @ wabs.T)[cube_of]
    c = max(4.0, 2.0 * np.sqrt(K / 16.0))
    tol = c * 2.0 ** -24 * S + 4 * 2.0 ** -24 * np.abs(ref64) + 1e-35
    if not hdq.dq_core_needs_bf16(fmt, core.shape[0], K, wabs.shape[0]):
        tol = tol + core_fp8_mfma_bound(core, wabs, fmt)[cube_of]
    if y_dtype == hdq.DTYPE_BF16:
        tol = tol + 2.0 ** -8 * 1.01 * np.abs(got)
    bad = np.abs(got - ref64) > tol
    assert not bad.any(), f"{int(bad.sum())} outputs beyond the per-element bound"
    return err


@pytest.mark.parametrize("grid,cube,K,N,fmt", [((3, 5, 7), (2, 2, 2), 64, 40, "nvfp4"),
                                               # K 96: the bf16 core GEMM and the combine route for MX
                                               ((3, 5, 7), (2, 2, 2), 96, 40, "mx"),
                                               ((4, 6, 10), (2, 2, 2), 256, 300, "mx"),
                                               ((3, 8, 8), (1, 2, 2), 512, 96, "p2"),
                                               # four 256-token tiles of the fused epilogue
                                               ((4, 12, 20), (2, 2, 2), 512, 520, "p2"),
                                               ((4, 12, 20), (2, 3, 4), 512, 264, "mx")])
@pytest.mark.parametrize("y_dtype", [hdq.DTYPE_BF16, hdq.DTYPE_F32])
def test_dq_linear_matches_oracle(grid, cube, K, N, fmt, y_dtype):
    say(f"dq linear grid={grid} cube={cube} K={K} N={N} {fmt} y={y_dtype}")
    err = linear_case(*grid, K, N, cube, FMTS[fmt], y_dtype=y_dtype)
    say(f"  relative Frobenius error {err:.3g}")
    # float32 output: 1e-5 where the core GEMM accumulates at float32
    # precision (bf16 route); the FP8 x FP4 MFMA's narrower sum (bounded per
    # element above) measures about 1.5e-5 on these inputs, so 1e-4 there
    fp8 = not hdq.dq_core_needs_bf16(FMTS[fmt], hdq.dq_cubes((*grid, cube)), K, N)
    assert err <= (1e-3 if y_dtype == hdq.DTYPE_BF16 else 1e-4 if fp8 else 1e-5), err


def test_dq_linear_full_size_sampled_rows():
    """13 x 30 x 45 tokens, K 3072 -> N 12288 (the FFN up-projection's shape),
    MX format: the first 256 and last 112 tokens against the oracle's result
    from its own codes of the whole grid."""
    say("dq linear full size")
    M = 13 * 30 * 45
    rows = np.r_[0:256, M - 112:M]
    err = linear_case(13, 30, 45, 3072, 12288, (2, 2, 2), hdq.FMT_NVFP4_MX, rows=rows)
    assert err <= 1e-3, err
