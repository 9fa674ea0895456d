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
    a = hdq.dq_quantize(to_dev(x16), (F, H, W, cube), fmt)
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
    ((4, 6, 10), (2, 3, 4), 256, "mx"), ((2, 3, 3), (2, 3, 3), 32, "nvfp4"), ((5, 4, 9), (4, 4, 4), 512, "mx")])
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


def linear_case(F, H, W, K, N, cube, fmt, rows=None, y_dtype=hdq.DTYPE_BF16, seed=0):
    x16 = synth.smooth_video_tokens(F, H, W, K, synth.rng_for(133, seed))
    w16 = synth.gaussian(N, K, 0.02, synth.rng_for(134, seed))
    a = hdq.dq_quantize(to_dev(x16), (F, H, W, cube), fmt)
    wq = hdq.quantize(to_dev(w16), 1, fmt)
    y = hdq.dq_linear(a, wq, hdq.dq_decode_weights(wq), y_dtype=y_dtype)
    torch.cuda.synchronize()
    q = O.dq_quantize(x16, F, H, W, cube, MX[fmt]) if rows is None else None
    wc, we, wst = O.quant_nvfp4(w16, 1, mx=MX[fmt])
    if rows is None:
        ref = O.dq_linear(q, wc, we, wst, K, F, H, W, cube)
        got = y.float().cpu().numpy()
    else:
        # sampled rows: the GPU's own codes (bit-exact with the oracle's, checked
        # above at this size) in the oracle's double GEMMs
        cube_of = O.dq_cube_of(F, H, W, cube)
        sub = dict(codes=u8(a.delta.codes)[rows], blk=u8(a.delta.blk_scale)[rows],
                   s_t=np.float32(a.delta.tensor_scale.item()), core=u8(a.core), core_scale=a.core_scale.cpu().numpy())
        yd = O.gemm_nvfp4(sub["codes"], sub["blk"], sub["s_t"], wc, we, wst, K)
        cubes = cube_of[rows]
        core = O.e4m3s_decode(sub["core"][cubes]).astype(np.float64) * sub["core_scale"][cubes].astype(np.float64)[:, None]
        ref = yd + (core @ O.dequant_nvfp4(wc, we, 1.0, K).astype(np.float64).T) * float(wst)
        got = y.float().cpu().numpy()[rows]
    if y_dtype == hdq.DTYPE_BF16:      # the oracle's result rounded to the output dtype
        ref = synth.bf16_bits_to_f32(synth.to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    return err


@pytest.mark.parametrize("grid,cube,K,N,fmt", [((3, 5, 7), (2, 2, 2), 64, 40, "nvfp4"),
                                               ((4, 6, 10), (2, 2, 2), 256, 300, "mx"),
                                               ((3, 8, 8), (1, 2, 2), 512, 96, "p2")])
@pytest.mark.parametrize("y_dtype", [hdq.DTYPE_BF16, hdq.DTYPE_F32])
def test_dq_linear_matches_oracle(grid, cube, K, N, fmt, y_dtype):
    say(f"dq linear grid={grid} cube={cube} K={K} N={N} {fmt} y={y_dtype}")
    err = linear_case(*grid, K, N, cube, FMTS[fmt], y_dtype=y_dtype)
    assert err <= (1e-3 if y_dtype == hdq.DTYPE_BF16 else 1e-5), err


def test_dq_linear_full_size_sampled_rows():
    """13 x 30 x 45 tokens, K 3072 -> N 12288 (the FFN up-projection's shape),
    MX format: the first 256 and last 112 tokens against the oracle."""
    say("dq linear full size")
    M = 13 * 30 * 45
    rows = np.r_[0:256, M - 112:M]
    err = linear_case(13, 30, 45, 3072, 12288, (2, 2, 2), hdq.FMT_NVFP4_MX, rows=rows)
    assert err <= 1e-3, err
