"""DeltaQuant token sets for the non-finite flag, shared by the oracle pin
and the GPU parity test (inputs only: values built by hand, with the oracle's
bf16 codec and cube map used to place them)."""
import numpy as np

import oracle as O
from bit_quantized_video_amd import synth


def nonfinite_cases():
    """Token sets (float32 values, exactly representable in bf16) for the
    non-finite flag: 2x2x2 cubes of a 2x2x4 grid, K 32."""
    F, H, W, K = 2, 2, 4, 32
    base = np.random.default_rng(9).standard_normal((F * H * W, K)).astype(np.float32)
    base = O.bf16_to_f32(synth.to_bf16_bits(base))
    big = np.float32(O.bf16_to_f32(np.array([0x7f7f], np.uint16))[0])   # largest finite bf16, 3.39e38
    cases = {}
    x = base.copy(); x[5, 3] = np.nan; cases["nan element"] = (x, True)
    x = base.copy(); x[0, 7] = np.inf; cases["+inf element"] = (x, True)
    x = base.copy(); x[9, 0] = -np.inf; x[1, 0] = np.inf; cases["+inf and -inf in one cube"] = (x, True)
    cube_of = O.dq_cube_of(F, H, W, (2, 2, 2))
    idx = np.flatnonzero(cube_of == 0)
    x = base.copy(); x[idx, 4] = big; cases["cube sum overflows"] = (x, True)
    # token 0 at +big, the other seven at -big/4: every partial sum stays
    # finite (mean -0.09375 big) but token 0's difference, 1.09375 big, does not
    x = base.copy(); x[idx, 4] = -big / 4; x[idx[0], 4] = big; cases["difference overflows"] = (x, True)
    x = base.copy(); x[idx, 4] = big / 8; x[idx[1], 5] = np.float32(1e-38); cases["large and tiny, finite"] = (x, False)
    return F, H, W, K, cases
