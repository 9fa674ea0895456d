"""Host logic of the benchmark's embedded difference plan (no GPU): every
layer call's difference chunks are planned exactly once, before that call's
own GEMM launch, and no launch carries more slices than the C-ABI takes."""
import argparse

import pytest

import bench
import bit_quantized_video_amd.hdq as H
from bit_quantized_video_amd import synth


@pytest.mark.parametrize("weight", ["capacity", "work"])
@pytest.mark.parametrize("blocks,timesteps", [(42, 3), (2, 3), (1, 1)])
def test_embed_plan_covers_every_chunk_in_time(blocks, timesteps, weight):
    M = synth.M_COGVIDEOX
    args = argparse.Namespace(timesteps=timesteps, blocks=blocks, dispatch="on", delta="embed",
                              embed_weight=weight)
    P = bench.embed_plan(args, H, synth, M, "cpu")
    plan = P["embed"]
    calls = [(t, b, li) for t in range(timesteps) for b in range(blocks)
             for li in range(len(synth.SCHEDULE_LAYERS))]
    assert len(plan) == len(calls)
    got = {}
    for k, slices in enumerate(plan):
        assert len(slices) <= H.DELTA_MAX_SLICES
        for j, c0, c1 in slices:
            assert k + 1 <= j < len(calls) and 0 <= c0 < c1   # before call j's own launch
            got.setdefault(j, []).append((c0, c1))
    for j in range(1, len(calls)):
        n = H.delta_chunks(M * synth.SCHEDULE_LAYERS[calls[j][2]][1])
        r = sorted(got[j])
        assert r[0][0] == 0 and r[-1][1] == n and all(a[1] == b[0] for a, b in zip(r, r[1:]))
        assert tuple(P["embed_parts"][j].shape) == (n, 2)
    assert 0 not in got       # call 0's difference runs on its own
