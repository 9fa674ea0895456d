"""The allocation-free fused selection + INT8 quantization
(hdq_select_quantize_int8_noalloc) against the workspace entry point
(hdq_select_quantize_int8) through the C ABI: decision, statistics, codes and
row scales bit for bit, on consecutive calls that share the library's fixed
scratch, the later ones smaller, with and without a previous-step difference,
on both routes (rows kept in registers, and the two passes for rows over
16384 columns); inputs over the fixed scratch are rejected before any work."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).to(DEV).view(torch.bfloat16)


def run_both(x, sums, hb):
    """The workspace call and the allocation-free call on the same input,
    each into its own outputs; returns both (decision, stats, codes, scales)."""
    rows, cols = x.shape
    d1, s1, q1 = hdq.select_quantize_int8(sums, x, hb)
    d2 = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    s2 = torch.full((5,), float("nan"), dtype=torch.float32, device=DEV)
    q2 = hdq.QuantizedTensor(hdq.FMT_INT8_ROW, rows, cols, hb, DEV)
    q2.codes.fill_(99)
    q2.row_scale.fill_(-1.0)
    hdq.select_quantize_int8_noalloc(sums, x, hb, d2, s2, q2)
    torch.cuda.synchronize()
    return (d1, s1, q1), (d2, s2, q2)


def assert_same(a, b, what):
    (d1, s1, q1), (d2, s2, q2) = a, b
    assert int(d1.item()) == int(d2.item()), what
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), what       # NaN delta included
    assert torch.equal(q1.codes, q2.codes), what
    assert torch.equal(q1.row_scale.view(torch.int32), q2.row_scale.view(torch.int32)), what
    assert q2.fmt == hdq.FMT_INT8_ROW and q2.had_block == q1.had_block


@pytest.mark.parametrize("shapes", [[(17776, 3072), (333, 1024)], [(4096, 20480), (1000, 12288), (9, 128)]])
def test_noalloc_matches_workspace_entry_point(shapes):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    for i, (rows, cols) in enumerate(shapes):
        say(f"noalloc select+int8 call {i}: {rows} x {cols}")
        x = synth.device_gaussian((rows, cols), 1.0, gen, DEV)
        if i % 2:
            x[:, 5] *= 300.0                           # outlier channel: the decision flips to bf16
        prev_out = synth.device_noisy_copy(x, 0.05 + 0.1 * i, gen)
        sums = hdq.delta_sums(x, prev_out)
        for hist in (sums, None):
            a, b = run_both(x, hist, 128)
            assert_same(a, b, (rows, cols, hist is None))
        say(f"noalloc call {i}: decision {int(a[0].item())}")


def test_noalloc_rejects_inputs_beyond_the_fixed_scratch():
    rows = hdq.NOALLOC_SCRATCH_BYTES // 48 + 1
    assert hdq.workspace_bytes(hdq.OP_SELECT_Q8, rows, 256, 0) > hdq.NOALLOC_SCRATCH_BYTES
    assert hdq.workspace_bytes(hdq.OP_SELECT_Q8, rows - 1, 256, 0) <= hdq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(rows, 256, dtype=torch.bfloat16, device=DEV)
    d = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.zeros(5, dtype=torch.float32, device=DEV)
    q = hdq.QuantizedTensor(hdq.FMT_INT8_ROW, rows, 256, 64, DEV)
    with pytest.raises(hdq.HdqError) as e:
        hdq.select_quantize_int8_noalloc(None, x, 64, d, s, q)
    assert e.value.status == hdq.ERR_TOO_LARGE
    # the largest accepted input still runs, and matches the workspace call
    xs = x[: rows - 1]
    xs.normal_()
    a, b = run_both(xs, None, 64)
    assert_same(a, b, "largest accepted")
