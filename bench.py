#!/usr/bin/env python
"""Benchmark of the DMPQ hot path on one MI355X.

Workload (one "step"): the dynamic mixed-precision schedule over 42
CogVideoX-5B-shaped transformer blocks x 4 linear layers (QKV 3072->9216,
attention out 3072->3072, FFN up 3072->12288, FFN down 12288->3072) x 3
denoising timesteps, M = 17776 tokens (13 latent frames x 1350 patches + 226
text tokens).  Per layer and timestep, on the device with no host round trip:
  1. hdq_select_precision: relative-L1 difference of the previous step's
     input/output (threshold 0.1: INT8 above, NVFP4 below) and the outlier
     ratio max|x|/mean|x| of the input (above 50: bf16 fallback);
  2. hdq_quantize, gated by that decision: block-Hadamard (128) rotation
     fused with INT8 per-token or NVFP4 quantization;
  3. hdq_linear, gated: INT8 x INT4, NVFP4 x NVFP4 or bf16 x bf16 GEMM.
Inputs are synthetic and resident in HBM before timing: per (block, layer)
two bf16 activations A ~ N(0, 1) and B = A + N(0, 0.1), the inputs of
alternating timesteps (t even: A, odd: B), so every step's input differs from
the previous step's; the previous step's output is the previous step's input
+ N(0, s), s ~ U(0.01, 0.3) per (block, layer, timestep); weights ~ N(0,
0.02) per (block, layer), prepared (rotated + quantized) before timing.

metric: effective TOPS = sum over layer calls of 2 M N K / step time (the
step time includes selection, quantization and the gated-off launches).
Per-kernel durations come from HIP events recorded on the stream the
kernels run on, inside the timed region.

Other modes: --config {1,2,3,4} times one single-layer configuration
(quantize + GEMM); --profile-copy runs a plain 1 GiB device copy (the
reference for HBM-counter calibration).
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS of fused Hadamard-quant+linear (CogVideoX-5B shapes); quant GB/s"
PEAK = {"int8": 5.0e15, "bf16": 2.5e15, "fp8": 5.0e15, "fp4": 10.1e15, "hbm": 8.0e12}
HB = 128
DELTA_T, RATIO_T = 0.1, 50.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--blocks", type=int, default=42)
    ap.add_argument("--timesteps", type=int, default=3)
    ap.add_argument("--fp4", choices=["nvfp4", "mx", "p2"], default="mx",
                    help="NVFP4 recipe of the headline run: MX-compatible (FP4 MFMA, default), "
                         "plain (exact, bf16 MFMA) or a power of two per 16-block (FP4 MFMA, two "
                         "passes); the schedule also times the other two")
    ap.add_argument("--config", type=int, default=5, help="5: schedule; 1-4: one linear layer")
    ap.add_argument("--delta", choices=["embed", "overlap", "inline"], default="embed",
                    help="previous-step difference: in chunks on extra workgroups of earlier layer "
                         "calls' GEMM launches (embed, default; needs --dispatch on), on a second "
                         "stream ahead of each layer call (overlap) or inside the selection pass "
                         "(inline)")
    ap.add_argument("--fuse", choices=["on", "off"], default="on",
                    help="selection fused with the INT8 per-token quantization of the input (on, "
                         "default; the codes are written whatever the decision) or separate")
    ap.add_argument("--dispatch", choices=["on", "off"], default="on",
                    help="one GEMM launch per layer call for the decided precision (on, default) "
                         "or one gated launch per precision")
    ap.add_argument("--embed-weight", choices=["capacity", "work"], default="capacity",
                    help="--delta embed: share the difference chunks among the GEMM launches by the CU "
                         "time each leaves free (the free CUs over the whole launch plus the workgroups "
                         "idle in its last tile round; default) or by GEMM work")
    ap.add_argument("--delta-ahead", type=int, default=2,
                    help="with --delta overlap: the difference of call k + D runs beside the GEMMs "
                         "of call k")
    ap.add_argument("--events", choices=["gemm", "all"], default="gemm",
                    help="HIP events in the timed steps: around each layer call's GEMM launch only "
                         "(default; the other kernels are timed in one instrumented step after the timed "
                         "ones), or around every kernel (each event record adds a marker to the stream, "
                         "which costs the step several percent)")
    ap.add_argument("--dq-steps", type=int, default=10,
                    help="timed calls of the DeltaQuant cube-delta path (quantize, linear) on the "
                         "13x30x45-token video grid, K 3072 -> N 12288; 0 skips it")
    ap.add_argument("--tdc-steps", type=int, default=12,
                    help="steps of the temporal-delta-cache trajectory measured after the schedule "
                         "(0: none)")
    ap.add_argument("--tdc-blocks", type=int, default=8,
                    help="blocks (x 4 linear modules) in the temporal-delta-cache trajectory")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config-reps", type=int, default=5,
                    help="timed repetitions of each single-layer configuration (1-4) the default run "
                         "reports beside the schedule; 0 skips them")
    ap.add_argument("--bf16-reps", type=int, default=5,
                    help="timed repetitions of the full-precision fallback layer calls (inputs whose "
                         "outlier ratio sends them to bf16); 0 skips them")
    ap.add_argument("--decisions-out", help="write the per-call precision decisions (call order) as JSON, "
                                            "for attributing one-launch GEMMs in profiles")
    ap.add_argument("--profile-copy", action="store_true")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers

class KernelTimes:
    """Accumulates (duration, algorithmic work) per kernel kind."""

    def __init__(self):
        self.t = {}
        self.work = {}
        self.bytes = {}
        self.n = {}

    def add(self, kind, ms, work, nbytes=0.0):
        self.t[kind] = self.t.get(kind, 0.0) + ms
        self.work[kind] = self.work.get(kind, 0.0) + work
        self.bytes[kind] = self.bytes.get(kind, 0.0) + nbytes
        self.n[kind] = self.n.get(kind, 0) + 1

    def summary(self):
        out = {}
        for k in sorted(self.t):
            out[k] = {"launches": self.n[k], "total_ms": round(self.t[k], 3),
                      "avg_us": round(1e3 * self.t[k] / self.n[k], 2),
                      "bytes_per_launch": self.bytes[k] / self.n[k],
                      "rate": self.work[k] / (self.t[k] * 1e-3) if self.t[k] > 0 else 0.0}
        return out


def quant_bytes(M, K, prec, decoded=False):
    """Algorithmic HBM bytes of one fused rotate+quantize of X [M, K] bf16
    (decoded: the NVFP4 codes' exact bf16 values written as well)."""
    if prec == "int8":
        return 2 * M * K + M * K + 4 * M
    return 2 * M * K + M * K // 2 + M * K // 16 + 4 + 4 + (2 * M * K if decoded else 0)


def stats_bytes(M, K):
    return 3 * 2 * M * K


def gemm_bytes(M, N, K, prec, fp4):
    """Algorithmic HBM bytes of one GEMM launch: each operand read once
    (codes + scales) and the bf16 output written once."""
    if prec == "int8":
        a, b = M * K + 4 * M, N * K // 2 + 4 * N
    elif prec == "bf16":
        a, b = 2 * M * K, 2 * N * K
    elif fp4 == "nvfp4":  # plain NVFP4: both operands' exact bf16 values
        a, b = 2 * M * K, 2 * N * K
    else:  # NVFP4 on the FP4 MFMA: packed E2M1 + one scale byte per 16 elements (MX: one per 32)
        g = 32 if fp4 == "mx" else 16
        a, b = M * K // 2 + M * K // g, N * K // 2 + N * K // g
    return a + b + 2 * M * N


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "schedule_hbm_traffic.txt")

# NVFP4 recipes: the oracle's mx argument, the format, a description
RECIPE_MX = {"nvfp4": 0, "mx": 1, "p2": 2}
RECIPE_FMT = {"nvfp4": lambda h: h.FMT_NVFP4, "mx": lambda h: h.FMT_NVFP4_MX, "p2": lambda h: h.FMT_NVFP4_P2}
RECIPE_NAME = {"mx": "MX-compatible (FP4 MFMA)", "nvfp4": "plain (bf16 MFMA)",
               "p2": "power of two per 16-block (FP4 MFMA, two passes)"}


# ------------------------------------------------------------------ copy

def profile_copy():
    n = 1 << 28
    x = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 5}))


def measure_copy_gbps(nbytes=1 << 30, reps=10):
    """Bandwidth of a plain device-to-device copy (read + write bytes / time),
    the practical ceiling for the HBM-bound kernels."""
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


# ------------------------------------------------------------ schedule (5)

def build_schedule(args, hdq, synth):
    dev = torch.device("cuda:0")
    M = synth.M_COGVIDEOX
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    recipes = {"mx": hdq.FMT_NVFP4_MX, "nvfp4": hdq.FMT_NVFP4, "p2": hdq.FMT_NVFP4_P2}
    s_levels = synth.schedule_noise_levels(args.blocks, args.timesteps)
    blocks = []
    t0 = time.time()
    for b in range(args.blocks):
        layers = []
        for li, (name, K, N) in enumerate(synth.SCHEDULE_LAYERS):
            # the inputs of even (A) and odd (B) timesteps; the previous
            # step's output is the previous step's input plus noise
            x = synth.device_gaussian((M, K), 1.0, gen, dev)
            x_odd = synth.device_noisy_copy(x, 0.1, gen)
            xs = (x, x_odd)
            prev_out = [synth.device_noisy_copy(xs[(t + 1) % 2], float(s_levels[b, li, t]), gen)
                        for t in range(args.timesteps)]
            w = synth.device_gaussian((N, K), 0.02, gen, dev)
            # plain NVFP4 also keeps its weights' exact bf16 values: the exact
            # GEMM then reads both operands decoded (same output bits)
            W = {r: hdq.LinearWeights(w, HB, fp4_fmt=f, fp4_decoded=(r == "nvfp4")) for r, f in recipes.items()}
            layers.append(dict(name=name, K=K, N=N, x=x, xs=xs, prev_out=prev_out, W=W))
        blocks.append(layers)
        if b % 6 == 5 or b == args.blocks - 1:
            torch.cuda.synchronize()
            log(f"setup: {b + 1}/{args.blocks} blocks, {torch.cuda.memory_allocated() / 2**30:.1f} GiB, "
                f"{time.time() - t0:.1f} s")
    # per layer type: quantized-activation buffers, outputs, workspaces
    shared = []
    for name, K, N in synth.SCHEDULE_LAYERS:
        shared.append(dict(
            xq8=hdq.QuantizedTensor(hdq.FMT_INT8_ROW, M, K, HB, dev),
            xq4={r: hdq.QuantizedTensor(f, M, K, HB, dev, decoded=(r == "nvfp4")) for r, f in recipes.items()},
            y=torch.empty(M, N, dtype=torch.bfloat16, device=dev)))
    ws_sel = torch.empty(hdq.workspace_bytes(hdq.OP_SELECT, M, 12288, M * 12288), dtype=torch.uint8,
                         device=dev)
    T, B, L = args.timesteps, args.blocks, len(synth.SCHEDULE_LAYERS)
    dec = torch.full((T, B, L, 1), -1, dtype=torch.int32, device=dev)
    sts = torch.zeros((T, B, L, 5), dtype=torch.float32, device=dev)
    # previous-step difference sums, computed on a second stream (default
    # priority) ahead of the layer calls that need them
    sums = torch.zeros((T, B, L, 2), dtype=torch.float64, device=dev)
    ws_delta = torch.empty_like(ws_sel)
    ws_sq8 = torch.empty(hdq.workspace_bytes(hdq.OP_SELECT_Q8, M, 12288), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    S = dict(M=M, recipes=recipes, blocks=blocks, shared=shared, ws_sel=ws_sel, dec=dec, sts=sts,
             s_levels=s_levels, sums=sums, ws_delta=ws_delta, ws_sq8=ws_sq8, side=side)
    if args.delta == "embed":
        if args.dispatch != "on":
            raise SystemExit("--delta embed needs --dispatch on")
        S.update(embed_plan(args, hdq, synth, M, dev))
    return S


def embed_plan(args, hdq, synth, M, dev):
    """--delta embed: which difference chunks each layer call's GEMM launch
    carries.  The difference of call k is needed by call k's selection, so
    its chunks must all have run by the GEMM launch of call k - 1 (call 0's
    runs as a separate pass at the start of the step).  The chunks of calls
    1.. form one queue in call order; launch k takes its share of the queue,
    proportional to the CU time its GEMM leaves free (--embed-weight
    capacity) or to its GEMM's work (so most chunks run beside a GEMM on the
    CUs it leaves free), or more when call k + 1's chunks would otherwise
    not be done in time."""
    calls = [(t, b, li) for t in range(args.timesteps) for b in range(args.blocks)
             for li in range(len(synth.SCHEDULE_LAYERS))]
    n = [hdq.delta_chunks(M * synth.SCHEDULE_LAYERS[li][1]) for _, _, li in calls]
    work = [2.0 * M * synth.SCHEDULE_LAYERS[li][1] * synth.SCHEDULE_LAYERS[li][2] for _, _, li in calls]
    if getattr(args, "embed_weight", "capacity") == "capacity":
        # CU time a launch leaves to its difference workgroups, in tile times
        # (a tile's time taken as proportional to K): the CUs the persistent
        # GEMM leaves free over all of its tile rounds, plus the GEMM
        # workgroups that have no tile in the last round
        cus = torch.cuda.get_device_properties(dev).multi_processor_count if torch.cuda.is_available() else 256
        wgs = (cus & ~7) - (16 if cus >= 128 else 0)
        def capacity(li):
            _, K, N = synth.SCHEDULE_LAYERS[li]
            tiles = -(-M // 256) * -(-N // 256)
            g = min(tiles, wgs)
            rounds = -(-tiles // g)
            return K * ((cus - g) * rounds + (g * rounds - tiles))
        work = [capacity(li) for _, _, li in calls]
    offs = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    parts = torch.full((int(offs[-1]), 2), float("nan"), dtype=torch.float64, device=dev)
    part_of = [parts[offs[k]:offs[k + 1]] for k in range(len(calls))]
    # queue positions: call k's chunks are [offs[k] - offs[1], offs[k + 1] - offs[1])
    total = int(offs[-1] - offs[1])
    rate = total / sum(work)
    plan, pos = [], 0
    for k in range(len(calls)):
        need = int(offs[k + 2] - offs[1]) - pos if k + 2 < len(offs) else 0
        take = min(total - pos, max(int(round(rate * work[k])), need))
        slices, end = [], pos + take
        while pos < end:
            j = int(np.searchsorted(offs[1:], pos + offs[1], side="right"))  # call owning queue pos
            c0 = pos + int(offs[1]) - int(offs[j])
            c1 = min(int(n[j]), end + int(offs[1]) - int(offs[j]))
            slices.append((j, c0, c1))
            pos += c1 - c0
        if len(slices) > hdq.DELTA_MAX_SLICES:
            raise SystemExit(f"embed plan: launch {k} spans {len(slices)} calls")
        plan.append(slices)
    assert pos == total
    return dict(embed=plan, embed_parts=part_of, embed_queue=torch.zeros(2, dtype=torch.int32, device=dev))


def rec(ev, i):
    """Records event i of a layer call's list, if that list has one."""
    if ev is not None and ev[i] is not None:
        ev[i].record()


def cur_in(L, t):
    """The layer's input at timestep t (A for even t, B for odd)."""
    return L["xs"][t % 2]


def prev_in(L, t):
    """The layer's input at the step before timestep t (its previous-step
    output is L["prev_out"][t])."""
    return L["xs"][(t + 1) % 2]


def run_schedule_step(S, args, hdq, recipe, events=None, side_events=None):
    """One step: every timestep, block and layer, NVFP4 layers in `recipe`.
    With `events`, records up to 7 HIP events per layer call on the main
    stream (select | q8 | q4 | g8 | g4 | gbf; None entries are skipped) and,
    with --delta overlap, 2 per call on the difference stream
    (`side_events`)."""
    calls = [(t, b, li) for t in range(args.timesteps) for b in range(len(S["blocks"]))
             for li in range(len(S["blocks"][b]))]
    main = torch.cuda.current_stream()
    side = S["side"]
    overlap = args.delta == "overlap"
    embed = args.delta == "embed"
    done = [None] * len(calls)

    def enqueue_delta(k, gate=None):
        t, b, li = calls[k]
        L = S["blocks"][b][li]
        if gate is not None:
            side.wait_event(gate)
        with torch.cuda.stream(side):
            se = side_events[k] if side_events is not None else None
            if se: se[0].record(side)
            hdq.delta_sums(prev_in(L, t), L["prev_out"][t], sums=S["sums"][t, b, li], ws=S["ws_delta"],
                           stream=side)
            if se: se[1].record(side)
            ev = torch.cuda.Event()
            ev.record(side)
        done[k] = ev

    ahead = max(1, args.delta_ahead)
    if overlap:
        side.wait_stream(main)  # the previous step's readers of the sums are enqueued before
        for k in range(min(ahead, len(calls))):
            enqueue_delta(k)
    if embed:
        # call 0's difference on its own; the others ride along earlier GEMM launches
        t, b, li = calls[0]
        L = S["blocks"][b][li]
        hdq.delta_sums(prev_in(L, t), L["prev_out"][t], sums=S["sums"][t, b, li], ws=S["ws_delta"])
    for k, (t, b, li) in enumerate(calls):
        L = S["blocks"][b][li]
        sh = S["shared"][li]
        d = S["dec"][t, b, li]
        st = S["sts"][t, b, li]
        ev = events[k] if events is not None else None
        if overlap:
            main.wait_event(done[k])
        fused = args.fuse == "on"
        if fused and args.delta == "inline":
            # the difference on the main stream, right before the selection
            hdq.delta_sums(prev_in(L, t), L["prev_out"][t], sums=S["sums"][t, b, li], ws=S["ws_delta"])
        rec(ev, 0)
        hist = S["embed_parts"][k] if embed and k > 0 else S["sums"][t, b, li]
        if fused:
            hdq.select_quantize_int8(hist, cur_in(L, t), HB, DELTA_T, RATIO_T, decision=d,
                                     stats=st, out=sh["xq8"], ws=S["ws_sq8"])
        elif overlap or embed:
            hdq.select_precision_sums(hist, cur_in(L, t), HB, DELTA_T, RATIO_T, decision=d,
                                      stats=st, ws=S["ws_sel"])
        else:
            hdq.select_precision(prev_in(L, t), L["prev_out"][t], cur_in(L, t), HB, DELTA_T, RATIO_T,
                                 decision=d, stats=st, ws=S["ws_sel"])
        rec(ev, 1)
        if not fused:
            hdq.quantize(cur_in(L, t), HB, hdq.FMT_INT8_ROW, out=sh["xq8"], decision=d)
        rec(ev, 2)
        hdq.quantize(cur_in(L, t), HB, S["recipes"][recipe], tensor_amax=st[4:5], out=sh["xq4"][recipe],
                     decision=d)
        rec(ev, 3)
        if overlap and k + ahead < len(calls):
            # the difference of a later call streams beside this call's
            # compute-bound GEMMs rather than beside its memory-bound passes
            gate = torch.cuda.Event()
            gate.record(main)
            enqueue_delta(k + ahead, gate)
        W = L["W"][recipe]
        if embed:
            sl = []
            for j, c0, c1 in S["embed"][k]:
                tj, bj, lj = calls[j]
                Lj = S["blocks"][bj][lj]
                sl.append((prev_in(Lj, tj), Lj["prev_out"][tj], c0, c1, S["embed_parts"][j]))
            hdq.linear_dispatch_delta(d, cur_in(L, t), sh["xq8"], sh["xq4"][recipe], W, sl, S["embed_queue"],
                                      y=sh["y"])
            rec(ev, 4)
        elif args.dispatch == "on":
            hdq.linear_dispatch(d, cur_in(L, t), sh["xq8"], sh["xq4"][recipe], W, y=sh["y"])
            rec(ev, 4)
        else:
            hdq.linear(hdq.PREC_INT8, None, W, decision=d, xq=sh["xq8"], y=sh["y"])
            rec(ev, 4)
            hdq.linear(hdq.PREC_NVFP4, None, W, decision=d, xq=sh["xq4"][recipe], y=sh["y"])
            rec(ev, 5)
            hdq.linear(hdq.PREC_BF16, cur_in(L, t), W, decision=d, y=sh["y"])
            rec(ev, 6)
    return len(calls)


def embed_bytes(S, args, synth):
    """Per layer call: the difference bytes (both tensors) its GEMM launch
    carries under --delta embed, else 0."""
    calls = [(t, b, li) for t in range(args.timesteps) for b in range(args.blocks)
             for li in range(len(synth.SCHEDULE_LAYERS))]
    if args.delta != "embed":
        return [0] * len(calls)
    from bit_quantized_video_amd.hdq import DELTA_CHUNK as hdq_chunk
    out = []
    for slices in S["embed"]:
        nb = 0
        for j, c0, c1 in slices:
            numel = S["M"] * synth.SCHEDULE_LAYERS[calls[j][2]][1]
            nb += 4 * (min(c1 * hdq_chunk, numel) - c0 * hdq_chunk)
        out.append(nb)
    return out


def schedule_kernel_times(S, args, events_per_step, synth, recipe, side_per_step=None):
    """Per-kernel durations from the recorded events, attributed by the
    device decision of each layer call."""
    M = S["M"]
    decisions = S["dec"].cpu().numpy().reshape(args.timesteps, args.blocks, -1)
    kt = KernelTimes()
    inline = args.delta == "inline"
    carried = embed_bytes(S, args, synth)
    fused = args.fuse == "on"
    dispatch = args.dispatch == "on"
    for s_i, evs in enumerate(events_per_step):
        side = side_per_step[s_i] if side_per_step is not None else None
        k = 0
        for t in range(args.timesteps):
            for b in range(args.blocks):
                for li, (name, K, N) in enumerate(synth.SCHEDULE_LAYERS):
                    ev = evs[k]
                    k += 1
                    d = int(decisions[t, b, li])
                    dt = [ev[i].elapsed_time(ev[i + 1]) if ev[i] is not None and ev[i + 1] is not None
                          else None for i in range(6)]
                    flops = 2.0 * M * N * K
                    q8, q4 = quant_bytes(M, K, "int8"), quant_bytes(M, K, "nvfp4", recipe == "nvfp4")
                    if dt[0] is None:
                        pass  # GEMM events only
                    elif fused:
                        # one pass: x read once, INT8 codes written
                        kt.add("select_quant_int8", dt[0], q8, q8)
                    else:
                        sel = stats_bytes(M, K) if inline else 2 * M * K
                        kt.add("select_stats", dt[0], sel, sel)
                        kt.add("quant_int8" if d == 1 else "quant_int8_gated_off", dt[1],
                               q8 if d == 1 else 0, q8 if d == 1 else 0)
                    if side is not None:
                        kt.add("delta_sums", side[k - 1][0].elapsed_time(side[k - 1][1]), 4 * M * K,
                               4 * M * K)
                    if dt[2] is not None:
                        kt.add("quant_nvfp4" if d == 0 else "quant_nvfp4_gated_off", dt[2],
                               q4 if d == 0 else 0, q4 if d == 0 else 0)
                    for kind, prec, dd, i in (("gemm_int8", "int8", 1, 3), ("gemm_nvfp4", "nvfp4", 0, 4),
                                              ("gemm_bf16", "bf16", 2, 5)):
                        on = d == dd
                        if dispatch:
                            # one launch (slot 3) ran the decided precision's GEMM
                            if on and dt[3] is not None:
                                kt.add(kind, dt[3], flops, gemm_bytes(M, N, K, prec, recipe) + carried[k - 1])
                            continue
                        if dt[i] is not None:
                            kt.add(kind if on else kind + "_gated_off", dt[i], flops if on else 0,
                                   gemm_bytes(M, N, K, prec, recipe) if on else 0)
    return kt, decisions


def cpu_baseline_schedule(S, args, synth):
    """The oracle on a bounded sample of the same workload: block 0's four
    layers at timestep 0 -- selection statistics over the full tensors, then
    quantize + GEMM on the first 256 and last 112 rows in the decided
    precision (all host threads in the GEMM loops; one thread on the first 8
    rows), scaled to all M rows.  Weight preparation is excluded (as on the
    GPU)."""
    import oracle as O
    M = S["M"]
    rows = np.r_[0:256, M - 112:M]  # first 256 rows and the ragged last 112
    R, R1 = len(rows), 8
    fp4_mx = RECIPE_MX[args.fp4]
    threads = O.num_threads()
    t_stats = t_quant = t_gemm = t1_quant = t1_gemm = 0.0
    flops_total = 0.0
    for li, (name, K, N) in enumerate(synth.SCHEDULE_LAYERS):
        L = S["blocks"][0][li]
        np16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        pi, po, x = np16(prev_in(L, 0)), np16(L["prev_out"][0]), np16(cur_in(L, 0))
        w = np16(L["W"][args.fp4].w_bf16)
        # weights (untimed preparation)
        qw, sw = O.quant_int(w, HB, 7)
        wc, we, wst = O.quant_nvfp4(w, HB, mx=fp4_mx)
        t0 = time.perf_counter()
        st = O.stats(pi, po, x, HB)
        d = O.decide(True, st[0], st[1], DELTA_T, RATIO_T)
        ts = time.perf_counter() - t0

        def rows_run(xs):
            t0 = time.perf_counter()
            if d == O.INT8:
                q = O.quant_int(xs, HB, 127)
            elif d == O.NVFP4:
                q = O.quant_nvfp4(xs, HB, amax=np.float32(st[4]), mx=fp4_mx)
            t1 = time.perf_counter()
            if d == O.INT8:
                O.gemm_int(q[0], q[1], qw, sw)
            elif d == O.NVFP4:
                O.gemm_nvfp4(*q, wc, we, wst, K)
            else:
                O.gemm_bf16(xs, w)
            return t1 - t0, time.perf_counter() - t1
        O.set_num_threads(threads)
        tq, tg = rows_run(np.ascontiguousarray(x[rows]))
        O.set_num_threads(1)
        tq1, tg1 = rows_run(np.ascontiguousarray(x[:R1]))
        O.set_num_threads(threads)
        t_stats += ts
        t_quant += tq * M / R
        t_gemm += tg * M / R
        t1_quant += tq1 * M / R1
        t1_gemm += tg1 * M / R1
        flops_total += 2.0 * M * N * K
        log(f"cpu baseline: {name} decision={d} stats {ts:.2f}s, {R} rows quant {tq:.2f}s gemm {tg:.2f}s, "
            f"{R1} rows one thread {tq1 + tg1:.2f}s")
    t_total = t_stats + t_quant + t_gemm
    t1_total = t_stats + t1_quant + t1_gemm
    return {"value": flops_total / t_total / 1e12, "unit": "TOPS", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "split_s": {"stats": round(t_stats, 3), "quantize": round(t_quant, 3), "gemm": round(t_gemm, 3)},
            "one_thread": {"value": round(flops_total / t1_total / 1e12, 6), "unit": "TOPS",
                           "split_s": {"stats": round(t_stats, 3), "quantize": round(t1_quant, 3),
                                       "gemm": round(t1_gemm, 3)}, "rows": R1},
            "sample": (f"block 0 x 4 layers at timestep 0: selection statistics over the full "
                       f"[17776, K] tensors (1 thread), rotate+quantize (1 thread) and GEMM (OpenMP, "
                       f"{threads} threads) in the decided precision on {R} of 17776 rows (the first 256 "
                       f"and the last 112), times scaled linearly to all rows; one_thread: the first {R1} "
                       f"rows with one thread; weight preparation untimed")}


def time_schedule(S, args, hdq, synth, recipe):
    """Warmup, then exactly args.steps timed steps with HIP events around
    each layer call's GEMM launch (--events gemm) or every kernel (all).
    With gemm events, one instrumented step after the timed ones times the
    other kernels.  Returns ms/step, per-kernel times, the decisions, and
    which step each kernel's times come from."""
    log(f"warmup ({recipe})")
    for _ in range(args.warmup):
        run_schedule_step(S, args, hdq, recipe)
    n_calls = args.timesteps * args.blocks * len(synth.SCHEDULE_LAYERS)
    overlap = args.delta == "overlap"
    gemm_slots = (3, 4) if args.dispatch == "on" else (3, 4, 5, 6)

    def make(slots):
        return [[torch.cuda.Event(enable_timing=True) if i in slots else None for i in range(7)]
                for _ in range(n_calls)]

    def make_side():
        return [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_calls)]

    all_slots = tuple(range(5 if args.dispatch == "on" else 7))
    timed_slots = gemm_slots if args.events == "gemm" else all_slots
    events = [make(timed_slots) for _ in range(args.steps)]
    side = [make_side() for _ in range(args.steps)] if overlap and args.events == "all" else None
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps ({recipe}, events: {args.events})")
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_schedule_step(S, args, hdq, recipe, events[s], side[s] if side else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt, decisions = schedule_kernel_times(S, args, events, synth, recipe, side)
    source = {k: "timed steps" for k in kt.t}
    if args.events == "gemm":
        # the other kernels: one instrumented (untimed) step
        ev1, side1 = [make(all_slots)], [make_side()] if overlap else None
        run_schedule_step(S, args, hdq, recipe, ev1[0], side1[0] if side1 else None)
        torch.cuda.synchronize()
        kt1, _ = schedule_kernel_times(S, args, ev1, synth, recipe, side1)
        for k in list(kt1.t):
            if not k.startswith("gemm"):
                kt.t[k], kt.work[k], kt.bytes[k], kt.n[k] = kt1.t[k], kt1.work[k], kt1.bytes[k], kt1.n[k]
                source[k] = "instrumented step"
    return 1e3 * elapsed / args.steps, kt, decisions, source


TDC_TAU_SKIP, TDC_TAU_ACC = 0.05, 0.15


def schedule_history(S, args, t, b, li):
    """The schedule's previous-step difference sums of call (t, b, li): its
    chunk partials under --delta embed (except call 0's pair), else its pair."""
    k = (t * args.blocks + b) * len(S["blocks"][b]) + li
    if args.delta == "embed" and k > 0:
        return S["embed_parts"][k]
    return S["sums"][t, b, li]


def tdc_trajectory(S, args, hdq, synth, recipe, use_tdc, dirs):
    """One synthetic denoising trajectory over the first args.tdc_blocks
    blocks' modules.  Module input at step t: x + a_t * d (d a fixed seeded
    direction, increments a_t - a_(t-1) = 0.3 * 0.6^t, so the trajectory
    smooths out).  A computed module runs the DMPQ path of the schedule
    (selection fused with INT8 quantization -- history: the schedule's
    difference sums when the module ran at the previous step, none after a
    skip -- the gated NVFP4 quantizer and the one-launch GEMM) into a fresh
    output buffer.  With use_tdc, the change of each new output against the
    module's cached one and the skip rule (hdq_tdc_decide, once per step for
    all modules, read back with one synchronization) decide which modules the
    next step skips.  The change runs as chunk partials inside the next
    computed module's GEMM launch (hdq_linear_dispatch_delta; part of the path
    time), the step's last one on its own before the rule (hdq_delta_sums;
    timed with the rule).  HIP events time the hot path (input formation
    excluded); returns per-step milliseconds and skip counts."""
    dev = torch.device("cuda:0")
    M = S["M"]
    mods = [(b, li) for b in range(args.tdc_blocks) for li in range(len(synth.SCHEDULE_LAYERS))]
    n = len(mods)
    ybuf = [[torch.empty(M, synth.SCHEDULE_LAYERS[li][2], dtype=torch.bfloat16, device=dev)
             for _ in range(2)] for _, li in mods]
    cur = [None] * n                      # index of the cached output buffer
    ran_prev = [False] * n
    state = torch.zeros(n, dtype=torch.int32, device=dev)
    c = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.zeros(n, dtype=torch.float32, device=dev)
    skip = torch.zeros(n, dtype=torch.int32, device=dev)
    skip_h = [0] * n
    dec_t = torch.zeros((n, 1), dtype=torch.int32, device=dev)
    sts_t = torch.zeros((n, 5), dtype=torch.float32, device=dev)
    xin = {li: torch.empty(M, K, dtype=torch.bfloat16, device=dev)
           for li, (_, K, _) in enumerate(synth.SCHEDULE_LAYERS)}
    # the change statistic as chunk partials: module i's are rows off[i] .. off[i + 1] - 1
    nch = [hdq.delta_chunks(M * synth.SCHEDULE_LAYERS[li][2]) for _, li in mods]
    off = np.concatenate([[0], np.cumsum(nch)]).astype(np.int64)
    parts = torch.zeros((int(off[-1]), 2), dtype=torch.float64, device=dev)
    part_of = [parts[off[i]:off[i + 1]] for i in range(n)]
    off_dev = torch.from_numpy(off).to(dev)
    queue = torch.zeros(2, dtype=torch.int32, device=dev)
    per_step, skips, change_ms, decide_ms = [], [], [], []
    a = 0.0
    for t in range(args.tdc_steps):
        a += 0.3 * 0.6 ** t
        evs = []
        state_h = [0] * n
        pending = []   # the last computed module's change, run inside the next module's GEMM launch
        for i, (b, li) in enumerate(mods):
            if use_tdc and skip_h[i]:
                ran_prev[i] = False
                continue
            L = S["blocks"][b][li]
            sh = S["shared"][li]
            torch.add(L["x"], dirs[i], alpha=a, out=xin[li])
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            hist = schedule_history(S, args, min(t, args.timesteps - 1), b, li) if ran_prev[i] else None
            d, st = dec_t[i], sts_t[i]
            hdq.select_quantize_int8(hist, xin[li], HB, DELTA_T, RATIO_T, decision=d, stats=st,
                                     out=sh["xq8"], ws=S["ws_sq8"])
            hdq.quantize(xin[li], HB, S["recipes"][recipe], tensor_amax=st[4:5], out=sh["xq4"][recipe],
                         decision=d)
            new = 0 if cur[i] is None else 1 - cur[i]
            if pending:
                hdq.linear_dispatch_delta(d, xin[li], sh["xq8"], sh["xq4"][recipe], L["W"][recipe], pending,
                                          queue, y=ybuf[i][new])
            else:
                hdq.linear_dispatch(d, xin[li], sh["xq8"], sh["xq4"][recipe], L["W"][recipe], y=ybuf[i][new])
            pending = []
            e[1].record()
            if use_tdc:
                if cur[i] is None:
                    state_h[i] = 1
                else:
                    state_h[i] = 2
                    pending = [(ybuf[i][cur[i]], ybuf[i][new], 0, nch[i], part_of[i])]
            e[2].record()
            evs.append(e)
            cur[i] = new
            ran_prev[i] = True
        ed = None
        if use_tdc:
            state.copy_(torch.tensor(state_h, dtype=torch.int32))
            ed = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ed[0].record()
            if pending:
                # the step's last computed module: its change on its own, as the
                # first pair of its range (the rest zero)
                old_y, new_y, _, _, pr = pending[0]
                hdq.delta_sums(old_y, new_y, sums=pr[0], ws=S["ws_delta"])
                pr[1:].zero_()
            hdq.tdc_decide(parts, state, c, acc, skip=skip, tau_skip=TDC_TAU_SKIP, tau_acc=TDC_TAU_ACC,
                           offsets=off_dev)
            ed[1].record()
            skip_h = skip.tolist()        # one synchronization per step
        torch.cuda.synchronize()
        path = sum(e[0].elapsed_time(e[1]) for e in evs)
        chg = sum(e[1].elapsed_time(e[2]) for e in evs)
        dec = ed[0].elapsed_time(ed[1]) if ed else 0.0
        per_step.append(path + chg + dec)
        change_ms.append(chg / max(1, len(evs)))
        decide_ms.append(dec)
        skips.append(n - len(evs))
    return per_step, skips, change_ms, decide_ms


def bench_tdc(S, args, hdq, synth):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    n_mod = args.tdc_blocks * len(synth.SCHEDULE_LAYERS)
    dirs = [synth.device_gaussian(S["blocks"][b][li]["x"].shape, 1.0, gen, dev)
            for b in range(args.tdc_blocks) for li in range(len(synth.SCHEDULE_LAYERS))]
    log(f"tdc trajectory: {n_mod} modules x {args.tdc_steps} steps")
    full = tdc_trajectory(S, args, hdq, synth, args.fp4, False, dirs)
    tdc = tdc_trajectory(S, args, hdq, synth, args.fp4, True, dirs)
    del dirs
    torch.cuda.empty_cache()
    ms_full, ms_tdc = float(np.mean(full[0])), float(np.mean(tdc[0]))
    return {"modules": n_mod, "steps": args.tdc_steps, "tau_skip": TDC_TAU_SKIP, "tau_acc": TDC_TAU_ACC,
            "skip_fraction": round(sum(tdc[1]) / (n_mod * args.tdc_steps), 4),
            "skips_per_step": tdc[1],
            "ms_per_step_full": round(ms_full, 3), "ms_per_step_tdc": round(ms_tdc, 3),
            "speedup": round(ms_full / ms_tdc, 3),
            "rule_us_avg": round(1e3 * float(np.mean(tdc[3])), 2),
            "input": "x + a_t d per module, a_t - a_(t-1) = 0.3 * 0.6^t; hot path timed with HIP "
                     "events (input formation excluded)",
            "change_statistic": "chunk partials inside the next computed module's GEMM launch (in the "
                                "path time); the step's last module's on its own, timed with the rule "
                                "(rule_us_avg)"}


def schedule_quality(S, hdq):
    """Output error of each precision on one NVFP4-sized layer (block 0 FFN
    up-projection): relative Frobenius distance of the bf16 output from the
    unquantized bf16 GEMM's."""
    L = S["blocks"][0][2]
    x, ref = L["x"], None
    out = {}
    for name, prec, W in (("bf16", hdq.PREC_BF16, L["W"]["mx"]), ("int8", hdq.PREC_INT8, L["W"]["mx"]),
                          ("nvfp4_mx", hdq.PREC_NVFP4, L["W"]["mx"]),
                          ("nvfp4", hdq.PREC_NVFP4, L["W"]["nvfp4"]),
                          ("nvfp4_p2", hdq.PREC_NVFP4, L["W"]["p2"])):
        y = hdq.linear(prec, x, W, y_dtype=hdq.DTYPE_F32)
        if ref is None:
            ref = y
            continue
        out[name] = float(torch.linalg.norm(y - ref) / torch.linalg.norm(ref))
    return out


def bench_schedule(args, hdq, synth):
    copy_gbps = measure_copy_gbps()
    log(f"device copy: {copy_gbps:.0f} GB/s")
    S = build_schedule(args, hdq, synth)
    M = S["M"]
    flops_step = sum(2.0 * M * N * K for _, K, N in synth.SCHEDULE_LAYERS) * args.blocks * args.timesteps
    n_calls = args.timesteps * args.blocks * len(synth.SCHEDULE_LAYERS)
    others = [r for r in ("mx", "nvfp4", "p2") if r != args.fp4]
    runs = {r: time_schedule(S, args, hdq, synth, r) for r in [args.fp4] + others}
    ms_per_step, kt, decisions, source = runs[args.fp4]
    if args.decisions_out:
        with open(args.decisions_out, "w") as fh:
            json.dump({"decisions": [int(v) for v in decisions.reshape(-1)]}, fh)
    ks = kt.summary()
    counts = {p: int((decisions == v).sum()) for p, v in (("nvfp4", 0), ("int8", 1), ("bf16", 2))}
    # dominant kernel: the critical-path kernel with the most time (the
    # difference pass on the second stream overlaps the GEMMs and is not one)
    main_kinds = ["gemm_int8", "gemm_nvfp4", "gemm_bf16", "quant_int8", "quant_nvfp4", "select_stats",
                  "select_quant_int8"]
    dom = max((k for k in main_kinds if k in ks), key=lambda k: ks[k]["total_ms"])
    roof = roofline_for(dom, ks[dom], args.fp4, copy_gbps)
    # quantization passes (with --fuse on, the INT8 one is the selection pass)
    q_kinds = ("quant_int8", "select_quant_int8", "quant_nvfp4")
    q_bytes = sum(kt.work[k] for k in q_kinds if k in kt.work)
    q_ms = sum(kt.t[k] for k in q_kinds if k in kt.t)
    # effective TOPS of the fused quant + linear alone (selected kernels only)
    ql_ms = q_ms + sum(kt.t.get(k, 0.0) for k in ("gemm_int8", "gemm_nvfp4", "gemm_bf16"))
    ql_flops = sum(kt.work.get(k, 0.0) for k in ("gemm_int8", "gemm_nvfp4", "gemm_bf16"))
    def other_line(r):
        o_ms, o_kt, _, _ = runs[r]
        o_ks = o_kt.summary()
        g = o_ks.get("gemm_nvfp4")
        return {"recipe": r, "value": round(flops_step / (o_ms * 1e-3) / 1e12, 2),
                "ms_per_step": round(o_ms, 3),
                "gemm_nvfp4": ({k: g[k] for k in ("launches", "total_ms", "avg_us")}
                               | {"rate_tflops": round(g["rate"] / 1e12, 1)}) if g else None}
    result = {
        "metric": METRIC,
        "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"mx": "int8+nvfp4_mx", "nvfp4": "int8+nvfp4", "p2": "int8+nvfp4_p2"}[args.fp4],
        "data": "synthetic",
        "config": {"workload": (f"DMPQ schedule: {args.blocks} CogVideoX-5B blocks x (QKV 3072->9216, "
                                f"out 3072->3072, FFN 3072->12288->3072) x {args.timesteps} timesteps, "
                                f"M=17776 tokens, Hadamard block 128, delta thresh 0.1, ratio thresh 50, "
                                f"NVFP4 recipe {RECIPE_NAME[args.fp4]}"),
                   "global_batch": M, "layer_calls_per_step": n_calls},
        "roofline": roof,
        "quant_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1) if q_ms > 0 else None,
        "copy_gbps": round(copy_gbps, 1),
        "quant_roofline": {k: roofline_for(k, ks[k], args.fp4, copy_gbps)
                           for k in ("quant_int8", "quant_nvfp4", "select_stats", "select_quant_int8",
                                     "delta_sums") if k in ks},
        "fused_quant_linear_tops": round(ql_flops / (ql_ms * 1e-3) / 1e12, 2) if ql_ms > 0 else None,
        "decisions": counts,
        "kernels": {k: {"launches": v["launches"], "total_ms": v["total_ms"], "avg_us": v["avg_us"],
                        "rate": round(v["rate"] / 1e12, 3), "timed_in": source.get(k),
                        "rate_unit": ("TB/s" if k.startswith(("quant", "select", "delta")) else
                                      "TOP/s" if k.startswith("gemm_int8") else "TFLOP/s")}
                    for k, v in ks.items()},
        "other_recipes": [other_line(r) for r in others],
        "quality_rel_err_vs_bf16": schedule_quality(S, hdq),
    }
    if args.fp4 != "nvfp4":
        # the at-spec recipe (E4M3 scale per 16 elements) beside the headline
        plain = other_line("nvfp4")
        result["value_plain_nvfp4"] = plain["value"]
        result["ms_per_step_plain_nvfp4"] = plain["ms_per_step"]
    if args.bf16_reps > 0:
        log("bf16 fallback layers")
        result["bf16_fallback"] = bench_bf16_fallback(S, args, hdq, synth, args.fp4)
    if args.tdc_steps > 0:
        result["tdc"] = bench_tdc(S, args, hdq, synth)
    if args.dq_steps > 0:
        result["deltaquant"] = bench_deltaquant(args, hdq, synth)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline_schedule(S, args, synth)
        result["cpu_baseline"]["value"] = round(result["cpu_baseline"]["value"], 6)
    if args.config_reps > 0:
        del S
        torch.cuda.empty_cache()
        result["configs"] = bench_configs(args, hdq, synth)
    return result


def cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_FILL = {}


def gpu_filler(ms=5.0):
    """Queues about `ms` of device copies (256 MiB each): the clocks leave
    their idle state, and launches enqueued behind it reach the GPU back to
    back instead of at the host's launch rate."""
    if "a" not in _FILL:
        _FILL["a"] = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
        _FILL["b"] = torch.empty_like(_FILL["a"])
    for _ in range(max(1, int(ms / 0.1))):
        _FILL["b"].copy_(_FILL["a"])


def event_time(fn, reps, warm=2):
    """Average milliseconds of fn() over reps launches (HIP events), timed
    behind a few milliseconds of queued copies so that the host enqueues the
    timed launches while they run."""
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_filler()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# the single-layer configurations and the paths each is run on
# (nvfp4: the exact GEMM on both operands' decoded bf16 values, which the
# quantizer writes beside the codes; nvfp4_staged: the same GEMM decoding the
# codes while it stages them)
CONFIG_PATHS = {1: ("int8", "nvfp4", "nvfp4_staged", "nvfp4_mx"), 2: ("int8",),
                3: ("nvfp4", "nvfp4_staged", "nvfp4_mx"), 4: ("int8",)}
PATH_FMT = {"int8": "FMT_INT8_ROW", "nvfp4": "FMT_NVFP4", "nvfp4_staged": "FMT_NVFP4", "nvfp4_mx": "FMT_NVFP4_MX"}


def bench_configs(args, hdq, synth):
    """The four single-layer configurations (1024^3 with outliers; CogVideoX-2B
    QKV INT8; CogVideoX-5B FFN up NVFP4; FFN down INT8) at full size: the fused
    rotate+quantize and the GEMM timed apart with HIP events (tensor amax given
    to the NVFP4 quantizer, as the selection pass supplies it), their rates
    against the roofline, a parity check of sampled output rows against the
    oracle, and the oracle's own times on those rows (all host threads and one
    thread, quantize and GEMM apart, scaled per row to all M rows)."""
    import oracle as O
    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    threads = O.num_threads()
    out = {}
    for cfg in (1, 2, 3, 4):
        c = synth.CONFIGS[cfg]
        M, K, N, hb = c["M"], c["K"], c["N"], c["had_block"]
        log(f"config {cfg}: {c['name']}")
        x16 = synth.config_activations(cfg)
        w16 = synth.config_weights(cfg)
        xd, wd = to_dev(x16), to_dev(w16)
        y_dtype = hdq.DTYPE_F32 if c["out"] == "f32" else hdq.DTYPE_BF16
        y = torch.empty(M, N, dtype=torch.float32 if y_dtype == hdq.DTYPE_F32 else torch.bfloat16, device=dev)
        rows = np.arange(M) if M <= 1024 else np.r_[0:256, M - 112:M]
        recs = {}
        for path in CONFIG_PATHS[cfg]:
            fmt = getattr(hdq, PATH_FMT[path])
            decoded = path == "nvfp4"
            W = hdq.LinearWeights(wd, hb, fp4_fmt=None if path == "int8" else fmt, keep_bf16=False,
                                  fp4_decoded=decoded)
            prec = hdq.PREC_INT8 if path == "int8" else hdq.PREC_NVFP4
            xq = hdq.QuantizedTensor(fmt, M, K, hb, dev, decoded=decoded)
            amax = None if path == "int8" else hdq.select_precision(None, None, xd, hb)[1][4:5]
            tq = event_time(lambda: hdq.quantize(xd, hb, fmt, tensor_amax=amax, out=xq), args.config_reps)
            tg = event_time(lambda: hdq.linear(prec, None, W, xq=xq, y=y, y_dtype=y_dtype), args.config_reps)
            flops = 2.0 * M * N * K
            qb = quant_bytes(M, K, "int8" if path == "int8" else "nvfp4", decoded)
            dt = {"int8": "int8", "nvfp4": "bf16", "nvfp4_staged": "bf16", "nvfp4_mx": "fp4"}[path]
            rec = {"quant_us": round(tq * 1e3, 1), "quant_gbps": round(qb / (tq * 1e-3) / 1e9, 1),
                   "quant_frac_hbm": round(qb / (tq * 1e-3) / PEAK["hbm"], 4),
                   "gemm_us": round(tg * 1e3, 1), "gemm_dtype": dt,
                   "gemm_rate": round(flops / (tg * 1e-3) / 1e12, 1),
                   "gemm_rate_unit": "TOP/s" if dt == "int8" else "TFLOP/s",
                   "gemm_frac": round(flops / (tg * 1e-3) / PEAK[dt], 4),
                   "effective_tops": round(flops / ((tq + tg) * 1e-3) / 1e12, 2)}
            # parity of the sampled rows and the oracle's times on them
            got = y.float().cpu().numpy()[rows] if y_dtype == hdq.DTYPE_F32 else \
                synth.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)[rows])
            xs = np.ascontiguousarray(x16[rows])
            mx = {"nvfp4_mx": 1}.get(path, 0)
            if path == "int8":
                qw, sw = O.quant_int(w16, hb, 7)
            else:
                wc, we, wst = O.quant_nvfp4(w16, hb, mx=mx)
                a_all = np.float32(O.rotated_amax(x16, hb))
            def oracle_rows(xr):
                t0 = time.perf_counter()
                if path == "int8":
                    q = O.quant_int(xr, hb, 127)
                else:
                    q = O.quant_nvfp4(xr, hb, amax=a_all, mx=mx)
                t1 = time.perf_counter()
                r = O.gemm_int(q[0], q[1], qw, sw)[0] if path == "int8" else O.gemm_nvfp4(*q, wc, we, wst, K)
                return r, t1 - t0, time.perf_counter() - t1
            sample = rows if path == "int8" or cfg == 1 else np.r_[0:64, M - 48:M]
            O.set_num_threads(threads)
            ref, cq, cg = oracle_rows(np.ascontiguousarray(x16[sample]))
            ref = ref.astype(np.float64)
            sel = np.searchsorted(rows, sample)
            if y_dtype == hdq.DTYPE_BF16:
                ref = synth.bf16_bits_to_f32(O.f32_to_bf16(ref.astype(np.float32))).astype(np.float64)
            else:
                ref = ref.astype(np.float32).astype(np.float64)
            g = got[sel].astype(np.float64)
            rec["parity"] = ({"rows": int(len(sample)), "bitexact": bool(np.array_equal(g, ref))} if path == "int8"
                             else {"rows": int(len(sample)),
                                   "rel_fro": float(np.linalg.norm(g - ref) / np.linalg.norm(ref))})
            n1 = 16 if path == "int8" else 4
            O.set_num_threads(1)
            _, cq1, cg1 = oracle_rows(np.ascontiguousarray(x16[:n1]))
            O.set_num_threads(threads)
            def cpu(tq_, tg_, n):
                sq, sg = tq_ / n * M, tg_ / n * M
                return {"quant_s": round(sq, 3), "gemm_s": round(sg, 3),
                        "quant_gbps": round(qb / sq / 1e9, 3), "effective_tops": round(flops / (sq + sg) / 1e12, 6)}
            rec["cpu_baseline"] = {"kind": "oracle", "cpu": cpu_model(), "host_cpus": os.cpu_count(),
                                   "all_cores": dict(cpu(cq, cg, len(sample)), threads=threads, rows=int(len(sample))),
                                   "one_thread": dict(cpu(cq1, cg1, n1), threads=1, rows=n1),
                                   "note": "oracle times on the rows named, scaled linearly to all M rows; the "
                                           "quantizer loops are single-threaded, the GEMM loops OpenMP; weight "
                                           "preparation and the NVFP4 tensor amax untimed"}
            recs[path] = rec
            del W, xq
            log(f"config {cfg} {path}: quant {rec['quant_us']} us, gemm {rec['gemm_us']} us "
                f"({rec['gemm_rate']} {rec['gemm_rate_unit']}), parity {rec['parity']}")
        out[str(cfg)] = {"workload": c["name"], "M": M, "K": K, "N": N, "had_block": hb,
                         "out": c["out"], "paths": recs}
        del xd, wd, y, x16, w16
        torch.cuda.empty_cache()
    return out


def bench_bf16_fallback(S, args, hdq, synth, recipe):
    """The full-precision fallback (purified delta refresh) at the schedule's
    layer shapes: block 0's inputs with one channel scaled x400, whose outlier
    ratio max|x|/mean|x| is far above 50, through the schedule's own sequence
    (selection fused with INT8 quantization, the gated NVFP4 quantizer, the
    one-launch GEMM); HIP events around the GEMM launch, which runs the bf16
    body."""
    dev = torch.device("cuda:0")
    M = S["M"]
    recs, tot_ms, tot_flops = {}, 0.0, 0.0
    for li, (name, K, N) in enumerate(synth.SCHEDULE_LAYERS):
        L = S["blocks"][0][li]
        sh = S["shared"][li]
        x = L["x"].clone()
        x[:, 7] *= 400.0
        d = torch.empty(1, dtype=torch.int32, device=dev)
        st = torch.empty(5, dtype=torch.float32, device=dev)
        hdq.select_quantize_int8(None, x, HB, DELTA_T, RATIO_T, decision=d, stats=st, out=sh["xq8"],
                                 ws=S["ws_sq8"])
        hdq.quantize(x, HB, S["recipes"][recipe], tensor_amax=st[4:5], out=sh["xq4"][recipe], decision=d)
        torch.cuda.synchronize()
        assert int(d.item()) == hdq.PREC_BF16, (name, float(st[1].item()))
        W = L["W"][recipe]
        ms = event_time(lambda: hdq.linear_dispatch(d, x, sh["xq8"], sh["xq4"][recipe], W, y=sh["y"]),
                        args.bf16_reps)
        flops = 2.0 * M * N * K
        tot_ms += ms
        tot_flops += flops
        recs[name] = {"gemm_us": round(ms * 1e3, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                      "frac": round(flops / (ms * 1e-3) / PEAK["bf16"], 4),
                      "ratio": round(float(st[1].item()), 1)}
        del x
    return {"workload": "bf16 fallback (outlier ratio above 50) at the schedule's four layer shapes, M=17776",
            "layers": recs, "tflops": round(tot_flops / (tot_ms * 1e-3) / 1e12, 1),
            "frac": round(tot_flops / (tot_ms * 1e-3) / PEAK["bf16"], 4), "peak_tflops": PEAK["bf16"] / 1e12}


def bench_deltaquant(args, hdq, synth):
    """DeltaQuant's cube-delta path on one FFN up-projection of the CogVideoX-5B
    video tokens (13 x 30 x 45 grid, K 3072 -> N 12288, 2 x 2 x 2 cubes, MX
    NVFP4 differences): per-call times of the activation quantization and of
    the linear, their rates against the roofline, and the output's relative
    error against the bf16 product beside plain NVFP4 (no cubes, no rotation)."""
    log("deltaquant")
    F, H, W, K, N, cube, fmt = 13, 30, 45, 3072, 12288, (2, 2, 2), hdq.FMT_NVFP4_MX
    grid = (F, H, W, cube)
    M, C = F * H * W, hdq.dq_cubes(grid)
    dev = torch.device("cuda:0")
    x16 = synth.smooth_video_tokens(F, H, W, K, synth.rng_for(140, 0))
    x = torch.from_numpy(x16.view(np.int16)).to(dev).view(torch.bfloat16)
    gen = torch.Generator(device=dev)
    gen.manual_seed(140)
    w = synth.device_gaussian((N, K), 0.02, gen, dev)
    W1 = hdq.LinearWeights(w, 1, fp4_fmt=fmt)    # no rotation: had_block 1
    wq = W1.w_fp4
    bf16_core = hdq.dq_core_needs_bf16(fmt, C, K, N)
    wdec = hdq.dq_decode_weights(wq) if bf16_core else None
    a = hdq.dq_quantize(x, grid, fmt)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(hdq.dq_linear_workspace_bytes(grid, K, N, fmt), dtype=torch.uint8, device=dev)

    def timed(fn, n):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        gpu_filler()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    q_ms = timed(lambda: hdq.dq_quantize(x, grid, fmt, out=a), args.dq_steps)
    l_ms = timed(lambda: hdq.dq_linear(a, wq, wdec, y=y, ws=ws), args.dq_steps)
    # algorithmic bytes of the quantization: x once, the difference codes and
    # block scales, the core codes and scales (and the core's bf16 values when
    # the core GEMM runs in bf16)
    q_bytes = M * K * 2 + M * K // 2 + M * K // 16 + C * K * (3 if bf16_core else 1) + C * 4
    # the linear: the core GEMM (FP8 x FP4 MFMA, or bf16) and the difference
    # GEMM (FP4 x FP4); its peak is the time-weighted one of the two
    core_flops, diff_flops = 2.0 * C * N * K, 2.0 * M * N * K
    flops = core_flops + diff_flops
    core_peak = PEAK["bf16" if bf16_core else "fp8"]
    peak = flops / (core_flops / core_peak + diff_flops / PEAK["fp4"])
    ref = x.float() @ w.float().T
    plain = hdq.linear(hdq.PREC_NVFP4, None, W1, xq=hdq.quantize(x, 1, fmt), y_dtype=hdq.DTYPE_F32)
    yd = hdq.dq_linear(a, wq, wdec, y_dtype=hdq.DTYPE_F32, ws=ws)
    nref = float(torch.linalg.vector_norm(ref))
    err = lambda t: round(float(torch.linalg.vector_norm(t - ref)) / nref, 5)
    ach = flops / (l_ms * 1e-3)
    out = {"workload": f"DeltaQuant cube-delta linear: 13x30x45 video tokens ({M}), K 3072 -> N 12288, "
                       f"2x2x2 cubes ({C}, ragged), FP8 E4M3 cores, NVFP4-MX differences, bf16 output",
           "quantize_us": round(q_ms * 1e3, 1),
           "quantize_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
           "quantize_roofline": {"bound": "hbm", "achieved": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                                 "peak": 8000.0, "unit": "GB/s",
                                 "frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / 8000.0, 3),
                                 "traffic": None},
           "linear_us": round(l_ms * 1e3, 1),
           "linear_tflops": round(ach / 1e12, 1),
           "linear_roofline": {"bound": "mfma", "achieved": round(ach / 1e12, 1),
                               "peak": round(peak / 1e12, 1), "unit": "TFLOP/s",
                               "peak_note": ("time-weighted: core GEMM %s (%.0f TFLOP/s), difference GEMM FP4 "
                                             "(%.0f TFLOP/s)" % ("bf16" if bf16_core else "FP8 x FP4",
                                                                 core_peak / 1e12, PEAK["fp4"] / 1e12)),
                               "frac": round(ach / peak, 3), "traffic": None},
           "rel_err_vs_bf16": err(yd), "plain_nvfp4mx_rel_err_vs_bf16": err(plain)}
    del ref, plain, yd
    return out


def stored_traffic(kind, recipe):
    """HBM bytes per launch for a bench kernel kind from the committed
    FETCH_SIZE/WRITE_SIZE summary, or None (absent, or the kernel changed
    since the counters were taken)."""
    from bit_quantized_video_amd import profsum
    suffix = {"mx": "_mx", "p2": "_p2"}.get(recipe, "")
    pkind = kind + suffix if kind in ("gemm_nvfp4", "quant_nvfp4") else kind
    try:
        return profsum.current_traffic(TRAFFIC_PROFILE, pkind)
    except (OSError, KeyError):
        return None


def roofline_for(kind, k, recipe, copy_gbps=None):
    traffic = stored_traffic(kind, recipe)
    traffic = None if traffic is None else round(traffic)
    alg = round(k["bytes_per_launch"])
    if kind.startswith("gemm"):
        dt = {"gemm_int8": "int8", "gemm_bf16": "bf16",
              "gemm_nvfp4": "bf16" if recipe == "nvfp4" else "fp4"}[kind]
        peak = PEAK[dt]
        ach = k["rate"]
        return {"kernel": kind, "bound": "mfma", "dtype": dt, "achieved": round(ach / 1e12, 1),
                "peak": round(peak / 1e12, 1), "unit": "TFLOP/s" if dt != "int8" else "TOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic, "traffic_unit": "bytes/launch",
                "algorithmic_bytes": alg, "avg_launch_us": k["avg_us"]}
    ach = k["rate"]
    return {"kernel": kind, "bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": 8000.0,
            "unit": "GB/s", "frac": round(ach / PEAK["hbm"], 4),
            "frac_of_copy": round(ach / 1e9 / copy_gbps, 4) if copy_gbps else None, "traffic": traffic,
            "traffic_unit": "bytes/launch", "algorithmic_bytes": alg, "avg_launch_us": k["avg_us"]}


# ---------------------------------------------------------- single layer

def bench_single(args, hdq, synth):
    import oracle as O  # noqa: F401  (only for the CPU-baseline leg)
    cfg = args.config
    c = synth.CONFIGS[cfg]
    M, K, N, hb = c["M"], c["K"], c["N"], c["had_block"]
    dev = torch.device("cuda:0")
    log(f"config {cfg}: generating")
    x16 = synth.config_activations(cfg)
    w16 = synth.config_weights(cfg)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    xd = to_dev(x16)
    path = c["paths"][0] if args.fp4 == "nvfp4" else ("nvfp4" if "nvfp4" in c["paths"] else "int8")
    fmt = hdq.FMT_INT8_ROW if path == "int8" else RECIPE_FMT[args.fp4](hdq)
    # plain NVFP4: the exact GEMM on both operands' decoded bf16 values
    decoded = path != "int8" and args.fp4 == "nvfp4"
    W = hdq.LinearWeights(to_dev(w16), hb, fp4_fmt=None if path == "int8" else fmt, fp4_decoded=decoded)
    prec = hdq.PREC_INT8 if path == "int8" else hdq.PREC_NVFP4
    y_dtype = hdq.DTYPE_F32 if c["out"] == "f32" else hdq.DTYPE_BF16
    xq = hdq.QuantizedTensor(fmt, M, K, hb, dev, decoded=decoded)
    amax = None
    if path != "int8":
        _, st = hdq.select_precision(None, None, xd, hb)
        amax = st[4:5]
    y = torch.empty(M, N, dtype=torch.float32 if y_dtype == hdq.DTYPE_F32 else torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        hdq.quantize(xd, hb, fmt, tensor_amax=amax, out=xq)
        hdq.linear(prec, None, W, xq=xq, y=y, y_dtype=y_dtype)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        hdq.quantize(xd, hb, fmt, tensor_amax=amax, out=xq)
        e[1].record()
        hdq.linear(prec, None, W, xq=xq, y=y, y_dtype=y_dtype)
        e[2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tq = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    tg = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    flops = 2.0 * M * N * K
    qb = quant_bytes(M, K, "int8" if path == "int8" else "nvfp4", decoded)
    dt = "int8" if path == "int8" else ("bf16" if args.fp4 == "nvfp4" else "fp4")
    res = {"metric": METRIC, "value": round(flops / ((tq + tg) * 1e-3) / 1e12, 2), "unit": "TOPS",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
           "config": {"workload": c["name"], "global_batch": M},
           "quant_gbps": round(qb / (tq * 1e-3) / 1e9, 1), "quant_ms": round(tq, 4),
           "gemm_ms": round(tg, 4),
           "roofline": {"kernel": f"gemm_{path}", "bound": "mfma", "dtype": dt,
                        "achieved": round(flops / (tg * 1e-3) / 1e12, 1), "peak": PEAK[dt] / 1e12,
                        "unit": "TFLOP/s" if dt != "int8" else "TOP/s",
                        "frac": round(flops / (tg * 1e-3) / PEAK[dt], 4), "traffic": None},
           "quant_roofline": {"bound": "hbm", "achieved": round(qb / (tq * 1e-3) / 1e9, 1), "peak": 8000.0,
                              "unit": "GB/s", "frac": round(qb / (tq * 1e-3) / PEAK["hbm"], 4)}}
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the work shards by tokens; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.profile_copy:
        profile_copy()
        return
    from bit_quantized_video_amd import hdq, synth
    if args.config == 5:
        res = bench_schedule(args, hdq, synth)
    else:
        res = bench_single(args, hdq, synth)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
