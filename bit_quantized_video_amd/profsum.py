"""Text summaries of rocprofv3 runs of the mixed-precision schedule benchmark.

Two modes, each reading the rocpd SQLite database(s) rocprofv3 writes:

  trace    per-kernel durations from a ``--kernel-trace --stats`` run: the
           profiler's own top-kernel table plus, for each step of the path, the
           launches that did work.  Every layer call launches all three
           precisions' quantizer and GEMM behind a device-side decision gate;
           the launches whose gate is closed return at once (a few
           microseconds) and are listed separately.
  traffic  HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run of
           the benchmark, calibrated against the same counters read for a
           plain device copy of known size.
  mfma     matrix-core utilisation of the GEMMs from one counter run:
           SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) over the SIMD-cycles
           of the launch (GRBM_GUI_ACTIVE, summed over the 8 XCDs, /8 x 1024
           SIMDs), and the MFMA op count (MOPS x 512) against 2 M N K.

The summary ends with machine-readable ``traffic`` lines (kind, bytes per
launch, hash of the sources the kernel is built from) that the benchmark reads
to fill its roofline record; it reports null once those sources changed.

Usage (paths are the rocprofv3 output databases; --decisions F is the
benchmark's --decisions-out file, which attributes each one-launch GEMM to
the precision its layer call decided):
  python3 -m bit_quantized_video_amd.profsum trace DB [--bench-json F] [--decisions F]
  python3 -m bit_quantized_video_amd.profsum traffic --fetch DB --write DB
          --copy-fetch DB --copy-write DB --copy-bytes N [--decisions F]
  python3 -m bit_quantized_video_amd.profsum mfma DB [--decisions F]
"""
import argparse
import hashlib
import json
import os
import re
import sqlite3
import sys
from collections import OrderedDict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# Step of the path -> kernel-name pattern (bf16-output GEMMs only: the
# schedule writes bf16; the f32-output variants belong to the quality check).
KINDS = OrderedDict([
    ("delta_sums", r"k_stats_partial<1>"),
    ("select_stats", r"k_stats_partial(<[02]>)?"),
    ("select_final_rows", r"k_stats_final_rows"),
    ("select_final", r"k_stats_final"),
    ("select_quant_int8", r"k_quant_int_rows<\d+, \d+, false, true(, \d+)?(, (true|false))?>"),
    ("quant_int8", r"k_quant_int_rows(_long)?<\d+, \d+, false(, false(, \d+)?(, (true|false))?)?>"),
    ("quant_nvfp4_mx", r"k_quant_nvfp4(_w32)?<3(, \d+)?(, (true|false))?>"),
    ("quant_nvfp4_p2", r"k_quant_nvfp4(_w32)?<4(, \d+)?(, (true|false))?>"),
    ("quant_nvfp4", r"k_quant_nvfp4(_w32)?<2(, \d+)?(, (true|false))?>"),
    ("decode_nvfp4", r"k_dq_decode_w"),
    ("gemm_int8", r"k_gemm_i8i4(_pipe)?<[\d, ]*1>"),
    ("gemm_nvfp4_mx", r"k_gemm_fp4mx_pipe<1, false>"),
    ("gemm_nvfp4_p2", r"k_gemm_fp4mx_pipe<1, true>"),
    ("gemm_nvfp4", r"k_gemm_bf16(_pipe|mfma)<[12], 1>"),
    ("gemm_bf16", r"k_gemm_bf16(_pipe|mfma)<0, 1>"),
])
# Sources each kind is built from (any change voids a stored traffic figure).
SOURCES = {
    "delta_sums": ["stats.hip"], "select_stats": ["stats.hip"], "select_final": ["stats.hip"],
    "select_final_rows": ["stats.hip"],
    "quant_int8": ["quant.hip"], "quant_nvfp4_mx": ["quant.hip"], "quant_nvfp4": ["quant.hip"],
    "quant_nvfp4_p2": ["quant.hip"], "decode_nvfp4": ["quant.hip"],
    "select_quant_int8": ["quant.hip", "stats.hip"],
    "gemm_int8": ["gemm_i8.hip", "gemm_i8_pipe.h", "gemm_dispatch.hip"],
    "gemm_nvfp4_mx": ["gemm_fp4.hip", "gemm_fp4_pipe.h", "gemm_dispatch.hip"],
    "gemm_nvfp4_p2": ["gemm_fp4.hip", "gemm_fp4_pipe.h", "gemm_dispatch.hip"],
    "gemm_nvfp4": ["gemm_bf16.hip", "gemm_bf16_pipe.h", "gemm_dispatch.hip"],
    "gemm_bf16": ["gemm_bf16.hip", "gemm_bf16_pipe.h", "gemm_dispatch.hip"],
    "gemm_dispatch": ["gemm_dispatch.hip", "gemm_i8_pipe.h", "gemm_fp4_pipe.h", "gemm_bf16_pipe.h"],
}
# One-launch GEMMs (bf16 output) that run the decided precision: the kind
# comes from the decision of the layer call (DECISIONS, in call order); the
# second template argument is the NVFP4 weights' format (2 plain, 3 MX, 4
# per-16 powers of two; 16 plain from operands decoded to bf16, 17 from
# decoded activations only).
DISPATCH = r"k_gemm_dispatch<1, (2|3|4|16|17)>"
FP4_KIND = {"2": "gemm_nvfp4", "3": "gemm_nvfp4_mx", "4": "gemm_nvfp4_p2", "16": "gemm_nvfp4", "17": "gemm_nvfp4"}
DECISIONS = None


def load_decisions(path):
    global DECISIONS
    if path:
        with open(path) as fh:
            DECISIONS = json.load(fh)["decisions"]


class Classifier:
    """Kernel name -> kind, counting one-launch GEMMs per recipe so that the
    i-th one takes the i-th layer call's decision."""

    def __init__(self):
        self.seen = {}

    def __call__(self, name):
        m = re.search(DISPATCH, name)
        if m is None:
            return classify(name)
        if not DECISIONS:
            return "gemm_dispatch"
        fmt = m.group(1)
        i = self.seen.get(fmt, 0)
        self.seen[fmt] = i + 1
        d = DECISIONS[i % len(DECISIONS)]
        return {1: "gemm_int8", 0: FP4_KIND[fmt], 2: "gemm_bf16"}[d]
COMMON_SOURCES = ["hdq_device.h", "hdq_internal.h", "../build.py"]
WEIGHT_PREP = r"k_quant_int_rows(_long)?<\d+, \d+, true(, false(, \d+)?(, (true|false))?)?>"
# A launch that did work: longer than this (trace; gated-off launches take a
# few microseconds, more when a concurrent stream shares the GPU, and the
# smallest GEMM that does work takes over 100) / moved more than this (PMC).
MIN_WORK_NS = {"gemm": 60_000, "quant": 12_000}
MIN_WORK_NS_DEFAULT = 12_000
MIN_WORK_KIB = 1024.0


def min_work_ns(kind):
    return MIN_WORK_NS.get(kind.split("_")[0], MIN_WORK_NS_DEFAULT)


def code_only(text):
    """Source text without comments and whitespace: a change to comments
    alone leaves the kernel, and so its measured traffic, as it was."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"(?m)^\s*#(?!\s*(include|define|if|else|elif|endif|pragma)).*$", " ", text)
    return "".join(text.split())


def sources_hash(kind):
    h = hashlib.sha256()
    for f in SOURCES[kind] + COMMON_SOURCES:
        with open(os.path.normpath(os.path.join(CSRC, f)), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def classify(name):
    for kind, pat in KINDS.items():
        if re.search(pat, name):
            return kind
    return None


def schedule_window(rows):
    """rows: (dispatch_id, name, ...) in dispatch order.  The schedule starts
    at the first dispatch after the last weight preparation (INT4 weight
    quantization) and ends at the last bf16-output GEMM."""
    last_prep = max((i for i, r in enumerate(rows) if re.search(WEIGHT_PREP, r[1])), default=-1)
    is_gemm = lambda n: re.search(DISPATCH, n) or (classify(n) or "").startswith("gemm")
    gemm = [i for i, r in enumerate(rows) if is_gemm(r[1])]
    end = max(gemm) if gemm else len(rows) - 1
    return rows[last_prep + 1:end + 1]


def short(name, n=90):
    name = name.split("(")[0]
    return name if len(name) <= n else name[:n - 3] + "..."


# ------------------------------------------------------------------- trace

def trace_summary(db, bench_json=None, command=None):
    c = sqlite3.connect(db)
    out = []
    if command:
        out.append(f"command: {command}")
    out.append(f"source: rocprofv3 kernel trace database ({os.path.basename(db)})")
    out.append("")
    out.append("profiler top kernels (all launches, gated-off ones included):")
    out.append(f"  {'calls':>7} {'total ms':>11} {'avg us':>10} {'%':>6}  kernel")
    for name, calls, tot, avg, pct in c.execute(
            "select name, total_calls, total_duration, average, percentage from top_kernels "
            "order by total_duration desc limit 20"):
        # rocpd reports total_duration and average in microseconds
        out.append(f"  {calls:>7} {tot / 1e3:>11.3f} {avg:>10.2f} {pct:>6.2f}  {short(name)}")
    rows = list(c.execute("select dispatch_id, name, duration, grid_x from kernels order by start"))
    win = schedule_window(rows)
    out.append("")
    out.append(f"schedule window: {len(win)} dispatches (after the last weight preparation)")
    out.append("launches that did work (GEMMs > 60 us, others > 12 us; finalize and difference passes")
    out.append("always) vs gated off, per step of the path:")
    out.append(f"  {'kind':<16} {'work':>6} {'avg us':>10} {'total ms':>10} {'off':>6} {'off avg us':>11}")
    per = OrderedDict((k, ([], [])) for k in list(KINDS) + ["gemm_dispatch"])
    cls = Classifier()
    for _, name, dur, _ in win:
        k = cls(name)
        if k is None:
            continue
        # the finalize and the difference pass are never gated off
        ungated = k.startswith("select_final") or k == "delta_sums"
        per[k][0 if ungated or dur > min_work_ns(k) else 1].append(dur)
    summary = {}
    for k, (w, off) in per.items():
        if not w and not off:
            continue
        aw = sum(w) / len(w) / 1e3 if w else 0.0
        ao = sum(off) / len(off) / 1e3 if off else 0.0
        summary[k] = aw
        out.append(f"  {k:<16} {len(w):>6} {aw:>10.2f} {sum(w) / 1e6:>10.3f} {len(off):>6} {ao:>11.2f}")
    if bench_json:
        with open(bench_json) as fh:
            line = [l for l in fh.read().splitlines() if l.startswith("{")][-1]
        b = json.loads(line)
        out.append("")
        out.append("same run, benchmark's own HIP-event averages (headline recipe, timed steps):")
        for k, v in b.get("kernels", {}).items():
            if k.endswith("_gated_off"):
                continue
            out.append(f"  {k:<16} launches {v['launches']:>5}  avg {v['avg_us']:>9.2f} us")
        rl = b.get("roofline", {})
        out.append(f"  roofline kernel {rl.get('kernel')}: achieved {rl.get('achieved')} {rl.get('unit')}, "
                   f"frac {rl.get('frac')}")
        out.append(f"  value {b.get('value')} {b.get('unit')}, {b.get('ms_per_step')} ms/step")
    return "\n".join(out) + "\n"


# ----------------------------------------------------------------- traffic

def pmc_rows(db, counter):
    c = sqlite3.connect(db)
    return list(c.execute(
        "select dispatch_id, kernel_name, sum(value), grid_size from counters_collection "
        "where counter_name = ? group by dispatch_id order by dispatch_id", (counter,)))


def copy_factor(db, counter, nbytes):
    rows = [r for r in pmc_rows(db, counter) if "copyBuffer" in r[1] and r[2] > MIN_WORK_KIB]
    if not rows:
        raise SystemExit(f"no copy dispatch with {counter} in {db}")
    kib = sum(r[2] for r in rows) / len(rows)
    return nbytes / (kib * 1024.0), kib, len(rows)


def traffic_summary(fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes, command=None):
    ff, ckf, nf = copy_factor(copy_fetch_db, "FETCH_SIZE", copy_bytes)
    wf, ckw, nw = copy_factor(copy_write_db, "WRITE_SIZE", copy_bytes)
    out = []
    if command:
        out.append(f"commands: {command}")
    out.append(f"calibration: a device copy of {copy_bytes} bytes ({nf} launches) reads FETCH_SIZE "
               f"{ckf:.0f} KiB and WRITE_SIZE {ckw:.0f} KiB per launch")
    out.append(f"  -> HBM bytes = FETCH_SIZE KiB x 1024 x {ff:.4f} + WRITE_SIZE KiB x 1024 x {wf:.4f}")
    out.append("  (FETCH_SIZE/WRITE_SIZE count L2-to-fabric traffic, so bytes served by the")
    out.append("   Infinity Cache are included: an upper bound on DRAM bytes)")
    out.append("")
    # Both runs execute the same deterministic command, so the schedule
    # windows align dispatch by dispatch; a launch did work if it fetched
    # more than MIN_WORK_KIB (gated-off launches read a few KiB of arguments).
    fwin = schedule_window(pmc_rows(fetch_db, "FETCH_SIZE"))
    wwin = schedule_window(pmc_rows(write_db, "WRITE_SIZE"))
    if [r[1] for r in fwin] != [r[1] for r in wwin]:
        raise SystemExit("FETCH_SIZE and WRITE_SIZE runs dispatched different kernel sequences")
    per = {}
    cls = Classifier()
    for (_, name, fkib, _), (_, _, wkib, _) in zip(fwin, wwin):
        k = cls(name)
        if k is None:
            continue
        d = per.setdefault(k, {"FETCH_SIZE": [], "WRITE_SIZE": [], "off": 0})
        if fkib > MIN_WORK_KIB:
            d["FETCH_SIZE"].append(fkib)
            d["WRITE_SIZE"].append(wkib)
        else:
            d["off"] += 1
    out.append("per launch that did work (schedule window; gated-off launches read < 1 MiB):")
    out.append(f"  {'kind':<16} {'launches':>8} {'FETCH KiB':>12} {'WRITE KiB':>12} {'HBM MB':>10}")
    lines = []
    for k in list(KINDS) + ["gemm_dispatch"]:
        if k not in per:
            continue
        d = per[k]
        if not d["FETCH_SIZE"] or not d["WRITE_SIZE"]:
            continue
        fk = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"])
        wk = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"])
        b = fk * 1024 * ff + wk * 1024 * wf
        out.append(f"  {k:<16} {len(d['FETCH_SIZE']):>8} {fk:>12.0f} {wk:>12.0f} {b / 1e6:>10.1f}")
        lines.append(f"traffic {k} {b:.0f} {sources_hash(k)}")
    out.append("")
    out.append("# kind, HBM bytes per launch, sources hash")
    out.extend(lines)
    return "\n".join(out) + "\n"


def read_traffic(path):
    """{kind: (bytes per launch, sources hash)} from a traffic summary."""
    res = {}
    if not os.path.exists(path):
        return res
    with open(path) as fh:
        for line in fh:
            p = line.split()
            if len(p) == 4 and p[0] == "traffic":
                res[p[1]] = (float(p[2]), p[3])
    return res


def current_traffic(path, kind):
    """Stored bytes per launch for `kind`, or None when absent or when the
    kernel's sources changed since the counters were taken."""
    t = read_traffic(path).get(kind)
    if t is None or t[1] != sources_hash(kind):
        return None
    return t[0]


# ------------------------------------------------------------------- mfma

MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
N_XCD, N_SIMD = 8, 256 * 4


def mfma_summary(db, command=None):
    c = sqlite3.connect(db)
    rows = list(c.execute(
        "select dispatch_id, kernel_name, counter_name, sum(value), grid_size from counters_collection "
        "group by dispatch_id, counter_name order by dispatch_id"))
    disp = OrderedDict()
    for d, name, cn, v, g in rows:
        disp.setdefault(d, [d, name, {}])[2][cn] = v
    win = schedule_window(list(disp.values()))
    per = OrderedDict()
    cls = Classifier()
    for _, name, cnt in win:
        k = cls(name)
        if k is None or not k.startswith("gemm"):
            continue
        mops = sum(cnt.get(n, 0.0) for n in MFMA_COUNTERS[2:])
        if mops <= 0:
            continue  # gated off
        e = per.setdefault(k, {"n": 0, "busy": 0.0, "gui": 0.0, "ops": 0.0})
        e["n"] += 1
        e["busy"] += cnt["SQ_VALU_MFMA_BUSY_CYCLES"]
        e["gui"] += cnt["GRBM_GUI_ACTIVE"] / N_XCD
        e["ops"] += 512.0 * mops
    out = []
    if command:
        out.append(f"command: {command}")
    out.append("MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs)")
    out.append("(busy cycles relative to the clock the kernel actually ran at; the datasheet")
    out.append(" fraction in the benchmark's roofline record is relative to 2.4 GHz)")
    out.append(f"  {'kind':<16} {'launches':>8} {'MFMA ops/launch':>16} {'cycles/launch':>14} {'util':>7}")
    for k, e in per.items():
        util = e["busy"] / (N_SIMD * e["gui"])
        out.append(f"  {k:<16} {e['n']:>8} {e['ops'] / e['n']:>16.4e} {e['gui'] / e['n']:>14.0f} {util:>7.3f}")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--bench-json")
    t.add_argument("--command")
    t.add_argument("--decisions")
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--copy-fetch", required=True)
    f.add_argument("--copy-write", required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--command")
    f.add_argument("--decisions")
    m = sub.add_parser("mfma")
    m.add_argument("db")
    m.add_argument("--command")
    m.add_argument("--decisions")
    a = ap.parse_args(argv)
    load_decisions(a.decisions)
    if a.mode == "trace":
        sys.stdout.write(trace_summary(a.db, a.bench_json, a.command))
    elif a.mode == "mfma":
        sys.stdout.write(mfma_summary(a.db, a.command))
    else:
        sys.stdout.write(traffic_summary(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes,
                                         a.command))


if __name__ == "__main__":
    main()
