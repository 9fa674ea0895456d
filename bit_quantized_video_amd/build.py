"""Builds libhdq.so (all HIP sources under csrc/) for gfx950 with hipcc.

Flags:
  -O3 --offload-arch=gfx950      CDNA4 code only
  -ffp-contract=off              no FMA contraction: every float expression
                                 rounds where written (quantized codes and the
                                 INT8 epilogue must match the reference rounding)
  -target-feature -packed-fp32-ops
                                 keep the compiler from emitting packed fp32
                                 VALU ops (the host pass warns that it does not
                                 know the feature; harmless)
Division and square root stay IEEE (hipcc's default correctly rounded fp32
divide), which the scale computations rely on.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libhdq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(jobs=None, verbose=False):
    """Compile every csrc/*.hip to an object (in parallel) and link libhdq.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    procs = []
    objs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *[f for f in FLAGS if f != "-shared"], "-I", INCLUDE, "-I", CSRC,
               "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append((src, "\n".join(noise)))
        elif verbose and noise:
            print("\n".join(noise))
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
