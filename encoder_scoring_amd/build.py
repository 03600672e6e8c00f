"""Build libencscore.so in-tree for gfx950 with hipcc (no JIT, no torch extension).

    python -m encoder_scoring_amd.build          # compile + link
    python -m encoder_scoring_amd.build --host   # also the g++ host-only library

The shared library lands next to this file, where the Python binding loads it.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libencscore.so")
HOST_LIB = os.path.join(HERE, "libencscore_host.so")

SOURCES = ["planner.cpp", "blob.cpp", "memplan.cpp", "layout.cpp", "model.hip", "ops.hip", "rowops.hip", "gemm.hip", "attn.hip"]
HOST_SOURCES = ["planner.cpp", "blob.cpp", "memplan.cpp", "layout.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libencscore)")


# Per-source extras: the attention kernels keep their MFMA accumulators in
# VGPRs (the default AGPR form costs a copy of every accumulator at each
# online-softmax rescale).
EXTRA_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src, obj):
    cmd = [_hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noisy = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return src, noisy


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, warn in ex.map(_compile, SOURCES, objs):
            if verbose or warn:
                print(f"[encscore build] {src}: {'ok' if not warn else chr(10).join(warn)}")
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_host(extra_flags=(), out=None):
    """Host-only part (planner, arena planner, blob parser, pass metadata and
    its checker) with g++, no HIP; used by the CPU tests.  `extra_flags`
    (e.g. sanitizers) and `out` (another output path) for special builds."""
    out = out or HOST_LIB
    cmd = ["g++", "-O2", "-g", "-fPIC", "-shared", "-std=c++17", "-Wall", *extra_flags,
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host build failed: {' '.join(cmd)}\n{r.stderr}")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--host", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(verbose=a.verbose))
    if a.host:
        print(build_host())


if __name__ == "__main__":
    sys.exit(main())
