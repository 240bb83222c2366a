"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_42_amd.build [--verbose]

Every source under csrc/ is compiled to an object (in parallel), then linked into
paged_kv_cache_42_amd/libpkv.so. HIP code is built with packed-FP32 instructions
disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpkv.so")

ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


# The kernels issue some global stores as inline assembly that the compiler's wait-count
# and hazard passes do not see (mfma_common.h); that they stay correct was checked on
# the output of this compiler release. Another release may schedule differently, so the
# build refuses it unless PKV_ALLOW_UNCHECKED_COMPILER=1 (then rerun the GPU tests,
# test_small_mixed_steps with 5000 chunk slots in particular, before trusting results).
CHECKED_COMPILER = ("HIP version: 7.2.", "AMD clang version 22.")


def compiler_version() -> str:
    r = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    return r.stdout.strip()


def check_compiler() -> str:
    """The hipcc version text; raises unless it is the release the kernels were checked on."""
    text = compiler_version()
    lines = text.splitlines()
    ok = all(any(line.startswith(p) for line in lines) for p in CHECKED_COMPILER)
    if not ok and os.environ.get("PKV_ALLOW_UNCHECKED_COMPILER") != "1":
        raise RuntimeError(
            "libpkv's inline-assembly stores were checked with " + " / ".join(CHECKED_COMPILER) +
            f"*, not with:\n{text}\nSet PKV_ALLOW_UNCHECKED_COMPILER=1 to build anyway, then rerun the GPU tests.")
    if not ok:
        print(f"warning: building libpkv with an unchecked compiler:\n{text}", file=sys.stderr)
    return text


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "c++", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    err = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x and x.strip())
    if err and verbose:
        print(err)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    version = check_compiler()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(LIB + ".buildinfo", "w") as f:      # which compiler made this library
        f.write(version + "\n")
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
