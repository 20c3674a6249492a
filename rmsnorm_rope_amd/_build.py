"""Build step for libh3qk: compiles the gfx950 HIP kernels and the C ABI into
rmsnorm_rope_amd/libh3qk.so with hipcc (in-tree, so the library travels with the sources)."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libh3qk.so")
SOURCES = [os.path.join(CSRC, f) for f in ("h3qk_kernels.hip", "h3_tensor_kernels.hip", "h3_block_kernels.hip",
                                             "h3qk_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "h3qk.h"), os.path.join(CSRC, "h3qk_internal.h"),
           os.path.join(CSRC, "h3qk_device.h")]
# test-only check kernels over the library's device helpers, built beside their sources
CHECK_SRC = os.path.join(ROOT, "tests", "hip", "h3check.hip")
CHECK_LIB = os.path.join(ROOT, "tests", "hip", "libh3check.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # the numerical contract: no contraction, no fast-math, IEEE denormals, correctly rounded
    # division and square root in device code
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (one hipcc per file), then link the library."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="h3qk_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(src) + ".o") for src in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            futs = [ex.submit(_run, [HIPCC, *FLAGS, *inc, "-c", "-o", obj, src], verbose)
                    for src, obj in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", LIB + ".tmp", *objs], verbose)
    os.replace(LIB + ".tmp", LIB)
    if os.path.exists(CHECK_SRC):
        _run([HIPCC, *FLAGS, *inc, "-shared", "-o", CHECK_LIB + ".tmp", CHECK_SRC], verbose)
        os.replace(CHECK_LIB + ".tmp", CHECK_LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    if any(os.path.getmtime(f) > t for f in SOURCES + HEADERS):
        return True
    if os.path.exists(CHECK_SRC):
        if not os.path.exists(CHECK_LIB):
            return True
        tc = os.path.getmtime(CHECK_LIB)
        return any(os.path.getmtime(f) > tc for f in [CHECK_SRC] + HEADERS)
    return False


if __name__ == "__main__":
    print(build(verbose=True))
