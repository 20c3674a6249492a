"""Helpers for the GPU parity tests: bit views of device tensors and comparisons that report
the ulp histogram of any deviation."""
import numpy as np


def bits(t):
    """numpy bit view of a tensor copied to the host (uint32 / uint16 / uint8)."""
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.float32:
        return a.numpy().view(np.uint32)
    if a.dtype in (torch.float16, torch.bfloat16, torch.int16):
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def _as_bits(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def _is_nan(b, dt):
    if dt == "f32":
        return (b & 0x7FFFFFFF) > 0x7F800000
    if dt == "f16":
        return (b & 0x7FFF) > 0x7C00
    if dt == "bf16":
        return (b & 0x7FFF) > 0x7F80
    if dt == "e4m3":
        return (b & 0x7F) == 0x7F
    return np.zeros(b.shape, bool)


def _ordinal(b, dt):
    """Monotone integer image of the encoding, so |a - b| counts ulps across zero."""
    b = b.astype(np.int64)
    sign_bit = {"f32": 1 << 31, "f16": 1 << 15, "bf16": 1 << 15, "e4m3": 1 << 7}[dt]
    mag = b & (sign_bit - 1)
    return np.where(b & sign_bit, -mag, mag)


def compare(got, ref, dt, what, max_ulp=0):
    """Element-wise comparison of two encodings of dtype dt.  NaN matches any NaN (payloads are
    not part of the contract); every other element must agree within max_ulp ulps.  Returns the
    ulp histogram {0: n, 1: n, '>1': n}."""
    g, r = _as_bits(got), _as_bits(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gn, rn = _is_nan(g, dt), _is_nan(r, dt)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({int(np.sum(gn != rn))})"
    m = ~rn
    d = np.abs(_ordinal(g[m], dt) - _ordinal(r[m], dt)) if dt != "raw" else (g[m] != r[m]).astype(np.int64)
    hist = {0: int(np.sum(d == 0)), 1: int(np.sum(d == 1)), ">1": int(np.sum(d > 1))}
    if int(d.max(initial=0)) > max_ulp:
        flat = np.flatnonzero(m)[d > max_ulp][:5]
        raise AssertionError(f"{what}: {int(np.sum(d > max_ulp))} elements beyond {max_ulp} ulp, histogram {hist}; "
                             f"first at flat {flat.tolist()}: got {g.ravel()[flat].tolist()} ref {r.ravel()[flat].tolist()}")
    return hist


def compare_raw(got, ref, what):
    g, r = np.asarray(got), np.asarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if not np.array_equal(g, r):
        bad = np.flatnonzero(g.ravel() != r.ravel())
        raise AssertionError(f"{what}: {bad.size} differing elements, first at {bad[:5].tolist()}: "
                             f"got {g.ravel()[bad[:5]].tolist()} ref {r.ravel()[bad[:5]].tolist()}")


def build_c_e2e(out_dir):
    """Compile tests/c/e2e_gpu.c (plain C99 with gcc) against the HIP runtime, libh3qk and the
    oracle library; returns the executable's path."""
    import os
    import subprocess

    import oracle
    import rmsnorm_rope_amd as h3
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    oracle_lib = oracle.build(force=False)
    libdirs = [os.path.dirname(h3.LIB_PATH), os.path.dirname(oracle_lib), "/opt/rocm/lib"]
    exe = os.path.join(str(out_dir), "e2e_gpu")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
           os.path.join(root, "tests", "c", "e2e_gpu.c"), "-o", exe,
           "-L", libdirs[0], "-lh3qk", "-L", libdirs[1], "-loracle_h3ref", "-L", libdirs[2], "-lamdhip64",
           "-Wl,-rpath," + ":".join(libdirs), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe
