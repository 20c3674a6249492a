"""The shorter reciprocal square root row_rstd takes when eps >= 2^-96 (rsqrt_rn_large: the
hardware square root corrected by two FMA residuals, then the hardware reciprocal with one FMA
Newton step) gives the bits of 1.0f / sqrtf(v), both correctly rounded, for every binary32 v in
[2^-96, +inf] and for every NaN pattern: an exhaustive check on the GPU through the library's
own device code (tests/hip/h3check.hip)."""
import ctypes
import os
import struct

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    torch.cuda.set_device(0)
    yield


def _bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


@pytest.mark.parametrize("lo,hi,what", [
    (_bits(2.0 ** -96), 0x7F800001, "every v in [2^-96, +inf]"),
    (0x7F800001, 0x80000000, "every positive-sign NaN"),
    (0xFF800001, 0xFFFFFFFF, "every negative-sign NaN but the last"),
])
def test_rsqrt_sequence_exhaustive(lo, hi, what):
    from rmsnorm_rope_amd import _build
    L = ctypes.CDLL(_build.CHECK_LIB)
    L.h3check_rsqrt.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert L.h3check_rsqrt(lo, hi, bad.data_ptr(), first.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    n = int(bad.item())
    print(f"[rsqrt] {what}: {hi - lo} values, {n} mismatches", flush=True)
    assert n == 0, [hex(int(x) & 0xFFFFFFFF) for x in first.tolist()[:min(n, 4)]]
