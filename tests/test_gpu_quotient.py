"""The cast's quotient (quotient() in the library's device code: RN(y / ds) from rcp = RN(1 / ds),
one product and FMA remainder corrections) against correctly rounded division, for every finite
binary32 y and 64 descales across the fast path's range [2^-60, 2^60]: the bits of y / ds wherever
|y / ds| is in [2^-12, 512), the same E4M3 code (a signed zero) below 2^-12, and a NaN or a
magnitude past 448 with the right sign at 512 and beyond (the exact path or the saturated code).
An exhaustive check on the GPU through tests/hip/rsqrt_check.hip, built with the library's flags."""
import ctypes

import numpy as np
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


def _descales():
    """Powers of two at both ends and the middle of the range, descales of the amax / 448 form for
    amaxes met in practice, and seeded random values with exponents across [2^-60, 2^60)."""
    ds = [2.0 ** e for e in (-60, -31, -9, -1, 0, 1, 7, 30, 59)]
    ds += [float(np.float32(a) / np.float32(448.0)) for a in (1e-3, 0.37, 1.0, 3.7, 17.3, 448.0, 1000.0, 65504.0)]
    rng = np.random.default_rng(2024)
    for _ in range(64 - len(ds)):
        ds.append(float(np.float32(2.0 ** rng.uniform(-60, 59.99))))
    return [np.float32(d) for d in ds]


@pytest.mark.parametrize("ds", _descales(), ids=lambda d: f"{float(d):.6g}")
def test_quotient_matches_division(ds):
    from rmsnorm_rope_amd import _build
    assert 2.0 ** -60 <= ds <= 2.0 ** 60
    L = ctypes.CDLL(_build.CHECK_LIB)
    L.h3check_quotient.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for lo, hi in ((0x00000000, 0x7F800000), (0x80000000, 0xFF800000)):  # finite y of either sign
        assert L.h3check_quotient(lo, hi, float(ds), bad.data_ptr(), first.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    n = int(bad.item())
    print(f"[quotient] ds = {float(ds):.9g}: {n} mismatches over every finite y", flush=True)
    assert n == 0, [hex(int(x) & 0xFFFFFFFF) for x in first.tolist()[:min(n, 4)]]
