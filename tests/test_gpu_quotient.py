"""The cast's quotient (quotient() in the library's device code: RN(y / ds) from rcp = RN(1 / ds),
one product and one FMA remainder correction) against correctly rounded division, on the GPU
through tests/hip/h3check.hip, built with the library's flags.

- Every pair of significands: ds and y each over all 2^23 significands of [1, 2) (and -y for every
  16th y), 2^46 quotients in (1/2, 2), compared bit for bit.  Multiplying y or ds by a power of two
  scales every intermediate of the sequence exactly as long as all of them stay normal binary32
  numbers, which holds for every descale in the fast path's range [2^-60, 2^60] and every quotient
  of magnitude in [2^-12, 512); so this sweep settles that whole region, whatever the exponents.
- Every finite y at 80 descales (the ends of the range, the largest significands at its edge
  exponents, amax / 448 descales met in practice, seeded random ones): the bits of y / ds wherever
  |y / ds| is in [2^-12, 512), the same E4M3 code (a signed zero) below 2^-12, and a NaN or a
  magnitude past 448 with the right sign at 512 and beyond (the exact path or the saturated code).
"""
import ctypes
import struct

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


def _f(bits):
    return np.float32(struct.unpack("<f", struct.pack("<I", bits))[0])


def _descales():
    """Powers of two at both ends and the middle of the range, the extreme significands at the edge
    exponents (2^-60 and 2^59 binades, and the last value below 2^60), descales of the amax / 448
    form for amaxes met in practice, and seeded random values with exponents across
    [2^-60, 2^60)."""
    ds = [2.0 ** e for e in (-60, -31, -9, -1, 0, 1, 7, 30, 59, 60)]
    lo, hi = 0x21800000, 0x5D800000  # bits of 2^-60 and 2^60
    ds += [float(_f(b)) for b in (lo + 1, lo + 2, lo + 0x400000, lo + 0x7FFFFF, hi - 0x800000 + 1,
                                  hi - 0x400000, hi - 2, hi - 1)]
    ds += [float(np.float32(a) / np.float32(448.0)) for a in (1e-3, 0.37, 1.0, 3.7, 17.3, 448.0, 1000.0, 65504.0)]
    rng = np.random.default_rng(2024)
    while len(ds) < 80:
        ds.append(float(np.float32(2.0 ** rng.uniform(-60, 59.99))))
    return [np.float32(d) for d in ds]


@pytest.mark.parametrize("ds", _descales(), ids=lambda d: f"{float(d):.9g}")
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


PAIR_PARTS = 16


@pytest.mark.parametrize("part", range(PAIR_PARTS))
def test_quotient_every_significand_pair(part):
    """Descale significands [part, part + 1) / 16 of [0, 2^23) against every y significand."""
    from rmsnorm_rope_amd import _build
    L = ctypes.CDLL(_build.CHECK_LIB)
    L.h3check_quotient_pairs.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    span = (1 << 23) // PAIR_PARTS
    j0 = part * span
    step = span // 8  # eight launches of 2^16 descales each (2^31 work-items per launch)
    for j in range(j0, j0 + span, step):
        assert L.h3check_quotient_pairs(j, j + step, bad.data_ptr(), first.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    n = int(bad.item())
    print(f"[quotient pairs] descale significands {j0:#x}..{j0 + span - 1:#x} x every y significand: "
          f"{n} mismatches", flush=True)
    f = [int(x) & 0xFFFFFFFF for x in first.tolist()]
    assert n == 0, [(hex(0x3F800000 + f[2 * k]), hex(0x3F800000 + f[2 * k + 1])) for k in range(min(n, 2))]
