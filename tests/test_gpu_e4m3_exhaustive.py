"""Exhaustive checks of the E4M3 encodings the cast passes use, on the GPU through the library's own
device code (tests/hip/h3check.hip, built with the library's flags).  The chain of trust:

1. the oracle's encoder (oracle/h3ref.c) is pinned on the CPU against a brute-force nearest-code
   search and torch's float8_e4m3fn cast (tests/test_oracle_pins.py);
2. the library's integer encoder f32_to_e4m3, run on the GPU, gives the oracle encoder's code for
   every one of the 2^32 binary32 bit patterns (compared on the host);
3. the gfx950 conversion instruction, as the fast path calls it (pack_e4m3 with hw = true), gives
   f32_to_e4m3's code for every binary32 of magnitude <= 448, and after the clip path's clamp
   (clamp_e4m3) for every non-NaN binary32, +-inf included;
4. the whole wave-level cast (cast_e4m3_wave) at descale 1, where the quotient is the value itself,
   gives f32_to_e4m3's codes and the right clip count for every bit pattern, with the waves filled
   in order (homogeneous waves: the fast path, the clip path, the exact path of NaN waves) and
   scattered (waves mixing in-range, clipped and NaN values).

The per-tensor E4M3 cast is the one in [TRT-21485] (TensorRT-LLM PR #21485), Summary and the
fused_fp8_qk commit; the encoding is OCP E4M3FN, round to nearest even, saturating."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F448 = 0x43E00000  # bits of 448.0
INF = 0x7F800000


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    torch.cuda.set_device(0)
    yield


def _lib():
    from rmsnorm_rope_amd import _build
    L = ctypes.CDLL(_build.CHECK_LIB)
    u32, vp, i = ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    L.h3check_e4m3_codes.argtypes = [u32, u32, vp, vp]
    L.h3check_e4m3_hw.argtypes = [u32, u32, i, vp, vp, vp]
    L.h3check_cast_wave.argtypes = [u32, u32, i, vp, vp, vp, vp]
    return L


def _counters():
    return (torch.zeros(1, dtype=torch.int64, device="cuda"), torch.zeros(4, dtype=torch.int32, device="cuda"),
            torch.cuda.current_stream().cuda_stream)


def _first(first, n):
    return [hex(int(x) & 0xFFFFFFFF) for x in first.tolist()[:min(n, 4)]]


@pytest.mark.parametrize("quarter", range(4))
def test_integer_encoder_matches_oracle(quarter):
    """f32_to_e4m3 on the GPU == the oracle's h3ref_e4m3_encode for every bit pattern of one quarter
    of the 2^32, in chunks of 2^28 compared on the host."""
    import oracle
    L = _lib()
    chunk = 1 << 28
    codes = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    total_bad = 0
    for c in range(4):
        lo = (quarter * 4 + c) * chunk
        assert L.h3check_e4m3_codes(lo, chunk, codes.data_ptr(), stream) == 0
        got = codes.cpu().numpy()
        x = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        ref = oracle.encode(x, "e4m3")
        bad = np.flatnonzero(got != ref)
        total_bad += bad.size
        assert bad.size == 0, (f"patterns from {lo:#x}: {bad.size} codes differ, first at "
                               f"{[hex(lo + int(b)) for b in bad[:4]]}: got {got[bad[:4]].tolist()} "
                               f"oracle {ref[bad[:4]].tolist()}")
    print(f"[e4m3 encoder] patterns {quarter * 4 * chunk:#x}..{(quarter + 1) * 4 * chunk - 1:#x}: "
          f"{total_bad} differences from the oracle", flush=True)


@pytest.mark.parametrize("lo,hi,clamp,what", [
    (0x00000000, F448, 0, "every v in [+0, 448], unclamped"),
    (0x80000000, 0x80000000 | F448, 0, "every v in [-448, -0], unclamped"),
    (0x00000000, INF, 1, "every v in [+0, +inf], clamped"),
    (0x80000000, 0x80000000 | INF, 1, "every v in [-inf, -0], clamped"),
])
def test_conversion_instruction(lo, hi, clamp, what):
    L = _lib()
    bad, first, stream = _counters()
    assert L.h3check_e4m3_hw(lo, hi, clamp, bad.data_ptr(), first.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    n = int(bad.item())
    print(f"[e4m3 conversion] {what}: {hi - lo + 1} values, {n} mismatches", flush=True)
    assert n == 0, _first(first, n)


# non-NaN patterns past 448 in magnitude, (448, +inf] of either sign: what a full sweep must count
CLIPPED_PATTERNS = 2 * (INF - F448)


@pytest.mark.parametrize("order,what", [
    (0, "waves filled in order"),
    (1, "waves of scattered patterns (NaNs included)"),
    (2, "waves of scattered patterns, NaNs made finite"),
])
def test_wave_cast(order, what):
    L = _lib()
    bad, first, stream = _counters()
    sat = torch.zeros(1, dtype=torch.int64, device="cuda")
    waves = 1 << 24
    step = 1 << 22
    for w0 in range(0, waves, step):
        assert L.h3check_cast_wave(w0, w0 + step, order, bad.data_ptr(), first.data_ptr(), sat.data_ptr(),
                                   stream) == 0
    torch.cuda.synchronize()
    n, s = int(bad.item()), int(sat.item())
    print(f"[e4m3 wave cast] {what}: 2^32 values, {n} mismatches, {s} clipped", flush=True)
    assert n == 0, _first(first, n)
    if order < 2:  # the identity and the multiplicative map visit every pattern once
        assert s == CLIPPED_PATTERNS, (s, CLIPPED_PATTERNS)
