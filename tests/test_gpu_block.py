"""GPU parity of the decoder-block elementwise ops (SwiGLU, scaled residual) against the oracle,
through the C ABI, bit for bit: the scaled residual in binary32 with the product rounded first;
SwiGLU as the binary64 value rounded once to the 16-bit output (the kernel's binary32 fast path is
used only where its rounding is certain; tests/test_gpu_swiglu_exhaustive.py covers every input
pair).  NaN outputs match any NaN."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits, compare

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    yield


def run_swiglu(xb, dt):
    import rmsnorm_rope_amd as h3
    N, F2 = xb.shape
    x = torch.from_numpy(xb.view(np.int16).copy()).cuda()
    y = torch.empty((N, F2 // 2), dtype=torch.int16, device="cuda")
    h3.h3_swiglu(x, dt, y, N, F2 // 2)
    torch.cuda.synchronize()
    return bits(y)


@pytest.mark.parametrize("N,F,dt", [(1797, 8192, "f16"), (1, 8, "f16"), (3, 24, "f16"), (257, 1000, "f16"),
                                    (64, 512, "bf16"), (1797, 8192, "bf16")])
def test_swiglu(N, F, dt):
    xb = synth.swiglu_input(N, F, dt)
    got = run_swiglu(xb, dt)
    ref = oracle.swiglu(xb, dt)
    hist = compare(got, ref, dt, "swiglu")
    print("swiglu", N, F, dt, "ulp histogram", hist, flush=True)


def test_swiglu_special_values():
    x = np.zeros((2, 16), np.float16)
    x[0, :8] = [0.0, 20.0, -20.0, 65504.0, -65504.0, -90.0, 1e-7, -1e-7]
    x[0, 8:] = [1.5, -2.0, 3.0, 1.0, 1.0, 4.0, 1.0, 1.0]
    x[1, :8] = [np.inf, -np.inf, np.nan, 5.0, -5.0, 0.5, -0.5, 11.0]
    x[1, 8:] = [1.0, 1.0, 1.0, np.inf, 0.0, -0.0, 2.0, 1e-3]
    got = run_swiglu(x.view(np.uint16), "f16")
    ref = oracle.swiglu(x.view(np.uint16), "f16")
    compare(got, ref, "f16", "swiglu specials")


def run_residual(res, br, sc, dt):
    import rmsnorm_rope_amd as h3
    N, C = res.shape
    r = torch.from_numpy(res).cuda()
    b = torch.from_numpy(br.view(np.int16).copy()).cuda()
    s = torch.from_numpy(np.ascontiguousarray(sc, np.float32)).cuda()
    o = torch.empty_like(r)
    h3.h3_scaled_residual(r, b, dt, s, s.numel(), o, N, C)
    torch.cuda.synchronize()
    return bits(o)


@pytest.mark.parametrize("N,C,dt,per_channel", [(3594, 2048, "f16", True), (3594, 2048, "f16", False),
                                                (1, 4, "f16", True), (5, 36, "bf16", True), (1000, 2048, "bf16", False)])
def test_scaled_residual(N, C, dt, per_channel):
    res, br, sc = synth.residual_inputs(N, C, dt)
    if not per_channel:
        sc = sc[:1]
    got = run_residual(res, br, sc, dt)
    ref = oracle.scaled_residual(res, br, sc, dt)
    compare(got, ref.view(np.uint32), "f32", "scaled residual")


def test_scaled_residual_no_contraction_and_specials():
    b = np.float16(1 + 2.0 ** -10)
    s = np.float32(1 + 2.0 ** -14 + 2.0 ** -23)
    p = np.float32(np.float32(b) * s)
    res = np.array([[-p, 1.0, -0.0, np.inf]], np.float32)
    br = np.array([[b, np.float16(0.0), np.float16(-0.0), np.float16(1.0)]], np.float16)
    sc = np.array([s, 2.0, 3.0, -np.inf], np.float32)
    got = run_residual(res, br.view(np.uint16), sc, "f16")
    ref = oracle.scaled_residual(res, br.view(np.uint16), sc, "f16")
    compare(got, ref.view(np.uint32), "f32", "scaled residual specials")
    assert got.view(np.float32)[0, 0] == 0.0
