"""Pins of the oracle's decoder-block elementwise ops (SwiGLU, scaled residual) and of its
binary64 -> 16-bit encoders.  No GPU."""
import numpy as np
import pytest
from scipy.special import expit

import oracle

F = np.float32


def _bf16_values():
    b = np.arange(0x7F80, dtype=np.uint32)  # finite non-negative bfloat16
    return (b << 16).view(np.float32).astype(np.float64)


def test_f64_encoders_against_nearest_value():
    """binary64 -> binary16 / bfloat16 with one RNE rounding: against numpy's float16 cast of the
    double (a single rounding) and a brute-force nearest search over the bfloat16 values, on random
    doubles, exact midpoints and their neighbours."""
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        [0.0, 65504.0, 65519.999, 65520.0, 1e300, 6e-8, 2.0 ** -25, 2.0 ** -26]])
    h = np.array([oracle.f16_encode_f64(float(x)) for x in v], np.uint16)
    with np.errstate(over="ignore"):
        assert np.array_equal(h, v.astype(np.float16).view(np.uint16))
    vals = _bf16_values()
    mids = (vals[:-1] + vals[1:]) / 2
    pick = rng.integers(0, mids.size, 3000)
    cand = np.concatenate([mids[pick], np.nextafter(mids[pick], 0), np.nextafter(mids[pick], np.inf),
                           rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000)])
    for x in cand:
        a = abs(x)
        k = np.searchsorted(vals, a)
        lo, hi = vals[max(k - 1, 0)], vals[min(k, vals.size - 1)]
        if a - lo < hi - a or (a - lo == hi - a and (max(k - 1, 0) % 2 == 0)):
            want = lo
        else:
            want = hi
        got = oracle.bf16_encode_f64(float(x))
        gv = float(np.array([got & 0x7FFF], np.uint32).__lshift__(16).view(np.float32)[0])
        assert gv == want and (got >> 15) == (1 if np.signbit(x) else 0), (x, got, want)


def test_swiglu_matches_library_sigmoid():
    """silu(g) u = g sigmoid(g) u with scipy's expit as the sigmoid, both in binary64 and rounded
    once: identical binary16 codes (a mismatch would need a rounding tie within 1e-16)."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((512, 2 * 384)) * 3).astype(np.float16)
    y = oracle.swiglu(x.view(np.uint16)).view(np.float16)
    g, u = x[:, :384].astype(np.float64), x[:, 384:].astype(np.float64)
    assert np.array_equal(y, (g * expit(g) * u).astype(np.float16))


def test_swiglu_special_values():
    x = np.zeros((1, 16), np.float16)
    x[0, :8] = [0.0, 20.0, -20.0, 65504.0, -65504.0, np.inf, -np.inf, np.nan]
    x[0, 8:] = [1.5, -2.0, 3.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    y = oracle.swiglu(x.view(np.uint16)).view(np.float16)
    assert y[0, 0] == 0                                   # silu(0) = 0
    assert y[0, 1] == np.float16(-40.0)                   # silu(20) = 20 (1 - 2e-9)
    assert y[0, 2] == np.float16(3 * -20 * np.exp(-20.0)) # tiny negative, exactly as defined
    assert y[0, 3] == np.float16(65504.0) and y[0, 4] == 0 and np.signbit(y[0, 4])
    assert np.isnan(y[0, 5]) or y[0, 5] == np.inf        # inf / (1 + 0) = inf
    assert y[0, 6] == 0 or np.isnan(y[0, 6])
    assert np.isnan(y[0, 7])


def test_swiglu_bf16():
    rng = np.random.default_rng(9)
    xf = rng.standard_normal((64, 2 * 64)).astype(np.float32) * 4
    xb = oracle.encode(xf, "bf16").reshape(xf.shape)
    y = oracle.swiglu(xb, "bf16")
    g = (xb[:, :64].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    u = (xb[:, 64:].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = np.array([oracle.bf16_encode_f64(float(v)) for v in (g * expit(g) * u).ravel()], np.uint16)
    assert np.array_equal(y.ravel(), want)


def test_scaled_residual_closed_forms():
    rng = np.random.default_rng(10)
    N, C = 64, 256
    res = rng.standard_normal((N, C)).astype(F)
    br = rng.standard_normal((N, C)).astype(np.float16)
    sc = (1 + 0.1 * rng.standard_normal(C)).astype(F)
    # scale 1: one rounding of res + branch (numpy's binary32 add)
    out = oracle.scaled_residual(res, br.view(np.uint16), np.ones(1, F))
    assert np.array_equal(out, res + br.astype(F))
    # zero branch leaves the residual
    out = oracle.scaled_residual(res, np.zeros((N, C), np.uint16), sc)
    assert np.array_equal(out, res)
    # a scalar scale equals a constant per-channel scale
    a = oracle.scaled_residual(res, br.view(np.uint16), np.full(1, 0.37, F))
    b = oracle.scaled_residual(res, br.view(np.uint16), np.full(C, 0.37, F))
    assert np.array_equal(a, b)
    # two roundings: within 1.5 ulp of the binary64 value
    out = oracle.scaled_residual(res, br.view(np.uint16), sc)
    exact = res.astype(np.float64) + br.astype(np.float64) * sc.astype(np.float64)
    ulp = np.spacing(np.abs(out).astype(F)).astype(np.float64)
    prod_ulp = np.spacing(np.abs(br.astype(F) * sc)).astype(np.float64)
    assert np.all(np.abs(out - exact) <= 0.5 * ulp + 0.5 * prod_ulp + 1e-45)


def test_scaled_residual_has_no_contraction():
    """b s rounded to binary32 first: with res = -RN(b s) the sum is exactly 0, while a fused
    multiply-add would return the product's rounding error (2^-24 - 2^-33 here)."""
    b = np.float16(1 + 2.0 ** -10)
    s = F(1 + 2.0 ** -14 + 2.0 ** -23)
    p = F(np.float32(b) * s)
    assert float(p) - float(b) * float(s) != 0       # the product does round
    out = oracle.scaled_residual(np.array([[-p]], F), np.array([[b]], np.float16).view(np.uint16), np.array([s], F))
    assert out[0, 0] == 0.0
