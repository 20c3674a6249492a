"""Pins of the oracle's static-scale FP8 cast and its saturation counter (TensorRT-LLM PR #21485:
the static scale table that replaces the dynamic amax pass, the E4M3 saturation log per tensor,
and the V cast of the per-tensor FP8 recipe).  No GPU.

Hand-built rows whose normalised values are exact (eps = 0, a one-hot row of 8 over D = 64 in a
dimension the rotation leaves alone, so 1/rms = 1 and y = 8 w) put elements exactly on and just
past the E4M3 range; V values are chosen on and off the E4M3 grid.  A wrong comparison (>= for >),
a count of NaN, a dropped V scale, counted padding, or codes not saturated fail one of them."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from oracle import twin

F = np.float32


def _spec(T=8, H=2, D=64, n=8, grid=(1, 2, 4), eps=0.0, valid=None, B=1):
    tl = grid
    cos, sin = synth.rope_tables(tl, n)
    return oracle.Spec(B, T, H, D, grid, n, tl, cos, sin, valid_len=valid, eps=eps)


def _f16(v):
    return np.asarray(v, np.float16).view(np.uint16)


def _one_hot_problem(sign_alt=True, dim=50, c=8.0, T=8, H=2, D=64):
    """qkv [1, T, 3 H D]: every Q and K row is c e_dim (sign alternating by token); V zero."""
    x = np.zeros((1, T, 3 * H * D), np.uint16)
    for i in range(T):
        s = -1.0 if (sign_alt and i % 2) else 1.0
        for h in range(2 * H):
            x[0, i, h * D + dim] = _f16(s * c)
    return x


def test_boundary_448_not_counted_just_past_counted():
    """y = 8 w exactly: Q at 448 (inside the range: code 0x7E, not counted), K one binary32 ulp past
    448 (counted, saturated to 0x7E), both with descale 1; then the same with descale 2 at 896."""
    sp = _spec()
    x = _one_hot_problem()
    for ds, wq50 in ((1.0, 56.0), (2.0, 112.0)):
        wq = np.ones(64, F); wk = np.ones(64, F)
        wq[50] = wq50
        wk[50] = np.nextafter(F(wq50), F(1e9))
        q, k, v, sat = oracle.qk_cast_e4m3_static(sp, x, "f16", wq, wk, [ds, ds])
        rows = sp.T * sp.H
        assert sat.tolist() == [0, rows, 0]
        sign = np.array([0x00, 0x80] * 4, np.uint8)[None, None, :]
        assert np.array_equal(q[..., 50], np.broadcast_to(sign | 0x7E, q[..., 50].shape))
        assert np.array_equal(k[..., 50], np.broadcast_to(sign | 0x7E, k[..., 50].shape))
        others = np.delete(np.arange(64), 50)
        # zeros stay zeros (a rotated zero pair can be -0 where cos < 0: code 0x80)
        assert not (q[..., others] & 0x7F).any() and not (k[..., others] & 0x7F).any()
        assert np.array_equal(v, np.zeros_like(v))                  # V copied (zeros)


def test_v_codes_and_counts():
    """V cast with descale 1 and 0.5: codes of values on the E4M3 grid, at the range end, past it
    (counted, saturated) and a tie at half the smallest subnormal (rounds to the even code 0)."""
    sp = _spec(T=8, H=2)
    x = np.zeros((1, 8, 3 * 2 * 64), np.uint16)
    vals = np.array([448, 450, -500, 464, 1.5, -0.0, 2.0 ** -10, 0.25], np.float64)
    want1 = [0x7E, 0x7E, 0xFE, 0x7E, 0x3C, 0x80, 0x00, 0x28]
    x[0, :, 2 * 2 * 64:2 * 2 * 64 + 8] = _f16(vals)  # V head 0, dims 0..7 of every token
    w = np.ones(64, F)
    q, k, v, sat = oracle.qk_cast_e4m3_static(sp, x, "f16", w, w, [1.0, 1.0, 1.0], v_fp8=True)
    assert v.dtype == np.uint8
    assert np.array_equal(v[0, 0, :, :8], np.tile(np.array(want1, np.uint8), (8, 1)))
    assert not v[0, 1].any() and not v[0, 0, :, 8:].any()
    assert sat.tolist() == [0, 0, 3 * 8]
    # descale 0.5: v = 224 is exactly 448 after scaling, 225 is past it
    x2 = np.zeros_like(x)
    x2[0, :, 256:259] = _f16([224, 225, -112])
    _, _, v2, sat2 = oracle.qk_cast_e4m3_static(sp, x2, "f16", w, w, [1.0, 1.0, 0.5], v_fp8=True)
    assert v2[0, 0, 0, :3].tolist() == [0x7E, 0x7E, 0xF6]  # -224 = -(1.75 * 2^7): E = 14, m = 6
    assert sat2.tolist() == [0, 0, 8]


def test_tiny_descale_saturates_every_valid_element_and_skips_padding():
    """descale 1e-30 on random data: every valid nonzero element is past the range, so the count is
    the number of nonzero valid elements and every code is +-448; padded tokens stay 0, uncounted."""
    wl = dataclasses.replace(synth.workloads()["fp8long"], T=40, valid=[29], grid=(1, 5, 8))
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    q, k, v, sat = oracle.qk_cast_e4m3_static(sp, x, "bf16", wq, wk, [1e-30] * 3, v_fp8=True)
    H, D, vl = wl.H, wl.D, 29
    y = twin.token_y(sp, x[0, :vl], np.arange(vl), "bf16", wq, wk)
    vin = x[0, :vl, 2 * H * D:]
    assert sat.tolist() == [np.count_nonzero(y[:, 0]), np.count_nonzero(y[:, 1]),
                            np.count_nonzero(vin & 0x7FFF)]
    assert sat[0] > 0.99 * vl * H * D
    for codes in (q, k, v):
        valid = codes[0, :, :vl]
        nz = valid & 0x7F
        assert np.all((nz == 0x7E) | (nz == 0))
        assert not codes[0, :, vl:].any()


def test_huge_descale_gives_zero_codes():
    wl = dataclasses.replace(synth.workloads()["tiny"])
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    q, k, v, sat = oracle.qk_cast_e4m3_static(sp, x, "f16", wq, wk, [2.0 ** 100] * 3, v_fp8=True)
    assert sat.tolist() == [0, 0, 0]
    for codes in (q, k, v):
        assert np.all((codes & 0x7F) == 0)


def test_descale_guard_reads_nonpositive_and_nan_as_one():
    wl = synth.workloads()["tiny"]
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    ref = oracle.qk_cast_e4m3_static(sp, x, "f16", wq, wk, [1.0, 1.0, 1.0], v_fp8=True)
    for bad in (0.0, -0.0, -3.0, float("nan"), float("-inf")):
        got = oracle.qk_cast_e4m3_static(sp, x, "f16", wq, wk, [bad, bad, bad], v_fp8=True)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)
    assert oracle.static_descale(float("inf")) == float("inf")
    assert oracle.static_descale(0.25) == 0.25


def test_static_at_dynamic_descale_equals_dynamic_cast():
    """With the descales the dynamic pass would use, the static cast writes the same codes and V."""
    wl = dataclasses.replace(synth.workloads()["fp8long"], T=300, valid=[250], grid=(1, 10, 30))
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    am = oracle.qk_amax(sp, x, "bf16", wq, wk)
    q, k, v, ds = oracle.qk_cast_e4m3(sp, x, "bf16", wq, wk, am)
    q2, k2, v2, sat = oracle.qk_cast_e4m3_static(sp, x, "bf16", wq, wk, ds)
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    assert sat[2] == 0
    # only elements whose quotient rounds just above 448 can count at the amax descale
    assert sat[0] <= 2 and sat[1] <= 2


def test_counts_fall_as_the_descale_grows():
    wl = dataclasses.replace(synth.workloads()["tile"], T=256, grid=(1, 16, 16))
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    am = oracle.qk_amax(sp, x, "f16", wq, wk)
    prev = None
    for f in (0.05, 0.1, 0.2, 0.4, 0.8, 1.0):
        ds = [am[0] * f / 448, am[1] * f / 448, 0.02 * f]
        sat = oracle.qk_cast_e4m3_static(sp, x, "f16", wq, wk, ds, v_fp8=True)[3]
        if prev is not None:
            assert np.all(sat <= prev)
        prev = sat
    assert prev[0] <= 2 and prev[1] <= 2


@pytest.mark.parametrize("v_fp8", [False, True])
def test_twin_matches_static_cast(v_fp8):
    """The numpy twin (independent encoder and reduction code) agrees on codes and counts with
    descales that clip roughly the top 1-5 % of each tensor; bf16, D = 128, offsets, padding."""
    wl = dataclasses.replace(synth.workloads()["fp8long"], T=500, valid=[433], grid=(1, 20, 25))
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    ds = [0.0045, 0.005, 0.0046]  # clip at about 2 standard deviations
    a = oracle.qk_cast_e4m3_static(sp, x, "bf16", wq, wk, ds, v_fp8=v_fp8)
    b = twin.qk_cast_static(sp, x, "bf16", wq, wk, ds, v_fp8=v_fp8)
    for u, w in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(w).view(np.uint8))
    n = 433 * wl.H * wl.D
    assert 0.005 * n < a[3][0] < 0.2 * n and 0.005 * n < a[3][1] < 0.2 * n
    if v_fp8:
        assert 0.005 * n < a[3][2] < 0.2 * n
    else:
        assert a[3][2] == 0


def test_token_subset_matches_full_static_cast():
    wl = dataclasses.replace(synth.workloads()["fp8long"], T=200, valid=[150], grid=(1, 10, 20))
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    ds = [0.012, 0.011, 0.0055]
    q, k, v, sat = oracle.qk_cast_e4m3_static(sp, x, "bf16", wq, wk, ds, v_fp8=True)
    toks = np.arange(200)
    s2 = np.zeros(3, np.uint64)
    tq, tk, tv, _ = oracle.qk_tokens(sp, x[0], toks, "bf16", wq, wk, fp8=True, descale=ds, v_fp8=True, sat=s2)
    assert np.array_equal(tq, q[0].transpose(1, 0, 2)) and np.array_equal(tk, k[0].transpose(1, 0, 2))
    assert np.array_equal(tv, v[0].transpose(1, 0, 2))
    assert np.array_equal(s2, sat)
