"""The seeded generator: host (numpy) and device-style (torch integer) paths give the same bits,
subsets regenerate exactly, and the workloads have the shapes and statistics they claim."""
import numpy as np
import torch

import synth


def test_numpy_and_torch_generators_agree():
    for dist, dt in (("normal", "f16"), ("x2_outliers", "f16"), ("normal", "bf16")):
        a = synth.values_np(1234, synth.S_QKV, np.arange(5000, 300000), dist, dt)
        b = synth.values_torch(1234, synth.S_QKV, 5000, 295000, dist, dt, "cpu", chunk=70000)
        assert np.array_equal(a, b.numpy().view(np.uint16))


def test_token_subset_regenerates_full_rows():
    wl = synth.workloads()["tiles8"]
    toks = np.array([0, 1, 12399, 12400, 8 * 12400 - 1])
    sub = synth.qkv_host(wl, toks)
    idx = toks[:, None] * wl.stride + np.arange(wl.stride)[None, :]
    full = synth.values_np(wl.seed, synth.S_QKV, idx.ravel(), wl.dist, wl.in_dtype).reshape(sub.shape)
    assert np.array_equal(sub, full)


def test_distributions():
    wl = synth.workloads()["tile"]
    x = synth.qkv_host(wl, np.arange(0, 7936, 5)).view(np.float16).astype(np.float64)
    frac_out = np.mean(np.abs(x) > 9.0)          # x2 values stay below 2 * 4.33
    assert 0.005 < frac_out < 0.012
    core = x[np.abs(x) <= 9.0]
    assert abs(core.std() - 2.0) < 0.05 and abs(core.mean()) < 0.02
    wl3 = synth.workloads()["latent"]
    y = synth.qkv_host(wl3, np.arange(0, 1000)).view(np.float16).astype(np.float64)
    assert abs(y.std() - 1.0) < 0.02
    wq, wk = synth.norm_weights(wl3)
    assert wq.dtype == np.float32 and abs(wq.mean() - 1) < 0.05 and 0.05 < wq.std() < 0.15
    assert not np.array_equal(wq, wk)


def test_workload_shapes():
    w = synth.workloads()
    assert [x.T for x in w.values()] == [32, 7936, 12400, 249984, 104448]
    for x in w.values():
        gt, gh, gw = x.grid
        assert x.valid_len.max() <= min(x.T, gt * gh * gw)
        assert x.D in (64, 128) and 6 * x.n <= x.D
    assert w["fp8long"].valid_len.tolist() == [104076]
    assert w["latent"].stride == 3072 and w["fp8long"].stride == 9216


def _decimal_cos_sin(x2, x, digits=40):
    """cos and sin from their Taylor series in decimal arithmetic, given x and x^2."""
    from decimal import Decimal, getcontext
    getcontext().prec = digits
    c, s = Decimal(0), Decimal(0)
    term_c, term_s = Decimal(1), Decimal(1)  # x^(2k) / (2k)!  and  x^(2k) / (2k + 1)!
    for k in range(30):
        c += term_c if k % 2 == 0 else -term_c
        s += term_s if k % 2 == 0 else -term_s
        term_c = term_c * x2 / ((2 * k + 1) * (2 * k + 2))
        term_s = term_s * x2 / ((2 * k + 2) * (2 * k + 3))
    return c, s * x


def test_rope_table_hand_values():
    """The frequency ladder theta^(-j/n), theta = 10000, pinned to values worked out by hand: with
    n = 8, j = 1 the frequency is 10^(-1/2), so at position p = 1 the angle x has x^2 = 1/10 exactly
    and cos, sin follow from their Taylor series in exact decimal arithmetic; at j = n - 1 = 7 the
    frequency is 10^(-7/2) (x^2 = 10^-7).  A ladder with theta^(-2j/n) or j/(n - 1) in the exponent
    gives other angles and fails here.  Rows: t part at row p, h part at P_t + p, w part at
    P_t + P_h + p (the ladder restarts on every axis)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 40
    tl = (31, 16, 16)
    cos, sin = synth.rope_tables(tl, 8)
    for j, x2 in ((1, Decimal(1) / 10), (7, Decimal(1) / 10 ** 7)):
        x = x2.sqrt()
        c, s = _decimal_cos_sin(x2, x)
        want_c, want_s = np.float32(float(c)), np.float32(float(s))
        for row in (1, tl[0] + 1, tl[0] + tl[1] + 1):
            assert cos[row, j] == want_c and sin[row, j] == want_s, (j, row, cos[row, j], want_c, sin[row, j], want_s)
    # a hand value that does not depend on the series: position 0 of every axis is the identity
    for row in (0, tl[0], tl[0] + tl[1]):
        assert np.all(cos[row] == 1.0) and np.all(sin[row] == 0.0)
    # and j = 0 is frequency 1: angle p itself
    assert cos[3, 0] == np.float32(np.cos(3.0)) and sin[tl[0] + 5, 0] == np.float32(np.sin(5.0))


def test_rope_table_ladder_closed_form():
    """Sampled entries of every workload's tables against cos / sin of p * theta^(-j/n) written out
    per entry with the math module (row base_a + p, column j), within one binary32 ulp (the libm
    argument and result may differ in the last binary64 bit from numpy's vector routines)."""
    import math
    rng = np.random.default_rng(5)
    for wl in synth.workloads().values():
        cos, sin = synth.rope_tables(wl.table_len, wl.n)
        base = (0, wl.table_len[0], wl.table_len[0] + wl.table_len[1])
        for a in range(3):
            for p in [0, 1, wl.table_len[a] - 1] + rng.integers(0, wl.table_len[a], 5).tolist():
                for j in [0, 1, wl.n - 1] + rng.integers(0, wl.n, 3).tolist():
                    ang = p * math.pow(10000.0, -j / wl.n)
                    for tab, f in ((cos, math.cos), (sin, math.sin)):
                        got, want = tab[base[a] + p, j], np.float32(f(ang))
                        assert abs(int(got.view(np.int32)) - int(want.view(np.int32))) <= 1, (wl.name, a, p, j)
