"""Pins of the CPU oracle against facts fixed outside it (closed forms, brute force, library
routines, hand-derived values).  No GPU.  Each test names what it pins and why a plausible
mistake in the oracle (dropped term, wrong sign or index, transposed operand, other reduction
order, other rounding) fails it."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import twin

F = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


def identity_rows(n):
    one, zero = np.ones(n, F), np.zeros(n, F)
    return [one] * 3, [zero] * 3


# --------------------------------------------------------------------------- encoders

def _f32_sweep(stride=97, lo=0, hi=1 << 32):
    return np.arange(lo, hi, stride, dtype=np.uint64).astype(np.uint32).view(F)


def test_f16_encoder_matches_numpy_cast():
    """binary32 -> binary16 RNE: numpy's float16 cast is the library routine; a strided sweep of all
    bit patterns plus every binary16 value, midpoint and the overflow boundary."""
    x = _f32_sweep(97)
    halves = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (halves[:-1] + halves[1:]) / 2  # exact in fp64, exactly representable in fp32
    extra = np.concatenate([halves, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                            [65504, 65519.99, 65520, 65536, 1e30, np.inf]]).astype(F)
    x = np.concatenate([x, extra, -extra])
    got = oracle.encode(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all(got[nan] & 0x3FF)


def test_bf16_encoder_matches_torch_cast():
    x = np.concatenate([_f32_sweep(89), np.array([np.inf, -np.inf, 3.3895314e38, 3.40282e38], F)])
    got = oracle.encode(x, "bf16")
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x7F)


def test_decoders_roundtrip_every_code():
    c16 = np.arange(65536, dtype=np.uint16)
    f = oracle.decode(c16, "f16")
    assert np.array_equal(f[~np.isnan(f)], c16.view(np.float16).astype(F)[~np.isnan(f)])
    fin = (c16 & 0x7C00) != 0x7C00
    assert np.array_equal(oracle.encode(f[fin], "f16"), c16[fin])
    b = oracle.decode(c16, "bf16")
    fin = (c16 & 0x7F80) != 0x7F80
    assert np.array_equal(oracle.encode(b[fin], "bf16"), c16[fin])
    c8 = np.arange(256, dtype=np.uint8)
    e = oracle.decode(c8, "e4m3")
    ok = (c8 & 0x7F) != 0x7F
    assert np.array_equal(oracle.encode(e[ok], "e4m3"), c8[ok])
    assert np.isnan(e[~ok]).all()
    # the format's published constants: max finite 448, min normal 2^-6, min subnormal 2^-9
    assert oracle.decode(np.array([0x7E], np.uint8), "e4m3")[0] == 448.0
    assert oracle.decode(np.array([0x08], np.uint8), "e4m3")[0] == 2.0 ** -6
    assert oracle.decode(np.array([0x01], np.uint8), "e4m3")[0] == 2.0 ** -9


def _e4m3_probe_points():
    vals = twin._E4M3
    mids = (vals[:-1] + vals[1:]) / 2
    pts = [vals, mids]
    for p in (mids, vals):
        q = p.astype(F)
        for k in range(1, 4):
            pts.append(np.nextafter(q, np.float32(0)) if k == 1 else q)
            q = np.nextafter(q, np.float32(1e9))
            pts.append(q)
    pts.append(np.array([448, 449, 463.99997, 464, 464.00003, 470, 480, 1e10, np.inf, 2.0 ** -10,
                         2.0 ** -10 * 1.0000001, 2.0 ** -126, 1e-45], np.float64))
    return np.concatenate(pts).astype(F)


def test_e4m3_encoder_brute_force_and_torch():
    """OCP E4M3FN, RNE, saturating: against a brute-force nearest-code search (twin) on every
    midpoint and its neighbours plus a strided sweep of [-480, 480], and against torch's
    float8_e4m3fn cast wherever that cast does not overflow to NaN (|v| < 464)."""
    hi = int(np.float32(480.0).view(np.uint32)) + 1
    pos = _f32_sweep(13, 0, hi)
    x = np.concatenate([pos, -pos, _e4m3_probe_points(), -_e4m3_probe_points(), np.array([np.nan], F)])
    got = oracle.encode(x, "e4m3")
    assert np.array_equal(got, twin.e4m3_encode(x))
    m = np.abs(x) < 464
    ref = torch.from_numpy(x[m].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[m], ref)
    assert got[np.argmax(x == np.float32(470))] == 0x7E and oracle.encode(np.array([-np.inf], F), "e4m3")[0] == 0xFE


@pytest.mark.slow
def test_e4m3_encoder_exhaustive_positive_range():
    """Every binary32 in [0, 480]: oracle encoder == torch cast (|v| < 464) and saturation above."""
    hi = int(np.float32(480.0).view(np.uint32)) + 1
    step = 1 << 25
    for lo in range(0, hi, step):
        x = np.arange(lo, min(hi, lo + step), dtype=np.uint32).view(F)
        got = oracle.encode(x, "e4m3")
        m = x < 464
        ref = torch.from_numpy(x[m].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got[m], ref)
        assert np.all(got[~m] == 0x7E)


# --------------------------------------------------------------------------- the reduction tree

def _tree_probe(D, x):
    """Run one row through the oracle with unit weight, eps = 0 and identity rotation."""
    c, s = identity_rows(8 if D == 64 else 16)
    return oracle.norm_rope_row(np.asarray(x, F), np.ones(D, F), 0.0, 8 if D == 64 else 16, c, s)


def _expected_from_ss(x, ss, D):
    ms = F(ss) * F(1.0 / D)
    r = F(1.0) / np.sqrt(ms)
    return np.asarray(x, F) * r


@pytest.mark.parametrize("D,ones_from,ss_tree,ss_other", [
    # D = 64, x_0 = 4096 (x^2 = 2^24), x_1..31 = 0, x_32..63 = 1.  Halving tree, by hand:
    #   o=32: a_0 = 2^24 + 1 -> 2^24 (tie to even); a_1..31 = 1
    #   o=16: a_0 = 2^24 + 1 -> 2^24;  a_1..15 = 2
    #   o=8:  a_0 = 2^24 + 2;          a_1..7 = 4
    #   o=4:  a_0 = 2^24 + 6;          a_1..3 = 8
    #   o=2:  a_0 = 2^24 + 14;         a_1 = 16
    #   o=1:  a_0 = 2^24 + 30
    # An adjacent-pairs tree gives 2^24 + 32, a left-to-right sum 2^24.
    (64, 32, 16777216 + 30, 16777216 + 32),
    # D = 128, x_0 = 4096, x_1..63 = 0, x_64..127 = 1.  o=64 folds the ones onto a_0..63:
    #   a_0 = 2^24 + 1 -> 2^24, a_1..63 = 1; the 64-tree on [2^24, 1 x 63] then gives
    #   +2, +4, +8, +16, +32 -> 2^24 + 62.  Two separate 64-trees added last give 2^24 + 64.
    (128, 64, 16777216 + 62, 16777216 + 64),
])
def test_reduction_tree_order(D, ones_from, ss_tree, ss_other):
    x = np.zeros(D, F)
    x[0] = 4096.0
    x[ones_from:] = 1.0
    y = _tree_probe(D, x)
    want = _expected_from_ss(x, ss_tree, D)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    # the pin discriminates: the other orders give other bits
    assert not np.array_equal(_expected_from_ss(x, ss_other, D), want)
    assert not np.array_equal(_expected_from_ss(x, 16777216, D), want)


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("c", [1.5, -0.75, 3.0, 2.0 ** -7])
def test_constant_row_closed_form(D, c):
    """x_d = c: every tree sum is exact, ss = D c^2, ms = c^2, r = 1/sqrt(c^2 + eps) rounded twice,
    y_d = (c r) w_d.  r is also within 1 ulp of the fp64 value."""
    n = D // 8
    w = (1.0 + 0.1 * np.random.default_rng(1).standard_normal(D)).astype(F)
    cr, sr = identity_rows(n)
    eps = F(1e-6)
    y = oracle.norm_rope_row(np.full(D, c, F), w, float(eps), n, cr, sr)
    c32 = F(c)
    r = F(1.0) / np.sqrt(c32 * c32 + eps)
    want = (c32 * r) * w
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    r64 = 1.0 / np.sqrt(float(c) ** 2 + float(eps))
    assert abs(float(r) - r64) <= ulp32(r)


@pytest.mark.parametrize("D", [64, 128])
def test_one_hot_row(D):
    """x = c e_k: ss = c^2 exactly, ms = c^2 / D; y_k = (c r) w_k and every other y is a signed
    zero."""
    n = D // 8
    w = (1.0 + 0.1 * np.random.default_rng(2).standard_normal(D)).astype(F)
    cr, sr = identity_rows(n)
    for k in (0, 5, D - 1):
        x = np.zeros(D, F)
        x[k] = F(-2.5)
        y = oracle.norm_rope_row(x, w, 1e-6, n, cr, sr)
        r = F(1.0) / np.sqrt(F(6.25) * F(1.0 / D) + F(1e-6))
        assert y[k] == (F(-2.5) * r) * w[k]
        others = np.delete(y, k)
        assert np.all(others == 0)


def test_unit_weight_rms():
    """With w = 1 and no rotation, rms(y) = sqrt(ms / (ms + eps)) to a few fp32 ulps."""
    rng = np.random.default_rng(3)
    for D in (64, 128):
        n = D // 8
        cr, sr = identity_rows(n)
        for scale in (1e-3, 1.0, 30.0):
            x = (rng.standard_normal(D) * scale).astype(F)
            y = oracle.norm_rope_row(x, np.ones(D, F), 1e-6, n, cr, sr).astype(np.float64)
            ms = np.mean(x.astype(np.float64) ** 2)
            want = np.sqrt(ms / (ms + float(F(1e-6))))
            assert abs(np.sqrt(np.mean(y ** 2)) - want) <= 4 * 2.0 ** -23 * want


def test_rotation_preserves_pair_norm_and_position_zero_is_identity():
    wl = synth.workloads()["tile"]
    cos, sin = synth.rope_tables(wl.table_len, wl.n)
    rng = np.random.default_rng(4)
    n, D = wl.n, wl.D
    w = (1 + 0.1 * rng.standard_normal(D)).astype(F)
    cr0, sr0 = identity_rows(n)
    # position 0 of every axis is exactly (1, 0) in the tables
    assert np.all(cos[[0, 31, 47]] == 1) and np.all(sin[[0, 31, 47]] == 0)
    for _ in range(50):
        x = rng.standard_normal(D).astype(F)
        rows = [rng.integers(0, wl.table_len[0]), wl.table_len[0] + rng.integers(0, wl.table_len[1]),
                wl.table_len[0] + wl.table_len[1] + rng.integers(0, wl.table_len[2])]
        y0 = oracle.norm_rope_row(x, w, 1e-6, n, cr0, sr0)
        y0b = oracle.norm_rope_row(x, w, 1e-6, n, [cos[0]] * 3, [sin[0]] * 3)
        assert np.array_equal(y0b, y0)  # +0 / -0 may differ in sign only; == treats them equal
        y1 = oracle.norm_rope_row(x, w, 1e-6, n, [cos[r] for r in rows], [sin[r] for r in rows])
        assert np.array_equal(y1[6 * n:], y0[6 * n:])  # pass-through dims untouched
        a = np.hypot(y0[:6 * n:2].astype(np.float64), y0[1:6 * n:2].astype(np.float64))
        b = np.hypot(y1[:6 * n:2].astype(np.float64), y1[1:6 * n:2].astype(np.float64))
        assert np.all(np.abs(a - b) <= 4 * 2.0 ** -23 * a + 1e-30)


@pytest.mark.parametrize("D", [64, 128])
def test_pair_probe_returns_table_entry(D):
    """eps = 0, w = 1 and x = 8 e_{2p} (or 8 e_{2p+1}), plus, for D = 128, x_{127} = 8 in the
    pass-through part: the squares sum to D exactly, so r = 1 and y = x; the rotation then gives
    (8c, 8s) (or (-8s, 8c)) with (c, s) the table entry of axis p / n at frequency p mod n, and
    zeros elsewhere.  Pins the pair -> (axis, frequency) map and the rotation's signs."""
    n = D // 8
    rng = np.random.default_rng(5)
    crow = [rng.uniform(-1, 1, n).astype(F) for _ in range(3)]
    srow = [rng.uniform(-1, 1, n).astype(F) for _ in range(3)]
    for p in range(3 * n):
        for odd in (0, 1):
            x = np.zeros(D, F)
            x[2 * p + odd] = 8.0
            if D == 128:
                x[127] = 8.0
            y = oracle.norm_rope_row(x, np.ones(D, F), 0.0, n, crow, srow)
            c, s = crow[p // n][p % n], srow[p // n][p % n]
            want = np.zeros(D, F)
            if D == 128:
                want[127] = 8.0
            if odd == 0:
                want[2 * p], want[2 * p + 1] = F(8) * c, F(8) * s
            else:
                want[2 * p], want[2 * p + 1] = -(F(8) * s), F(8) * c
            assert np.array_equal(y, want), (p, odd)


def test_all_zero_tensor():
    wl = synth.Workload("z", 1, (2, 4, 4), 32, 2, 128, 16, "bf16", "zeros", 7, fp8=True)
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    am = oracle.qk_amax(sp, x, "bf16", wq, wk)
    assert np.all(am == 0)
    q, k, v, ds = oracle.qk_cast_e4m3(sp, x, "bf16", wq, wk, am)
    # y' is a signed zero (the sign follows w and the rotation), so every code is +-0
    assert np.all(ds == 1) and not (q & 0x7F).any() and not (k & 0x7F).any() and not v.any()


def test_descale():
    assert oracle.descale(0.0) == 1.0 and oracle.descale(-0.0) == 1.0
    assert oracle.descale(448.0) == 1.0
    for a in (1e-30, 0.37, 3.0, 1e30):
        assert oracle.descale(a) == F(F(a) / F(448.0))


# --------------------------------------------------------------------------- layout

def test_position_decode_brute_force():
    """Token i -> (t, h, w): the t-major, w-fastest enumeration of the grid, plus offsets, plus the
    axis base rows of the tables."""
    wl = synth.workloads()["tiles8"]
    sp = oracle.spec_from_workload(wl, T=31 * 20 * 20)
    off = synth.pos_offsets(wl)
    Pt, Ph, _ = wl.table_len
    for b in (0, 5):
        for i, (t, h, w) in enumerate(itertools.product(range(31), range(20), range(20))):
            if i % 7:
                continue
            rows = oracle.token_rows(sp, b, i)
            assert list(rows) == [t + off[b, 0], Pt + h + off[b, 1], Pt + Ph + w + off[b, 2]]


def test_offsets_and_tables_shape():
    wl = synth.workloads()["tiles8"]
    off = synth.pos_offsets(wl)
    assert off.shape == (8, 3) and np.all(off[:, 0] == 0)
    assert np.all((off[:, 1:] >= 0) & (off[:, 1:] < 64)) and len(np.unique(off[:, 1:])) > 4
    assert wl.table_len == (31, 83, 83)
    cos, sin = synth.rope_tables(wl.table_len, wl.n)
    assert cos.shape == (31 + 83 + 83, 8)
    # frequency ladder restarts on every axis: row 1 of each axis part is the same
    assert np.array_equal(cos[1], cos[31 + 1]) and np.array_equal(sin[1], sin[31 + 83 + 1])
    assert np.abs(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2 - 1).max() < 2e-7


def test_permute_index_map():
    """V out[b, h, i, :] is the input's V slice of head h at token i (numpy transpose is the
    reference); Q / K land at the same (b, h, i) as the per-token computation."""
    wl = synth.Workload("perm", 2, (2, 3, 5), 30, 3, 64, 8, "f16", "normal", 11, valid=[30, 17])
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    q, k, v = oracle.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk)
    ref_v = x.reshape(2, 30, 3, 3, 64)[:, :, 2].transpose(0, 2, 1, 3).copy()
    ref_v[1, :, 17:] = 0
    assert np.array_equal(v, ref_v)
    toks = np.array([0, 7, 29, 30 + 3, 30 + 16, 30 + 17, 30 + 29])
    tq, tk, tv, ty = oracle.qk_tokens(sp, x.reshape(60, -1)[toks], toks, "f16", wq, wk)
    for j, t in enumerate(toks):
        b, i = divmod(int(t), 30)
        assert np.array_equal(q[b, :, i], tq[j]) and np.array_equal(k[b, :, i], tk[j])
        assert np.array_equal(v[b, :, i], tv[j])
    # padded rows are zero, the valid ones are not
    assert not q[1, :, 17:].any() and q[1, :, :17].all()


def test_row_stride_and_batch_stride():
    """A padded row stride / batch stride reads the same values as the packed layout."""
    wl = synth.Workload("s", 2, (2, 2, 4), 16, 2, 64, 8, "f16", "normal", 12)
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    ref = oracle.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk)
    wide = np.zeros((2, 16 + 3, 384 + 40), np.uint16)
    wide[:, :16, :384] = x
    sp2 = oracle.spec_from_workload(wl, row_stride=424, batch_stride=19 * 424)
    got = oracle.qk_rmsnorm_rope_permute(sp2, wide, "f16", wq, wk)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)


# --------------------------------------------------------------------------- amax / cast

def test_amax_is_max_abs_and_head_order_free():
    wl = synth.Workload("am", 2, (3, 4, 5), 64, 3, 128, 16, "bf16", "normal", 13, valid=[60, 0])
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    am = oracle.qk_amax(sp, x, "bf16", wq, wk)
    q, k, _ = oracle.qk_rmsnorm_rope_permute(sp, x, "bf16", wq, wk, "f32", "f32")
    assert am[0] == np.abs(q).max() and am[1] == np.abs(k).max()
    # padded rows excluded: item 1 has none valid, item 0 stops at 60
    assert np.abs(q[0, :, :60]).max() == am[0] and not q[1].any()
    # permuting the heads of Q and K leaves the per-tensor maxima unchanged
    xp = x.reshape(2, 64, 3, 3, 128)[:, :, :, [2, 0, 1]].reshape(x.shape)
    assert np.array_equal(oracle.qk_amax(sp, xp, "bf16", wq, wk), am)


def test_cast_codes_are_encoded_quotients():
    wl = synth.Workload("cast", 1, (3, 4, 5), 64, 2, 128, 16, "bf16", "normal", 14, valid=[55])
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    am = oracle.qk_amax(sp, x, "bf16", wq, wk)
    q8, k8, v, ds = oracle.qk_cast_e4m3(sp, x, "bf16", wq, wk, am)
    q, k, v2 = oracle.qk_rmsnorm_rope_permute(sp, x, "bf16", wq, wk, "f32", "f32")
    assert ds[0] == am[0] / F(448) and ds[1] == am[1] / F(448)
    assert np.array_equal(q8, twin.e4m3_encode(q / ds[0])) and np.array_equal(k8, twin.e4m3_encode(k / ds[1]))
    assert np.array_equal(v, v2)
    # the amax element lands on +-448 (code 0x7E / 0xFE) up to the rounding of the descale
    dec = np.abs(twin.e4m3_decode(q8))
    assert dec.max() == 448.0
    # dequantised codes are within half an E4M3 step (relative 2^-4) of y' for normal codes
    qq = twin.e4m3_decode(q8).astype(np.float64) * ds[0]
    big = np.abs(q) / ds[0] >= 2.0 ** -6
    assert np.all(np.abs(qq[big] - q[big]) <= 2.0 ** -4 * np.abs(q[big]) + 1e-30)


# --------------------------------------------------------------------------- accuracy + twin

def test_accuracy_against_fp64():
    """The binary32 chain stays within a few ulps (of the row's scale) of an fp64 evaluation of
    the same formulas on the same fp32 inputs and tables."""
    wl = synth.workloads()["tile"]
    sp = oracle.spec_from_workload(wl)
    toks = np.arange(0, 7936, 37)
    rows = synth.qkv_host(wl, toks)
    wq, wk = synth.norm_weights(wl)
    _, _, _, y = oracle.qk_tokens(sp, rows, toks, "f16", wq, wk)
    H, D, n = wl.H, wl.D, wl.n
    x = twin.f16_decode(rows[:, :2 * H * D]).astype(np.float64).reshape(-1, 2, H, D)
    worst = 0.0
    for j, t in enumerate(toks):
        r3 = oracle.token_rows(sp, 0, int(t))
        c = np.concatenate([sp.cos[r] for r in r3]).astype(np.float64)
        s = np.concatenate([sp.sin[r] for r in r3]).astype(np.float64)
        for si, w in ((0, wq), (1, wk)):
            xs = x[j, si]
            r = 1.0 / np.sqrt(np.mean(xs ** 2, axis=1) + float(F(1e-6)))
            yy = xs * r[:, None] * w.astype(np.float64)[None, :]
            e, f = yy[:, 0:6 * n:2].copy(), yy[:, 1:6 * n:2].copy()
            yy[:, 0:6 * n:2] = e * c - f * s
            yy[:, 1:6 * n:2] = e * s + f * c
            scale = np.abs(yy).max(axis=1, keepdims=True)
            err = np.abs(y[j, si].astype(np.float64) - yy) / (scale * 2.0 ** -23)
            worst = max(worst, err.max())
    assert worst <= 8, worst


@pytest.mark.parametrize("name", ["tiny", "tile"])
def test_twin_matches_c_oracle_full(name):
    wl = synth.workloads()[name]
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    a = oracle.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk)
    b = twin.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk)
    for u, w in zip(a, b):
        assert np.array_equal(u.view(np.uint8), w.view(np.uint8))


def test_twin_matches_c_oracle_offsets_and_fp8():
    """Offsets (eight tiles, truncated T), bf16 + D = 128 + valid length + amax + cast."""
    wl = dataclasses_replace(synth.workloads()["tiles8"], T=600)
    sp = oracle.spec_from_workload(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    for u, w in zip(oracle.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk, "bf16", "f32"),
                    twin.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk, "bf16", "f32")):
        assert np.array_equal(u.view(np.uint8), w.view(np.uint8))
    wl4 = dataclasses_replace(synth.workloads()["fp8long"], T=700, valid=[611])
    sp4 = oracle.spec_from_workload(wl4)
    x4 = synth.qkv_host(wl4)
    wq, wk = synth.norm_weights(wl4)
    am = oracle.qk_amax(sp4, x4, "bf16", wq, wk)
    assert np.array_equal(am, twin.qk_amax(sp4, x4, "bf16", wq, wk))
    a = oracle.qk_cast_e4m3(sp4, x4, "bf16", wq, wk, am)
    b = twin.qk_rmsnorm_rope_permute(sp4, x4, "bf16", wq, wk, fp8_amax=am)
    for u, w in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(w).view(np.uint8))


def dataclasses_replace(wl, **kw):
    import dataclasses
    return dataclasses.replace(wl, **kw)


# --------------------------------------------------------------------------- stored values

def test_golden_tiny_outputs():
    """Digest of the oracle's outputs on the tiny workload, written by tests/golden/make_golden.py
    (which calls only the oracle); any change to the oracle's arithmetic shows up here."""
    import hashlib
    with open(os.path.join(GOLDEN, "oracle_digests.json")) as f:
        g = json.load(f)
    for name, ent in g.items():
        wl = synth.workloads()[ent["workload"]]
        sp = oracle.spec_from_workload(wl)
        x = synth.qkv_host(wl)
        assert hashlib.sha256(x.tobytes()).hexdigest() == ent["input_sha256"]
        wq, wk = synth.norm_weights(wl)
        outs = oracle.qk_rmsnorm_rope_permute(sp, x, wl.in_dtype, wq, wk, ent["q_dt"], ent["k_dt"])
        for key, arr in zip(("q", "k", "v"), outs):
            assert hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest() == ent[key + "_sha256"], (name, key)
