"""Pins of the oracle's V cast (third per-tensor scale) and of its per-tensor passes for one
separately projected [B, S, H, D] tensor (TensorRT-LLM PR #21485: the per-tensor FP8 recipe that
casts Q, K and V; norm_rope_tensor; the split launch mode over the packed QKV).  No GPU.

The per-tensor passes run on Q, K and V slices of a packed QKV must reproduce the fused pass
(pinned on its own); V's amax and codes are checked against brute force with numpy's own float16
decoding and the twin's table-search E4M3 encoder; the [B, T, H, D] layout against a transpose;
the identity path against numpy and torch casts."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import twin

F = np.float32


def W(name, **kw):
    return dataclasses.replace(synth.workloads()[name], **kw)


def _problem(wl):
    sp = oracle.spec_from_workload(wl, batch_stride=wl.T * wl.stride)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    return sp, x, wq, wk


def _tensor_spec(sp, row_stride=None, batch_stride=None):
    """The same problem seen as one tensor of sp.H heads with the given token stride."""
    rs = sp.row_stride if row_stride is None else row_stride
    return oracle.Spec(sp.B, sp.T, sp.H, sp.D, sp.grid, sp.n, sp.table_len, sp.cos, sp.sin, pos_offset=sp.off,
                       valid_len=sp.vl, eps=sp.eps, row_stride=rs,
                       batch_stride=sp.batch_stride if batch_stride is None else batch_stride)


CASES = [
    ("tiles8", dict(B=2, T=120, valid=[120, 77])),
    ("fp8long", dict(T=90, valid=[83], grid=(1, 9, 10))),
]


@pytest.mark.parametrize("name,kw", CASES)
def test_tensor_passes_on_packed_slices_match_fused(name, kw):
    wl = W(name, **kw)
    sp, x, wq, wk = _problem(wl)
    H, D = wl.H, wl.D
    flat = x.reshape(-1)
    q, k, v = oracle.qk_rmsnorm_rope_permute(sp, x, wl.in_dtype, wq, wk, "f32", "bf16")
    ts = _tensor_spec(sp)  # token stride 3 H D: the packed QKV's rows
    tq = oracle.tensor_norm_rope(ts, flat, wl.in_dtype, wq, "f32")
    tk = oracle.tensor_norm_rope(ts, flat[H * D:], wl.in_dtype, wk, "bf16")
    tv = oracle.tensor_norm_rope(ts, flat[2 * H * D:], wl.in_dtype, None, wl.in_dtype)
    assert np.array_equal(tq.view(np.uint32), q.view(np.uint32))
    assert np.array_equal(tk, k) and np.array_equal(tv, v)
    # [B, T, H, D] is the transpose of [B, H, T, D]
    tq1 = oracle.tensor_norm_rope(ts, flat, wl.in_dtype, wq, "f32", layout=1)
    assert np.array_equal(tq1.view(np.uint32), tq.transpose(0, 2, 1, 3).view(np.uint32))
    # amax of the Q slice is the fused pass's Q amax
    am = oracle.qk_amax(sp, x, wl.in_dtype, wq, wk)
    assert oracle.tensor_amax(ts, flat, wl.in_dtype, wq) == am[0]
    assert oracle.tensor_amax(ts, flat[H * D:], wl.in_dtype, wk) == am[1]


def test_standalone_tensor_equals_packed_slice():
    """A compact [B, S, H, D] tensor (token stride H D) gives the outputs of the same values read
    out of a packed QKV with token stride 3 H D."""
    wl = W("tiles8", B=2, T=64, valid=[64, 50])
    sp, x, wq, wk = _problem(wl)
    H, D = wl.H, wl.D
    kslice = np.ascontiguousarray(x[:, :, H * D:2 * H * D])           # [B, T, H D]
    ts_packed = _tensor_spec(sp)
    ts_compact = _tensor_spec(sp, row_stride=H * D, batch_stride=wl.T * H * D)
    a = oracle.tensor_norm_rope(ts_packed, x.reshape(-1)[H * D:], "f16", wk, "f16", layout=1)
    b = oracle.tensor_norm_rope(ts_compact, kslice, "f16", wk, "f16", layout=1)
    assert np.array_equal(a, b)


def test_identity_path_is_a_plain_conversion():
    wl = W("tiles8", B=1, T=40, valid=[33])
    sp, x, wq, wk = _problem(wl)
    H, D = wl.H, wl.D
    ts = _tensor_spec(sp)
    vbits = x[0, :, 2 * H * D:].reshape(40, H, D)
    vf = oracle.tensor_norm_rope(ts, x.reshape(-1)[2 * H * D:], "f16", None, "f32", layout=1)
    ref = vbits.view(np.float16).astype(F)
    ref[33:] = 0
    assert np.array_equal(vf[0].view(np.uint32), ref.view(np.uint32))
    vb = oracle.tensor_norm_rope(ts, x.reshape(-1)[2 * H * D:], "f16", None, "bf16", layout=1)
    refb = torch.from_numpy(vbits.view(np.float16).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    refb[33:] = 0
    assert np.array_equal(vb[0], refb)


@pytest.mark.parametrize("name,kw", CASES)
def test_v_amax_and_codes_brute_force(name, kw):
    wl = W(name, **kw)
    sp, x, wq, wk = _problem(wl)
    H, D = wl.H, wl.D
    am = oracle.qkv_amax(sp, x, wl.in_dtype, wq, wk)
    assert np.array_equal(am[:2], oracle.qk_amax(sp, x, wl.in_dtype, wq, wk))
    vals = []
    for b in range(wl.B):
        vl = int(wl.valid_len[b])
        vals.append(twin.decode_in(x[b, :vl, 2 * H * D:3 * H * D], wl.in_dtype).ravel())
    assert am[2] == np.max(np.abs(np.concatenate(vals)))
    q, k, v, ds = oracle.qkv_cast_e4m3(sp, x, wl.in_dtype, wq, wk, am)
    q2, k2, _, ds2 = oracle.qk_cast_e4m3(sp, x, wl.in_dtype, wq, wk, am[:2])
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(ds[:2], ds2)
    assert ds[2] == np.float32(am[2]) / np.float32(448.0)
    for b in range(wl.B):
        vl = int(wl.valid_len[b])
        vv = twin.decode_in(x[b, :vl, 2 * H * D:3 * H * D], wl.in_dtype).reshape(vl, H, D)
        want = twin.e4m3_encode((vv / ds[2]).astype(F)).transpose(1, 0, 2)
        assert np.array_equal(v[b, :, :vl], want)
        assert not v[b, :, vl:].any()


def _put(x, wl, b, i, e, val):
    """Write val (binary32) into element e of token i of item b, encoded in the input dtype."""
    enc = (np.array([val], np.float16).view(np.uint16) if wl.in_dtype == "f16"
           else oracle.encode(np.array([val], F), "bf16"))
    x[b, i, e] = enc[0]


@pytest.mark.parametrize("in_dtype", ["f16", "bf16"])
def test_amax_planted_maxima_and_nan(in_dtype):
    """Planted values decide each amax: V's maximum |v| is a planted 7.5 (K holds a planted 6.0,
    so reading the wrong heads shows), a planted value in a padding row is ignored, and a NaN in
    one Q row (or one V element) makes that tensor's amax NaN while the others stay finite."""
    wl = W("tiles8", B=2, T=40, valid=[40, 21], grid=(1, 5, 8), in_dtype=in_dtype)
    sp, x, wq, wk = _problem(wl)
    x = x.copy()
    H, D = wl.H, wl.D
    _put(x, wl, 1, 5, 2 * H * D + 3 * D + 17, -7.5)   # V, item 1, valid token
    _put(x, wl, 0, 9, H * D + 2 * D + 1, 6.0)         # K
    _put(x, wl, 1, 30, 2 * H * D + 5, 9.0)            # V in a padding row of item 1
    am = oracle.qkv_amax(sp, x, in_dtype, wq, wk)
    assert am[2] == np.float32(7.5)
    assert np.isfinite(am).all()
    xq = x.copy()
    _put(xq, wl, 0, 3, 4 * D + 2, np.nan)              # one Q element: its row's y' is all NaN
    aq = oracle.qkv_amax(sp, xq, in_dtype, wq, wk)
    assert np.isnan(aq[0]) and aq[1] == am[1] and aq[2] == am[2]
    assert np.isnan(oracle.qk_amax(sp, xq, in_dtype, wq, wk)[0])
    xv = x.copy()
    _put(xv, wl, 0, 0, 2 * H * D, np.nan)
    av = oracle.qkv_amax(sp, xv, in_dtype, wq, wk)
    assert np.isnan(av[2]) and av[0] == am[0] and av[1] == am[1]
    xp = x.copy()
    _put(xp, wl, 1, 35, 0, np.nan)                      # NaN in a padding row: ignored
    assert np.array_equal(oracle.qkv_amax(sp, xp, in_dtype, wq, wk), am)
    ts = _tensor_spec(sp)
    assert np.isnan(oracle.tensor_amax(ts, xq.reshape(-1), in_dtype, wq))


def test_tensor_cast_against_its_own_f32_output():
    """Codes of the per-tensor cast are the twin's E4M3 encoding of (f32 output / descale), with
    the descale closed form amax / 448, the static guard, and the clip count from numpy."""
    wl = W("fp8long", T=90, valid=[83], grid=(1, 9, 10))
    sp, x, wq, wk = _problem(wl)
    ts = _tensor_spec(sp)
    flat = x.reshape(-1)
    y = oracle.tensor_norm_rope(ts, flat, "bf16", wq, "f32", layout=1)
    am = oracle.tensor_amax(ts, flat, "bf16", wq)
    assert am == np.max(np.abs(y))
    codes, ds, sat = oracle.tensor_cast_e4m3(ts, flat, "bf16", wq, float(am), False, layout=1)
    assert ds == np.float32(am) / np.float32(448.0)
    assert np.array_equal(codes, twin.e4m3_encode((y / ds).astype(F)))
    assert sat <= 2
    for d in (0.004, 0.0, -1.0, float("nan")):
        c2, ds2, sat2 = oracle.tensor_cast_e4m3(ts, flat, "bf16", wq, d, True, layout=1)
        use = np.float32(d) if d > 0 else np.float32(1.0)
        assert ds2 == use
        qt = (y / use).astype(F)
        assert np.array_equal(c2, twin.e4m3_encode(qt))
        valid = np.zeros(y.shape, bool)
        valid[:, :83] = True
        assert sat2 == int(np.count_nonzero(np.abs(qt[valid]) > 448.0))
    assert oracle.tensor_cast_e4m3(ts, flat, "bf16", wq, 0.004, True)[2] > 0


def test_empty_tensor_amax_is_zero_and_descale_one():
    wl = W("fp8long", T=24, valid=[0], grid=(1, 4, 6))
    sp, x, wq, wk = _problem(wl)
    ts = _tensor_spec(sp)
    assert oracle.tensor_amax(ts, x.reshape(-1), "bf16", wq) == 0.0
    codes, ds, sat = oracle.tensor_cast_e4m3(ts, x.reshape(-1), "bf16", wq, 0.0, False)
    assert ds == 1.0 and sat == 0 and not codes.any()
