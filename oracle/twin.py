"""Vectorised numpy re-implementation of the oracle (test infrastructure only).

Written separately from h3ref.c so that the two can be checked against each other: numpy binary32
arithmetic (one rounding per ufunc, never fused), the halving reduction tree as explicit slice adds
(never np.sum), and encoders built differently from the C ones (numpy's own float16 cast, an
integer bfloat16 rounding, and an E4M3 nearest-value search over the code table).
"""
from __future__ import annotations

import numpy as np

F = np.float32


def f16_decode(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(F)


def bf16_decode(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(F)


def f16_encode(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, F).astype(np.float16).view(np.uint16)


def bf16_encode(x):
    u = np.asarray(x, F).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


def _e4m3_table():
    vals = []
    for c in range(0x7F):  # finite non-negative codes 0x00..0x7E
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.array(vals, dtype=np.float64)


_E4M3 = _e4m3_table()


def e4m3_encode(x):
    """Nearest finite E4M3FN value (ties to the even code), saturating at 448; NaN -> 0x7F|sign."""
    x = np.asarray(x, F)
    a = np.abs(x.astype(np.float64))
    sign = (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 1, len(_E4M3) - 1)
    lo = hi - 1
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a > 448.0, np.uint8(0x7E), code)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def e4m3_decode(c):
    c = np.asarray(c, np.uint8)
    mag = np.append(_E4M3, np.nan)[c & 0x7F]
    return np.where(c & 0x80, -mag, mag).astype(F)


def decode_in(bits, dt):
    return bf16_decode(bits) if dt == "bf16" else f16_decode(bits)


def encode_out(y, dt):
    if dt == "f32":
        return np.asarray(y, F)
    if dt == "f16":
        return f16_encode(y)
    if dt == "bf16":
        return bf16_encode(y)
    return e4m3_encode(y)


def norm_rope(x, w, eps, n, cos_rows, sin_rows):
    """x [R, D] f32; cos_rows/sin_rows [R, 3n] (t part, then h, then w).  Returns y' [R, D]."""
    x = np.asarray(x, F)
    D = x.shape[1]
    a = x * x
    o = D // 2
    while o >= 1:
        a = a[:, :o] + a[:, o:2 * o]
        o //= 2
    ss = a[:, 0]
    ms = ss * F(1.0 / D)
    v = ms + F(eps)
    r = F(1.0) / np.sqrt(v)
    y = (x * r[:, None]) * np.asarray(w, F)[None, :]
    e, f = y[:, 0:6 * n:2].copy(), y[:, 1:6 * n:2].copy()
    y[:, 0:6 * n:2] = e * cos_rows - f * sin_rows
    y[:, 1:6 * n:2] = e * sin_rows + f * cos_rows
    return y


def _positions(spec, b, i):
    gt, gh, gw = spec.grid
    off = spec.off[b]                                          # [n_tok, 3]
    return np.stack([i // (gh * gw) + off[:, 0], (i // gw) % gh + off[:, 1], i % gw + off[:, 2]], axis=-1)


def _table_rows(spec, pos):
    base = np.array([0, spec.table_len[0], spec.table_len[0] + spec.table_len[1]])
    assert np.all(pos >= 0) and np.all(pos < np.array(spec.table_len))
    return pos + base


def token_y(spec, rows_bits, tokens, in_dt, w_q, w_k):
    """y' [n_tok, 2, H, D] for the valid tokens among `tokens` (rows_bits [n_tok, row_stride])."""
    H, D, n = spec.H, spec.D, spec.n
    tokens = np.asarray(tokens, np.int64)
    b, i = tokens // spec.T, tokens % spec.T
    rows = _table_rows(spec, _positions(spec, b, i))          # [n_tok, 3]
    cs = np.concatenate([spec.cos[rows[:, a]] for a in range(3)], axis=1)  # [n_tok, 3n]
    sn = np.concatenate([spec.sin[rows[:, a]] for a in range(3)], axis=1)
    x = decode_in(rows_bits[:, :2 * H * D], in_dt).reshape(-1, 2, H, D)
    out = np.empty(x.shape, F)
    for s, w in ((0, w_q), (1, w_k)):
        xs = x[:, s].reshape(-1, D)
        c = np.repeat(cs, H, axis=0)
        si = np.repeat(sn, H, axis=0)
        out[:, s] = norm_rope(xs, w, spec.eps, n, c, si).reshape(-1, H, D)
    return out


def qk_rmsnorm_rope_permute(spec, qkv_bits, in_dt, w_q, w_k, q_dt="f32", k_dt="f16", fp8_amax=None):
    """Whole-problem outputs, head-major [B, H, T, D].  With fp8_amax, Q/K are E4M3 codes of
    y' / descale and the descales are returned as a 4th value."""
    B, T, H, D = spec.B, spec.T, spec.H, spec.D
    flat = np.asarray(qkv_bits, np.uint16).reshape(-1)
    q = np.zeros((B, H, T, D), np.uint8 if fp8_amax is not None else {"f32": F}.get(q_dt, np.uint16))
    k = np.zeros((B, H, T, D), np.uint8 if fp8_amax is not None else {"f32": F}.get(k_dt, np.uint16))
    v = np.zeros((B, H, T, D), np.uint16)
    ds = None
    if fp8_amax is not None:
        am = np.asarray(fp8_amax, F)
        ds = np.where(am > 0, am / F(448.0), F(1.0)).astype(F)
    for b in range(B):
        vl = int(spec.vl[b])
        if vl == 0:
            continue
        i = np.arange(vl)
        start = b * spec.batch_stride + i[:, None] * spec.row_stride
        rows_bits = flat[start + np.arange(3 * H * D)[None, :]]
        y = token_y(spec, rows_bits, b * T + i, in_dt, w_q, w_k)   # [vl, 2, H, D]
        if ds is not None:
            q[b, :, :vl] = e4m3_encode(y[:, 0] / ds[0]).transpose(1, 0, 2)
            k[b, :, :vl] = e4m3_encode(y[:, 1] / ds[1]).transpose(1, 0, 2)
        else:
            q[b, :, :vl] = encode_out(y[:, 0], q_dt).transpose(1, 0, 2)
            k[b, :, :vl] = encode_out(y[:, 1], k_dt).transpose(1, 0, 2)
        v[b, :, :vl] = rows_bits[:, 2 * H * D:].reshape(vl, H, D).transpose(1, 0, 2)
    if ds is not None:
        return q, k, v, ds
    return q, k, v


def qk_amax(spec, qkv_bits, in_dt, w_q, w_k):
    B, T, H, D = spec.B, spec.T, spec.H, spec.D
    flat = np.asarray(qkv_bits, np.uint16).reshape(-1)
    am = np.zeros(2, F)
    for b in range(B):
        vl = int(spec.vl[b])
        if vl == 0:
            continue
        i = np.arange(vl)
        start = b * spec.batch_stride + i[:, None] * spec.row_stride
        y = token_y(spec, flat[start + np.arange(3 * H * D)[None, :]], b * T + i, in_dt, w_q, w_k)
        for s in range(2):
            m = np.abs(y[:, s])
            am[s] = np.nan if (np.isnan(m).any() or np.isnan(am[s])) else max(am[s], m.max())
    return am


def qk_cast_static(spec, qkv_bits, in_dt, w_q, w_k, descale, v_fp8=False):
    """FP8 cast with caller descales: (q, k, v, sat).  A descale that is not > 0 counts as 1; V is
    cast with descale[2] when v_fp8, else copied; sat [3] counts |quotient| > 448 per tensor."""
    B, T, H, D = spec.B, spec.T, spec.H, spec.D
    flat = np.asarray(qkv_bits, np.uint16).reshape(-1)
    d = np.ones(3, F)
    given = np.asarray(descale, F).ravel()
    d[:given.size] = given
    ds = np.where(d > 0, d, F(1.0)).astype(F)
    if not v_fp8:
        ds[2] = F(1.0)
    q = np.zeros((B, H, T, D), np.uint8)
    k = np.zeros((B, H, T, D), np.uint8)
    v = np.zeros((B, H, T, D), np.uint8 if v_fp8 else np.uint16)
    sat = np.zeros(3, np.uint64)
    for b in range(B):
        vl = int(spec.vl[b])
        if vl == 0:
            continue
        i = np.arange(vl)
        start = b * spec.batch_stride + i[:, None] * spec.row_stride
        rows_bits = flat[start + np.arange(3 * H * D)[None, :]]
        y = token_y(spec, rows_bits, b * T + i, in_dt, w_q, w_k)   # [vl, 2, H, D]
        vb = rows_bits[:, 2 * H * D:].reshape(vl, H, D)
        parts = [(0, y[:, 0], q), (1, y[:, 1], k)]
        if v_fp8:
            parts.append((2, decode_in(vb, in_dt), v))
        else:
            v[b, :, :vl] = vb.transpose(1, 0, 2)
        for s, val, out in parts:
            with np.errstate(over="ignore", invalid="ignore"):
                quo = (val / ds[s]).astype(F)
                sat[s] += np.uint64(np.count_nonzero(np.abs(quo) > F(448.0)))
            out[b, :, :vl] = e4m3_encode(quo).transpose(1, 0, 2)
    return q, k, v, sat
