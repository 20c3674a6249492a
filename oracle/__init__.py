"""CPU oracle for the fused QK RMSNorm + 3-axis RoPE + head-major permute, amax and E4M3 cast.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's CPU-baseline leg are the
only users.  The product path never imports this package.  The arithmetic lives in the plain C
file h3ref.c (binary32, one rounding per written operation, no contraction), built with gcc into
liboracle_h3ref.so beside it; this module only marshals numpy arrays to it.  `twin.py` is a
separate numpy re-implementation used to cross-check the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "h3ref.c")
# H3REF_LIB names a prebuilt substitute library (the mutation test loads deliberately broken
# builds of h3ref.c through it); it is used as given and never rebuilt.
LIB_OVERRIDE = os.environ.get("H3REF_LIB")
LIB = LIB_OVERRIDE or os.path.join(HERE, "liboracle_h3ref.so")

DT = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
NP_DT = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(force: bool = True, src: str = SRC, out: str = None) -> str:
    """Compile the oracle with gcc (plain x86-64 SSE binary32: no FMA, no FTZ).  `src` / `out`
    build another copy of the source elsewhere (the mutation test)."""
    out = out or os.path.join(HERE, "liboracle_h3ref.so")
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not LIB_OVERRIDE and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.POINTER(Problem)
        vp, fp = ctypes.c_void_p, ctypes.c_void_p
        i64 = ctypes.c_int64
        L.h3ref_qk_rmsnorm_rope_permute.argtypes = [P, vp, ctypes.c_int, fp, fp, vp, ctypes.c_int, vp, ctypes.c_int, vp]
        L.h3ref_qk_amax.argtypes = [P, vp, ctypes.c_int, fp, fp, fp]
        L.h3ref_qk_cast_e4m3.argtypes = [P, vp, ctypes.c_int, fp, fp, fp, vp, vp, vp, fp]
        L.h3ref_qk_tokens.argtypes = [P, vp, ctypes.c_int, fp, fp, vp, i64, ctypes.c_int, fp, vp,
                                      ctypes.c_int, vp, ctypes.c_int, vp, fp]
        L.h3ref_qk_cast_e4m3_static.argtypes = [P, vp, ctypes.c_int, fp, fp, fp, ctypes.c_int, vp, vp, vp, vp]
        L.h3ref_qk_tokens_ex.argtypes = [P, vp, ctypes.c_int, fp, fp, vp, i64, ctypes.c_int, fp, ctypes.c_int,
                                         vp, ctypes.c_int, vp, ctypes.c_int, vp, fp, vp]
        L.h3ref_qkv_amax.argtypes = [P, vp, ctypes.c_int, fp, fp, fp]
        L.h3ref_qkv_cast_e4m3.argtypes = [P, vp, ctypes.c_int, fp, fp, fp, vp, vp, vp, fp]
        L.h3ref_tensor_norm_rope.argtypes = [P, vp, ctypes.c_int, fp, vp, ctypes.c_int, ctypes.c_int]
        L.h3ref_tensor_amax.argtypes = [P, vp, ctypes.c_int, fp, fp]
        L.h3ref_tensor_cast_e4m3.argtypes = [P, vp, ctypes.c_int, fp, ctypes.c_float, ctypes.c_int, vp,
                                             ctypes.c_int, fp, vp]
        L.h3ref_qk_sage.argtypes = [P, vp, ctypes.c_int, fp, fp, ctypes.c_float, fp, fp, vp]
        L.h3ref_static_descale.argtypes = [ctypes.c_float]
        L.h3ref_static_descale.restype = ctypes.c_float
        L.h3ref_norm_rope_row.argtypes = [fp, ctypes.c_int, fp, ctypes.c_float, ctypes.c_int, vp, vp, fp]
        L.h3ref_token_rows.argtypes = [P, ctypes.c_int, i64, vp]
        for n in ("f16", "bf16"):
            getattr(L, f"h3ref_{n}_encode").argtypes = [ctypes.c_float]
            getattr(L, f"h3ref_{n}_encode").restype = ctypes.c_uint16
            getattr(L, f"h3ref_{n}_decode").argtypes = [ctypes.c_uint16]
            getattr(L, f"h3ref_{n}_decode").restype = ctypes.c_float
            getattr(L, f"h3ref_{n}_encode_array").argtypes = [fp, vp, i64]
        L.h3ref_e4m3_encode.argtypes = [ctypes.c_float]
        L.h3ref_e4m3_encode.restype = ctypes.c_uint8
        L.h3ref_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.h3ref_e4m3_decode.restype = ctypes.c_float
        L.h3ref_e4m3_encode_array.argtypes = [fp, vp, i64]
        L.h3ref_f16_encode_f64.argtypes = [ctypes.c_double]
        L.h3ref_f16_encode_f64.restype = ctypes.c_uint16
        L.h3ref_bf16_encode_f64.argtypes = [ctypes.c_double]
        L.h3ref_bf16_encode_f64.restype = ctypes.c_uint16
        L.h3ref_swiglu.argtypes = [vp, vp, i64, i64, ctypes.c_int]
        L.h3ref_scaled_residual.argtypes = [fp, vp, fp, i64, fp, i64, i64, ctypes.c_int]
        L.h3ref_descale.argtypes = [ctypes.c_float]
        L.h3ref_descale.restype = ctypes.c_float
        _lib = L
    return _lib


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("row_stride", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
        ("grid", ctypes.c_int32 * 3),
        ("pos_offset", ctypes.c_void_p), ("valid_len", ctypes.c_void_p),
        ("n", ctypes.c_int32), ("table_len", ctypes.c_int32 * 3),
        ("cos_tab", ctypes.c_void_p), ("sin_tab", ctypes.c_void_p),
        ("eps", ctypes.c_float),
    ]


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Spec:
    """Problem description for the oracle; keeps the numpy arrays it points into alive."""

    def __init__(self, B, T, H, D, grid, n, table_len, cos_tab, sin_tab, pos_offset=None,
                 valid_len=None, eps=1e-6, row_stride=None, batch_stride=None):
        self.B, self.T, self.H, self.D, self.n = B, T, H, D, n
        self.grid = tuple(grid)
        self.table_len = tuple(table_len)
        self.cos = np.ascontiguousarray(cos_tab, dtype=np.float32)
        self.sin = np.ascontiguousarray(sin_tab, dtype=np.float32)
        self.off = np.ascontiguousarray(np.zeros((B, 3), np.int32) if pos_offset is None else pos_offset, dtype=np.int32)
        self.vl = np.ascontiguousarray(np.full(B, T, np.int32) if valid_len is None else valid_len, dtype=np.int32)
        self.eps = float(eps)
        self.row_stride = 3 * H * D if row_stride is None else int(row_stride)
        self.batch_stride = T * self.row_stride if batch_stride is None else int(batch_stride)
        assert self.off.shape == (B, 3) and self.vl.shape == (B,)
        assert self.cos.shape == (sum(self.table_len), n) and self.sin.shape == self.cos.shape

    def c(self) -> Problem:
        p = Problem()
        p.B, p.T, p.H, p.D = self.B, self.T, self.H, self.D
        p.row_stride, p.batch_stride = self.row_stride, self.batch_stride
        p.grid = (ctypes.c_int32 * 3)(*self.grid)
        p.pos_offset, p.valid_len = _ptr(self.off), _ptr(self.vl)
        p.n = self.n
        p.table_len = (ctypes.c_int32 * 3)(*self.table_len)
        p.cos_tab, p.sin_tab = _ptr(self.cos), _ptr(self.sin)
        p.eps = self.eps
        return p


def spec_from_workload(wl, **over) -> Spec:
    """Oracle spec for a synth.Workload (tables, offsets, valid lengths from the generator)."""
    import synth
    cos, sin = synth.rope_tables(wl.table_len, wl.n)
    kw = dict(B=wl.B, T=wl.T, H=wl.H, D=wl.D, grid=wl.grid, n=wl.n, table_len=wl.table_len,
              cos_tab=cos, sin_tab=sin, pos_offset=synth.pos_offsets(wl), valid_len=wl.valid_len,
              eps=wl.eps, row_stride=wl.stride)
    kw.update(over)
    return Spec(**kw)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def qk_rmsnorm_rope_permute(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k, q_dt="f32", k_dt="f16"):
    """Head-major (Q, K, V) for the whole problem.  qkv holds the 16-bit input bits."""
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    assert qkv.size >= (spec.B - 1) * spec.batch_stride + spec.T * spec.row_stride
    shape = (spec.B, spec.H, spec.T, spec.D)
    q = np.empty(shape, NP_DT[q_dt]); k = np.empty(shape, NP_DT[k_dt]); v = np.empty(shape, np.uint16)
    wq, wk = _f32(w_q), _f32(w_k)
    P = spec.c()
    rc = lib().h3ref_qk_rmsnorm_rope_permute(ctypes.byref(P), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk),
                                             _ptr(q), DT[q_dt], _ptr(k), DT[k_dt], _ptr(v))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return q, k, v


def qk_amax(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k) -> np.ndarray:
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    wq, wk = _f32(w_q), _f32(w_k)
    amax = np.zeros(2, np.float32)
    P = spec.c()
    rc = lib().h3ref_qk_amax(ctypes.byref(P), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk), _ptr(amax))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return amax


def qk_cast_e4m3(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k, amax):
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    wq, wk, am = _f32(w_q), _f32(w_k), _f32(amax)
    shape = (spec.B, spec.H, spec.T, spec.D)
    q = np.empty(shape, np.uint8); k = np.empty(shape, np.uint8); v = np.empty(shape, np.uint16)
    ds = np.zeros(2, np.float32)
    P = spec.c()
    rc = lib().h3ref_qk_cast_e4m3(ctypes.byref(P), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk), _ptr(am),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(ds))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return q, k, v, ds


def qk_cast_e4m3_static(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k, descale, v_fp8: bool = False):
    """FP8 cast with caller descales ([2], or [3] with v_fp8).  Returns (q, k, v, sat) with sat the
    uint64 [3] clip counts; v is uint8 codes when v_fp8, else the 16-bit bit copy."""
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    wq, wk = _f32(w_q), _f32(w_k)
    ds = np.ones(3, np.float32)
    d = _f32(descale).ravel()
    ds[:d.size] = d
    shape = (spec.B, spec.H, spec.T, spec.D)
    q = np.empty(shape, np.uint8); k = np.empty(shape, np.uint8)
    v = np.empty(shape, np.uint8 if v_fp8 else np.uint16)
    sat = np.zeros(3, np.uint64)
    P = spec.c()
    rc = lib().h3ref_qk_cast_e4m3_static(ctypes.byref(P), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk), _ptr(ds),
                                         int(v_fp8), _ptr(q), _ptr(k), _ptr(v), _ptr(sat))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return q, k, v, sat


def qkv_amax(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k) -> np.ndarray:
    """amax of Q and K (normalised, rotated) and of V (the input values) over the valid rows."""
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    wq, wk = _f32(w_q), _f32(w_k)
    amax = np.zeros(3, np.float32)
    rc = lib().h3ref_qkv_amax(ctypes.byref(spec.c()), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk), _ptr(amax))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return amax


def qkv_cast_e4m3(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k, amax):
    """Dynamic cast of Q, K and V; returns (q, k, v codes, descale[3])."""
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    wq, wk, am = _f32(w_q), _f32(w_k), _f32(amax)
    assert am.size == 3
    shape = (spec.B, spec.H, spec.T, spec.D)
    q = np.empty(shape, np.uint8); k = np.empty(shape, np.uint8); v = np.empty(shape, np.uint8)
    ds = np.zeros(3, np.float32)
    rc = lib().h3ref_qkv_cast_e4m3(ctypes.byref(spec.c()), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk), _ptr(am),
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(ds))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return q, k, v, ds


def _tensor_args(spec, x, w):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.size >= (spec.B - 1) * spec.batch_stride + (spec.T - 1) * spec.row_stride + spec.H * spec.D
    wp = None if w is None else _f32(w)
    return x, wp, (0 if wp is None else _ptr(wp))


def _out_shape(spec, layout):
    return (spec.B, spec.H, spec.T, spec.D) if layout == 0 else (spec.B, spec.T, spec.H, spec.D)


def tensor_norm_rope(spec: Spec, x: np.ndarray, in_dt: str, w, out_dt: str, layout: int = 0) -> np.ndarray:
    """One separately projected tensor (spec.H = its heads, spec.row_stride = its token stride):
    norm + RoPE with weight w, or the identity when w is None; layout 0 [B,H,T,D], 1 [B,T,H,D]."""
    x, wp, wptr = _tensor_args(spec, x, w)
    out = np.empty(_out_shape(spec, layout), NP_DT[out_dt])
    rc = lib().h3ref_tensor_norm_rope(ctypes.byref(spec.c()), _ptr(x), DT[in_dt], wptr, _ptr(out), DT[out_dt],
                                      layout)
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return out


def tensor_amax(spec: Spec, x: np.ndarray, in_dt: str, w) -> float:
    x, wp, wptr = _tensor_args(spec, x, w)
    a = np.zeros(1, np.float32)
    rc = lib().h3ref_tensor_amax(ctypes.byref(spec.c()), _ptr(x), DT[in_dt], wptr, _ptr(a))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return a[0]


def tensor_cast_e4m3(spec: Spec, x: np.ndarray, in_dt: str, w, scale: float, is_descale: bool, layout: int = 0):
    """Codes E4M3(y' / ds): ds from an amax (is_descale False) or a caller descale (True).
    Returns (codes, descale, clip count)."""
    x, wp, wptr = _tensor_args(spec, x, w)
    out = np.empty(_out_shape(spec, layout), np.uint8)
    ds = np.zeros(1, np.float32)
    sat = np.zeros(1, np.uint64)
    rc = lib().h3ref_tensor_cast_e4m3(ctypes.byref(spec.c()), _ptr(x), DT[in_dt], wptr, ctypes.c_float(scale),
                                      int(is_descale), _ptr(out), layout, _ptr(ds), _ptr(sat))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return out, ds[0], int(sat[0])


def qk_sage(spec: Spec, qkv: np.ndarray, in_dt: str, w_q, w_k, kv_scale: float):
    """Sage emission: (Q f32, K * kv_scale f32, V * kv_scale f16 bits), head-major [B, H, T, D]."""
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    wq, wk = _f32(w_q), _f32(w_k)
    shape = (spec.B, spec.H, spec.T, spec.D)
    q = np.empty(shape, np.float32); k = np.empty(shape, np.float32); v = np.empty(shape, np.uint16)
    rc = lib().h3ref_qk_sage(ctypes.byref(spec.c()), _ptr(qkv), DT[in_dt], _ptr(wq), _ptr(wk),
                             ctypes.c_float(kv_scale), _ptr(q), _ptr(k), _ptr(v))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return q, k, v


def static_descale(d: float) -> float:
    return lib().h3ref_static_descale(ctypes.c_float(d))


def qk_tokens(spec: Spec, qkv_rows: np.ndarray, tokens, in_dt: str, w_q, w_k, q_dt="f32", k_dt="f16",
              fp8=False, amax=None, descale=None, v_fp8=False, sat=None):
    """Outputs for selected tokens only.  qkv_rows [n_tok, row_stride] holds their input rows.
    fp8: descales from amax (dynamic) or, when `descale` is given, the caller's static descales
    (guarded like the library); v_fp8 casts V with descale[2].  Returns (q, k, v, y) with q, k, v
    [n_tok, H, D] and y the f32 y' [n_tok, 2, H, D]; `sat` (uint64 [3]) is added to."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    n = tokens.size
    rows = np.ascontiguousarray(qkv_rows, dtype=np.uint16).reshape(n, spec.row_stride)
    wq, wk = _f32(w_q), _f32(w_k)
    ds = np.ones(3, np.float32)
    if fp8 and descale is not None:
        d = _f32(descale).ravel()
        for j in range(d.size):
            ds[j] = static_descale(float(d[j]))
    elif fp8:
        am = _f32(np.zeros(2) if amax is None else amax).ravel()
        for j in range(am.size):
            ds[j] = descale_of(float(am[j]))
    qd, kd = ("e4m3", "e4m3") if fp8 else (q_dt, k_dt)
    shape = (n, spec.H, spec.D)
    q = np.empty(shape, NP_DT[qd]); k = np.empty(shape, NP_DT[kd])
    v = np.empty(shape, np.uint8 if (fp8 and v_fp8) else np.uint16)
    y = np.empty((n, 2, spec.H, spec.D), np.float32)
    counts = np.zeros(3, np.uint64) if sat is None else sat
    assert counts.dtype == np.uint64 and counts.size == 3 and counts.flags.c_contiguous
    P = spec.c()
    rc = lib().h3ref_qk_tokens_ex(ctypes.byref(P), _ptr(rows), DT[in_dt], _ptr(wq), _ptr(wk), _ptr(tokens), n,
                                  int(fp8), _ptr(ds), int(v_fp8), _ptr(q), DT[qd], _ptr(k), DT[kd], _ptr(v), _ptr(y),
                                  _ptr(counts))
    if rc:
        raise ValueError(f"oracle: position outside the tables (rc={rc})")
    return q, k, v, y


def qk_tokens_store(spec: Spec, qkv_rows: np.ndarray, tokens, in_dt: str, w_q, w_k, q_dt="f32", k_dt="f16",
                    threads: int = 1):
    """The non-FP8 outputs (q, k, v [n_tok, H, D]) of selected tokens, the token list split into
    `threads` contiguous blocks that run h3ref_qk_tokens_ex at the same time on host threads (ctypes
    releases the interpreter lock during the call, and the oracle's row buffers are per thread).
    Rows are independent, so the result does not depend on `threads`.  Used to time the oracle on
    one core and on all cores; y' is not written out."""
    from concurrent.futures import ThreadPoolExecutor
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    n = tokens.size
    rows = np.ascontiguousarray(qkv_rows, dtype=np.uint16).reshape(n, spec.row_stride)
    wq, wk = _f32(w_q), _f32(w_k)
    ds = np.ones(3, np.float32)
    shape = (n, spec.H, spec.D)
    q = np.empty(shape, NP_DT[q_dt]); k = np.empty(shape, NP_DT[k_dt]); v = np.empty(shape, np.uint16)
    P = spec.c()
    L = lib()
    cuts = [n * j // threads for j in range(threads + 1)]

    def block(j):
        a, b = cuts[j], cuts[j + 1]
        if b <= a:
            return 0
        return L.h3ref_qk_tokens_ex(ctypes.byref(P), _ptr(rows[a:b]), DT[in_dt], _ptr(wq), _ptr(wk),
                                    _ptr(tokens[a:b]), b - a, 0, _ptr(ds), 0, _ptr(q[a:b]), DT[q_dt], _ptr(k[a:b]),
                                    DT[k_dt], _ptr(v[a:b]), None, None)

    if threads == 1:
        rcs = [block(0)]
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            rcs = list(ex.map(block, range(threads)))
    if any(rcs):
        raise ValueError(f"oracle: position outside the tables (rc={rcs})")
    return q, k, v


def norm_rope_row(x, w, eps, n, crow, srow):
    """One row through the oracle's norm + rotation; crow/srow: three length-n arrays (t, h, w)."""
    x, w = _f32(x), _f32(w)
    D = x.size
    c = [_f32(r) for r in crow]
    s = [_f32(r) for r in srow]
    cp = (ctypes.c_void_p * 3)(*[_ptr(a) for a in c])
    sp = (ctypes.c_void_p * 3)(*[_ptr(a) for a in s])
    y = np.empty(D, np.float32)
    lib().h3ref_norm_rope_row(_ptr(x), D, _ptr(w), ctypes.c_float(eps), n, ctypes.cast(cp, ctypes.c_void_p),
                              ctypes.cast(sp, ctypes.c_void_p), _ptr(y))
    return y


def token_rows(spec: Spec, b: int, i: int):
    rows = np.zeros(3, np.int32)
    P = spec.c()
    rc = lib().h3ref_token_rows(ctypes.byref(P), b, i, _ptr(rows))
    return None if rc else rows


def encode(x: np.ndarray, dt: str) -> np.ndarray:
    x = _f32(x).ravel()
    if dt == "e4m3":
        y = np.empty(x.size, np.uint8)
        lib().h3ref_e4m3_encode_array(_ptr(x), _ptr(y), x.size)
    else:
        y = np.empty(x.size, np.uint16)
        getattr(lib(), f"h3ref_{dt}_encode_array")(_ptr(x), _ptr(y), x.size)
    return y


def decode(bits: np.ndarray, dt: str) -> np.ndarray:
    fn = getattr(lib(), f"h3ref_{dt}_decode")
    return np.array([fn(int(b)) for b in np.ravel(bits)], dtype=np.float32)


def descale(amax: float) -> float:
    return lib().h3ref_descale(ctypes.c_float(amax))


descale_of = descale


def swiglu(x_bits: np.ndarray, in_dt: str = "f16", threads: int = 1) -> np.ndarray:
    """x_bits [N, 2F] 16-bit -> y bits [N, F]: silu(gate) * up in binary64, one rounding.  With
    threads > 1 the rows are split into contiguous blocks evaluated on host threads at once (the C
    loop keeps no state, and ctypes releases the interpreter lock during the call)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    N, F2 = x.shape
    y = np.empty((N, F2 // 2), np.uint16)
    L = lib()
    cuts = [N * j // threads for j in range(threads + 1)]

    def block(j):
        a, b = cuts[j], cuts[j + 1]
        if b > a:
            L.h3ref_swiglu(_ptr(x[a:b]), _ptr(y[a:b]), b - a, F2 // 2, DT[in_dt])

    if threads == 1:
        block(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(block, range(threads)))
    return y


def scaled_residual(res: np.ndarray, branch_bits: np.ndarray, scale: np.ndarray, in_dt: str = "f16") -> np.ndarray:
    res = np.ascontiguousarray(res, dtype=np.float32)
    br = np.ascontiguousarray(branch_bits, dtype=np.uint16)
    sc = np.ascontiguousarray(scale, dtype=np.float32).ravel()
    N, C = res.shape
    out = np.empty_like(res)
    lib().h3ref_scaled_residual(_ptr(res), _ptr(br), _ptr(sc), sc.size, _ptr(out), N, C, DT[in_dt])
    return out


def f16_encode_f64(v: float) -> int:
    return lib().h3ref_f16_encode_f64(ctypes.c_double(v))


def bf16_encode_f64(v: float) -> int:
    return lib().h3ref_bf16_encode_f64(ctypes.c_double(v))
