"""Python binding of libh3qk (include/h3qk.h): the same entry points, argument marshalling only.

Every computation runs in the gfx950 kernels of rmsnorm_rope_amd/libh3qk.so.  Device buffers
are passed as torch tensors (their data_ptr) or as raw integer device addresses; the stream
defaults to torch's current stream.  There is no fallback: if the library is not built, or a
call returns an error code, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "F32", "F16", "BF16", "E4M3FN", "MAX_BATCH", "SAT_WORDS", "H3Error", "QkDesc", "make_desc", "lib",
    "h3_qk_rmsnorm_rope_permute", "h3_qk_amax", "h3_qk_cast_e4m3", "h3_qk_cast_e4m3_static",
    "h3_qk_cast_e4m3_static_noalloc",
    "h3_qk_rmsnorm_rope_permute_sage", "h3_qkv_amax", "h3_qkv_cast_e4m3", "h3_tensor_norm_rope", "h3_tensor_amax", "h3_tensor_cast_e4m3",
    "LAYOUT_BHTD", "LAYOUT_BTHD", "h3_swiglu", "h3_scaled_residual",
    "h3_last_error", "h3_abi_version",
    "EXPORTS",
]

F32, F16, BF16, E4M3FN = 0, 1, 2, 3
MAX_BATCH = 64
SAT_SLOTS = 128
SAT_WORDS = 16 * (SAT_SLOTS + 1)  # uint64 words of a clip-counter buffer (counts in words 0..2)
LAYOUT_BHTD, LAYOUT_BTHD = 0, 1
_DT = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": E4M3FN, "e4m3fn": E4M3FN}
ERRORS = {0: "H3_OK", -1: "H3_EINVAL", -2: "H3_EUNSUPPORTED", -3: "H3_EALIGN", -4: "H3_ERANGE",
          -5: "H3_EALIAS", -6: "H3_ELAUNCH"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libh3qk.so")

# every function include/h3qk.h declares
EXPORTS = ("h3_qk_rmsnorm_rope_permute", "h3_qk_amax", "h3_qk_cast_e4m3", "h3_qk_cast_e4m3_static",
           "h3_qk_cast_e4m3_static_noalloc",
           "h3_qk_rmsnorm_rope_permute_sage", "h3_qkv_amax", "h3_qkv_cast_e4m3", "h3_tensor_norm_rope",
           "h3_tensor_amax", "h3_tensor_cast_e4m3", "h3_swiglu", "h3_scaled_residual", "h3_last_error", "h3_abi_version")


class H3Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} -> {ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class QkDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("row_stride", ctypes.c_int64), ("batch_stride", ctypes.c_int64),
        ("grid", ctypes.c_int32 * 3),
        ("pos_offset", (ctypes.c_int32 * 3) * MAX_BATCH),
        ("valid_len", ctypes.c_int32 * MAX_BATCH),
        ("pairs_per_axis", ctypes.c_int32),
        ("table_len", ctypes.c_int32 * 3),
        ("cos_tab", ctypes.c_void_p), ("sin_tab", ctypes.c_void_p),
        ("eps", ctypes.c_float),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        D = ctypes.POINTER(QkDesc)
        L.h3_qk_rmsnorm_rope_permute.argtypes = [D, vp, i32, vp, vp, vp, i32, vp, i32, vp, vp]
        L.h3_qk_amax.argtypes = [D, vp, i32, vp, vp, vp, vp]
        L.h3_qk_cast_e4m3.argtypes = [D, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.h3_qk_cast_e4m3_static.argtypes = [D, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp]
        L.h3_qk_cast_e4m3_static_noalloc.argtypes = [D, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp]
        L.h3_qk_rmsnorm_rope_permute_sage.argtypes = [D, vp, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp]
        L.h3_qkv_amax.argtypes = [D, vp, i32, vp, vp, vp, vp]
        L.h3_qkv_cast_e4m3.argtypes = [D, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.h3_tensor_norm_rope.argtypes = [D, vp, i32, vp, vp, i32, i32, vp]
        L.h3_tensor_amax.argtypes = [D, vp, i32, vp, vp, vp]
        L.h3_tensor_cast_e4m3.argtypes = [D, vp, i32, vp, vp, i32, vp, i32, vp, vp, vp]
        L.h3_swiglu.argtypes = [vp, i32, vp, ctypes.c_int64, ctypes.c_int64, vp]
        L.h3_scaled_residual.argtypes = [vp, vp, i32, vp, ctypes.c_int64, vp, ctypes.c_int64, ctypes.c_int64, vp]
        for f in EXPORTS[:-2]:
            getattr(L, f).restype = i32
        L.h3_last_error.restype = ctypes.c_char_p
        L.h3_last_error.argtypes = []
        L.h3_abi_version.restype = i32
        L.h3_abi_version.argtypes = []
        _lib = L
    return _lib


_NOT_CONTIGUOUS = "tensor arguments must be contiguous (token and batch strides go in the descriptor)"


def _ptr(x) -> Optional[int]:
    """Device address of a tensor argument (or an integer address as given).  A tensor must be a
    contiguous device tensor: the library reads and writes flat memory, and strides other than the
    descriptor's would silently address the wrong elements."""
    if x is None:
        return None
    is_cuda = getattr(x, "is_cuda", None)
    if is_cuda is not None:  # a torch tensor: the two checks at the cost of three attribute reads
        if not is_cuda:
            raise ValueError(f"tensor arguments must be device tensors, got one on {x.device}")
        if not x.is_contiguous():
            raise ValueError(_NOT_CONTIGUOUS)
        return x.data_ptr()
    if hasattr(x, "data_ptr"):  # another tensor-like object
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError(_NOT_CONTIGUOUS)
        dev = getattr(x, "device", None)
        if dev is not None and getattr(dev, "type", "cuda") != "cuda":
            raise ValueError(f"tensor arguments must be device tensors, got one on {dev}")
        return x.data_ptr()
    return int(x)


def _dt(x) -> int:
    return _DT[x] if isinstance(x, str) else int(x)


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise H3Error(fn, rc, lib().h3_last_error().decode())


def make_desc(B: int, T: int, H: int, D: int, grid: Sequence[int], pairs_per_axis: int,
              table_len: Sequence[int], cos_tab, sin_tab, pos_offset=None, valid_len=None,
              eps: float = 1e-6, row_stride: Optional[int] = None,
              batch_stride: Optional[int] = None) -> QkDesc:
    """Fill an h3_qk_desc.  cos_tab / sin_tab are device buffers; pos_offset ([B][3]) and
    valid_len ([B]) are host values (defaults: zeros and T)."""
    d = QkDesc()
    d.B, d.T, d.H, d.D = int(B), int(T), int(H), int(D)
    d.row_stride = 3 * H * D if row_stride is None else int(row_stride)
    d.batch_stride = T * d.row_stride if batch_stride is None else int(batch_stride)
    for a in range(3):
        d.grid[a] = int(grid[a])
        d.table_len[a] = int(table_len[a])
    for b in range(min(int(B), MAX_BATCH)):
        for a in range(3):
            d.pos_offset[b][a] = 0 if pos_offset is None else int(pos_offset[b][a])
        d.valid_len[b] = int(T) if valid_len is None else int(valid_len[b])
    d.pairs_per_axis = int(pairs_per_axis)
    d.cos_tab, d.sin_tab = _ptr(cos_tab), _ptr(sin_tab)
    d.eps = float(eps)
    return d


def h3_qk_rmsnorm_rope_permute(desc: QkDesc, qkv, in_dt, w_q, w_k, q_out, q_dt, k_out, k_dt, v_out,
                               stream=None) -> None:
    rc = lib().h3_qk_rmsnorm_rope_permute(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k),
                                          _ptr(q_out), _dt(q_dt), _ptr(k_out), _dt(k_dt), _ptr(v_out),
                                          _stream(stream))
    _check("h3_qk_rmsnorm_rope_permute", rc)


def h3_qk_amax(desc: QkDesc, qkv, in_dt, w_q, w_k, amax_qk, stream=None) -> None:
    rc = lib().h3_qk_amax(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k), _ptr(amax_qk),
                          _stream(stream))
    _check("h3_qk_amax", rc)


def h3_qk_cast_e4m3(desc: QkDesc, qkv, in_dt, w_q, w_k, amax_qk, q_codes, k_codes, v_out, descale_qk,
                    stream=None) -> None:
    rc = lib().h3_qk_cast_e4m3(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k),
                               _ptr(amax_qk), _ptr(q_codes), _ptr(k_codes), _ptr(v_out), _ptr(descale_qk),
                               _stream(stream))
    _check("h3_qk_cast_e4m3", rc)


def h3_qk_cast_e4m3_static(desc: QkDesc, qkv, in_dt, w_q, w_k, descale_qkv, q_codes, k_codes, v_out, v_dt,
                           sat_qkv=None, stream=None) -> None:
    rc = lib().h3_qk_cast_e4m3_static(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k),
                                      _ptr(descale_qkv), _ptr(q_codes), _ptr(k_codes), _ptr(v_out), _dt(v_dt),
                                      _ptr(sat_qkv), _stream(stream))
    _check("h3_qk_cast_e4m3_static", rc)


def h3_qk_cast_e4m3_static_noalloc(desc: QkDesc, qkv, in_dt, w_q, w_k, descale_qkv, q_codes, k_codes, v_out,
                                   v_dt, sat_counts=None, stream=None) -> None:
    rc = lib().h3_qk_cast_e4m3_static_noalloc(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k),
                                              _ptr(descale_qkv), _ptr(q_codes), _ptr(k_codes), _ptr(v_out),
                                              _dt(v_dt), _ptr(sat_counts), _stream(stream))
    _check("h3_qk_cast_e4m3_static_noalloc", rc)


def h3_qk_rmsnorm_rope_permute_sage(desc: QkDesc, qkv, in_dt, w_q, w_k, kv_scale: float, q_out, k_out, v_out,
                                    stream=None) -> None:
    rc = lib().h3_qk_rmsnorm_rope_permute_sage(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k),
                                               ctypes.c_float(kv_scale), _ptr(q_out), _ptr(k_out), _ptr(v_out),
                                               _stream(stream))
    _check("h3_qk_rmsnorm_rope_permute_sage", rc)


def h3_qkv_amax(desc: QkDesc, qkv, in_dt, w_q, w_k, amax_qkv, stream=None) -> None:
    rc = lib().h3_qkv_amax(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k), _ptr(amax_qkv),
                           _stream(stream))
    _check("h3_qkv_amax", rc)


def h3_qkv_cast_e4m3(desc: QkDesc, qkv, in_dt, w_q, w_k, amax_qkv, q_codes, k_codes, v_codes, descale_qkv,
                     stream=None) -> None:
    rc = lib().h3_qkv_cast_e4m3(ctypes.byref(desc), _ptr(qkv), _dt(in_dt), _ptr(w_q), _ptr(w_k), _ptr(amax_qkv),
                                _ptr(q_codes), _ptr(k_codes), _ptr(v_codes), _ptr(descale_qkv), _stream(stream))
    _check("h3_qkv_cast_e4m3", rc)


def h3_tensor_norm_rope(desc: QkDesc, x, in_dt, w, out, out_dt, out_layout=LAYOUT_BHTD, stream=None) -> None:
    rc = lib().h3_tensor_norm_rope(ctypes.byref(desc), _ptr(x), _dt(in_dt), _ptr(w), _ptr(out), _dt(out_dt),
                                   int(out_layout), _stream(stream))
    _check("h3_tensor_norm_rope", rc)


def h3_tensor_amax(desc: QkDesc, x, in_dt, w, amax, stream=None) -> None:
    rc = lib().h3_tensor_amax(ctypes.byref(desc), _ptr(x), _dt(in_dt), _ptr(w), _ptr(amax), _stream(stream))
    _check("h3_tensor_amax", rc)


def h3_tensor_cast_e4m3(desc: QkDesc, x, in_dt, w, scale, scale_is_descale: bool, codes, out_layout=LAYOUT_BHTD,
                        descale=None, sat=None, stream=None) -> None:
    rc = lib().h3_tensor_cast_e4m3(ctypes.byref(desc), _ptr(x), _dt(in_dt), _ptr(w), _ptr(scale),
                                   int(bool(scale_is_descale)), _ptr(codes), int(out_layout), _ptr(descale),
                                   _ptr(sat), _stream(stream))
    _check("h3_tensor_cast_e4m3", rc)


def h3_swiglu(x, dt, y, N: int, F: int, stream=None) -> None:
    rc = lib().h3_swiglu(_ptr(x), _dt(dt), _ptr(y), int(N), int(F), _stream(stream))
    _check("h3_swiglu", rc)


def h3_scaled_residual(res, branch, branch_dt, scale, scale_len: int, out, N: int, C: int, stream=None) -> None:
    rc = lib().h3_scaled_residual(_ptr(res), _ptr(branch), _dt(branch_dt), _ptr(scale), int(scale_len), _ptr(out),
                                  int(N), int(C), _stream(stream))
    _check("h3_scaled_residual", rc)


def h3_last_error() -> str:
    return lib().h3_last_error().decode()


def h3_abi_version() -> int:
    return lib().h3_abi_version()
