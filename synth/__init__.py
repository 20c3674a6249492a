"""Seeded synthetic inputs for the fused QK RMSNorm + 3-axis RoPE + head-major permute workloads.

Every generated element is a pure function of (seed, stream, flat index): a SplitMix64 finaliser
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) hashes the
counter, and the top 16 bits of the hash index a 65536-entry table of standard-normal quantiles
that is already rounded to the storage dtype.  Because the per-element path is integer arithmetic
plus a table lookup, the host (numpy) and the device (torch integer ops) produce identical bits,
and any subset of tokens can be regenerated on its own.

This module is shared by the tests, the bench and the smoke check.  It holds none of the
operation's arithmetic: it only makes the inputs (activations, norm weights, per-item position
offsets and the rotary cos/sin tables the caller owns).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB

# substreams
S_QKV, S_WQ, S_WK, S_OFF = 1, 2, 3, 4

# P(outlier) for the "x2_outliers" distribution: low 32 bits of the hash below this threshold.
OUTLIER_THRESHOLD = 42949673  # ~= 0.01 * 2**32

THETA = 10000.0


def _mix64_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return _mix64_int(seed * _GOLDEN + (stream << 32) + stream)


# ----------------------------------------------------------------------------- host (numpy)

def hash_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """uint64 hash of each counter in idx (any integer array)."""
    key = np.uint64(stream_key(seed, stream))
    with np.errstate(over="ignore"):
        z = (idx.astype(np.uint64) + np.uint64(1)) * np.uint64(_GOLDEN) + key
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_C1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_C2)
        z = z ^ (z >> np.uint64(31))
    return z


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


_QCACHE: dict = {}


def normal_quantiles() -> np.ndarray:
    """fp64 standard-normal quantiles at the 65536 bin centres (k + 1/2) / 65536."""
    if "q" not in _QCACHE:
        from scipy.special import ndtri
        _QCACHE["q"] = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0)
    return _QCACHE["q"]


def value_tables(dist: str, dtype: str) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """(regular, outlier) uint16 bit tables for a distribution and a 16-bit storage dtype."""
    q = normal_quantiles()
    if dist == "normal":
        reg, out = q, None
    elif dist == "x2_outliers":
        reg, out = 2.0 * q, 40.0 * q
    elif dist == "zeros":
        reg, out = np.zeros_like(q), None
    else:
        raise ValueError(dist)

    def enc(v):
        if dtype == "f16":
            return v.astype(np.float16).view(np.uint16)
        if dtype == "bf16":
            return _f32_to_bf16_bits(v.astype(np.float32))
        raise ValueError(dtype)

    return enc(reg), (None if out is None else enc(out))


def values_np(seed: int, stream: int, idx: np.ndarray, dist: str, dtype: str) -> np.ndarray:
    """uint16 bit patterns of the synthetic activations at flat indices idx."""
    reg, out = value_tables(dist, dtype)
    h = hash_np(seed, stream, idx)
    v = reg[(h >> np.uint64(48)).astype(np.int64)]
    if out is not None:
        low = h & np.uint64(0xFFFFFFFF)
        v = np.where(low < np.uint64(OUTLIER_THRESHOLD), out[(h >> np.uint64(48)).astype(np.int64)], v)
    return v


# ----------------------------------------------------------------------------- device (torch)

def _to_i64(c: int) -> int:
    c &= _M64
    return c - (1 << 64) if c >= (1 << 63) else c


def _lsr(z, k: int):
    return (z >> k) & ((1 << (64 - k)) - 1)


def hash_torch(seed: int, stream: int, idx):
    """Same hash as hash_np, on an int64 torch tensor (wrapping arithmetic)."""
    key = _to_i64(stream_key(seed, stream))
    z = (idx + 1) * _to_i64(_GOLDEN) + key
    z = (z ^ _lsr(z, 30)) * _to_i64(_C1)
    z = (z ^ _lsr(z, 27)) * _to_i64(_C2)
    return z ^ _lsr(z, 31)


def values_torch(seed: int, stream: int, start: int, count: int, dist: str, dtype: str, device,
                 out=None, chunk: int = 1 << 25):
    """int16 tensor of the bit patterns for flat indices [start, start+count), made on `device`."""
    import torch
    reg, outl = value_tables(dist, dtype)
    treg = torch.from_numpy(reg.view(np.int16).copy()).to(device)
    tout = None if outl is None else torch.from_numpy(outl.view(np.int16).copy()).to(device)
    if out is None:
        out = torch.empty(count, dtype=torch.int16, device=device)
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        idx = torch.arange(start + c0, start + c0 + n, dtype=torch.int64, device=device)
        h = hash_torch(seed, stream, idx)
        u = _lsr(h, 48)
        v = treg[u]
        if tout is not None:
            low = h & 0xFFFFFFFF
            v = torch.where(low < OUTLIER_THRESHOLD, tout[u], v)
        out[c0:c0 + n] = v
        del idx, h, u, v
    return out


# ----------------------------------------------------------------------------- workloads

@dataclasses.dataclass
class Workload:
    name: str
    B: int
    grid: Tuple[int, int, int]      # (Gt, Gh, Gw) latent token grid, t-major, w fastest
    T: int                          # padded tokens per item
    H: int
    D: int
    n: int                          # rotated pairs per axis
    in_dtype: str                   # "f16" | "bf16"
    dist: str                       # "normal" | "x2_outliers"
    seed: int
    valid: Optional[Sequence[int]] = None   # per-item valid length (None: all T)
    offset_hw_max: int = 0          # h/w offsets drawn from [0, offset_hw_max)
    q_dtype: str = "f32"
    k_dtype: str = "f16"
    fp8: bool = False
    eps: float = 1e-6
    row_stride: Optional[int] = None

    @property
    def stride(self) -> int:
        return self.row_stride if self.row_stride is not None else 3 * self.H * self.D

    @property
    def valid_len(self) -> np.ndarray:
        if self.valid is None:
            return np.full(self.B, self.T, dtype=np.int32)
        return np.asarray(self.valid, dtype=np.int32)

    @property
    def table_len(self) -> Tuple[int, int, int]:
        gt, gh, gw = self.grid
        m = max(self.offset_hw_max - 1, 0)
        return (gt, gh + m, gw + m)

    def qkv_numel(self) -> int:
        return self.B * self.T * self.stride


def workloads() -> dict:
    """The five seeded configurations: tiny, one tile, eight tiles, full latent, FP8 long sequence."""
    w = [
        Workload("tiny", 1, (2, 4, 4), 32, 2, 64, 8, "f16", "normal", 1000),
        Workload("tile", 1, (31, 16, 16), 7936, 16, 64, 8, "f16", "x2_outliers", 1001),
        Workload("tiles8", 8, (31, 20, 20), 12400, 16, 64, 8, "f16", "normal", 1002, offset_hw_max=64),
        Workload("latent", 1, (62, 48, 84), 249984, 16, 64, 8, "f16", "normal", 1003),
        Workload("fp8long", 1, (31, 34, 99), 104448, 24, 128, 16, "bf16", "normal", 1004,
                 valid=[104076], fp8=True, q_dtype="e4m3", k_dtype="e4m3"),
    ]
    return {x.name: x for x in w}


def by_index(i: int) -> Workload:
    return list(workloads().values())[i]


def norm_weights(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """w_q, w_k: fp32 [D], 1 + 0.1 z with z standard normal (53-bit uniform through ndtri)."""
    from scipy.special import ndtri
    res = []
    for s in (S_WQ, S_WK):
        h = hash_np(wl.seed, s, np.arange(wl.D))
        u = ((h >> np.uint64(11)).astype(np.float64) + 0.5) / float(1 << 53)
        res.append((1.0 + 0.1 * ndtri(u)).astype(np.float32))
    return res[0], res[1]


def pos_offsets(wl: Workload) -> np.ndarray:
    """int32 [B, 3] per-item (t, h, w) position offsets: t = 0, h and w uniform in [0, max)."""
    off = np.zeros((wl.B, 3), dtype=np.int32)
    if wl.offset_hw_max > 0:
        h = hash_np(wl.seed, S_OFF, np.arange(2 * wl.B))
        u = (h >> np.uint64(32)).astype(np.float64) / float(1 << 32)
        off[:, 1:] = np.floor(u * wl.offset_hw_max).astype(np.int32).reshape(wl.B, 2)
    return off


def rope_tables(table_len: Tuple[int, int, int], n: int, theta: float = THETA):
    """Caller-owned rotary tables, fp32 [(P_t + P_h + P_w), n], axis-major (t rows, then h, then w).

    Row `base_a + p` holds cos / sin of p * theta**(-j/n) for j < n, evaluated in fp64 and rounded
    to fp32; the frequency ladder restarts on every axis.  Position 0 gives exactly (1, 0).
    """
    rows_c, rows_s = [], []
    inv = theta ** (-(np.arange(n, dtype=np.float64) / n))
    for P in table_len:
        ang = np.arange(P, dtype=np.float64)[:, None] * inv[None, :]
        rows_c.append(np.cos(ang))
        rows_s.append(np.sin(ang))
    return (np.concatenate(rows_c).astype(np.float32), np.concatenate(rows_s).astype(np.float32))


def qkv_host(wl: Workload, tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """uint16 bits of the fused QKV input: [B, T, stride], or [len(tokens), stride] for the given
    flat token ids (b * T + i)."""
    if tokens is None:
        idx = np.arange(wl.qkv_numel(), dtype=np.int64)
        return values_np(wl.seed, S_QKV, idx, wl.dist, wl.in_dtype).reshape(wl.B, wl.T, wl.stride)
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = tokens[:, None] * wl.stride + np.arange(wl.stride, dtype=np.int64)[None, :]
    return values_np(wl.seed, S_QKV, idx, wl.dist, wl.in_dtype)


def qkv_device(wl: Workload, device="cuda"):
    """The same fused QKV input made on the device: torch int16 [B, T, stride] (viewed by the
    caller as float16 / bfloat16)."""
    v = values_torch(wl.seed, S_QKV, 0, wl.qkv_numel(), wl.dist, wl.in_dtype, device)
    return v.view(wl.B, wl.T, wl.stride)


# ----------------------------------------------------------------------------- decoder-block ops

S_SWIGLU, S_RES, S_BRANCH, S_SCALE = 5, 6, 7, 8

# Shapes of the isolated decoder-block measurements of the vllm-omni MiniMax-H3 VAE review thread:
# SwiGLU on the w1 output [1, 1797, 16384]; scaled residual on [2, 1797, 2048].
SWIGLU_SHAPE = (1797, 8192)          # (N, F): x is [N, 2F]
RESIDUAL_SHAPE = (2 * 1797, 2048)    # (N, C)


def vae_qk_workload() -> Workload:
    """Q and K of the same thread's isolated Q/K RMSNorm + RoPE measurement, [2, 1797, 32, 64] f16,
    each a separate tensor.  The thread gives only the shape: the 3 x 599 x 1 token grid and n = 8
    rotated pairs per axis are this generator's choice."""
    return Workload("vae_qk", 2, (3, 599, 1), 1797, 32, 64, 8, "f16", "normal", 3001)


def swiglu_input(N: int, F: int, dtype: str = "f16", seed: int = 2000) -> np.ndarray:
    """uint16 bits [N, 2F]: standard normal x 3 (so the gate spans silu's curved region)."""
    idx = np.arange(N * 2 * F, dtype=np.int64)
    q = normal_quantiles()
    h = hash_np(seed, S_SWIGLU, idx)
    v = (3.0 * q)[(h >> np.uint64(48)).astype(np.int64)]
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16).reshape(N, 2 * F)
    return _f32_to_bf16_bits(v.astype(np.float32)).reshape(N, 2 * F)


def residual_inputs(N: int, C: int, dtype: str = "f16", seed: int = 2001):
    """(res fp32 [N, C], branch 16-bit bits [N, C], scale fp32 [C] = 1 + 0.1 z)."""
    q = normal_quantiles()
    idx = np.arange(N * C, dtype=np.int64)
    res = q[(hash_np(seed, S_RES, idx) >> np.uint64(48)).astype(np.int64)].astype(np.float32).reshape(N, C)
    braw = q[(hash_np(seed, S_BRANCH, idx) >> np.uint64(48)).astype(np.int64)]
    branch = (braw.astype(np.float16).view(np.uint16) if dtype == "f16"
              else _f32_to_bf16_bits(braw.astype(np.float32))).reshape(N, C)
    sc = q[(hash_np(seed, S_SCALE, np.arange(C)) >> np.uint64(48)).astype(np.int64)]
    scale = (1.0 + 0.1 * sc).astype(np.float32)
    return res, branch, scale
