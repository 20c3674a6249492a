"""Device-side setup of a seeded synthetic problem: uploads the generated inputs (activations,
weights, tables), fills the libh3qk descriptor and allocates outputs.  Glue only: no arithmetic
of the operation.  Shared by the GPU tests, the bench and the smoke check."""
from __future__ import annotations

import numpy as np

import synth

_TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16", "e4m3": "uint8"}


def torch_dtype(dt: str):
    import torch
    return getattr(torch, _TORCH_DT[dt])


class DeviceProblem:
    """Inputs of a synth.Workload resident on the device plus its h3_qk_desc."""

    def __init__(self, wl: synth.Workload, device="cuda", qkv_bits: np.ndarray = None):
        import torch
        import rmsnorm_rope_amd as h3
        self.wl = wl
        self.device = device
        if qkv_bits is None:
            self.qkv = synth.qkv_device(wl, device)                      # int16 [B, T, stride]
        else:
            self.qkv = torch.from_numpy(np.ascontiguousarray(qkv_bits).view(np.int16)).to(device)
        wq, wk = synth.norm_weights(wl)
        self.wq_host, self.wk_host = wq, wk
        self.wq = torch.from_numpy(wq).to(device)
        self.wk = torch.from_numpy(wk).to(device)
        cos, sin = synth.rope_tables(wl.table_len, wl.n)
        self.cos = torch.from_numpy(cos).to(device)
        self.sin = torch.from_numpy(sin).to(device)
        self.off = synth.pos_offsets(wl)
        self.desc = h3.make_desc(wl.B, wl.T, wl.H, wl.D, wl.grid, wl.n, wl.table_len, self.cos, self.sin,
                                 pos_offset=self.off, valid_len=wl.valid_len, eps=wl.eps,
                                 row_stride=wl.stride, batch_stride=wl.T * wl.stride)

    @property
    def in_dt(self) -> str:
        return self.wl.in_dtype

    def out(self, dt: str):
        import torch
        wl = self.wl
        return torch.empty((wl.B, wl.H, wl.T, wl.D), dtype=torch_dtype(dt), device=self.device)

    def qkv_host(self) -> np.ndarray:
        """uint16 copy of the device input (what the kernels read)."""
        return self.qkv.cpu().numpy().view(np.uint16)

    # --- the three passes through the C ABI ------------------------------------------
    def run_store(self, q_dt="f32", k_dt="f16", outs=None, stream=None):
        import rmsnorm_rope_amd as h3
        q, k, v = outs if outs is not None else (self.out(q_dt), self.out(k_dt), self.out(self.in_dt))
        h3.h3_qk_rmsnorm_rope_permute(self.desc, self.qkv, self.in_dt, self.wq, self.wk, q, q_dt, k, k_dt, v,
                                      stream=stream)
        return q, k, v

    def run_sage(self, kv_scale, outs=None, stream=None):
        """Sage emission: (Q f32, K * kv_scale f32, V * kv_scale f16)."""
        import rmsnorm_rope_amd as h3
        q, k, v = outs if outs is not None else (self.out("f32"), self.out("f32"), self.out("f16"))
        h3.h3_qk_rmsnorm_rope_permute_sage(self.desc, self.qkv, self.in_dt, self.wq, self.wk, kv_scale, q, k, v,
                                           stream=stream)
        return q, k, v

    def run_amax(self, amax=None, stream=None):
        import torch
        import rmsnorm_rope_amd as h3
        if amax is None:
            amax = torch.empty(2, dtype=torch.float32, device=self.device)
        h3.h3_qk_amax(self.desc, self.qkv, self.in_dt, self.wq, self.wk, amax, stream=stream)
        return amax

    def run_cast(self, amax, outs=None, stream=None):
        import torch
        import rmsnorm_rope_amd as h3
        if outs is None:
            outs = (self.out("e4m3"), self.out("e4m3"), self.out(self.in_dt),
                    torch.empty(2, dtype=torch.float32, device=self.device))
        q, k, v, ds = outs
        h3.h3_qk_cast_e4m3(self.desc, self.qkv, self.in_dt, self.wq, self.wk, amax, q, k, v, ds, stream=stream)
        return q, k, v, ds


    def run_cast_static(self, descale, v_fp8=False, count=True, outs=None, stream=None):
        """Static-scale cast: descale is a device fp32 tensor ([2] or [3]).  Returns
        (q, k, v, sat) with sat the device int64 clip-counter buffer [SAT_WORDS] whose first three
        words are the counts (None when count is False)."""
        import torch
        import rmsnorm_rope_amd as h3
        if outs is None:
            outs = (self.out("e4m3"), self.out("e4m3"), self.out("e4m3" if v_fp8 else self.in_dt),
                    torch.empty(h3.SAT_WORDS, dtype=torch.int64, device=self.device) if count else None)
        q, k, v, sat = outs
        h3.h3_qk_cast_e4m3_static(self.desc, self.qkv, self.in_dt, self.wq, self.wk, descale, q, k, v,
                                  "e4m3" if v_fp8 else self.in_dt, sat, stream=stream)
        return q, k, v, sat


def oracle_spec(wl: synth.Workload):
    import oracle
    return oracle.spec_from_workload(wl, batch_stride=wl.T * wl.stride)


def algorithmic_bytes(wl: synth.Workload, mode: str, q_dt="f32", k_dt="f16") -> int:
    """Bytes the pass must move: read each needed input element once, write each output once
    (tables, weights and the 8-byte amax/descale are excluded)."""
    size = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
    valid = int(np.sum(wl.valid_len))
    tok_all = wl.B * wl.T
    hd = wl.H * wl.D
    if mode == "store":
        return valid * 3 * hd * 2 + tok_all * hd * (size[q_dt] + size[k_dt] + 2)
    if mode == "sage":
        return valid * 3 * hd * 2 + tok_all * hd * (4 + 4 + 2)
    if mode == "amax":
        return valid * 2 * hd * 2
    if mode == "amax_v":
        return valid * 3 * hd * 2
    if mode == "cast":
        return valid * 3 * hd * 2 + tok_all * hd * (1 + 1 + 2)
    if mode == "cast_v8":
        return valid * 3 * hd * 2 + tok_all * hd * (1 + 1 + 1)
    raise ValueError(mode)
