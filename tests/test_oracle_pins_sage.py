"""Pins of the oracle's sage emission (stable-diffusion.cpp PR #19, sage commit: F32 Q, F32 K
times kv_scale and F16 V times kv_scale, head-major, with the unfused chain's rounding points).
No GPU.  K and V are checked against one binary32 multiplication (numpy) of the independently
pinned f32 outputs and input values, V's rounding against numpy's float16 cast; a power-of-two
scale against exact scaling; scale 1 against the plain store."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth

F = np.float32


def W(name, **kw):
    return dataclasses.replace(synth.workloads()[name], **kw)


def _problem(wl):
    sp = oracle.spec_from_workload(wl, batch_stride=wl.T * wl.stride)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    return sp, x, wq, wk


def _v_values(wl, x):
    H, D = wl.H, wl.D
    vb = x[:, :, 2 * H * D:3 * H * D].reshape(wl.B, wl.T, H, D).transpose(0, 2, 1, 3)
    if wl.in_dtype == "bf16":
        return (vb.astype(np.uint32) << 16).view(F)
    return vb.view(np.float16).astype(F)


@pytest.mark.parametrize("name,kw", [("tile", dict(T=300, grid=(2, 10, 15))),
                                     ("tiles8", dict(B=2, T=77, valid=[77, 40])),
                                     ("fp8long", dict(T=64, valid=[60], grid=(1, 8, 8)))])
@pytest.mark.parametrize("s", [1.0, 0.125, 0.08838834764831845, 3.7])
def test_sage_is_one_rounding_of_the_scaled_outputs(name, kw, s):
    wl = W(name, **kw)
    sp, x, wq, wk = _problem(wl)
    q, k, v = oracle.qk_sage(sp, x, wl.in_dtype, wq, wk, s)
    yq, yk, _ = oracle.qk_rmsnorm_rope_permute(sp, x, wl.in_dtype, wq, wk, "f32", "f32")
    assert np.array_equal(q.view(np.uint32), yq.view(np.uint32))
    sf = F(s)
    assert np.array_equal(k.view(np.uint32), (yk * sf).astype(F).view(np.uint32))
    with np.errstate(over="ignore"):
        vref = (_v_values(wl, x) * sf).astype(F).astype(np.float16).view(np.uint16)
    valid = np.zeros(vref.shape, bool)
    for b in range(wl.B):
        valid[b, :, :int(wl.valid_len[b])] = True
    vref = np.where(valid, vref, np.uint16(0))
    assert np.array_equal(v, vref)
    if s == 0.125:  # a power of two scales exactly
        assert np.array_equal(k, yk / 8)


def test_sage_scale_one_is_the_plain_store():
    wl = W("tile", T=200, grid=(1, 10, 20))
    sp, x, wq, wk = _problem(wl)
    q, k, v = oracle.qk_sage(sp, x, "f16", wq, wk, 1.0)
    yq, yk, yv = oracle.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk, "f32", "f32")
    assert np.array_equal(v, yv)  # f16 input: V * 1 rounds back to itself
    assert np.array_equal(k.view(np.uint32), yk.view(np.uint32))
