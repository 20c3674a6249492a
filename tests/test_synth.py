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
