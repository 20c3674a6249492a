"""GPU parity, through the C ABI, of the FP8 recipe with V cast (h3_qkv_amax, h3_qkv_cast_e4m3)
and of the one-tensor passes (h3_tensor_norm_rope, h3_tensor_amax, h3_tensor_cast_e4m3) against
the CPU oracle: bit-exact outputs, amaxes, descales, codes and clip counts, on ragged and padded
cases, both layouts, Q/K (normalised) and V (identity), packed slices and compact tensors."""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth
from synth.problem import DeviceProblem, oracle_spec
from tests.gpu_util import bits, compare, compare_raw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    torch.cuda.set_device(0)
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def W(name, **kw):
    return dataclasses.replace(synth.workloads()[name], **kw)


# ----------------------------------------------------------------------------- fused Q, K, V FP8

FP8_CASES = [
    ("fp8long", dict(T=203, valid=[190])),
    ("fp8long", dict(T=64, valid=[64], H=3)),
    ("fp8long", dict(B=3, T=50, valid=[50, 0, 17], offset_hw_max=0)),
    ("fp8long", dict(T=31, valid=[0])),
    ("fp8long", dict(T=40, valid=[40], D=64, n=8, in_dtype="f16")),
    ("tiles8", dict(B=2, T=333, valid=[333, 101])),
]


def check_qkv_fp8(wl, qkv_bits=None):
    say(f"[qkv-fp8] {wl.name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} in={wl.in_dtype} valid={list(wl.valid_len)[:4]}")
    import rmsnorm_rope_amd as h3
    pb = DeviceProblem(wl, "cuda", qkv_bits=qkv_bits)
    amax = torch.empty(3, dtype=torch.float32, device="cuda")
    h3.h3_qkv_amax(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, amax)
    q, k, v = pb.out("e4m3"), pb.out("e4m3"), pb.out("e4m3")
    ds = torch.empty(3, dtype=torch.float32, device="cuda")
    h3.h3_qkv_cast_e4m3(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, amax, q, k, v, ds)
    torch.cuda.synchronize()
    sp = oracle_spec(wl)
    x = pb.qkv_host()
    ra = oracle.qkv_amax(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host)
    compare(bits(amax), ra, "f32", "amax_qkv")
    rq, rk, rv, rds = oracle.qkv_cast_e4m3(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, ra)
    compare(bits(ds), rds, "f32", "descale_qkv")
    compare(bits(q), rq, "e4m3", "Q codes")
    compare(bits(k), rk, "e4m3", "K codes")
    compare(bits(v), rv, "e4m3", "V codes")
    return ra


@pytest.mark.parametrize("name,kw", FP8_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(FP8_CASES)])
def test_qkv_fp8_small(name, kw):
    check_qkv_fp8(W(name, **kw))


def test_qkv_fp8_nan_in_v():
    wl = W("fp8long", T=16, valid=[16], H=2, grid=(1, 4, 4))
    x = synth.qkv_host(wl).copy()
    x[0, 5, 2 * 2 * 128 + 9] = 0x7FC0
    ra = check_qkv_fp8(wl, qkv_bits=x)
    assert np.isnan(ra[2]) and not np.isnan(ra[0])


def test_full_fp8long_qkv():
    ra = check_qkv_fp8(synth.workloads()["fp8long"])
    say(f"[full] fp8long amax_qkv {ra.tolist()}")


# ----------------------------------------------------------------------------- one tensor

class TensorCase:
    """One tensor of a synthetic workload on the device: slot s (0 Q, 1 K, 2 V) of the packed
    QKV read in place with the packed row stride, or copied out as a compact [B, T, H, D] tensor."""

    def __init__(self, wl, slot, compact, qkv_bits=None, pb=None):
        import rmsnorm_rope_amd as h3
        self.wl, self.slot, self.compact = wl, slot, compact
        self.pb = pb or DeviceProblem(wl, "cuda", qkv_bits=qkv_bits)
        H, D, T = wl.H, wl.D, wl.T
        if compact:
            self.x = self.pb.qkv[:, :, slot * H * D:(slot + 1) * H * D].contiguous()
            rs, bs, self.xptr = H * D, T * H * D, self.x.data_ptr()
        else:
            self.x = self.pb.qkv
            rs, bs = wl.stride, T * wl.stride
            self.xptr = self.pb.qkv.data_ptr() + 2 * slot * H * D
        self.desc = h3.make_desc(wl.B, T, H, D, wl.grid, wl.n, wl.table_len, self.pb.cos, self.pb.sin,
                                 pos_offset=self.pb.off, valid_len=wl.valid_len, eps=wl.eps,
                                 row_stride=rs, batch_stride=bs)
        self.w = None if slot == 2 else (self.pb.wq if slot == 0 else self.pb.wk)
        self.w_host = None if slot == 2 else (self.pb.wq_host if slot == 0 else self.pb.wk_host)
        self.spec = oracle.Spec(wl.B, T, H, D, wl.grid, wl.n, wl.table_len, *synth.rope_tables(wl.table_len, wl.n),
                                pos_offset=self.pb.off, valid_len=wl.valid_len, eps=wl.eps, row_stride=rs,
                                batch_stride=bs)

    def host_x(self):
        a = self.x.cpu().numpy().view(np.uint16).reshape(-1)
        return a if self.compact else a[self.slot * self.wl.H * self.wl.D:]

    def out(self, dt, layout):
        wl = self.wl
        shape = (wl.B, wl.H, wl.T, wl.D) if layout == 0 else (wl.B, wl.T, wl.H, wl.D)
        from synth.problem import torch_dtype
        return torch.empty(shape, dtype=torch_dtype(dt), device="cuda")


def check_tensor_store(tc, out_dt, layout):
    import rmsnorm_rope_amd as h3
    wl = tc.wl
    say(f"[tensor-store] {wl.name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} in={wl.in_dtype} slot={tc.slot} "
        f"compact={tc.compact} out={out_dt} layout={layout}")
    out = tc.out(out_dt, layout)
    h3.h3_tensor_norm_rope(tc.desc, tc.xptr, wl.in_dtype, tc.w, out, out_dt, layout)
    torch.cuda.synchronize()
    ref = oracle.tensor_norm_rope(tc.spec, tc.host_x(), wl.in_dtype, tc.w_host, out_dt, layout)
    return compare(bits(out), ref, out_dt, f"out slot {tc.slot}")


def check_tensor_fp8(tc, layout, static_descale=None, count=True):
    import rmsnorm_rope_amd as h3
    wl = tc.wl
    say(f"[tensor-fp8] {wl.name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} in={wl.in_dtype} slot={tc.slot} "
        f"compact={tc.compact} layout={layout} static={static_descale}")
    xh = tc.host_x()
    ram = oracle.tensor_amax(tc.spec, xh, wl.in_dtype, tc.w_host)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    h3.h3_tensor_amax(tc.desc, tc.xptr, wl.in_dtype, tc.w, amax)
    torch.cuda.synchronize()
    compare(bits(amax), np.array([ram], np.float32), "f32", "amax")
    if static_descale is None:
        scale, is_ds, use = amax, False, float(ram)
    else:
        scale = torch.tensor([static_descale], dtype=torch.float32, device="cuda")
        is_ds, use = True, static_descale
    codes = tc.out("e4m3", layout)
    ds = torch.empty(1, dtype=torch.float32, device="cuda")
    sat = torch.empty(h3.SAT_WORDS, dtype=torch.int64, device="cuda") if count else None
    h3.h3_tensor_cast_e4m3(tc.desc, tc.xptr, wl.in_dtype, tc.w, scale, is_ds, codes, layout, ds, sat)
    torch.cuda.synchronize()
    rc, rds, rsat = oracle.tensor_cast_e4m3(tc.spec, xh, wl.in_dtype, tc.w_host, use, is_ds, layout)
    compare(bits(ds), np.array([rds], np.float32), "f32", "descale")
    compare(bits(codes), rc, "e4m3", "codes")
    if count:
        got = sat[:3].cpu().numpy().astype(np.uint64).tolist()
        say(f"  clip counts gpu {got} oracle {rsat}")
        assert got == [rsat, 0, 0]
    return rsat


TENSOR_CASES = [
    ("tiles8", dict(B=2, T=150, valid=[150, 61])),
    ("tiny", dict(T=29, valid=[23], grid=(2, 4, 4))),
    ("fp8long", dict(T=90, valid=[83], grid=(1, 9, 10))),
    ("fp8long", dict(T=64, valid=[64], H=3, grid=(1, 8, 8))),
    ("fp8long", dict(T=40, valid=[40], H=6, D=64, n=8, in_dtype="f16", grid=(1, 5, 8))),
]


@pytest.mark.parametrize("slot", [0, 1, 2])
@pytest.mark.parametrize("name,kw", TENSOR_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(TENSOR_CASES)])
def test_tensor_store(name, kw, slot):
    wl = W(name, **kw)
    tc = TensorCase(wl, slot, compact=False)
    for out_dt, layout in (("f32", 0), ("f32", 1), ("f16", 1), ("bf16", 0), ("bf16", 1)):
        check_tensor_store(tc, out_dt, layout)
    check_tensor_store(TensorCase(wl, slot, compact=True), "f16", 1)


@pytest.mark.parametrize("slot", [0, 2])
@pytest.mark.parametrize("name,kw", TENSOR_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(TENSOR_CASES)])
def test_tensor_fp8(name, kw, slot):
    wl = W(name, **kw)
    tc = TensorCase(wl, slot, compact=(slot == 2))
    check_tensor_fp8(tc, 0)
    check_tensor_fp8(tc, 1, static_descale=0.0045)


@pytest.mark.parametrize("bad", [0.0, float("nan"), 1e-30, 2.0 ** 100])
def test_tensor_fp8_special_descales(bad):
    wl = W("fp8long", T=24, valid=[21], H=2, grid=(1, 4, 6))
    check_tensor_fp8(TensorCase(wl, 1, compact=False), 1, static_descale=bad)


def test_tensor_slices_match_fused_on_the_gpu():
    """The per-tensor store over the Q, K and V parts of a packed QKV writes, bit for bit, what the
    fused pass writes (eight tiles, full size, both on the GPU)."""
    import rmsnorm_rope_amd as h3
    wl = synth.workloads()["tiles8"]
    pb = DeviceProblem(wl, "cuda")
    q, k, v = pb.run_store("f32", "f16")
    for slot, ref, dt in ((0, q, "f32"), (1, k, "f16"), (2, v, "f16")):
        tc = TensorCase(wl, slot, compact=False, pb=pb)
        out = tc.out(dt, 0)
        h3.h3_tensor_norm_rope(tc.desc, tc.xptr, wl.in_dtype, tc.w, out, dt, 0)
        torch.cuda.synchronize()
        compare_raw(bits(out), bits(ref), f"slot {slot}")
        del out
    say("[full] tiles8 per-tensor slices match the fused pass")


def test_vae_qk_shape_compact_q_and_k():
    """Q and K as separate compact [2, 1797, 32, 64] f16 tensors into f16 [B, T, H, D], the shape
    the bench times against the thread's isolated Q/K measurement: every output compared."""
    wl = synth.vae_qk_workload()
    pb = DeviceProblem(wl, "cuda")
    for slot in (0, 1):
        check_tensor_store(TensorCase(wl, slot, compact=True, pb=pb), "f16", 1)
    say("[full] vae_qk Q and K match the oracle")


def test_full_fp8long_tensor_v_cast():
    wl = synth.workloads()["fp8long"]
    rsat = check_tensor_fp8(TensorCase(wl, 2, compact=False), 1, static_descale=3.0 / 448)
    say(f"[full] fp8long V per-tensor static cast clip count {rsat}")
    assert rsat > 0


def test_full_fp8long_tensor_k_bthd():
    """The one-tensor FP8 recipe the bench times, at full size: the FP8 long sequence's K heads as a
    compact bf16 [1, 104448, 24, 128] tensor; amax, dynamic cast to [B, T, H, D] codes and the
    16-bit norm + RoPE store, every element against the oracle."""
    wl = synth.workloads()["fp8long"]
    tc = TensorCase(wl, 1, compact=True)
    check_tensor_fp8(tc, 1)
    check_tensor_store(tc, "bf16", 1)
    say("[full] fp8long K heads as one tensor: amax, cast and bf16 store match the oracle")
