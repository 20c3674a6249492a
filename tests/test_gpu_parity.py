"""GPU parity of libh3qk against the CPU oracle, through the C ABI.

Bar: bit-exact Q/K/V, amax, descales and E4M3 codes (the contract in include/h3qk.h has one
result per input); NaN payloads are not part of the contract.  Every comparison reports its ulp
histogram.  Small and ragged cases compare every element; the full-size workloads (one tile,
eight tiles, the full latent, the FP8 long sequence) also compare every element, with the
oracle run over the whole input copied back from the device."""
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


def check_store(wl, q_dt="f32", k_dt="f16", qkv_bits=None, pb=None):
    say(f"[store] {wl.name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} n={wl.n} in={wl.in_dtype} q={q_dt} k={k_dt}")
    pb = pb or DeviceProblem(wl, "cuda", qkv_bits=qkv_bits)
    q, k, v = pb.run_store(q_dt, k_dt)
    torch.cuda.synchronize()
    x = pb.qkv_host()
    rq, rk, rv = oracle.qk_rmsnorm_rope_permute(oracle_spec(wl), x, wl.in_dtype, pb.wq_host, pb.wk_host, q_dt, k_dt)
    hq = compare(bits(q), rq, q_dt, "Q")
    hk = compare(bits(k), rk, k_dt, "K")
    compare_raw(bits(v), rv, "V")
    return hq, hk


# ----------------------------------------------------------------------------- small / ragged

SMALL = [
    ("tiny", {}),
    ("tiny", dict(T=1, grid=(1, 1, 1))),
    ("tiny", dict(T=7, grid=(1, 1, 7))),
    ("tiny", dict(T=9, grid=(1, 3, 3))),
    ("tiny", dict(T=33, grid=(3, 3, 4))),
    ("tiny", dict(H=1)),
    ("tiny", dict(H=3, T=45, grid=(5, 3, 3))),
    ("tiny", dict(B=3, T=40, grid=(2, 4, 5), valid=[40, 0, 13], offset_hw_max=9)),
    ("tiny", dict(H=24, T=20, grid=(1, 4, 5), in_dtype="bf16")),
    ("tiny", dict(D=128, n=16, T=24, grid=(2, 3, 4), in_dtype="bf16")),
    ("tiny", dict(D=128, n=16, H=5, T=17, grid=(1, 1, 17))),
    ("tiny", dict(n=0)),
    ("tiny", dict(n=5)),
    ("tiny", dict(n=10)),
    ("tiny", dict(D=128, n=21, T=16, grid=(2, 2, 4))),
    ("tiny", dict(eps=0.0)),
    ("tiny", dict(eps=1e-2)),
    ("tiny", dict(row_stride=3 * 2 * 64 + 24)),
    ("tile", dict(T=3000, grid=(31, 16, 16), valid=[2999])),
    ("tiles8", dict(T=257, B=5, valid=[257, 256, 1, 0, 100])),
    ("tiny", dict(B=64, T=9, grid=(1, 3, 3), valid=[i % 10 for i in range(64)], offset_hw_max=5)),  # max batch
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_store_small(name, kw):
    check_store(W(name, **kw))


@pytest.mark.parametrize("q_dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k_dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("in_dt", ["f16", "bf16"])
def test_store_dtype_matrix(q_dt, k_dt, in_dt):
    check_store(W("tiny", T=40, grid=(2, 4, 5), B=2, valid=[40, 31], in_dtype=in_dt), q_dt, k_dt)
    check_store(W("tiny", T=12, grid=(1, 3, 4), B=2, valid=[12, 5], D=128, n=16, in_dtype=in_dt), q_dt, k_dt)


def test_store_max_row_stride():
    """The largest row stride the ABI accepts (2^26 elements): token 8 of a group starts 7 * 2^27
    bytes past the group's first token, the far end of the 32-bit lane offsets."""
    wl = W("tiny", T=9, grid=(1, 3, 3), row_stride=1 << 26)
    x = np.zeros((1, 9, 1 << 26), np.uint16)
    x[:, :, :3 * wl.H * wl.D] = synth.qkv_host(W("tiny", T=9, grid=(1, 3, 3)))
    check_store(wl, qkv_bits=x)
    check_fp8(dataclasses.replace(wl, fp8=True), qkv_bits=x)


def _tables_at_4_bytes(pb):
    """Re-point pb's descriptor at copies of its rotary tables that start 4 bytes past an 8-byte
    boundary (the kernels then read the entries one by one instead of in pairs)."""
    import rmsnorm_rope_amd as h3
    wl = pb.wl
    keep = []
    for t in (pb.cos, pb.sin):
        buf = torch.empty(t.numel() + 2, dtype=torch.float32, device="cuda")
        view = buf[1:1 + t.numel()]
        view.copy_(t.reshape(-1))
        assert view.data_ptr() % 8 == 4
        keep.append((buf, view))
    pb.tables_at_4 = keep
    pb.desc = h3.make_desc(wl.B, wl.T, wl.H, wl.D, wl.grid, wl.n, wl.table_len, keep[0][1], keep[1][1],
                           pos_offset=pb.off, valid_len=wl.valid_len, eps=wl.eps,
                           row_stride=wl.stride, batch_stride=wl.T * wl.stride)
    return pb


@pytest.mark.parametrize("name,kw", [("tiles8", dict(B=2, T=150, valid=[150, 61])),
                                     ("fp8long", dict(T=90, valid=[83], grid=(1, 9, 10), D=64, n=8, in_dtype="f16"))])
def test_tables_4_byte_aligned(name, kw):
    """Rotary tables that are 4- but not 8-byte aligned (the ABI's minimum): the same bits."""
    wl = W(name, **kw)
    check_store(wl, pb=_tables_at_4_bytes(DeviceProblem(wl, "cuda")))
    wf = dataclasses.replace(wl, fp8=True)
    check_fp8(wf, pb=_tables_at_4_bytes(DeviceProblem(wf, "cuda")))


def test_store_padded_batch_stride():
    wl = W("tiny", B=2, T=16, grid=(1, 4, 4))
    pb = DeviceProblem(wl, "cuda")
    import rmsnorm_rope_amd as h3
    # re-lay the input with a wider batch stride (extra 3 tokens of junk between items)
    x = pb.qkv_host()
    wide = np.full((2, 19, wl.stride), 0x7E00, np.uint16)   # NaN junk must never be read
    wide[:, :16] = x
    pb.qkv = torch.from_numpy(wide.view(np.int16)).cuda()
    pb.desc = h3.make_desc(wl.B, wl.T, wl.H, wl.D, wl.grid, wl.n, wl.table_len, pb.cos, pb.sin,
                           row_stride=wl.stride, batch_stride=19 * wl.stride)
    q, k, v = pb.run_store()
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qk_rmsnorm_rope_permute(oracle_spec(wl), x, "f16", pb.wq_host, pb.wk_host)
    compare(bits(q), rq, "f32", "Q")
    compare(bits(k), rk, "f16", "K")
    compare_raw(bits(v), rv, "V")


# ----------------------------------------------------------------------------- crafted inputs

def _crafted(wl, fill):
    x = np.zeros((wl.B, wl.T, wl.stride), np.float32)
    fill(x)
    if wl.in_dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return oracle.encode(x, "bf16").reshape(x.shape)


@pytest.mark.parametrize("D", [64, 128])
def test_reduction_tree_rows(D):
    """Rows whose sum of squares depends on the reduction order (2^24 plus ones placed so that
    other trees give other bits): the GPU must take the contract's halving tree."""
    wl = W("tiny", D=D, n=D // 8, T=8, grid=(1, 2, 4), H=2)

    def fill(x):
        for s in range(3):
            for h in range(2):
                base = (s * 2 + h) * D
                x[:, :, base] = 4096.0
                x[:, :, base + D // 2:base + D] = 1.0
                x[:, 1::2, base + 1:base + D // 2] = 1.0
    check_store(wl, qkv_bits=_crafted(wl, fill))


def test_special_rows():
    """Constant, one-hot, tiny (binary16 subnormal), large, zero, +-inf and NaN rows."""
    wl = W("tiny", T=16, grid=(2, 2, 4), H=4)
    rng = np.random.default_rng(0)

    def fill(x):
        D = 64
        x[:, :, :] = rng.standard_normal(x.shape)
        x[:, 0, :] = 1.5                                   # constant
        x[:, 1, :] = 0.0
        x[:, 1, 5::64] = -2.5                              # one-hot per head
        x[:, 2, :] = rng.standard_normal(x.shape[-1]) * 2.0 ** -20  # f16 subnormals
        x[:, 3, :] = rng.standard_normal(x.shape[-1]) * 1e4  # towards the f16 range
        x[:, 4, :] = 0.0                                   # zero rows
        x[:, 5, 3] = np.inf
        x[:, 6, 70] = -np.inf
        x[:, 7, 200] = np.nan
        x[:, 8, :] = 6e-8                                  # smallest f16 subnormal
    check_store(wl, qkv_bits=_crafted(wl, fill))
    check_store(wl, "bf16", "bf16", qkv_bits=_crafted(wl, fill))
    # eps = 0: a zero row has 1/rms = 1/0 = inf and every y' = 0 * inf = NaN, on both sides
    check_store(dataclasses.replace(wl, eps=0.0), qkv_bits=_crafted(wl, fill))


def test_special_rows_fp8_and_sage():
    """The same special rows through the cast (NaN rows, inf, saturation) and the sage emission,
    with and without eps."""
    import rmsnorm_rope_amd as h3
    wl = W("fp8long", T=16, valid=[14], H=2, grid=(1, 4, 4))
    rng = np.random.default_rng(1)

    def fill(x):
        x[:, :, :] = rng.standard_normal(x.shape)
        x[:, 1, :] = 0.0
        x[:, 2, :] = rng.standard_normal(x.shape[-1]) * 2.0 ** -130   # bf16 subnormals
        x[:, 3, :] = rng.standard_normal(x.shape[-1]) * 1e30
        x[:, 4, 7] = np.inf
        x[:, 5, 300] = np.nan
        x[:, 6, :] = 0.0
        x[:, 6, 9::128] = 3.0
    for eps in (1e-6, 0.0):
        w = dataclasses.replace(wl, eps=eps)
        check_fp8(w, qkv_bits=_crafted(w, fill))
        pb = DeviceProblem(w, "cuda", qkv_bits=_crafted(w, fill))
        q, k, v = pb.run_sage(0.3)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.qk_sage(oracle_spec(w), pb.qkv_host(), w.in_dtype, pb.wq_host, pb.wk_host, 0.3)
        compare(bits(q), rq, "f32", "sage Q")
        compare(bits(k), rk, "f32", "sage K")
        compare(bits(v), rv, "f16", "sage V")


# ----------------------------------------------------------------------------- FP8 amax + cast

def check_fp8(wl, qkv_bits=None, amax_override=None, pb=None):
    say(f"[fp8] {wl.name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} in={wl.in_dtype} valid={list(wl.valid_len)[:4]}")
    pb = pb or DeviceProblem(wl, "cuda", qkv_bits=qkv_bits)
    amax = pb.run_amax()
    if amax_override is not None:
        amax = torch.tensor(amax_override, dtype=torch.float32, device="cuda")
    q8, k8, v8, ds = pb.run_cast(amax)
    torch.cuda.synchronize()
    sp = oracle_spec(wl)
    x = pb.qkv_host()
    ra = oracle.qk_amax(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host)
    if amax_override is None:
        compare(bits(amax), ra, "f32", "amax")
        use = ra
    else:
        use = np.asarray(amax_override, np.float32)
    rq, rk, rv, rds = oracle.qk_cast_e4m3(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, use)
    compare(bits(ds), rds, "f32", "descale")
    compare(bits(q8), rq, "e4m3", "Q codes")
    compare(bits(k8), rk, "e4m3", "K codes")
    compare_raw(bits(v8), rv, "V")
    return ra


FP8_SMALL = [
    ("fp8long", dict(T=203, valid=[190])),
    ("fp8long", dict(T=64, valid=[64], H=3)),
    ("fp8long", dict(B=3, T=50, valid=[50, 0, 17], offset_hw_max=0)),
    ("fp8long", dict(T=31, valid=[0])),                      # nothing valid: amax 0, descale 1
    ("fp8long", dict(T=40, valid=[40], D=64, n=8, in_dtype="f16")),
    ("tiny", dict(fp8=True, in_dtype="bf16", valid=[20])),
]


@pytest.mark.parametrize("name,kw", FP8_SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(FP8_SMALL)])
def test_fp8_small(name, kw):
    check_fp8(W(name, **kw))


def test_fp8_static_scale_saturates():
    """A caller-provided amax smaller than the data (a static scale) drives codes past 448:
    they saturate to +-448 on both sides."""
    wl = W("fp8long", T=48, valid=[48], H=2)
    check_fp8(wl, amax_override=[0.5, 2.0])


def test_fp8_zero_and_nan():
    wl = W("fp8long", T=16, valid=[16], H=2, grid=(1, 4, 4))
    check_fp8(wl, qkv_bits=_crafted(wl, lambda x: None))
    def nan_fill(x):
        x[:] = np.random.default_rng(1).standard_normal(x.shape)
        x[0, 3, 5] = np.nan
    ra = check_fp8(wl, qkv_bits=_crafted(wl, nan_fill))
    assert np.isnan(ra[0]) and not np.isnan(ra[1])


def test_fp8_subnormal_amax():
    """Q weights of 2^-130 make every Q output y' (and so its amax) a binary32 subnormal, and the
    descale amax / 448 a subnormal too, below the cast's fast range: the magnitude maximum must
    compare subnormals as they are, on the fused pass, on the Q/K/V pass and on the one-tensor
    pass, and the cast takes its exact path."""
    import rmsnorm_rope_amd as h3
    wl = W("fp8long", T=24, valid=[21], H=2, grid=(1, 4, 6))
    pb = DeviceProblem(wl, "cuda")
    pb.wq_host = (pb.wq_host * np.float32(2.0 ** -130)).astype(np.float32)
    pb.wq = torch.from_numpy(pb.wq_host).to("cuda")
    sp, x = oracle_spec(wl), pb.qkv_host()
    ra = oracle.qk_amax(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host)
    assert 0.0 < ra[0] < np.float32(2.0 ** -126) and ra[1] > 1.0, ra
    amax = pb.run_amax()
    q8, k8, v8, ds = pb.run_cast(amax)
    am3 = torch.empty(3, dtype=torch.float32, device="cuda")
    h3.h3_qkv_amax(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, am3)
    torch.cuda.synchronize()
    compare(bits(amax), ra, "f32", "amax")
    compare(bits(am3)[:2], ra, "f32", "Q/K/V pass amax of Q and K")
    rq, rk, rv, rds = oracle.qk_cast_e4m3(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, ra)
    assert 0.0 < rds[0] < np.float32(2.0 ** -126), rds
    compare(bits(ds), rds, "f32", "descale")
    compare(bits(q8), rq, "e4m3", "Q codes")
    compare(bits(k8), rk, "e4m3", "K codes")
    compare_raw(bits(v8), rv, "V")
    # the Q heads alone as one tensor
    H, D = wl.H, wl.D
    qx = pb.qkv[:, :, :H * D].contiguous()
    desc = h3.make_desc(wl.B, wl.T, H, D, wl.grid, wl.n, wl.table_len, pb.cos, pb.sin, pos_offset=pb.off,
                        valid_len=wl.valid_len, eps=wl.eps, row_stride=H * D, batch_stride=wl.T * H * D)
    ta = torch.empty(1, dtype=torch.float32, device="cuda")
    h3.h3_tensor_amax(desc, qx, wl.in_dtype, pb.wq, ta)
    torch.cuda.synchronize()
    tsp = oracle.spec_from_workload(wl, row_stride=H * D, batch_stride=wl.T * H * D)
    rt = oracle.tensor_amax(tsp, bits(qx), wl.in_dtype, pb.wq_host)
    assert rt.view(np.uint32) == ra[:1].view(np.uint32)[0]
    compare(bits(ta), np.array([rt], np.float32), "f32", "one-tensor amax of Q")


# ----------------------------------------------------------------------------- full-size workloads

def _full_store(name):
    wl = synth.workloads()[name]
    pb = DeviceProblem(wl, "cuda")
    say(f"[full] {name}: generated on device, running kernel")
    hq, hk = check_store(wl, pb=pb)
    say(f"[full] {name}: Q ulp histogram {hq}, K {hk}")


def test_full_tile():
    _full_store("tile")


def test_full_tiles8():
    _full_store("tiles8")


def test_full_latent():
    _full_store("latent")


def test_full_fp8long():
    wl = synth.workloads()["fp8long"]
    ra = check_fp8(wl)
    say(f"[full] fp8long amax {ra.tolist()}")


def test_full_fp8long_store_f32():
    """The store pass on the full long sequence with binary32 Q and K (whole-line binary32 rows at
    D = 128), every output element against the oracle."""
    wl = synth.workloads()["fp8long"]
    pb = DeviceProblem(wl, "cuda")
    hq, hk = check_store(wl, "f32", "f32", pb=pb)
    say(f"[full] fp8long store f32/f32: Q ulp histogram {hq}, K {hk}")


# ----------------------------------------------------------------------------- determinism / streams

def test_repeat_and_side_stream():
    wl = W("tiles8", T=400, B=2, valid=[400, 333])
    pb = DeviceProblem(wl, "cuda")
    a = [bits(t) for t in pb.run_store()]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = pb.run_store(stream=s)
    s.synchronize()
    b = [bits(t) for t in outs]
    for u, w in zip(a, b):
        compare_raw(u, w, "repeat")
    a1 = bits(pb.run_amax())
    a2 = bits(pb.run_amax())
    compare_raw(a1, a2, "amax repeat")


def test_generator_on_device_matches_host():
    wl = synth.workloads()["tile"]
    dev = synth.qkv_device(wl, "cuda")[0, 1000:1100].cpu().numpy().view(np.uint16)
    host = synth.qkv_host(wl, np.arange(1000, 1100))
    assert np.array_equal(dev, host)

