"""A seeded stress matrix of small cases (256 by default; --stress-cases N runs N) through the C ABI,
every output bit-exact against the oracle: D in {64, 128} x input f16/bf16 x T in {1, 7, 32, 33,
1797} x H in {1, 2, 16, 24}, item offsets and valid lengths, output dtypes, and row distributions
(normal, x20 outliers, binary16 / bfloat16 subnormal rows, constant rows, one-hot rows, all-zero
rows).  Every fourth case also runs the FP8 amax + cast pair, another fourth the static-scale cast
with V codes and clip counters (descales at a quarter, one and three times the data's own scale),
another fourth a one-tensor pass (random slot, packed or compact input, layout, and store or
dynamic / static cast); every eighth case the Q/K/V FP8 recipe, and another eighth the sage
emission."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from synth.problem import DeviceProblem, oracle_spec
from tests.gpu_util import bits, compare, compare_raw
from tests.test_gpu_tensor import TensorCase, check_tensor_fp8, check_tensor_store

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


def _grid_for(T, rng):
    """A (Gt, Gh, Gw) grid with at least T positions."""
    gw = int(rng.integers(1, 9))
    gh = int(rng.integers(1, 6))
    gt = -(-T // (gh * gw))
    return (gt, gh, gw)


def _case(k):
    rng = np.random.default_rng(9000 + k)
    D = int(rng.choice([64, 128]))
    in_dt = str(rng.choice(["f16", "bf16"]))
    T = int(rng.choice([1, 7, 32, 33, 1797]))
    H = int(rng.choice([1, 2, 16, 24]))
    if T * H > 1797 * 2 and D == 128:  # keep every case small
        T = int(rng.choice([1, 7, 32, 33]))
    B = int(rng.choice([1, 1, 2, 3]))
    n = D // 8 if rng.random() < 0.7 else int(rng.integers(0, D // 6 + 1))
    grid = _grid_for(T, rng)
    gsize = grid[0] * grid[1] * grid[2]
    valid = [int(min(T, gsize) if rng.random() < 0.6 else rng.integers(0, min(T, gsize) + 1)) for _ in range(B)]
    wl = synth.Workload(f"stress{k}", B, grid, T, H, D, n, in_dt, str(rng.choice(["normal", "x2_outliers"])),
                        9000 + k, valid=valid, offset_hw_max=int(rng.choice([0, 0, 5])),
                        eps=float(rng.choice([1e-6, 1e-6, 0.0, 1e-2])))
    dist = str(rng.choice(["plain", "subnormal", "constant", "onehot", "zero"]))
    q_dt, k_dt = [str(x) for x in rng.choice(["f32", "f16", "bf16"], 2)]
    return wl, dist, q_dt, k_dt, rng


def _inputs(wl, dist, rng):
    x = synth.qkv_host(wl).copy()
    if dist == "plain" or wl.T < 2:
        return x
    rows = rng.choice(wl.T, size=max(1, wl.T // 4), replace=False)
    hd3 = 3 * wl.H * wl.D
    if dist == "zero":
        x[:, rows, :hd3] = 0
        return x
    vals = np.zeros((len(rows), hd3), np.float32)
    if dist == "subnormal":
        vals[:] = rng.standard_normal(vals.shape) * (2.0 ** -20 if wl.in_dtype == "f16" else 2.0 ** -130)
    elif dist == "constant":
        vals[:] = float(rng.choice([1.5, -0.75, 3.0]))
    elif dist == "onehot":
        vals[:, int(rng.integers(0, wl.D))::wl.D] = float(rng.choice([2.5, -4.0]))
    enc = (vals.astype(np.float16).view(np.uint16) if wl.in_dtype == "f16"
           else oracle.encode(vals, "bf16").reshape(vals.shape))
    x[:, rows, :hd3] = enc
    return x


def test_stress_matrix(request):
    n_cases = request.config.getoption("--stress-cases")
    import rmsnorm_rope_amd as h3
    counts = {"store": 0, "fp8": 0, "static": 0, "qkv": 0, "tensor": 0, "sage": 0}
    for k in range(n_cases):
        wl, dist, q_dt, k_dt, rng = _case(k)
        tag = (f"case {k}: B={wl.B} T={wl.T} H={wl.H} D={wl.D} n={wl.n} in={wl.in_dtype} {wl.dist}/{dist} "
               f"valid={list(wl.valid_len)} eps={wl.eps} q={q_dt} k={k_dt}")
        print(tag, flush=True)
        x = _inputs(wl, dist, rng)
        pb = DeviceProblem(wl, "cuda", qkv_bits=x)
        sp = oracle_spec(wl)
        q, kk, v = pb.run_store(q_dt, k_dt)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.qk_rmsnorm_rope_permute(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, q_dt, k_dt)
        compare(bits(q), rq, q_dt, f"{tag} Q")
        compare(bits(kk), rk, k_dt, f"{tag} K")
        compare_raw(bits(v), rv, f"{tag} V")
        counts["store"] += 1
        if k % 4 == 0:
            amax = pb.run_amax()
            q8, k8, v8, ds = pb.run_cast(amax)
            torch.cuda.synchronize()
            ra = oracle.qk_amax(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host)
            compare(bits(amax), ra, "f32", f"{tag} amax")
            oq, ok, ov, ods = oracle.qk_cast_e4m3(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, ra)
            compare(bits(ds), ods, "f32", f"{tag} descale")
            compare(bits(q8), oq, "e4m3", f"{tag} Q codes")
            compare(bits(k8), ok, "e4m3", f"{tag} K codes")
            compare_raw(bits(v8), ov, f"{tag} V copy")
            counts["fp8"] += 1
        if k % 4 == 2:  # static descales around the data's own scale, V codes, clip counters
            ra3 = oracle.qkv_amax(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host)
            fac = rng.choice([0.25, 1.0, 3.0], 3)
            ds_h = np.where(np.isfinite(ra3) & (ra3 > 0), ra3 / np.float32(448.0) * fac, 1.0).astype(np.float32)
            q8, k8, v8, sat = pb.run_cast_static(torch.from_numpy(ds_h).cuda(), v_fp8=True)
            torch.cuda.synchronize()
            oq, ok, ov, osat = oracle.qk_cast_e4m3_static(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, ds_h, v_fp8=True)
            compare(bits(q8), oq, "e4m3", f"{tag} static Q codes")
            compare(bits(k8), ok, "e4m3", f"{tag} static K codes")
            compare(bits(v8), ov, "e4m3", f"{tag} static V codes")
            assert np.array_equal(sat[:3].cpu().numpy().astype(np.uint64), osat), (tag, sat[:3].tolist(), osat)
            counts["static"] += 1
        if k % 8 == 3:  # the Q/K/V recipe: three amaxes, then Q, K and V codes
            am3 = torch.empty(3, dtype=torch.float32, device="cuda")
            h3.h3_qkv_amax(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, am3)
            q8, k8, v8 = pb.out("e4m3"), pb.out("e4m3"), pb.out("e4m3")
            ds3 = torch.empty(3, dtype=torch.float32, device="cuda")
            h3.h3_qkv_cast_e4m3(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, am3, q8, k8, v8, ds3)
            torch.cuda.synchronize()
            ra3 = oracle.qkv_amax(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host)
            compare(bits(am3), ra3, "f32", f"{tag} qkv amax")
            oq, ok, ov, ods = oracle.qkv_cast_e4m3(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, ra3)
            compare(bits(ds3), ods, "f32", f"{tag} qkv descales")
            compare(bits(q8), oq, "e4m3", f"{tag} qkv Q codes")
            compare(bits(k8), ok, "e4m3", f"{tag} qkv K codes")
            compare(bits(v8), ov, "e4m3", f"{tag} qkv V codes")
            counts["qkv"] += 1
        if k % 4 == 3:  # one tensor: a random slot, packed or compact, layout and output
            slot = int(rng.integers(0, 3))
            tc = TensorCase(wl, slot, compact=bool(rng.integers(0, 2)), pb=pb)
            layout = int(rng.integers(0, 2))
            if rng.random() < 0.5:
                check_tensor_store(tc, str(rng.choice(["f32", "f16", "bf16"])), layout)
            else:
                sd = None if rng.random() < 0.5 else float(rng.choice([0.0045, 0.01, 0.05]))
                check_tensor_fp8(tc, layout, static_descale=sd)
            counts["tensor"] += 1
        if k % 8 == 1:
            s = float(rng.choice([0.125, 0.0883883, 2.5]))
            sq, sk, sv = pb.run_sage(s)
            torch.cuda.synchronize()
            oq, ok, ov = oracle.qk_sage(sp, x, wl.in_dtype, pb.wq_host, pb.wk_host, s)
            compare(bits(sq), oq, "f32", f"{tag} sage Q")
            compare(bits(sk), ok, "f32", f"{tag} sage K")
            compare(bits(sv), ov, "f16", f"{tag} sage V")
            counts["sage"] += 1
        del pb
    print(f"[stress] {counts}", flush=True)
    assert counts["store"] == n_cases
