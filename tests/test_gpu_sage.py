"""GPU parity of the sage emission (h3_qk_rmsnorm_rope_permute_sage: F32 Q, F32 K * kv_scale,
F16 V * kv_scale, head-major) against the CPU oracle through the C ABI: bit-exact on ragged,
padded and batched cases, f16 and bf16 inputs, D = 64 and 128, and the full one-tile and
eight-tile workloads."""
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


def W(name, **kw):
    return dataclasses.replace(synth.workloads()[name], **kw)


def check_sage(wl, s, pb=None):
    print(f"[sage] {wl.name} B={wl.B} T={wl.T} H={wl.H} D={wl.D} in={wl.in_dtype} kv_scale={s}", flush=True)
    pb = pb or DeviceProblem(wl, "cuda")
    q, k, v = pb.run_sage(s)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qk_sage(oracle_spec(wl), pb.qkv_host(), wl.in_dtype, pb.wq_host, pb.wk_host, s)
    hq = compare(bits(q), rq, "f32", "Q")
    hk = compare(bits(k), rk, "f32", "K")
    compare(bits(v), rv, "f16", "V")
    return hq, hk


CASES = [
    ("tiny", {}),
    ("tile", dict(T=1000, grid=(4, 16, 16), valid=[997])),
    ("tiles8", dict(B=3, T=333, valid=[333, 0, 200])),
    ("fp8long", dict(T=90, valid=[83], grid=(1, 9, 10), fp8=False, q_dtype="f32", k_dtype="f16")),
    ("tiny", dict(in_dtype="bf16", H=3)),
]


@pytest.mark.parametrize("s", [1.0, 0.125, 0.08838834764831845, 7.3])
@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_sage_small(name, kw, s):
    check_sage(W(name, **kw), s)


@pytest.mark.parametrize("name", ["tile", "tiles8"])
def test_sage_full(name):
    hq, hk = check_sage(synth.workloads()[name], 0.125)
    print(f"[full] sage {name}: Q {hq}, K {hk}", flush=True)
