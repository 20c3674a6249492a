"""SwiGLU (h3_swiglu, through the C ABI) against the CPU oracle for every (gate, up) pair of 16-bit
values: 2^32 pairs per dtype, f16 and bf16, so the kernel's binary32 fast path and its decision to
fall back to binary64 are checked on the whole input domain.  The op is [OMNI-6607]'s SwiGLU
(vllm-omni PR #6607, "Operations" table, SwiGLU row: the gate's silu times the up half, taken on the
FP16 output of the w1 projection), computed as silu(g) * u in binary64 and rounded once to the
output dtype; NaN outputs match any NaN (payloads are not part of the contract).

Each call covers 4096 gate values (one per row, repeated across the row's F = 65536 gate columns)
against all 65536 up values; the oracle runs on the host threads at the same time."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import bits, compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROWS = 4096          # gate values per call
F = 1 << 16          # every up value
CALLS_PER_TEST = 4   # 4 calls x 4096 gate values = a quarter of the gate values per test


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    torch.cuda.set_device(0)
    yield


def _threads():
    import os
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


@pytest.mark.parametrize("quarter", range(4))
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_swiglu_every_input_pair(dt, quarter):
    import rmsnorm_rope_amd as h3
    up = np.arange(F, dtype=np.uint32).astype(np.uint16)
    x_host = np.empty((ROWS, 2 * F), np.uint16)
    x_host[:, F:] = up[None, :]
    x_dev = torch.empty((ROWS, 2 * F), dtype=torch.int16, device="cuda")
    y_dev = torch.empty((ROWS, F), dtype=torch.int16, device="cuda")
    nt = _threads()
    hist_total = {0: 0, 1: 0, ">1": 0}
    for c in range(CALLS_PER_TEST):
        g0 = (quarter * CALLS_PER_TEST + c) * ROWS
        gates = np.arange(g0, g0 + ROWS, dtype=np.uint32).astype(np.uint16)
        x_host[:, :F] = gates[:, None]
        x_dev.copy_(torch.from_numpy(x_host.view(np.int16)))
        h3.h3_swiglu(x_dev, dt, y_dev, ROWS, F)
        torch.cuda.synchronize()
        ref = oracle.swiglu(x_host, dt, threads=nt)
        got = bits(y_dev)
        if np.array_equal(got, ref):
            hist = {0: got.size, 1: 0, ">1": 0}
        else:  # NaN payloads may differ; anything else fails with the ulp histogram
            hist = compare(got, ref, dt, f"swiglu {dt} gates {g0:#06x}..{g0 + ROWS - 1:#06x}")
        for k in hist_total:
            hist_total[k] += hist[k]
    print(f"[swiglu {dt}] gate values {quarter * CALLS_PER_TEST * ROWS:#06x}.."
          f"{(quarter + 1) * CALLS_PER_TEST * ROWS - 1:#06x} x every up value: ulp histogram {hist_total}", flush=True)
