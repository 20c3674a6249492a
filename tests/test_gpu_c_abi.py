"""libh3qk driven from a plain C program (tests/c/e2e_gpu.c): HIP runtime buffers, the fused store,
the FP8 amax + cast pair and the static cast with V codes and clip counters on three ragged
padded problems, every output compared bit for bit with the C oracle, and a rejected call.  No
Python or PyTorch in that process: the boundary is usable as a C library on its own."""
import subprocess

import pytest

from tests.gpu_util import build_c_e2e

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    yield


def test_c_program_end_to_end(tmp_path):
    exe = build_c_e2e(tmp_path)
    print(f"[c-abi] running {exe}", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "all outputs bit-identical to the oracle" in r.stdout
    assert r.stdout.count("ok ") >= 3 * 13
