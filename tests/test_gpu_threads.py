"""Host threads calling the C ABI at once, each on its own stream: the lazily filled device caches
(device attributes, occupancy of the persistent amax kernels) and the per-thread error text must
hold up.  Every thread's outputs must equal, bit for bit, those of the same calls made one at a
time, and a thread whose calls are rejected must read its own error text while the others run."""
import dataclasses
import threading

import pytest

import synth
from synth.problem import DeviceProblem
from tests.gpu_util import bits, compare_raw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROUNDS = 12


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    torch.cuda.set_device(0)
    yield


def _problems():
    base = synth.workloads()
    return [
        DeviceProblem(dataclasses.replace(base["fp8long"], T=403, valid=[390], seed=7001), "cuda"),
        DeviceProblem(dataclasses.replace(base["tiles8"], B=2, T=777, valid=[777, 300], seed=7002), "cuda"),
        DeviceProblem(dataclasses.replace(base["fp8long"], T=256, valid=[256], H=5, seed=7003), "cuda"),
        DeviceProblem(dataclasses.replace(base["tile"], T=1000, valid=[999], seed=7004), "cuda"),
    ]


def _run(pb, stream, outs=None):
    """Store, amax and cast of one problem on `stream`; returns the output tensors."""
    import rmsnorm_rope_amd as h3
    if outs is None:
        outs = {"store": (pb.out("f32"), pb.out("f16"), pb.out(pb.in_dt)),
                "amax": torch.empty(2, dtype=torch.float32, device="cuda"),
                "cast": (pb.out("e4m3"), pb.out("e4m3"), pb.out(pb.in_dt),
                         torch.empty(2, dtype=torch.float32, device="cuda"))}
    pb.run_store("f32", "f16", outs=outs["store"], stream=stream)
    pb.run_amax(outs["amax"], stream=stream)
    pb.run_cast(outs["amax"], outs=outs["cast"], stream=stream)
    return outs


def _snapshot(outs):
    return [bits(t).copy() for v in outs.values() for t in (v if isinstance(v, tuple) else (v,))]


def test_concurrent_threads_match_serial_calls():
    import rmsnorm_rope_amd as h3
    pbs = _problems()
    ref = []
    for pb in pbs:
        o = _run(pb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ref.append(_snapshot(o))
    streams = [torch.cuda.Stream() for _ in pbs]  # default priority
    outs = [None] * len(pbs)
    errors = [None] * len(pbs)
    rejected = []
    start = threading.Barrier(len(pbs) + 1)

    def worker(k):
        try:
            torch.cuda.set_device(0)
            start.wait()
            o = None
            for _ in range(ROUNDS):
                o = _run(pbs[k], streams[k].cuda_stream, o)
            streams[k].synchronize()
            outs[k] = o
        except BaseException as e:  # reported by the main thread
            errors[k] = e

    def rejecter():
        # a descriptor with an unsupported head size, over and over: each call fails on the host
        # and this thread must read its own message every time
        bad = type(pbs[0].desc).from_buffer_copy(pbs[0].desc)
        bad.D = 96
        amax = torch.empty(2, dtype=torch.float32, device="cuda")
        start.wait()
        for _ in range(200):
            try:
                h3.h3_qk_amax(bad, pbs[0].qkv, pbs[0].in_dt, pbs[0].wq, pbs[0].wk, amax,
                              stream=streams[0].cuda_stream)
                rejected.append("accepted")
            except h3.H3Error as e:
                rejected.append(str(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(pbs))]
    threads.append(threading.Thread(target=rejecter))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
        assert not t.is_alive(), "a worker thread did not finish"
    for k, e in enumerate(errors):
        assert e is None, f"thread {k}: {e!r}"
    for k, o in enumerate(outs):
        got = _snapshot(o)
        assert len(got) == len(ref[k])
        for i, (a, b) in enumerate(zip(got, ref[k])):
            compare_raw(a, b, f"thread {k} output {i}")
    assert len(rejected) == 200
    assert all("head dim D must be 64 or 128" in r for r in rejected), set(rejected)
    print(f"[threads] {len(pbs)} threads x {ROUNDS} rounds bit-identical to serial calls; "
          f"200 rejected calls each saw its own error: {rejected[0]}", flush=True)
