"""Host logic of bench.py without a GPU: the PMC traffic summary (counter scaling by the copy
calibration, the kernel-source digest that invalidates it), the interleaved timing's medians, and
the one-GPU guard."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

STORE = "void h3::(anonymous namespace)::qk_kernel<64, 1, 0, 1, 0, 8, 0>(h3::QkParams)"
COPY = "__amd_rocclr_copyBuffer"


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "X", "Counter_Value": value})


def test_pmc_summary_scales_by_the_copy_and_records_the_digest(tmp_path, monkeypatch):
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy_kib = (1 << 31) / 1024.0
    # the store kernel: 750,000 KiB fetched (counter reads half the bytes, like the copy below) and
    # 2,000,000 KiB written per dispatch; a PyTorch kernel in the same run is ignored
    _counters(tmp_path / "pmc_FETCH_SIZE" / "a", [(STORE, 750000.0), (STORE, 750000.0), ("other", 5.0)])
    _counters(tmp_path / "pmc_WRITE_SIZE" / "a", [(STORE, 1999000.0), (STORE, 2001000.0)])
    _counters(tmp_path / "pmccopy_FETCH_SIZE" / "a", [(COPY, copy_kib / 2)])
    _counters(tmp_path / "pmccopy_WRITE_SIZE" / "a", [(COPY, copy_kib)])
    bench.pmc_summary(str(tmp_path))
    kv = dict(ln.strip().split("=", 1) for ln in open(out) if "=" in ln and not ln.startswith("#"))
    assert kv["kernel_sha256_16"] == bench.kernel_digest()
    assert int(kv["dispatches_fetch"]) == 2 and int(kv["dispatches_write"]) == 2
    assert float(kv["fetch_scale"]) == 2.0 and float(kv["write_scale"]) == 1.0
    assert int(kv["hbm_read_bytes_per_launch"]) == 750000 * 2 * 1024
    assert int(kv["hbm_write_bytes_per_launch"]) == 2000000 * 1024
    assert bench.measured_traffic(3583770624) == float(750000 * 2 * 1024 + 2000000 * 1024)
    # a summary taken on other kernel sources is not used
    text = out.read_text().replace(bench.kernel_digest(), "0" * 16)
    out.write_text(text)
    assert bench.measured_traffic(3583770624) is None


def test_measured_traffic_without_a_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic(1) is None


def test_time_interleaved_takes_the_median_of_each_pass(monkeypatch):
    calls = []
    per_call = {"a": iter([3.0, 1.0, 2.0]), "b": iter([10.0, 30.0, 20.0])}

    def fake(fn, steps, warmup, stream):
        name = fn()
        calls.append(name)
        return 0.0, next(per_call[name])

    monkeypatch.setattr(bench, "time_launches", fake)
    t = bench.time_interleaved({"a": lambda: "a", "b": lambda: "b"}, 5, 1, None, rounds=3)
    assert t == {"a": 2.0, "b": 20.0}
    assert calls == ["a", "b", "a", "b", "a", "b"]  # the passes taken in turn, round after round


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_oracle_on_all_cores_matches_one_thread():
    """The CPU baseline's driver: the oracle's token entry on disjoint blocks run by 8 host threads
    at once gives the bits of one thread and of the whole-problem entry (head-major there)."""
    import numpy as np

    import oracle
    import synth
    from synth.problem import oracle_spec
    wl = synth.workloads()["tile"]
    sp = oracle_spec(wl)
    x = synth.qkv_host(wl)
    wq, wk = synth.norm_weights(wl)
    toks = np.arange(wl.T)
    one = oracle.qk_tokens_store(sp, x[0], toks, "f16", wq, wk, threads=1)
    many = oracle.qk_tokens_store(sp, x[0], toks, "f16", wq, wk, threads=8)
    for a, b in zip(one, many):
        assert np.array_equal(a, b)
    q, k, v = oracle.qk_rmsnorm_rope_permute(sp, x, "f16", wq, wk, "f32", "f16")
    for whole, tok in zip((q, k, v), many):
        assert np.array_equal(whole[0].transpose(1, 0, 2), tok)
