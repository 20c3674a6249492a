"""Benchmark of libh3qk on one MI355X.

One step = one pass of the fused RMSNorm + 3-axis RoPE + head-major permute over the full-latent
workload (token grid 62x48x84, T = 249,984, H = 16, D = 64, fp16 fused QKV [1, 249984, 3072] ->
Q fp32, K/V fp16 head-major), inputs resident in HBM, launched through the C ABI on torch's
current stream.  Prints one JSON line: throughput in algorithmic GB/s (read every input element
once, write every output element once), tokens/ms, the roofline fraction of the fused kernel
(HIP events on the launch stream around the timed region), the FP8 long-sequence recipe (the amax
pass then the cast pass, and each alone) under "fp8_pair", and the CPU oracle timed on one host
thread and on all of them.  --extra adds the one-tile, eight-tile, static-scale, sage, one-tensor
and decoder-block passes under "extra".
"""
import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused QK-norm+RoPE+permute GB/s and tokens/ms; % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_latent.txt")
KERNEL_SRCS = [os.path.join(ROOT, "rmsnorm_rope_amd", "csrc", f) for f in ("h3qk_kernels.hip", "h3qk_device.h",
                                                                       "h3qk_internal.h")]


def kernel_digest() -> str:
    """Digest of the sources the fused kernels are built from (kernel file and device helpers)."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_alg):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, when it was taken on the
    current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for ln in open(TRAFFIC_FILE):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sha256_16") != kernel_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_launches(launch, steps, warmup, stream):
    """Run `launch` warmup times untimed, then `steps` times back to back between two HIP events
    recorded on `stream` (synchronised on both sides).  Returns (total ms of the timed region,
    average ms per launch = total / steps).  No event sits between the timed launches, so the
    average is the launch-to-launch time of a steady stream of calls."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        launch()
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    return total, total / steps


def time_interleaved(launches, steps, warmup, stream, rounds=3):
    """Time each of several passes (name -> launch) with time_launches, the passes taken in turn
    and the whole sequence repeated `rounds` times; returns name -> median ms per launch.  The
    part's clock drifts under sustained load, so passes compared with one another are timed
    alternately rather than one after the other."""
    per = {name: [] for name in launches}
    for _ in range(rounds):
        for name, fn in launches.items():
            per[name].append(time_launches(fn, steps, warmup, stream)[1])
    return {name: sorted(v)[len(v) // 2] for name, v in per.items()}


def time_graph(launch, calls, replays, warmup=2):
    """Capture `calls` back-to-back invocations of `launch` (which must take torch's current
    stream at call time) in one HIP graph, replay it `warmup` times untimed, then `replays` times
    between two events; returns ms per invocation."""
    import torch
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()  # first-call work (device queries) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            launch()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(replays):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (replays * calls)


def host_cpu() -> str:
    """The host CPU model and the number of CPUs this process may use."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return f"{model}, {n} CPUs available to the process"


def host_threads() -> int:
    """Host threads for the all-cores oracle run: the CPUs this process may use, at most 16 (one
    GPU's share of its host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def cpu_baseline(pb, budget_s=10.0):
    """The oracle (plain C, unchanged) on the same workload, as its token entry point
    h3ref_qk_tokens_ex run on one host thread and on all of them (disjoint contiguous token blocks,
    one per thread: rows are independent, so the outputs are the same bits).  The one-thread run
    takes a prefix of the tokens sized by a short calibration to about budget_s seconds; the
    all-cores run takes the whole workload, repeated until about budget_s seconds have been spent."""
    import numpy as np

    import oracle
    from synth.problem import algorithmic_bytes, oracle_spec
    wl = pb.wl
    assert wl.B == 1
    x = pb.qkv_host()[0]
    sp = oracle_spec(wl)
    oracle.lib()

    def run(ts, threads):
        t = time.perf_counter()
        oracle.qk_tokens_store(sp, x[:ts], np.arange(ts), wl.in_dtype, pb.wq_host, pb.wk_host, "f32", "f16",
                               threads=threads)
        return time.perf_counter() - t

    def timed(ts, threads):
        runs, total = 0, 0.0
        while runs == 0 or total < budget_s * 0.8:
            total += run(ts, threads)
            runs += 1
        spent = total / runs
        sub = dataclasses.replace(wl, T=ts, valid=[ts])
        return spent, runs, algorithmic_bytes(sub, "store")

    ts = min(wl.T, 2048)
    dt = run(ts, 1)
    tok1 = min(wl.T, max(ts, int(ts * budget_s / max(dt, 1e-3))))
    s1, r1, b1 = timed(tok1, 1)
    nt = host_threads()
    sn, rn, bn = timed(wl.T, nt)
    what = f"tokens of the {wl.name} workload (all {wl.H} heads, Q f32, K/V f16, token-major outputs)"
    return {"value": round(bn / sn / 1e9, 3), "unit": "GB/s", "cores": nt, "kind": "oracle",
            "tokens_per_ms": round(wl.T / sn / 1e3, 2), "seconds": round(sn, 3), "runs": rn, "host": host_cpu(),
            "sample": f"all {wl.T} {what}, {nt} host threads on disjoint token blocks, each running the C "
                      f"oracle's token entry point",
            "single_thread": {"value": round(b1 / s1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "tokens_per_ms": round(tok1 / s1 / 1e3, 2), "seconds": round(s1, 2), "runs": r1,
                              "sample": f"first {tok1} of {wl.T} {what}, one host thread"}}


def bench_store(wl, steps, warmup, rotate=1):
    import torch

    from synth.problem import DeviceProblem, algorithmic_bytes
    pbs = [DeviceProblem(wl, "cuda") for _ in range(rotate)]
    outs = [(pb.out("f32"), pb.out("f16"), pb.out(wl.in_dtype)) for pb in pbs]
    stream = torch.cuda.current_stream()
    it = [0]

    def launch():
        j = it[0] % rotate
        it[0] += 1
        pbs[j].run_store("f32", "f16", outs=outs[j], stream=stream.cuda_stream)

    total, per = time_launches(launch, steps, warmup, stream)
    nbytes = algorithmic_bytes(wl, "store")
    return pbs[0], {"ms_per_step": total / steps, "kernel_ms": per, "bytes": nbytes}


def bench_store_dtypes(wl, steps, warmup, combos=(("bf16", "bf16"), ("f32", "bf16"), ("f32", "f32"))):
    """The store pass on one workload for several (Q, K) output dtypes (V keeps the input dtype),
    timed in turn; returns one entry per combination."""
    import torch

    from synth.problem import DeviceProblem, algorithmic_bytes
    pb = DeviceProblem(wl, "cuda")
    stream = torch.cuda.current_stream()
    outs = {c: (pb.out(c[0]), pb.out(c[1]), pb.out(wl.in_dtype)) for c in combos}
    launches = {f"{q}/{k}": (lambda c=(q, k): pb.run_store(c[0], c[1], outs=outs[c], stream=stream.cuda_stream))
                for q, k in combos}
    per = time_interleaved(launches, steps, warmup, stream)
    res = {}
    for q, k in combos:
        ms, nbytes = per[f"{q}/{k}"], algorithmic_bytes(wl, "store", q, k)
        res[f"q_{q}_k_{k}"] = {"us_per_call": round(ms * 1e3, 2), "GBs": round(nbytes / ms / 1e6, 1),
                               "frac_of_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": nbytes}
    return res


def bench_fp8(wl, steps, warmup):
    import torch

    from synth.problem import DeviceProblem, algorithmic_bytes
    pb = DeviceProblem(wl, "cuda")
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    outs = (pb.out("e4m3"), pb.out("e4m3"), pb.out(wl.in_dtype), torch.empty(2, dtype=torch.float32, device="cuda"))
    stream = torch.cuda.current_stream()
    ba, bc = algorithmic_bytes(wl, "amax"), algorithmic_bytes(wl, "cast")
    # static descales (no amax pass) with V cast and clip counters: descales at the data's own
    # amax / 448 (a table calibrated on like data: nothing clips), and at about two standard
    # deviations (a few per cent of every tensor saturates: every wave counts)
    import rmsnorm_rope_amd as h3
    pb.run_amax(amax)
    vdt = torch.bfloat16 if wl.in_dtype == "bf16" else torch.float16
    vmax = float(pb.qkv.view(vdt)[..., 2 * wl.H * wl.D:3 * wl.H * wl.D].abs().amax().item())
    cal = torch.cat([amax / 448.0, torch.tensor([vmax / 448.0], device="cuda")]).float().contiguous()
    clip = torch.tensor([0.0045, 0.005, 0.0046], dtype=torch.float32, device="cuda")
    souts = (pb.out("e4m3"), pb.out("e4m3"), pb.out("e4m3"), torch.empty(h3.SAT_WORDS, dtype=torch.int64, device="cuda"))
    bs = algorithmic_bytes(wl, "cast_v8")
    # dynamic recipe with V cast: amax of Q, K and V in one pass, then the cast with V codes
    am3 = torch.empty(3, dtype=torch.float32, device="cuda")
    ds3 = torch.empty(3, dtype=torch.float32, device="cuda")
    vo = pb.out("e4m3")
    sid = stream.cuda_stream
    # the dynamic pair as a caller runs it, amax then cast back to back on the same input, over
    # two input sets taken in turn (each amax pass starts on lines no earlier pass left in cache)
    pb2 = DeviceProblem(wl, "cuda")
    amax2 = torch.empty(2, dtype=torch.float32, device="cuda")
    outs2 = (pb2.out("e4m3"), pb2.out("e4m3"), pb2.out(wl.in_dtype), torch.empty(2, dtype=torch.float32, device="cuda"))
    sets = ((pb, amax, outs), (pb2, amax2, outs2))
    turn = [0]

    def pair():
        p_, a_, o_ = sets[turn[0] & 1]
        turn[0] += 1
        p_.run_amax(a_, stream=sid)
        p_.run_cast(a_, outs=o_, stream=sid)

    t = time_interleaved({
        "pair": pair,
        "amax": lambda: pb.run_amax(amax, stream=sid),
        "cast": lambda: pb.run_cast(amax, outs=outs, stream=sid),
        "static": lambda: pb.run_cast_static(cal, v_fp8=True, outs=souts, stream=sid),
        "static_clip": lambda: pb.run_cast_static(clip, v_fp8=True, outs=souts, stream=sid),
        "qkv_amax": lambda: h3.h3_qkv_amax(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, am3, stream=sid),
        "qkv_cast": lambda: h3.h3_qkv_cast_e4m3(pb.desc, pb.qkv, pb.in_dt, pb.wq, pb.wk, am3, souts[0], souts[1],
                                                vo, ds3, stream=sid),
    }, steps, warmup, stream)
    pp, pa, pc, ps, pk, pa3, pc3 = (t[k] for k in ("pair", "amax", "cast", "static", "static_clip", "qkv_amax",
                                                   "qkv_cast"))
    ba3 = algorithmic_bytes(wl, "amax_v")
    return {"qkv_amax_us": round(pa3 * 1e3, 2), "qkv_amax_GBs": round(ba3 / pa3 / 1e6, 1),
            "qkv_cast_us": round(pc3 * 1e3, 2), "qkv_cast_GBs": round(bs / pc3 / 1e6, 1),
            "qkv_pair_frac_of_peak": round((ba3 + bs) / (pa3 + pc3) / 1e6 / HBM_PEAK_GBS, 4),
            "static_v8_us": round(ps * 1e3, 2), "static_v8_GBs": round(bs / ps / 1e6, 1),
            "static_v8_frac_of_peak": round(bs / ps / 1e6 / HBM_PEAK_GBS, 4),
            "static_v8_clip2sd_us": round(pk * 1e3, 2), "static_v8_clip2sd_GBs": round(bs / pk / 1e6, 1),
            "amax_us": round(pa * 1e3, 2), "amax_GBs": round(ba / pa / 1e6, 1),
            "cast_us": round(pc * 1e3, 2), "cast_GBs": round(bc / pc / 1e6, 1),
            "pair_us": round(pp * 1e3, 2), "pair_GBs": round((ba + bc) / pp / 1e6, 1),
            "pair_frac_of_peak": round((ba + bc) / pp / 1e6 / HBM_PEAK_GBS, 4),
            "valid_tokens_per_ms": round(int(wl.valid_len.sum()) / pp, 1),
            "amax_plus_cast_us": round((pa + pc) * 1e3, 2),
            "timing": "median of 3 rounds, the seven passes timed in turn in each round; pair = amax then "
                      "cast back to back, two input sets taken in turn; amax_plus_cast = the sum of the "
                      "two passes timed alone"}


def bench_fp8_pair(wl, steps, warmup):
    """The dynamic FP8 recipe as a caller runs it on the long-sequence workload: the amax pass then
    the cast pass (Q/K E4M3 codes with their descales, V a bf16 copy), back to back on the same
    input, over two input sets taken in turn so that no amax pass starts on lines the pass before
    it left in the last-level cache; and each pass alone.  Medians of three rounds, the three timed
    in turn."""
    import torch

    from synth.problem import DeviceProblem, algorithmic_bytes
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    sets = []
    for _ in range(2):
        pb = DeviceProblem(wl, "cuda")
        amax = torch.empty(2, dtype=torch.float32, device="cuda")
        outs = (pb.out("e4m3"), pb.out("e4m3"), pb.out(wl.in_dtype), torch.empty(2, dtype=torch.float32, device="cuda"))
        sets.append((pb, amax, outs))
    turn = [0]

    def pair():
        p_, a_, o_ = sets[turn[0] & 1]
        turn[0] += 1
        p_.run_amax(a_, stream=sid)
        p_.run_cast(a_, outs=o_, stream=sid)

    pb, amax, outs = sets[0]
    t = time_interleaved({"pair": pair, "amax": lambda: pb.run_amax(amax, stream=sid),
                          "cast": lambda: pb.run_cast(amax, outs=outs, stream=sid)}, steps, warmup, stream)
    ba, bc = algorithmic_bytes(wl, "amax"), algorithmic_bytes(wl, "cast")
    pp, pa, pc = t["pair"], t["amax"], t["cast"]
    return {"workload": "FP8 long sequence: T=104448 (104076 valid, grid 31x34x99), H=24, D=128, bf16 fused QKV "
                        "[1,104448,9216] -> Q/K E4M3 codes head-major with descales, V bf16",
            "pair_us": round(pp * 1e3, 2), "pair_GBs": round((ba + bc) / pp / 1e6, 1),
            "pair_frac_of_peak": round((ba + bc) / pp / 1e6 / HBM_PEAK_GBS, 4),
            "valid_tokens_per_ms": round(int(wl.valid_len.sum()) / pp, 1),
            "amax_us": round(pa * 1e3, 2), "amax_GBs": round(ba / pa / 1e6, 1),
            "amax_frac_of_peak": round(ba / pa / 1e6 / HBM_PEAK_GBS, 4),
            "cast_us": round(pc * 1e3, 2), "cast_GBs": round(bc / pc / 1e6, 1),
            "cast_frac_of_peak": round(bc / pc / 1e6 / HBM_PEAK_GBS, 4),
            "bytes_amax": ba, "bytes_cast": bc,
            "kernels": {"amax": "qk_amax_kernel<D=128, bf16> (after a one-block clear of amax[2])",
                        "cast": "qk_kernel<D=128, bf16 -> E4M3, cast>"},
            "timing": "HIP events on the launch stream; median of 3 rounds, the pair, the amax pass and the cast "
                      "pass timed in turn; pair = amax then cast back to back over two input sets taken in turn"}


def bench_sage(wl, steps, warmup, kv_scale=0.125):
    """Sage emission on the workload: F32 Q, F32 K * kv_scale, F16 V * kv_scale head-major."""
    import torch

    from synth.problem import DeviceProblem, algorithmic_bytes
    pb = DeviceProblem(wl, "cuda")
    outs = (pb.out("f32"), pb.out("f32"), pb.out("f16"))
    stream = torch.cuda.current_stream()
    _, pk = time_launches(lambda: pb.run_sage(kv_scale, outs=outs, stream=stream.cuda_stream), steps, warmup, stream)
    nb = algorithmic_bytes(wl, "sage")
    return {"us_per_call": round(pk * 1e3, 2), "GBs": round(nb / pk / 1e6, 1),
            "frac_of_peak": round(nb / pk / 1e6 / HBM_PEAK_GBS, 4), "tokens_per_ms": round(wl.B * wl.T / pk, 1)}


def bench_tensor(wl, steps, warmup):
    """One separately projected tensor: the K heads of the workload copied out as a compact
    [B, T, H, D] f16 tensor, normalised and rotated into f16 [B, T, H, D] (the layout of the
    asynchronous Ulysses input); and V through the identity path (a plain streaming copy)."""
    import torch

    import rmsnorm_rope_amd as h3
    from synth.problem import DeviceProblem
    pb = DeviceProblem(wl, "cuda")
    H, D, T = wl.H, wl.D, wl.T
    kx = pb.qkv[:, :, H * D:2 * H * D].contiguous()
    del pb.qkv
    desc = h3.make_desc(wl.B, T, H, D, wl.grid, wl.n, wl.table_len, pb.cos, pb.sin, pos_offset=pb.off,
                        valid_len=wl.valid_len, eps=wl.eps, row_stride=H * D, batch_stride=T * H * D)
    out = torch.empty((wl.B, T, H, D), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    t = time_interleaved({
        "k": lambda: h3.h3_tensor_norm_rope(desc, kx, "f16", pb.wk, out, "f16", h3.LAYOUT_BTHD, stream=sid),
        "v": lambda: h3.h3_tensor_norm_rope(desc, kx, "f16", None, out, "f16", h3.LAYOUT_BTHD, stream=sid),
    }, steps, warmup, stream)
    pk, pv = t["k"], t["v"]
    nb = int(wl.valid_len.sum()) * H * D * 2 + wl.B * T * H * D * 2
    return {"shape": [wl.B, T, H, D], "k_norm_rope_us": round(pk * 1e3, 2), "k_GBs": round(nb / pk / 1e6, 1),
            "k_frac_of_peak": round(nb / pk / 1e6 / HBM_PEAK_GBS, 4),
            "identity_us": round(pv * 1e3, 2), "identity_GBs": round(nb / pv / 1e6, 1),
            "timing": "median of 3 rounds, the two passes timed in turn in each round"}


def bench_tensor_fp8(wl, steps, warmup):
    """The FP8 recipe on one separately projected 128-dim tensor: the K heads of the long sequence
    copied out as a compact bf16 [B, T, H, D] tensor (the asynchronous Ulysses input form); the
    amax pass, then the cast to E4M3 codes [B, T, H, D] with its dynamic descale, back to back over
    two input sets taken in turn; and the 16-bit norm + RoPE store of the same tensor."""
    import torch

    import rmsnorm_rope_amd as h3
    from synth.problem import DeviceProblem
    pb = DeviceProblem(wl, "cuda")
    H, D, T = wl.H, wl.D, wl.T
    xs = [pb.qkv[:, :, H * D:2 * H * D].contiguous() for _ in range(2)]
    del pb.qkv
    desc = h3.make_desc(wl.B, T, H, D, wl.grid, wl.n, wl.table_len, pb.cos, pb.sin, pos_offset=pb.off,
                        valid_len=wl.valid_len, eps=wl.eps, row_stride=H * D, batch_stride=T * H * D)
    am = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in xs]
    ds = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in xs]
    codes = [torch.empty((wl.B, T, H, D), dtype=torch.uint8, device="cuda") for _ in xs]
    out = torch.empty((wl.B, T, H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    turn = [0]

    def pair():
        j = turn[0] & 1
        turn[0] += 1
        h3.h3_tensor_amax(desc, xs[j], wl.in_dtype, pb.wk, am[j], stream=sid)
        h3.h3_tensor_cast_e4m3(desc, xs[j], wl.in_dtype, pb.wk, am[j], False, codes[j], h3.LAYOUT_BTHD,
                               descale=ds[j], stream=sid)

    t = time_interleaved({
        "pair": pair,
        "amax": lambda: h3.h3_tensor_amax(desc, xs[0], wl.in_dtype, pb.wk, am[0], stream=sid),
        "cast": lambda: h3.h3_tensor_cast_e4m3(desc, xs[0], wl.in_dtype, pb.wk, am[0], False, codes[0],
                                               h3.LAYOUT_BTHD, descale=ds[0], stream=sid),
        "store": lambda: h3.h3_tensor_norm_rope(desc, xs[0], wl.in_dtype, pb.wk, out, "bf16", h3.LAYOUT_BTHD,
                                                stream=sid),
    }, steps, warmup, stream)
    nv = int(wl.valid_len.sum()) * H * D
    b_amax = nv * 2
    b_cast = nv * 2 + wl.B * T * H * D * 1
    b_store = nv * 2 + wl.B * T * H * D * 2
    pp, pa, pc, ps = (t[k] for k in ("pair", "amax", "cast", "store"))
    return {"shape": [wl.B, T, H, D], "pair_us": round(pp * 1e3, 2),
            "pair_GBs": round((b_amax + b_cast) / pp / 1e6, 1),
            "pair_frac_of_peak": round((b_amax + b_cast) / pp / 1e6 / HBM_PEAK_GBS, 4),
            "amax_us": round(pa * 1e3, 2), "amax_GBs": round(b_amax / pa / 1e6, 1),
            "cast_us": round(pc * 1e3, 2), "cast_GBs": round(b_cast / pc / 1e6, 1),
            "store_bf16_us": round(ps * 1e3, 2), "store_bf16_GBs": round(b_store / ps / 1e6, 1),
            "store_bf16_frac_of_peak": round(b_store / ps / 1e6 / HBM_PEAK_GBS, 4),
            "timing": "median of 3 rounds, the four passes timed in turn in each round; pair = amax then cast "
                      "back to back, two input sets taken in turn"}


def bench_qk_tensors_2x1797(steps, warmup, rotate=8):
    """Q and K as separate [2, 1797, 32, 64] f16 tensors, each normalised and rotated into f16
    [B, T, H, D] by one one-tensor call (two calls per step): the operator shape of the isolated Q/K
    RMSNorm + RoPE measurement in the B300 validation comment of the vllm-omni MiniMax-H3 VAE review
    thread (another machine and its own rotary layout: context only).  Timed twice: on one buffer
    set (its 59 MB stay in the last-level cache, as in a back-to-back operator loop) and rotating
    over `rotate` sets (cold).  The grid and n are the generator's choice (the thread gives only
    the shape)."""
    import torch

    import rmsnorm_rope_amd as h3
    import synth
    from synth.problem import DeviceProblem
    wl = synth.vae_qk_workload()
    pb = DeviceProblem(wl, "cuda")
    H, D, T = wl.H, wl.D, wl.T
    desc = h3.make_desc(wl.B, T, H, D, wl.grid, wl.n, wl.table_len, pb.cos, pb.sin, pos_offset=pb.off,
                        valid_len=wl.valid_len, eps=wl.eps, row_stride=H * D, batch_stride=T * H * D)
    qx = pb.qkv[:, :, :H * D].contiguous()
    kx = pb.qkv[:, :, H * D:2 * H * D].contiguous()
    del pb.qkv
    sets = [(qx, kx, torch.empty_like(qx), torch.empty_like(kx))]
    for _ in range(rotate - 1):
        sets.append(tuple(t.clone() for t in sets[0]))
    stream = torch.cuda.current_stream()
    res = {"shape": "Q and K each [2, 1797, 32, 64] f16 -> f16 [B, T, H, D]", "grid": list(wl.grid), "n": wl.n}
    nb = 2 * 2 * qx.numel() * 2
    for label, nsets in (("hot", 1), ("rotated", rotate)):
        it = [0]

        def step():
            q, k, qo, ko = sets[it[0] % nsets]
            it[0] += 1
            h3.h3_tensor_norm_rope(desc, q, "f16", pb.wq, qo, "f16", h3.LAYOUT_BTHD,
                                   stream=stream.cuda_stream)
            h3.h3_tensor_norm_rope(desc, k, "f16", pb.wk, ko, "f16", h3.LAYOUT_BTHD,
                                   stream=stream.cuda_stream)

        _, per = time_launches(step, steps, warmup, stream)
        res[f"{label}_us_per_qk_pair"] = round(per * 1e3, 2)
        res[f"{label}_GBs"] = round(nb / per / 1e6, 1)
    q, k, qo, ko = sets[0]

    def pair():  # on torch's current stream at call time (the capture stream under capture)
        h3.h3_tensor_norm_rope(desc, q, "f16", pb.wq, qo, "f16", h3.LAYOUT_BTHD)
        h3.h3_tensor_norm_rope(desc, k, "f16", pb.wk, ko, "f16", h3.LAYOUT_BTHD)

    g_ms = time_graph(pair, calls=20, replays=10)
    res["graph_hot_us_per_qk_pair"] = round(g_ms * 1e3, 2)
    res["graph_note"] = "20 pairs captured in one HIP graph, replayed on one buffer set"
    res["pages_context_us"] = 28.877
    return res


def bench_tile_scaling(steps, warmup, rotate=8):
    """The fixed cost of one store launch at decoder-tile sizes: the one-tile workload (token grid
    31x16x16, H = 16, D = 64) and the same problem with its first T / 2 ... T / 16 tokens valid, each
    over `rotate` buffer sets (inputs from HBM), launched back to back; a least-squares line
    time = fixed + bytes / rate through the five points.  The full tile is also timed from a HIP
    graph of 8 calls over the 8 sets (no host launch between the kernels)."""
    import numpy as np
    import torch

    import synth
    from synth.problem import DeviceProblem, algorithmic_bytes
    base = synth.workloads()["tile"]
    stream = torch.cuda.current_stream()
    pts = []
    for div in (1, 2, 4, 8, 16):
        t = base.T // div
        wl = dataclasses.replace(base, T=t, valid=[t])
        pbs = [DeviceProblem(wl, "cuda") for _ in range(rotate)]
        outs = [(pb.out("f32"), pb.out("f16"), pb.out("f16")) for pb in pbs]
        it = [0]

        def launch():
            j = it[0] % rotate
            it[0] += 1
            pbs[j].run_store("f32", "f16", outs=outs[j], stream=stream.cuda_stream)

        per = time_interleaved({"x": launch}, steps, warmup, stream)["x"]
        nb = algorithmic_bytes(wl, "store")
        pts.append({"tokens": t, "bytes": nb, "us": round(per * 1e3, 2)})
        if div == 1:
            def graph_calls():
                for j in range(rotate):
                    pbs[j].run_store("f32", "f16", outs=outs[j])
            g_ms = time_graph(graph_calls, calls=1, replays=max(10, steps // 2))
            tile_graph_us = round(g_ms / rotate * 1e3, 2)
        del pbs, outs
    x = np.array([p["bytes"] for p in pts], float)
    y = np.array([p["us"] for p in pts], float)
    slope, fixed = np.polyfit(x, y, 1)
    return {"points": pts, "fixed_us": round(float(fixed), 2), "rate_GBs": round(1e-3 / float(slope), 1),
            "tile_graph_us_per_call": tile_graph_us,
            "note": "least-squares line us = fixed + bytes / rate over the five sizes; 8 buffer sets rotated"}


def bench_block_ops(steps, warmup, rotate=8):
    """SwiGLU on [1797, 2 x 8192] f16 and the scaled residual on [2 x 1797, 2048] (fp32 residual,
    f16 branch, per-channel scale), each with `rotate` buffer sets so the 256 MB MALL holds none."""
    import numpy as np
    import torch

    import rmsnorm_rope_amd as h3
    import synth
    stream = torch.cuda.current_stream()
    N, F = synth.SWIGLU_SHAPE
    xb = synth.swiglu_input(N, F)
    xs = [torch.from_numpy(xb.view(np.int16).copy()).cuda() for _ in range(rotate)]
    ys = [torch.empty((N, F), dtype=torch.int16, device="cuda") for _ in range(rotate)]
    it = [0]

    def sw():
        j = it[0] % rotate
        it[0] += 1
        h3.h3_swiglu(xs[j], "f16", ys[j], N, F, stream=stream.cuda_stream)

    _, psw = time_launches(sw, steps, warmup, stream)
    Nr, C = synth.RESIDUAL_SHAPE
    res, br, sc = synth.residual_inputs(Nr, C)
    rs = [torch.from_numpy(res).cuda() for _ in range(rotate)]
    bs = [torch.from_numpy(br.view(np.int16).copy()).cuda() for _ in range(rotate)]
    os_ = [torch.empty_like(rs[0]) for _ in range(rotate)]
    s = torch.from_numpy(sc).cuda()

    def rr():
        j = it[0] % rotate
        it[0] += 1
        h3.h3_scaled_residual(rs[j], bs[j], "f16", s, C, os_[j], Nr, C, stream=stream.cuda_stream)

    _, prr = time_launches(rr, steps, warmup, stream)
    bsw, brr = N * F * 6, Nr * C * 10
    return {"swiglu": {"shape": [N, 2 * F], "us_per_call": round(psw * 1e3, 2), "GBs": round(bsw / psw / 1e6, 1),
                       "frac_of_peak": round(bsw / psw / 1e6 / HBM_PEAK_GBS, 4), "buffer_sets_rotated": rotate},
            "scaled_residual": {"shape": [Nr, C], "us_per_call": round(prr * 1e3, 2), "GBs": round(brr / prr / 1e6, 1),
                                "frac_of_peak": round(brr / prr / 1e6 / HBM_PEAK_GBS, 4),
                                "buffer_sets_rotated": rotate}}


def pmc_summary(root):
    """Write profiles/traffic_latent.txt from four rocprofv3 --pmc runs under `root`:
    pmc_FETCH_SIZE, pmc_WRITE_SIZE (this bench) and pmccopy_FETCH_SIZE, pmccopy_WRITE_SIZE
    (--copy-calibration).  Counters are KiB per dispatch; each is scaled by the ratio of the
    copy's known bytes to what the same counter read for the copy."""
    import csv
    import glob

    def per_dispatch(d, key):
        vals = []
        for f in glob.glob(os.path.join(root, d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if key in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
        assert vals, (d, key)
        return sum(vals) / len(vals), len(vals)

    kern = "qk_kernel<64, 1, 0, 1, 0, 8, 0>"
    fk, nf = per_dispatch("pmc_FETCH_SIZE", kern)
    wk, nw = per_dispatch("pmc_WRITE_SIZE", kern)
    cf, _ = per_dispatch("pmccopy_FETCH_SIZE", "copyBuffer")
    cw, _ = per_dispatch("pmccopy_WRITE_SIZE", "copyBuffer")
    copy_kib = (1 << 31) / 1024.0
    fs, ws = copy_kib / cf, copy_kib / cw
    rd, wr = fk * fs * 1024, wk * ws * 1024
    lines = [
        "# HBM traffic of the fused store kernel on the full-latent workload, from rocprofv3 --pmc.",
        "# Commands (repository root R, output directory OUT, run from /tmp with TMPDIR=/tmp), one counter per run:",
        "#   rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_FETCH_SIZE -o run --output-format csv -- "
        "python3 $R/bench.py --steps 5 --warmup 1 --no-cpu-baseline",
        "#   rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_WRITE_SIZE -o run --output-format csv -- "
        "python3 $R/bench.py --steps 5 --warmup 1 --no-cpu-baseline",
        "#   the same two with -d .../pmccopy_<counter> -- python3 $R/bench.py --copy-calibration "
        "(a 2 GiB device copy: 2 GiB read, 2 GiB written)",
        "#   python3 bench.py --pmc-summary $OUT",
        f"kernel_sha256_16={kernel_digest()}",
        f"dispatches_fetch={nf}",
        f"dispatches_write={nw}",
        f"fetch_kib_per_dispatch={fk:.1f}",
        f"write_kib_per_dispatch={wk:.1f}",
        f"copy_fetch_kib={cf:.1f}",
        f"copy_write_kib={cw:.1f}",
        f"fetch_scale={fs:.5f}",
        f"write_scale={ws:.5f}",
        f"hbm_read_bytes_per_launch={rd:.0f}",
        f"hbm_write_bytes_per_launch={wr:.0f}",
        f"hbm_bytes_per_launch={rd + wr:.0f}",
        "algorithmic_bytes_per_launch=3583770624",
        f"traffic_over_algorithmic={(rd + wr) / 3583770624:.5f}",
    ]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_calibration(nbytes=1 << 31, steps=10):
    """A plain device copy of known size (torch's copy kernel), for scaling the PMC byte counters."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "launches": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 20 untimed launches: after the host synchronisation that precedes the timed region, the full
    # latent's first ~10 launches run 640-650 us before settling at 612-620 us (rocprofv3 traces);
    # 5 warm-up launches measured 618.6-620.1 us on average, 20 and 40 measured 612.8-614.1 us
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true", help="also time the tile, eight-tile and FP8 workloads")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", metavar="DIR", help="write the traffic summary from rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only (one process, one MI355X); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch

    import synth
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return

    wl = synth.workloads()["latent"]
    pb, r = bench_store(wl, args.steps, args.warmup)
    nbytes = r["bytes"]
    value = nbytes / (r["ms_per_step"] * 1e-3) / 1e9
    achieved = nbytes / (r["kernel_ms"] * 1e-3) / 1e9
    tokens = wl.B * wl.T
    traffic = measured_traffic(nbytes)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "full latent 62x48x84: B=1, T=249984, H=16, D=64, fp16 fused QKV [1,249984,3072] "
                               "-> Q fp32, K/V fp16 head-major [1,16,249984,64]",
                   "global_batch": wl.B, "seq_len": wl.T, "parallelism": "none (one GPU)"},
        "tokens_per_ms": round(tokens / r["ms_per_step"], 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "qk_kernel<D=64, f16 -> f32/f16, store>", "bytes_per_launch": nbytes,
                     "avg_launch_us": round(r["kernel_ms"] * 1e3, 2),
                     "timing": f"HIP events on the launch stream around {args.steps} back-to-back calls after "
                               f"{args.warmup} untimed ones; each call is one launch of this kernel and nothing "
                               f"else, so the region's length / {args.steps} is the kernel's average launch "
                               f"duration (gaps between the queued launches included)"},
    }
    out["fp8_pair"] = bench_fp8_pair(synth.workloads()["fp8long"], args.steps, args.warmup)
    if args.extra:
        extra = {"note": "us_per_call: average over back-to-back calls of the timed region (a call may launch "
                          "a clear and a total kernel around the main one)"}
        for name, rot in (("tile", 8), ("tiles8", 1)):
            w = synth.workloads()[name]
            _, rr = bench_store(w, max(10, args.steps // 2), args.warmup, rotate=rot)
            extra[name] = {"us_per_call": round(rr["kernel_ms"] * 1e3, 2),
                           "GBs": round(rr["bytes"] / rr["kernel_ms"] / 1e6, 1),
                           "frac_of_peak": round(rr["bytes"] / rr["kernel_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                           "tokens_per_ms": round(w.B * w.T / rr["kernel_ms"], 1),
                           "buffer_sets_rotated": rot}
        tiny = synth.workloads()["tiny"]
        tpb, rr = bench_store(tiny, max(20, args.steps), args.warmup)
        touts = (tpb.out("f32"), tpb.out("f16"), tpb.out(tiny.in_dtype))
        g_ms = time_graph(lambda: tpb.run_store("f32", "f16", outs=touts), calls=50, replays=20)
        extra["tiny"] = {"us_per_call": round(rr["kernel_ms"] * 1e3, 2),
                         "graph_us_per_call": round(g_ms * 1e3, 2),
                         "note": "launch-bound: latency; graph_us_per_call: 50 calls captured in one HIP graph"}
        extra["fp8long"] = bench_fp8(synth.workloads()["fp8long"], max(10, args.steps // 2), args.warmup)
        shard = dataclasses.replace(synth.workloads()["fp8long"], T=13056, valid=[13056])
        extra["fp8long_shard8"] = bench_fp8(shard, max(10, args.steps // 2), args.warmup)
        extra["fp8long_shard8"]["note"] = "one of 8 sequence shards (T = 13,056), uncounted"
        extra["fp8long_store"] = bench_store_dtypes(synth.workloads()["fp8long"], max(10, args.steps // 2),
                                                    args.warmup)
        extra["fp8_latent_d64"] = bench_fp8(synth.workloads()["latent"], max(10, args.steps // 2), args.warmup)
        extra["fp8_latent_d64"]["note"] = ("the FP8 passes at D = 64 (f16 in) on the full latent, uncounted; "
                                           "static_v8_clip2sd uses the long sequence's clipping descales")
        extra["fp8long_tensor_k"] = bench_tensor_fp8(synth.workloads()["fp8long"], max(10, args.steps // 2),
                                                     args.warmup)
        extra["sage_latent"] = bench_sage(synth.workloads()["latent"], max(10, args.steps // 2), args.warmup)
        extra["tensor_latent_k"] = bench_tensor(synth.workloads()["latent"], max(10, args.steps // 2), args.warmup)
        extra["qk_tensors_2x1797x32x64"] = bench_qk_tensors_2x1797(max(20, args.steps), args.warmup)
        extra.update(bench_block_ops(max(20, args.steps), args.warmup))
        extra["tile_scaling"] = bench_tile_scaling(max(20, args.steps), args.warmup)
        out["extra"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pb)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
