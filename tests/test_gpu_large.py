"""Sizes past the 32-bit limits, through the C ABI: one item of T = 2^20 + 3 tokens (a ragged last
token group, five padding tokens), H = 16, D = 128, bf16.  Every output plane holds more than 2^31
elements (Q f32: 8.6 GB), so any 32-bit truncation of an element or byte offset would land rows in
the wrong place.  The oracle computes sampled tokens one by one (the first and last groups, the
padding tail, the tokens around the 2^30- and 2^31-element offsets of the planes and around 2^32
bytes of the input, and seeded random tokens); every head of every sampled token is compared bit
for bit.

The FP8 amax needs the maximum over all 2^24 rows, which the oracle cannot compute here.  Token 0
carries planted one-hot rows instead: for any row, |x_d| r <= sqrt(D) and a rotation keeps the
length of each pair, so no output can exceed sqrt(D) max|w| (up to rounding); a row whose whole
energy sits in the dimension of largest |w| at token 0 (all angles 0) reaches that bound, while a
row of the generator's normal samples (|x| below 4.2, rms near 1) stays under half of it.  The
oracle's value at the planted row is therefore the exact amax of the whole tensor, and the codes
of the sampled tokens follow from it."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits, compare, compare_raw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

T = (1 << 20) + 3
H, D, N = 16, 128, 16
GRID = (2, 725, 724)          # 1,049,800 positions >= T
VALID = T - 5
A = 3.0                       # the planted value (exact in bf16)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rmsnorm_rope_amd import _build
    if _build.stale():
        _build.build()
    torch.cuda.set_device(0)
    yield


def _workload():
    return synth.Workload("large", 1, GRID, T, H, D, N, "bf16", "normal", 7100, valid=[VALID])


def _plant(rows_or_x, token_axis_first, wq, wk):
    """One-hot rows at token 0: Q of head 0 at argmax |w_q|, K of head 1 at argmax |w_k|."""
    dq, dk = int(np.argmax(np.abs(wq))), int(np.argmax(np.abs(wk)))
    a_bits = int(oracle.encode(np.array([A], np.float32), "bf16")[0])
    spans = ((0 * D, dq), (H * D + 1 * D, dk))
    for lo, d in spans:
        if token_axis_first:
            rows_or_x[0, lo:lo + D] = 0
            rows_or_x[0, lo + d] = a_bits
        else:  # device tensor [1, T, stride] of int16
            rows_or_x[0, 0, lo:lo + D] = 0
            rows_or_x[0, 0, lo + d] = a_bits - (1 << 16) if a_bits >= (1 << 15) else a_bits


def _sample_tokens():
    """Sampled tokens: both ends, the padding tail, the tokens around the 2^30- and 2^31-element
    offsets of a [H, T, D] output plane (2^32 bytes of f32, 2^31 elements), around 2^32 bytes of
    the input, and seeded random ones."""
    rng = np.random.default_rng(7101)
    toks = {0, 1, 7, 8, 9, T - 1, T - 2, T - 3, T - 4, T - 5, T - 6, T - 8, T - 9, VALID - 1}
    for e in (1 << 30, 1 << 31):
        for h in range(H):  # element (h T + t) D of the plane
            t = e // D - h * T
            if 0 <= t < T:
                toks.update(u for u in (t - 1, t, t + 1) if 0 <= u < T)
    t_in = (1 << 32) // (3 * H * D * 2)  # input byte offset t * row bytes
    toks.update((t_in - 1, t_in, t_in + 1, t_in + 2))
    toks.update(int(t) for t in rng.integers(0, T, 600))
    return np.array(sorted(toks), np.int64)


def _gather(out, toks_dev):
    """[1, H, T, D] device tensor -> host [n, H, D] at the sampled tokens."""
    return out[0].index_select(1, toks_dev).permute(1, 0, 2).contiguous().cpu()


def test_large_item_store_amax_cast():
    import rmsnorm_rope_amd as h3
    wl = _workload()
    stride = 3 * H * D
    print(f"[large] B=1 T={T} H={H} D={D} bf16: {T * stride * 2 / 1e9:.1f} GB input", flush=True)
    wq, wk = synth.norm_weights(wl)
    x = torch.empty((1, T, stride), dtype=torch.int16, device="cuda")
    synth.values_torch(wl.seed, synth.S_QKV, 0, T * stride, wl.dist, wl.in_dtype, "cuda", out=x.view(-1))
    _plant(x, False, wq, wk)
    cos, sin = synth.rope_tables(wl.table_len, N)
    dcos, dsin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    dwq, dwk = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    desc = h3.make_desc(1, T, H, D, GRID, N, wl.table_len, dcos, dsin, valid_len=[VALID], eps=wl.eps,
                        row_stride=stride, batch_stride=T * stride)

    toks = _sample_tokens()
    rows = synth.qkv_host(wl, toks).copy()
    _plant(rows, True, wq, wk)
    spec = oracle.spec_from_workload(wl, batch_stride=T * stride)
    toks_dev = torch.from_numpy(toks).cuda()
    print(f"[large] {toks.size} sampled tokens", flush=True)

    # store: Q f32, K f16, V bf16 copy
    q = torch.empty((1, H, T, D), dtype=torch.float32, device="cuda")
    k = torch.empty((1, H, T, D), dtype=torch.float16, device="cuda")
    v = torch.empty((1, H, T, D), dtype=torch.bfloat16, device="cuda")
    h3.h3_qk_rmsnorm_rope_permute(desc, x, "bf16", dwq, dwk, q, "f32", k, "f16", v)
    torch.cuda.synchronize()
    rq, rk, rv, ry = oracle.qk_tokens(spec, rows, toks, "bf16", wq, wk, "f32", "f16")
    compare(bits(_gather(q, toks_dev)), rq, "f32", "large Q")
    compare(bits(_gather(k, toks_dev)), rk, "f16", "large K")
    compare_raw(bits(_gather(v, toks_dev)), rv, "large V")
    del q, k, v
    torch.cuda.empty_cache()

    # amax: attained at the planted rows (see the module docstring)
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    h3.h3_qk_amax(desc, x, "bf16", dwq, dwk, amax)
    torch.cuda.synchronize()
    live = toks < VALID
    want = np.array([np.abs(ry[live, 0]).max(), np.abs(ry[live, 1]).max()], np.float32)
    bound = np.sqrt(D) * np.array([np.abs(wq).max(), np.abs(wk).max()])
    assert np.all(want > 0.99 * bound), (want, bound)
    others = np.abs(ry[live][1:]).reshape(-1, 2, H * D).max(axis=(0, 2))  # sampled rows but token 0
    assert np.all(others < 0.6 * want), (others, want)
    compare(bits(amax.cpu()), want, "f32", "large amax")

    # cast with that amax
    q8 = torch.empty((1, H, T, D), dtype=torch.uint8, device="cuda")
    k8 = torch.empty((1, H, T, D), dtype=torch.uint8, device="cuda")
    v16 = torch.empty((1, H, T, D), dtype=torch.bfloat16, device="cuda")
    ds = torch.empty(2, dtype=torch.float32, device="cuda")
    h3.h3_qk_cast_e4m3(desc, x, "bf16", dwq, dwk, amax, q8, k8, v16, ds)
    torch.cuda.synchronize()
    cq, ck, cv, _ = oracle.qk_tokens(spec, rows, toks, "bf16", wq, wk, fp8=True, amax=want)
    compare(bits(ds.cpu()), np.array([oracle.descale_of(float(a)) for a in want], np.float32), "f32", "large descale")
    compare(bits(_gather(q8, toks_dev)), cq, "e4m3", "large Q codes")
    compare(bits(_gather(k8, toks_dev)), ck, "e4m3", "large K codes")
    compare_raw(bits(_gather(v16, toks_dev)), cv, "large V copy")
    print(f"[large] store, amax {want.tolist()} and cast match the oracle at {toks.size} tokens", flush=True)
