"""The C-ABI library on a machine without a GPU: it loads, exports every symbol include/h3qk.h
declares, and validates arguments on the host before any HIP call (no compute call is made:
every case here fails validation, so nothing reaches the runtime)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import rmsnorm_rope_amd as h3
from rmsnorm_rope_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if _build.stale():
        _build.build()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "h3qk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(h3_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(h3.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", h3.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (h3_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(h3.lib(), n)


def test_header_constants_match_binding():
    src = open(os.path.join(ROOT, "include", "h3qk.h")).read()
    assert int(re.search(r"#define H3_SAT_SLOTS (\d+)", src).group(1)) == h3.SAT_SLOTS
    assert int(re.search(r"#define H3_MAX_BATCH (\d+)", src).group(1)) == h3.MAX_BATCH
    assert h3.SAT_WORDS == 16 * (h3.SAT_SLOTS + 1)


def test_header_is_c99_and_every_entry_point_links(tmp_path):
    """A plain C99 program includes include/h3qk.h, links against the library and calls every entry
    point (each fails host validation; no GPU call)."""
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-o", str(exe),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", os.path.dirname(h3.LIB_PATH), "-lh3qk",
           "-Wl,-rpath," + os.path.dirname(h3.LIB_PATH)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 failure(s)" in out.stdout


def test_c_end_to_end_program_builds(tmp_path):
    """The pure-C GPU program (tests/c/e2e_gpu.c, run by the gpu tests) compiles and links here."""
    from tests.gpu_util import build_c_e2e
    assert os.path.exists(build_c_e2e(tmp_path))


def test_binding_refuses_host_and_strided_tensors():
    """The binding passes flat device addresses: a host tensor or a non-contiguous view is refused
    before the library is called."""
    import torch
    with pytest.raises(ValueError, match="device tensors"):
        h3._ptr(torch.zeros(4))
    class FakeStrided:  # a device tensor that is not contiguous (no GPU needed to model one)
        device = type("dev", (), {"type": "cuda"})()
        def is_contiguous(self): return False
        def data_ptr(self): return BASE
    with pytest.raises(ValueError, match="contiguous"):
        h3._ptr(FakeStrided())
    class FakeStridedTensor:  # the same through the attributes of a torch tensor
        is_cuda = True
        def is_contiguous(self): return False
        def data_ptr(self): return BASE
    with pytest.raises(ValueError, match="contiguous"):
        h3._ptr(FakeStridedTensor())
    FakeStridedTensor.is_contiguous = lambda self: True
    assert h3._ptr(FakeStridedTensor()) == BASE
    with pytest.raises(ValueError, match="device tensors"):
        h3._ptr(torch.zeros(4).t())
    assert h3._ptr(BASE) == BASE and h3._ptr(None) is None


def test_abi_version():
    assert h3.h3_abi_version() == 1


# fake, well-aligned device addresses: validation never dereferences them
BASE = 0x7F0000000000


def desc(**kw):
    a = dict(B=1, T=32, H=2, D=64, grid=(2, 4, 4), pairs_per_axis=8, table_len=(2, 4, 4),
             cos_tab=BASE + 0x10000000, sin_tab=BASE + 0x11000000)
    a.update(kw)
    return h3.make_desc(**a)


def call(d=None, qkv=BASE, in_dt=h3.F16, wq=BASE + 0x20000000, wk=BASE + 0x21000000,
         q=BASE + 0x30000000, q_dt=h3.F32, k=BASE + 0x40000000, k_dt=h3.F16, v=BASE + 0x50000000):
    d = desc() if d is None else d
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_rmsnorm_rope_permute(d, qkv, in_dt, wq, wk, q, q_dt, k, k_dt, v, stream=0)
    return e.value


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), "H3_EINVAL"), (dict(B=65), "H3_EINVAL"), (dict(T=0), "H3_EINVAL"), (dict(H=0), "H3_EINVAL"),
    (dict(D=96), "H3_EUNSUPPORTED"), (dict(D=256), "H3_EUNSUPPORTED"),
    (dict(pairs_per_axis=11), "H3_EUNSUPPORTED"), (dict(pairs_per_axis=-1), "H3_EUNSUPPORTED"),
    (dict(eps=float("nan")), "H3_EINVAL"), (dict(eps=-1.0), "H3_EINVAL"),
    (dict(row_stride=3 * 2 * 64 - 8), "H3_EINVAL"), (dict(row_stride=3 * 2 * 64 + 4), "H3_EALIGN"),
    (dict(B=2, batch_stride=32 * 384 - 8), "H3_EINVAL"),
    (dict(grid=(0, 4, 4)), "H3_EINVAL"), (dict(table_len=(2, 4, 3)), "H3_ERANGE"),
    (dict(valid_len=[33]), "H3_ERANGE"), (dict(valid_len=[-1]), "H3_ERANGE"),
    (dict(T=40, valid_len=[33]), "H3_ERANGE"),             # more valid tokens than grid positions
    (dict(pos_offset=[[1, 0, 0]]), "H3_ERANGE"), (dict(pos_offset=[[0, -1, 0]]), "H3_ERANGE"),
    (dict(cos_tab=0), "H3_EINVAL"), (dict(sin_tab=BASE + 2), "H3_EALIGN"),
    (dict(table_len=(2, 4, (1 << 27) - 5)), "H3_EINVAL"),  # (P_t + P_h + P_w) * n = 2^30 + 8 entries
])
def test_descriptor_validation(kw, code):
    assert call(desc(**kw)).name == code


def test_pointer_validation():
    assert call(qkv=0).name == "H3_EINVAL"
    assert call(q=0).name == "H3_EINVAL"
    assert call(qkv=BASE + 8).name == "H3_EALIGN"
    assert call(wq=BASE + 0x20000004).name == "H3_EALIGN"
    assert call(q=BASE + 0x30000008).name == "H3_EALIGN"
    assert call(in_dt=h3.F32).name == "H3_EUNSUPPORTED"
    assert call(q_dt=h3.E4M3FN).name == "H3_EUNSUPPORTED"
    assert call(k_dt=7).name == "H3_EUNSUPPORTED"


def test_alias_validation():
    # q_out inside the input
    assert call(q=BASE + 4096).name == "H3_EALIAS"
    # k_out overlapping q_out (q is 32*2*64*4 = 16 KiB)
    assert call(k=BASE + 0x30000000 + 8192).name == "H3_EALIAS"
    # v_out on a weight
    assert call(v=BASE + 0x20000000).name == "H3_EALIAS"
    # outputs adjacent but not overlapping are fine up to validation (checked via amax path below)
    e = call(q=BASE + 0x30000000, k=BASE + 0x30000000 + 16384 - 16)
    assert e.name == "H3_EALIAS"
    msg = h3.h3_last_error()
    assert "k_out" in msg and "q_out" in msg


def test_amax_and_cast_validation():
    d = desc(D=128, pairs_per_axis=16)
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_amax(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, 0, stream=0)
    assert e.value.name == "H3_EINVAL"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_amax(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 64, stream=0)
    assert e.value.name == "H3_EALIAS"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_cast_e4m3(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x60000000,
                           BASE + 0x30000000, BASE + 0x30000000 + 128, BASE + 0x50000000, BASE + 0x61000000,
                           stream=0)
    assert e.value.name == "H3_EALIAS"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_cast_e4m3(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x60000000,
                           BASE + 0x30000000, BASE + 0x40000000, BASE + 0x50000000, BASE + 0x60000000,
                           stream=0)
    assert e.value.name == "H3_EALIAS"  # descale on top of amax
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_cast_e4m3(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x60000000,
                           BASE + 0x30000000, BASE + 0x40000000, BASE + 0x50000000, BASE + 0x61000004,
                           stream=0)
    assert e.value.name == "H3_EALIGN"


def _static(d, descale=BASE + 0x60000000, q=BASE + 0x30000000, k=BASE + 0x40000000, v=BASE + 0x50000000,
            v_dt=h3.E4M3FN, sat=BASE + 0x61000000):
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qk_cast_e4m3_static(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, descale, q, k, v, v_dt,
                                  sat, stream=0)
    return e.value.name, h3.h3_last_error()


def test_static_cast_validation():
    d = desc(D=128, pairs_per_axis=16)
    assert _static(d, descale=0)[0] == "H3_EINVAL"
    assert _static(d, v=0)[0] == "H3_EINVAL"
    assert _static(d, v_dt=h3.F16)[0] == "H3_EUNSUPPORTED"          # neither in_dt (bf16) nor E4M3
    assert _static(d, v_dt=h3.F32)[0] == "H3_EUNSUPPORTED"
    assert _static(d, descale=BASE + 0x60000002)[0] == "H3_EALIGN"
    assert _static(d, sat=BASE + 0x61000004)[0] == "H3_EALIGN"
    name, msg = _static(d, sat=BASE + 0x60000000 - 8 * h3.SAT_WORDS + 8)  # counter tail on the descales
    assert name == "H3_EALIAS" and "sat_qkv" in msg and "descale_qkv" in msg
    name, msg = _static(d, sat=BASE + 0x50000000 + 32 * 2 * 128 - 8)  # counter on the V codes' tail
    assert name == "H3_EALIAS" and "v_out" in msg
    name, msg = _static(d, k=BASE + 0x30000000 + 32 * 2 * 128 - 16)  # K codes on Q codes
    assert name == "H3_EALIAS" and "k_codes" in msg
    # V copied (v_dt = in_dt): the V output is 2 bytes per element, so a K placed one code plane after
    # V's start overlaps it, while with V codes it does not
    name, msg = _static(d, v=BASE + 0x50000000, k=BASE + 0x50000000 + 32 * 2 * 128, v_dt=h3.BF16)
    assert name == "H3_EALIAS" and "v_out" in msg
    # with V as codes that layout passes the overlap checks; an unaligned counter then still fails
    assert _static(d, v=BASE + 0x50000000, k=BASE + 0x50000000 + 32 * 2 * 128, sat=BASE + 0x61000001)[0] == "H3_EALIGN"


def test_static_cast_noalloc_validation():
    """The allocation-free static cast validates like h3_qk_cast_e4m3_static, with a three-word
    counts output in place of the counter buffer (every case fails before any HIP call)."""
    d = desc(D=128, pairs_per_axis=16)

    def call(descale=BASE + 0x60000000, v=BASE + 0x50000000, v_dt=h3.E4M3FN, sat=BASE + 0x61000000):
        with pytest.raises(h3.H3Error) as e:
            h3.h3_qk_cast_e4m3_static_noalloc(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, descale,
                                              BASE + 0x30000000, BASE + 0x40000000, v, v_dt, sat, stream=0)
        return e.value.name, h3.h3_last_error()
    assert call(descale=0)[0] == "H3_EINVAL"
    assert call(v_dt=h3.F32)[0] == "H3_EUNSUPPORTED"
    assert call(sat=BASE + 0x61000004)[0] == "H3_EALIGN"
    name, msg = call(sat=BASE + 0x60000000 - 16)  # the counts' last word on the first descale
    assert name == "H3_EALIAS" and "sat_counts" in msg and "descale_qkv" in msg
    name, msg = call(sat=BASE + 0x50000000 + 32 * 2 * 128 - 16)  # on the V codes' tail
    assert name == "H3_EALIAS" and "sat_counts" in msg and "v_out" in msg


def test_sage_validation():
    d = desc()
    def sage(scale=0.125, q=BASE + 0x30000000, k=BASE + 0x40000000, v=BASE + 0x50000000):
        with pytest.raises(h3.H3Error) as e:
            h3.h3_qk_rmsnorm_rope_permute_sage(d, BASE, h3.F16, BASE + 0x20000000, BASE + 0x21000000, scale, q, k, v,
                                               stream=0)
        return e.value.name, h3.h3_last_error()
    assert sage(scale=float("nan"))[0] == "H3_EINVAL"
    assert sage(scale=float("inf"))[0] == "H3_EINVAL"
    assert sage(v=0)[0] == "H3_EINVAL"
    name, msg = sage(k=BASE + 0x30000000 + 32 * 2 * 64 * 4 - 16)   # K f32 on Q f32's tail
    assert name == "H3_EALIAS" and "k_out" in msg


def test_qkv_fp8_validation():
    d = desc(D=128, pairs_per_axis=16)
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qkv_amax(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x20000000 + 508, stream=0)
    assert e.value.name == "H3_EALIAS"                                     # amax_qkv tail on w_q
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qkv_amax(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x60000002, stream=0)
    assert e.value.name == "H3_EALIGN"
    n = 32 * 2 * 128
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qkv_cast_e4m3(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x60000000,
                            BASE + 0x30000000, BASE + 0x40000000, BASE + 0x40000000 + n - 16, BASE + 0x61000000,
                            stream=0)
    assert e.value.name == "H3_EALIAS" and "v_codes" in h3.h3_last_error()
    with pytest.raises(h3.H3Error) as e:
        h3.h3_qkv_cast_e4m3(d, BASE, h3.BF16, BASE + 0x20000000, BASE + 0x21000000, BASE + 0x60000000,
                            BASE + 0x30000000, BASE + 0x40000000, BASE + 0x50000000, BASE + 0x60000008,
                            stream=0)
    assert e.value.name == "H3_EALIAS" and "descale_qkv" in h3.h3_last_error()  # on amax_qkv[2]


def _tensor_store(d, x=BASE, w=BASE + 0x20000000, out=BASE + 0x30000000, out_dt=h3.F16, layout=0):
    with pytest.raises(h3.H3Error) as e:
        h3.h3_tensor_norm_rope(d, x, h3.BF16, w, out, out_dt, layout, stream=0)
    return e.value.name, h3.h3_last_error()


def test_tensor_validation():
    d = desc(D=128, pairs_per_axis=16, row_stride=2 * 128)          # one tensor of H = 2 heads
    assert _tensor_store(d, out_dt=h3.E4M3FN)[0] == "H3_EUNSUPPORTED"
    assert _tensor_store(d, layout=2)[0] == "H3_EUNSUPPORTED"
    assert _tensor_store(d, x=0)[0] == "H3_EINVAL"
    assert _tensor_store(d, out=0)[0] == "H3_EINVAL"
    assert _tensor_store(d, w=BASE + 0x20000004)[0] == "H3_EALIGN"
    name, msg = _tensor_store(d, out=BASE + 4096)                    # out inside x
    assert name == "H3_EALIAS" and "x" in msg
    assert _tensor_store(desc(D=128, pairs_per_axis=16, row_stride=2 * 128 - 8))[0] == "H3_EINVAL"
    # identity (w = NULL) passes weight checks; an aliasing output still fails
    assert _tensor_store(d, w=0, out=BASE + 64)[0] == "H3_EALIAS"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_tensor_amax(d, BASE, h3.BF16, 0, BASE + 16, stream=0)
    assert e.value.name == "H3_EALIAS"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_tensor_amax(d, BASE, h3.BF16, 0, 0, stream=0)
    assert e.value.name == "H3_EINVAL"

    def cast(scale=BASE + 0x60000000, is_ds=1, codes=BASE + 0x30000000, descale=BASE + 0x61000000,
             sat=BASE + 0x62000000):
        with pytest.raises(h3.H3Error) as e:
            h3.h3_tensor_cast_e4m3(d, BASE, h3.BF16, BASE + 0x20000000, scale, is_ds, codes, 0, descale, sat, stream=0)
        return e.value.name, h3.h3_last_error()
    assert cast(scale=0)[0] == "H3_EINVAL"
    assert h3.lib().h3_tensor_cast_e4m3(ctypes.byref(d), BASE, h3.BF16, BASE + 0x20000000, BASE + 0x60000000, 2,
                                        BASE + 0x30000000, 0, None, None, None) == -1
    assert cast(descale=BASE + 0x60000000)[0] == "H3_EALIAS"       # descale on the scale input
    name, msg = cast(sat=BASE + 0x30000000 + 32 * 2 * 128 - 8)      # counters on the codes' tail
    assert name == "H3_EALIAS" and "sat" in msg
    assert cast(sat=BASE + 0x62000004)[0] == "H3_EALIGN"


def test_null_descriptor():
    rc = h3.lib().h3_qk_rmsnorm_rope_permute(None, BASE, 1, BASE, BASE, BASE, 0, BASE, 1, BASE, None)
    assert rc == -1 and "desc" in h3.h3_last_error()


def test_block_op_validation():
    with pytest.raises(h3.H3Error) as e:
        h3.h3_swiglu(BASE, h3.F16, BASE + 0x40000000, 4, 12, stream=0)
    assert e.value.name == "H3_EUNSUPPORTED"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_swiglu(BASE, h3.F16, BASE + 64, 4, 16, stream=0)       # y inside x
    assert e.value.name == "H3_EALIAS"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_swiglu(BASE + 8, h3.F16, BASE + 0x40000000, 4, 16, stream=0)
    assert e.value.name == "H3_EALIGN"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_swiglu(BASE, h3.F32, BASE + 0x40000000, 4, 16, stream=0)
    assert e.value.name == "H3_EUNSUPPORTED"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_swiglu(0, h3.F16, BASE + 0x40000000, 4, 16, stream=0)
    assert e.value.name == "H3_EINVAL"
    R, Bq, S, O = BASE, BASE + 0x10000000, BASE + 0x20000000, BASE + 0x30000000
    with pytest.raises(h3.H3Error) as e:
        h3.h3_scaled_residual(R, Bq, h3.F16, S, 3, O, 4, 8, stream=0)     # scale_len not 1 or C
    assert e.value.name == "H3_EINVAL"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_scaled_residual(R, Bq, h3.F16, S, 1, O, 4, 6, stream=0)     # C not a multiple of 4
    assert e.value.name == "H3_EUNSUPPORTED"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_scaled_residual(R, Bq, h3.F16, S, 1, R + 16, 4, 8, stream=0)  # out overlaps res
    assert e.value.name == "H3_EALIAS"
    with pytest.raises(h3.H3Error) as e:
        h3.h3_scaled_residual(R, Bq + 4, h3.F16, S, 8, O, 4, 8, stream=0)
    assert e.value.name == "H3_EALIGN"


def test_elementwise_launch_covers_the_largest_accepted_size(tmp_path):
    """The decoder-block ops accept up to 2^32 - 1 vectors (N * F / 8 for SwiGLU, N * C / 4 for the
    scaled residual).  Their block count is taken in 64 bits (a 32-bit sum would wrap to zero blocks
    at the top of that range and the call would return success having written nothing), and the
    multiply-high division that maps a vector to its row is exact there.  Host code of the library's
    internal header, compiled with g++ (no GPU)."""
    src = tmp_path / "blocks.cpp"
    src.write_text(r'''
#include <cstdio>
#include "h3qk_internal.h"
int main() {
    int bad = 0;
    const uint64_t top = 0xFFFFFFFFull;  // the largest vector count the host accepts
    const uint64_t per = 512;            // vectors per block of the elementwise kernels
    const uint64_t vs[] = {1, 511, 512, 513, top - 512, top - 511, top - 1, top};
    for (uint64_t v : vs) {
        const uint64_t b = h3::blocks_for(v, per);
        if (b == 0 || b * per < v || (b - 1) * per >= v) { std::printf("blocks %llu\n", (unsigned long long)v); ++bad; }
        if (b > (1ull << 23)) { std::printf("more than 2^23 blocks at %llu\n", (unsigned long long)v); ++bad; }
    }
    const uint32_t ds[] = {1u, 2u, 3u, 7u, 256u, 1000u, 1024u, 4095u, 1u << 27};
    for (uint32_t d : ds) {
        const h3::DivMagic m = h3::div_magic(d);
        const uint64_t ns[] = {0, 1, (uint64_t)d - 1, (uint64_t)d, 0x7FFFFFFF, top - d, top - 1, top};
        for (uint64_t n : ns) {
            if (n > top) continue;
            if (h3::div_apply((uint32_t)n, m) != (uint32_t)n / d) { std::printf("div %llu / %u\n", (unsigned long long)n, d); ++bad; }
        }
    }
    std::printf("%d failure(s)\n", bad);
    return bad != 0;
}
''')
    exe = tmp_path / "blocks"
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-DH3QK_NO_HIP", "-I", os.path.join(ROOT, "rmsnorm_rope_amd", "csrc"),
                        "-o", str(exe), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and "0 failure(s)" in out.stdout, out.stdout + out.stderr
