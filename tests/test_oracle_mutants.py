"""Mutation check of the oracle's pins: each mutant is a copy of oracle/h3ref.c with one plausible
mistake planted (a dropped term, a wrong sign, index or operand order, a wrong constant or
boundary, a skipped rounding), built with gcc into a temporary library and loaded by the pin tests
in a child process (H3REF_LIB).  Every mutant must make at least one pin fail.  The comparisons
against the numpy twin and the stored digests are left out: they re-derive the oracle's own
formulas or outputs and do not count as pins.  CPU only; nothing here touches a GPU."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_pins.py", "test_oracle_pins_block.py", "test_oracle_pins_sage.py",
    "test_oracle_pins_static.py", "test_oracle_pins_tensor.py")]
NOT_PINS = "not twin_matches and not golden"

# (name, text in h3ref.c, replacement)
MUTANTS = [
    ("rotation: sign of the sine term", "y[2 * p] = ec - fs;", "y[2 * p] = ec + fs;"),
    ("rotation: second output from the wrong products", "y[2 * p + 1] = es + fc;", "y[2 * p + 1] = fc - es;"),
    ("rotation: axes interleaved instead of blocked", "int axis = p / n, j = p % n;", "int axis = p % 3, j = p / 3;"),
    ("rotation: last rotated pair left alone", "for (int p = 0; p < 3 * n; ++p) {", "for (int p = 0; p < 3 * n - 1; ++p) {"),
    ("rms: eps dropped", "float v = ms + eps;", "float v = ms;"),
    ("rms: mean over D - 1", "float ms = a[0] * (1.0f / (float)D);", "float ms = a[0] / (float)(D - 1);"),
    ("rms: sequential sum instead of the halving tree",
     "for (int o = D / 2; o >= 1; o /= 2)\n        for (int d = 0; d < o; ++d) a[d] = a[d] + a[d + o];",
     "for (int d = 1; d < D; ++d) a[0] = a[0] + a[d];"),
    ("rms: weight applied before 1/rms", "float t = x[d] * r;\n        y[d] = t * w[d];",
     "float t = x[d] * w[d];\n        y[d] = t * r;"),
    ("rms: reciprocal square root rounded once",
     "float sq = sqrtf(v);\n    float r = 1.0f / sq;", "float sq = sqrtf(v);\n    float r = (float)(1.0 / sqrt((double)v));"),
    ("position: w offset taken from the h axis", "pos[2] = i % gw + P->pos_offset[3 * b + 2];",
     "pos[2] = i % gw + P->pos_offset[3 * b + 1];"),
    ("position: h index not reduced modulo Gh", "pos[1] = (i / gw) % gh + P->pos_offset[3 * b + 1];",
     "pos[1] = (i / gw) % (gh + 1) + P->pos_offset[3 * b + 1];"),
    ("rounding: ties away from even", "if (rem > half || (rem == half && (q & 1))) q += 1;",
     "if (rem >= half) q += 1;"),
    ("f16: overflow threshold one step low", "if (a >= 0x477FF000) return (uint16_t)(sign | 0x7C00);",
     "if (a >= 0x477FE000) return (uint16_t)(sign | 0x7C00);"),
    ("e4m3: no saturation (NaN code past 448)", "if (a > 0x43E00000) return (uint8_t)(sign | 0x7E);",
     "if (a > 0x43E00000) return (uint8_t)(sign | 0x7F);"),
    ("e4m3: subnormal step 2^-10", "if (e >= -6) return", "if (e >= -7) return"),
    ("descale: 240 instead of 448", "return amax > 0.0f ? amax / 448.0f : 1.0f;", "return amax > 0.0f ? amax / 240.0f : 1.0f;"),
    ("descale: zero amax kept", "float h3ref_descale(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }",
     "float h3ref_descale(float amax) { return amax / 448.0f; }"),
    ("static descale: negative values accepted", "float h3ref_static_descale(float d) { return d > 0.0f ? d : 1.0f; }",
     "float h3ref_static_descale(float d) { return d != 0.0f ? d : 1.0f; }"),
    ("clip count: quotients equal to 448 counted", "if (sat && fabsf(q) > 448.0f) *sat += 1;",
     "if (sat && fabsf(q) >= 448.0f) *sat += 1;"),
    ("cast: V codes with the Q descale", "cast_one(load_in(row, in_dt, vi + d), so->ds[2],",
     "cast_one(load_in(row, in_dt, vi + d), so->ds[0],"),
    ("amax: NaN ignored", "if (isnan(m) || isnan(amax[s])) amax[s] = NAN;", "if (0) amax[s] = NAN;"),
    ("V amax: read from the K heads", "float m = fabsf(load_in(row, in_dt, 2 * (int64_t)H * D + e));",
     "float m = fabsf(load_in(row, in_dt, 1 * (int64_t)H * D + e));"),
    ("store: padding rows of V copied", "((uint16_t *)v)[o + d] = padded ? 0 : row[vi + d];",
     "((uint16_t *)v)[o + d] = row[vi + d];"),
    ("tensor: [B, T, H, D] laid out as [B, H, T, D]", "return (((int64_t)b * P->T + i) * P->H + h) * P->D + d;",
     "return (((int64_t)b * P->H + h) * P->T + i) * P->D + d;"),
    ("sage: K not scaled", "float ks = yqk[((int64_t)H + h) * D + d] * kv_scale;",
     "float ks = yqk[((int64_t)H + h) * D + d];"),
    ("sage: V rounded once from binary64",
     "float vs = load_in(row, in_dt, ((int64_t)2 * H + h) * D + d) * kv_scale;\n                    v[o] = h3ref_f16_encode(vs);",
     "double vs = (double)load_in(row, in_dt, ((int64_t)2 * H + h) * D + d) * kv_scale;\n"
     "                    uint16_t h3ref_f16_encode_f64(double);\n                    v[o] = h3ref_f16_encode_f64(vs);"),
    ("SwiGLU: gate and up swapped", "double s = g / (1.0 + exp(-g));\n            double v = s * u;",
     "double s = u / (1.0 + exp(-u));\n            double v = s * g;"),
    ("f16 decode: subnormal step 2^-25", "if (E == 0)       v = ldexpf((float)m, -24);",
     "if (E == 0)       v = ldexpf((float)m, -25);"),
    ("bf16 encode: NaN not kept quiet", "return (uint16_t)((x >> 16) | 0x40);", "return (uint16_t)(x >> 16);"),
    ("e4m3 decode: subnormal step 2^-10", "float v = (E == 0) ? ldexpf((float)m, -9)",
     "float v = (E == 0) ? ldexpf((float)m, -10)"),
    ("Q/K/V cast: V with the K descale", "h3ref_descale(amax[1]), h3ref_descale(amax[2])}, 0};",
     "h3ref_descale(amax[1]), h3ref_descale(amax[1])}, 0};"),
    ("static cast: V descale unguarded", "v_fp8 ? h3ref_static_descale(descale[2]) : 1.0f},",
     "v_fp8 ? descale[2] : 1.0f},"),
    ("tensor cast: padding rows cast instead of zeroed",
     "out[o] = rc == 1 ? 0 : cast_one(y[(int64_t)h * P->D + d], ds, sat);",
     "out[o] = rc == 1 ? 0x38 : cast_one(y[(int64_t)h * P->D + d], ds, sat);"),
    ("tensor amax: starts at one", "    *amax = 0.0f;\n", "    *amax = 1.0f;\n"),
    ("sage: padding rows of K left at one", "if (rc == 1) { q[o] = 0.0f; k[o] = 0.0f; v[o] = 0; continue; }",
     "if (rc == 1) { q[o] = 0.0f; k[o] = 1.0f; v[o] = 0; continue; }"),
    ("SwiGLU: sign of the exponent", "double s = g / (1.0 + exp(-g));", "double s = g / (1.0 + exp(g));"),
    ("residual: per-channel scale ignored", "float t = b * scale[scale_len == 1 ? 0 : c];",
     "float t = b * scale[0];"),
    ("residual: product and sum rounded once",
     "float t = b * scale[scale_len == 1 ? 0 : c];\n            out[n * C + c] = res[n * C + c] + t;",
     "out[n * C + c] = (float)((double)res[n * C + c] + (double)b * (double)scale[scale_len == 1 ? 0 : c]);"),
]


def _pins(lib, expr):
    env = dict(os.environ, H3REF_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES, "-k", expr]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-400:]


def _caught(lib):
    """Fast pins first; the exhaustive encoder pins only when those all pass."""
    rc, out = _pins(lib, f"{NOT_PINS} and not encoder")
    if rc == 1:
        return True, out
    assert rc == 0, out  # 0 passed, 1 failed; anything else is a broken run
    rc, out = _pins(lib, f"{NOT_PINS} and encoder")
    assert rc in (0, 1), out
    return rc == 1, out


def test_mutant_texts_are_unique():
    src = open(oracle.SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.skipif(oracle.LIB_OVERRIDE is not None, reason="already running under a substitute oracle")
def test_every_mutant_fails_a_pin():
    src = open(oracle.SRC).read()
    with tempfile.TemporaryDirectory(prefix="h3ref_mut_") as tmp:
        libs = []
        for k, (name, old, new) in enumerate(MUTANTS):
            assert src.count(old) == 1, name
            c = os.path.join(tmp, f"m{k}.c")
            with open(c, "w") as f:
                f.write(src.replace(old, new))
            libs.append(oracle.build(src=c, out=os.path.join(tmp, f"m{k}.so")))
        # the unmutated library passes the same pins (a broken harness would "catch" everything)
        rc, out = _pins(oracle.build(out=os.path.join(tmp, "base.so")), f"{NOT_PINS} and not encoder")
        assert rc == 0, out
        workers = max(1, min(8, (os.cpu_count() or 2) - 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(_caught, libs))
    survivors = [MUTANTS[k][0] for k, (ok, _) in enumerate(results) if not ok]
    print(f"[mutants] {len(MUTANTS) - len(survivors)} of {len(MUTANTS)} caught by the pins", flush=True)
    assert not survivors, f"mutants no pin catches: {survivors}"
