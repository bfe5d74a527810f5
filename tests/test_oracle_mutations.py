"""Mutation check of the oracle's pins: each plausible slip planted into a
scratch copy of oracle/moe_oracle.c must make at least one pin in
test_oracle_pins.py or test_oracle_formats.py fail.

For every mutation the copy is compiled with the oracle's own flags, and the
pin suite runs in a child process that loads that build (MOE_ORACLE_LIB).  An
unmutated copy must pass the same suite, so a failure is the mutation's doing.
The repository's oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
HDR = os.path.join(ROOT, "oracle", "moe_oracle.h")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_oracle_formats.py")]

# (name, exact text in moe_oracle.c, replacement): each one a slip that a
# reader of the pages could plausibly make.
MUTATIONS = [
    ("nibble order", "(k % 2 == 0) ? (byte & 0xF) : (byte >> 4)", "(k % 2 == 0) ? (byte >> 4) : (byte & 0xF)"),
    ("code offset", "(double)(code - 8) * scale", "(double)(code - 7) * scale"),
    ("scale group index", "s[(int64_t)n * (K / G) + k / G]", "s[(int64_t)n * (K / G) + (k / G + 1) % (K / G)]"),
    ("gate row", "g += wq_at(w13_q, w13_s, H, G, r, k) * x[k];",
     "g += wq_at(w13_q, w13_s, H, G, (r + 1) % I, k) * x[k];"),
    ("up row", "u += wq_at(w13_q, w13_s, H, G, I + r, k) * x[k];",
     "u += wq_at(w13_q, w13_s, H, G, I + (r + 1) % I, k) * x[k];"),
    ("gate/up swap", "h[r] = silu(g) * u;\n  }\n#pragma omp parallel for schedule(static)\n  for (int32_t n = 0; n < H; ++n) {\n"
     "    double acc = 0.0;\n    for (int32_t r = 0; r < I; ++r) acc += wq_at",
     "h[r] = silu(u) * g;\n  }\n#pragma omp parallel for schedule(static)\n  for (int32_t n = 0; n < H; ++n) {\n"
     "    double acc = 0.0;\n    for (int32_t r = 0; r < I; ++r) acc += wq_at"),
    ("SiLU sign", "return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    ("down input index", "wq_at(w2_q, w2_s, I, G, n, r) * h[r]", "wq_at(w2_q, w2_s, I, G, n, (r + 1) % I) * h[r]"),
    ("down transposed", "acc += wq_at(w2_q, w2_s, I, G, n, r) * h[r];",
     "acc += wq_at(w2_q, w2_s, I, G, (n + r) % H, r) * h[r];"),
    ("tie-break", "if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;",
     "if (!taken[e] && (best < 0 || l[e] >= l[best])) best = e;"),
    ("softmax denominator", "denom += exp(l[ids[(int64_t)t * k + j]] - l0);", "denom += exp(l[ids[(int64_t)t * k + j]]);"),
    ("dropped routing weight", "ot[n] += wj * y[n];", "ot[n] += y[n];"),
    ("dropped shared term", "for (int32_t n = 0; n < H; ++n) ot[n] += y[n];",
     "for (int32_t n = 0; n < H; ++n) ot[n] += 0.0 * y[n];"),
    ("shared gate/up swap", "g += oracle_bf16_to_f64(sh_w13[(int64_t)r * H + k]) * x[k];\n"
     "      u += oracle_bf16_to_f64(sh_w13[(int64_t)(I + r) * H + k]) * x[k];",
     "u += oracle_bf16_to_f64(sh_w13[(int64_t)r * H + k]) * x[k];\n"
     "      g += oracle_bf16_to_f64(sh_w13[(int64_t)(I + r) * H + k]) * x[k];"),
    ("gap from the wrong rank", "gap[t] = l[ids[(int64_t)t * k + k - 1]] - l[next];",
     "gap[t] = l[ids[(int64_t)t * k]] - l[next];"),
    ("permutation not stable", "perm[cursor[e]++] = (int32_t)p;",
     "perm[offsets[e + 1] - 1 - (cursor[e]++ - offsets[e])] = (int32_t)p;"),
    ("RMS mean over H - 1", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)(H - 1) + eps)"),
    ("RMS eps dropped", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
    ("RMS multiplies", "oracle_bf16_to_f64(y[(int64_t)t * H + h]) / d)", "oracle_bf16_to_f64(y[(int64_t)t * H + h]) * d)"),
    ("bf16 subnormal step", "if (qexp < -133) qexp = -133;", "if (qexp < -126) qexp = -126;"),
    ("bf16 ties away from zero", "r = nearbyint(ldexp(a, -qexp));", "r = floor(ldexp(a, -qexp) + 0.5);"),
    ("E4M3 exponent bias 8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("E4M3 subnormal step", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("E4M3 ties to odd", "(d == best_d && (c & 1) == 0 && (best & 1) == 1)", "(d == best_d && (c & 1) == 1 && (best & 1) == 0)"),
    ("E4M3 overflow to NaN", "if (a >= 448.0) return (uint8_t)(sign | 0x7E);", "if (a >= 448.0) return (uint8_t)(sign | 0x7F);"),
    ("LM head scale 240", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 240.0f : 1.0f"),
    ("LM head multiplies by the scale", "(float)oracle_bf16_to_f64(w[(int64_t)v * H + h]) / sv)",
     "(float)oracle_bf16_to_f64(w[(int64_t)v * H + h]) * sv)"),
    ("LM head product drops the scale", "out[(int64_t)t * V + v] = (double)s[v] * acc;", "out[(int64_t)t * V + v] = acc;"),
    ("E2M1 subnormal 0.25", "e == 0 ? 0.5 * m :", "e == 0 ? 0.25 * m :"),
    ("E2M1 exponent bias 0", "ldexp(1.0 + m / 2.0, e - 1)", "ldexp(1.0 + m / 2.0, e)"),
    ("E8M0 bias 128", "ldexp(1.0, (int)c - 127)", "ldexp(1.0, (int)c - 128)"),
    ("MXFP4 scale group shifted", "oracle_e8m0_to_f64(((const uint8_t*)s)[(int64_t)n * (K / 32) + k / 32])",
     "oracle_e8m0_to_f64(((const uint8_t*)s)[(int64_t)n * (K / 32) + (k / 32 + 1) % (K / 32)])"),
    ("FP8 block of 64 columns", "sf[(int64_t)(n / 128) * kb + k / 128]", "sf[(int64_t)(n / 128) * kb + (k / 64) % kb]"),
    ("format ignored by the forward", "expert_fmt(cfg, ex->fmt, ex->w13_q[e]", "expert_fmt(cfg, ORACLE_FMT_INT4_G32, ex->w13_q[e]"),
]


def _gcc():
    return shutil.which("gcc")


def _build(src_text, d):
    src = os.path.join(d, "moe_oracle.c")
    with open(src, "w") as f:
        f.write(src_text)
    shutil.copy(HDR, os.path.join(d, "moe_oracle.h"))
    lib = os.path.join(d, "libmoe_oracle.so")
    subprocess.run([_gcc(), "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", src, "-o", lib, "-lm"],
                   check=True)
    return lib


def _pins_pass(lib):
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode == 0, r.stdout[-400:]


@pytest.fixture(scope="module")
def original():
    with open(SRC) as f:
        return f.read()


@pytest.mark.skipif(_gcc() is None, reason="gcc is needed to build the oracle")
def test_unmutated_copy_passes_the_pins(original, tmp_path):
    ok, tail = _pins_pass(_build(original, str(tmp_path)))
    assert ok, tail


@pytest.mark.skipif(_gcc() is None, reason="gcc is needed to build the oracle")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught_by_a_pin(original, tmp_path, name, old, new):
    assert original.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
    ok, tail = _pins_pass(_build(original.replace(old, new), str(tmp_path)))
    assert not ok, f"mutation '{name}' passed every pin:\n{tail}"
