"""The oracle's pins catch plausible mistakes.

Each mutant below is a copy of oracle/oracle.c with one planted mistake of
the kind a careful reader could still make: a dropped term, a rounding taken
twice or at the wrong point, a wrong sign, index or stride, a swapped
operand, a misplaced tie rule. Every mutant is compiled with the oracle's
own flags and the pinning tests (test_oracle_codecs.py, test_oracle_ops.py)
run against it in a subprocess; each mutant must make at least one pin fail.
The unmodified source, compiled the same way, must pass them all.

CPU only. The mistakes are planted in the oracle, never in GPU code.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
PIN_TESTS = [os.path.join(ROOT, "tests", "test_oracle_codecs.py"),
             os.path.join(ROOT, "tests", "test_oracle_ops.py")]

# name -> [(exact text in oracle.c, replacement[, occurrences]), ...]
MUTANTS = {
    "bf16 ties round away from zero": [
        ("r = (bf16_bits_of_representable(lo) & 1u) ? hi : lo; /* tie: even */", "r = hi;")],
    "bf16 subnormal spacing off by one binade": [
        ("if (m < 0x1p-126) return 0x1p-133;", "if (m < 0x1p-126) return 0x1p-134;")],
    "exact sum rounded twice (TwoSum error dropped)": [
        ("    return bf16_round(s, err);\n}", "    return bf16_round(s, 0.0 * err);\n}")],
    "E4M3 ties round up": [
        ("else c = (lo & 1) ? hi : lo; /* tie: even code (even mantissa) */", "else c = hi;")],
    "E4M3 subnormal exponent wrong": [
        ("ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)")],
    "E2M1 ties round down": [
        ("else c = (lo & 1) ? hi : lo; /* tie: even code */\n    return (uint8_t)(sign | c);\n}\n\nvoid",
         "else c = lo;\n    return (uint8_t)(sign | c);\n}\n\nvoid")],
    "LayerNorm epsilon dropped": [
        ("*factor32 = (float)(1.0 / sqrt(var + (double)eps));", "*factor32 = (float)(1.0 / sqrt(var));")],
    "LayerNorm variance unbiased": [
        ("const double var = ss / (double)n;", "const double var = ss / (double)(n - 1);")],
    "normalised row not rounded to bf16": [
        ("const float norm = bf(oracle_bf16_from_f32(t));", "const float norm = t;")],
    "modulation uses scale instead of 1 + scale": [
        ("const float one_plus_scale = 1.0f + bf(scale[j]);", "const float one_plus_scale = bf(scale[j]);")],
    "FP8 multiplies by the scale instead of its reciprocal": [
        ("const float scaled = bf(y[j]) * inv;", "const float scaled = bf(y[j]) / inv;")],
    "gated residual: bias add not rounded to bf16": [
        ("if (bias) xb = bf(oracle_bf16_from_f32(xb + bf(bias[j])));", "if (bias) xb = xb + bf(bias[j]);")],
    "gated residual rounded twice": [
        ("rr[j] = oracle_bf16_of_exact_sum(product, (double)bf(resr[j]));",
         "rr[j] = oracle_bf16_from_f32((float)product + bf(resr[j]));")],
    "RMSNorm epsilon dropped": [
        ("return (float)(1.0 / sqrt(ms + (double)eps));", "return (float)(1.0 / sqrt(ms));")],
    "RMSNorm weight dropped": [
        ("scratch[i] = oracle_bf16_from_f32(t * bf(w[i]));", "scratch[i] = oracle_bf16_from_f32(t);")],
    "RoPE rotates the wrong way": [
        ("out[2 * p] = oracle_bf16_of_exact_sum(n0 * c, -(n1 * s));",
         "out[2 * p] = oracle_bf16_of_exact_sum(n0 * c, n1 * s);"),
        ("out[2 * p + 1] = oracle_bf16_of_exact_sum(n1 * c, n0 * s);",
         "out[2 * p + 1] = oracle_bf16_of_exact_sum(n1 * c, -(n0 * s));")],
    "RoPE pairs halves (NeoX) instead of neighbours": [
        ("const double n0 = (double)bf(scratch[2 * p]);", "const double n0 = (double)bf(scratch[p]);"),
        ("const double n1 = (double)bf(scratch[2 * p + 1]);",
         "const double n1 = (double)bf(scratch[p + head_dim / 2]);")],
    "RoPE cos/sin swapped": [
        ("const double c = (double)cos_row[p];\n        const double s = (double)sin_row[p];",
         "const double c = (double)sin_row[p];\n        const double s = (double)cos_row[p];")],
    "joint layout puts image rows first": [
        ("const int is_txt = j < txt_rows;\n        const int64_t i = is_txt ? j : j - txt_rows;",
         "const int is_txt = j >= img_rows;\n        const int64_t i = is_txt ? j - img_rows : j;")],
    "bias_mul_add rounded twice": [
        ("y[o] = oracle_bf16_of_exact_sum(product, (double)bf(residual[o]));",
         "y[o] = oracle_bf16_from_f32((float)product + bf(residual[o]));")],
    "bias_mul_add: bias add not rounded to bf16": [
        ("const float b = bias ? bf(oracle_bf16_from_f32(bf(x[o]) + bf(bias[j])))",
         "const float b = bias ? (bf(x[o]) + bf(bias[j]))")],
    "token cat reads the MLP branch with the attention stride": [
        ("memcpy(dst + a_cols, b + r * b_cols,", "memcpy(dst + a_cols, b + r * a_cols,")],
    "FP4 scale divides the group maximum by 4": [
        ("const float sp = (amax / 6.0f) * g;", "const float sp = (amax / 4.0f) * g;")],
    "FP4 element scale inverted": [
        ("g / (float)oracle_e4m3_decode(s8)", "(float)oracle_e4m3_decode(s8) / g")],
    "FP4 nibbles swapped": [
        ("(uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));", "(uint8_t)(codes[2 * k + 1] | (codes[2 * k] << 4));")],
    "FP4 pad-row scales not zero": [
        ("memset(scales, 0, (size_t)(rows_padded * groups));", "memset(scales, 0x38, (size_t)(rows_padded * groups));", 2)],
    "norm FP4 quantises the input row instead of y": [
        ("y + r * hidden, hidden, g);", "x + r * hidden, hidden, g);")],
    "128x4 scale layout with the 32 and 4 row factors swapped": [
        ("const int64_t inner = (r % 32) * 16 + (r / 32) * 4 + k % 4;",
         "const int64_t inner = (r % 4) * 128 + (r / 4) * 4 + k % 4;")],
    "128x4 scale layout with tiles in column order": [
        ("const int64_t tile = (m / 128) * tiles_per_row + k / 4;",
         "const int64_t tile = (k / 4) * (rows_padded / 128) + m / 128;")],
    "residual norm FP4 normalises x instead of the new residual": [
        ("oracle_norm_modulate_fp4(y, packed, scales, s_pre, pre, r_out, scale, shift, g, rows,",
         "oracle_norm_modulate_fp4(y, packed, scales, s_pre, pre, x, scale, shift, g, rows,")],
    "RMS inverse through binary32 sqrt and division": [
        ("return (float)(1.0 / sqrt(ms + (double)eps));",
         "return 1.0f / sqrtf((float)(ms + (double)eps));")],
    "RMSNorm mean of squares over n - 1": [
        ("const double ms = ss / (double)n;", "const double ms = ss / (double)(n - 1);")],
    "RMSNorm weight applied to the inverse first": [
        ("const float t = bf(x[i]) * inv;\n        scratch[i] = oracle_bf16_from_f32(t * bf(w[i]));",
         "const float t = inv * bf(w[i]);\n        scratch[i] = oracle_bf16_from_f32(bf(x[i]) * t);")],
    "RoPE products rounded to binary32": [
        ("out[2 * p] = oracle_bf16_of_exact_sum(n0 * c, -(n1 * s));",
         "out[2 * p] = oracle_bf16_of_exact_sum((float)(n0 * c), -(double)(float)(n1 * s));"),
        ("out[2 * p + 1] = oracle_bf16_of_exact_sum(n1 * c, n0 * s);",
         "out[2 * p + 1] = oracle_bf16_of_exact_sum((float)(n1 * c), (float)(n0 * s));")],
    "LayerNorm sum accumulated in binary32": [
        ("double sum = 0.0;\n    for (int64_t i = 0; i < n; ++i) sum += (double)bf(v[i]);",
         "float sum = 0.0f;\n    for (int64_t i = 0; i < n; ++i) sum += bf(v[i]);")],
    "modulation multiply and add rounded separately": [
        ("const float modulated = fmaf(norm, one_plus_scale, bf(shift[j]));",
         "const float modulated = norm * one_plus_scale + bf(shift[j]);")],
    "FP4 scale as amax * (g / 6)": [
        ("const float sp = (amax / 6.0f) * g;", "const float sp = amax * (g / 6.0f);")],
    "FP4 scale as (amax * g) / 6": [
        ("const float sp = (amax / 6.0f) * g;", "const float sp = (amax * g) / 6.0f;")],
    "FP4 element value as (x * g) / scale": [
        ("const float t = bf(grp[k]) * kscale;",
         "const float t = (s8 == 0) ? 0.0f : (bf(grp[k]) * g) / (float)oracle_e4m3_decode(s8);")],
}


def _mutate(source, edits):
    """Applies (old, new) or (old, new, count) edits; `old` must occur exactly
    once (or `count` times, all replaced)."""
    for old, new, *count in edits:
        n = count[0] if count else 1
        assert source.count(old) == n, f"mutation anchor not found exactly {n} times: {old!r}"
        source = source.replace(old, new)
    return source


def _run_pins(lib_path):
    env = dict(os.environ, DIT_ORACLE_LIB=lib_path, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu"]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:]


def _build_and_run(tmp, name, source):
    import oracle

    slug = "".join(ch if ch.isalnum() else "_" for ch in name)[:60]
    src = os.path.join(tmp, f"{slug}.c")
    lib = os.path.join(tmp, f"{slug}.so")
    with open(src, "w") as f:
        f.write(source)
    oracle.compile_source(src, lib)
    return _run_pins(lib)


def test_every_planted_mistake_fails_a_pin():
    with open(ORACLE_C) as f:
        original = f.read()
    sources = {name: _mutate(original, edits) for name, edits in MUTANTS.items()}
    with tempfile.TemporaryDirectory() as tmp:
        # The harness itself: the unmodified oracle passes every pin.
        rc, out = _build_and_run(tmp, "unmodified", original)
        assert rc == 0, "the unmodified oracle must pass its pins:\n" + out
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = dict(zip(sources, ex.map(lambda kv: _build_and_run(tmp, *kv),
                                               sources.items())))
    survivors = [name for name, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
    broken = {name: out for name, (rc, out) in results.items() if rc not in (0, 1)}
    assert not broken, f"pin runs that errored instead of failing: {broken}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutation_anchor_is_unique(name):
    with open(ORACLE_C) as f:
        _mutate(f.read(), MUTANTS[name])
