"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/hbl_oracle.c (a wrong rounding rule, a
butterfly sign, a dropped scale factor, a transposed operand, a wrong bit layout, ...),
builds that copy, and runs the oracle's pin tests against it in a subprocess: at least one
pin must fail.  A control case builds the unchanged source the same way and must pass, so
a failure of the harness itself cannot pass for a caught mistake.  CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hbl_oracle.c")
PIN_FILES = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f != os.path.basename(__file__))

# (name, text to replace, replacement, which occurrence of the text, 0-based)
MUTATIONS = [
    ("weights: ties away from zero", "float r = rintf(W[n * K + k] / alpha);",
     "float r = roundf(W[n * K + k] / alpha);", 0),
    ("alpha: half the mean", "S += row_sum[n];", "S += row_sum[n] * 0.5;", 0),
    ("fwht f32: butterfly sign", "v[j + h] = a - b;", "v[j + h] = b - a;", 0),
    ("fwht f64: butterfly sign", "v[j + h] = a - b;", "v[j + h] = b - a;", 1),
    ("fwht f32: stages in descending order", "for (int64_t h = 1; h < n; h *= 2)",
     "for (int64_t h = n / 2; h >= 1; h /= 2)", 0),
    ("rms: sum of x instead of x^2", "ss += (double)xf * (double)xf;", "ss += (double)xf;", 0),
    ("absmean: sum of z instead of |z|", "sa += (double)fabsf(z[k]);", "sa += (double)z[k];", 0),
    ("absmean codes: ties away from zero", "float v = rintf(z[k] * s);", "float v = roundf(z[k] * s);", 0),
    ("absmax codes: ties away from zero", "float v = rintf(z[k] * s);", "float v = roundf(z[k] * s);", 1),
    ("absmean deq: 1/sqrt(K) dropped", "d = d * hK;", "d = d;", 0),
    ("absmax deq: 1/sqrt(K) dropped", "d = d * hK;", "d = d;", 1),
    ("deq: RMS factor dropped", "d = d * r;", "d = d;", 0),
    ("absmean: scale guard only at zero", "if (b < 0x1p-120f) {", "if (b == 0.0f) {", 0),
    ("absmax: scale guard only at zero", "if (g < 0x1p-120f) {", "if (g == 0.0f) {", 0),
    ("qkv: scale guard only at zero", "const float s = g < 0x1p-120f ? 0.0f", "const float s = g == 0.0f ? 0.0f", 0),
    ("gemm: transposed weights", "s += (int32_t)q[m * K + k] * (int32_t)T[n * K + k];",
     "s += (int32_t)q[m * K + k] * (int32_t)T[k * N + n];", 0),
    ("dequant: scales multiplied first", "float v = (float)acc[m * N + n] * deq[m];\n      y[m * N + n] = v * alpha;",
     "y[m * N + n] = (float)acc[m * N + n] * (deq[m] * alpha);", 0),
    ("weight packing: natural field order", "int p = 4 * (c % 4) + c / 4;", "int p = c;", 0),
    ("INT4 packing: natural nibble order", "int c0 = (j % 4) + 8 * (j / 4);", "int c0 = 2 * j;", 0),
    ("swiglu: sign of the exponent", "double s = gv / (1.0 + exp(-gv));", "double s = gv / (1.0 + exp(gv));", 0),
    ("bf16: truncation", "const double v = rint((double)f / q) * q;", "const double v = trunc((double)f / q) * q;", 0),
    ("qkv: offset dropped", "v = rintf(v + c);", "v = rintf(v);", 0),
    ("qkv: scale over g instead of 2g", "const float s = g < 0x1p-120f ? 0.0f : L / (2.0f * g);",
     "const float s = g < 0x1p-120f ? 0.0f : L / g;", 0),
    ("b-bit packing: MSB first", "if ((v >> b) & 1u) out[r * rb + bit / 8] |= (uint8_t)(1u << (bit % 8));",
     "if ((v >> b) & 1u) out[r * rb + bit / 8] |= (uint8_t)(1u << (7 - bit % 8));", 0),
    ("fp6: exponent bias dropped", "code = ((e + 1u) << 3) | m;", "code = (e << 3) | m;", 0),
    ("fp4: sign in bit 2", "nib[i] = t == 0 ? 0u : ((t < 0 ? 8u : 0u) | 2u);",
     "nib[i] = t == 0 ? 0u : ((t < 0 ? 4u : 0u) | 2u);", 0),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.find(old, start + 1)
        if start < 0:
            return None
    return text[:start] + new + text[start + len(old):]


def _run_pins(tmp_path, source):
    sys.path.insert(0, ROOT)
    import oracle.oracle as oo

    src = tmp_path / "hbl_oracle.c"
    src.write_text(source)
    lib = tmp_path / "liboracle.so"
    subprocess.run(oo.compile_command(str(src), str(lib)), check=True, capture_output=True)
    env = dict(os.environ, HBL_ORACLE_LIB=str(lib), OMP_NUM_THREADS=os.environ.get("OMP_NUM_THREADS", "4"))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                           *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_control_unchanged_source_passes(tmp_path):
    r = _run_pins(tmp_path, open(SRC).read())
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new,nth", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, nth):
    mutated = _replace_nth(open(SRC).read(), old, new, nth)
    assert mutated is not None, f"the oracle no longer contains occurrence {nth} of: {old}"
    r = _run_pins(tmp_path, mutated)
    assert r.returncode == 1 and " failed" in r.stdout, f"{name}: no pin failed\n{r.stdout[-1500:]}"
