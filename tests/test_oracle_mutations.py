"""The pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of the C oracle (a dropped term, a wrong
sign, index or operand order, a truncating cast, a missing clamp, a wrong block
or scale rule), rebuilds it in a scratch directory and runs the pins against the
mutant: at least one pin must fail.  The oracle in the repository is never
touched.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "c", "rnl_oracle.c")

# name -> (text in the oracle, replacement)
MUTATIONS = {
    "sum of squares drops the last term": (
        "for (int64_t k = 0; k < K; ++k) {\n    const double v = (double)bf16_to_f32(x[k]);",
        "for (int64_t k = 0; k < K - 1; ++k) {\n    const double v = (double)bf16_to_f32(x[k]);"),
    "eps dropped": ("const float var = ms + eps;\n  const float sd = sqrtf(var);",
                    "const float var = ms;\n  const float sd = sqrtf(var);"),
    "1/K off by one": ("const float c = 1.0f / (float)K;\n  return (float)S * c;",
                       "const float c = 1.0f / (float)(K + 1);\n  return (float)S * c;"),
    "rstd off by a little": ("return 1.0f / sd;", "return 1.0f / sd + 1e-7f;"),
    "gamma applied before rstd": (
        "float v = bf16_to_f32(x[k]) * r;\n    if (c->gamma != NULL) v = v * bf16_to_f32(c->gamma[k]); "
        "/* (x * rstd) * gamma: two roundings */",
        "float v = bf16_to_f32(x[k]);\n    if (c->gamma != NULL) v = v * bf16_to_f32(c->gamma[k]);\n    v = v * r;"),
    "bf16 cast truncates": ("return (uint16_t)(((uint64_t)u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)(u >> 16);"),
    "normed rows not cast to bf16": ("for (int64_t i = 0; i < T * K; ++i) a[i] = bf16_round(n[i]);",
                                     "for (int64_t i = 0; i < T * K; ++i) a[i] = n[i];"),
    "bf16 weight transposed": (
        "for (int64_t k = 0; k < c->K; ++k) acc += (double)a[k] * (double)bf16_to_f32(w[k]);",
        "for (int64_t k = 0; k < c->K; ++k) acc += (double)a[k] * (double)bf16_to_f32(c->wb[k * c->N + j]);"),
    "fp32 weight transposed": (
        "for (int64_t k = 0; k < c->K; ++k) acc += (double)a[k] * (double)w[k];",
        "for (int64_t k = 0; k < c->K; ++k) acc += (double)a[k] * (double)c->wf[k * c->N + j];"),
    "quant rounds half away from zero": ("float r = rintf(n * s);", "float r = roundf(n * s);"),
    "quant does not saturate": ("if (r > 127.0f) r = 127.0f;", "if (r > 200.0f) r = 127.0f;"),
    "quant scale inverted": ("const float s = amax == 0.0f ? 0.0f : 127.0f / amax;",
                             "const float s = amax == 0.0f ? 0.0f : amax / 127.0f;"),
    "int8 weight transposed": (
        "for (int64_t k = 0; k < c->K; ++k) s += (int64_t)a[k] * (int64_t)w[k];",
        "for (int64_t k = 0; k < c->K; ++k) s += (int64_t)a[k] * (int64_t)c->w[k * c->N + j];"),
    "dequant drops the weight scale": ("const float sm = x_scale[t] * w_scale[j];", "const float sm = x_scale[t];"),
    "residual add truncates": (
        "for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(bf16_to_f32(x[i]) + bf16_to_f32(r[i]));",
        "for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)(((uint32_t)x[i] << 16) + ((uint32_t)r[i] << 16) >> 16);"),
    "rope sign flipped": ("n[i] = a - b;", "n[i] = a + b;"),
    "rope pairs neighbours": ("const float lo = n[i], hi = n[i + h];", "const float lo = n[2 * i], hi = n[2 * i + 1];"),
    "head gamma skipped": ("if (gamma != NULL) v = v * bf16_to_f32(gamma[k]);\n        n[k] = v;", "n[k] = v;"),
    "e4m3 exponent bias": ("code = (uint8_t)(((e + 7) << 3) | m);", "code = (uint8_t)(((e + 8) << 3) | m);"),
    "e4m3 does not saturate": ("if (r > 448.0) r = 448.0;", "if (r > 480.0) r = 448.0;"),
    "mx scale rounds the exponent up": ("sh = E - 1 - 8;", "sh = E - 8;"),
    "mx blocks of 32": ("const uint8_t s = sc[r * nb + k / 64];", "const uint8_t s = sc[r * nb + (k / 32) % nb];"),
}


@pytest.fixture(scope="module")
def source():
    return open(SRC).read()


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, source, tmp_path):
    before, after = MUTATIONS[name]
    assert source.count(before) == 1, f"the text to mutate is not unique in the oracle: {before!r}"
    for d in ("oracle", "synthetic", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    (tmp_path / "oracle" / "c" / "rnl_oracle.c").write_text(source.replace(before, after))
    subprocess.run([sys.executable, "-m", "oracle.build_oracle"], cwd=tmp_path, check=True, capture_output=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-k", "c]",
                        "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode == 1, f"no pin fails with '{name}' planted\n{r.stdout[-2000:]}"
