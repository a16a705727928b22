"""Each plausible mistake in the oracle must fail at least one pin.

The mistakes are planted in copies of ``oracle/kq_oracle.c`` compiled into a
temporary directory, on the CPU; the real oracle is never modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kq_oracle.c")

# (label, exact text in kq_oracle.c, replacement)
MUTANTS = [
    ("q4k nibbles swapped",
     "y[64 * c + l] = D0 * (float)(q & 15) - M0;", "y[64 * c + l] = D0 * (float)(q >> 4) - M0;"),
    ("q4k min sign",
     "y[64 * c + 32 + l] = D1 * (float)(q >> 4) - M1;", "y[64 * c + 32 + l] = D1 * (float)(q >> 4) + M1;"),
    ("q4k high scale bits dropped",
     "sc[j] = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);", "sc[j] = (s[j + 4] & 0x0F);"),
    ("q4k high min bits from wrong byte",
     "mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);", "mn[j] = (s[j + 4] >> 4) | ((s[j - 4] >> 6) << 4);"),
    ("q4k scale and min transposed",
     "float D0 = d * (float)sc[2 * c], M0 = dmin * (float)mn[2 * c];",
     "float D0 = d * (float)mn[2 * c], M0 = dmin * (float)sc[2 * c];"),
    ("q4k d and dmin swapped",
     "float d = h2f(rd16(b)), dmin = h2f(rd16(b + 2));", "float dmin = h2f(rd16(b)), d = h2f(rd16(b + 2));"),
    ("q6k offset 31",
     "y[v] = (d * (float)sc[v / 16]) * (float)(q6k_code(b, v) - 32);",
     "y[v] = (d * (float)sc[v / 16]) * (float)(q6k_code(b, v) - 31);"),
    ("q6k scale index v/32",
     "y[v] = (d * (float)sc[v / 16]) * (float)(q6k_code(b, v) - 32);",
     "y[v] = (d * (float)sc[v / 32]) * (float)(q6k_code(b, v) - 32);"),
    ("q6k qh shift g",
     "int high = (qh[32 * h + l] >> (2 * g)) & 3;", "int high = (qh[32 * h + l] >> g) & 3;"),
    ("q6k ql half swapped",
     "int lowbyte = ql[64 * h + (g & 1) * 32 + l];", "int lowbyte = ql[64 * h + (g >> 1) * 32 + l];"),
    ("q8 constant 128", "float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    ("q8 ties to even", "float v = roundf(x[i] * id);", "float v = rintf(x[i] * id);"),
    ("q8 division instead of reciprocal", "float v = roundf(x[i] * id);", "float v = roundf(x[i] / d);"),
    ("q8 sequential source sum",
     "for (int i = 0; i < h; ++i) a[i] = a[i] + a[i + h];",
     "for (int i = 0; i < h; ++i) a[i] = (h == 16 && i == 0) ? (float)({double t = 0; for (int z = 0; z < 32; ++z) t += x[z]; t;}) : a[i] * (h == 16 ? 0.0f : 1.0f);"),
    ("f16 ties away", "double q = nearbyint(ldexp(v, 10 - E));", "double q = floor(ldexp(v, 10 - E) + 0.5);"),
    ("q8 dequant from the source sum",
     "float d8 = h2f(rd16(blk));", "float d8 = h2f(rd16(blk + 2));"),
    ("residual dropped", "acc += (double)*res;", "(void)0;"),
    ("den signed", "dsum += fabs(T);", "dsum += T;"),
    ("last block dropped", "for (int64_t j = 0; j < k / 32; ++j) {", "for (int64_t j = 0; j < k / 32 - 1; ++j) {"),
    ("products in f32", "double p = (double)wr[32 * j + i] * (double)xr[32 * j + i];",
     "double p = (double)(wr[32 * j + i] * xr[32 * j + i]);"),
    ("rms sum in natural order", "        a[l] = acc;",
     "        a[l] = l ? 0.0f : ({float t = 0.0f; for (int64_t i = 0; i < n; ++i) t = fmaf(h[i], h[i], t); t;});"),
    ("rms reciprocal dropped", "float r = 1.0f / sqrtf(ss / (float)n + eps);",
     "float r = sqrtf(ss / (float)n + eps);"),
    ("rms eps outside the root", "float r = 1.0f / sqrtf(ss / (float)n + eps);",
     "float r = 1.0f / (sqrtf(ss / (float)n) + eps);"),
    ("rms mean over n-1", "float r = 1.0f / sqrtf(ss / (float)n + eps);",
     "float r = 1.0f / sqrtf(ss / (float)(n - 1) + eps);"),
    ("rms residual dropped", "h[i] = res ? x[row * n + i] + res[row * n + i] : x[row * n + i];",
     "h[i] = x[row * n + i];"),
    ("rms gain dropped", "for (int64_t i = 0; i < n; ++i) yr[i] = (h[i] * r) * g[i];",
     "for (int64_t i = 0; i < n; ++i) yr[i] = h[i] * r;"),
    ("silu sign", "static float silu_f32(float t) { return t / (1.0f + exp_f32(-t)); }",
     "static float silu_f32(float t) { return t / (1.0f + exp_f32(t)); }"),
    ("exp degree 5", "    p = fmaf(p, r, 1.0f / 720.0f);", "    p = 0.0f;"),
    ("exp second reduction constant dropped", "    r = fmaf(-k, -2.12194440054690583e-4f, r);", "    (void)0;"),
    ("exp saturation at the wrong end", "    if (a < -110.0f) return 0.0f;", "    if (a < -110.0f) return INFINITY;"),
    ("q8 NaN product coded -127", "if (v != v) v = 0.0f;", "if (v != v) v = -127.0f;"),
    ("swiglu up dropped", "yr[i] = silu_f32(gate[row * n + i]) * up[row * n + i];",
     "yr[i] = silu_f32(gate[row * n + i]);"),
]


def _fails_some_pin(path):
    with oracle.using_library(path):
        for pin in PINS:
            try:
                pin(oracle)
            except AssertionError:
                return pin.__name__
            except Exception as e:  # a crash on bad data also counts as caught
                return f"{pin.__name__} ({type(e).__name__})"
    return None


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(label, old, new, tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {label!r} not unique"
    mutant = os.path.join(tmp_path, "mutant.c")
    with open(mutant, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp_path, "libmutant.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-w", "-o", lib, mutant, "-lm"])
    caught = _fails_some_pin(lib)
    assert caught, f"mutant {label!r} passed every pin"
