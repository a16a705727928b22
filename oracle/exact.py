"""Exact-rational checker for tiny inputs -- TEST INFRASTRUCTURE ONLY.

An independent second implementation, in Python ``fractions.Fraction``, of
what ``kq_oracle.c`` computes.  It rounds to binary32/binary16 with its own
routines (round to nearest, ties to even), so every f32 operation of the
q8_1 quantiser and of the GGUF-order Q4_K dequantisation is reproduced as an
exact value followed by one explicit rounding.  The matmul is the exact
rational sum of the products of f32 weights and dequantised activations.

It is slow (pure Python) and meant for inputs of a few superblocks.
"""
from __future__ import annotations

from fractions import Fraction
import math


# ---------------------------------------------------------- roundings ------

def _round_half_even(fr: Fraction) -> int:
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_binary(v: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round v to the binary format with ``mant_bits`` significand bits
    (including the implicit one), minimum normal exponent ``emin`` and
    maximum exponent ``emax``; ties to even; overflow gives +-inf (as float)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # normalise so that 2^e <= a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)  # subnormals share the minimum exponent's quantum
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    q = _round_half_even(a / quantum)
    r = q * quantum
    if r >= Fraction(2) ** (emax + 1):
        return Fraction(sign) * Fraction(10) ** 400  # sentinel for overflow
    return sign * r


def f32(v: Fraction) -> Fraction:
    return round_binary(Fraction(v), 24, -126, 127)


def f16(v: Fraction) -> Fraction:
    return round_binary(Fraction(v), 11, -14, 15)


def f16_bits(v: Fraction, negative: bool | None = None) -> int:
    """Bit pattern of a value already representable in binary16.  ``negative``
    gives the sign of a zero (a nonzero value that rounded to zero keeps its
    sign, as IEEE rounding does)."""
    v = Fraction(v)
    neg = (v < 0) if negative is None else negative
    sign = 0x8000 if neg else 0
    a = abs(v)
    if a == 0:
        return sign
    if a >= Fraction(10) ** 300:
        return sign | 0x7C00
    if a < Fraction(1, 2 ** 14):
        q = a * 2 ** 24
        assert q.denominator == 1
        return sign | int(q)
    e = 0
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    q = a / Fraction(2) ** (e - 10)
    assert q.denominator == 1 and 1024 <= q < 2048
    return sign | ((e + 15) << 10) | (int(q) - 1024)


def f16_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 31
    mant = bits & 1023
    if e == 0:
        return sign * Fraction(mant, 2 ** 24)
    if e == 31:
        raise ValueError("inf/nan")
    return sign * Fraction(1024 + mant) * Fraction(2) ** (e - 25)


def round_half_away(v: Fraction) -> int:
    a = abs(v)
    q = math.floor(a + Fraction(1, 2))
    return q if v >= 0 else -q


# -------------------------------------------------------------- q8_1 -------

def quantize_block(x):
    """x: 32 binary32 values (floats).  Returns (d_bits, s_bits, codes)."""
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    d = f32(amax / 127)
    idv = f32(1 / d) if d != 0 else Fraction(0)
    codes = []
    for v in xs:
        q = round_half_away(f32(v * idv))
        codes.append(max(-127, min(127, q)))
    a = list(xs)
    h = 16
    while h >= 1:
        for i in range(h):
            a[i] = f32(a[i] + a[i + h])
        h //= 2
    return f16_bits(f16(d)), f16_bits(f16(a[0]), negative=a[0] < 0), codes


# ------------------------------------------------------------ weights ------

def _u16(b, off):
    return b[off] | (b[off + 1] << 8)


def q4k_superblock(b):
    """144 bytes -> 256 exact f32 weight values (GGUF order)."""
    d = f16_value(_u16(b, 0))
    dmin = f16_value(_u16(b, 2))
    s = b[4:16]
    sc = [0] * 8
    mn = [0] * 8
    for j in range(8):
        if j < 4:
            sc[j] = s[j] & 63
            mn[j] = s[j + 4] & 63
        else:
            sc[j] = (s[j + 4] & 0xF) | ((s[j - 4] >> 6) << 4)
            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)
    qs = b[16:144]
    out = [None] * 256
    for v in range(256):
        c, rest = divmod(v, 64)
        hi, l = divmod(rest, 32)
        byte = qs[32 * c + l]
        q = (byte >> 4) if hi else (byte & 15)
        j = 2 * c + hi
        D = f32(d * sc[j])
        Mn = f32(dmin * mn[j])
        out[v] = f32(f32(D * q) - Mn)
    return out


def q6k_superblock(b):
    """210 bytes -> 256 exact f32 weight values."""
    d = f16_value(_u16(b, 208))
    ql = b[0:128]
    qh = b[128:192]
    sc = [x - 256 if x > 127 else x for x in b[192:208]]
    out = [None] * 256
    for v in range(256):
        h, rest = divmod(v, 128)
        g, l = divmod(rest, 32)
        lowbyte = ql[64 * h + 32 * (g % 2) + l]
        low = (lowbyte & 15) if g < 2 else (lowbyte >> 4)
        high = (qh[32 * h + l] >> (2 * g)) & 3
        q = (low | (high << 4)) - 32
        out[v] = f32(f32(d * sc[v // 16]) * q)
    return out


def weights(kind: str, row_bytes, k: int):
    row_bytes = [int(v) for v in row_bytes]
    out = []
    step = 144 if kind == "q4k" else 210
    fn = q4k_superblock if kind == "q4k" else q6k_superblock
    for s in range(k // 256):
        out.extend(fn(row_bytes[s * step:(s + 1) * step]))
    return out


def activation(xq_row, k: int):
    xq_row = [int(v) for v in xq_row]
    out = []
    for b in range(k // 32):
        blk = xq_row[b * 36:(b + 1) * 36]
        d8 = f16_value(_u16(blk, 0))
        for i in range(32):
            c = blk[4 + i]
            out.append(d8 * (c - 256 if c > 127 else c))
    return out


def dot(kind: str, w_row, xq_row, k: int, residual=None):
    """Exact value of one output, and sum of |products| (for error bounds)."""
    w = weights(kind, w_row, k)
    x = activation(xq_row, k)
    tot = sum(wi * xi for wi, xi in zip(w, x))
    mag = sum(abs(wi * xi) for wi, xi in zip(w, x))
    if residual is not None:
        tot += Fraction(float(residual))
        mag += abs(Fraction(float(residual)))
    return tot, mag
