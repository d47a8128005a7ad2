"""Exact-rational reference for tiny inputs -- TEST INFRASTRUCTURE ONLY.

A second, independent route to the same numbers as oracle.c, written from the definitions
rather than from the algorithm's steps, used to pin oracle.c on small inputs:

* every weight is formed as an exact rational from its binary16 scales and integer fields
  (rustdoc "Module numerics", Structs Scale / Segment / CodedRow);
* the activation scale is found by brute force over every candidate m * 2^e near amax/127
  (Functions wide_scale / block_scale), and each code is Python's round-half-even of the
  exact quotient (Functions rne_div / rne);
* a block's (or 256-element group's) value is the exact dot of the exact weights with the
  dequantized activations, sum(w_i * c_i * s_i), which the method's two-term / sixteen-term
  exact sums equal (module description; rustdoc "Module lane", description);
* binary32 rounding is done on Fractions: nearest, ties to even, on the gradual-underflow
  grid, overflow to infinity, then a subnormal flushed to a zero of its sign (Functions
  scaled_to_f32, ftz); fadd is the same rounding of the exact sum of two binary32 values.

The SUM_WINDOW floor is not modelled here (the exact sum is used whole); the tests that pin
the window build their terms explicitly.  Slow by design: pure Python.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np

F0 = Fraction(0)


def f16_value(h: int) -> Fraction:
    """binary16 bits -> exact value; raises on inf/NaN (an Unreadable block)."""
    s, E, M = (h >> 15) & 1, (h >> 10) & 31, h & 1023
    if E == 31:
        raise ValueError("unreadable block scale")
    v = Fraction(M, 1 << 24) if E == 0 else Fraction(1024 + M) * Fraction(2) ** (E - 25)
    return -v if s else v


def f32_value(x) -> Fraction:
    """binary32 value (finite) -> exact Fraction."""
    return Fraction(float(np.float32(x)))


def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]


def bits_f32(u: int) -> np.float32:
    return np.frombuffer(struct.pack("<I", u & 0xFFFFFFFF), dtype=np.float32)[0]


def ftz(x) -> np.float32:
    u = f32_bits(x)
    if (u & 0x7F800000) == 0:
        u &= 0x80000000
    return bits_f32(u)


def _floor_log2(a: Fraction) -> int:
    """floor(log2 a) for a > 0, exactly."""
    k = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** k > a:
        k -= 1
    while Fraction(2) ** (k + 1) <= a:
        k += 1
    return k


def round_f32(x: Fraction, negative_zero: bool = False) -> np.float32:
    """Nearest binary32 to x, ties to even, on the gradual-underflow grid; overflow -> inf;
    then a subnormal result -> zero of its sign.  x == 0 -> +0 (or -0 if negative_zero)."""
    if x == 0:
        return bits_f32(0x80000000 if negative_zero else 0)
    sign = 0x80000000 if x < 0 else 0
    a = abs(x)
    k = _floor_log2(a)
    qexp = max(k - 23, -149)
    quantum = Fraction(2) ** qexp
    n = round(a / quantum)                      # Fraction.__round__: half to even
    val = n * quantum
    if val >= Fraction(2) ** 128:
        return bits_f32(sign | 0x7F800000)
    if val < Fraction(2) ** -126:
        return bits_f32(sign)                   # flushed (includes a rounding to 0)
    f = float(val)                              # exact: val is a normal binary32 value
    return bits_f32(f32_bits(f) | sign)


def fadd(a, b) -> np.float32:
    """binary32 add with ftz of the result (operands are normal or zero here)."""
    fa, fb = np.float32(a), np.float32(b)
    if np.isinf(fa) or np.isinf(fb) or np.isnan(fa) or np.isnan(fb):
        with np.errstate(all="ignore"):
            return np.float32(fa + fb)
    s = f32_value(fa) + f32_value(fb)
    if s == 0:
        # IEEE: an exact zero sum is +0 unless both operands are -0
        both_neg = (f32_bits(fa) >> 31) and (f32_bits(fb) >> 31)
        return bits_f32(0x80000000 if both_neg else 0)
    return round_f32(s)


# --- activation quantization ---------------------------------------------------------------

def least_scale(amax: Fraction, bits: int) -> tuple[int, int]:
    """Brute force: among all m * 2^e with m of exactly `bits` significant bits and e within
    a wide window around amax/127, the least one with 127 * m * 2^e >= amax."""
    lo, hi = 1 << (bits - 1), (1 << bits) - 1
    t = amax / 127
    k = _floor_log2(t)
    best = None
    for e in range(k - bits - 6, k + 6):
        for m in range(lo, hi + 1):
            v = Fraction(m) * Fraction(2) ** e
            if 127 * v >= amax and (best is None or v < best[0]):
                best = (v, m, e)
    return best[1], best[2]


def quantize_block(x: np.ndarray, bits: int):
    """One activation block -> (m, e, codes) with the readings of oracle.c (ftz'd reads,
    NaN code 0 and passed over, all-zero block -> (2^(bits-1), 0))."""
    vals = []
    for v in x:
        f = ftz(v)
        vals.append(None if np.isnan(f) else f32_value(f))
    finite = [abs(v) for v in vals if v is not None]
    amax = max(finite) if finite else F0
    if amax == 0:
        m, e = 1 << (bits - 1), 0
    else:
        m, e = least_scale(amax, bits)
    s = Fraction(m) * Fraction(2) ** e
    codes = [0 if v is None else round(v / s) for v in vals]
    assert all(abs(c) <= 127 for c in codes)
    return m, e, codes


def quantize(x: np.ndarray, mode: int, blk: int = 256):
    """Row x (1-D f32) -> (codes list, [(m, e)] per activation block).  PerBlock blocks are
    `blk` elements (the weight format's own block) with 8 bits, Sub32 blocks 32 with 4."""
    blk, bits = (blk, 8) if mode == 0 else (32, 4)
    codes, scales = [], []
    for b in range(len(x) // blk):
        m, e, c = quantize_block(x[b * blk:(b + 1) * blk], bits)
        codes += c
        scales.append((m, e))
    return codes, scales


# --- weights and the dot -------------------------------------------------------------------

def q4k_weights(f: dict, r: int) -> list[Fraction]:
    """Exact weights of row r: w = d*sc*q - dmin*mn."""
    C = f["cols"]
    w = []
    for i in range(C):
        b, j = i // 256, i // 32
        d = f16_value(int(f["d"][r, b]))
        dm = f16_value(int(f["dmin"][r, b]))
        w.append(d * int(f["sc"][r, j]) * int(f["q"][r, i]) - dm * int(f["mn"][r, j]))
    return w


def q6k_weights(f: dict, r: int) -> list[Fraction]:
    """Exact weights of row r: w = d*sc*(q - 32)."""
    C = f["cols"]
    return [f16_value(int(f["d"][r, i // 256])) * int(f["sc"][r, i // 16]) * (int(f["q"][r, i]) - 32)
            for i in range(C)]


def b32_weights(f: dict, r: int) -> list[Fraction]:
    """Exact weights of row r of a 32-element-block matrix: Q8_0-style w = d*q (int8 q),
    Q4_0-style w = d*(q - 8)."""
    off = 0 if f["fmt"] == "q8_0" else 8
    return [f16_value(int(f["d"][r, i // 32])) * (int(f["q"][r, i]) - off) for i in range(f["cols"])]


def dot_row(weights: list[Fraction], codes: list[int], scales: list[tuple[int, int]], mode: int,
            ablk: int = 256, piece: int = 256) -> np.float32:
    """Row value: per piece (`piece` elements: the weight block under PerBlock, the 256-element
    group under Sub32) the exact sum(w_i * c_i * s_i), rounded once, the rounded pieces added
    in order from +0; NaN -> 0x7FC00000.  Activation scales cover `ablk` elements."""
    if mode != 0:
        ablk = 32
    y = np.float32(0.0)
    for b in range(len(weights) // piece):
        X = F0
        for i in range(b * piece, (b + 1) * piece):
            m, e = scales[i // ablk]
            X += weights[i] * codes[i] * m * Fraction(2) ** e
        y = fadd(y, round_f32(X))
    if np.isnan(y):
        y = bits_f32(0x7FC00000)
    return y


def gemv(f: dict, x: np.ndarray, mode: int) -> np.ndarray:
    """All rows of a tiny matrix against one f32 activation row."""
    b32 = f["fmt"] in ("q8_0", "q4_0")
    blk = 32 if b32 else 256
    codes, scales = quantize(np.asarray(x, np.float32).reshape(-1), mode, blk)
    wfun = {"q4k": q4k_weights, "q6k": q6k_weights}.get(f["fmt"], b32_weights)
    piece = 32 if (b32 and mode == 0) else 256
    return np.array([dot_row(wfun(f, r), codes, scales, mode, blk, piece) for r in range(f["rows"])],
                    dtype=np.float32)
