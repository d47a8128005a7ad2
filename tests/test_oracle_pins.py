"""Pins of the CPU oracle against things other than itself (no GPU).

Each test fixes part of oracle.c with a closed form, an invariant, a library routine or an
exact-rational brute force (oracle/exact.py), chosen so that a plausible mistake in the
oracle fails at least one of them (test_mutants_are_caught plants such mistakes).

Citations name the rustdoc page ("Module numerics" / "Module lane" of
logicaffeine_compile::spatial::decode_engine) and the item on it.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32bits(x) -> int:
    return int(np.array([x], np.float32).view(np.uint32)[0])


def ftz_np(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float32).copy()
    u = a.view(np.uint32)
    sub = (u & 0x7F800000) == 0
    u[sub] &= 0x80000000
    return a


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# --- scaled_to_f32 (Functions scaled_to_f32, ftz) ------------------------------------------

def test_r32_vectors_closed_forms():
    rows = [r for r in read_table("r32_vectors.txt")]
    assert len(rows) >= 14
    for r in rows:
        v, e, want = int(r[0]), int(r[1]), int(r[2], 16)
        assert f32bits(oracle.scaled_to_f32(v, e)) == want, (v, e)
        assert f32bits(exact.round_f32(Fraction(v) * Fraction(2) ** e)) == want, (v, e)


def test_r32_matches_numpy_cast_where_f64_is_exact():
    """Library special case: for |v| < 2^53, v*2^e is exact in float64, and numpy's
    float64 -> float32 cast is IEEE nearest-even with gradual underflow; followed by ftz it
    must equal the oracle's single rounding."""
    g = np.random.Generator(np.random.PCG64(7))
    n = 20000
    nbits = g.integers(1, 54, n)
    v = (g.integers(0, 2 ** 62, n, dtype=np.int64) >> (63 - nbits)).astype(np.int64)
    v[g.random(n) < 0.5] *= -1
    e = g.integers(-200, 110, n)
    with np.errstate(over="ignore"):
        ref = ftz_np(np.ldexp(v.astype(np.float64), e).astype(np.float32))
    got = np.array([oracle.scaled_to_f32(int(a), int(b)) for a, b in zip(v, e)], np.float32)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_exact_sum_no_terms_is_plus_zero_and_single_terms():
    assert f32bits(oracle.exact_sum([], [])) == 0
    assert f32bits(oracle.exact_sum([0, 0], [3, -9])) == 0
    assert oracle.exact_sum([3], [-1]) == np.float32(1.5)
    # exact cancellation of two terms at different exponents is +0
    assert f32bits(oracle.exact_sum([4, -1], [-2, 0])) == 0


# --- activation scales and codes (Functions wide_scale, block_scale, rne_div, quantize) ----

def test_least_scale_closed_forms():
    for r in read_table("least_scale.txt"):
        amax, bits, m, e, code = float(r[0]), int(r[1]), int(r[2]), int(r[3]), int(r[4])
        assert oracle.least_scale(amax, bits) == (m, e), r
        assert exact.least_scale(Fraction(amax), bits) == (m, e), r
        assert oracle.rne_div(amax, m, e) == code, r


def _pred(m, e, bits):
    lo = 1 << (bits - 1)
    return Fraction(m - 1) * Fraction(2) ** e if m > lo else Fraction(2 * lo - 1) * Fraction(2) ** (e - 1)


@pytest.mark.parametrize("bits", [8, 4])
def test_least_scale_is_least(bits):
    """127*s >= amax > 127*pred(s), pred(s) the next smaller admissible value; random amax
    over many binades, including exact boundaries 127*m*2^e."""
    g = np.random.Generator(np.random.PCG64(11 + bits))
    lo = 1 << (bits - 1)
    amaxes = list(np.exp2(g.uniform(-120, 120, 3000)).astype(np.float32))
    amaxes += [np.float32(127 * m * 2.0 ** e) for m in range(lo, 2 * lo) for e in (-30, 0, 11)]
    amaxes += [np.nextafter(a, np.float32(np.inf)) for a in amaxes[-50:]]
    for a in amaxes:
        a = np.float32(a)
        if not (a > 0 and np.isfinite(a)) or a < 2 ** -126:
            continue
        m, e = oracle.least_scale(float(a), bits)
        assert lo <= m < 2 * lo
        s = Fraction(m) * Fraction(2) ** e
        A = Fraction(float(a))
        assert 127 * s >= A > 127 * _pred(m, e, bits), (a, m, e)


@pytest.mark.parametrize("bits", [8, 4])
def test_least_scale_brute_force(bits):
    g = np.random.Generator(np.random.PCG64(21 + bits))
    for a in np.exp2(g.uniform(-60, 60, 150)).astype(np.float32):
        assert oracle.least_scale(float(a), bits) == exact.least_scale(Fraction(float(a)), bits)


@pytest.mark.parametrize("mode", [oracle.PERBLOCK, oracle.SUB32])
def test_codes_match_numpy_rint(mode):
    """Library cross-check: numpy.rint(float64(x) / float64(s)) (half to even) equals every
    code.  fl64(x/s) cannot land on a half-integer unless x/s is one (|x/s| <= 127)."""
    x = gen.act_outliers(8, 4096, 5)
    codes, m, e, s16 = oracle.quantize(x, mode)
    ablk = 256 if mode == oracle.PERBLOCK else 32
    s = (m.astype(np.float64) * np.exp2(e.astype(np.float64))).repeat(ablk, axis=1)
    ref = np.rint(x.astype(np.float64) / s)
    assert np.array_equal(ref, codes.astype(np.float64))
    assert np.abs(codes).max() <= 127
    assert np.array_equal(s16, codes.reshape(8, -1, 16).astype(np.int32).sum(axis=2))


def test_codes_ties_go_to_even_and_scale_is_exact_fraction():
    m, e = 130, -14
    s = m * 2.0 ** e
    # amax element fixes the scale; the others sit exactly on half-integers of s
    halves = [0.5, 1.5, 2.5, -0.5, -3.5, 100.5, -125.5]
    x = np.zeros(256, np.float32)
    x[0] = 1.0
    for i, h in enumerate(halves):
        x[1 + i] = np.float32(h * s)
        assert float(x[1 + i]) == h * s
    codes, mm, ee, _ = oracle.quantize(x[None], oracle.PERBLOCK)
    assert (int(mm[0, 0]), int(ee[0, 0])) == (m, e)
    want = [0, 2, 2, 0, -4, 100, -126]
    assert list(codes[0, 1:1 + len(halves)]) == want


@pytest.mark.parametrize("mode", [oracle.PERBLOCK, oracle.SUB32])
def test_scaling_law(mode):
    """scale(2^k x) = 2^k scale(x) with identical codes (no under/overflow)."""
    x = gen.act_normal(2, 1024, 3)
    c0, m0, e0, _ = oracle.quantize(x, mode)
    for k in (-20, -1, 1, 7, 30):
        xk = (x.astype(np.float64) * 2.0 ** k).astype(np.float32)
        c1, m1, e1, _ = oracle.quantize(xk, mode)
        assert np.array_equal(c0, c1) and np.array_equal(m0, m1) and np.array_equal(e1, e0 + k)


def test_quantize_special_values():
    x = np.zeros((1, 256), np.float32)
    codes, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    assert (int(m[0, 0]), int(e[0, 0])) == (128, 0) and not codes.any()
    x[0, 3] = np.nan
    x[0, 4] = np.float32(2.0 ** -130)            # subnormal: read as 0
    x[0, 5] = np.float32(1.0)
    codes, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    assert (int(m[0, 0]), int(e[0, 0])) == (130, -14)
    assert codes[0, 3] == 0 and codes[0, 4] == 0 and codes[0, 5] == 126
    x[0, 7] = np.inf
    with pytest.raises(oracle.OracleError) as ei:
        oracle.quantize(x, oracle.PERBLOCK)
    assert ei.value.status == 1


def test_sub32_generator_hits_its_exponents():
    x, t = gen.sub32_act(0)
    _, m, e, _ = oracle.quantize(x, oracle.SUB32)
    assert np.array_equal(e.astype(np.int32), t)
    assert e.min() == -12 and e.max() == 4
    assert ((m >= 8) & (m <= 15)).all()


# --- block scales (Structs Scale, Unreadable) ----------------------------------------------

def test_f16_scale_decoding():
    assert oracle.f16_scale(0x3C00) == (1024, -10)          # 1.0
    assert oracle.f16_scale(0x0001) == (1, -24)             # least subnormal 2^-24
    assert oracle.f16_scale(0x0000) == (0, -24)
    assert oracle.f16_scale(0xBC00) == (-1024, -10)
    assert oracle.f16_scale(0x7BFF) == (2047, 5)            # 65504
    for h in [0x0001, 0x03FF, 0x0400, 0x3555, 0x7BFF, 0x8123]:
        sig, ex = oracle.f16_scale(h)
        assert Fraction(sig) * Fraction(2) ** ex == Fraction(float(np.array([h], np.uint16).view(np.float16)[0]))
    for h in (0x7C00, 0xFC00, 0x7E00):
        with pytest.raises(oracle.OracleError):
            oracle.f16_scale(h)


def test_unreadable_block_is_refused():
    f = gen.q4k_fields(2, 256, 1)
    f["d"][1, 0] = 0x7C00
    c, m, e, _ = oracle.quantize(gen.act_normal(1, 256, 2), oracle.PERBLOCK)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    assert ei.value.status == 3


# --- block value closed forms (module description: PerBlock and Sub32; Module lane) --------

def _const_q4k(rows, cols, q, sc, mn, d, dmin):
    G = cols // 256
    return {"fmt": "q4k", "rows": rows, "cols": cols,
            "q": np.full((rows, cols), q, np.uint8), "sc": np.full((rows, cols // 32), sc, np.uint8),
            "mn": np.full((rows, cols // 32), mn, np.uint8), "d": np.full((rows, G), d, np.uint16),
            "dmin": np.full((rows, G), dmin, np.uint16)}


def test_q4k_block_closed_form():
    """d = 2^-10, dmin = 2^-12, sc = mn = 1, q = 1, x = 127/128 everywhere: codes all 127,
    s = 2^-7, block value 256 * (2^-10 - 2^-12) * 127 * 2^-7 = 381/2048; four blocks add
    exactly to 381/512.  With q = 0 only the offset term is left: -127/2048 per block."""
    x = np.full((1, 1024), 0.9921875, np.float32)
    c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    assert (c == 127).all() and (m == 128).all() and (e == -14).all()
    f = _const_q4k(3, 1024, 1, 1, 1, 0x1400, 0x0C00)
    out = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    assert (out == np.float32(381 / 512)).all() and out[0] == np.float32(0.744140625)
    f0 = _const_q4k(1, 1024, 0, 1, 1, 0x1400, 0x0C00)
    assert oracle.gemv(f0, c, m, e, oracle.PERBLOCK)[0] == np.float32(-4 * 127 / 2048)
    # Sub32 reading of the same row: every 32-block has scale (8, -10) = 2^-7 too
    c2, m2, e2, _ = oracle.quantize(x, oracle.SUB32)
    assert (m2 == 8).all() and (e2 == -10).all()
    assert (oracle.gemv(f, c2, m2, e2, oracle.SUB32) == np.float32(381 / 512)).all()


def test_q6k_block_closed_form():
    """d = 2^-10, sc = 1, q = 33 (weight 2^-10), codes 127 at s = 2^-7: 127 * 2^-9 a block."""
    x = np.full((1, 512), 0.9921875, np.float32)
    c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    f = {"fmt": "q6k", "rows": 1, "cols": 512, "q": np.full((1, 512), 33, np.uint8),
         "sc": np.ones((1, 32), np.int8), "d": np.full((1, 2), 0x1400, np.uint16)}
    assert oracle.gemv(f, c, m, e, oracle.PERBLOCK)[0] == np.float32(2 * 127 / 512)
    f["q"][:] = 0                                  # weight -32 * 2^-10
    f["sc"][:] = -128                              # coefficient -128 * -32 = COEF_BOUND
    assert oracle.gemv(f, c, m, e, oracle.PERBLOCK)[0] == np.float32(2 * 256 * 4096 * 127 * 2.0 ** -17)


def test_sub32_group_closed_form():
    """Per-32 blocks at different exponents: block j of the group is 127/128 * 2^k_j, so its
    scale is 8 * 2^(-10 + k_j) and codes 127; with d = 2^-10, dmin = 0, sc = q = 1 the
    group value is sum_j 32 * 2^-10 * 127 * 2^(-7 + k_j), rounded once (it spans 30 bits, so
    the rounding is visible)."""
    ks = [0, -3, 5, 1, -12, 4, 2, 0]
    x = np.concatenate([np.full(32, 0.9921875 * 2.0 ** k, np.float32) for k in ks])[None]
    c, m, e, _ = oracle.quantize(x, oracle.SUB32)
    assert list(e[0]) == [-10 + k for k in ks] and (c == 127).all()
    f = _const_q4k(1, 256, 1, 1, 0, 0x1400, 0x0000)
    want = sum(Fraction(32 * 127) * Fraction(2) ** (-17 + k) for k in ks)
    got = oracle.gemv(f, c, m, e, oracle.SUB32)[0]
    assert f32bits(got) == f32bits(exact.round_f32(want))
    assert Fraction(float(got)) != want


def test_sub32_group_values_beside_binary32_boundaries():
    """Hand-laid Sub32 groups (workloads.gen.sub32_boundary_rows): with F = 8 * 2^16 on block 0
    and 8 on block 1, the integer sums are IC = 2^32 + 768 (768 without block 0) and IO = 8, so
    a group is 2^emin * (d * IC - dmin * IO) with emin = -16 (or -128 for the second row).  Its
    one rounding, by exact rationals, is the oracle's output; for dmin = +-2^-24 the value lies
    2^-37 beside the midpoint 2^16 + 3 * 2^-8, where rounding to binary64 first (which lands on
    the midpoint) and then to binary32 gives the other neighbour."""
    f, x = gen.sub32_boundary_rows()
    c, m, e, _ = oracle.quantize(x, oracle.SUB32)
    assert list(e[0]) == [0, -16] + [-8] * 6 and list(e[1]) == [-112, -128] + [-120] * 6
    assert (m == 8).all()
    two = Fraction(2)
    d = [1, 1, 1, -1, 1, two ** -24, -two ** -24]
    dmin = [two ** -24, -two ** -24, 0, two ** -24, two ** -24, 0, 0]
    IC = [2 ** 32 + 768] * 4 + [768] * 3
    for k, emin in ((0, -16), (1, -128)):
        got = oracle.gemv(f, c[k:k + 1], m[k:k + 1], e[k:k + 1], oracle.SUB32)
        for r in range(7):
            want = two ** emin * (d[r] * IC[r] - dmin[r] * 8)
            if k == 1 and r >= 5:
                assert float(got[r]) == 0.0                  # below 2^-126: flushed
                continue
            assert f32bits(got[r]) == f32bits(exact.round_f32(want)), (k, r)
    got0 = oracle.gemv(f, c[:1], m[:1], e[:1], oracle.SUB32)
    assert float(got0[0]) == 2.0 ** 16 + 2.0 ** -7 and float(got0[1]) == 2.0 ** 16 + 2.0 ** -6
    assert float(got0[2]) == 2.0 ** 16 + 2.0 ** -6                 # the exact tie, to even
    assert float(np.float32(float(two ** -16 * (IC[0] - dmin[0] * 8)))) != float(got0[0])


# --- integer sums (Module lane: the excess-form identity) ----------------------------------

def test_excess_form_identity_on_random_units():
    """sum((q - z) a) = P' - 128 Q - z S' + 2048 z and sum(a) = S' - 2048 over 16-element units
    with a' = a + 128; and the two-word form for 16-bit a = 256 hi + lo."""
    g = np.random.Generator(np.random.PCG64(31))
    for qmax, z in ((16, 0), (64, 32)):
        q = g.integers(0, qmax, (5000, 16)).astype(np.int64)
        a = g.integers(-128, 128, (5000, 16)).astype(np.int64)
        ap = a + 128
        P, Q, S = (q * ap).sum(1), q.sum(1), ap.sum(1)
        assert np.array_equal(P - 128 * Q - z * S + 128 * 16 * z, ((q - z) * a).sum(1))
        assert np.array_equal(S - 128 * 16, a.sum(1))
        a16 = g.integers(-32768, 32768, (5000, 16)).astype(np.int64)
        hi, lo = a16 >> 8, a16 & 255
        hip = hi + 128
        Ph, Sh = (q * hip).sum(1), hip.sum(1)
        Pl, Sl = (q * lo).sum(1), lo.sum(1)
        two_word = 256 * (Ph - 128 * Q - z * Sh + 128 * 16 * z) + (Pl - z * Sl)
        assert np.array_equal(two_word, ((q - z) * a16).sum(1))


def test_oracle_sums_equal_the_lane_route():
    """The oracle's element-by-element sums equal the lane page's route: per 16-unit P', Q,
    S' in excess form, corrected by the identity, weighted by the unit's scale."""
    f = gen.q4k_fields(64, 1024, 41)
    c, _, _, _ = oracle.quantize(gen.act_outliers(1, 1024, 42), oracle.PERBLOCK)
    Cs, Os = oracle.sub_sums(f, c[0])
    q = f["q"].astype(np.int64).reshape(64, -1, 16)
    ap = c[0].astype(np.int64).reshape(-1, 16)[None] + 128
    P, Q, S = (q * ap).sum(2), q.sum(2), ap.sum(2)
    unit_coef = P - 128 * Q                          # z = 0
    unit_a = S - 2048
    sc = f["sc"].astype(np.int64).repeat(2, axis=1)
    mn = f["mn"].astype(np.int64).repeat(2, axis=1)
    assert np.array_equal((sc * unit_coef).reshape(64, -1, 2).sum(2), Cs)
    assert np.array_equal((mn * unit_a).reshape(64, -1, 2).sum(2), Os)
    f6 = gen.q6k_fields(32, 512, 43)
    c6, _, _, _ = oracle.quantize(gen.act_normal(1, 512, 44), oracle.PERBLOCK)
    C6 = oracle.sub_sums(f6, c6[0])
    q6 = f6["q"].astype(np.int64).reshape(32, -1, 16)
    ap6 = c6[0].astype(np.int64).reshape(-1, 16)[None] + 128
    via = (q6 * ap6).sum(2) - 128 * q6.sum(2) - 32 * ap6.sum(2) + 2048 * 32
    assert np.array_equal(f6["sc"].astype(np.int64) * via, C6)
    assert np.abs(C6).max() <= 16 * 4096 * 127


# --- brute force on tiny rows (exact rationals) --------------------------------------------

def _adversarial_q4k(seed, rows, cols):
    f = gen.q4k_fields(rows, cols, seed)
    g = np.random.Generator(np.random.PCG64(seed + 1))
    G = cols // 256
    # subnormal, zero and large binary16 scales, far-apart d/dmin exponents
    choices = np.array([0x0000, 0x0001, 0x0003, 0x03FF, 0x0400, 0x1400, 0x3C00, 0x7BFF, 0x8001, 0x2E66], np.uint16)
    for key in ("d", "dmin"):
        pick = g.random((rows, G)) < 0.4
        f[key][pick] = g.choice(choices, size=int(pick.sum()))
    # all-zero sub-scales in some blocks, extreme codes in others
    f["sc"][g.random(f["sc"].shape) < 0.1] = 0
    f["q"][g.random(f["q"].shape) < 0.05] = 15
    return f


def _adversarial_x(seed, cols, mode, spread=None):
    """Activation row with all-zero, tiny (partly subnormal), huge, NaN and tie-laden blocks.
    Under Sub32 the per-32 blocks of one group stay within 2^+-20 of each other by default,
    so the SUM_WINDOW floor is not engaged (the Fraction reference sums exactly)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(cols).astype(np.float32)
    blk = 256 if mode == oracle.PERBLOCK else 32
    lo_k, hi_k = spread if spread else ((-120, 100) if mode == oracle.PERBLOCK else (-20, 20))
    nb = cols // blk
    for b in range(nb):
        kind = g.integers(0, 7)
        sl = slice(b * blk, (b + 1) * blk)
        if kind == 0:
            x[sl] = 0.0                                         # all-zero block
        elif kind == 1:
            x[sl] *= np.float32(2.0 ** lo_k)                    # tiny
        elif kind == 2:
            x[sl] *= np.float32(2.0 ** hi_k)                    # huge
        elif kind == 3:
            x[b * blk + 1] = np.nan
        elif kind == 4:
            x[sl] = np.round(x[sl] * 4) / 4                     # many exact ties
    return x


@pytest.mark.parametrize("mode", [oracle.PERBLOCK, oracle.SUB32])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_q4k_rows_brute_force(mode, seed):
    for cols in (256, 768):
        f = _adversarial_q4k(1000 * seed + cols, 6, cols)
        x = _adversarial_x(77 * seed + cols, cols, mode)
        c, m, e, _ = oracle.quantize(x[None], mode)
        got = oracle.gemv(f, c, m, e, mode)
        want = exact.gemv(f, x, mode)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)
        ec, es = exact.quantize(x, mode)
        assert list(c[0]) == ec and list(zip(m[0].tolist(), e[0].tolist())) == es


@pytest.mark.parametrize("mode", [oracle.PERBLOCK, oracle.SUB32])
def test_q6k_rows_brute_force(mode):
    for seed, cols in ((5, 256), (6, 512)):
        f = gen.q6k_fields(6, cols, seed)
        g = np.random.Generator(np.random.PCG64(seed))
        pick = g.random(f["d"].shape) < 0.5
        f["d"][pick] = g.choice(np.array([0, 1, 0x03FF, 0x7BFF, 0x8400], np.uint16), size=int(pick.sum()))
        x = _adversarial_x(seed + 9, cols, mode)
        c, m, e, _ = oracle.quantize(x[None], mode)
        got = oracle.gemv(f, c, m, e, mode)
        want = exact.gemv(f, x, mode)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_near_underflow_and_overflow_pieces():
    """Pieces straddling 2^-126 (flushed or kept) and past the top of binary32 (inf), and
    an inf + -inf row (NaN, canonical)."""
    f = _const_q4k(4, 512, 1, 1, 0, 0x0001, 0x0000)      # d = 2^-24
    f["q"][1] = 0
    f["sc"][2] = 63
    x = np.full((1, 512), np.float32(2.0 ** -100), np.float32)
    c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    got = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    want = exact.gemv(f, x[0], oracle.PERBLOCK)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    big = _const_q4k(2, 512, 15, 63, 0, 0x7BFF, 0x0000)
    big["d"][1, 1] = 0xFBFF                                  # -65504 in block 1 of row 1
    xb = np.full((1, 512), np.float32(3.0e38), np.float32)
    c, m, e, _ = oracle.quantize(xb, oracle.PERBLOCK)
    out = oracle.gemv(big, c, m, e, oracle.PERBLOCK)
    assert np.isposinf(out[0])
    assert f32bits(out[1]) == 0x7FC00000


# --- the row fold (module description: pieces added in order; Functions fadd) --------------

def _pieces(f, c, m, e, mode):
    """Per-block pieces through single-block matrices (a one-block row is 0 + piece)."""
    G = f["cols"] // 256
    nsc = 1 if mode == oracle.PERBLOCK else 8
    out = []
    for b in range(G):
        fb = dict(f)
        fb["cols"] = 256
        for k, per in (("q", 256), ("sc", 8), ("mn", 8), ("d", 1), ("dmin", 1)):
            fb[k] = np.ascontiguousarray(f[k][:, b * per:(b + 1) * per])
        out.append(oracle.gemv(fb, c[:, b * 256:(b + 1) * 256], m[:, b * nsc:(b + 1) * nsc],
                               e[:, b * nsc:(b + 1) * nsc], mode))
    return np.stack(out, axis=1)


def test_fold_is_sequential_float32_and_order_matters():
    f, x = gen.tiny_q4k()
    c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    out = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    p = _pieces(f, c, m, e, oracle.PERBLOCK)
    y = np.zeros(f["rows"], np.float32)
    for b in range(p.shape[1]):
        y = ftz_np(y + p[:, b])
    assert np.array_equal(y.view(np.uint32), out.view(np.uint32))
    tree = ftz_np(ftz_np(p[:, 0] + p[:, 1]) + ftz_np(p[:, 2] + p[:, 3]))
    assert not np.array_equal(tree.view(np.uint32), out.view(np.uint32))   # the check has teeth
    # and the reassociated order stays within the bound a stated 1e-5 tolerance allows
    assert np.max(np.abs(tree - out) / np.maximum(np.abs(out), 1e-30)) < 1e-5


def test_fold_keeps_negative_zero_through_a_flushed_piece():
    """One row of three blocks under an activation block of all 2^-112 (codes 126, scale
    130 * 2^-126) whose pieces are 800u, -801u and -1u, u = 16380 * 2^-142: the first two cancel
    to a negative subnormal partial sum, which the flushed add turns into -0; the third piece is
    itself a negative subnormal, so it is -0, and -0 + -0 stays -0.  Had that piece been +0 (or
    been added as +0 + piece), the row would end at +0."""
    f = gen.q4k_fields(1, 768, 77)
    f["q"][0, :768] = 1
    f["q"][0, 256:768] = 0
    f["sc"][0, :24] = 0
    f["sc"][0, :8] = 1
    f["mn"][0, :24] = 1
    f["mn"][0, :8] = 0
    f["d"][0, :3] = [800, 0, 0]                     # binary16 subnormals k * 2^-24
    f["dmin"][0, :3] = [0, 801, 1]
    x = np.full((1, 768), np.float32(2.0 ** -112))
    c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    assert int(c[0, 0]) == 126 and int(m[0, 0]) == 130 and int(e[0, 0]) == -126
    unit = 16380.0 * 2.0 ** -142
    # the pieces from the exact sum of each block's two products (C * d * s and -O * dmin * s)
    p0 = oracle.exact_sum([32256 * 800 * 130], [-150])
    p1 = oracle.exact_sum([-32256 * 801 * 130], [-150])
    p2 = oracle.exact_sum([-32256 * 1 * 130], [-150])
    assert p0 == np.float32(800 * unit) and p1 == np.float32(-801 * unit)
    assert f32bits(p2) == 0x80000000
    y = ftz_np(np.float32(0.0) + np.float32(p0))
    y = ftz_np(y + np.float32(p1))
    assert f32bits(y) == 0x80000000
    assert f32bits(ftz_np(y + np.float32(p2))) == 0x80000000
    assert f32bits(ftz_np(y + np.float32(0.0))) == 0
    out = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    assert f32bits(out[0]) == 0x80000000


def test_exponent_invariance():
    f, x = gen.tiny_q4k()
    for mode in (oracle.PERBLOCK, oracle.SUB32):
        base = oracle.gemv(f, *oracle.quantize(x, mode)[:3], mode)
        for k in (-6, -1, 2, 9):
            xk = (x.astype(np.float64) * 2.0 ** k).astype(np.float32)
            got = oracle.gemv(f, *oracle.quantize(xk, mode)[:3], mode)
            assert np.array_equal(got, (base.astype(np.float64) * 2.0 ** k).astype(np.float32))


def test_close_to_the_float64_dequantized_dot():
    """Sanity bound: |out - sum w_i c_i s| <= sum_b |X_b - piece_b| + G * 2^-24 * sum_b |piece_b|,
    with X_b, piece_b bounded via |piece_b| ~ |X_b| (2^-24 relative each)."""
    f, x = gen.tiny_q4k()
    c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK)
    out = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    d = f["d"].view(np.float16).astype(np.float64)
    dm = f["dmin"].view(np.float16).astype(np.float64)
    w = (d.repeat(256, 1) * f["sc"].astype(np.float64).repeat(32, 1) * f["q"]
         - dm.repeat(256, 1) * f["mn"].astype(np.float64).repeat(32, 1))
    xs = c[0] * (m[0].astype(np.float64) * np.exp2(e[0])).repeat(256)
    X = (w * xs).reshape(f["rows"], -1, 256).sum(2)
    ref = X.sum(1)
    bound = 8 * 2.0 ** -24 * np.abs(X).sum(1) + 1e-30
    assert (np.abs(out - ref) <= bound).all()


def test_gemm_columns_are_gemvs():
    f = gen.q4k_fields(64, 1024, 51)
    xs = gen.act_normal(5, 1024, 52)
    c, m, e, _ = oracle.quantize(xs, oracle.PERBLOCK)
    out = oracle.gemm(f, c, m, e, oracle.PERBLOCK).reshape(5, 64)
    for k in range(5):
        assert np.array_equal(out[k], oracle.gemv(f, c[k:k + 1], m[k:k + 1], e[k:k + 1], oracle.PERBLOCK))


def test_thread_count_does_not_change_bits():
    f = gen.q4k_fields(512, 1024, 61)
    c, m, e, _ = oracle.quantize(gen.act_normal(1, 1024, 62), oracle.PERBLOCK)
    oracle.set_threads(1)
    a = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    oracle.set_threads(4)
    b = oracle.gemv(f, c, m, e, oracle.PERBLOCK)
    oracle.set_threads(1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --- SUM_WINDOW (value not printed; reading: 64) -------------------------------------------

def _windowed_sum_fraction(vs, es, W=64):
    """The reading of exact_sum written over Fractions: terms whose exponent is more than W
    below the largest-magnitude term's exponent are floored to a multiple of 2^(L - W)."""
    if not vs:
        return exact.round_f32(Fraction(0))
    mags = [abs(Fraction(v) * Fraction(2) ** e) for v, e in zip(vs, es)]
    L = es[max(range(len(vs)), key=lambda i: (mags[i], -i))]
    q = Fraction(2) ** (L - W)
    tot = Fraction(0)
    for v, e in zip(vs, es):
        t = Fraction(v) * Fraction(2) ** e
        if e < L - W:
            t = (t / q).__floor__() * q
        tot += t
    return exact.round_f32(tot)


def test_exact_sum_window_reading():
    """Parity unpinned by the pages (SUM_WINDOW's value is not printed): the oracle agrees
    with the Fraction form of the reading, and inside the window the sum is exact."""
    g = np.random.Generator(np.random.PCG64(71))
    for _ in range(400):
        n = int(g.integers(1, 17))
        vs = [int(v) for v in g.integers(-2 ** 40, 2 ** 40, n)]
        es = [int(e) for e in g.integers(-150, 40, n)]
        got = oracle.exact_sum(vs, es)
        assert f32bits(got) == f32bits(_windowed_sum_fraction(vs, es)), (vs, es)
    # inside the window the sum is the exact one
    vs, es = [1 << 30, 3, -5], [0, -60, -64]
    exact_val = Fraction(1 << 30) + Fraction(3, 2 ** 60) - Fraction(5, 2 ** 64)
    assert f32bits(oracle.exact_sum(vs, es)) == f32bits(exact.round_f32(exact_val))


def test_sub32_rows_with_the_window_engaged():
    """Sub32 groups whose 32-blocks lie 2^+-120 apart: the oracle's rows equal the Fraction
    form of the SUM_WINDOW reading applied to the sixteen terms of each group.  Parity
    unpinned by the pages (the window's value is not printed)."""
    engaged = 0
    for seed in (3, 4):
        f = _adversarial_q4k(500 + seed, 6, 768)
        x = _adversarial_x(600 + seed, 768, oracle.SUB32, spread=(-120, 100))
        c, m, e, _ = oracle.quantize(x[None], oracle.SUB32)
        got = oracle.gemv(f, c, m, e, oracle.SUB32)
        Cs, Os = oracle.sub_sums(f, c[0])
        for r in range(f["rows"]):
            y = np.float32(0)
            for b in range(3):
                sd, ed = oracle.f16_scale(int(f["d"][r, b]))
                sm, em = oracle.f16_scale(int(f["dmin"][r, b]))
                vs, es = [], []
                for j in range(8 * b, 8 * b + 8):
                    vs += [int(m[0, j]) * sd * int(Cs[r, j]), -int(m[0, j]) * sm * int(Os[r, j])]
                    es += [int(e[0, j]) + ed, int(e[0, j]) + em]
                piece = _windowed_sum_fraction(vs, es)
                engaged += exact.round_f32(sum(Fraction(v) * Fraction(2) ** k for v, k in zip(vs, es))) != piece
                y = exact.fadd(y, piece)
            assert f32bits(got[r]) == f32bits(y)
    assert engaged > 0


# --- 32-element weight blocks (Q8_0- and Q4_0-style) ----------------------------------------

def _adversarial_b32(fmt, seed, rows, cols):
    f = gen.q8_0_fields(rows, cols, seed) if fmt == "q8_0" else gen.q4_0_fields(rows, cols, seed)
    g = np.random.Generator(np.random.PCG64(seed + 1))
    choices = np.array([0x0000, 0x0001, 0x0003, 0x03FF, 0x0400, 0x1400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF], np.uint16)
    pick = g.random(f["d"].shape) < 0.4
    f["d"][pick] = g.choice(choices, size=int(pick.sum()))
    hi = 127 if fmt == "q8_0" else 15
    lo = -128 if fmt == "q8_0" else 0
    f["q"][g.random(f["q"].shape) < 0.05] = hi
    f["q"][g.random(f["q"].shape) < 0.05] = lo
    return f


def _b32_x(seed, cols, mode):
    """Adversarial activations with PerBlock blocks of 32 elements (the format's own block)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(cols).astype(np.float32)
    lo_k, hi_k = (-120, 100) if mode == oracle.PERBLOCK else (-20, 20)
    for b in range(cols // 32):
        kind = g.integers(0, 7)
        sl = slice(b * 32, (b + 1) * 32)
        if kind == 0:
            x[sl] = 0.0
        elif kind == 1:
            x[sl] *= np.float32(2.0 ** lo_k)
        elif kind == 2:
            x[sl] *= np.float32(2.0 ** hi_k)
        elif kind == 3:
            x[b * 32 + 1] = np.nan
        elif kind == 4:
            x[sl] = np.round(x[sl] * 4) / 4
    return x


def _b32_quant(fmt, x, mode, mutant=0):
    return oracle.quantize(np.asarray(x, np.float32).reshape(1, -1), mode, block=oracle.act_block(fmt, mode),
                           mutant=mutant)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("mode", [0, 1])
def test_b32_closed_form(fmt, mode):
    """All weights d*1 with d = 2^-10 and x = 127*128*2^-14 everywhere: codes 127 under
    s = 2^-7 (PerBlock over 32: m = 128, e = -14; Sub32: m = 8, e = -10), so every 32-block
    is 2^-7 * 2^-10 * 32 * 127 and a 256-element row 8 of them: 127/512 exactly."""
    f = gen.q8_0_fields(2, 512, 5) if fmt == "q8_0" else gen.q4_0_fields(2, 512, 5)
    f["q"][:] = 1 if fmt == "q8_0" else 9
    f["d"][:] = 0x1400
    x = np.full(512, np.float32(0.9921875), np.float32)
    c, m, e, _ = _b32_quant(fmt, x, mode)
    assert (c == 127).all()
    assert (m == (128 if mode == 0 else 8)).all() and (e == (-14 if mode == 0 else -10)).all()
    out = oracle.gemv(f, c, m, e, mode)
    assert (out == np.float32(254 / 512)).all()
    if fmt == "q4_0":                                        # codes 8 are the value 0
        f["q"][:] = 8
        assert (oracle.gemv(f, c, m, e, mode) == 0).all()


@pytest.mark.parametrize("mode", [0, 1])
def test_q4_0_equals_q8_0_shifted(mode):
    """A Q4_0-style code q is the value q - 8: the same matrix stored as Q8_0 codes q - 8 gives
    the same bits (two code paths of the oracle)."""
    f4 = _adversarial_b32("q4_0", 41, 37, 1024)
    f8 = {"fmt": "q8_0", "rows": 37, "cols": 1024, "q": (f4["q"].astype(np.int16) - 8).astype(np.int8),
          "d": f4["d"].copy()}
    x = _b32_x(42, 1024, mode)
    c, m, e, _ = _b32_quant("q4_0", x, mode)
    assert np.array_equal(oracle.gemv(f4, c, m, e, mode).view(np.uint32), oracle.gemv(f8, c, m, e, mode).view(np.uint32))


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("mode", [0, 1])
def test_b32_fraction_brute_force(fmt, mode):
    """Tiny adversarial rows against the exact-rational reference (subnormal, zero, huge and
    negative binary16 scales; tiny, huge, NaN, all-zero and tie-laden activation blocks)."""
    for seed in (1, 2, 3):
        f = _adversarial_b32(fmt, 500 + seed, 4, 512)
        x = _b32_x(600 + seed, 512, mode)
        c, m, e, _ = _b32_quant(fmt, x, mode)
        got = oracle.gemv(f, c, m, e, mode)
        want = exact.gemv(f, x, mode)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (fmt, mode, seed)


# --- argmax ([numerics] Functions argmax) ---------------------------------------------------

def _argmax_cases():
    for r in read_table("argmax.txt"):
        vals = [] if r[1] == "-" else [int(h, 16) for h in r[1:]]
        yield int(r[0]), np.array(vals, np.uint32).view(np.float32)


def test_argmax_hand_cases():
    for want, x in _argmax_cases():
        assert oracle.argmax(x) == want, (want, x)


def test_argmax_matches_numpy_first_occurrence():
    """numpy's argmax returns the first of equal maxima and compares -0 == +0; with NaNs it is
    taken over the non-NaN entries (nanargmax would confuse a NaN with a real -inf).  Rows are
    drawn from few values so ties and signed zeros are common."""
    g = np.random.Generator(np.random.PCG64(31))
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, -2.5, np.inf, -np.inf], np.float32)
    for _ in range(2000):
        n = int(g.integers(1, 40))
        x = g.choice(pool, n)
        assert oracle.argmax(x) == int(np.argmax(x))
        y = x.copy()
        y[g.random(n) < 0.3] = np.nan
        keep = np.flatnonzero(~np.isnan(y))
        want = 0 if keep.size == 0 else int(keep[np.argmax(y[keep])])
        assert oracle.argmax(y) == want


# --- planted mistakes --------------------------------------------------------------------

def _quick_pins(mutant: int) -> bool:
    """True when every quick pin passes for the oracle variant `mutant`."""
    try:
        for r in read_table("r32_vectors.txt"):
            if f32bits(oracle.scaled_to_f32(int(r[0]), int(r[1]), mutant)) != int(r[2], 16):
                return False
        for r in read_table("least_scale.txt"):
            amax, bits, m, e, code = float(r[0]), int(r[1]), int(r[2]), int(r[3]), int(r[4])
            if oracle.least_scale(amax, bits, mutant) != (m, e) or oracle.rne_div(amax, m, e, mutant) != code:
                return False
        for mode in (oracle.PERBLOCK, oracle.SUB32):
            for seed in (1, 2):
                f = _adversarial_q4k(1000 * seed + 768, 6, 768)
                x = _adversarial_x(77 * seed + 768, 768, mode)
                c, m, e, _ = oracle.quantize(x[None], mode, mutant=mutant)
                got = oracle.gemv(f, c, m, e, mode, mutant=mutant)
                if not np.array_equal(got.view(np.uint32), exact.gemv(f, x, mode).view(np.uint32)):
                    return False
        f, x = gen.tiny_q4k()
        c, m, e, _ = oracle.quantize(x, oracle.PERBLOCK, mutant=mutant)
        out = oracle.gemv(f, c, m, e, oracle.PERBLOCK, mutant=mutant)
        p = _pieces(f, c, m, e, oracle.PERBLOCK)
        y = np.zeros(f["rows"], np.float32)
        for b in range(p.shape[1]):
            y = ftz_np(y + p[:, b])
        if not np.array_equal(y.view(np.uint32), out.view(np.uint32)):
            return False
        xt = np.zeros((1, 256), np.float32)
        xt[0, 0] = 1.0
        for i, h in enumerate([0.5, 1.5, 2.5, -0.5, -3.5]):
            xt[0, 1 + i] = np.float32(h * 130 * 2.0 ** -14)
        c, m, e, _ = oracle.quantize(xt, oracle.PERBLOCK, mutant=mutant)
        if list(c[0, 1:6]) != [0, 2, 2, 0, -4]:
            return False
        xs = np.zeros((1, 256), np.float32)
        xs[0, 4] = np.float32(2.0 ** -130)
        xs[0, 5] = np.float32(2.0 ** -127)
        c, m, e, _ = oracle.quantize(xs, oracle.PERBLOCK, mutant=mutant)
        if (int(m[0, 0]), int(e[0, 0])) != (128, 0):
            return False
        for want, x in _argmax_cases():
            if oracle.argmax(x, mutant) != want:
                return False
        for fmt in ("q8_0", "q4_0"):
            f = _adversarial_b32(fmt, 800, 3, 256)
            x = _b32_x(801, 256, oracle.PERBLOCK)
            c, m, e, _ = _b32_quant(fmt, x, oracle.PERBLOCK, mutant)
            got = oracle.gemv(f, c, m, e, oracle.PERBLOCK, mutant=mutant)
            if not np.array_equal(got.view(np.uint32), exact.gemv(f, x, oracle.PERBLOCK).view(np.uint32)):
                return False
    except oracle.OracleError:
        return False
    return True


@pytest.mark.slow
def test_mutants_are_caught():
    assert _quick_pins(0)
    for mutant in range(1, 14):
        assert not _quick_pins(mutant), f"oracle mutant {mutant} passes every quick pin"
