"""Pins of the oracle's int8 KV cache ([numerics] Functions cache_row, int8_codes, quantize_head,
int8_score, weighted_int8; Constants INV_127, VALUE_BLOCK), against numpy's binary16
conversion, hand-derived closed forms, the already pinned activation quantizer, and Fraction
brute force written from the definitions.  Four planted mistakes must each fail a quick pin."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact

F16_FINITE = np.arange(0, 0x7C00, dtype=np.uint16)
F16_VALUES = F16_FINITE.view(np.float16).astype(np.float64)


def f16_nearest(v: float) -> int:
    """Brute force over every finite binary16: the nearest to v (|v| below the overflow
    threshold), ties to the even significand."""
    a = abs(v)
    d = np.abs(F16_VALUES - a)
    best = np.flatnonzero(d == d.min())
    h = int(best[0]) if len(best) == 1 else int(best[np.argmin(best & 1)])
    return h | (0x8000 if v < 0 or (v == 0 and np.signbit(v)) else 0)


def test_f16_rne_matches_numpy_and_brute_force():
    g = np.random.default_rng(3)
    xs = np.concatenate([
        (g.standard_normal(4000) * 2.0 ** g.integers(-30, 17, 4000)).astype(np.float32),
        np.array([65504, 65519.99, 65520, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
                  (2.0 ** -14) * (1 - 2.0 ** -11), 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -0.0, 0.0], np.float32)])
    for x in xs:
        with np.errstate(over="ignore"):
            want = int(np.array([x], np.float32).astype(np.float16).view(np.uint16)[0])
        assert oracle.f16_rne(x) == want, x
    for x in xs[:300]:
        if abs(float(x)) < 65520:
            assert oracle.f16_rne(x) == f16_nearest(float(x)), x


def test_cache_row_closed_forms():
    # amax 127: 127 * f32(1/127) rounds to 1.0 in binary32, so the scale is 1 and every code is the
    # nearest integer of x itself (ties to even)
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [127, 63.5, -0.5, 1.5, 2.5, -2.5, 0.49, -126.5]
    s, c = oracle.kv_cache_rows(x)
    assert int(s[0]) == 0x3C00
    assert list(c[0, :8]) == [127, 64, 0, 2, 2, -2, 0, -126]
    # amax 1: f32(1/127) = 0.00787401571... lies 1032.06 steps of 2^-17 above 0: binary16 1032 * 2^-17
    # (0x2008); its reciprocal is 127.0077..., so 1, 0.5, -1, 0.25 code as 127, 64, -127, 32
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [1, 0.5, -1, 0.25]
    s, c = oracle.kv_cache_rows(x)
    assert int(s[0]) == 0x2008
    assert list(c[0, :4]) == [127, 64, -127, 32]
    # zero row, denormals only (read as zero), NaN passed over, and a scale past binary16's top
    x = np.zeros((4, 32), np.float32)
    x[1, 3] = np.float32(1e-40)
    x[2, :3] = [np.nan, 127.0, -63.5]
    x[3, 0] = 1e7
    s, c = oracle.kv_cache_rows(x)
    assert int(s[0]) == 0 and not c[0].any()
    assert int(s[1]) == 0 and not c[1].any()
    assert int(s[2]) == 0x3C00 and list(c[2, :3]) == [0, 127, -64]
    assert int(s[3]) == 0x7C00 and not c[3].any()


def test_cache_row_brute_force():
    g = np.random.default_rng(11)
    inv127 = np.float32(1) / np.float32(127)
    for r in range(40):
        hd = 64
        x = (g.standard_normal(hd) * 2.0 ** int(g.integers(-12, 12))).astype(np.float32)
        if r % 5 == 0:
            x[g.integers(0, hd, 3)] = np.round(x[:3] * 4) / 4
        s, c = oracle.kv_cache_rows(x[None])
        amax = np.float32(np.max(np.abs(x)))
        h = f16_nearest(float(np.float32(amax * inv127)))
        assert int(s[0]) == h
        inv = np.float32(1) / np.float32(np.array([h], np.uint16).view(np.float16)[0])
        for i in range(hd):
            p = Fraction(float(np.float32(x[i] * inv)))
            want = max(-127, min(127, round(p)))
            assert int(c[0, i]) == want, (r, i)


def test_quantize_heads_reduce_to_the_activation_quantizer():
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 256)).astype(np.float32)
    x[1, 10] = np.nan
    for mode in (oracle.PERBLOCK, oracle.SUB32):
        c, m, e = oracle.kv_quantize_heads(x, mode)
        oc, om, oe, _ = oracle.quantize(x, mode)
        assert np.array_equal(c, oc) and np.array_equal(m, om) and np.array_equal(e, oe)
    # a 128-element head under PerBlock is one block: the brute-force scale and codes
    for seed in range(6):
        q = (np.random.default_rng(seed).standard_normal(128) * 2.0 ** (seed - 3)).astype(np.float32)
        c, m, e = oracle.kv_quantize_heads(q, oracle.PERBLOCK)
        bm, be, bc = exact.quantize_block(q, 8)
        assert (int(m[0, 0]), int(e[0, 0])) == (bm, be) and list(c[0]) == list(bc)


def _score_fraction(qc, qm, qe, ks, kc, mode):
    hd = qc.size
    B = hd if mode == oracle.PERBLOCK else 32
    d = exact.f16_value(int(ks))
    tot = Fraction(0)
    for b in range(hd // B):
        P = int(np.dot(qc[b * B:(b + 1) * B].astype(np.int64), kc[b * B:(b + 1) * B].astype(np.int64)))
        tot += Fraction(int(qm[b])) * Fraction(2) ** int(qe[b]) * P * d
    return exact.ftz(exact.round_f32(tot))


def test_scores_fraction_brute_force_and_head_groups():
    g = np.random.default_rng(21)
    nh, nkv, npos, hd = 4, 2, 37, 64
    q = (g.standard_normal((nh, hd)) * 2.0 ** g.integers(-8, 8, (nh, 1))).astype(np.float32)
    k = (g.standard_normal((nkv * npos, hd)) * 2.0 ** g.integers(-8, 8, (nkv * npos, 1))).astype(np.float32)
    ks, kc = oracle.kv_cache_rows(k)
    ks, kc = ks.reshape(nkv, npos), kc.reshape(nkv, npos, hd)
    for mode in (oracle.PERBLOCK, oracle.SUB32):
        qc, qm, qe = oracle.kv_quantize_heads(q, mode)
        got = oracle.kv_scores(mode, qc, qm, qe, ks, kc)
        for h in range(nh):
            for j in range(npos):
                want = _score_fraction(qc[h], qm[h], qe[h], ks[h // 2, j], kc[h // 2, j], mode)
                assert got[h, j].view(np.uint32) == want.view(np.uint32), (mode, h, j)
    # closed form: a query of all 127 codes under scale 1 (m = 128, e = -7) against a key of all
    # 1 codes under scale 1 scores 127 * 64 = 8128
    qc = np.full((1, 64), 127, np.int8)
    got = oracle.kv_scores(oracle.PERBLOCK, qc, np.array([[128]], np.uint8), np.array([[-7]], np.int16),
                           np.array([[0x3C00]], np.uint16), np.ones((1, 1, 64), np.int8))
    assert float(got[0, 0]) == 8128.0
    # a key whose scale is not finite scores the canonical NaN
    got = oracle.kv_scores(oracle.PERBLOCK, qc, np.array([[128]], np.uint8), np.array([[-7]], np.int16),
                           np.array([[0x7C00]], np.uint16), np.ones((1, 1, 64), np.int8))
    assert got.view(np.uint32)[0, 0] == 0x7FC00000


def _weighted_fraction(p, vs, vc):
    npos, hd = vc.shape
    y = np.zeros(hd, np.float32)
    for j0 in range(0, npos, oracle.VALUE_BLOCK):
        js = range(j0, min(npos, j0 + oracle.VALUE_BLOCK))
        w = [exact.ftz(np.float32(np.float32(p[j]) * np.float32(np.array([vs[j]], np.uint16).view(np.float16)[0])))
             for j in js]
        amax = max(abs(Fraction(float(v))) for v in w)
        E = 0 if amax == 0 else exact.least_scale(amax, 1)[1]
        u = [round(Fraction(float(v)) / Fraction(2) ** E) for v in w]
        for e in range(hd):
            T = sum(u[i] * int(vc[j, e]) for i, j in enumerate(js))
            y[e] = exact.fadd(y[e], exact.ftz(exact.round_f32(Fraction(T) * Fraction(2) ** E)))
    return y


def test_weighted_fraction_brute_force():
    g = np.random.default_rng(31)
    nh, nkv, npos, hd = 2, 1, 75, 16
    v = (g.standard_normal((npos, hd)) * 2.0 ** g.integers(-6, 6, (npos, 1))).astype(np.float32)
    vs, vc = oracle.kv_cache_rows(v)
    logits = g.standard_normal((nh, npos)) * 3
    p = (np.exp(logits) / np.exp(logits).sum(1, keepdims=True)).astype(np.float32)
    p[1, 40:50] = 0                                     # a partly zero block
    got = oracle.kv_weighted(p, vs[None], vc[None])
    for h in range(nh):
        want = _weighted_fraction(p[h], vs, vc)
        assert np.array_equal(got[h].view(np.uint32), want.view(np.uint32)), h


def test_weighted_closed_forms():
    # one-hot probabilities under value scale 1: w = (1, 0, ...), the least power of two with
    # 127 * 2^E >= 1 is 2^-6, u_0 = 64, and each element's piece is exactly its value code
    vc = np.arange(-8, 8, dtype=np.int8).reshape(1, 16).repeat(40, 0)
    vc[0] = np.arange(16) - 5
    vs = np.full(40, 0x3C00, np.uint16)
    p = np.zeros((1, 40), np.float32)
    p[0, 0] = 1.0
    got = oracle.kv_weighted(p, vs[None], vc[None])
    assert list(got[0]) == [float(t) for t in np.arange(16) - 5]
    # a value row whose scale is not finite makes its block's pieces NaN
    vs[33] = 0x7C00
    got = oracle.kv_weighted(p, vs[None], vc[None])
    assert np.all(got.view(np.uint32) == 0x7FC00000)


def _order_case():
    """Three blocks whose pieces are 1, 2^-24, 2^-24 (one position each: p = 1 or 2^-24 under
    value scale 1 and value code 1): added in block order the two small pieces each tie to
    even and vanish (1.0); the last block first would give 1 + 2^-23."""
    npos = 96
    p = np.zeros((1, npos), np.float32)
    p[0, 0], p[0, 32], p[0, 64] = 1.0, 2.0 ** -24, 2.0 ** -24
    vs = np.full(npos, 0x3C00, np.uint16)
    vc = np.ones((npos, 1), np.int8)
    return p, vs, vc


def test_weighted_adds_blocks_in_order():
    p, vs, vc = _order_case()
    got = oracle.kv_weighted(p, vs[None], vc[None])
    assert float(got[0, 0]) == 1.0


def _flushed_sign_case():
    """Two heads, each over its own KV head of 96 positions (scales 1.0), hand-worked: head 0's
    blocks give the pieces 2^-125, -5 * 2^-127 and 0 (block 0: w = 2^-125, E = -131 as
    127 * 2^-132 < 2^-125 <= 127 * 2^-131, code 64, value 1; block 1: w = 5 * 2^-127, E = -131,
    code 80, value -1); head 1 has the zero block first.  The running sum 2^-125 - 5 * 2^-127 =
    -2^-127 is subnormal and flushes to -0: head 1 ends there (-0), while head 0 adds the zero
    block's +0 after it (-0 + +0 = +0 under round to nearest)."""
    npos, hd = 96, 32
    p = np.zeros((2, npos), np.float32)
    vs = np.full((2, npos), 0x3C00, np.uint16)
    vc = np.zeros((2, npos, hd), np.int8)
    for h, b0 in ((0, 0), (1, 32)):
        p[h, b0] = np.float32(2.0 ** -125)
        vc[h, b0, :] = 1
        p[h, b0 + 32] = np.float32(5 * 2.0 ** -127)
        vc[h, b0 + 32, :] = -1
    return p, vs, vc


def test_weighted_flushes_a_subnormal_running_sum_to_a_signed_zero():
    p, vs, vc = _flushed_sign_case()
    got = oracle.kv_weighted(p, vs, vc).view(np.uint32)
    assert (got[0] == 0x00000000).all()
    assert (got[1] == 0x80000000).all()


def _kv_quick_pins(mutant: int) -> bool:
    try:
        for x in (np.float32(1 + 2.0 ** -11), np.float32(2.0 ** -25), np.float32(1 + 3 * 2.0 ** -11)):
            if oracle.f16_rne(x, mutant) != int(np.array([x], np.float32).astype(np.float16).view(np.uint16)[0]):
                return False
        x = np.zeros((1, 32), np.float32)
        x[0, :8] = [127, 63.5, -0.5, 1.5, 2.5, -2.5, 0.49, -126.5]
        s, c = oracle.kv_cache_rows(x, mutant)
        if int(s[0]) != 0x3C00 or list(c[0, :8]) != [127, 64, 0, 2, 2, -2, 0, -126]:
            return False
        g = np.random.default_rng(31)
        v = (g.standard_normal((75, 16)) * 2.0 ** g.integers(-6, 6, (75, 1))).astype(np.float32)
        vs, vc = oracle.kv_cache_rows(v)
        p = g.random((1, 75)).astype(np.float32)
        got = oracle.kv_weighted(p, vs[None], vc[None], mutant)
        if not np.array_equal(got[0].view(np.uint32), _weighted_fraction(p[0], vs, vc).view(np.uint32)):
            return False
        p, vs, vc = _order_case()
        if float(oracle.kv_weighted(p, vs[None], vc[None], mutant)[0, 0]) != 1.0:
            return False
    except oracle.OracleError:
        return False
    return True


@pytest.mark.slow
def test_kv_mutants_are_caught():
    assert _kv_quick_pins(0)
    for mutant in (14, 15, 16, 17):
        assert not _kv_quick_pins(mutant), f"oracle mutant {mutant} passes every KV quick pin"
