"""Seeded synthetic inputs for the exact block-quantized GEMV.

This module only draws random numbers and lays them out as the logical fields of a
block-format matrix and as f32 activation rows. It computes nothing the method computes
(no activation scale, no code, no dot product), so both the CPU oracle and the GPU path
can take their inputs from here without sharing any of the arithmetic under test.

Every generator takes an explicit seed and uses numpy's PCG64 bit generator, so a
(shape, seed) pair names an input exactly.

Logical fields (one matrix of R rows and C columns, C a multiple of 256):

Q4_K-style (256-element blocks, 8 sub-blocks of 32):
    q     uint8 [R, C]        codes 0..15
    sc    uint8 [R, C/32]     sub-block scales 0..63
    mn    uint8 [R, C/32]     sub-block offsets 0..63
    d     uint16 [R, C/256]   first block scale, binary16 bits
    dmin  uint16 [R, C/256]   second block scale, binary16 bits

Q6_K-style (256-element blocks, 16 sub-blocks of 16):
    q     uint8 [R, C]        codes 0..63 (the weight uses q - 32)
    sc    int8  [R, C/16]     sub-block scales -128..127
    d     uint16 [R, C/256]   block scale, binary16 bits
"""
from __future__ import annotations

import numpy as np

BLOCK = 256

# Seeds, fixed once per role and never reused across roles.
SEED_TINY_W, SEED_TINY_X = 100, 101
SEED_ATTN_W, SEED_FFN_W = 110, 111
SEED_GATE_W = 112                  # the FFN gate projection, beside the up projection (seed 111)
SEED_K_W, SEED_V_W = 113, 114      # 1024 x 4096 K and V projections (Llama-8B grouped-query shapes)
SEED_Q8_W, SEED_Q4_0_W = 150, 151  # 14336 x 4096 Q8_0-style and Q4_0-style matrices
SEED_REP_X = 1_000_000          # repetition k of the decode workload uses SEED_REP_X + k
SEED_OUT_W, SEED_OUT_X = 120, 121
SEED_SUB32_X = 130              # repetition k uses SEED_SUB32_X + k
SEED_BATCH_X = 140              # batch of N columns uses SEED_BATCH_X + N
SEED_KV = 160                   # decode attention over a cached context: keys, values, query, weights


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f16_bits_of(values: np.ndarray) -> np.ndarray:
    """binary16 bits of float64 values: numpy's conversion (nearest, ties to even, subnormals kept)."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def q4k_fields(rows: int, cols: int, seed: int, scale_exp: int = -8) -> dict:
    """Q4_K-style matrix: q ~ U{0..15}, sc, mn ~ U{0..63}, d, dmin = f16(|N(0,1)| * 2^scale_exp)."""
    assert cols % BLOCK == 0
    g = _rng(seed)
    q = g.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    sc = g.integers(0, 64, size=(rows, cols // 32), dtype=np.uint8)
    mn = g.integers(0, 64, size=(rows, cols // 32), dtype=np.uint8)
    d = f16_bits_of(np.abs(g.standard_normal((rows, cols // BLOCK))) * 2.0 ** scale_exp)
    dmin = f16_bits_of(np.abs(g.standard_normal((rows, cols // BLOCK))) * 2.0 ** scale_exp)
    return {"fmt": "q4k", "rows": rows, "cols": cols, "q": q, "sc": sc, "mn": mn, "d": d, "dmin": dmin}


def q6k_fields(rows: int, cols: int, seed: int, scale_exp: int = -10) -> dict:
    """Q6_K-style matrix: q ~ U{0..63}, sc ~ U{-128..127}, d = f16(|N(0,1)| * 2^scale_exp)."""
    assert cols % BLOCK == 0
    g = _rng(seed)
    q = g.integers(0, 64, size=(rows, cols), dtype=np.uint8)
    sc = g.integers(-128, 128, size=(rows, cols // 16), dtype=np.int8)
    d = f16_bits_of(np.abs(g.standard_normal((rows, cols // BLOCK))) * 2.0 ** scale_exp)
    return {"fmt": "q6k", "rows": rows, "cols": cols, "q": q, "sc": sc, "d": d}


def q8_0_fields(rows: int, cols: int, seed: int, scale_exp: int = -8) -> dict:
    """Q8_0-style matrix (32-element blocks): q ~ U{-128..127} int8, one d = f16(|N(0,1)| * 2^scale_exp)
    per 32 weights."""
    assert cols % BLOCK == 0
    g = _rng(seed)
    q = g.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    d = f16_bits_of(np.abs(g.standard_normal((rows, cols // 32))) * 2.0 ** scale_exp)
    return {"fmt": "q8_0", "rows": rows, "cols": cols, "q": q, "d": d}


def q4_0_fields(rows: int, cols: int, seed: int, scale_exp: int = -8) -> dict:
    """Q4_0-style matrix (32-element blocks): q ~ U{0..15} (value q - 8), one d = f16(|N(0,1)| *
    2^scale_exp) per 32 weights."""
    assert cols % BLOCK == 0
    g = _rng(seed)
    q = g.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    d = f16_bits_of(np.abs(g.standard_normal((rows, cols // 32))) * 2.0 ** scale_exp)
    return {"fmt": "q4_0", "rows": rows, "cols": cols, "q": q, "d": d}


def slice_rows(fields: dict, idx) -> dict:
    """The same matrix restricted to the rows `idx` (any numpy index over rows)."""
    out = {}
    for k, v in fields.items():
        out[k] = v[idx] if isinstance(v, np.ndarray) else v
    out["rows"] = int(out["q"].shape[0])
    return out


def act_normal(n: int, cols: int, seed: int) -> np.ndarray:
    """n activation rows ~ N(0,1), float32."""
    return _rng(seed).standard_normal((n, cols), dtype=np.float32)


def act_outliers(n: int, cols: int, seed: int, rate: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """N(0,1) float32 rows where each element independently (probability `rate`) is multiplied
    by `factor` in float32."""
    g = _rng(seed)
    x = g.standard_normal((n, cols), dtype=np.float32)
    mask = g.random((n, cols)) < rate
    x[mask] = x[mask] * np.float32(factor)
    return x


def act_sub32(n: int, cols: int, seed: int, e_lo: int = -12, e_hi: int = 4) -> tuple[np.ndarray, np.ndarray]:
    """Laplace(0,1) float32 rows whose 32-element blocks are rescaled so that each block's
    largest magnitude lies in [127*8*2^t, 127*15*2^t] for a per-block target t drawn uniformly
    from e_lo..e_hi; blocks 0 and 1 of every row take t = e_lo and t = e_hi.

    Returns (x, t) with t int32 [n, cols/32]. Under a per-32 scale with a 4-bit significand the
    least admissible scale of such a block has exponent t, which the tests assert of the
    quantizer rather than assume here.
    """
    g = _rng(seed)
    nb = cols // 32
    lap = g.laplace(0.0, 1.0, size=(n, nb, 32))
    t = g.integers(e_lo, e_hi + 1, size=(n, nb)).astype(np.int32)
    t[:, 0] = e_lo
    if nb > 1:
        t[:, 1] = e_hi
    u = g.uniform(8.0, 15.0, size=(n, nb))
    target = np.float32(127.0) * u * np.exp2(t.astype(np.float64))   # wanted largest magnitude
    target = target.astype(np.float32).astype(np.float64)
    peak = np.max(np.abs(lap), axis=2)
    peak[peak == 0] = 1.0
    x = (lap / peak[..., None]) * target[..., None]
    x = x.astype(np.float32).reshape(n, cols)
    return x, t


# --- the named workloads -------------------------------------------------------------------

def tiny_q4k():
    """256 x 1024 Q4_K-style matrix and one N(0,1) activation row (PerBlock)."""
    return q4k_fields(256, 1024, SEED_TINY_W), act_normal(1, 1024, SEED_TINY_X)


def llama_q4k(which: str):
    """Llama-8B-shaped Q4_K-style matrices: 'attn' 4096 x 4096 (also the Q projection),
    'ffn' 14336 x 4096 (the up projection), 'gate' 14336 x 4096, 'k' and 'v' 1024 x 4096."""
    if which == "attn":
        return q4k_fields(4096, 4096, SEED_ATTN_W)
    if which == "ffn":
        return q4k_fields(14336, 4096, SEED_FFN_W)
    if which == "gate":
        return q4k_fields(14336, 4096, SEED_GATE_W)
    if which == "k":
        return q4k_fields(1024, 4096, SEED_K_W)
    if which == "v":
        return q4k_fields(1024, 4096, SEED_V_W)
    raise ValueError(which)


def decode_act(rep: int, cols: int = 4096) -> np.ndarray:
    """Activation row of decode repetition `rep`: N(0,1) with 1% outliers x20."""
    return act_outliers(1, cols, SEED_REP_X + rep)


def output_q6k():
    """128256 x 4096 Q6_K-style output projection and its N(0,1) activation row."""
    return q6k_fields(128256, 4096, SEED_OUT_W), act_normal(1, 4096, SEED_OUT_X)


def sub32_act(rep: int, cols: int = 4096):
    return act_sub32(1, cols, SEED_SUB32_X + rep)


def batch_act(n: int, cols: int = 4096) -> np.ndarray:
    return act_normal(n, cols, SEED_BATCH_X + n)


# --- attention over an int8 KV cache -----------------------------------------------------

def kv_rows(n: int, hd: int, seed: int) -> np.ndarray:
    """n cached key or value rows of hd elements, float32: N(0,1) times a per-row magnitude
    2^u with u uniform in [-3, 3] (rows of one context differ in size)."""
    g = _rng(seed)
    x = g.standard_normal((n, hd))
    x *= np.exp2(g.uniform(-3.0, 3.0, size=(n, 1)))
    return x.astype(np.float32)


def attn_weights(nh: int, npos: int, seed: int) -> np.ndarray:
    """Per-head attention weights over npos positions, float32, each row positive and summing
    to about 1: exp of N(0, 2^2) draws, normalised in float64 (a peaked, uneven mix)."""
    g = _rng(seed)
    z = g.standard_normal((nh, npos)) * 2.0
    w = np.exp(z - z.max(axis=1, keepdims=True)) if npos else z
    if npos:
        w /= w.sum(axis=1, keepdims=True)
    return w.astype(np.float32)


def kv_decode(nh: int = 32, nkv: int = 8, npos: int = 4096, hd: int = 128, seed: int = SEED_KV):
    """One decode step's attention inputs (Llama-8B grouped-query shapes by default): the
    context's keys and values f32 [nkv, npos, hd], the query f32 [nh, hd] and the weights
    f32 [nh, npos]."""
    keys = kv_rows(nkv * npos, hd, seed).reshape(nkv, npos, hd)
    vals = kv_rows(nkv * npos, hd, seed + 1).reshape(nkv, npos, hd)
    query = act_normal(nh, hd, seed + 2)
    weights = attn_weights(nh, npos, seed + 3)
    return keys, vals, query, weights


# --- hand-laid inputs ----------------------------------------------------------------------

def sub32_boundary_rows():
    """A 7 x 256 Q4_K-style matrix and two activation rows laid out by hand so that Sub32 group
    values fall on or just beside a binary32 rounding boundary, where a binary64 value rounded
    again to binary32 would be off, and (second row) below the binary32 normal range.

    Activation row 0: block 0 holds 1016 and 256 (the scale 8 * 2^0, codes 127 and 32), block 1
    holds 127, 12, -11 and -127 times 2^-13 (the scale 8 * 2^-16, codes of those values), each
    of the other six blocks one element 1016 * 2^-8 (weights 0 there; the group's exponents
    span 16 places).  Row 1 is row 0 times 2^-112.  Weights: nibble 8 at element 1
    (against the code 32) and at element 33 (against the code 12), every other nibble 0;
    sub-block scales 32 and 1, offset 1 on sub-block 1 alone.  The rows differ in d and dmin
    (binary16 bits) and in whether sub-block 0 counts:
        row  d       dmin    sc[0]
        0    0x3C00  0x0001  32      1.0, 2^-24
        1    0x3C00  0x8001  32      1.0, -2^-24
        2    0x3C00  0x0000  32      1.0, 0
        3    0xBC00  0x0001  32      -1.0, 2^-24
        4    0x3C00  0x0001  0       1.0, 2^-24
        5    0x0001  0x0000  0       2^-24, 0
        6    0x8001  0x0000  0       -2^-24, 0
    """
    rows, cols = 7, 256
    x = np.zeros((2, cols), np.float32)
    x[0, 0], x[0, 1] = 1016.0, 256.0
    x[0, 32:36] = np.array([127.0, 12.0, -11.0, -127.0]) * 2.0 ** -13
    x[0, 64::32] = 1016.0 * 2.0 ** -8
    x[1] = x[0] * np.float32(2.0 ** -112)
    q = np.zeros((rows, cols), np.uint8)
    q[:, 1] = 8
    q[:, 33] = 8
    sc = np.zeros((rows, cols // 32), np.uint8)
    sc[:, 0], sc[:, 1] = 32, 1
    sc[4:, 0] = 0
    mn = np.zeros((rows, cols // 32), np.uint8)
    mn[:, 1] = 1
    d = np.array([[0x3C00], [0x3C00], [0x3C00], [0xBC00], [0x3C00], [0x0001], [0x8001]], np.uint16)
    dmin = np.array([[0x0001], [0x8001], [0x0000], [0x0001], [0x0001], [0x0000], [0x0000]], np.uint16)
    f = {"fmt": "q4k", "rows": rows, "cols": cols, "q": q, "sc": sc, "mn": mn, "d": d, "dmin": dmin}
    return f, x
