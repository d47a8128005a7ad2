"""GPU parity for attention over an int8 KV cache, bit for bit against the oracle
([numerics] Functions cache_row, int8_codes, quantize_head, int8_score, weighted_int8;
Constants INV_127, VALUE_BLOCK): cache rows with zero, denormal, subnormal-scale, overflowing,
NaN and infinite rows; query heads under both scalings and every head size; scores with grouped
query heads, special key scales and Sub32 query blocks spread past the exact sum's window;
weighted sums over ragged, empty and poisoned blocks; the decode shapes at full size; and the
chain cache -> query -> scores -> weights -> weighted sum."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
HDS = [32, 64, 128, 256]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import block_format_gemv_amd as q
    oracle.set_threads(8)
    return q


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).reshape(-1)


def same_bits(got, want, what):
    g, w = f32_bits(got), f32_bits(want)
    bad = np.nonzero(g != w)[0]
    assert len(bad) == 0, f"{what}: {len(bad)} mismatches; first at {bad[0]}: got {g[bad[0]]:08x} want {w[bad[0]]:08x}"


def u16_dev(a: np.ndarray):
    """uint16 bits as a device int16 tensor (same bytes)."""
    return dev(np.ascontiguousarray(a, np.uint16).view(np.int16))


def u16_host(t) -> np.ndarray:
    return host(t).view(np.uint16)


def pack_scales(m: np.ndarray, e: np.ndarray) -> np.ndarray:
    """(m, e) -> the 4-byte scale records {int16 e; uint8 m; uint8 pad} as int32 words."""
    w = (e.astype(np.int64) & 0xFFFF) | (m.astype(np.int64) << 16)
    return w.astype(np.uint32).view(np.int32)


def unpack_scales(words: np.ndarray):
    w = words.astype(np.int64) & 0xFFFFFFFF
    return ((w >> 16) & 0xFF).astype(np.uint8), (w & 0xFFFF).astype(np.uint16).view(np.int16)


# --- cache rows ---------------------------------------------------------------------------

def special_rows(hd: int, seed: int) -> np.ndarray:
    """Rows that reach every branch of the cache-row scale and code."""
    g = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(hd, np.float32))                                          # zero scale
    rows.append((g.standard_normal(hd) * 1e-39).astype(np.float32))                # denormals only
    rows.append((g.standard_normal(hd) * 1e-5).astype(np.float32))                 # subnormal binary16 scale
    rows.append((g.standard_normal(hd) * 1e-9).astype(np.float32))                 # scale rounds to 0
    rows.append(np.clip(g.standard_normal(hd) * 3e38, -3.4e38, 3.4e38).astype(np.float32))   # scale overflows
    r = g.standard_normal(hd).astype(np.float32); r[3] = np.nan; rows.append(r)    # NaN passed over
    r = g.standard_normal(hd).astype(np.float32); r[5] = -np.inf; rows.append(r)   # infinite amax
    r = np.zeros(hd, np.float32); r[0] = 127.0
    r[1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -3.5]; rows.append(r)        # ties to even
    r = (g.standard_normal(hd) * 4000).astype(np.float32); r[0] = 65504.0 * 127; rows.append(r)
    r = g.standard_normal(hd).astype(np.float32); r[2] = -0.0; r[4] = 1e-40; rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("hd", HDS)
def test_cache_rows(qg, hd):
    x = np.concatenate([gen.kv_rows(27, hd, 7 + hd), special_rows(hd, hd)])   # 37 rows: ragged
    say(f"cache rows hd={hd} n={len(x)}")
    want_s, want_c = oracle.kv_cache_rows(x)
    n = len(x)
    scales = torch.full((n,), 0x5555, dtype=torch.int16, device=DEV)
    codes = torch.full((n, hd), 99, dtype=torch.int8, device=DEV)
    qg.qg_kv_cache_rows(n, hd, dev(x), scales, codes)
    torch.cuda.synchronize()
    assert np.array_equal(u16_host(scales), want_s)
    assert np.array_equal(host(codes), want_c)


def test_cache_rows_scale_rounds_twice(qg):
    """Row maxima whose product with binary32 1/127 lands, once rounded to binary32, on the
    other side of a binary16 rounding boundary than the exact product: the scale is the binary16
    of the binary32 product (two roundings), never the exact product rounded once."""
    g = np.random.default_rng(11)
    inv = np.float32(1.0) / np.float32(127.0)
    a = (g.uniform(1.0, 2.0, 400000) * 2.0 ** g.integers(-10, 12, 400000)).astype(np.float32)
    once = (a.astype(np.float64) * np.float64(inv)).astype(np.float16)     # exact product: 48 bits
    twice = (a * inv).astype(np.float32).astype(np.float16)
    amax = a[once != twice][:64]
    assert len(amax) >= 16
    hd = 64
    x = (g.uniform(-1.0, 1.0, (len(amax), hd)) * amax[:, None]).astype(np.float32)
    x[:, 0] = amax
    want_s, want_c = oracle.kv_cache_rows(x)
    assert np.array_equal(want_s, twice[once != twice][:64].view(np.uint16))
    n = len(x)
    scales = torch.zeros(n, dtype=torch.int16, device=DEV)
    codes = torch.zeros((n, hd), dtype=torch.int8, device=DEV)
    qg.qg_kv_cache_rows(n, hd, dev(x), scales, codes)
    torch.cuda.synchronize()
    assert np.array_equal(u16_host(scales), want_s)
    assert np.array_equal(host(codes), want_c)


def test_cache_rows_one_row_and_empty(qg):
    x = gen.kv_rows(1, 128, 5)
    want_s, want_c = oracle.kv_cache_rows(x)
    scales = torch.zeros(1, dtype=torch.int16, device=DEV)
    codes = torch.zeros((1, 128), dtype=torch.int8, device=DEV)
    qg.qg_kv_cache_rows(1, 128, dev(x), scales, codes)
    qg.qg_kv_cache_rows(0, 128, None, None, None)
    torch.cuda.synchronize()
    assert np.array_equal(u16_host(scales), want_s) and np.array_equal(host(codes), want_c)


# --- query heads --------------------------------------------------------------------------

def special_heads(nh: int, hd: int, mode: int, seed: int) -> np.ndarray:
    if mode == oracle.SUB32:
        q, _ = gen.act_sub32(nh, hd, seed)
    else:
        q = gen.act_outliers(nh, hd, seed)
    q[1] = 0.0                                          # an all-zero head
    q[2, :] = (q[2, :] * 1e-39).astype(np.float32)      # denormals read as zero
    q[3, 1] = np.nan
    q[4, hd - 1] = 1e-40
    q[5, 7] = 3e38                                      # the largest scales
    return q


@pytest.mark.parametrize("hd", HDS)
@pytest.mark.parametrize("mode", [0, 1], ids=["perblock", "sub32"])
def test_quantize_heads(qg, mode, hd):
    nh = 13                                             # 13 * hd elements: a ragged last wave
    q = special_heads(nh, hd, mode, 40 + hd + mode)
    say(f"quantize heads mode={mode} hd={hd} nh={nh}")
    want_c, want_m, want_e = oracle.kv_quantize_heads(q, mode)
    nb = 1 if mode == qg.PERBLOCK else hd // 32
    codes = torch.full((nh, hd), 99, dtype=torch.int8, device=DEV)
    scales = torch.full((nh, nb), -1, dtype=torch.int32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    qg.qg_kv_quantize_heads(mode, nh, hd, dev(q), codes, scales, flag)
    torch.cuda.synchronize()
    m, e = unpack_scales(host(scales))
    assert np.array_equal(host(codes), want_c)
    assert np.array_equal(m, want_m) and np.array_equal(e, want_e)
    assert int(flag.item()) == 0


@pytest.mark.parametrize("mode", [0, 1], ids=["perblock", "sub32"])
def test_quantize_heads_infinite(qg, mode):
    hd, nh = 128, 4
    q = gen.act_normal(nh, hd, 77)
    q[2, 33] = np.inf
    want_c, want_m, want_e = oracle.kv_quantize_heads(q, mode, check=False)
    with pytest.raises(oracle.OracleError):
        oracle.kv_quantize_heads(q, mode)
    nb = 1 if mode == qg.PERBLOCK else hd // 32
    codes = torch.zeros((nh, hd), dtype=torch.int8, device=DEV)
    scales = torch.zeros((nh, nb), dtype=torch.int32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    qg.qg_kv_quantize_heads(mode, nh, hd, dev(q), codes, scales, flag)
    torch.cuda.synchronize()
    m, e = unpack_scales(host(scales))
    assert int(flag.item()) == 1
    assert np.array_equal(host(codes), want_c)
    assert np.array_equal(m, want_m) and np.array_equal(e, want_e)


# --- scores -------------------------------------------------------------------------------

SPECIAL_KEY_SCALES = [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x3C00, 0x7C00, 0xFC00, 0x7E00, 0x7D01]


def run_scores(qg, mode, qc, qm, qe, ks, kc):
    nh, hd = qc.shape
    nkv, npos = ks.shape
    out = torch.full((nh, npos), 7.0, dtype=torch.float32, device=DEV)
    qg.qg_kv_scores(mode, nh, nkv, npos, hd, dev(qc), dev(pack_scales(qm, qe)), u16_dev(ks), dev(kc), out)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("hd", HDS)
@pytest.mark.parametrize("mode", [0, 1], ids=["perblock", "sub32"])
def test_scores(qg, mode, hd):
    nh, nkv, npos = 8, 2, 300                           # grouped heads; 300 = 256 + a ragged tail
    keys = gen.kv_rows(nkv * npos, hd, 90 + hd)
    ks, kc = oracle.kv_cache_rows(keys)
    ks = ks.reshape(nkv, npos).copy()
    kc = kc.reshape(nkv, npos, hd)
    ks[0, :len(SPECIAL_KEY_SCALES)] = SPECIAL_KEY_SCALES
    ks[1, -len(SPECIAL_KEY_SCALES):] = SPECIAL_KEY_SCALES
    if mode == qg.SUB32:
        q, _ = gen.act_sub32(nh, hd, 60 + hd)
    else:
        q = gen.act_outliers(nh, hd, 60 + hd)
    q[3] = 0.0
    qc, qm, qe = oracle.kv_quantize_heads(q, mode)
    say(f"scores mode={mode} hd={hd} nh={nh} nkv={nkv} npos={npos}")
    want = oracle.kv_scores(mode, qc, qm, qe, ks, kc)
    same_bits(run_scores(qg, mode, qc, qm, qe, ks, kc), want, f"scores mode={mode} hd={hd}")


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_scores_sub32_past_the_window(qg, hd):
    """Sub32 query blocks whose exponents lie far apart, so that the exact sum floors the small
    terms below its window (the largest term first among equals)."""
    nh, nkv, npos = 4, 4, 70
    g = np.random.default_rng(hd)
    keys = gen.kv_rows(nkv * npos, hd, 300 + hd)
    ks, kc = oracle.kv_cache_rows(keys)
    ks, kc = ks.reshape(nkv, npos), kc.reshape(nkv, npos, hd)
    nb = hd // 32
    qc = g.integers(-127, 128, size=(nh, hd)).astype(np.int8)
    qm = g.integers(8, 16, size=(nh, nb)).astype(np.uint8)
    qe = g.integers(-40, 40, size=(nh, nb)).astype(np.int16)
    qe[:, 0] = -120                                     # 200 binades below block 1
    qe[:, 1] = 80
    qe[1, :] = 5                                        # equal exponents: ties between terms
    qm[1, :] = 8
    say(f"scores past the window hd={hd}")
    want = oracle.kv_scores(qg.SUB32, qc, qm, qe, ks, kc)
    same_bits(run_scores(qg, qg.SUB32, qc, qm, qe, ks, kc), want, f"window hd={hd}")


def test_scores_one_position_and_heads_per_kv(qg):
    hd = 128
    for nh, nkv, npos in [(4, 4, 1), (6, 1, 33), (2, 2, 257)]:
        keys = gen.kv_rows(nkv * npos, hd, nh * 1000 + npos)
        ks, kc = oracle.kv_cache_rows(keys)
        ks, kc = ks.reshape(nkv, npos), kc.reshape(nkv, npos, hd)
        q = gen.act_normal(nh, hd, npos)
        for mode in (0, 1):
            qc, qm, qe = oracle.kv_quantize_heads(q, mode)
            want = oracle.kv_scores(mode, qc, qm, qe, ks, kc)
            same_bits(run_scores(qg, mode, qc, qm, qe, ks, kc), want, f"nh={nh} nkv={nkv} npos={npos} mode={mode}")


# --- weighted sum -------------------------------------------------------------------------

def run_weighted(qg, probs, vs, vc, fill=7.0, passes=1):
    """qg_kv_weighted (passes=1) or qg_kv_weighted_with_workspace (passes=2, over a workspace
    filled with NaN beforehand, a few words longer than needed, so that a piece left unwritten
    shows)."""
    nh, npos = probs.shape
    nkv, _, hd = vc.shape
    out = torch.full((nh, hd), fill, dtype=torch.float32, device=DEV)
    args = (dev(probs), u16_dev(vs), dev(vc)) if npos else (None, None, None)
    if passes == 1:
        qg.qg_kv_weighted(nh, nkv, npos, hd, *args, out)
    else:
        need = qg.qg_kv_weighted_workspace(nh, npos, hd)
        ws = torch.full((need // 4 + 5,), float("nan"), dtype=torch.float32, device=DEV)
        qg.qg_kv_weighted_with_workspace(nh, nkv, npos, hd, *args, out, ws)
    torch.cuda.synchronize()
    return host(out)


@pytest.fixture(params=[1, 2], ids=["one_pass", "two_pass"])
def passes(request):
    return request.param


def cached_values(nkv, npos, hd, seed):
    vals = gen.kv_rows(nkv * npos, hd, seed)
    vs, vc = oracle.kv_cache_rows(vals)
    return vs.reshape(nkv, npos).copy(), vc.reshape(nkv, npos, hd)


@pytest.mark.parametrize("hd", HDS)
@pytest.mark.parametrize("npos", [1, 31, 32, 33, 300, 1000])
def test_weighted(qg, hd, npos, passes):
    nh, nkv = 8, 2
    vs, vc = cached_values(nkv, npos, hd, 500 + hd + npos)
    probs = gen.attn_weights(nh, npos, 600 + npos)
    say(f"weighted hd={hd} npos={npos} passes={passes}")
    want = oracle.kv_weighted(probs, vs, vc)
    same_bits(run_weighted(qg, probs, vs, vc, passes=passes), want, f"weighted hd={hd} npos={npos}")


@pytest.mark.parametrize("hd", [32, 128, 256])
def test_weighted_special_blocks(qg, hd, passes):
    """One head per KV head, each with one special block: zero weights, weights whose products
    are subnormal (read as zero), a NaN weight, an infinite product, tiny equal products (the
    scale near the bottom), the largest value scale, and value scales that are not finite
    (NaN pieces)."""
    nh = nkv = 8
    npos = 32 * 9 + 5
    vs, vc = cached_values(nkv, npos, hd, 700 + hd)
    probs = gen.attn_weights(nh, npos, 800 + hd)
    probs[0, 0:32] = 0.0                                # all-zero block: E = 0, pieces +0
    probs[1, 32:64] = 1e-41                             # subnormal weights ...
    probs[1, 40] = 1e-30                                # ... beside one tiny normal one
    probs[2, 70] = np.nan                               # a NaN weight codes as 0
    probs[3, 100] = 3e38                                # times a scale of 2: an infinite product
    vs[3, 100] = 0x4000
    probs[4, 128:160] = np.float32(2.0 ** -120)         # tiny products: E near the bottom
    probs[5, 160:192] = np.float32(1.0)
    vs[5, 160:192] = 0x7BFF                             # the largest finite value scale
    vs[6, 200] = 0x7C00                                 # an infinite value scale
    vs[7, 260] = 0x7E01                                 # a NaN value scale
    say(f"weighted special blocks hd={hd} passes={passes}")
    want = oracle.kv_weighted(probs, vs, vc)
    same_bits(run_weighted(qg, probs, vs, vc, passes=passes), want, f"weighted special hd={hd}")
    assert np.isnan(want[3]).all() and np.isnan(want[6]).all() and np.isnan(want[7]).all()
    assert np.isfinite(want[[0, 1, 2, 4, 5]]).all()


@pytest.mark.parametrize("nh,nkv,npos,hd", [(40, 2, 100, 64), (36, 1, 65, 256), (64, 2, 97, 32),
                                            (5, 5, 129, 128), (16, 1, 32, 128)])
def test_weighted_grouped_heads(qg, nh, nkv, npos, hd, passes):
    """Query heads per KV head from 1 to 32: the two-pass form codes them 16 at a time from
    one read of the block's value rows."""
    vs, vc = cached_values(nkv, npos, hd, 900 + nh + npos)
    probs = gen.attn_weights(nh, npos, 950 + nh)
    probs[nh - 1, npos - 1] = np.nan
    say(f"weighted grouped nh={nh} nkv={nkv} npos={npos} hd={hd} passes={passes}")
    want = oracle.kv_weighted(probs, vs, vc)
    same_bits(run_weighted(qg, probs, vs, vc, passes=passes), want, f"grouped nh={nh} nkv={nkv}")


def test_weighted_workspace_reused_across_shapes(qg):
    """One workspace, sized for the largest call, serves calls of other shapes in turn; each
    result matches the oracle and the one-pass entry point."""
    shapes = [(32, 8, 1000, 128), (8, 2, 33, 64), (32, 8, 1000, 128), (4, 4, 1, 256), (8, 1, 0, 32)]
    need = max(qg.qg_kv_weighted_workspace(nh, npos, hd) for nh, _, npos, hd in shapes)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    for k, (nh, nkv, npos, hd) in enumerate(shapes):
        vs, vc = cached_values(nkv, npos, hd, 1000 + k)
        probs = gen.attn_weights(nh, npos, 1100 + k)
        out = torch.full((nh, hd), 7.0, dtype=torch.float32, device=DEV)
        args = (dev(probs), u16_dev(vs), dev(vc)) if npos else (None, None, None)
        say(f"weighted workspace reuse {k}: nh={nh} nkv={nkv} npos={npos} hd={hd}")
        qg.qg_kv_weighted_with_workspace(nh, nkv, npos, hd, *args, out, ws)
        torch.cuda.synchronize()
        want = oracle.kv_weighted(probs, vs, vc)
        same_bits(host(out), want, f"reuse {k}")
        same_bits(host(out), run_weighted(qg, probs, vs, vc), f"reuse {k} against one pass")


def test_weighted_order_of_blocks(qg, passes):
    """Three blocks whose pieces are 1, 2^-24, 2^-24: added in order they give 1; the order of
    the blocks decides the result."""
    hd, npos = 32, 96
    vc = np.zeros((1, npos, hd), np.int8)
    vs = np.full((1, npos), 0x3C00, np.uint16)        # scale 1
    probs = np.zeros((1, npos), np.float32)
    probs[0, 0] = 1.0
    vc[0, 0, :] = 1
    probs[0, 32] = np.float32(2.0 ** -24)
    vc[0, 32, :] = 1
    probs[0, 64] = np.float32(2.0 ** -24)
    vc[0, 64, :] = 1
    want = oracle.kv_weighted(probs, vs, vc)
    assert (want == 1.0).all()
    same_bits(run_weighted(qg, probs, vs, vc, passes=passes), want, "order")


def test_weighted_flushed_running_sum_keeps_its_sign(qg, passes):
    """A running sum of -2^-127 flushes to -0; a zero block after it gives +0 (hand-worked
    two-head case: pieces 2^-125, -5 * 2^-127, then 0 for head 0; the zero block first for
    head 1)."""
    hd, npos = 32, 96
    p = np.zeros((2, npos), np.float32)
    vs = np.full((2, npos), 0x3C00, np.uint16)
    vc = np.zeros((2, npos, hd), np.int8)
    for h, b0 in ((0, 0), (1, 32)):
        p[h, b0] = np.float32(2.0 ** -125)
        vc[h, b0, :] = 1
        p[h, b0 + 32] = np.float32(5 * 2.0 ** -127)
        vc[h, b0 + 32, :] = -1
    want = oracle.kv_weighted(p, vs, vc)
    assert (want[0].view(np.uint32) == 0).all() and (want[1].view(np.uint32) == 0x80000000).all()
    same_bits(run_weighted(qg, p, vs, vc, passes=passes), want, "flushed sign")


def test_weighted_empty_context(qg, passes):
    vc = np.zeros((2, 0, 64), np.int8)
    vs = np.zeros((2, 0), np.uint16)
    probs = np.zeros((4, 0), np.float32)
    want = oracle.kv_weighted(probs, vs, vc)
    got = run_weighted(qg, probs, vs, vc, fill=7.0, passes=passes)
    assert (want == 0).all()
    same_bits(got, want, "empty")


# --- the decode shapes at full size, and the chain ---------------------------------------

@pytest.fixture(scope="module")
def decode():
    return gen.kv_decode()                             # 32 heads, 8 KV heads, 4096 positions, hd 128


@pytest.mark.parametrize("mode", [0, 1], ids=["perblock", "sub32"])
def test_decode_full_size_chain(qg, decode, mode):
    keys, vals, query, weights = decode
    nkv, npos, hd = keys.shape
    nh = query.shape[0]
    say(f"decode chain mode={mode} nh={nh} nkv={nkv} npos={npos} hd={hd}")
    # the cache, written by the library from the f32 rows
    ks_d = torch.zeros(nkv * npos, dtype=torch.int16, device=DEV)
    kc_d = torch.zeros((nkv * npos, hd), dtype=torch.int8, device=DEV)
    vs_d = torch.zeros(nkv * npos, dtype=torch.int16, device=DEV)
    vc_d = torch.zeros((nkv * npos, hd), dtype=torch.int8, device=DEV)
    qg.qg_kv_cache_rows(nkv * npos, hd, dev(keys.reshape(-1, hd)), ks_d, kc_d)
    qg.qg_kv_cache_rows(nkv * npos, hd, dev(vals.reshape(-1, hd)), vs_d, vc_d)
    nb = 1 if mode == qg.PERBLOCK else hd // 32
    qc_d = torch.zeros((nh, hd), dtype=torch.int8, device=DEV)
    qs_d = torch.zeros((nh, nb), dtype=torch.int32, device=DEV)
    qg.qg_kv_quantize_heads(mode, nh, hd, dev(query), qc_d, qs_d, None)
    sc_d = torch.zeros((nh, npos), dtype=torch.float32, device=DEV)
    qg.qg_kv_scores(mode, nh, nkv, npos, hd, qc_d, qs_d, ks_d, kc_d, sc_d)
    torch.cuda.synchronize()

    ks, kc = oracle.kv_cache_rows(keys.reshape(-1, hd))
    vs, vc = oracle.kv_cache_rows(vals.reshape(-1, hd))
    assert np.array_equal(u16_host(ks_d), ks) and np.array_equal(host(kc_d), kc)
    assert np.array_equal(u16_host(vs_d), vs) and np.array_equal(host(vc_d), vc)
    qc, qm, qe = oracle.kv_quantize_heads(query, mode)
    m, e = unpack_scales(host(qs_d))
    assert np.array_equal(host(qc_d), qc) and np.array_equal(m, qm) and np.array_equal(e, qe)
    want_sc = oracle.kv_scores(mode, qc, qm, qe, ks.reshape(nkv, npos), kc.reshape(nkv, npos, hd))
    same_bits(host(sc_d), want_sc, f"decode scores mode={mode}")

    # the caller's softmax, here in float64 on the CPU from the oracle's scores; then the
    # weighted sum over the library's value cache against the oracle's
    s = want_sc.astype(np.float64)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    out = torch.zeros((nh, hd), dtype=torch.float32, device=DEV)
    qg.qg_kv_weighted(nh, nkv, npos, hd, dev(p), vs_d, vc_d, out)
    out2 = torch.zeros((nh, hd), dtype=torch.float32, device=DEV)
    ws = torch.empty(qg.qg_kv_weighted_workspace(nh, npos, hd), dtype=torch.uint8, device=DEV)
    qg.qg_kv_weighted_with_workspace(nh, nkv, npos, hd, dev(p), vs_d, vc_d, out2, ws)
    torch.cuda.synchronize()
    want = oracle.kv_weighted(p, vs.reshape(nkv, npos), vc.reshape(nkv, npos, hd))
    same_bits(host(out), want, f"decode weighted mode={mode}")
    same_bits(host(out2), want, f"decode weighted, two passes, mode={mode}")


def test_decode_full_size_weighted(qg, decode, passes):
    keys, vals, query, weights = decode
    nkv, npos, hd = vals.shape
    vs, vc = oracle.kv_cache_rows(vals.reshape(-1, hd))
    vs, vc = vs.reshape(nkv, npos), vc.reshape(nkv, npos, hd)
    want = oracle.kv_weighted(weights, vs, vc)
    same_bits(run_weighted(qg, weights, vs, vc, passes=passes), want, "decode weighted")
