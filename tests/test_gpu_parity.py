"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for bit.

Activation codes, scales and code sums are compared byte for byte; integer block sums
exactly; every f32 output by its bits (compared as uint32, NaN canonical), never within a
tolerance.  Shapes span several tiles with ragged tails; the named workloads run at full
size in the launch configuration the benchmark times, every output of every repetition
compared with the oracle's.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import block_format_gemv_amd as q
    q.qg_set_tuning(q.TUNE_WAVES_PER_WG, 0)
    q.qg_set_tuning(q.TUNE_MFMA_MIN_COLS, 0)
    q.qg_set_tuning(q.TUNE_MFMA_COL_TILES, 0)
    q.qg_set_tuning(q.TUNE_COLS_KERNEL, 0)
    q.qg_set_tuning(q.TUNE_MFMA_TABLES, 0)
    q.qg_set_tuning(q.TUNE_MFMA_FORM, 0)
    q.qg_set_tuning(q.TUNE_GEMM_ROW_TILES, 0)
    q.qg_set_tuning(q.TUNE_GEMV_QUARTER, 0)
    oracle.set_threads(8)
    return q


DEV = "cuda:0"


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(a) -> np.ndarray:
    a = a.detach().cpu().numpy() if hasattr(a, "detach") else np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def first_mismatch(got, want):
    g, w = bits(got).reshape(-1), bits(want).reshape(-1)
    bad = np.nonzero(g != w)[0]
    if len(bad) == 0:
        return None
    i = bad[0]
    return f"{len(bad)} mismatches; first at {i}: got {g[i]:08x} want {w[i]:08x}"


def gpu_quant(q, x: np.ndarray, mode: int, fmt=None):
    xd = dev(x.astype(np.float32))
    a = q.quantize_act(xd, mode, fmt or q.Q4K)
    m, e = a.scale_fields()
    return a, a.codes.cpu().numpy(), m, e, a.csums.cpu().numpy()


class Mat:
    """A matrix's logical fields, its image on the GPU, and its format code."""

    def __init__(self, q, fields):
        self.f = fields
        self.fmt = q.FMT_CODES[fields["fmt"]]
        self.rows, self.cols = fields["rows"], fields["cols"]
        self.img = dev(q.pack(fields))


def run_gemv(q, M: Mat, act, out=None):
    return q.gemv(M.fmt, M.rows, M.cols, M.img, act, out=out)


# --- the quantizer -------------------------------------------------------------------------

def _quant_inputs():
    g = np.random.Generator(np.random.PCG64(5))
    x = gen.act_outliers(4, 4096, 9)
    adv = g.standard_normal((6, 1024)).astype(np.float32)
    adv[0, :256] = 0                                         # all-zero block
    adv[1, 3] = np.nan                                       # NaN: code 0, passed over
    adv[1, 700] = np.nan
    adv[2] *= np.float32(2.0 ** -126)                        # many subnormals (read as 0)
    adv[3] *= np.float32(2.0 ** 120)                         # huge
    adv[4] = np.round(adv[4] * 8) / 8                        # many exact ties
    adv[5, 256:512] = np.float32(1.0)                        # exact boundary 127*m*2^e cases
    adv[5, 300] = np.float32(127.0 * 130 * 2.0 ** -14)
    sub, _ = gen.sub32_act(3)
    return [("outliers", x), ("adversarial", adv), ("sub32", sub), ("normal", gen.act_normal(64, 4096, 140 + 64))]


@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_matches_oracle(qg, mode):
    for name, x in _quant_inputs():
        say("quantize", name, x.shape, "mode", mode)
        _, c, m, e, s = gpu_quant(qg, x, mode)
        oc, om, oe, os_ = oracle.quantize(x, mode)
        assert np.array_equal(c, oc), name
        assert np.array_equal(m, om) and np.array_equal(e, oe), name
        assert np.array_equal(s, os_), name


def _tie_rows(mode: int, nblocks: int, seed: int) -> np.ndarray:
    """Activation rows built on the quantizer's grid: per activation block a scale s = m*2^e,
    an element at exactly 127*s (the least-scale boundary) or one binary32 step either side
    of it, and the other elements at exact half-integer multiples of s (ties), one step
    either side of a tie, or exact multiples of s.  Every value is exact in binary32."""
    g = np.random.Generator(np.random.PCG64(seed))
    blk, lo, hi = (256, 128, 256) if mode == 0 else (32, 8, 16)
    x = np.empty((nblocks, blk), np.float32)
    for b in range(nblocks):
        m = int(g.integers(lo, hi))
        e = int(g.integers(-118, 100))
        n = g.integers(-127, 127, blk)
        kind = g.integers(0, 4, blk)
        half = np.ldexp((2.0 * n + 1.0) * m, e - 1).astype(np.float32)        # (n + 1/2) * s
        v = np.where(kind == 0, half, np.where(kind == 1, np.nextafter(half, np.float32(np.inf)),
                     np.where(kind == 2, np.nextafter(half, np.float32(-np.inf)),
                              np.ldexp(float(m) * n, e).astype(np.float32))))
        top = np.float32(np.ldexp(127.0 * m, e))
        top = [top, np.nextafter(top, np.float32(np.inf)), np.nextafter(top, np.float32(0))][b % 3]
        v[int(g.integers(0, blk))] = top if b % 2 else -top
        x[b] = v.astype(np.float32)
    return x.reshape(-1, 1024)


@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_ties_and_grid_boundaries(qg, mode):
    """Codes of exact ties (to even) and of values one binary32 step from a tie, and the
    least scale when the block's largest magnitude is exactly 127*m*2^e or one step off it:
    the quantizer, the one-launch quantize + GEMV and the oracle agree bit for bit."""
    x = _tie_rows(mode, 4096 if mode == 0 else 8192, 77 + mode)
    say("quantize ties", x.shape, "mode", mode)
    _, c, m, e, s = gpu_quant(qg, x, mode)
    oc, om, oe, os_ = oracle.quantize(x, mode)
    assert np.array_equal(m, om) and np.array_equal(e, oe)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)
    f = gen.q4k_fields(64, 1024, 5)
    M = Mat(qg, f)
    for r in range(0, x.shape[0], 97):
        out, fc, fm, fe, fs = _fused(qg, M, x[r:r + 1], mode)
        assert np.array_equal(fc, oc[r:r + 1]) and np.array_equal(fm, om[r:r + 1]) and np.array_equal(fe, oe[r:r + 1])
        assert first_mismatch(out, oracle.gemv(f, oc[r:r + 1], om[r:r + 1], oe[r:r + 1], mode)) is None, r


def test_quantize_infinity_raises_the_flag(qg):
    x = gen.act_normal(2, 1024, 4)
    x[1, 600] = np.inf
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    for mode in (0, 1):
        flag.zero_()
        a = qg.quantize_act(dev(x), mode, err_flag=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1
        with pytest.raises(qg.QGError) as ei:
            qg.check(flag)
        assert ei.value.status == qg.E_NONFINITE
        oc, om, oe, os_ = oracle.quantize(x, mode, check=False)
        m, e = a.scale_fields()
        assert np.array_equal(a.codes.cpu().numpy(), oc) and np.array_equal(m, om) and np.array_equal(e, oe)
    flag.zero_()
    qg.quantize_act(dev(gen.act_normal(1, 1024, 5)), 0, err_flag=flag)
    qg.check(flag)
    assert int(flag.item()) == 0


# --- GEMV on assorted shapes ----------------------------------------------------------------

def _adversarial_fields(fmt, rows, cols, seed):
    if fmt == "q4k":
        f = gen.q4k_fields(rows, cols, seed)
        keys = ("d", "dmin")
    else:
        f = gen.q6k_fields(rows, cols, seed)
        keys = ("d",)
    g = np.random.Generator(np.random.PCG64(seed + 99))
    choices = np.array([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF, 0x2E66], np.uint16)
    for k in keys:
        pick = g.random(f[k].shape) < 0.05
        f[k][pick] = g.choice(choices, size=int(pick.sum()))
    return f


SHAPES = [(1, 256), (3, 768), (63, 1024), (65, 1280), (257, 4096), (9, 14336), (130, 3072), (2, 32768)]


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemv_shapes(qg, fmt, mode):
    for rows, cols in SHAPES:
        say("gemv", fmt, "mode", mode, "shape", rows, cols)
        f = _adversarial_fields(fmt, rows, cols, rows * 131 + cols)
        M = Mat(qg, f)
        x = gen.act_outliers(1, cols, rows + cols)
        if mode == 1:
            x, _ = gen.act_sub32(1, cols, rows + cols)
        act, c, m, e, _ = gpu_quant(qg, x, mode)
        out = run_gemv(qg, M, act)
        want = oracle.gemv(f, c, m, e, mode)
        assert first_mismatch(out, want) is None, (rows, cols, first_mismatch(out, want))


def test_gemv_tiny_workload(qg):
    f, x = gen.tiny_q4k()
    M = Mat(qg, f)
    act, c, m, e, _ = gpu_quant(qg, x, 0)
    out = run_gemv(qg, M, act)
    want = oracle.gemv(f, c, m, e, 0)
    assert first_mismatch(out, want) is None
    assert np.isfinite(want).all() and np.abs(want).max() > 0


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_block_sums_exact(qg, fmt):
    for rows, cols in [(5, 768), (64, 4096)]:
        f = _adversarial_fields(fmt, rows, cols, 7 + rows)
        M = Mat(qg, f)
        x = gen.act_outliers(1, cols, 3 + rows)
        act, c, _, _, _ = gpu_quant(qg, x, 0)
        per = 32 if fmt == "q4k" else 16
        cs = torch.empty((rows, cols // per), dtype=torch.int32, device=DEV)
        os_ = torch.empty((rows, cols // 32), dtype=torch.int32, device=DEV) if fmt == "q4k" else None
        qg.qg_block_sums(M.fmt, rows, cols, M.img, act.codes, cs, os_)
        if fmt == "q4k":
            oC, oO = oracle.sub_sums(f, c[0])
            assert np.array_equal(cs.cpu().numpy(), oC) and np.array_equal(os_.cpu().numpy(), oO)
        else:
            assert np.array_equal(cs.cpu().numpy(), oracle.sub_sums(f, c[0]))


def test_edge_pieces(qg):
    """Pieces that flush at 2^-126, overflow to inf, and inf - inf rows (canonical NaN)."""
    f = gen.q4k_fields(6, 512, 1)
    f["d"][:] = 0x0001
    f["dmin"][:] = 0
    f["d"][2:4] = 0x7BFF
    f["d"][3, 1] = 0xFBFF
    M = Mat(qg, f)
    for scale in (2.0 ** -100, 2.0 ** -60, 3.0e38):
        x = np.full((1, 512), np.float32(scale), np.float32)
        x[0, ::3] *= -1
        act, c, m, e, _ = gpu_quant(qg, x, 0)
        out = run_gemv(qg, M, act)
        want = oracle.gemv(f, c, m, e, 0)
        assert first_mismatch(out, want) is None, scale
    assert (bits(out)[3] == 0x7FC00000) or np.isinf(want[3])


def test_sub32_window_engaged(qg):
    """Sub32 groups whose 32-blocks lie 2^+-120 apart engage the SUM_WINDOW floor (value not
    printed by the pages; reading 64 places): GPU and oracle take the same reading."""
    g = np.random.Generator(np.random.PCG64(17))
    for fmt in ("q4k", "q6k"):
        f = _adversarial_fields(fmt, 40, 1024, 23)
        M = Mat(qg, f)
        x = g.standard_normal((1, 1024)).astype(np.float32)
        k = g.integers(-120, 101, 32)
        x = (x.reshape(32, 32) * np.exp2(k)[:, None]).astype(np.float32).reshape(1, 1024)
        act, c, m, e, _ = gpu_quant(qg, x, 1)
        out = run_gemv(qg, M, act)
        want = oracle.gemv(f, c, m, e, 1)
        assert first_mismatch(out, want) is None, fmt


def test_launch_configuration_does_not_change_bits(qg):
    f = _adversarial_fields("q4k", 1000, 4096, 5)
    M = Mat(qg, f)
    act, c, m, e, _ = gpu_quant(qg, gen.act_outliers(1, 4096, 8), 0)
    ref = bits(run_gemv(qg, M, act))
    try:
        for w in (4, 8, 16):
            qg.qg_set_tuning(qg.TUNE_WAVES_PER_WG, w)
            say("waves per workgroup", w)
            assert np.array_equal(bits(run_gemv(qg, M, act)), ref), w
    finally:
        qg.qg_set_tuning(qg.TUNE_WAVES_PER_WG, 0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty(1000, dtype=torch.float32, device=DEV)
        qg.qg_gemv_q(M.fmt, 0, 1000, 4096, M.img, act.codes, act.scales, act.csums, out, stream=s)
    s.synchronize()
    assert np.array_equal(bits(out), ref)
    assert np.array_equal(ref, bits(oracle.gemv(f, c, m, e, 0)))


def test_binding_refuses_short_buffers(qg):
    M = Mat(qg, gen.q4k_fields(8, 512, 1))
    act, _, _, _, _ = gpu_quant(qg, gen.act_normal(1, 512, 2), 0)
    # 8 rows fill one 64-row group; 65 rows would need two
    with pytest.raises(qg.QGError):
        qg.qg_gemv_q(M.fmt, 0, 65, 512, M.img, act.codes, act.scales, act.csums,
                     torch.empty(65, dtype=torch.float32, device=DEV))
    with pytest.raises(qg.QGError):
        qg.qg_gemv_q(M.fmt, 0, 8, 512, M.img, act.codes, act.scales, act.csums,
                     torch.empty(4, dtype=torch.float32, device=DEV))


# --- the named workloads at full size ------------------------------------------------------

@pytest.fixture(scope="module")
def llama(qg):
    say("packing the 4096x4096 and 14336x4096 Q4_K-style matrices")
    return {k: Mat(qg, gen.llama_q4k(k)) for k in ("attn", "ffn")}


def test_decode_workload_every_row_all_1000_reps(qg, llama):
    """Both Llama-8B-shaped matrices, 1000 repetitions with fresh activations each, every row
    of every repetition against the oracle: the benchmark's one-launch step
    (qg_quantize_gemv) and the two-launch path (qg_quantize_act, then qg_gemv_q); the
    quantized rows of both paths (codes, scales and code sums) byte for byte too."""
    reps = 1000
    xs = np.concatenate([gen.decode_act(k) for k in range(reps)])
    oc, om, oe, osum = oracle.quantize(xs, 0)
    xd = dev(xs)
    for name, M in llama.items():
        say("decode workload", name, M.rows, "x", M.cols, "reps", reps)
        want = oracle.gemm(M.f, oc, om, oe, 0).reshape(reps, M.rows)
        one = torch.empty((reps, M.rows), dtype=torch.float32, device=DEV)
        two = torch.empty((reps, M.rows), dtype=torch.float32, device=DEV)
        a1 = qg.alloc_act(reps, M.cols, 0)
        a2 = qg.alloc_act(reps, M.cols, 0)
        for k in range(reps):
            ak1 = qg.Act(a1.codes[k:k + 1], a1.scales[k:k + 1], a1.csums[k:k + 1], 0)
            ak2 = qg.Act(a2.codes[k:k + 1], a2.scales[k:k + 1], a2.csums[k:k + 1], 0)
            qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, xd[k], 0, act=ak1, out=one[k])
            qg.quantize_act(xd[k:k + 1], 0, out=ak2)
            run_gemv(qg, M, ak2, out=two[k])
        torch.cuda.synchronize()
        for a in (a1, a2):
            m, e = a.scale_fields()
            assert np.array_equal(a.codes.cpu().numpy(), oc), name
            assert np.array_equal(a.csums.cpu().numpy(), osum), name
            assert np.array_equal(m.astype(np.int64), om.astype(np.int64)), name
            assert np.array_equal(e.astype(np.int64), oe.astype(np.int64)), name
        assert first_mismatch(one, want) is None, ("one launch", name)
        assert first_mismatch(two, want) is None, ("two launches", name)
        del one, two, a1, a2


@pytest.mark.parametrize("quarter", [1, 2])
def test_gemv_row_group_split_both_ways(qg, llama, quarter):
    """The one-column Q4_K PerBlock GEMV with 16-row workgroups (1) and with 64-row ones (2),
    forced, one launch and two: every shape of at most 16 blocks per row, the 14336-row matrix
    for 20 repetitions and a three-matrix launch, all against the oracle."""
    try:
        qg.qg_set_tuning(qg.TUNE_GEMV_QUARTER, quarter)
        for rows, cols in [s for s in SHAPES if s[1] <= 4096] + [(4096, 4096), (4100, 2048), (8191, 512)]:
            say("row-group split", quarter, "shape", rows, cols)
            f = _adversarial_fields("q4k", rows, cols, rows * 7 + cols + quarter)
            M = Mat(qg, f)
            x = gen.act_outliers(1, cols, rows + 5 * cols)
            out, c, m, e, s = _fused(qg, M, x, 0)
            oc, om, oe, os_ = oracle.quantize(x, 0)
            assert np.array_equal(c, oc) and np.array_equal(m, om) and np.array_equal(e, oe)
            assert np.array_equal(s, os_)
            want = oracle.gemv(f, oc, om, oe, 0)
            assert first_mismatch(out, want) is None, (rows, cols, first_mismatch(out, want))
            act, _, _, _, _ = gpu_quant(qg, x, 0)
            assert first_mismatch(run_gemv(qg, M, act), want) is None, (rows, cols)
        M = llama["ffn"]
        reps = 20
        xs = np.concatenate([gen.decode_act(2000 + k) for k in range(reps)])
        oc, om, oe, _ = oracle.quantize(xs, 0)
        want = oracle.gemm(M.f, oc, om, oe, 0).reshape(reps, M.rows)
        xd = dev(xs)
        one = torch.empty((reps, M.rows), dtype=torch.float32, device=DEV)
        for k in range(reps):
            qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, xd[k], 0, out=one[k])
        say("row-group split", quarter, "14336 x 4096,", reps, "reps")
        assert first_mismatch(one, want) is None
        shapes = [70, 0, 4096]
        mats = [Mat(qg, _adversarial_fields("q4k", max(r, 1), 1024, 90 + r)) for r in shapes]
        x = gen.act_outliers(1, 1024, 91)
        act = qg.alloc_act(1, 1024, 0)
        outs = [torch.full((max(r, 1),), -7.0, dtype=torch.float32, device=DEV) for r in shapes]
        qg.qg_quantize_gemv_multi(qg.Q4K, 0, shapes, 1024, [M.img for M in mats], dev(x.reshape(-1)), act.codes,
                                  act.scales, act.csums, None, outs)
        oc, om, oe, _ = oracle.quantize(x, 0)
        for r, M, o in zip(shapes, mats, outs):
            if r == 0:
                assert float(o[0].item()) == -7.0
            else:
                assert first_mismatch(o, oracle.gemv(M.f, oc, om, oe, 0)) is None, r
    finally:
        qg.qg_set_tuning(qg.TUNE_GEMV_QUARTER, 0)


def test_output_projection_q6k_logits(qg):
    say("generating the 128256x4096 Q6_K-style matrix")
    f, x = gen.output_q6k()
    M = Mat(qg, f)
    act, c, m, e, _ = gpu_quant(qg, x, 0)
    out = run_gemv(qg, M, act)
    say("oracle over 128256 rows")
    want = oracle.gemv(f, c, m, e, 0)
    assert first_mismatch(out, want) is None
    del M
    torch.cuda.empty_cache()


def test_sub32_workload_every_row_100_reps(qg, llama):
    """Sub32 on the 14336x4096 matrix, 100 repetitions (the exponents of each row span
    -12..4), every row of every repetition against the oracle, for the one-launch step and
    the two-launch path."""
    M = llama["ffn"]
    reps = 100
    xs, ts = zip(*(gen.sub32_act(k) for k in range(reps)))
    xs = np.concatenate(xs)
    oc, om, oe, osum = oracle.quantize(xs, 1)
    assert np.array_equal(oe.astype(np.int32), np.concatenate(ts).astype(np.int32))
    say("oracle: Sub32 over", M.rows, "rows x", reps, "reps")
    want = oracle.gemm(M.f, oc, om, oe, 1).reshape(reps, M.rows)
    xd = dev(xs)
    one = torch.empty((reps, M.rows), dtype=torch.float32, device=DEV)
    two = torch.empty((reps, M.rows), dtype=torch.float32, device=DEV)
    a1 = qg.alloc_act(reps, M.cols, 1)
    a2 = qg.alloc_act(reps, M.cols, 1)
    for k in range(reps):
        ak1 = qg.Act(a1.codes[k:k + 1], a1.scales[k:k + 1], a1.csums[k:k + 1], 1)
        ak2 = qg.Act(a2.codes[k:k + 1], a2.scales[k:k + 1], a2.csums[k:k + 1], 1)
        qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, xd[k], 1, act=ak1, out=one[k])
        qg.quantize_act(xd[k:k + 1], 1, out=ak2)
        run_gemv(qg, M, ak2, out=two[k])
    torch.cuda.synchronize()
    for a in (a1, a2):
        m, e = a.scale_fields()
        assert np.array_equal(a.codes.cpu().numpy(), oc)
        assert np.array_equal(a.csums.cpu().numpy(), osum)
        assert np.array_equal(m.astype(np.int64), om.astype(np.int64))
        assert np.array_equal(e.astype(np.int64), oe.astype(np.int64))
    assert first_mismatch(one, want) is None, "one launch"
    assert first_mismatch(two, want) is None, "two launches"


@pytest.mark.parametrize("n", [2, 8, 64])
def test_batched_columns(qg, llama, n):
    """The batched workload on both matrices: every (r, c) against the oracle, and columns 0
    and n-1 bit for bit equal to the GEMV of that column."""
    xs = gen.batch_act(n)
    for name, M in llama.items():
        say("gemm", name, "n", n)
        act, c, m, e, _ = gpu_quant(qg, xs, 0)
        out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
        want = oracle.gemm(M.f, c, m, e, 0).reshape(n, M.rows)
        assert first_mismatch(out, want) is None, (name, n)
        one = qg.alloc_act(1, M.cols, 0)
        for k in (0, n - 1):
            one.codes.copy_(act.codes[k:k + 1])
            one.scales.copy_(act.scales[k:k + 1])
            one.csums.copy_(act.csums[k:k + 1])
            assert np.array_equal(bits(run_gemv(qg, M, one)), bits(out[k]))


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("mode", [0, 1])
def test_several_columns_one_column_machinery(qg, fmt, mode):
    """Several activation columns below the matrix-core threshold (2 to 13 columns, batches of
    2, 4 and 8 per workgroup, ragged rows, 1 to 16 blocks per row): the oracle's bits, and the
    same bits as the kernel that stages the columns in LDS."""
    try:
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 65536)
        for rows, cols, n in ((70, 4096, 2), (130, 3072, 3), (64, 1024, 4), (9, 256, 5), (200, 4096, 8),
                              (65, 2048, 9), (33, 4096, 13)):
            say("several columns", fmt, "mode", mode, "shape", rows, cols, "n", n)
            f = _adversarial_fields(fmt, rows, cols, rows + 7 * cols + n)
            M = Mat(qg, f)
            xs = gen.act_outliers(n, cols, rows + n) if mode == 0 else gen.act_sub32(n, cols, rows + n)[0]
            act, c, m, e, _ = gpu_quant(qg, xs, mode)
            qg.qg_set_tuning(qg.TUNE_COLS_KERNEL, 0)
            out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
            want = oracle.gemm(f, c, m, e, mode).reshape(n, rows)
            assert first_mismatch(out, want) is None, (rows, cols, n, first_mismatch(out, want))
            qg.qg_set_tuning(qg.TUNE_COLS_KERNEL, 1)
            staged = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
            assert np.array_equal(bits(staged), bits(out)), (rows, cols, n)
    finally:
        qg.qg_set_tuning(qg.TUNE_COLS_KERNEL, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 0)


# --- batched columns on the int8 matrix cores -----------------------------------------------

@pytest.mark.parametrize("ncol", [3, 8, 16, 17, 33, 64, 100])
def test_matrix_core_gemm_matches_oracle(qg, ncol):
    """Q4_K PerBlock batches run on v_mfma_i32_16x16x64_i8 (by default from 2 or 5 columns; here
    forced for every count); every (row, column) must carry the oracle's bits in every form,
    across column-tile and row-tile (for the column-resident form: waves per workgroup)
    settings, ragged rows and columns, and block scales that take both the near-exponent and
    the general combine."""
    f = _adversarial_fields("q4k", 130, 1280, 900 + ncol)
    M = Mat(qg, f)
    xs = gen.act_outliers(ncol, 1280, 901 + ncol)
    xs[min(3, ncol - 1), 256:512] = 0.0                         # an all-zero activation block
    act, c, m, e, _ = gpu_quant(qg, xs, 0)
    want = oracle.gemm(f, c, m, e, 0).reshape(ncol, 130)
    try:
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 1)                # matrix cores for any column count
        # derived, staged (at most 16 columns), shared operands, split, column-resident
        for form in (0, 1, 2, 3, 4):
            if form == 1 and ncol > 16:
                continue
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, form)
            for ct in ((0, 1, 2) if form == 4 else (0, 1, 2, 4)):   # 0: derived from the column count
                qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, ct)
                for rt in ((0, 1, 2, 4) if form in (1, 3, 4) and ct == 0 else (0,)):
                    qg.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, rt)
                    for tab in ((0, 1) if form == 2 else (0,)):     # shared operands: scale tables or not
                        qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, tab)
                        say("matrix-core gemm", ncol, "form", form, "column tiles", ct, "row tiles", rt, "tables off", tab)
                        out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
                        assert first_mismatch(out, want) is None, (ncol, form, ct, rt, tab, first_mismatch(out, want))
                    qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, 0)
                qg.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 65536)          # force the vector-ALU kernel
        out_valu = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
        assert first_mismatch(out_valu, want) is None
    finally:
        qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, 0)
        qg.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 0)


@pytest.mark.parametrize("ncol", [64, 100])
def test_matrix_core_gemm_16_blocks(qg, ncol):
    """Rows of 16 blocks through the shared-operand kernel, whose block loop is unrolled when
    compiled, and the column-resident kernel, compiled for 16 blocks too: ragged rows and
    columns, block scales that take both the near-exponent and the general combine, and (in the
    second run) a row of tiny activations, which makes its batch of columns take the flushed
    combine; with and without the scale tables."""
    rows, cols = 130, 4096
    f = _adversarial_fields("q4k", rows, cols, 4400 + ncol)
    for r in (1, 66):
        _subnormal_partial_q4k(f, r)
    M = Mat(qg, f)
    for tiny in (False, True):
        xs = gen.act_outliers(ncol, cols, 4401 + ncol)
        if tiny:
            xs[ncol - 3, :] = np.float32(2.0 ** -112)
        act, c, m, e, _ = gpu_quant(qg, xs, 0)
        want = oracle.gemm(f, c, m, e, 0).reshape(ncol, rows)
        try:
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 2)      # the shared-operand form on these 130 rows too
            for tab in (0, 1):
                qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, tab)
                say("matrix-core gemm, 16 blocks", ncol, "tiny row", tiny, "tables off", tab)
                out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
                assert first_mismatch(out, want) is None, (ncol, tiny, tab, first_mismatch(out, want))
            qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, 0)
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 4)      # the column-resident form, one or two column tiles
            for ct in (0, 1, 2):
                qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, ct)
                say("matrix-core gemm, 16 blocks, column-resident", ncol, "tiny row", tiny, "column tiles", ct)
                out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
                assert first_mismatch(out, want) is None, (ncol, tiny, "resident", ct, first_mismatch(out, want))
        finally:
            qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, 0)
            qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, 0)
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 0)


@pytest.mark.parametrize("cols", [6144, 8192, 12288])
def test_matrix_core_gemm_long_rows(qg, cols):
    """Rows of 24, 32 and 48 blocks through the shared-operand kernel: at 24 blocks the scale
    tables fit in LDS beside the operand stages (the block loop runs with three prefetch
    buffers), at 32 and 48 they do not and each block loads its own scales; 40 columns, ragged
    rows, far block-scale pairs and one row of tiny activations; and the form the dispatch
    derives for these 70 rows (split); the column-resident form at 24 and 32 blocks."""
    rows, ncol = 70, 40
    f = _adversarial_fields("q4k", rows, cols, 5100 + cols // 256)
    _subnormal_partial_q4k(f, 3)
    M = Mat(qg, f)
    xs = gen.act_outliers(ncol, cols, 5101 + cols // 256)
    xs[7, :] = np.float32(2.0 ** -112)
    act, c, m, e, _ = gpu_quant(qg, xs, 0)
    want = oracle.gemm(f, c, m, e, 0).reshape(ncol, rows)
    try:
        for form in ((2, 0, 4) if cols <= 8192 else (2, 0)):   # column-resident: one column tile to 32 blocks
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, form)
            say("matrix-core gemm, long rows", cols, "form", form)
            out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
            assert first_mismatch(out, want) is None, (cols, form, first_mismatch(out, want))
    finally:
        qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 0)


@pytest.mark.parametrize("cols,ncol", [(1280, 5), (1280, 64), (3072, 16), (4096, 1), (4096, 2), (4096, 8), (4096, 33),
                                       (4096, 100), (6144, 40), (8192, 17)])
def test_split_gemm_matches_oracle(qg, cols, ncol):
    """The split and staged matrix-core GEMMs (every wave one block, every load issued at once)
    in every row-tile x column-tile shape: ragged rows (three 64-row groups, the last partial) and
    columns, rows of 5 blocks (one partial round of waves), 16 (one round), 24 and 32 (two
    rounds), block scales that take both the near-exponent and the general combine, a row whose
    partial sum passes through the subnormal range, and a column of tiny activations."""
    rows = 130
    f = _adversarial_fields("q4k", rows, cols, 6100 + cols // 256 + ncol)
    _subnormal_partial_q4k(f, 65)
    M = Mat(qg, f)
    xs = gen.act_outliers(ncol, cols, 6101 + ncol)
    xs[ncol - 1, :] = np.float32(2.0 ** -112)
    if ncol > 3:
        xs[2, 256:512] = 0.0                                    # an all-zero activation block
    act, c, m, e, _ = gpu_quant(qg, xs, 0)
    want = oracle.gemm(f, c, m, e, 0).reshape(ncol, rows)
    try:
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 1)
        qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 3)
        for rtt in (0, 1, 2, 4):
            for ct in (0, 1, 2, 4):
                if rtt * ct > 8:
                    continue
                qg.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, rtt)
                qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, ct)
                say("split gemm", rows, "x", cols, "n", ncol, "row tiles", rtt, "column tiles", ct)
                out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
                assert first_mismatch(out, want) is None, (rtt, ct, first_mismatch(out, want))
        qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, 0)
        if cols <= 4096 and ncol <= 16:
            # the staged form (at most 16 columns staged in LDS), every row-tile count
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 1)
            for rtt in (0, 1, 2, 4):
                qg.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, rtt)
                say("staged gemm", rows, "x", cols, "n", ncol, "row tiles", rtt)
                out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
                assert first_mismatch(out, want) is None, ("staged", rtt, first_mismatch(out, want))
    finally:
        qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 0)
        qg.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 0)


def _subnormal_partial_q4k(f, r):
    """Row r of a Q4_K-style matrix (at least 3 blocks) whose PerBlock pieces, under an
    activation block of all 2^-112 (codes 126, scale 130 * 2^-126), are 16380*k*2^-142 with
    k = 800, -801, 8 in blocks 0, 1, 2: normal, but the first two cancel to a subnormal
    partial sum, which the flush turns into -0 before block 2 is added."""
    f["q"][r, :768] = 1
    f["q"][r, 256:512] = 0
    f["sc"][r, :24] = 1
    f["sc"][r, 8:16] = 0
    f["mn"][r, :24] = 0
    f["mn"][r, 8:16] = 1
    f["d"][r, :3] = [800, 0, 8]                     # binary16 subnormals k * 2^-24
    f["dmin"][r, :3] = [0, 801, 0]


def _negative_zero_tail_q4k(f, r):
    """Row r as in _subnormal_partial_q4k, but block 2's piece is -1 * 16380 * 2^-142: a negative
    subnormal, flushed to -0 and added to the partial sum that is already -0, which stays -0 (an
    add of +0 there would give +0)."""
    _subnormal_partial_q4k(f, r)
    f["q"][r, 512:768] = 0
    f["sc"][r, 16:24] = 0
    f["mn"][r, 16:24] = 1
    f["d"][r, 2] = 0
    f["dmin"][r, 2] = 1


@pytest.mark.parametrize("ncol,tiny", [(16, (3, 15)), (64, (0, 63)), (100, (70,))])
def test_subnormal_partial_sums_gemv_and_gemm(qg, ncol, tiny):
    """Rows whose running sum passes through the subnormal range (one of them then adds a piece
    that is itself flushed to -0, keeping the -0), through the GEMV and every GEMM form: all
    must give the oracle's bits, which differ from unflushed adds.  With 100
    columns the tiny activation row lies in the second batch of 64 only, so the first batch
    takes the matrix-core kernel's plain-add combine and the second its flushed one."""
    rows, cols = 70, 768
    f = gen.q4k_fields(rows, cols, 77)
    for r in (0, 5, 69):
        _subnormal_partial_q4k(f, r)
    _negative_zero_tail_q4k(f, 33)
    M = Mat(qg, f)
    xs = gen.act_outliers(ncol, cols, 78)
    for t in tiny:
        xs[t, :] = np.float32(2.0 ** -112)
    act, c, m, e, _ = gpu_quant(qg, xs, 0)
    t0 = tiny[0]
    assert int(c[t0, 0]) == 126 and int(m[t0, 0]) == 130 and int(e[t0, 0]) == -126
    want = oracle.gemm(f, c, m, e, 0).reshape(ncol, rows)
    # unflushed adds of the three pieces (exact binary32 values) give other bits
    unit = np.float32(16380.0 * 2.0 ** -142)
    plain = np.float32(np.float32(np.float32(0) + np.float32(800 * unit)) + np.float32(-801 * unit))
    plain = np.float32(plain + np.float32(8 * unit))
    assert plain.view(np.uint32) != bits(want[t0])[0]
    assert bits(want[t0])[0] == np.float32(8 * unit).view(np.uint32)
    assert bits(want[t0])[33] == 0x80000000                     # -0 kept through a -0 piece
    one = qg.alloc_act(1, cols, 0)
    one.codes.copy_(act.codes[t0:t0 + 1]); one.scales.copy_(act.scales[t0:t0 + 1]); one.csums.copy_(act.csums[t0:t0 + 1])
    assert first_mismatch(run_gemv(qg, M, one), want[t0]) is None
    try:
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 1)
        # staged, shared (tables or not), split, column-resident
        for form, tab in ((1, 0), (2, 0), (2, 1), (3, 0), (4, 0)):
            if form == 1 and ncol > 16:
                continue
            qg.qg_set_tuning(qg.TUNE_MFMA_FORM, form)
            qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, tab)
            say("subnormal partial sums, gemm form", form, "tables off", tab, "columns", ncol)
            out = qg.gemm(M.fmt, M.rows, M.cols, M.img, act)
            assert first_mismatch(out, want) is None, (form, tab, first_mismatch(out, want))
    finally:
        qg.qg_set_tuning(qg.TUNE_MFMA_FORM, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_TABLES, 0)
        qg.qg_set_tuning(qg.TUNE_MFMA_MIN_COLS, 0)


@pytest.mark.parametrize("span", [15, 16, 17, 20])
def test_sub32_exponent_spans(qg, span):
    """Sub32 groups whose activation exponents span 15 to 20 places (the factored exact sum
    takes up to 16, wider groups take the pairwise one): the quantized-row GEMV and the
    one-launch step give the oracle's bits, on near and far block-scale pairs."""
    rows, cols = 200, 4096
    f = _adversarial_fields("q4k", rows, cols, 300 + span)
    M = Mat(qg, f)
    x, t = gen.act_sub32(2, cols, 310 + span, e_lo=-12, e_hi=-12 + span)
    g8 = t.reshape(2, -1, 8)
    assert (g8.max(axis=2) - g8.min(axis=2)).max() == span
    say("sub32 exponent span", span)
    for k in range(2):
        c, m, e, _ = oracle.quantize(x[k:k + 1], 1)
        assert np.array_equal(e.reshape(-1), t[k])
        want = oracle.gemv(f, c, m, e, 1)
        act, gc, gm, ge, _ = gpu_quant(qg, x[k:k + 1], 1)
        assert np.array_equal(gc, c) and np.array_equal(ge, e)
        assert first_mismatch(run_gemv(qg, M, act), want) is None, (span, k)
        out, *_ = _fused(qg, M, x[k:k + 1], 1)
        assert first_mismatch(out, want) is None, (span, k)


def test_sub32_pieces_on_binary32_boundaries(qg):
    """Sub32 group values on a binary32 rounding boundary and one binary64 step either side of
    it (where a binary64 rounding taken first lands on the boundary), and group values below the
    binary32 normal range: two columns at once, the quantized-row GEMV and the one-launch step
    give the oracle's bits."""
    f, x = gen.sub32_boundary_rows()
    M = Mat(qg, f)
    c, m, e, _ = oracle.quantize(x, 1)
    want = oracle.gemm(f, c, m, e, 1).reshape(2, f["rows"])
    say("sub32 boundary rows")
    act, gc, gm, ge, _ = gpu_quant(qg, x, 1)
    assert np.array_equal(gc, c) and np.array_equal(ge, e)
    assert first_mismatch(qg.gemm(M.fmt, M.rows, M.cols, M.img, act), want) is None
    for k in range(2):
        one, *_ = gpu_quant(qg, x[k:k + 1], 1)
        assert first_mismatch(run_gemv(qg, M, one), want[k]) is None, k
        out, *_ = _fused(qg, M, x[k:k + 1], 1)
        assert first_mismatch(out, want[k]) is None, k


@pytest.mark.parametrize("cols", [4096, 8192])
def test_subnormal_partial_sums_wide_rows(qg, cols):
    """The same cancelling rows at 16 blocks (one wave per block) and 32 blocks (two tiles
    per wave), their later blocks zero: the quantized-row GEMV and the one-launch step give
    the oracle's bits, 8 units where unflushed adds would give 7."""
    rows = 70
    f = gen.q4k_fields(rows, cols, 79)
    for r in (0, 5, 69):
        _subnormal_partial_q4k(f, r)
        f["q"][r, 768:] = 0
        f["mn"][r, 24:] = 0
    M = Mat(qg, f)
    x = np.full((1, cols), np.float32(2.0 ** -112), np.float32)
    c, m, e, _ = oracle.quantize(x, 0)
    want = oracle.gemv(f, c, m, e, 0)
    unit = np.float32(16380.0 * 2.0 ** -142)
    assert bits(want)[0] == np.float32(8 * unit).view(np.uint32)
    act, gc, gm, ge, _ = gpu_quant(qg, x, 0)
    assert np.array_equal(gc, c)
    say("subnormal partial sums, wide rows", cols)
    assert first_mismatch(run_gemv(qg, M, act), want) is None
    out, *_ = _fused(qg, M, x, 0)
    assert first_mismatch(out, want) is None


# --- quantize + GEMV in one launch ------------------------------------------------------------

def _fused(qg, M, x: np.ndarray, mode: int, err_flag=None):
    out, act = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, dev(x.reshape(-1)), mode, err_flag=err_flag)
    m, e = act.scale_fields()
    return out, act.codes.cpu().numpy(), m, e, act.csums.cpu().numpy()


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("mode", [0, 1])
def test_fused_quantize_gemv_shapes(qg, fmt, mode):
    """qg_quantize_gemv against the oracle's quantize then dot: the output row and the
    quantized row it writes, on every shape (one launch up to 64 blocks per row, the
    two-launch form above)."""
    for rows, cols in SHAPES + [(70, 16384), (3, 16640)]:
        say("fused", fmt, "mode", mode, "shape", rows, cols)
        f = _adversarial_fields(fmt, rows, cols, rows * 17 + cols)
        M = Mat(qg, f)
        x = gen.act_outliers(1, cols, rows + 3 * cols)
        if mode == 1:
            x, _ = gen.act_sub32(1, cols, rows + 3 * cols)
        out, c, m, e, s = _fused(qg, M, x, mode)
        oc, om, oe, os_ = oracle.quantize(x, mode)
        assert np.array_equal(c, oc) and np.array_equal(m, om) and np.array_equal(e, oe) and np.array_equal(s, os_)
        want = oracle.gemv(f, oc, om, oe, mode)
        assert first_mismatch(out, want) is None, (rows, cols, first_mismatch(out, want))


def test_fused_launch_configuration_and_streams(qg):
    f = _adversarial_fields("q4k", 1000, 4096, 15)
    M = Mat(qg, f)
    x = gen.act_outliers(1, 4096, 18)
    ref, c, m, e, _ = _fused(qg, M, x, 0)
    ref = bits(ref)
    assert np.array_equal(ref, bits(oracle.gemv(f, c, m, e, 0)))
    try:
        for w in (4, 8, 16):
            qg.qg_set_tuning(qg.TUNE_WAVES_PER_WG, w)
            say("fused, waves per workgroup", w)
            assert np.array_equal(bits(_fused(qg, M, x, 0)[0]), ref), w
    finally:
        qg.qg_set_tuning(qg.TUNE_WAVES_PER_WG, 0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, _ = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, dev(x.reshape(-1)), 0, stream=s)
    s.synchronize()
    assert np.array_equal(bits(out), ref)


def test_fused_infinity_flag_and_zero_rows(qg):
    f = gen.q4k_fields(100, 1024, 41)
    M = Mat(qg, f)
    x = gen.act_normal(1, 1024, 42)
    x[0, 300] = -np.inf
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    for mode in (0, 1):
        flag.zero_()
        out, c, m, e, _ = _fused(qg, M, x, mode, err_flag=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1
        oc, om, oe, _ = oracle.quantize(x, mode, check=False)
        assert np.array_equal(c, oc) and np.array_equal(m, om) and np.array_equal(e, oe)
        assert first_mismatch(out, oracle.gemv(f, oc, om, oe, mode)) is None
    # rows = 0: the call only quantizes
    act = qg.alloc_act(1, 1024, 0)
    xg = gen.act_normal(1, 1024, 43)
    qg.qg_quantize_gemv(M.fmt, 0, 0, 1024, None, dev(xg.reshape(-1)), act.codes, act.scales, act.csums, None, None)
    assert np.array_equal(act.codes.cpu().numpy(), oracle.quantize(xg, 0)[0])


def test_stream_read_diagnostic(qg):
    """The measured-ceiling read: zeros never meet a nonzero magic; a 16-byte piece at the
    right place does (lane 0 of the first wave reads bytes 0..15 of every chunk it owns)."""
    buf = torch.zeros(9 * 1024 * 3 + 512, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    qg.qg_stream_read(buf, buf.numel(), 0x1234, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1
    buf[0:4] = torch.tensor([0x34, 0x12, 0, 0], dtype=torch.uint8, device=DEV)
    qg.qg_stream_read(buf, buf.numel(), 0x1234, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0x1234


@pytest.mark.parametrize("w,k,wgs,flags", [(16, 9, 0, 0), (4, 1, 0, 1), (8, 4, 3, 0), (1, 16, 2, 1)])
def test_stream_read_shape_diagnostic(qg, w, k, wgs, flags):
    """The launch-shape read: every shape reads every chunk (a magic planted in the last
    chunk's first word, the rest zero, reaches the sink through the lane that reads it), and a
    shape outside the documented sets is refused."""
    nchunks = 9 * 7 + 5
    buf = torch.zeros(nchunks * 1024 + 100, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    qg.qg_stream_read_shape(buf, buf.numel(), w, k, wgs, flags, 0x1234, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1
    off = (nchunks - 1) * 1024
    buf[off:off + 4] = torch.tensor([0x34, 0x12, 0, 0], dtype=torch.uint8, device=DEV)
    qg.qg_stream_read_shape(buf, buf.numel(), w, k, wgs, flags, 0x1234, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0x1234
    with pytest.raises(qg.QGError):
        qg.qg_stream_read_shape(buf, buf.numel(), w, 3, wgs, flags, 0x1234, sink)


# --- several matrices sharing one activation row ------------------------------------------

@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("mode", [0, 1])
def test_multi_matrix_launch_matches_single_calls(qg, fmt, mode):
    """One launch over matrices of ragged row counts (one of them empty) gives every matrix the
    bits of its own call and of the oracle; the quantized row is the one-matrix call's."""
    cols = 1280
    shapes = [130, 64, 0, 5, 300]
    mats = []
    for k, rows in enumerate(shapes):
        f = _adversarial_fields(fmt, max(rows, 1), cols, 700 + 13 * k)
        if rows == 0:
            mats.append(None)
            continue
        mats.append(Mat(qg, f))
    x = gen.act_outliers(1, cols, 77) if mode == 0 else gen.act_sub32(1, cols, 77)[0]
    xd = dev(x.reshape(-1))
    images = [M.img if M else None for M in mats]
    outs = [torch.full((max(r, 1),), -7.0, dtype=torch.float32, device=DEV) for r in shapes]
    act = qg.alloc_act(1, cols, mode)
    fmt_code = qg.FMT_CODES[fmt]
    qg.qg_quantize_gemv_multi(fmt_code, mode, shapes, cols, images, xd, act.codes, act.scales, act.csums, None, outs)
    oc, om, oe, os_ = oracle.quantize(x, mode)
    m, e = act.scale_fields()
    assert np.array_equal(act.codes.cpu().numpy(), oc) and np.array_equal(m, om) and np.array_equal(e, oe)
    assert np.array_equal(act.csums.cpu().numpy(), os_)
    outs2 = [torch.full((max(r, 1),), -7.0, dtype=torch.float32, device=DEV) for r in shapes]
    qg.qg_gemv_q_multi(fmt_code, mode, shapes, cols, images, act.codes, act.scales, act.csums, outs2)
    for k, M in enumerate(mats):
        if M is None:
            assert float(outs[k][0].item()) == -7.0 and float(outs2[k][0].item()) == -7.0
            continue
        say("multi", fmt, "mode", mode, "matrix", k, M.rows)
        single, _ = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, xd, mode)
        want = oracle.gemv(M.f, oc, om, oe, mode)
        assert np.array_equal(bits(outs[k]), bits(single)), k
        assert np.array_equal(bits(outs2[k]), bits(single)), k
        assert first_mismatch(outs[k], want) is None, k


def test_multi_matrix_gate_up_workload(qg, llama):
    """The decode layer's gate and up projections (two 14336 x 4096 matrices) in one launch."""
    up = llama["ffn"]
    gate = Mat(qg, gen.q4k_fields(14336, 4096, gen.SEED_GATE_W))
    x = gen.decode_act(3)
    xd = dev(x.reshape(-1))
    outs = [torch.empty(14336, dtype=torch.float32, device=DEV) for _ in range(2)]
    act = qg.alloc_act(1, 4096, 0)
    qg.qg_quantize_gemv_multi(qg.Q4K, 0, [14336, 14336], 4096, [gate.img, up.img], xd, act.codes, act.scales,
                              act.csums, None, outs)
    oc, om, oe, _ = oracle.quantize(x, 0)
    for M, o in ((gate, outs[0]), (up, outs[1])):
        assert first_mismatch(o, oracle.gemv(M.f, oc, om, oe, 0)) is None


# --- argmax of the output row --------------------------------------------------------------

def _fused_argmax(qg, M, x: np.ndarray, mode: int):
    key = torch.zeros(1, dtype=torch.int64, device=DEV)
    act = qg.alloc_act(1, M.cols, mode)
    out = torch.empty(M.rows, dtype=torch.float32, device=DEV)
    qg.qg_quantize_gemv_argmax(M.fmt, mode, M.rows, M.cols, M.img, dev(x.reshape(-1)), act.codes, act.scales,
                               act.csums, None, out, key)
    return qg.qg_argmax_index(int(key.item()) & 0xFFFFFFFFFFFFFFFF), out


def test_argmax_of_logits_q6k_output(qg):
    """The 128256-row Q6_K output projection: the fused argmax equals the oracle's argmax of
    the oracle's logits, and the logits are the plain call's bits."""
    f, x = gen.output_q6k()
    M = Mat(qg, f)
    idx, out = _fused_argmax(qg, M, x, 0)
    c, m, e, _ = oracle.quantize(x, 0)
    want = oracle.gemv(f, c, m, e, 0)
    assert first_mismatch(out, want) is None
    assert idx == oracle.argmax(want)
    del M
    torch.cuda.empty_cache()


def test_argmax_ties_nan_and_zeros(qg):
    """Equal maxima in several workgroups (the first wins), NaN rows passed over, and a matrix
    whose every row is NaN (index 0)."""
    cols = 512
    f = gen.q4k_fields(300, cols, 61)
    x = gen.act_normal(1, cols, 62)
    c, m, e, _ = oracle.quantize(x, 0)
    base = oracle.gemv(f, c, m, e, 0)
    top = int(np.argmax(base))
    for r in (7, 100, 299):                                # copies of the top row, above and below it
        for k in ("q", "sc", "mn", "d", "dmin"):
            f[k][r] = f[k][top]
    want = oracle.gemv(f, c, m, e, 0)
    idx, out = _fused_argmax(qg, Mat(qg, f), x, 0)
    assert first_mismatch(out, want) is None
    assert idx == oracle.argmax(want) == min(7, top)
    # rows of inf - inf (canonical NaN) are passed over; all of them NaN gives 0.  With the
    # largest scales and activations every piece overflows: block 0 (codes 15) to +inf, block 1
    # (codes 0, only the offset term) to -inf, so a row is NaN unless its block 1 keeps codes 15.
    g = gen.q4k_fields(130, cols, 63)
    g["d"][:] = 0x7BFF
    g["dmin"][:] = 0x7BFF
    g["sc"][:] = 63
    g["mn"][:] = 63
    g["q"][:, :256] = 15
    g["q"][:, 256:] = 0
    xb = np.full((1, cols), np.float32(3.0e38), np.float32)
    c2, m2, e2, _ = oracle.quantize(xb, 0)
    for finite_rows in ((70, 71), ()):
        h = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in g.items()}
        for r in finite_rows:
            h["q"][r, 256:] = 15
        want2 = oracle.gemv(h, c2, m2, e2, 0)
        assert np.isnan(want2).sum() == h["rows"] - len(finite_rows)
        idx2, out2 = _fused_argmax(qg, Mat(qg, h), xb, 0)
        assert first_mismatch(out2, want2) is None
        assert idx2 == oracle.argmax(want2) == (finite_rows[0] if finite_rows else 0)
