"""GPU parity for the 32-element-block formats (Q8_0- and Q4_0-style), bit for bit against
the oracle: the quantizer's 32-element PerBlock blocks, the GEMV from quantized codes and
the one-launch quantize + GEMV on shapes with ragged row groups and up to 128 blocks per row,
several matrices in one launch, the fused argmax, batched columns, the launch configuration,
and the full-size 14336 x 4096 matrices."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
FMTS = ["q8_0", "q4_0"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qg():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import block_format_gemv_amd as q
    q.qg_set_tuning(q.TUNE_WAVES_PER_WG, 0)
    oracle.set_threads(8)
    return q


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(a) -> np.ndarray:
    a = a.detach().cpu().numpy() if hasattr(a, "detach") else np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).reshape(-1)


def first_mismatch(got, want):
    g, w = bits(got), bits(want)
    bad = np.nonzero(g != w)[0]
    if len(bad) == 0:
        return None
    i = bad[0]
    return f"{len(bad)} mismatches; first at {i}: got {g[i]:08x} want {w[i]:08x}"


def fields(fmt, rows, cols, seed, adversarial=True):
    f = (gen.q8_0_fields if fmt == "q8_0" else gen.q4_0_fields)(rows, cols, seed)
    if adversarial:
        # zero, subnormal, largest and negative binary16 scales on 5% of the blocks, and a few
        # rows of extreme codes
        g = np.random.Generator(np.random.PCG64(seed + 99))
        choices = np.array([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF, 0x2E66], np.uint16)
        pick = g.random(f["d"].shape) < 0.05
        f["d"][pick] = g.choice(choices, size=int(pick.sum()))
        f["q"][0, :] = -128 if fmt == "q8_0" else 0
        if rows > 2:
            f["q"][2, :] = 127 if fmt == "q8_0" else 15
    return f


class Mat:
    def __init__(self, q, f):
        self.f = f
        self.fmt = q.FMT_CODES[f["fmt"]]
        self.rows, self.cols = f["rows"], f["cols"]
        self.img = dev(q.pack(f))


def act_row(cols, seed, mode):
    return gen.act_outliers(1, cols, seed) if mode == 0 else gen.act_sub32(1, cols, seed)[0]


def oracle_act(fmt, x, mode):
    return oracle.quantize(x, mode, block=oracle.act_block(fmt, mode))


SHAPES = [(1, 256), (3, 768), (63, 1024), (65, 1280), (257, 4096), (9, 14336), (130, 3072), (2, 32768)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_blocks_of_32(qg, fmt, mode):
    g = np.random.Generator(np.random.PCG64(21))
    x = gen.act_outliers(3, 2048, 22)
    x[1, :32] = 0                                          # an all-zero 32-element block
    x[1, 40] = np.nan
    x[2] *= np.float32(2.0 ** -120)
    x[0, 64:96] = np.round(g.standard_normal(32) * 8).astype(np.float32) / 8
    say("quantize", fmt, "mode", mode)
    a = qg.quantize_act(dev(x), mode, qg.FMT_CODES[fmt])
    m, e = a.scale_fields()
    oc, om, oe, os_ = oracle_act(fmt, x, mode)
    assert m.shape == (3, 2048 // 32)
    assert np.array_equal(a.codes.cpu().numpy(), oc)
    assert np.array_equal(m, om) and np.array_equal(e, oe)
    assert np.array_equal(a.csums.cpu().numpy(), os_)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [0, 1])
def test_gemv_and_fused_shapes(qg, fmt, mode):
    for rows, cols in SHAPES:
        say("b32", fmt, "mode", mode, "shape", rows, cols)
        f = fields(fmt, rows, cols, rows * 31 + cols)
        M = Mat(qg, f)
        x = act_row(cols, rows + 5 * cols, mode)
        out, act = qg.quantize_gemv(M.fmt, rows, cols, M.img, dev(x.reshape(-1)), mode)
        oc, om, oe, os_ = oracle_act(fmt, x, mode)
        m, e = act.scale_fields()
        assert np.array_equal(act.codes.cpu().numpy(), oc)
        assert np.array_equal(m, om) and np.array_equal(e, oe)
        assert np.array_equal(act.csums.cpu().numpy(), os_)
        want = oracle.gemv(f, oc, om, oe, mode)
        assert first_mismatch(out, want) is None, (rows, cols, first_mismatch(out, want))
        two = qg.gemv(M.fmt, rows, cols, M.img, act)
        assert first_mismatch(two, want) is None, (rows, cols, first_mismatch(two, want))


@pytest.mark.parametrize("fmt", FMTS)
def test_launch_configuration_does_not_change_bits(qg, fmt):
    f = fields(fmt, 300, 4096, 5)
    M = Mat(qg, f)
    x = act_row(4096, 6, 0)
    ref, act = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, dev(x.reshape(-1)), 0)
    oc, om, oe, _ = oracle_act(fmt, x, 0)
    assert first_mismatch(ref, oracle.gemv(f, oc, om, oe, 0)) is None
    try:
        for w in (4, 8, 16):
            qg.qg_set_tuning(qg.TUNE_WAVES_PER_WG, w)
            say("b32 waves per workgroup", w)
            out, _ = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, dev(x.reshape(-1)), 0)
            assert np.array_equal(bits(out), bits(ref)), w
            out2 = qg.gemv(M.fmt, M.rows, M.cols, M.img, act)
            assert np.array_equal(bits(out2), bits(ref)), w
    finally:
        qg.qg_set_tuning(qg.TUNE_WAVES_PER_WG, 0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [0, 1])
def test_batched_columns(qg, fmt, mode):
    rows, cols, n = 200, 1536, 5
    f = fields(fmt, rows, cols, 44)
    M = Mat(qg, f)
    x = gen.act_outliers(n, cols, 45) if mode == 0 else gen.act_sub32(n, cols, 45)[0]
    act = qg.quantize_act(dev(x), mode, M.fmt)
    out = qg.gemm(M.fmt, rows, cols, M.img, act)
    oc, om, oe, _ = oracle_act(fmt, x, mode)
    want = oracle.gemm(f, oc, om, oe, mode)
    assert first_mismatch(out, want) is None, first_mismatch(out, want)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [0, 1])
def test_multi_matrix_launch(qg, fmt, mode):
    cols = 1280
    shapes = [130, 0, 64, 7]
    mats = [Mat(qg, fields(fmt, r, cols, 800 + k)) if r else None for k, r in enumerate(shapes)]
    x = act_row(cols, 81, mode)
    xd = dev(x.reshape(-1))
    code = qg.FMT_CODES[fmt]
    images = [M.img if M else None for M in mats]
    outs = [torch.full((max(r, 1),), -7.0, dtype=torch.float32, device=DEV) for r in shapes]
    act = qg.alloc_act(1, cols, mode, DEV, code)
    say("b32 multi", fmt, "mode", mode)
    qg.qg_quantize_gemv_multi(code, mode, shapes, cols, images, xd, act.codes, act.scales, act.csums, None, outs)
    oc, om, oe, os_ = oracle_act(fmt, x, mode)
    m, e = act.scale_fields()
    assert np.array_equal(act.codes.cpu().numpy(), oc) and np.array_equal(m, om) and np.array_equal(e, oe)
    outs2 = [torch.full((max(r, 1),), -7.0, dtype=torch.float32, device=DEV) for r in shapes]
    qg.qg_gemv_q_multi(code, mode, shapes, cols, images, act.codes, act.scales, act.csums, outs2)
    for k, M in enumerate(mats):
        if M is None:
            assert float(outs[k][0].item()) == -7.0 and float(outs2[k][0].item()) == -7.0
            continue
        want = oracle.gemv(M.f, oc, om, oe, mode)
        assert first_mismatch(outs[k], want) is None, k
        assert first_mismatch(outs2[k], want) is None, k


@pytest.mark.parametrize("fmt", FMTS)
def test_fused_argmax(qg, fmt):
    rows, cols = 3000, 2048
    f = fields(fmt, rows, cols, 90, adversarial=False)
    M = Mat(qg, f)
    x = act_row(cols, 91, 0)
    act = qg.alloc_act(1, cols, 0, DEV, M.fmt)
    out = torch.empty(rows, dtype=torch.float32, device=DEV)
    key = torch.zeros(1, dtype=torch.int64, device=DEV)
    say("b32 argmax", fmt)
    qg.qg_quantize_gemv_argmax(M.fmt, 0, rows, cols, M.img, dev(x.reshape(-1)), act.codes, act.scales, act.csums,
                               None, out, key)
    oc, om, oe, _ = oracle_act(fmt, x, 0)
    want = oracle.gemv(f, oc, om, oe, 0)
    assert first_mismatch(out, want) is None
    assert qg.qg_argmax_index(int(key.item())) == oracle.argmax(want)


def test_infinity_flag(qg):
    f = fields("q8_0", 70, 512, 3, adversarial=False)
    M = Mat(qg, f)
    x = gen.act_normal(1, 512, 4)
    x[0, 100] = np.inf
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    for mode in (0, 1):
        flag.zero_()
        out, act = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, dev(x.reshape(-1)), mode, err_flag=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1
        oc, om, oe, _ = oracle.quantize(x, mode, block=32, check=False)
        m, e = act.scale_fields()
        assert np.array_equal(act.codes.cpu().numpy(), oc) and np.array_equal(m, om) and np.array_equal(e, oe)
        assert first_mismatch(out, oracle.gemv(f, oc, om, oe, mode)) is None


@pytest.mark.parametrize("fmt,seed", [("q8_0", gen.SEED_Q8_W), ("q4_0", gen.SEED_Q4_0_W)])
def test_full_size_matrix(qg, fmt, seed):
    """The 14336 x 4096 matrix the benchmark times, every row against the oracle, for three
    decode rows through the fused path and the two-launch path."""
    f = (gen.q8_0_fields if fmt == "q8_0" else gen.q4_0_fields)(14336, 4096, seed)
    M = Mat(qg, f)
    for k in range(3):
        say("b32 full size", fmt, "decode row", k)
        x = gen.decode_act(k)
        out, act = qg.quantize_gemv(M.fmt, M.rows, M.cols, M.img, dev(x.reshape(-1)), 0)
        oc, om, oe, _ = oracle_act(fmt, x, 0)
        want = oracle.gemv(f, oc, om, oe, 0)
        assert first_mismatch(out, want) is None, (k, first_mismatch(out, want))
        assert np.array_equal(bits(qg.gemv(M.fmt, M.rows, M.cols, M.img, act)), bits(out))


def _subnormal_partial_row(fmt, cols, at):
    """A row whose pieces (one per 32-element block, PerBlock) are normal but tiny (about
    2^-120) and cancel so that partial sums of the row are subnormal: blocks at+0 and at+1 give
    +p and -p' with p' - p one binary16 step of d, and block at+2 a piece the flushed and the
    unflushed running sums treat differently.  Activations are all 2^-110, so every block has
    the same codes and scale."""
    nb = cols // 32
    if fmt == "q8_0":
        q = np.ones(cols, np.int8)
        plus, minus = 1, -1
    else:
        q = np.full(cols, 9, np.uint8)
        plus, minus = 9, 7
    d = np.full(nb, 0x0400, np.uint16)                      # 2^-14
    q[32 * (at + 1):32 * (at + 2)] = minus
    q[32 * at:32 * (at + 1)] = plus
    d[at] = 0x0800                                          # 2^-13
    d[at + 1] = 0x0801                                      # 2^-13 (1 + 2^-10)
    d[at + 2] = 0x0001                                      # 2^-24
    return q, d


@pytest.mark.parametrize("fmt", FMTS)
def test_subnormal_partial_sums_are_flushed(qg, fmt):
    """Rows whose running sum passes through the subnormal range: every partial sum is flushed
    as in the oracle (the producers flag the tiny pieces and the row is added with the flush);
    one round (256 columns) and several rounds (8192 columns, pattern in a later round)."""
    for cols, at in ((256, 0), (8192, 130), (8192, 0)):
        rows = 70
        f = fields(fmt, rows, cols, 60 + at, adversarial=False)
        f["d"][:] = 0x0400
        for r in (0, 5, 69):
            q, d = _subnormal_partial_row(fmt, cols, at)
            f["q"][r], f["d"][r] = q, d
        M = Mat(qg, f)
        x = np.full((1, cols), np.float32(2.0 ** -110))
        say("b32 subnormal partial sums", fmt, cols, at)
        out, act = qg.quantize_gemv(M.fmt, rows, cols, M.img, dev(x.reshape(-1)), 0)
        oc, om, oe, _ = oracle_act(fmt, x, 0)
        want = oracle.gemv(f, oc, om, oe, 0)
        assert first_mismatch(out, want) is None, (cols, at, first_mismatch(out, want))
        # the case is a real one: adding the same pieces without the flush gives other bits
        code = int(oc[0, 0])
        s = float(om[0, 0]) * 2.0 ** int(oe[0, 0])
        w = np.float32(0)
        q0, d0 = f["q"][0], f["d"][0]
        for j in range(cols // 32):
            wq = q0[32 * j:32 * j + 32].astype(np.int64) - (0 if fmt == "q8_0" else 8)
            C = int(wq.sum()) * code
            p = np.float32(C * float(np.uint16(d0[j]).view(np.float16)) * s)
            w = np.float32(w + p)
        assert w.view(np.uint32) != bits(want)[0], "the row does not reach a subnormal partial sum"
