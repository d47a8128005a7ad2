"""Host-side checks of libqgemv.so (no GPU): the library loads and exports every entry point
include/qgemv.h declares; the packer writes exactly the documented tile layout (checked by
an independent numpy unpacker written from the header's description); argument
validation refuses bad calls before any GPU work, with a reason."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import block_format_gemv_amd as qg
from workloads import gen

from image_layout import _tiles, unpack_b32, unpack_q4k, unpack_q6k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qg_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 11
    L = ctypes.CDLL(qg.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qg.EXPORTS)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("rows,cols", [(1, 256), (5, 768), (64, 1024), (70, 512)])
def test_b32_pack_roundtrip(fmt, rows, cols):
    f = (gen.q8_0_fields if fmt == "q8_0" else gen.q4_0_fields)(rows, cols, rows * 13 + cols)
    code = qg.FMT_CODES[fmt]
    img = qg.pack(f)
    assert img.nbytes == qg.qg_image_bytes(code, rows, cols)
    u = unpack_b32(img, code == qg.Q8_0, rows, cols)
    assert np.array_equal(u["q"], f["q"]) and np.array_equal(u["d"], f["d"])
    if rows % 64:
        t, G, groups = _tiles(img, rows, cols, 17408 if code == qg.Q8_0 else 9216)
        lanes = np.arange(64) >= rows % 64
        assert not t[-1].reshape(G, -1, 64, 16)[:, :, lanes].any()


def test_b32_pack_refusals():
    f = gen.q4_0_fields(3, 256, 5)
    f["q"][2, 200] = 16
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f)
    assert ei.value.status == qg.E_INVALID
    f = gen.q8_0_fields(3, 512, 5)
    f["d"][1, 9] = 0x7C00                                        # +inf
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f)
    assert ei.value.status == qg.E_UNREADABLE and "row 1" in ei.value.reason
    img = np.zeros(qg.qg_image_bytes(qg.Q8_0, 3, 512), np.uint8)
    with pytest.raises(qg.QGError) as ei:
        qg.qg_pack_b32(qg.Q4K, 3, 512, f["q"], f["d"], img)
    assert ei.value.status == qg.E_INVALID


@pytest.mark.parametrize("rows,cols", [(1, 256), (5, 768), (64, 1024), (3, 2048), (37, 4096), (130, 1280)])
def test_q4k_pack_roundtrip(rows, cols):
    f = gen.q4k_fields(rows, cols, rows * 7 + cols)
    img = qg.pack(f)
    assert img.nbytes == qg.qg_image_bytes(qg.Q4K, rows, cols) == -(-rows // 64) * (cols // 256) * 9216
    u = unpack_q4k(img, rows, cols)
    for k in ("q", "sc", "mn", "d", "dmin"):
        assert np.array_equal(u[k], f[k]), k
    # zero padding past the last row, in every tile of the last row group
    if rows % 64:
        t, G, groups = _tiles(img, rows, cols, 9216)
        lanes = np.arange(64) >= rows % 64
        assert not t[-1, :, :8192].reshape(G, 8, 64, 16)[:, :, lanes].any()
        assert not t[-1, :, 8192:].reshape(G, 64, 16)[:, lanes].any()


@pytest.mark.parametrize("rows,cols", [(1, 256), (5, 768), (64, 1024), (9, 4096)])
def test_q6k_pack_roundtrip(rows, cols):
    f = gen.q6k_fields(rows, cols, rows * 11 + cols)
    img = qg.pack(f)
    assert img.nbytes == qg.qg_image_bytes(qg.Q6K, rows, cols) == -(-rows // 64) * (cols // 256) * 13440
    u = unpack_q6k(img, rows, cols)
    for k in ("q", "sc", "d"):
        assert np.array_equal(u[k], f[k]), k


def test_pack_refuses_unreadable_and_out_of_range_fields():
    f = gen.q4k_fields(4, 512, 3)
    f["dmin"][2, 1] = 0x7E00                                     # NaN
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f)
    assert ei.value.status == qg.E_UNREADABLE and "row 2 block 1" in ei.value.reason
    f = gen.q4k_fields(4, 512, 3)
    f["q"][1, 7] = 16
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f)
    assert ei.value.status == qg.E_INVALID
    f = gen.q4k_fields(4, 512, 3)
    f["mn"][0, 3] = 64
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f)
    assert ei.value.status == qg.E_INVALID
    f6 = gen.q6k_fields(2, 256, 4)
    f6["d"][1, 0] = 0xFC00                                       # -inf
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f6)
    assert ei.value.status == qg.E_UNREADABLE and "row 1 block 0" in ei.value.reason
    f6 = gen.q6k_fields(2, 256, 4)
    f6["q"][0, 0] = 64
    with pytest.raises(qg.QGError) as ei:
        qg.pack(f6)
    assert ei.value.status == qg.E_INVALID


def test_image_bytes_and_reads():
    assert qg.qg_image_bytes(qg.Q4K, 14336, 4096) == 33_030_144
    assert qg.qg_image_bytes(qg.Q4K, 4096, 4096) == 9_437_184
    assert qg.qg_image_bytes(qg.Q6K, 128256, 4096) == 430_940_160
    assert qg.qg_image_bytes(qg.Q4K, 256, 1024) == 147_456
    assert qg.qg_image_bytes(qg.Q4K, 4, 100) == 0
    assert qg.qg_image_bytes(qg.Q8_0, 14336, 4096) == 14336 // 64 * 16 * 17408
    assert qg.qg_image_bytes(qg.Q4_0, 65, 512) == 2 * 2 * 9216
    assert qg.qg_image_bytes(5, 4, 256) == 0 and qg.qg_image_bytes(0, 4, 256) == 0
    for fmt in qg.FORMATS:
        for mode in (qg.PERBLOCK, qg.SUB32):
            assert qg.qg_reads(fmt, mode)
    assert not qg.qg_reads(0, 0) and not qg.qg_reads(qg.Q4K, 7)


def _raw(name):
    return getattr(qg.lib(), name)


def test_validation_refuses_before_any_gpu_work():
    """Every refusal below returns before the library touches the GPU, so it runs here."""
    L = qg.lib()
    fake = ctypes.c_void_p(0x1000)           # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x1001)
    assert L.qg_gemv_q(qg.Q4K, qg.PERBLOCK, 8, 100, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert "multiple of 256" in qg.qg_last_error()
    assert L.qg_gemv_q(qg.Q4K, qg.PERBLOCK, 8, 65536, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_gemv_q(9, qg.PERBLOCK, 8, 256, fake, fake, fake, fake, fake, None) == qg.E_INVALID
    assert L.qg_gemv_q(qg.Q4K, 5, 8, 256, fake, fake, fake, fake, fake, None) == qg.E_INVALID
    assert L.qg_gemv_q(qg.Q4K, qg.PERBLOCK, 8, 256, None, fake, fake, fake, fake, None) == qg.E_INVALID
    assert "image is NULL" in qg.qg_last_error()
    assert L.qg_gemv_q(qg.Q4K, qg.PERBLOCK, 8, 256, odd, fake, fake, fake, fake, None) == qg.E_INVALID
    assert "aligned" in qg.qg_last_error()
    assert L.qg_gemv_q(qg.Q4K, qg.PERBLOCK, -1, 256, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_gemm_q(qg.Q4K, qg.PERBLOCK, 8, 256, -2, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_gemm_q(qg.Q4K, qg.PERBLOCK, 8, 256, 3, fake, fake, fake, fake, None, None) == qg.E_INVALID
    assert L.qg_quantize_act(qg.Q4K, qg.SUB32, 1, 300, fake, fake, fake, fake, None, None) == qg.E_SHAPE
    assert L.qg_quantize_act(qg.Q4K, qg.SUB32, 1, 256, odd, fake, fake, fake, None, None) == qg.E_INVALID
    assert L.qg_block_sums(qg.Q6K, 4, 512, fake, fake, None, None, None) == qg.E_INVALID
    assert L.qg_quantize_gemv(qg.Q4K, qg.PERBLOCK, 8, 300, fake, fake, fake, fake, fake, None, fake, None) == qg.E_SHAPE
    assert L.qg_quantize_gemv(qg.Q4K, qg.PERBLOCK, 8, 256, fake, odd, fake, fake, fake, None, fake, None) == qg.E_INVALID
    assert "x is not 16-byte aligned" in qg.qg_last_error()
    assert L.qg_quantize_gemv(qg.Q4K, qg.PERBLOCK, 8, 256, fake, fake, None, fake, fake, None, fake, None) == qg.E_INVALID
    assert "codes is NULL" in qg.qg_last_error()
    assert L.qg_quantize_gemv(qg.Q4K, qg.PERBLOCK, 8, 256, None, fake, fake, fake, fake, None, fake, None) == qg.E_INVALID
    assert "image is NULL" in qg.qg_last_error()
    assert L.qg_set_tuning(77, 1) == qg.E_INVALID
    assert L.qg_set_tuning(qg.TUNE_WAVES_PER_WG, 3) == qg.E_INVALID
    assert L.qg_set_tuning(qg.TUNE_MFMA_COL_TILES, 3) == qg.E_INVALID
    assert L.qg_set_tuning(qg.TUNE_MFMA_TABLES, 2) == qg.E_INVALID
    assert L.qg_set_tuning(qg.TUNE_MFMA_FORM, 5) == qg.E_INVALID
    assert L.qg_set_tuning(5, 0) == qg.E_INVALID                # no longer a key
    assert L.qg_set_tuning(qg.TUNE_GEMM_ROW_TILES, 3) == qg.E_INVALID
    assert L.qg_set_tuning(qg.TUNE_GEMV_QUARTER, 3) == qg.E_INVALID
    assert L.qg_set_tuning(qg.TUNE_GEMV_QUARTER, 2) == qg.OK and L.qg_set_tuning(qg.TUNE_GEMV_QUARTER, 0) == qg.OK
    rows2 = (ctypes.c_int64 * 2)(8, 8)
    imgs2 = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    outs2 = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    assert L.qg_gemv_q_multi(qg.Q4K, qg.PERBLOCK, 0, rows2, 256, imgs2, fake, fake, fake, outs2, None) == qg.E_SHAPE
    assert L.qg_gemv_q_multi(qg.Q4K, qg.PERBLOCK, 9, rows2, 256, imgs2, fake, fake, fake, outs2, None) == qg.E_SHAPE
    imgs_bad = (ctypes.c_void_p * 2)(0x1000, None)
    assert L.qg_gemv_q_multi(qg.Q4K, qg.PERBLOCK, 2, rows2, 256, imgs_bad, fake, fake, fake, outs2, None) == qg.E_INVALID
    assert "images[1]" in qg.qg_last_error()
    assert L.qg_quantize_gemv_multi(qg.Q4K, qg.PERBLOCK, 2, rows2, 300, imgs2, fake, fake, fake, fake, None, outs2,
                                    None) == qg.E_SHAPE
    assert L.qg_quantize_gemv_multi(qg.Q4K, qg.PERBLOCK, 2, rows2, 256, imgs2, odd, fake, fake, fake, None, outs2,
                                    None) == qg.E_INVALID
    assert L.qg_quantize_gemv_argmax(qg.Q4K, qg.PERBLOCK, 8, 256, fake, fake, fake, fake, fake, None, fake, None,
                                     None) == qg.E_INVALID
    assert "argmax_key is NULL" in qg.qg_last_error()
    # empty work is not an error and launches nothing
    assert L.qg_gemv_q(qg.Q4K, qg.PERBLOCK, 0, 256, None, None, None, None, None, None) == qg.OK
    assert L.qg_quantize_act(qg.Q4K, qg.PERBLOCK, 0, 256, None, None, None, None, None, None) == qg.OK


def test_kv_validation_refuses_before_any_gpu_work():
    """The int8 KV cache entry points refuse bad head sizes, uneven grouped heads, bad
    scalings, null and misaligned pointers before any GPU work, and launch nothing for empty
    work (every call below returns here, where there is no GPU)."""
    L = qg.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    assert L.qg_kv_cache_rows(4, 48, fake, fake, fake, None) == qg.E_SHAPE
    assert "head size" in qg.qg_last_error()
    assert L.qg_kv_cache_rows(-1, 64, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_kv_cache_rows(4, 64, None, fake, fake, None) == qg.E_INVALID
    assert L.qg_kv_cache_rows(4, 64, fake, fake, odd, None) == qg.E_INVALID
    assert L.qg_kv_cache_rows(0, 64, None, None, None, None) == qg.OK
    assert L.qg_kv_quantize_heads(2, 4, 64, fake, fake, fake, None, None) == qg.E_INVALID
    assert L.qg_kv_quantize_heads(qg.SUB32, 4, 96, fake, fake, fake, None, None) == qg.E_SHAPE
    assert L.qg_kv_quantize_heads(qg.SUB32, 4, 64, odd, fake, fake, None, None) == qg.E_INVALID
    assert L.qg_kv_quantize_heads(qg.PERBLOCK, 4, 64, fake, fake, None, None, None) == qg.E_INVALID
    assert L.qg_kv_quantize_heads(qg.PERBLOCK, 70000, 64, fake, fake, fake, None, None) == qg.E_SHAPE
    assert L.qg_kv_quantize_heads(qg.PERBLOCK, 0, 64, None, None, None, None, None) == qg.OK
    assert L.qg_kv_scores(qg.PERBLOCK, 6, 4, 10, 64, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert "KV heads" in qg.qg_last_error()
    assert L.qg_kv_scores(qg.PERBLOCK, 8, 0, 10, 64, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_kv_scores(qg.SUB32, 8, 2, -1, 64, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_kv_scores(qg.SUB32, 8, 2, 1 << 26, 64, fake, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_kv_scores(qg.SUB32, 8, 2, 10, 64, fake, fake, fake, odd, fake, None) == qg.E_INVALID
    assert L.qg_kv_scores(3, 8, 2, 10, 64, fake, fake, fake, fake, fake, None) == qg.E_INVALID
    assert L.qg_kv_scores(qg.SUB32, 8, 2, 0, 64, None, None, None, None, None, None) == qg.OK
    assert L.qg_kv_weighted(8, 3, 10, 64, fake, fake, fake, fake, None) == qg.E_SHAPE
    assert L.qg_kv_weighted(8, 2, 10, 64, fake, fake, fake, None, None) == qg.E_INVALID
    assert L.qg_kv_weighted(8, 2, 10, 64, fake, odd, ctypes.c_void_p(0x1001), fake, None) == qg.E_INVALID
    assert L.qg_kv_weighted(0, 2, 10, 64, None, None, None, None, None) == qg.OK


def test_kv_weighted_workspace_size_and_refusals():
    """qg_kv_weighted_workspace: one f32 piece per (head, 32-position block, element), the last
    block possibly short; qg_kv_weighted_with_workspace refuses a short, null or misaligned
    workspace and everything qg_kv_weighted refuses, before any GPU work (no GPU here)."""
    L = qg.lib()
    for nh, npos, hd in [(32, 4096, 128), (8, 1, 64), (4, 33, 32), (6, 0, 256), (0, 100, 128), (1, 31, 256)]:
        assert qg.qg_kv_weighted_workspace(nh, npos, hd) == nh * (-(-npos // 32)) * hd * 4
    with pytest.raises(qg.QGError) as ei:
        qg.qg_kv_weighted_workspace(4, 10, 48)
    assert ei.value.status == qg.E_SHAPE
    with pytest.raises(qg.QGError):
        qg.qg_kv_weighted_workspace(4, -1, 64)
    assert L.qg_kv_weighted_workspace(4, 10, 64, None) == qg.E_INVALID
    fake = ctypes.c_void_p(0x1000)
    need = 8 * 1 * 64 * 4
    args = (fake, fake, fake, fake)
    assert L.qg_kv_weighted_with_workspace(8, 2, 10, 64, *args, fake, need - 1, None) == qg.E_INVALID
    assert "workspace" in qg.qg_last_error()
    assert L.qg_kv_weighted_with_workspace(8, 2, 10, 64, *args, None, need, None) == qg.E_INVALID
    assert L.qg_kv_weighted_with_workspace(8, 2, 10, 64, *args, ctypes.c_void_p(0x1008), need, None) == qg.E_INVALID
    assert L.qg_kv_weighted_with_workspace(8, 3, 10, 64, *args, fake, need, None) == qg.E_SHAPE
    assert L.qg_kv_weighted_with_workspace(8, 2, 10, 96, *args, fake, need, None) == qg.E_SHAPE
    assert L.qg_kv_weighted_with_workspace(8, 2, 10, 64, fake, fake, fake, None, fake, need, None) == qg.E_INVALID
    assert L.qg_kv_weighted_with_workspace(0, 2, 10, 64, None, None, None, None, None, 0, None) == qg.OK
    # the fixed workspace of qg_kv_weighted_noalloc: 4 MiB, refused beyond it before any GPU work
    assert qg.KV_NOALLOC_BYTES == 4 << 20
    assert L.qg_kv_weighted_noalloc(64, 8, 8192, 128, *args, None) == qg.E_SHAPE
    assert "fixed workspace" in qg.qg_last_error()
    assert L.qg_kv_weighted_noalloc(8, 3, 10, 64, *args, None) == qg.E_SHAPE
    assert L.qg_kv_weighted_noalloc(8, 2, 10, 64, fake, fake, fake, None, None) == qg.E_INVALID
    assert L.qg_kv_weighted_noalloc(0, 2, 10, 64, None, None, None, None, None) == qg.OK


def test_kv_binding_refuses_short_buffers():
    """The binding checks buffer sizes the C ABI cannot see."""
    import torch
    x = torch.zeros(4 * 64 - 1, dtype=torch.float32)
    with pytest.raises(qg.QGError) as ei:
        qg.qg_kv_cache_rows(4, 64, x, torch.zeros(4, dtype=torch.int16), torch.zeros(256, dtype=torch.int8))
    assert ei.value.status == qg.E_SHAPE
    with pytest.raises(qg.QGError):
        qg.qg_kv_scores(qg.SUB32, 4, 2, 8, 64, torch.zeros(256, dtype=torch.int8),
                        torch.zeros(4, dtype=torch.int32), torch.zeros(16, dtype=torch.int16),
                        torch.zeros(1024, dtype=torch.int8), torch.zeros(32, dtype=torch.float32))


def test_argmax_key_decoding():
    """qg_argmax_index: key 0 is "none" (index 0); otherwise the low word is ~row."""
    assert qg.qg_argmax_index(0) == 0
    for row in (0, 1, 5, 14335, 128255, 2**31 - 1):
        key = (0x80000000 << 32) | (0xFFFFFFFF - row)
        assert qg.qg_argmax_index(key) == row


def test_check_maps_the_nonfinite_flag():
    """check(): a clear flag passes, a set one raises QG_E_NONFINITE (host flag: no device)."""
    import torch
    qg.check(torch.zeros(1, dtype=torch.int32))
    qg.check(None)
    with pytest.raises(qg.QGError) as ei:
        qg.check(torch.ones(1, dtype=torch.int32))
    assert ei.value.status == qg.E_NONFINITE
