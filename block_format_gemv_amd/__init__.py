"""Python binding of libqgemv.so: the exact block-quantized GEMV / GEMM for MI355X (gfx950).

The functions named qg_* mirror the C ABI of include/qgemv.h one for one and only marshal
arguments: torch tensors on the ROCm device are passed as device pointers, numpy arrays as
host pointers, and the stream defaults to torch's current stream.  Every step of the path
runs in the library's HIP kernels; there is no CPU fallback.  A nonzero status raises
QGError with the library's reason.

Convenience wrappers (pack, quantize_act, gemv, quantize_gemv, gemm) allocate outputs with torch and
call the qg_* functions.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemv.so")

Q4K, Q6K, Q8_0, Q4_0 = 1, 2, 3, 4
FORMATS = (Q4K, Q6K, Q8_0, Q4_0)
PERBLOCK, SUB32 = 0, 1
OK, E_INVALID, E_SHAPE, E_UNSUPPORTED, E_UNREADABLE, E_NONFINITE, E_RUNTIME = range(7)
TUNE_WAVES_PER_WG, TUNE_MFMA_MIN_COLS, TUNE_MFMA_COL_TILES, TUNE_MFMA_FORM = 1, 2, 3, 4
TUNE_COLS_KERNEL = 6
TUNE_MFMA_TABLES = 7
TUNE_GEMM_ROW_TILES = 8
TUNE_GEMV_QUARTER = 9
BLOCK = 256
MAX_COLS = 32768
MAX_MATRICES = 8

EXPORTS = ("qg_reads", "qg_image_bytes", "qg_pack_q4k", "qg_pack_q6k", "qg_pack_b32", "qg_quantize_act",
           "qg_gemv_q", "qg_gemm_q", "qg_quantize_gemv", "qg_quantize_gemv_argmax", "qg_argmax_index",
           "qg_quantize_gemv_multi", "qg_gemv_q_multi", "qg_block_sums", "qg_stream_read", "qg_stream_read_shape", "qg_set_tuning",
           "qg_time_next_launch", "qg_last_error", "qg_version", "qg_kv_cache_rows", "qg_kv_quantize_heads",
           "qg_kv_scores", "qg_kv_weighted", "qg_kv_weighted_workspace", "qg_kv_weighted_with_workspace",
           "qg_kv_weighted_noalloc")
VALUE_BLOCK = 32
KV_HEAD_SIZES = (32, 64, 128, 256)


class QGError(RuntimeError):
    def __init__(self, status: int, reason: str):
        super().__init__(f"status {status}: {reason}")
        self.status = status
        self.reason = reason


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    L.qg_reads.argtypes = [i32, i32]
    L.qg_image_bytes.argtypes = [i32, i64, i64]
    L.qg_image_bytes.restype = ctypes.c_size_t
    L.qg_pack_q4k.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
    L.qg_pack_q6k.argtypes = [i64, i64, vp, vp, vp, vp]
    L.qg_pack_b32.argtypes = [i32, i64, i64, vp, vp, vp]
    L.qg_quantize_act.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp]
    L.qg_gemv_q.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp]
    L.qg_gemm_q.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.qg_quantize_gemv.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    L.qg_block_sums.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
    L.qg_stream_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_uint32, vp, vp]
    L.qg_stream_read_shape.argtypes = [vp, ctypes.c_size_t, i32, i32, i64, i32, ctypes.c_uint32, vp, vp]
    L.qg_quantize_gemv_argmax.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.qg_argmax_index.argtypes = [ctypes.c_uint64]
    L.qg_argmax_index.restype = ctypes.c_int64
    L.qg_quantize_gemv_multi.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    L.qg_gemv_q_multi.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp]
    L.qg_set_tuning.argtypes = [i32, i64]
    L.qg_kv_cache_rows.argtypes = [i64, i64, vp, vp, vp, vp]
    L.qg_kv_quantize_heads.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
    L.qg_kv_scores.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.qg_kv_weighted.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp]
    L.qg_kv_weighted_workspace.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    L.qg_kv_weighted_with_workspace.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.qg_kv_weighted_noalloc.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp]
    L.qg_time_next_launch.argtypes = [vp, vp]
    L.qg_last_error.restype = ctypes.c_char_p
    return L


_lib = _load()


def lib():
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise QGError(status, _lib.qg_last_error().decode(errors="replace"))


def _dptr(t):
    """Device pointer of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _hptr(a: np.ndarray):
    if not a.flags.c_contiguous:
        raise ValueError("expected a C-contiguous array")
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# --- the C ABI, one for one ----------------------------------------------------------------

def qg_reads(fmt: int, mode: int) -> bool:
    return bool(_lib.qg_reads(fmt, mode))


def qg_image_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(_lib.qg_image_bytes(fmt, rows, cols))


def qg_pack_q4k(rows, cols, q, sc, mn, d, dmin, image) -> None:
    _check(_lib.qg_pack_q4k(rows, cols, _hptr(q), _hptr(sc), _hptr(mn), _hptr(d), _hptr(dmin), _hptr(image)))


def qg_pack_q6k(rows, cols, q, sc, d, image) -> None:
    _check(_lib.qg_pack_q6k(rows, cols, _hptr(q), _hptr(sc), _hptr(d), _hptr(image)))


def qg_pack_b32(fmt, rows, cols, q, d, image) -> None:
    _check(_lib.qg_pack_b32(fmt, rows, cols, _hptr(q), _hptr(d), _hptr(image)))


def _need(t, nbytes: int, name: str) -> None:
    """Refuse a device buffer smaller than the call will touch (the C ABI cannot see sizes)."""
    if t is None:
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise QGError(E_SHAPE, f"{name} holds {have} bytes, the call needs {nbytes}")


def act_block(fmt: int, mode: int) -> int:
    """Elements per activation scale: 32 under Sub32 or for a 32-element-block format, else 256."""
    return 32 if mode == SUB32 or fmt in (Q8_0, Q4_0) else BLOCK


def _nsc(fmt: int, mode: int, cols: int) -> int:
    return cols // act_block(fmt, mode)


def _check_act(fmt, mode, n, cols, codes, scales, csums):
    _need(codes, n * cols, "codes")
    _need(scales, 4 * n * _nsc(fmt, mode, cols), "scales")
    _need(csums, 4 * n * (cols // 16), "csums")


def qg_quantize_act(fmt, mode, n, cols, x, codes, scales, csums, err_flag=None, stream=None) -> None:
    if cols > 0 and cols % BLOCK == 0 and mode in (PERBLOCK, SUB32):
        _need(x, 4 * n * cols, "x")
        _check_act(fmt, mode, n, cols, codes, scales, csums)
        _need(err_flag, 4, "err_flag")
    _check(_lib.qg_quantize_act(fmt, mode, n, cols, _dptr(x), _dptr(codes), _dptr(scales), _dptr(csums),
                                _dptr(err_flag), _stream(stream)))


def _check_gemm(fmt, mode, rows, cols, n, image, codes, scales, csums, out):
    if cols > 0 and cols % BLOCK == 0 and mode in (PERBLOCK, SUB32) and fmt in FORMATS and rows > 0:
        _need(image, qg_image_bytes(fmt, rows, cols), "image")
        _check_act(fmt, mode, n, cols, codes, scales, csums)
        _need(out, 4 * n * rows, "out")


def qg_gemv_q(fmt, mode, rows, cols, image, codes, scales, csums, out, stream=None) -> None:
    _check_gemm(fmt, mode, rows, cols, 1, image, codes, scales, csums, out)
    _check(_lib.qg_gemv_q(fmt, mode, rows, cols, _dptr(image), _dptr(codes), _dptr(scales), _dptr(csums),
                          _dptr(out), _stream(stream)))


def qg_gemm_q(fmt, mode, rows, cols, n, image, codes, scales, csums, out, stream=None) -> None:
    _check_gemm(fmt, mode, rows, cols, n, image, codes, scales, csums, out)
    _check(_lib.qg_gemm_q(fmt, mode, rows, cols, n, _dptr(image), _dptr(codes), _dptr(scales), _dptr(csums),
                          _dptr(out), _stream(stream)))


def qg_quantize_gemv(fmt, mode, rows, cols, image, x, codes, scales, csums, err_flag, out, stream=None) -> None:
    if cols > 0 and cols % BLOCK == 0 and mode in (PERBLOCK, SUB32) and fmt in FORMATS:
        _need(x, 4 * cols, "x")
        _check_act(fmt, mode, 1, cols, codes, scales, csums)
        _need(err_flag, 4, "err_flag")
        if rows > 0:
            _need(image, qg_image_bytes(fmt, rows, cols), "image")
            _need(out, 4 * rows, "out")
    _check(_lib.qg_quantize_gemv(fmt, mode, rows, cols, _dptr(image), _dptr(x), _dptr(codes), _dptr(scales),
                                 _dptr(csums), _dptr(err_flag), _dptr(out), _stream(stream)))


def qg_quantize_gemv_argmax(fmt, mode, rows, cols, image, x, codes, scales, csums, err_flag, out, argmax_key,
                            stream=None) -> None:
    """argmax_key: device int64 [1] holding 0 before the call."""
    if cols > 0 and cols % BLOCK == 0 and mode in (PERBLOCK, SUB32) and fmt in FORMATS:
        _need(x, 4 * cols, "x")
        _check_act(fmt, mode, 1, cols, codes, scales, csums)
        _need(err_flag, 4, "err_flag")
        _need(argmax_key, 8, "argmax_key")
        if rows > 0:
            _need(image, qg_image_bytes(fmt, rows, cols), "image")
            _need(out, 4 * rows, "out")
    _check(_lib.qg_quantize_gemv_argmax(fmt, mode, rows, cols, _dptr(image), _dptr(x), _dptr(codes), _dptr(scales),
                                        _dptr(csums), _dptr(err_flag), _dptr(out), _dptr(argmax_key),
                                        _stream(stream)))


def qg_argmax_index(key: int) -> int:
    return int(_lib.qg_argmax_index(ctypes.c_uint64(key & 0xFFFFFFFFFFFFFFFF)))


def _multi_args(fmt, mode, rows, cols, images, outs):
    """Host arrays for the *_multi calls (kept alive by the caller's frame)."""
    nmat = len(rows)
    if not (len(images) == len(outs) == nmat):
        raise QGError(E_INVALID, "rows, images and outs differ in length")
    if cols > 0 and cols % BLOCK == 0 and fmt in FORMATS:
        for m in range(nmat):
            if rows[m] > 0:
                _need(images[m], qg_image_bytes(fmt, rows[m], cols), f"images[{m}]")
                _need(outs[m], 4 * rows[m], f"outs[{m}]")
    r = (ctypes.c_int64 * max(nmat, 1))(*[int(v) for v in rows])
    im = (ctypes.c_void_p * max(nmat, 1))(*[_dptr(t) for t in images])
    ou = (ctypes.c_void_p * max(nmat, 1))(*[_dptr(t) for t in outs])
    return nmat, r, im, ou


def qg_quantize_gemv_multi(fmt, mode, rows, cols, images, x, codes, scales, csums, err_flag, outs,
                           stream=None) -> None:
    """rows: list of ints; images, outs: lists of device tensors (one per matrix)."""
    nmat, r, im, ou = _multi_args(fmt, mode, rows, cols, images, outs)
    if cols > 0 and cols % BLOCK == 0 and mode in (PERBLOCK, SUB32):
        _need(x, 4 * cols, "x")
        _check_act(fmt, mode, 1, cols, codes, scales, csums)
        _need(err_flag, 4, "err_flag")
    _check(_lib.qg_quantize_gemv_multi(fmt, mode, nmat, r, cols, im, _dptr(x), _dptr(codes), _dptr(scales),
                                       _dptr(csums), _dptr(err_flag), ou, _stream(stream)))


def qg_gemv_q_multi(fmt, mode, rows, cols, images, codes, scales, csums, outs, stream=None) -> None:
    nmat, r, im, ou = _multi_args(fmt, mode, rows, cols, images, outs)
    if cols > 0 and cols % BLOCK == 0 and mode in (PERBLOCK, SUB32):
        _check_act(fmt, mode, 1, cols, codes, scales, csums)
    _check(_lib.qg_gemv_q_multi(fmt, mode, nmat, r, cols, im, _dptr(codes), _dptr(scales), _dptr(csums), ou,
                                _stream(stream)))


def qg_block_sums(fmt, rows, cols, image, codes, csum_out, osum_out=None, stream=None) -> None:
    if cols > 0 and cols % BLOCK == 0 and fmt in (Q4K, Q6K) and rows > 0:
        per = 32 if fmt == Q4K else 16
        _need(image, qg_image_bytes(fmt, rows, cols), "image")
        _need(codes, cols, "codes")
        _need(csum_out, 4 * rows * (cols // per), "csum_out")
        if fmt == Q4K:
            _need(osum_out, 4 * rows * (cols // 32), "osum_out")
    _check(_lib.qg_block_sums(fmt, rows, cols, _dptr(image), _dptr(codes), _dptr(csum_out), _dptr(osum_out),
                              _stream(stream)))


def _kv_shape_ok(nh, nkv, npos, hd) -> bool:
    return hd in KV_HEAD_SIZES and nkv >= 1 and nh >= 0 and nh % nkv == 0 and npos >= 0


def qg_kv_cache_rows(n, hd, x, scales, codes, stream=None) -> None:
    if hd in KV_HEAD_SIZES and n > 0:
        _need(x, 4 * n * hd, "x")
        _need(scales, 2 * n, "scales")
        _need(codes, n * hd, "codes")
    _check(_lib.qg_kv_cache_rows(n, hd, _dptr(x), _dptr(scales), _dptr(codes), _stream(stream)))


def qg_kv_quantize_heads(mode, nh, hd, q, codes, scales, err_flag=None, stream=None) -> None:
    if hd in KV_HEAD_SIZES and nh > 0 and mode in (PERBLOCK, SUB32):
        _need(q, 4 * nh * hd, "q")
        _need(codes, nh * hd, "codes")
        _need(scales, 4 * nh * (1 if mode == PERBLOCK else hd // 32), "scales")
        _need(err_flag, 4, "err_flag")
    _check(_lib.qg_kv_quantize_heads(mode, nh, hd, _dptr(q), _dptr(codes), _dptr(scales), _dptr(err_flag),
                                     _stream(stream)))


def qg_kv_scores(mode, nh, nkv, npos, hd, qcodes, qscales, kscales, kcodes, out, stream=None) -> None:
    if _kv_shape_ok(nh, nkv, npos, hd) and nh > 0 and npos > 0 and mode in (PERBLOCK, SUB32):
        _need(qcodes, nh * hd, "qcodes")
        _need(qscales, 4 * nh * (1 if mode == PERBLOCK else hd // 32), "qscales")
        _need(kscales, 2 * nkv * npos, "kscales")
        _need(kcodes, nkv * npos * hd, "kcodes")
        _need(out, 4 * nh * npos, "out")
    _check(_lib.qg_kv_scores(mode, nh, nkv, npos, hd, _dptr(qcodes), _dptr(qscales), _dptr(kscales), _dptr(kcodes),
                             _dptr(out), _stream(stream)))


def qg_kv_weighted(nh, nkv, npos, hd, probs, vscales, vcodes, out, stream=None) -> None:
    if _kv_shape_ok(nh, nkv, npos, hd) and nh > 0:
        _need(out, 4 * nh * hd, "out")
        if npos > 0:
            _need(probs, 4 * nh * npos, "probs")
            _need(vscales, 2 * nkv * npos, "vscales")
            _need(vcodes, nkv * npos * hd, "vcodes")
    _check(_lib.qg_kv_weighted(nh, nkv, npos, hd, _dptr(probs), _dptr(vscales), _dptr(vcodes), _dptr(out),
                               _stream(stream)))


def qg_kv_weighted_workspace(nh, npos, hd) -> int:
    """Bytes of workspace qg_kv_weighted_with_workspace needs."""
    n = ctypes.c_size_t(0)
    _check(_lib.qg_kv_weighted_workspace(nh, npos, hd, ctypes.byref(n)))
    return n.value


def qg_kv_weighted_with_workspace(nh, nkv, npos, hd, probs, vscales, vcodes, out, workspace, stream=None) -> None:
    """qg_kv_weighted in two passes over a caller's workspace (all of the tensor's bytes)."""
    if _kv_shape_ok(nh, nkv, npos, hd) and nh > 0:
        _need(out, 4 * nh * hd, "out")
        if npos > 0:
            _need(probs, 4 * nh * npos, "probs")
            _need(vscales, 2 * nkv * npos, "vscales")
            _need(vcodes, nkv * npos * hd, "vcodes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.qg_kv_weighted_with_workspace(nh, nkv, npos, hd, _dptr(probs), _dptr(vscales), _dptr(vcodes),
                                              _dptr(out), _dptr(workspace), ws_bytes, _stream(stream)))


KV_NOALLOC_BYTES = 4 << 20


def qg_kv_weighted_noalloc(nh, nkv, npos, hd, probs, vscales, vcodes, out, stream=None) -> None:
    """qg_kv_weighted over the library's fixed per-device workspace (no allocation)."""
    if _kv_shape_ok(nh, nkv, npos, hd) and nh > 0:
        _need(out, 4 * nh * hd, "out")
        if npos > 0:
            _need(probs, 4 * nh * npos, "probs")
            _need(vscales, 2 * nkv * npos, "vscales")
            _need(vcodes, nkv * npos * hd, "vcodes")
    _check(_lib.qg_kv_weighted_noalloc(nh, nkv, npos, hd, _dptr(probs), _dptr(vscales), _dptr(vcodes), _dptr(out),
                                       _stream(stream)))


def qg_stream_read(buf, nbytes: int, magic: int, sink, stream=None) -> None:
    """Diagnostic streaming read (the measured ceiling); see qgemv.h."""
    _need(buf, nbytes, "buf")
    _need(sink, 4, "sink")
    _check(_lib.qg_stream_read(_dptr(buf), nbytes, magic & 0xFFFFFFFF, _dptr(sink), _stream(stream)))


def qg_stream_read_shape(buf, nbytes: int, waves_per_wg: int, kib_per_wave: int, wgs: int, flags: int, magic: int,
                         sink, stream=None) -> None:
    """Diagnostic streaming read in a chosen launch geometry; see qgemv.h."""
    _need(buf, nbytes, "buf")
    _need(sink, 4, "sink")
    _check(_lib.qg_stream_read_shape(_dptr(buf), nbytes, waves_per_wg, kib_per_wave, wgs, flags, magic & 0xFFFFFFFF,
                                     _dptr(sink), _stream(stream)))


def check(err_flag, stream=None) -> None:
    """Wait for the work queued on `stream` (the current stream by default), then map the
    non-finite flag that qg_quantize_act, qg_quantize_gemv(_multi, _argmax) and
    qg_kv_quantize_heads set when an activation block holds +-inf to a refusal: QGError with
    status QG_E_NONFINITE if the flag is set.  The flag is left as it is (the caller clears it
    before the next call).  A flag in host memory is read as it is."""
    import torch
    if err_flag is None:
        return
    if err_flag.is_cuda:
        if stream is None:
            torch.cuda.current_stream(err_flag.device).synchronize()
        elif isinstance(stream, int):
            torch.cuda.synchronize(err_flag.device)
        else:
            stream.synchronize()
    if int(err_flag.reshape(-1)[0].item()) != 0:
        raise QGError(E_NONFINITE, "an activation block holds an infinity (the non-finite flag is set)")


def qg_set_tuning(key: int, value: int) -> None:
    _check(_lib.qg_set_tuning(key, value))


def qg_time_next_launch(start_event, stop_event) -> None:
    """Raw hipEvent_t handles (ints) or None."""
    _check(_lib.qg_time_next_launch(ctypes.c_void_p(start_event) if start_event else None,
                                    ctypes.c_void_p(stop_event) if stop_event else None))


def qg_last_error() -> str:
    return _lib.qg_last_error().decode(errors="replace")


def qg_version() -> int:
    return int(_lib.qg_version())


# --- convenience wrappers ------------------------------------------------------------------

FMT_CODES = {"q4k": Q4K, "q6k": Q6K, "q8_0": Q8_0, "q4_0": Q4_0}


def pack(fields: dict) -> np.ndarray:
    """Logical fields (see workloads/gen.py for the layout) -> host image (uint8)."""
    fmt = FMT_CODES[fields["fmt"]]
    rows, cols = int(fields["rows"]), int(fields["cols"])
    img = np.empty(qg_image_bytes(fmt, rows, cols), np.uint8)
    c = {k: np.ascontiguousarray(v) for k, v in fields.items() if isinstance(v, np.ndarray)}
    if fmt == Q4K:
        qg_pack_q4k(rows, cols, c["q"].astype(np.uint8, copy=False), c["sc"].astype(np.uint8, copy=False),
                    c["mn"].astype(np.uint8, copy=False), c["d"].astype(np.uint16, copy=False),
                    c["dmin"].astype(np.uint16, copy=False), img)
    elif fmt == Q6K:
        qg_pack_q6k(rows, cols, c["q"].astype(np.uint8, copy=False), c["sc"].astype(np.int8, copy=False),
                    c["d"].astype(np.uint16, copy=False), img)
    else:
        q = c["q"].astype(np.int8 if fmt == Q8_0 else np.uint8, copy=False)
        qg_pack_b32(fmt, rows, cols, q, c["d"].astype(np.uint16, copy=False), img)
    return img


class Act:
    """A quantized activation batch on the GPU: codes [n, C] int8, scales [n, nsc] as int32
    words (qg_act_scale), csums [n, C/16] int32."""

    def __init__(self, codes, scales, csums, mode):
        self.codes, self.scales, self.csums, self.mode = codes, scales, csums, mode

    @property
    def n(self):
        return int(self.codes.shape[0])

    def scale_fields(self):
        """(m uint8 [n, nsc], e int16 [n, nsc]) as host numpy arrays."""
        raw = self.scales.cpu().numpy().view(np.uint8).reshape(self.n, -1, 4)
        e = raw[..., 0:2].copy().view(np.int16)[..., 0]
        return raw[..., 2].copy(), e


def alloc_act(n: int, cols: int, mode: int, device="cuda", fmt: int = Q4K):
    import torch
    nsc = _nsc(fmt, mode, cols)
    codes = torch.empty((n, cols), dtype=torch.int8, device=device)
    scales = torch.empty((n, nsc), dtype=torch.int32, device=device)
    csums = torch.empty((n, cols // 16), dtype=torch.int32, device=device)
    return Act(codes, scales, csums, mode)


def quantize_act(x, mode: int, fmt: int = Q4K, err_flag=None, stream=None, out: Act | None = None) -> Act:
    """x: float32 [n, C] (or [C]) on the GPU -> Act."""
    if x.dim() == 1:
        x = x.unsqueeze(0)
    n, cols = x.shape
    a = out if out is not None else alloc_act(n, cols, mode, x.device, fmt)
    qg_quantize_act(fmt, mode, n, cols, x, a.codes, a.scales, a.csums, err_flag, stream)
    return a


def gemv(fmt: int, rows: int, cols: int, image, act: Act, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=act.codes.device)
    qg_gemv_q(fmt, act.mode, rows, cols, image, act.codes, act.scales, act.csums, out, stream)
    return out


def quantize_gemv(fmt: int, rows: int, cols: int, image, x, mode: int, act: Act | None = None, out=None,
                  err_flag=None, stream=None):
    """One f32 activation row x [C] on the GPU: quantize and multiply in one call.
    Returns (out [rows], the Act holding the quantized row)."""
    import torch
    a = act if act is not None else alloc_act(1, cols, mode, x.device, fmt)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=x.device)
    qg_quantize_gemv(fmt, mode, rows, cols, image, x, a.codes, a.scales, a.csums, err_flag, out, stream)
    return out, a


def gemm(fmt: int, rows: int, cols: int, image, act: Act, out=None, stream=None):
    """out[c, r] (a [n, rows] view of the flat out[c*rows + r])."""
    import torch
    if out is None:
        out = torch.empty((act.n, rows), dtype=torch.float32, device=act.codes.device)
    qg_gemm_q(fmt, act.mode, rows, cols, act.n, image, act.codes, act.scales, act.csums, out, stream)
    return out
