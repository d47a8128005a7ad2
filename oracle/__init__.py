"""CPU oracle of the exact block-quantized GEMV -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this package.
The product path (block_format_gemv_amd) never imports it, and it never imports the product.

The arithmetic lives in oracle.c (built to liboracle.so by oracle/build.py); this module
only marshals numpy arrays into it.  oracle/exact.py is a second, independent reference in
exact rationals for tiny inputs, used to pin oracle.c.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

PERBLOCK, SUB32 = 0, 1
STATUS = {0: "ok", 1: "nonfinite", 2: "shape", 3: "unreadable", 4: "range", 5: "internal"}

_libs: dict = {}


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what}: {STATUS.get(status, status)}")
        self.status = status


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def lib(mutant: int = 0):
    """The oracle library (mutant > 0: a variant with one planted mistake, built on demand)."""
    if mutant in _libs:
        return _libs[mutant]
    path = _build.lib_path(mutant)
    if mutant or not os.path.exists(path):
        _build.build(mutant)
    L = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    L.or_quantize.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp]
    L.or_gemm_q4k.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.or_gemm_q6k.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.or_sub_sums_q4k.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
    L.or_sub_sums_q6k.argtypes = [i64, i64, vp, vp, vp, vp]
    L.or_scaled_to_f32.argtypes = [ctypes.c_int64, ctypes.c_int]
    L.or_scaled_to_f32.restype = ctypes.c_float
    L.or_ftz.argtypes = [ctypes.c_float]
    L.or_ftz.restype = ctypes.c_float
    L.or_exact_sum_i64.argtypes = [ctypes.c_int, vp, vp, vp]
    L.or_least_scale.argtypes = [ctypes.c_int, ctypes.c_float, vp, vp]
    L.or_rne_div.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_int]
    L.or_rne_div.restype = ctypes.c_int64
    L.or_f16_scale.argtypes = [ctypes.c_uint16, vp, vp]
    L.or_set_threads.argtypes = [ctypes.c_int]
    L.or_gemm_b32.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.or_argmax.argtypes = [vp, i64]
    L.or_f16_rne.argtypes = [ctypes.c_float]
    L.or_f16_rne.restype = ctypes.c_uint16
    L.or_kv_cache_rows.argtypes = [i64, i64, vp, vp, vp]
    L.or_kv_quantize_heads.argtypes = [i32, i64, i64, vp, vp, vp, vp]
    L.or_kv_scores.argtypes = [i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.or_kv_weighted.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp]
    L.or_argmax.restype = ctypes.c_int64
    _libs[mutant] = L
    return L


def set_threads(n: int, mutant: int = 0) -> None:
    lib(mutant).or_set_threads(int(n))


def quantize(x: np.ndarray, mode: int, block: int = 256, mutant: int = 0, check: bool = True):
    """Activation rows x (f32 [n, C]) -> (codes int8 [n,C], m uint8 [n,nb], e int16 [n,nb],
    sums16 int32 [n, C/16]); nb = C/block (PerBlock) or C/32 (Sub32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    n, cols = x.shape
    ablk = block if mode == PERBLOCK else 32
    nb = cols // ablk
    codes = np.zeros((n, cols), np.int8)
    m = np.zeros((n, nb), np.uint8)
    e = np.zeros((n, nb), np.int16)
    s16 = np.zeros((n, cols // 16), np.int32)
    st = lib(mutant).or_quantize(mode, block, n, cols, _p(x), _p(codes), _p(m), _p(e), _p(s16))
    if st and check:
        raise OracleError(st, "quantize")
    return codes, m, e, s16


B32_FMT = {"q8_0": 3, "q4_0": 4}


def act_block(fmt: str, mode: int) -> int:
    """Elements per activation scale: the weight format's own block under PerBlock, 32 under Sub32."""
    if mode == SUB32:
        return 32
    return 32 if fmt in B32_FMT else 256


def gemm(fields: dict, codes: np.ndarray, m: np.ndarray, e: np.ndarray, mode: int, mutant: int = 0) -> np.ndarray:
    """out f32 [ncol * rows] with out[c*rows + r] = dot(row r, activation column c)."""
    codes = np.ascontiguousarray(codes, np.int8)
    if codes.ndim == 1:
        codes = codes[None]
    m = np.ascontiguousarray(m, np.uint8).reshape(codes.shape[0], -1)
    e = np.ascontiguousarray(e, np.int16).reshape(codes.shape[0], -1)
    ncol = codes.shape[0]
    rows, cols = fields["rows"], fields["cols"]
    out = np.zeros(ncol * rows, np.float32)
    L = lib(mutant)
    f = {k: np.ascontiguousarray(v) for k, v in fields.items() if isinstance(v, np.ndarray)}
    if fields["fmt"] == "q4k":
        st = L.or_gemm_q4k(mode, rows, cols, ncol, _p(f["q"]), _p(f["sc"]), _p(f["mn"]), _p(f["d"]),
                           _p(f["dmin"]), _p(codes), _p(m), _p(e), _p(out))
    elif fields["fmt"] == "q6k":
        st = L.or_gemm_q6k(mode, rows, cols, ncol, _p(f["q"]), _p(f["sc"]), _p(f["d"]),
                           _p(codes), _p(m), _p(e), _p(out))
    else:
        q = np.ascontiguousarray(f["q"]).view(np.uint8)            # stored bytes (int8 for Q8_0)
        st = L.or_gemm_b32(B32_FMT[fields["fmt"]], mode, rows, cols, ncol, _p(q), _p(f["d"]),
                           _p(codes), _p(m), _p(e), _p(out))
    if st:
        raise OracleError(st, "gemm")
    return out


def gemv(fields: dict, codes, m, e, mode: int, mutant: int = 0) -> np.ndarray:
    return gemm(fields, codes, m, e, mode, mutant)


def sub_sums(fields: dict, codes: np.ndarray):
    """Integer sums per (row, sub-block) for one code row: Q4_K -> (C, O) int64 [rows, C/32];
    Q6_K -> C int64 [rows, C/16]."""
    codes = np.ascontiguousarray(codes, np.int8).reshape(-1)
    rows, cols = fields["rows"], fields["cols"]
    L = lib()
    if fields["fmt"] == "q4k":
        C = np.zeros((rows, cols // 32), np.int64)
        O = np.zeros((rows, cols // 32), np.int64)
        st = L.or_sub_sums_q4k(rows, cols, _p(np.ascontiguousarray(fields["q"])), _p(np.ascontiguousarray(fields["sc"])),
                               _p(np.ascontiguousarray(fields["mn"])), _p(codes), _p(C), _p(O))
        if st:
            raise OracleError(st, "sub_sums")
        return C, O
    C = np.zeros((rows, cols // 16), np.int64)
    st = L.or_sub_sums_q6k(rows, cols, _p(np.ascontiguousarray(fields["q"])), _p(np.ascontiguousarray(fields["sc"])),
                           _p(codes), _p(C))
    if st:
        raise OracleError(st, "sub_sums")
    return C


def scaled_to_f32(v: int, exp: int, mutant: int = 0) -> np.float32:
    return np.float32(lib(mutant).or_scaled_to_f32(int(v), int(exp)))


def exact_sum(vs, es, mutant: int = 0) -> np.float32:
    v = np.ascontiguousarray(vs, np.int64)
    e = np.ascontiguousarray(es, np.int32)
    out = np.zeros(1, np.float32)
    st = lib(mutant).or_exact_sum_i64(len(v), _p(v), _p(e), _p(out))
    if st:
        raise OracleError(st, "exact_sum")
    return out[0]


def least_scale(amax: float, bits: int, mutant: int = 0):
    lo = 1 << (bits - 1)
    m = np.zeros(1, np.int32)
    e = np.zeros(1, np.int32)
    st = lib(mutant).or_least_scale(lo, float(np.float32(amax)), _p(m), _p(e))
    if st:
        raise OracleError(st, "least_scale")
    return int(m[0]), int(e[0])


def rne_div(x: float, m: int, e: int, mutant: int = 0) -> int:
    return int(lib(mutant).or_rne_div(float(np.float32(x)), int(m), int(e)))


def argmax(x: np.ndarray, mutant: int = 0) -> int:
    """[numerics] argmax of a binary32 row: first of equals, +0 == -0, NaN passed over, 0 if none."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    return int(lib(mutant).or_argmax(_p(x), x.size))


def f16_scale(h: int):
    sig = np.zeros(1, np.int64)
    ex = np.zeros(1, np.int32)
    st = lib().or_f16_scale(int(h), _p(sig), _p(ex))
    if st:
        raise OracleError(st, "f16_scale")
    return int(sig[0]), int(ex[0])


# --- int8 KV cache ([numerics] cache_row, quantize_head, int8_score, weighted_int8) ----------

VALUE_BLOCK = 32


def f16_rne(x: float, mutant: int = 0) -> int:
    """binary32 -> binary16 bits, nearest even, subnormals kept, past the top infinite."""
    return int(lib(mutant).or_f16_rne(float(np.float32(x))))


def kv_cache_rows(x: np.ndarray, mutant: int = 0):
    """Rows x f32 [n, hd] -> (scales uint16 [n] (binary16 bits), codes int8 [n, hd])."""
    x = np.ascontiguousarray(x, np.float32)
    if x.ndim == 1:
        x = x[None]
    n, hd = x.shape
    scales = np.zeros(n, np.uint16)
    codes = np.zeros((n, hd), np.int8)
    st = lib(mutant).or_kv_cache_rows(n, hd, _p(x), _p(scales), _p(codes))
    if st:
        raise OracleError(st, "kv_cache_rows")
    return scales, codes


def kv_quantize_heads(q: np.ndarray, mode: int, mutant: int = 0, check: bool = True):
    """Query heads f32 [nh, hd] -> (codes int8 [nh, hd], m uint8 [nh, nb], e int16 [nh, nb])."""
    q = np.ascontiguousarray(q, np.float32)
    if q.ndim == 1:
        q = q[None]
    nh, hd = q.shape
    nb = 1 if mode == PERBLOCK else hd // 32
    codes = np.zeros((nh, hd), np.int8)
    m = np.zeros((nh, nb), np.uint8)
    e = np.zeros((nh, nb), np.int16)
    st = lib(mutant).or_kv_quantize_heads(mode, nh, hd, _p(q), _p(codes), _p(m), _p(e))
    if st and check:
        raise OracleError(st, "kv_quantize_heads")
    return codes, m, e


def kv_scores(mode: int, qc, qm, qe, kscales, kcodes, mutant: int = 0) -> np.ndarray:
    """int8_score of every query head against every key row of its KV head.
    qc int8 [nh, hd]; qm, qe [nh, nb]; kscales uint16 [nkv, npos]; kcodes int8 [nkv, npos, hd].
    -> f32 [nh, npos]."""
    qc = np.ascontiguousarray(qc, np.int8)
    qm = np.ascontiguousarray(qm, np.uint8)
    qe = np.ascontiguousarray(qe, np.int16)
    ks = np.ascontiguousarray(kscales, np.uint16)
    kc = np.ascontiguousarray(kcodes, np.int8)
    nh, hd = qc.shape
    nkv, npos = ks.shape
    out = np.zeros((nh, npos), np.float32)
    st = lib(mutant).or_kv_scores(mode, nh, nkv, npos, hd, _p(qc), _p(qm), _p(qe), _p(ks), _p(kc), _p(out))
    if st:
        raise OracleError(st, "kv_scores")
    return out


def kv_weighted(probs, vscales, vcodes, mutant: int = 0) -> np.ndarray:
    """weighted_int8 per head: probs f32 [nh, npos]; vscales uint16 [nkv, npos];
    vcodes int8 [nkv, npos, hd] -> f32 [nh, hd]."""
    p = np.ascontiguousarray(probs, np.float32)
    vs = np.ascontiguousarray(vscales, np.uint16)
    vc = np.ascontiguousarray(vcodes, np.int8)
    nh, npos = p.shape
    nkv = vs.shape[0]
    hd = vc.shape[2]
    out = np.zeros((nh, hd), np.float32)
    st = lib(mutant).or_kv_weighted(nh, nkv, npos, hd, _p(p), _p(vs), _p(vc), _p(out))
    if st:
        raise OracleError(st, "kv_weighted")
    return out
