"""Independent unpackers of the weight images, written from the tile layouts described in
include/qgemv.h: image bytes back to the logical fields (numpy only, no library import), for
the packer's round-trip tests."""
from __future__ import annotations

import numpy as np


def _tiles(img: np.ndarray, rows: int, cols: int, tile_bytes: int):
    """Image -> array [groups, G, tile_bytes]; tile (g, b) holds rows 64g..64g+63 of block b."""
    G = cols // 256
    groups = -(-rows // 64)
    return img.reshape(groups, G, tile_bytes), G, groups


def unpack_q4k(img: np.ndarray, rows: int, cols: int) -> dict:
    t, G, groups = _tiles(img, rows, cols, 9216)
    chunks = t[..., :8192].reshape(groups, G, 8, 64, 16)        # [g, b, chunk i, lane, byte k]
    meta = t[..., 8192:].reshape(groups, G, 64, 16)             # [g, b, lane, 16]
    sub = np.concatenate([chunks & 15, chunks >> 4], axis=4)    # element 32i + (k | 16 + k)
    q = sub.transpose(0, 3, 1, 2, 4).reshape(groups * 64, cols)[:rows]
    m = meta.transpose(0, 2, 1, 3).reshape(groups * 64, G, 16)[:rows].astype(np.uint64)
    d = (m[..., 0] | (m[..., 1] << 8)).astype(np.uint16)
    dmin = (m[..., 2] | (m[..., 3] << 8)).astype(np.uint16)
    sc = np.zeros((rows, G, 8), np.uint8)
    mn = np.zeros((rows, G, 8), np.uint8)
    for r in range(rows):
        for b in range(G):
            bits = int.from_bytes(bytes(m[r, b, 4:16].astype(np.uint8)), "little")
            for j in range(8):
                field = (bits >> (12 * j)) & 0xFFF
                sc[r, b, j] = field & 63
                mn[r, b, j] = field >> 6
    return {"q": q, "sc": sc.reshape(rows, G * 8), "mn": mn.reshape(rows, G * 8), "d": d, "dmin": dmin}


def unpack_q6k(img: np.ndarray, rows: int, cols: int) -> dict:
    t, G, groups = _tiles(img, rows, cols, 13440)
    ql = t[..., :8192].reshape(groups, G, 8, 64, 16)
    qh = t[..., 8192:12288].reshape(groups, G, 4, 64, 16)
    sc = t[..., 12288:13312].reshape(groups, G, 64, 16).view(np.int8)
    d = t[..., 13312:13440].reshape(groups, G, 64, 2).astype(np.uint16)
    low = np.concatenate([ql & 15, ql >> 4], axis=4)             # [g, b, i, lane, 32]
    low = low.transpose(0, 1, 3, 2, 4).reshape(groups, G, 64, 256)
    high = np.zeros((groups, G, 64, 256), np.uint8)
    for h in range(4):
        for f in range(4):
            high[..., 64 * h + 16 * f:64 * h + 16 * f + 16] = (qh[:, :, h] >> (2 * f)) & 3
    q = (low | (high << 4)).transpose(0, 2, 1, 3).reshape(groups * 64, cols)[:rows]
    dd = (d[..., 0] | (d[..., 1] << 8)).transpose(0, 2, 1).reshape(groups * 64, G)[:rows]
    scs = sc.transpose(0, 2, 1, 3).reshape(groups * 64, G * 16)[:rows]
    return {"q": q, "sc": scs, "d": dd}


def unpack_b32(img: np.ndarray, q8: bool, rows: int, cols: int) -> dict:
    """Q8_0-style (q8): sixteen chunks of 16 int8 codes (elements 16i..16i+15) then the eight
    f16 scales; Q4_0-style: eight nibble-split chunks (one 32-element block each) then the
    scales."""
    tb = 17408 if q8 else 9216
    t, G, groups = _tiles(img, rows, cols, tb)
    if q8:
        codes = t[..., :16384].reshape(groups, G, 16, 64, 16).transpose(0, 1, 3, 2, 4).reshape(groups, G, 64, 256)
        dpart = t[..., 16384:]
    else:
        ch = t[..., :8192].reshape(groups, G, 8, 64, 16)
        codes = np.concatenate([ch & 15, ch >> 4], axis=4).transpose(0, 1, 3, 2, 4).reshape(groups, G, 64, 256)
        dpart = t[..., 8192:]
    q = codes.transpose(0, 2, 1, 3).reshape(groups * 64, cols)[:rows]
    if q8:
        q = q.view(np.int8)
    dp = dpart.reshape(groups, G, 64, 8, 2).astype(np.uint16)
    d = (dp[..., 0] | (dp[..., 1] << 8)).transpose(0, 2, 1, 3).reshape(groups * 64, G * 8)[:rows]
    return {"q": q, "d": d}
