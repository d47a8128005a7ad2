// pack.cpp -- host-side weight-image packer (the tile layouts are documented in qgemv.h).
//
// The pages store a weight as "a scale times an integer" with the codes and scales kept as
// stored ("Module numerics" of logicaffeine_compile::spatial::decode_engine, Structs
// CodedRow, Segment, Scale, Unreadable).  The packer only rearranges those fields into
// tiles of 64 rows x one block so that every GPU load is a contiguous 1 KiB per wave; it
// validates every field and refuses a block whose scale is inf or NaN.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "qg_internal.hpp"

namespace qg {
namespace {

bool f16_unreadable(uint16_t h) { return ((h >> 10) & 31) == 31; }

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" size_t qg_image_bytes(int fmt, int64_t rows, int64_t cols)
{
    if ((fmt < QG_Q4K || fmt > QG_Q4_0) || rows < 0 || cols <= 0 || cols % QG_BLOCK) return 0;
    const int64_t groups = (rows + kTileRows - 1) / kTileRows;
    const int64_t tiles = groups * (cols / QG_BLOCK);
    const int tb = fmt == QG_Q4K ? kTileBytesQ4K : fmt == QG_Q6K ? kTileBytesQ6K : fmt == QG_Q8_0 ? kTileBytesQ8_0
                                                                                                 : kTileBytesQ4_0;
    return (size_t)tiles * (size_t)tb;
}

extern "C" int qg_pack_q4k(int64_t rows, int64_t cols, const uint8_t *q, const uint8_t *sc, const uint8_t *mn,
                           const uint16_t *d, const uint16_t *dmin, void *image_host)
{
    if (rows < 0 || cols <= 0 || cols % QG_BLOCK)
        return fail(QG_E_SHAPE, "qg_pack_q4k: cols %lld is not a positive multiple of 256", (long long)cols);
    if (rows > 0 && (!q || !sc || !mn || !d || !dmin || !image_host))
        return fail(QG_E_INVALID, "qg_pack_q4k: null pointer");
    const int64_t G = cols / QG_BLOCK;
    // validate everything before writing anything
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < G; b++) {
            if (f16_unreadable(d[r * G + b]) || f16_unreadable(dmin[r * G + b]))
                return fail(QG_E_UNREADABLE, "qg_pack_q4k: row %lld block %lld has an inf/NaN scale",
                            (long long)r, (long long)b);
        }
        for (int64_t i = 0; i < cols; i++)
            if (q[r * cols + i] > 15)
                return fail(QG_E_INVALID, "qg_pack_q4k: code %u at row %lld col %lld exceeds 15",
                            q[r * cols + i], (long long)r, (long long)i);
        for (int64_t j = 0; j < cols / 32; j++)
            if (sc[r * (cols / 32) + j] > 63 || mn[r * (cols / 32) + j] > 63)
                return fail(QG_E_INVALID, "qg_pack_q4k: sub-scale/offset above 63 at row %lld sub-block %lld",
                            (long long)r, (long long)j);
    }
    const size_t bytes = qg_image_bytes(QG_Q4K, rows, cols);
    uint8_t *img = static_cast<uint8_t *>(image_host);
    memset(img, 0, bytes);
    for (int64_t r = 0; r < rows; r++) for (int64_t b = 0; b < G; b++) {
        uint8_t *tile = img + ((r / kTileRows) * G + b) * kTileBytesQ4K;
        const int l = (int)(r % kTileRows);
        const uint8_t *qb = q + r * cols + b * QG_BLOCK;
        for (int i = 0; i < 8; i++) {
            uint8_t *dst = tile + 1024 * i + 16 * l;
            for (int k = 0; k < 16; k++)
                dst[k] = (uint8_t)(qb[32 * i + k] | (qb[32 * i + 16 + k] << 4));
        }
        uint8_t *meta = tile + 8192 + 16 * l;
        const uint16_t dv = d[r * G + b], mv = dmin[r * G + b];
        meta[0] = (uint8_t)(dv & 0xFF);
        meta[1] = (uint8_t)(dv >> 8);
        meta[2] = (uint8_t)(mv & 0xFF);
        meta[3] = (uint8_t)(mv >> 8);
        // 96-bit little-endian field string: sub-block j at bits 12j (sc) and 12j+6 (mn)
        uint8_t bitsbuf[12] = {0};
        for (int j = 0; j < 8; j++) {
            const uint32_t field = (uint32_t)sc[r * (cols / 32) + b * 8 + j] | ((uint32_t)mn[r * (cols / 32) + b * 8 + j] << 6);
            for (int t = 0; t < 12; t++)
                if ((field >> t) & 1u) {
                    const int bit = 12 * j + t;
                    bitsbuf[bit >> 3] |= (uint8_t)(1u << (bit & 7));
                }
        }
        memcpy(meta + 4, bitsbuf, 12);
    }
    return QG_OK;
}

extern "C" int qg_pack_q6k(int64_t rows, int64_t cols, const uint8_t *q, const int8_t *sc, const uint16_t *d,
                           void *image_host)
{
    if (rows < 0 || cols <= 0 || cols % QG_BLOCK)
        return fail(QG_E_SHAPE, "qg_pack_q6k: cols %lld is not a positive multiple of 256", (long long)cols);
    if (rows > 0 && (!q || !sc || !d || !image_host)) return fail(QG_E_INVALID, "qg_pack_q6k: null pointer");
    const int64_t G = cols / QG_BLOCK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < G; b++)
            if (f16_unreadable(d[r * G + b]))
                return fail(QG_E_UNREADABLE, "qg_pack_q6k: row %lld block %lld has an inf/NaN scale",
                            (long long)r, (long long)b);
        for (int64_t i = 0; i < cols; i++)
            if (q[r * cols + i] > 63)
                return fail(QG_E_INVALID, "qg_pack_q6k: code %u at row %lld col %lld exceeds 63",
                            q[r * cols + i], (long long)r, (long long)i);
    }
    const size_t bytes = qg_image_bytes(QG_Q6K, rows, cols);
    uint8_t *img = static_cast<uint8_t *>(image_host);
    memset(img, 0, bytes);
    for (int64_t r = 0; r < rows; r++) for (int64_t b = 0; b < G; b++) {
        uint8_t *tile = img + ((r / kTileRows) * G + b) * kTileBytesQ6K;
        const int l = (int)(r % kTileRows);
        const uint8_t *qb = q + r * cols + b * QG_BLOCK;
        for (int i = 0; i < 8; i++) {
            uint8_t *dst = tile + 1024 * i + 16 * l;
            for (int k = 0; k < 16; k++)
                dst[k] = (uint8_t)((qb[32 * i + k] & 15) | ((qb[32 * i + 16 + k] & 15) << 4));
        }
        for (int h = 0; h < 4; h++) {
            uint8_t *dst = tile + 8192 + 1024 * h + 16 * l;
            for (int k = 0; k < 16; k++) {
                uint8_t v = 0;
                for (int f = 0; f < 4; f++) v |= (uint8_t)(((qb[64 * h + 16 * f + k] >> 4) & 3) << (2 * f));
                dst[k] = v;
            }
        }
        memcpy(tile + 12288 + 16 * l, sc + r * (cols / 16) + b * 16, 16);
        const uint16_t dv = d[r * G + b];
        tile[13312 + 2 * l] = (uint8_t)(dv & 0xFF);
        tile[13312 + 2 * l + 1] = (uint8_t)(dv >> 8);
    }
    return QG_OK;
}

extern "C" int qg_pack_b32(int fmt, int64_t rows, int64_t cols, const void *q_host, const uint16_t *d_host,
                           void *image_host)
{
    if (fmt != QG_Q8_0 && fmt != QG_Q4_0) return fail(QG_E_INVALID, "qg_pack_b32: format %d has no 32-element blocks", fmt);
    if (rows < 0 || cols <= 0 || cols % QG_BLOCK)
        return fail(QG_E_SHAPE, "qg_pack_b32: cols %lld is not a positive multiple of 256", (long long)cols);
    if (rows > 0 && (!q_host || !d_host || !image_host)) return fail(QG_E_INVALID, "qg_pack_b32: null pointer");
    const uint8_t *q = static_cast<const uint8_t *>(q_host);
    const int64_t G = cols / QG_BLOCK, nb = cols / 32;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < nb; j++)
            if (f16_unreadable(d_host[r * nb + j]))
                return fail(QG_E_UNREADABLE, "qg_pack_b32: row %lld block %lld has an inf/NaN scale", (long long)r,
                            (long long)j);
        if (fmt == QG_Q4_0)
            for (int64_t i = 0; i < cols; i++)
                if (q[r * cols + i] > 15)
                    return fail(QG_E_INVALID, "qg_pack_b32: code %u at row %lld col %lld exceeds 15", q[r * cols + i],
                                (long long)r, (long long)i);
    }
    const int tb = fmt == QG_Q8_0 ? kTileBytesQ8_0 : kTileBytesQ4_0;
    const int doff = fmt == QG_Q8_0 ? 16384 : 8192;
    uint8_t *img = static_cast<uint8_t *>(image_host);
    memset(img, 0, qg_image_bytes(fmt, rows, cols));
    for (int64_t r = 0; r < rows; r++) for (int64_t b = 0; b < G; b++) {
        uint8_t *tile = img + ((r / kTileRows) * G + b) * tb;
        const int l = (int)(r % kTileRows);
        const uint8_t *qb = q + r * cols + b * QG_BLOCK;
        if (fmt == QG_Q8_0) {
            for (int i = 0; i < 16; i++) memcpy(tile + 1024 * i + 16 * l, qb + 16 * i, 16);
        } else {
            for (int i = 0; i < 8; i++) {
                uint8_t *dst = tile + 1024 * i + 16 * l;
                for (int k = 0; k < 16; k++) dst[k] = (uint8_t)(qb[32 * i + k] | (qb[32 * i + 16 + k] << 4));
            }
        }
        uint8_t *dd = tile + doff + 16 * l;
        for (int j = 0; j < 8; j++) {
            const uint16_t dv = d_host[r * nb + b * 8 + j];
            dd[2 * j] = (uint8_t)(dv & 0xFF);
            dd[2 * j + 1] = (uint8_t)(dv >> 8);
        }
    }
    return QG_OK;
}
