// abi.cpp -- the extern "C" entry points: argument validation, reasons, launches.
//
// Refusals happen before any work, each with a reason naming what was wrong (the pages'
// convention of refusing up front with a reason: bankML forward.md, "Technical usage",
// plan; "Module numerics", Structs Unreadable and Functions reads).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "qg_internal.hpp"

namespace qg {

namespace {
thread_local char g_reason[512] = "";
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;
thread_local Tuning g_tuning = {};   // per thread, as the reason string

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];
}  // namespace

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_reason, sizeof g_reason, fmt, ap);
    va_end(ap);
    return status;
}

const Tuning &tuning() { return g_tuning; }

void take_timing_events(hipEvent_t *start, hipEvent_t *stop)
{
    *start = g_ev_start;
    *stop = g_ev_stop;
    g_ev_start = g_ev_stop = nullptr;
}

int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::call_once(g_cu_once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cu_count[dev] = n;
    });
    return g_cu_count[dev];
}

}  // namespace qg

using namespace qg;

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_fmt_mode(const char *who, int fmt, int mode)
{
    if (fmt < QG_Q4K || fmt > QG_Q4_0) return fail(QG_E_INVALID, "%s: unknown format %d", who, fmt);
    if (mode != QG_PERBLOCK && mode != QG_SUB32) return fail(QG_E_INVALID, "%s: unknown scaling %d", who, mode);
    if (!qg_reads(fmt, mode)) return fail(QG_E_UNSUPPORTED, "%s: format %d is not read under scaling %d", who, fmt, mode);
    return QG_OK;
}

int check_cols(const char *who, int64_t cols)
{
    if (cols <= 0 || cols % QG_BLOCK)
        return fail(QG_E_SHAPE, "%s: cols %lld is not a positive multiple of %d", who, (long long)cols, QG_BLOCK);
    if (cols > QG_MAX_COLS) return fail(QG_E_SHAPE, "%s: cols %lld exceeds %d", who, (long long)cols, QG_MAX_COLS);
    return QG_OK;
}

int check_ptr(const char *who, const char *name, const void *p, uintptr_t align)
{
    if (!p) return fail(QG_E_INVALID, "%s: %s is NULL", who, name);
    if (!aligned(p, align)) return fail(QG_E_INVALID, "%s: %s is not %u-byte aligned", who, name, (unsigned)align);
    return QG_OK;
}

// head size and head counts of the KV-cache calls
int check_kv(const char *who, int64_t nh, int64_t nkv, int64_t npos, int64_t hd)
{
    if (hd != 32 && hd != 64 && hd != 128 && hd != 256)
        return fail(QG_E_SHAPE, "%s: head size %lld is not 32, 64, 128 or 256", who, (long long)hd);
    if (nkv < 1 || nh < 0 || nh % nkv)
        return fail(QG_E_SHAPE, "%s: %lld heads do not share %lld KV heads evenly", who, (long long)nh, (long long)nkv);
    if (nh > 65535) return fail(QG_E_SHAPE, "%s: %lld heads exceed 65535", who, (long long)nh);
    if (npos < 0 || npos > ((int64_t)1 << 31) / hd)
        return fail(QG_E_SHAPE, "%s: %lld positions out of range", who, (long long)npos);
    return QG_OK;
}

int check_act(const char *who, const int8_t *codes, const qg_act_scale *scales, const int32_t *csums)
{
    int st;
    if ((st = check_ptr(who, "codes", codes, 16))) return st;
    if ((st = check_ptr(who, "scales", scales, 4))) return st;
    if ((st = check_ptr(who, "csums", csums, 4))) return st;
    return QG_OK;
}

}  // namespace

extern "C" {

int qg_version(void) { return 100; }

const char *qg_last_error(void) { return g_reason; }

int qg_reads(int fmt, int mode)
{
    const bool f = fmt == QG_Q4K || fmt == QG_Q6K || fmt == QG_Q8_0 || fmt == QG_Q4_0;
    const bool m = mode == QG_PERBLOCK || mode == QG_SUB32;
    return f && m ? 1 : 0;
}

int qg_set_tuning(int key, int64_t value)
{
    if (value < 0) return fail(QG_E_INVALID, "qg_set_tuning: negative value");
    switch (key) {
    case QG_TUNE_WAVES_PER_WG:
        if (value != 0 && value != 4 && value != 8 && value != 16)
            return fail(QG_E_INVALID, "qg_set_tuning: waves per workgroup must be 0, 4, 8 or 16");
        g_tuning.waves_per_wg = (int)value;
        return QG_OK;
    case QG_TUNE_MFMA_MIN_COLS:
        g_tuning.mfma_min_cols = value > 65536 ? 65536 : (int)value;
        return QG_OK;
    case QG_TUNE_MFMA_COL_TILES:
        if (value != 0 && value != 1 && value != 2 && value != 4)
            return fail(QG_E_INVALID, "qg_set_tuning: column tiles must be 0, 1, 2 or 4");
        g_tuning.mfma_col_tiles = (int)value;
        return QG_OK;
    case QG_TUNE_MFMA_FORM:
        if (value > 4) return fail(QG_E_INVALID, "qg_set_tuning: form must be 0, 1, 2, 3 or 4");
        g_tuning.mfma_form = (int)value;
        return QG_OK;
    case QG_TUNE_COLS_KERNEL:
        if (value > 1) return fail(QG_E_INVALID, "qg_set_tuning: the several-column kernel choice must be 0 or 1");
        g_tuning.cols_off = (int)value;
        return QG_OK;
    case QG_TUNE_MFMA_TABLES:
        if (value > 1) return fail(QG_E_INVALID, "qg_set_tuning: the scale tables choice must be 0 or 1");
        g_tuning.mfma_pre_off = (int)value;
        return QG_OK;
    case QG_TUNE_GEMM_ROW_TILES:
        if (value != 0 && value != 1 && value != 2 && value != 4)
            return fail(QG_E_INVALID, "qg_set_tuning: row tiles must be 0, 1, 2 or 4");
        g_tuning.gemm_row_tiles = (int)value;
        return QG_OK;
    case QG_TUNE_GEMV_QUARTER:
        if (value > 2) return fail(QG_E_INVALID, "qg_set_tuning: the 16-row GEMV choice must be 0, 1 or 2");
        g_tuning.gemv_quarter = (int)value;
        return QG_OK;
    default:
        return fail(QG_E_INVALID, "qg_set_tuning: unknown key %d", key);
    }
}

int qg_time_next_launch(void *start_event, void *stop_event)
{
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(QG_E_INVALID, "qg_time_next_launch: give both events or neither");
    g_ev_start = static_cast<hipEvent_t>(start_event);
    g_ev_stop = static_cast<hipEvent_t>(stop_event);
    return QG_OK;
}

int qg_quantize_act(int fmt, int mode, int64_t n, int64_t cols, const float *x, int8_t *codes,
                    qg_act_scale *scales, int32_t *csums, int32_t *err_flag, void *stream)
{
    const char *who = "qg_quantize_act";
    int st;
    if ((st = check_fmt_mode(who, fmt, mode))) return st;
    if ((st = check_cols(who, cols))) return st;
    if (n < 0 || n > (int64_t)1 << 24) return fail(QG_E_SHAPE, "%s: n %lld out of range", who, (long long)n);
    if (n == 0) return QG_OK;
    if ((st = check_ptr(who, "x", x, 16))) return st;
    if ((st = check_act(who, codes, scales, csums))) return st;
    if (err_flag && !aligned(err_flag, 4)) return fail(QG_E_INVALID, "%s: err_flag is not 4-byte aligned", who);
    return launch_quantize(mode, act_block(fmt, mode), n, cols, x, codes, scales, csums, err_flag,
                           static_cast<hipStream_t>(stream));
}

static int gemm_common(const char *who, int fmt, int mode, int64_t rows, int64_t cols, int64_t n,
                       const void *image, const int8_t *codes, const qg_act_scale *scales,
                       const int32_t *csums, float *out, void *stream)
{
    int st;
    if ((st = check_fmt_mode(who, fmt, mode))) return st;
    if ((st = check_cols(who, cols))) return st;
    if (rows < 0 || rows > 0x7fffffff) return fail(QG_E_SHAPE, "%s: rows %lld out of range", who, (long long)rows);
    if (n < 0 || n > 65535) return fail(QG_E_SHAPE, "%s: n %lld out of range", who, (long long)n);
    if (rows == 0 || n == 0) return QG_OK;
    if ((st = check_ptr(who, "image", image, 16))) return st;
    if ((st = check_act(who, codes, scales, csums))) return st;
    if ((st = check_ptr(who, "out", out, 4))) return st;
    // the matrix cores from 2 columns on fewer than 8192 rows, from 5 on more (below that the
    // one-column machinery's workgroups already fill the chip and it is faster)
    const int min_cols = g_tuning.mfma_min_cols > 0 ? g_tuning.mfma_min_cols : rows < 8192 ? 2 : 5;
    if (fmt == QG_Q4K && mode == QG_PERBLOCK && n >= min_cols)
        return launch_gemm_mfma(rows, cols, n, image, codes, scales, out, static_cast<hipStream_t>(stream));
    return launch_gemv(fmt, mode, rows, cols, n, image, codes, scales, csums, out, static_cast<hipStream_t>(stream));
}

int qg_gemv_q(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const int8_t *codes,
              const qg_act_scale *scales, const int32_t *csums, float *out, void *stream)
{
    return gemm_common("qg_gemv_q", fmt, mode, rows, cols, 1, image, codes, scales, csums, out, stream);
}

int qg_gemm_q(int fmt, int mode, int64_t rows, int64_t cols, int64_t n, const void *image, const int8_t *codes,
              const qg_act_scale *scales, const int32_t *csums, float *out, void *stream)
{
    return gemm_common("qg_gemm_q", fmt, mode, rows, cols, n, image, codes, scales, csums, out, stream);
}

static int quantize_gemv_common(const char *who, int fmt, int mode, int64_t rows, int64_t cols, const void *image,
                                const float *x, int8_t *codes, qg_act_scale *scales, int32_t *csums,
                                int32_t *err_flag, float *out, uint64_t *argmax_key, void *stream)
{
    int st;
    if ((st = check_fmt_mode(who, fmt, mode))) return st;
    if ((st = check_cols(who, cols))) return st;
    if (rows < 0 || rows > 0x7fffffff) return fail(QG_E_SHAPE, "%s: rows %lld out of range", who, (long long)rows);
    if ((st = check_ptr(who, "x", x, 16))) return st;
    if ((st = check_act(who, codes, scales, csums))) return st;
    if (err_flag && !aligned(err_flag, 4)) return fail(QG_E_INVALID, "%s: err_flag is not 4-byte aligned", who);
    if (rows > 0) {
        if ((st = check_ptr(who, "image", image, 16))) return st;
        if ((st = check_ptr(who, "out", out, 4))) return st;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (rows > 0)
        return launch_gemv_fused(fmt, mode, rows, cols, image, x, codes, scales, csums, err_flag, out,
                                 reinterpret_cast<unsigned long long *>(argmax_key), s);
    // no rows to multiply: only the quantized row
    return launch_quantize(mode, act_block(fmt, mode), 1, cols, x, codes, scales, csums, err_flag, s);
}

int qg_quantize_gemv(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const float *x,
                     int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag, float *out,
                     void *stream)
{
    return quantize_gemv_common("qg_quantize_gemv", fmt, mode, rows, cols, image, x, codes, scales, csums, err_flag,
                                out, nullptr, stream);
}

int qg_quantize_gemv_argmax(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const float *x,
                            int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag, float *out,
                            uint64_t *argmax_key, void *stream)
{
    const char *who = "qg_quantize_gemv_argmax";
    int st;
    if ((st = check_ptr(who, "argmax_key", argmax_key, 8))) return st;
    return quantize_gemv_common(who, fmt, mode, rows, cols, image, x, codes, scales, csums, err_flag, out, argmax_key,
                                stream);
}

int64_t qg_argmax_index(uint64_t key) { return key == 0 ? 0 : (int64_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu)); }

static int check_multi(const char *who, int fmt, int mode, int nmat, const int64_t *rows, int64_t cols,
                       const void *const *images, float *const *outs)
{
    int st;
    if ((st = check_fmt_mode(who, fmt, mode))) return st;
    if ((st = check_cols(who, cols))) return st;
    if (nmat < 1 || nmat > QG_MAX_MATRICES)
        return fail(QG_E_SHAPE, "%s: nmat %d is not in 1..%d", who, nmat, QG_MAX_MATRICES);
    if (!rows || !images || !outs) return fail(QG_E_INVALID, "%s: rows, images or outs is NULL", who);
    for (int m = 0; m < nmat; m++) {
        if (rows[m] < 0 || rows[m] > 0x7fffffff)
            return fail(QG_E_SHAPE, "%s: rows[%d] = %lld out of range", who, m, (long long)rows[m]);
        if (rows[m] == 0) continue;
        if (!images[m] || !aligned(images[m], 16)) return fail(QG_E_INVALID, "%s: images[%d] is NULL or not 16-byte aligned", who, m);
        if (!outs[m] || !aligned(outs[m], 4)) return fail(QG_E_INVALID, "%s: outs[%d] is NULL or not 4-byte aligned", who, m);
    }
    return QG_OK;
}

int qg_quantize_gemv_multi(int fmt, int mode, int nmat, const int64_t *rows, int64_t cols, const void *const *images,
                           const float *x, int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag,
                           float *const *outs, void *stream)
{
    const char *who = "qg_quantize_gemv_multi";
    int st;
    if ((st = check_multi(who, fmt, mode, nmat, rows, cols, images, outs))) return st;
    if ((st = check_ptr(who, "x", x, 16))) return st;
    if ((st = check_act(who, codes, scales, csums))) return st;
    if (err_flag && !aligned(err_flag, 4)) return fail(QG_E_INVALID, "%s: err_flag is not 4-byte aligned", who);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t total = 0;
    for (int m = 0; m < nmat; m++) total += rows[m];
    if (total == 0) return launch_quantize(mode, act_block(fmt, mode), 1, cols, x, codes, scales, csums, err_flag, s);
    // the quantized row is written by the launch's first workgroup, which belongs to the
    // first matrix with rows
    return launch_gemv_multi(fmt, mode, nmat, rows, cols, images, x, nullptr, nullptr, codes, scales, csums, err_flag,
                             outs, s);
}

int qg_gemv_q_multi(int fmt, int mode, int nmat, const int64_t *rows, int64_t cols, const void *const *images,
                    const int8_t *codes, const qg_act_scale *scales, const int32_t *csums, float *const *outs,
                    void *stream)
{
    const char *who = "qg_gemv_q_multi";
    int st;
    if ((st = check_multi(who, fmt, mode, nmat, rows, cols, images, outs))) return st;
    if ((st = check_act(who, codes, scales, csums))) return st;
    return launch_gemv_multi(fmt, mode, nmat, rows, cols, images, nullptr, codes, scales, nullptr, nullptr, nullptr,
                             nullptr, outs, static_cast<hipStream_t>(stream));
}

int qg_stream_read(const void *buf, size_t bytes, uint32_t magic, uint32_t *sink, void *stream)
{
    const char *who = "qg_stream_read";
    int st;
    if (bytes < 1024) return QG_OK;
    if ((st = check_ptr(who, "buf", buf, 16))) return st;
    if ((st = check_ptr(who, "sink", sink, 4))) return st;
    return launch_stream_read(buf, bytes, magic, sink, static_cast<hipStream_t>(stream));
}

int qg_stream_read_shape(const void *buf, size_t bytes, int waves_per_wg, int kib_per_wave, int64_t wgs, int flags,
                         uint32_t magic, uint32_t *sink, void *stream)
{
    const char *who = "qg_stream_read_shape";
    int st;
    if (waves_per_wg != 1 && waves_per_wg != 2 && waves_per_wg != 4 && waves_per_wg != 8 && waves_per_wg != 16)
        return fail(QG_E_INVALID, "%s: %d waves per workgroup is not one of 1, 2, 4, 8, 16", who, waves_per_wg);
    if (kib_per_wave != 1 && kib_per_wave != 2 && kib_per_wave != 4 && kib_per_wave != 8 && kib_per_wave != 9 &&
        kib_per_wave != 16)
        return fail(QG_E_INVALID, "%s: %d KiB per wave is not one of 1, 2, 4, 8, 9, 16", who, kib_per_wave);
    if (wgs < 0 || wgs > 0x7fffffff) return fail(QG_E_INVALID, "%s: workgroup count %lld", who, (long long)wgs);
    if (flags & ~1) return fail(QG_E_INVALID, "%s: unknown flags 0x%x", who, flags);
    if (bytes < 1024) return QG_OK;
    if ((st = check_ptr(who, "buf", buf, 16))) return st;
    if ((st = check_ptr(who, "sink", sink, 4))) return st;
    return launch_stream_read_shape(buf, bytes, waves_per_wg, kib_per_wave, wgs, flags, magic, sink,
                                    static_cast<hipStream_t>(stream));
}

int qg_kv_cache_rows(int64_t n, int64_t hd, const float *x, uint16_t *scales, int8_t *codes, void *stream)
{
    const char *who = "qg_kv_cache_rows";
    int st;
    if ((st = check_kv(who, 0, 1, 0, hd))) return st;
    if (n < 0 || n > 0x7fffffffLL * 4) return fail(QG_E_SHAPE, "%s: %lld rows out of range", who, (long long)n);
    if (n == 0) return QG_OK;
    if ((st = check_ptr(who, "x", x, 4))) return st;
    if ((st = check_ptr(who, "scales", scales, 2))) return st;
    if ((st = check_ptr(who, "codes", codes, 4))) return st;
    return launch_kv_cache_rows(n, hd, x, scales, codes, static_cast<hipStream_t>(stream));
}

int qg_kv_quantize_heads(int mode, int64_t nh, int64_t hd, const float *q, int8_t *codes, qg_act_scale *scales,
                         int32_t *err_flag, void *stream)
{
    const char *who = "qg_kv_quantize_heads";
    int st;
    if (mode != QG_PERBLOCK && mode != QG_SUB32) return fail(QG_E_INVALID, "%s: unknown scaling %d", who, mode);
    if ((st = check_kv(who, nh, 1, 0, hd))) return st;
    if (nh == 0) return QG_OK;
    if ((st = check_ptr(who, "q", q, 16))) return st;
    if ((st = check_ptr(who, "codes", codes, 4))) return st;
    if ((st = check_ptr(who, "scales", scales, 4))) return st;
    if (err_flag && (st = check_ptr(who, "err_flag", err_flag, 4))) return st;
    return launch_kv_quantize_heads(mode, nh, hd, q, codes, scales, err_flag, static_cast<hipStream_t>(stream));
}

int qg_kv_scores(int mode, int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const int8_t *qcodes,
                 const qg_act_scale *qscales, const uint16_t *kscales, const int8_t *kcodes, float *out, void *stream)
{
    const char *who = "qg_kv_scores";
    int st;
    if (mode != QG_PERBLOCK && mode != QG_SUB32) return fail(QG_E_INVALID, "%s: unknown scaling %d", who, mode);
    if ((st = check_kv(who, nh, nkv, npos, hd))) return st;
    if (nh == 0 || npos == 0) return QG_OK;
    if ((st = check_ptr(who, "qcodes", qcodes, 4))) return st;
    if ((st = check_ptr(who, "qscales", qscales, 4))) return st;
    if ((st = check_ptr(who, "kscales", kscales, 2))) return st;
    if ((st = check_ptr(who, "kcodes", kcodes, 16))) return st;
    if ((st = check_ptr(who, "out", out, 4))) return st;
    return launch_kv_scores(mode, nh, nkv, npos, hd, qcodes, qscales, kscales, kcodes, out,
                            static_cast<hipStream_t>(stream));
}

int qg_kv_weighted(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs, const uint16_t *vscales,
                   const int8_t *vcodes, float *out, void *stream)
{
    const char *who = "qg_kv_weighted";
    int st;
    if ((st = check_kv(who, nh, nkv, npos, hd))) return st;
    if (nh == 0) return QG_OK;
    if ((st = check_ptr(who, "out", out, 4))) return st;
    if (npos > 0) {
        if ((st = check_ptr(who, "probs", probs, 4))) return st;
        if ((st = check_ptr(who, "vscales", vscales, 2))) return st;
        if ((st = check_ptr(who, "vcodes", vcodes, 4))) return st;
    }
    return launch_kv_weighted(nh, nkv, npos, hd, probs, vscales, vcodes, out, static_cast<hipStream_t>(stream));
}

int qg_kv_weighted_workspace(int64_t nh, int64_t npos, int64_t hd, size_t *bytes)
{
    const char *who = "qg_kv_weighted_workspace";
    int st;
    if ((st = check_kv(who, nh, 1, npos, hd))) return st;
    if (bytes == nullptr) return fail(QG_E_INVALID, "%s: bytes is null", who);
    *bytes = kv_weighted_workspace_bytes(nh, npos, hd);
    return QG_OK;
}

int qg_kv_weighted_with_workspace(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                                  const uint16_t *vscales, const int8_t *vcodes, float *out, void *workspace,
                                  size_t ws_bytes, void *stream)
{
    const char *who = "qg_kv_weighted_with_workspace";
    int st;
    if ((st = check_kv(who, nh, nkv, npos, hd))) return st;
    if (nh == 0) return QG_OK;
    if ((st = check_ptr(who, "out", out, 4))) return st;
    const size_t need = kv_weighted_workspace_bytes(nh, npos, hd);
    if (ws_bytes < need)
        return fail(QG_E_INVALID, "%s: workspace of %zu bytes, %zu needed", who, ws_bytes, need);
    if (npos > 0) {
        if ((st = check_ptr(who, "probs", probs, 4))) return st;
        if ((st = check_ptr(who, "vscales", vscales, 2))) return st;
        if ((st = check_ptr(who, "vcodes", vcodes, 4))) return st;
        if ((st = check_ptr(who, "workspace", workspace, 16))) return st;
    }
    return launch_kv_weighted_two_pass(nh, nkv, npos, hd, probs, vscales, vcodes, static_cast<float *>(workspace),
                                       out, static_cast<hipStream_t>(stream));
}

int qg_kv_weighted_noalloc(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                           const uint16_t *vscales, const int8_t *vcodes, float *out, void *stream)
{
    const char *who = "qg_kv_weighted_noalloc";
    int st;
    if ((st = check_kv(who, nh, nkv, npos, hd))) return st;
    if (nh == 0) return QG_OK;
    const size_t need = kv_weighted_workspace_bytes(nh, npos, hd);
    if (need > QG_KV_NOALLOC_BYTES)
        return fail(QG_E_SHAPE, "%s: the pieces need %zu bytes, the fixed workspace holds %zu", who, need,
                    (size_t)QG_KV_NOALLOC_BYTES);
    if ((st = check_ptr(who, "out", out, 4))) return st;
    if (npos > 0) {
        if ((st = check_ptr(who, "probs", probs, 4))) return st;
        if ((st = check_ptr(who, "vscales", vscales, 2))) return st;
        if ((st = check_ptr(who, "vcodes", vcodes, 4))) return st;
    }
    return launch_kv_weighted_noalloc(nh, nkv, npos, hd, probs, vscales, vcodes, out, static_cast<hipStream_t>(stream));
}

int qg_block_sums(int fmt, int64_t rows, int64_t cols, const void *image, const int8_t *codes,
                  int32_t *csum_out, int32_t *osum_out, void *stream)
{
    const char *who = "qg_block_sums";
    int st;
    if (fmt < QG_Q4K || fmt > QG_Q4_0) return fail(QG_E_INVALID, "%s: unknown format %d", who, fmt);
    if (is_b32(fmt)) return fail(QG_E_UNSUPPORTED, "%s: no sub-block sums view for format %d", who, fmt);
    if ((st = check_cols(who, cols))) return st;
    if (rows < 0 || rows > 0x7fffffff) return fail(QG_E_SHAPE, "%s: rows %lld out of range", who, (long long)rows);
    if (rows == 0) return QG_OK;
    if ((st = check_ptr(who, "image", image, 16))) return st;
    if ((st = check_ptr(who, "codes", codes, 16))) return st;
    if ((st = check_ptr(who, "csum_out", csum_out, 4))) return st;
    if (fmt == QG_Q4K && (st = check_ptr(who, "osum_out", osum_out, 4))) return st;
    return launch_block_sums(fmt, rows, cols, image, codes, csum_out, osum_out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
