// qg_internal.hpp -- host-side internals shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

// image tile geometry (see the layout in qgemv.h)
constexpr int kTileRows = 64;     // rows per tile (one 256-element block each)
constexpr int kTileBytesQ4K = 64 * 144;   // 9216
constexpr int kTileBytesQ6K = 64 * 210;   // 13440
constexpr int kTileBytesQ8_0 = 64 * 272;  // 17408
constexpr int kTileBytesQ4_0 = 64 * 144;  // 9216

// formats with 32-element weight blocks (PerBlock activation blocks of 32 too)
constexpr bool is_b32(int fmt) { return fmt == QG_Q8_0 || fmt == QG_Q4_0; }
// elements per activation scale for (format, scaling)
constexpr int act_block(int fmt, int mode) { return (mode == QG_SUB32 || is_b32(fmt)) ? 32 : 256; }

// per-thread failure reason
int fail(int status, const char *fmt, ...);

struct Tuning {
    int waves_per_wg;     // waves per GEMV workgroup (4, 8, 16); 0 = derived from the block count
    int mfma_min_cols;    // columns from which a Q4_K PerBlock GEMM uses the matrix cores; 0 = derived
    int mfma_col_tiles;   // matrix-core GEMM (shared, split): 1, 2 or 4 column tiles per workgroup; 0 = derived
    int mfma_form;        // matrix-core GEMM: 1 staged, 2 shared operands, 3 split; 0 = derived
    int cols_off;         // 1: several columns take the LDS-staged kernel, not the one-column machinery
    int mfma_pre_off;     // 1: the shared-operand GEMM loads its scales per block, not into tables
    int gemm_row_tiles;   // staged and split matrix-core GEMM: 16-row tiles per workgroup (1, 2, 4); 0 = derived
    int gemv_quarter;     // one-column Q4_K PerBlock GEMV: 1 = 16-row workgroups, 2 = 64-row ones; 0 = derived
};
const Tuning &tuning();

int device_cu_count();   // compute units of the current device

// events the next GEMV launch on this thread records around its kernel (both null: none);
// taking them clears them
void take_timing_events(hipEvent_t *start, hipEvent_t *stop);

// kernel launchers (return QG_OK or a failure already reported through fail())
// block: elements per activation scale (act_block)
int launch_quantize(int mode, int block, int64_t n, int64_t cols, const float *x, int8_t *codes,
                    qg_act_scale *scales, int32_t *csums, int32_t *err_flag, hipStream_t s);

int launch_gemv(int fmt, int mode, int64_t rows, int64_t cols, int64_t ncol, const void *image,
                const int8_t *codes, const qg_act_scale *scales, const int32_t *csums, float *out,
                hipStream_t s);

// one activation row: quantize it and run the GEMV in one launch
// argmax: null, or a 64-bit key word the row's argmax is folded into (atomic max)
int launch_gemv_fused(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const float *x,
                      int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag, float *out,
                      unsigned long long *argmax, hipStream_t s);

// several matrices, one activation row: from x (quantized on the fly, written to *_out) when x
// is not null, else from codes_in / scales_in
int launch_gemv_multi(int fmt, int mode, int nmat, const int64_t *rows, int64_t cols, const void *const *images,
                      const float *x, const int8_t *codes_in, const qg_act_scale *scales_in, int8_t *codes_out,
                      qg_act_scale *scales_out, int32_t *csums_out, int32_t *err_flag, float *const *outs,
                      hipStream_t s);

int launch_gemm_mfma(int64_t rows, int64_t cols, int64_t ncol, const void *image, const int8_t *codes,
                     const qg_act_scale *scales, float *out, hipStream_t s);

// diagnostic: read `bytes` (a multiple of 1 KiB is read; the rest ignored) with the GEMV's
// load pattern; sink[0] is written only if some lane's XOR of what it read equals magic
int launch_stream_read(const void *buf, size_t bytes, uint32_t magic, uint32_t *sink, hipStream_t s);
// diagnostic: the same in a chosen launch geometry (qg_stream_read_shape)
int launch_stream_read_shape(const void *buf, size_t bytes, int waves_per_wg, int kib_per_wave, int64_t wgs,
                             int flags, uint32_t magic, uint32_t *sink, hipStream_t s);
int launch_kv_cache_rows(int64_t n, int64_t hd, const float *x, uint16_t *scales, int8_t *codes, hipStream_t s);
int launch_kv_quantize_heads(int mode, int64_t nh, int64_t hd, const float *q, int8_t *codes, qg_act_scale *scales,
                             int32_t *err_flag, hipStream_t s);
int launch_kv_scores(int mode, int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const int8_t *qcodes,
                     const qg_act_scale *qscales, const uint16_t *kscales, const int8_t *kcodes, float *out,
                     hipStream_t s);
int launch_kv_weighted(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs, const uint16_t *vscales,
                       const int8_t *vcodes, float *out, hipStream_t s);
size_t kv_weighted_workspace_bytes(int64_t nh, int64_t npos, int64_t hd);
void launch_kv_fold_pieces(int64_t total, int hd, int64_t nblk, int64_t nkv, const float *pieces, float *out,
                           hipStream_t s);
int launch_kv_weighted_noalloc(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                               const uint16_t *vscales, const int8_t *vcodes, float *out, hipStream_t s);
int launch_kv_weighted_two_pass(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                                const uint16_t *vscales, const int8_t *vcodes, float *ws, float *out, hipStream_t s);

int launch_block_sums(int fmt, int64_t rows, int64_t cols, const void *image, const int8_t *codes,
                      int32_t *csum_out, int32_t *osum_out, hipStream_t s);

}  // namespace qg

static_assert(sizeof(qg_act_scale) == 4, "qg_act_scale must be 4 bytes");
