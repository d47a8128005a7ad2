/*
 * qgemv.h -- C ABI of libqgemv.so: the exact block-quantized matrix-row x activation-row
 * dot product (decode GEMV) and its batched-column form (GEMM) on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (rustdoc "Module numerics" of logicaffeine_compile::spatial::decode_engine,
 * module description, and "Module lane", module description):
 *   - a weight is exactly a block scale times an integer: Q4_K-style w = d*sc*q - dmin*mn,
 *     Q6_K-style w = d*sc*(q - 32);
 *   - activations are quantized under scales m*2^e to the exact nearest integer codes,
 *     either per weight block with an 8-bit significand (PerBlock) or per 32 elements with a
 *     4-bit significand (Sub32);
 *   - per 256-element block the terms (block scale x integer sum, second scale x offset sum,
 *     times the activation scale) are summed exactly and rounded to binary32 once, a
 *     subnormal result flushed to a zero of its sign;
 *   - a row's rounded pieces are added in ascending block order with binary32 adds (each
 *     result flushed), from +0.  A NaN output is 0x7FC00000.
 * Output bits depend only on the inputs: not on the stream, the launch configuration, the
 * tuning knobs or, for qg_gemm_q, on the number of columns.
 *
 * Conventions for every entry point:
 *   - Pointers named *_host are host memory; every other data pointer is device memory
 *     (hipMalloc / torch on the ROCm device).  All memory is owned by the caller; the
 *     library allocates no device memory and keeps no state except a per-thread reason
 *     string and the per-thread tuning knobs (qg_set_tuning).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Launches are asynchronous on it;
 *     the returned status covers only argument validation and launch errors.
 *   - Device pointers must be 16-byte aligned (4-byte for scales, csums, out, err_flag).
 *   - Errors return a nonzero qg_status and set a reason readable with qg_last_error().
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight block formats.  The first two use 256-element blocks, the last two 32-element ones. */
typedef enum {
    QG_Q4K = 1,   /* 4-bit codes, 8 sub-blocks of 32 with 6-bit scale and offset, f16 d, dmin */
    QG_Q6K = 2,   /* 6-bit codes offset by -32, 16 sub-blocks of 16 with int8 scales, f16 d */
    QG_Q8_0 = 3,  /* 32-element blocks: int8 codes, one f16 d per block (w = d*q) */
    QG_Q4_0 = 4   /* 32-element blocks: 4-bit codes offset by -8, one f16 d per block (w = d*(q-8)) */
} qg_format;

/* How an activation row is scaled ("Module numerics", Enums ActScaling). */
typedef enum {
    QG_PERBLOCK = 0,  /* one scale per weight block (256 or 32 elements), m in 128..255 */
    QG_SUB32 = 1      /* one scale per 32 elements, m in 8..15; a 256-group rounds once */
} qg_act_scaling;

/* An activation block's scale m * 2^e ("Module numerics", Structs ActScale).  For PerBlock
 * 128 <= m <= 255; for Sub32 8 <= m <= 15.  An all-zero block gets m = 128 (or 8), e = 0.
 * A block holding +-inf gets m = 0, e = 0 and raises the error flag. */
typedef struct {
    int16_t e;
    uint8_t m;
    uint8_t pad;
} qg_act_scale;

typedef enum {
    QG_OK = 0,
    QG_E_INVALID = 1,      /* null or misaligned pointer, bad enum, field out of range */
    QG_E_SHAPE = 2,        /* cols not a positive multiple of 256, cols > QG_MAX_COLS, n < 1 */
    QG_E_UNSUPPORTED = 3,  /* a (format, scaling) pair qg_reads() rejects */
    QG_E_UNREADABLE = 4,   /* a block scale is inf or NaN ("Module numerics", Structs Unreadable) */
    QG_E_NONFINITE = 5,    /* an activation is +-inf (reported through err_flag) */
    QG_E_RUNTIME = 6       /* a HIP call failed */
} qg_status;

#define QG_BLOCK 256
#define QG_MAX_COLS 32768
#define QG_MAX_MATRICES 8     /* matrices per qg_*_multi call */

/* Whether the kernels read matrices of `fmt` under `mode` ("Module numerics", Functions
 * reads).  1 for each of the four formats under PerBlock and Sub32; else 0. */
int qg_reads(int fmt, int mode);

/*
 * Weight image ------------------------------------------------------------------------
 *
 * A matrix of R rows and C columns (C = 256*G) is cut into tiles of 64 consecutive rows x
 * one 256-element block: tile (g, b) holds rows 64g .. 64g+63 of block b (rows past R are
 * zero padding) and sits at byte offset (g*G + b) * tile_bytes.  Lane l of a tile is row
 * 64g + l.
 *
 * Q4_K-style tile, 9216 bytes (= 64 x 144):
 *   chunk i (i = 0..7) at byte 1024*i: 16 bytes per lane at 1024*i + 16*l.  Byte k (0..15)
 *       holds the code of element 32i+k in its low nibble and of element 32i+16+k in its
 *       high nibble.
 *   meta at byte 8192: 16 bytes per lane at 8192 + 16*l:
 *       bytes 0..1  d    (binary16 bits, little endian)
 *       bytes 2..3  dmin (binary16 bits)
 *       bytes 4..15 a 96-bit little-endian field string; sub-block j's scale sc_j is bits
 *                   12j .. 12j+5 and its offset mn_j bits 12j+6 .. 12j+11.
 *
 * Q6_K-style tile, 13440 bytes (= 64 x 210):
 *   ql chunk i (i = 0..7) at byte 1024*i, 16 bytes per lane: byte k holds the low 4 bits of
 *       the code of element 32i+k (low nibble) and of element 32i+16+k (high nibble).
 *   qh chunk h (h = 0..3) at byte 8192 + 1024*h, 16 bytes per lane: byte k holds the high 2
 *       bits of the codes of elements 64h+k, 64h+16+k, 64h+32+k, 64h+48+k at bit pairs
 *       0-1, 2-3, 4-5, 6-7.
 *   scales at byte 12288, 16 bytes per lane: sub-block k's int8 scale in byte k.
 *   d at byte 13312, 2 bytes per lane: binary16 bits.
 *
 * The 32-element-block formats keep the same tiles of 64 rows x 256 elements (eight of
 * their blocks):
 * Q8_0-style tile, 17408 bytes (= 64 x 272):
 *   chunk i (i = 0..15) at byte 1024*i, 16 bytes per lane: the int8 codes of elements
 *       16i .. 16i+15 of the tile.
 *   d at byte 16384, 16 bytes per lane: the binary16 bits of the eight blocks' scales.
 * Q4_0-style tile, 9216 bytes (= 64 x 144):
 *   chunk i (i = 0..7) at byte 1024*i: block i's 32 codes, nibble-split as in the Q4_K-style
 *       tile (byte k: element 32i+k low, 32i+16+k high).
 *   d at byte 8192, 16 bytes per lane: the binary16 bits of the eight blocks' scales.
 */

/* Bytes of the image of an R x C matrix: ceil(R/64) * (C/256) * 64 * (144, 210, 272 or 144
 * for Q4_K, Q6_K, Q8_0, Q4_0).  0 for a bad format or shape. */
size_t qg_image_bytes(int fmt, int64_t rows, int64_t cols);

/* Pack Q4_K-style logical fields (host memory, row-major) into an image (host memory,
 * qg_image_bytes(QG_Q4K, rows, cols) bytes, no alignment needed):
 *   q    uint8  [rows][cols]      codes 0..15
 *   sc   uint8  [rows][cols/32]   sub-block scales 0..63
 *   mn   uint8  [rows][cols/32]   sub-block offsets 0..63
 *   d    uint16 [rows][cols/256]  binary16 bits of the block scale
 *   dmin uint16 [rows][cols/256]  binary16 bits of the second block scale
 * The weight of element i of block b is d*sc_j*q_i - dmin*mn_j with j the sub-block
 * ("Module numerics", Structs CodedRow, Segment, Scale).  Errors: QG_E_INVALID for a field
 * out of range, QG_E_UNREADABLE for an inf/NaN scale (the reason names row and block),
 * QG_E_SHAPE for a bad shape.  Nothing is written to the image on error. */
int qg_pack_q4k(int64_t rows, int64_t cols, const uint8_t *q_host, const uint8_t *sc_host,
                const uint8_t *mn_host, const uint16_t *d_host, const uint16_t *dmin_host,
                void *image_host);

/* Pack Q6_K-style logical fields into an image (host memory):
 *   q   uint8  [rows][cols]      codes 0..63 (the weight uses q - 32)
 *   sc  int8   [rows][cols/16]   sub-block scales -128..127
 *   d   uint16 [rows][cols/256]  binary16 bits of the block scale
 * Weight w = d*sc_k*(q_i - 32), k = i/16; |sc*(q-32)| <= 4096 ("Module numerics",
 * Constants COEF_BOUND).  Errors as qg_pack_q4k. */
int qg_pack_q6k(int64_t rows, int64_t cols, const uint8_t *q_host, const int8_t *sc_host,
                const uint16_t *d_host, void *image_host);

/* Pack a matrix with 32-element blocks ("Module numerics", module description: the matrix
 * format's own block, 32 or 256 elements) into an image (host memory):
 *   fmt  QG_Q8_0: q int8 [rows][cols] codes, w = d*q
 *        QG_Q4_0: q uint8 [rows][cols] codes 0..15, w = d*(q - 8)
 *   q    [rows][cols] as above (passed as bytes)
 *   d    uint16 [rows][cols/32]  binary16 bits of each block's scale
 * Errors as qg_pack_q4k (the reason of QG_E_UNREADABLE names the row and 32-element block). */
int qg_pack_b32(int fmt, int64_t rows, int64_t cols, const void *q_host, const uint16_t *d_host,
                void *image_host);

/* Quantize n activation rows ("Module numerics", Functions quantize_blocks (PerBlock) and
 * quantize (Sub32), absmax, wide_scale, block_scale, rne_div):
 *   x       f32 [n][cols]                       device
 *   codes   int8 [n][cols]                      device, out: rne(x / s), |code| <= 127
 *   scales  qg_act_scale [n][cols/B]            device, out; B = 32 under Sub32; under PerBlock
 *                                                the weight format's block (256 or 32)
 *   csums   int32 [n][cols/16]                  device, out: sum of the codes of each run of
 *                                                16 elements (the activation-side unit sums
 *                                                of "Module lane")
 *   err_flag int32 [1]                          device; set to 1 when a block holds +-inf.
 *                                                Never cleared by the library (clear it
 *                                                before the call).  May be NULL.
 * Each element is read with denormals as zero; the scale is the least m*2^e with
 * 127*m*2^e >= the block's largest magnitude (NaN passed over); a NaN element gets code 0.
 * fmt selects the PerBlock block: the weight format's own (256 for Q4_K and Q6_K, 32 for
 * Q8_0 and Q4_0), so scales are [n][cols/32] whenever mode is Sub32 or fmt is Q8_0 / Q4_0. */
int qg_quantize_act(int fmt, int mode, int64_t n, int64_t cols, const float *x, int8_t *codes,
                    qg_act_scale *scales, int32_t *csums, int32_t *err_flag, void *stream);

/* Decode GEMV ("Module numerics", Functions dot; "Module lane", Functions lane and group):
 *   image   the packed matrix (device), qg_image_bytes(fmt, rows, cols) bytes
 *   codes, scales, csums   one quantized activation row as written by qg_quantize_act
 *   out     f32 [rows] (device)
 * out[r] = the engine's f32 for row r . activation. */
int qg_gemv_q(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const int8_t *codes,
              const qg_act_scale *scales, const int32_t *csums, float *out, void *stream);

/* Batched columns: n activation rows (codes [n][cols], scales [n][cols/B], csums
 * [n][cols/16]) against the same matrix; out f32 [n*rows] with out[c*rows + r] equal, bit
 * for bit, to qg_gemv_q of row r with activation c. */
int qg_gemm_q(int fmt, int mode, int64_t rows, int64_t cols, int64_t n, const void *image,
              const int8_t *codes, const qg_act_scale *scales, const int32_t *csums, float *out,
              void *stream);

/* Quantize one activation row and run the decode GEMV on it, in one launch:
 *   x       f32 [cols] (device, 16-byte aligned)
 *   codes, scales, csums, err_flag   as qg_quantize_act with n = 1 (codes, scales and csums
 *           required: they receive the quantized row)
 *   image, out   as qg_gemv_q
 * out and the quantized row are bit for bit those of qg_quantize_act followed by qg_gemv_q
 * (the pages' dot of a row with a quantized activation row: "Module numerics", Functions
 * quantize and dot).  Every workgroup quantizes the blocks it needs itself; the first
 * writes the quantized row out.  rows = 0 only quantizes. */
int qg_quantize_gemv(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const float *x,
                     int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag, float *out,
                     void *stream);

/* qg_quantize_gemv plus the argmax of the output row, per "Module numerics", Functions argmax:
 * the row holding the greatest output, the lowest such row when several hold equal values
 * (+0 and -0 count as equal), NaN outputs skipped, and row 0 when every output is NaN.  It is
 * the greedy pick over an output projection's logits.
 *   argmax_key  device uint64 [1], 8-byte aligned; must hold 0 before the call (the caller
 *               clears it).  Each workgroup folds its rows into it with an atomic max of a
 *               key whose order is the value's, then the lower row's; the result is
 *               independent of workgroup order.  qg_argmax_index decodes it.
 * out and the quantized row are as qg_quantize_gemv writes them. */
int qg_quantize_gemv_argmax(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const float *x,
                            int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag, float *out,
                            uint64_t *argmax_key, void *stream);

/* The row index an argmax key stands for (host; 0 for the key 0: no row, or every row NaN). */
int64_t qg_argmax_index(uint64_t key);

/* Several matrices that share one activation row, in one launch (a decode layer's Q, K and V
 * projections, or its gate and up projections).  The matrices share fmt, mode and cols;
 *   nmat      1 .. QG_MAX_MATRICES
 *   rows      host int64 [nmat], each >= 0
 *   images    host array [nmat] of device images (qg_image_bytes(fmt, rows[m], cols) each)
 *   outs      host array [nmat] of device f32 outputs (rows[m] each)
 * qg_quantize_gemv_multi quantizes x as qg_quantize_gemv does (every workgroup the blocks it
 * needs; the first writes the quantized row to codes / scales / csums); qg_gemv_q_multi
 * takes an already quantized row.  Every outs[m] is bit for bit the one-matrix call's. */
int qg_quantize_gemv_multi(int fmt, int mode, int nmat, const int64_t *rows, int64_t cols,
                           const void *const *images, const float *x, int8_t *codes, qg_act_scale *scales,
                           int32_t *csums, int32_t *err_flag, float *const *outs, void *stream);
int qg_gemv_q_multi(int fmt, int mode, int nmat, const int64_t *rows, int64_t cols, const void *const *images,
                    const int8_t *codes, const qg_act_scale *scales, const int32_t *csums, float *const *outs,
                    void *stream);

/*
 * int8 KV cache ------------------------------------------------------------------------
 *
 * Attention over cached int8 rows on the same exact machinery ("Module numerics", Functions
 * cache_row, int8_codes, quantize_head, int8_score, weighted_int8, attend_int8; Constants
 * INV_127, VALUE_BLOCK).  The softmax between the scores and the weighted sum is the caller's.
 * Head sizes hd are 32, 64, 128 or 256.  nh query heads share nkv KV heads evenly: query head
 * h reads KV head h / (nh / nkv).  A KV cache of one KV head is npos rows: scales uint16 [npos]
 * (binary16 bits) and codes int8 [npos][hd]; the calls take [nkv][npos] and [nkv][npos][hd].
 * All buffers are device memory; QG_E_SHAPE for a bad head size, head counts that do not
 * divide, or sizes out of range; QG_E_INVALID for a bad pointer or enum.
 */
#define QG_VALUE_BLOCK 32   /* positions per block of the weighted sum */

/* Cache n rows x f32 [n][hd] (cache_row): per row the binary16 scale of amax * (1/127), amax
 * the largest magnitude (a denormal read as 0, a NaN passed over) and the product formed in
 * binary32, rounded to nearest even with subnormals kept (past the top it is infinite); the
 * codes are each x times the scale's binary32 reciprocal, to the nearest integer (ties to
 * even), within +-127 (a NaN product 0; all zero when the scale is zero).
 *   scales  uint16 [n]       out
 *   codes   int8 [n][hd]     out (4-byte aligned) */
int qg_kv_cache_rows(int64_t n, int64_t hd, const float *x, uint16_t *scales, int8_t *codes, void *stream);

/* Quantize nh query heads q f32 [nh][hd] (16-byte aligned) as the array reads them
 * (quantize_head): PerBlock, the whole head one block under an 8-bit significand scale;
 * Sub32, 32-element blocks under 4-bit ones; the rules of qg_quantize_act.
 *   codes   int8 [nh][hd]                       out
 *   scales  qg_act_scale [nh][1] (PerBlock) or [nh][hd/32] (Sub32)   out
 *   err_flag int32 [1] or NULL: set to 1 when a block holds +-inf (never cleared). */
int qg_kv_quantize_heads(int mode, int64_t nh, int64_t hd, const float *q, int8_t *codes, qg_act_scale *scales,
                         int32_t *err_flag, void *stream);

/* Scores (int8_score) of every query head against every cached key row of its KV head:
 * out[h][j] = R32(sum over the query's blocks b of m_b 2^e_b * (sum_i c_i k_ji) * d_j), the
 * terms summed exactly and rounded once (ftz); a key whose scale is not finite scores NaN
 * (0x7FC00000).  No softmax scale is applied.
 *   qcodes, qscales  one quantized head per query head, as qg_kv_quantize_heads writes them
 *   kscales uint16 [nkv][npos], kcodes int8 [nkv][npos][hd] (16-byte aligned)
 *   out     f32 [nh][npos] */
int qg_kv_scores(int mode, int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const int8_t *qcodes,
                 const qg_act_scale *qscales, const uint16_t *kscales, const int8_t *kcodes, float *out,
                 void *stream);

/* The weighted sum (weighted_int8) of every query head over its KV head's cached value rows:
 * w_j = p_j * d_j in binary32; per block of QG_VALUE_BLOCK positions (the last one possibly
 * shorter) the least power of two 2^E with 127 * 2^E >= the block's largest |w_j| (a denormal
 * read as 0, a NaN passed over; E = 0 for an all-zero block) and codes u_j = rne(w_j / 2^E);
 * per value element e the piece R32(2^E * sum_j u_j v_je); out[h][e] adds the pieces in block
 * order (binary32, each sum flushed; NaN -> 0x7FC00000).  A block holding an infinite w_j or a
 * value row whose scale is not finite gives NaN.  npos = 0 gives zeros.
 *   probs   f32 [nh][npos]
 *   vscales uint16 [nkv][npos], vcodes int8 [nkv][npos][hd]
 *   out     f32 [nh][hd] */
int qg_kv_weighted(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs, const uint16_t *vscales,
                   const int8_t *vcodes, float *out, void *stream);

/* Bytes of workspace qg_kv_weighted_with_workspace needs for nh heads over npos positions of
 * head size hd: one f32 piece per (head, block of QG_VALUE_BLOCK positions, value element),
 * nh * ceil(npos / QG_VALUE_BLOCK) * hd * 4.  Written to *bytes; QG_E_SHAPE for a head size or
 * count qg_kv_weighted refuses, QG_E_INVALID for a null bytes. */
int qg_kv_weighted_workspace(int64_t nh, int64_t npos, int64_t hd, size_t *bytes);

/* qg_kv_weighted in two passes, bit for bit the same result (weighted_int8): the first pass
 * reads each KV head's value rows once for every query head that shares them and writes each
 * block's pieces to the workspace, f32 [nh][ceil(npos / QG_VALUE_BLOCK)][hd]; the second adds
 * every head's pieces in block order.  The arguments are qg_kv_weighted's, plus
 *   workspace  device memory of ws_bytes >= qg_kv_weighted_workspace's figure (16-byte
 *              aligned), the caller's, overwritten; NULL allowed when that figure is 0.
 * QG_E_INVALID when ws_bytes is short or a pointer is null or misaligned.  Calls on one stream
 * may share a workspace; calls on concurrent streams need one each.  Honours
 * qg_time_next_launch (the events span both passes). */
int qg_kv_weighted_with_workspace(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                                  const uint16_t *vscales, const int8_t *vcodes, float *out, void *workspace,
                                  size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc): qg_kv_weighted_with_workspace over a fixed
 * workspace the library holds on each device, QG_KV_NOALLOC_BYTES long and kept until the
 * process ends, so that the call allocates nothing.  Same arguments as qg_kv_weighted and the
 * same bits.  QG_E_SHAPE when the pieces need more than QG_KV_NOALLOC_BYTES (nh *
 * ceil(npos / QG_VALUE_BLOCK) * hd * 4 bytes: 32 heads over 8192 positions of head size 128
 * fit); QG_E_RUNTIME when the workspace's device address cannot be had.  Every call on one
 * device uses the same workspace: calls on one stream follow each other safely, calls that
 * overlap on one GPU (concurrent streams or host threads) race and give wrong results.
 * Honours qg_time_next_launch. */
#define QG_KV_NOALLOC_BYTES ((size_t)4 << 20)
int qg_kv_weighted_noalloc(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                           const uint16_t *vscales, const int8_t *vcodes, float *out, void *stream);

/* Integer sums per (row, sub-block), before any scale ("Module lane", Functions
 * block_sums), for one activation row:
 *   Q4K: csum_out int32 [rows][cols/32] = sum sc_j*q*c over sub-block j,
 *        osum_out int32 [rows][cols/32] = sum mn_j*c.
 *   Q6K: csum_out int32 [rows][cols/16] = sum sc_k*(q-32)*c over sub-block k; osum_out is
 *        not written (may be NULL).
 * A debugging view of the kernels' integer stage; Q4_K and Q6_K only (QG_E_UNSUPPORTED
 * otherwise). */
int qg_block_sums(int fmt, int64_t rows, int64_t cols, const void *image, const int8_t *codes,
                  int32_t *csum_out, int32_t *osum_out, void *stream);

/* Diagnostic, not part of the method: reads the first floor(bytes / 1024) KiB of buf once
 * with the GEMV's load pattern (each wave nine contiguous 1 KiB chunks, non-temporal 16-byte
 * loads) and nothing else, to measure the streaming ceiling a launch of that size reaches.
 *   buf    device, 16-byte aligned; bytes < 1024 launches nothing
 *   sink   device uint32 [1]; written (with magic) only if, for some lane, the XOR of the
 *          16-byte pieces it read equals magic: a dependence that keeps the loads from
 *          being optimised away (an all-zero buffer never writes a nonzero magic)
 * Honours qg_time_next_launch. */
int qg_stream_read(const void *buf, size_t bytes, uint32_t magic, uint32_t *sink, void *stream);

/* Diagnostic, not part of the method: the same plain read of the first floor(bytes / 1024)
 * KiB of buf in a chosen launch geometry, for a sweep of launch shapes:
 *   waves_per_wg  1, 2, 4, 8 or 16 waves of 64 lanes per workgroup
 *   kib_per_wave  1, 2, 4, 8, 9 or 16: contiguous 1 KiB chunks each wave reads per pass, all of
 *                 a pass's loads issued before any is used (16 bytes per lane per chunk)
 *   wgs           0: one pass, as many workgroups as the bytes need; > 0: that many
 *                 workgroups in a grid-stride loop over the bytes
 *   flags         bit 0: ordinary loads (default: non-temporal loads)
 *   magic, sink   as qg_stream_read
 * QG_E_INVALID for a value outside these sets.  Honours qg_time_next_launch. */
int qg_stream_read_shape(const void *buf, size_t bytes, int waves_per_wg, int kib_per_wave, int64_t wgs, int flags,
                         uint32_t magic, uint32_t *sink, void *stream);

/* Speed-only tuning knobs; they never change output bits.  The knobs are per thread: a value
 * set by qg_set_tuning applies to the later calls made on the same thread (the library's only
 * state besides the reason string; other threads keep their own values).
 *   QG_TUNE_WAVES_PER_WG  waves per GEMV workgroup, splitting a 64-row group's blocks:
 *                         4, 8 or 16 (0 = one wave per block, at most 16).  16 applies
 *                         only to a single column of at most 16 blocks; otherwise 8 is used
 *   QG_TUNE_MFMA_MIN_COLS number of columns from which qg_gemm_q on a Q4_K PerBlock matrix
 *                         runs on the int8 matrix cores (0 = derived: 2 on fewer than 8192
 *                         rows, 5 on more; above 65535 = never)
 *   QG_TUNE_MFMA_FORM     the matrix-core GEMM's form: 1 = staged (at most 16 columns of rows of
 *                         at most 16 blocks: every wave one block, the columns' codes staged in
 *                         LDS), 2 = shared operands (weight operands built once per workgroup in
 *                         LDS), 3 = split (every wave one block, the activation operands loaded per
 *                         wave), 4 = column-resident (every block's activation codes of 16 or 32
 *                         columns staged in LDS once, every wave one 16-row tile over all blocks;
 *                         rows of at most 16 blocks with two column tiles, 32 with one); 0 =
 *                         derived from the shape
 *   QG_TUNE_MFMA_COL_TILES 1, 2 or 4: 16-column tiles per workgroup of the shared-operand,
 *                         split and (1 or 2) column-resident forms; 0 = derived (one for the split
 *                         form, from the columns for the shared-operand form, two for the
 *                         column-resident form on rows of at most 16 blocks)
 *   QG_TUNE_COLS_KERNEL   several columns below the matrix-core threshold (Q4_K/Q6_K, at most 16
 *                         blocks per row): 0 = the one-column kernel's machinery, NC columns per
 *                         wave (default); 1 = the kernel that stages the columns in LDS
 *   QG_TUNE_MFMA_TABLES   the shared-operand form: 0 = read every block's block scales, sub-block
 *                         fields and activation scales into LDS tables at the start where they
 *                         fit (default); 1 = load them with each block
 *   QG_TUNE_GEMM_ROW_TILES the staged and split forms: 16-row tiles per workgroup, 1, 2 or 4; the
 *                         column-resident form: waves (16-row tiles) per workgroup, 1, 2 or 4 (0 =
 *                         derived from the rows and columns)
 *   QG_TUNE_GEMV_QUARTER  one column of a Q4_K PerBlock matrix of at most 16 blocks per row,
 *                         without argmax: 1 = workgroups of 16 rows (four per 64-row group, so
 *                         a matrix of few row groups still fills the chip), 2 = workgroups of 64
 *                         rows, 0 = derived (16 rows below 128 row groups in the launch).  A
 *                         waves-per-workgroup setting takes the 64-row workgroups */
enum {
    QG_TUNE_WAVES_PER_WG = 1,
    QG_TUNE_MFMA_MIN_COLS = 2,
    QG_TUNE_MFMA_COL_TILES = 3,
    QG_TUNE_MFMA_FORM = 4,
    /* 5 is not used */
    QG_TUNE_COLS_KERNEL = 6,
    QG_TUNE_MFMA_TABLES = 7,
    QG_TUNE_GEMM_ROW_TILES = 8,
    QG_TUNE_GEMV_QUARTER = 9
};
int qg_set_tuning(int key, int64_t value);

/* Measurement hook: the next qg_gemv_q / qg_gemm_q / qg_quantize_gemv / qg_*_multi /
 * qg_stream_read call made on this thread launches its (GEMV, GEMM or read) kernel with hipExtLaunchKernelGGL, which records start_event as the kernel begins and
 * stop_event as it ends (hipEvent_t handles owned by the caller; both NULL cancels).
 * Later launches are not timed.  Changes no output bits. */
int qg_time_next_launch(void *start_event, void *stop_event);

/* The reason for the last nonzero status returned on this thread ("" if none). */
const char *qg_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
