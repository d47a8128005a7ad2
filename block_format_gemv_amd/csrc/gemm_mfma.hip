// gemm_mfma.hip -- batched-column GEMM of a Q4_K-style image under PerBlock scaling on the
// int8 matrix cores (v_mfma_i32_16x16x64_i8).
//
// The method's per-block integer sums ("Module lane", Functions block_sums) are a dense
// contraction once there are enough columns: per 256-element block,
//     C = sum sc_j * q_i * a_i,   O = sum mn_j * a_i   (j = the element's 32-element sub-block).
// A 6-bit sub-scale times a 4-bit code does not fit an int8 operand, so the sub-scale is
// split as sc = 8h + l (h, l <= 7): h*q and l*q are at most 105 and
//     C = 8 * sum (h*q)*a + sum (l*q)*a,
// three int8 products per block (the third with mn repeated per element), accumulated
// exactly in int32.  Each (row, column, block) is then combined and rounded once and added
// in block order exactly as in the GEMV ("Module numerics", module description; Functions
// exact_sum, scaled_to_f32, fadd), so every output carries the GEMV's bits.
//
// Operand roles: the MFMA's M dimension is 16 activation columns, N is 16 weight rows, so
// lane l of a result owns weight row l%16 and activation columns 4*(l/16) .. +3.
//
// The shared-operand form (more than 16 columns): a workgroup owns one 64-row group and 16*CW
// columns: wave (r, c) computes rows 16r..16r+15
// against columns 16c..16c+15.  Per block the workgroup builds, once, the weight operands of
// its 64 rows (wave (r, c) prepares the 64-element steps c, c+CW, .. of row quarter r) and the
// activation operands of its columns in an LDS stage; every wave reads what it needs from
// there.  Two stages alternate, and each thread's global loads run two blocks ahead.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMaxLds = 160 * 1024;   // LDS a gfx950 workgroup may use
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// each byte of q (at most 15) times k (at most 7): the products stay below 128, so the two
// 16-bit halves multiply without carries between bytes
__device__ __forceinline__ int bytes_times(uint32_t q, uint32_t k)
{
    const us2 a = __builtin_bit_cast(us2, q);
    const us2 b = {(unsigned short)k, (unsigned short)k};
    return __builtin_bit_cast(int, a * b);
}

// 12-bit (sc | mn << 6) field of sub-block j (0..7, any value) of the 96-bit string (y, z, w)
__device__ __forceinline__ uint32_t field_at(uint32_t y, uint32_t z, uint32_t w, int j)
{
    const int bit = 12 * j;                 // 0 .. 84
    const int word = bit >> 5, off = bit & 31;
    const uint32_t lo = word == 0 ? y : word == 1 ? z : w;
    const uint32_t hi = word == 0 ? z : w;  // word 2 never straddles (84 + 12 <= 96)
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> off) & 0xFFFu;
}

// One LDS stage (bytes).
template <int CW>
struct Stage {
    static constexpr int kBH = 0;                          // uint4 [4 row quarters][4 steps][64 lanes]: h*q
    static constexpr int kBL = kBH + 4 * 4 * 64 * 16;      // uint4 [4][4][64]: l*q
    static constexpr int kBO = kBL + 4 * 4 * 64 * 16;      // uint32 [4][4][64]: mn repeated
    static constexpr int kA = kBO + 4 * 4 * 64 * 4;        // uint4 [CW][4 steps][64 lanes]: activation codes
    static constexpr int kS = kA + CW * 4 * 64 * 16;       // double [16*CW]: activation scale m*2^e
    static constexpr int kW = kS + 16 * CW * 8;            // uint32 [16*CW]: qg_act_scale words
    static constexpr int kM = kW + 16 * CW * 4;            // uint32 [64]: d | dmin << 16 per row
    static constexpr int kBytes = (kM + 64 * 4 + 15) / 16 * 16;
};

// What one thread loads for one block, two blocks ahead of its use.
template <int CW>
struct Pref {
    uint4 ch[4 / CW];   // code chunk of each step this wave prepares
    uint4 meta;         // its row's d, dmin and sub-block fields
    uint4 a;            // 16 activation codes (its share of the stage's operands)
    uint32_t scw;       // a column's qg_act_scale word (used by threads < 16*CW)
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// float ftz through the class test: a subnormal becomes a zero of its sign
__device__ __forceinline__ float ftz_c(float x)
{
    const bool sub = __builtin_amdgcn_classf(x, 0x090);    // negative or positive subnormal (binary32 test)
    return sub ? __uint_as_float(__float_as_uint(x) & 0x80000000u) : x;
}

// grid: x = 64-row group, y = batch of 16*CW activation columns.  PRE: the block scales and
// sub-block fields of the group's rows and the activation scales of its columns, for every
// block, are read into LDS tables once at the start (when they fit), so that a block's loads
// are only its code chunks and activation codes: fewer vector-memory instructions per block.
template <int CW, bool PRE, int GT = 0>
__global__ __launch_bounds__(256 * CW) void gemm_mfma_q4k(const uint8_t *image, int rows, int G_arg,
                                                          const int8_t *__restrict__ codes,
                                                          const uint32_t *__restrict__ scw, int ncol,
                                                          float *__restrict__ out)
{
    using St = Stage<CW>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int G = GT ? GT : G_arg;   // GT: a block count known when compiling (the loop unrolls)
    const int C = G * 256;
    const int g = blockIdx.x;
    const int colbase = blockIdx.y * 16 * CW;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = wid & 3;                 // row quarter
    const int c = wid >> 2;                // column tile
    const int n = lane & 15;               // weight row within the quarter / activation column within the tile
    const int grp = lane >> 4;             // K group (16 of each 64-element step)
    const int trow = 16 * r + n;           // row within the 64-row tile

    // this thread's share of the activation operands: (column tile ta, step pa, lane la)
    const int ta = tid >> 8, pa = (tid >> 6) & 3, la = tid & 63;
    const int acol = min(colbase + 16 * ta + (la & 15), ncol - 1);
    const int8_t *abase = codes + (size_t)acol * C + 64 * pa + 16 * (la >> 4);
    const int scol = min(colbase + min(tid, 16 * CW - 1), ncol - 1);   // every thread loads one (in bounds)
    const uint8_t *gbase = image + (size_t)g * G * kTileBytesQ4K;
    // PRE tables after the two stages: uint4 [G][64] row metas, double [G][16*CW] activation
    // scales m*2^e, uint32 [G][16*CW] qg_act_scale words
    uint4 *t_meta = reinterpret_cast<uint4 *>(lds + 2 * St::kBytes);
    double *t_S = reinterpret_cast<double *>(lds + 2 * St::kBytes + (size_t)G * 64 * 16);
    uint32_t *t_W = reinterpret_cast<uint32_t *>(t_S + (size_t)G * 16 * CW);

    auto load = [&](Pref<CW> &pf, int b) __attribute__((always_inline)) {
        const uint8_t *tile = gbase + (size_t)b * kTileBytesQ4K;
#pragma unroll
        for (int k = 0; k < 4 / CW; k++) {
            const int p = c + k * CW;
            pf.ch[k] = ld16(tile + 1024 * (2 * p + (grp >> 1)) + 16 * trow);
        }
        if constexpr (!PRE) pf.meta = ld16(tile + 8192 + 16 * trow);
        pf.a = ld16(abase + (size_t)b * 256);
        if constexpr (!PRE) pf.scw = scw[(size_t)scol * G + b];
    };

    // prepare this wave's weight steps and this thread's activation share into stage st
    auto stage_write = [&](const Pref<CW> &pf, unsigned char *st, int b) __attribute__((always_inline)) {
        const uint4 meta = PRE ? t_meta[(size_t)b * 64 + trow] : pf.meta;
#pragma unroll
        for (int k = 0; k < 4 / CW; k++) {
            const int p = c + k * CW;
            const uint32_t f = field_at(meta.y, meta.z, meta.w, 2 * p + (grp >> 1));
            const uint32_t sc = f & 63u, hi = sc >> 3, lo = sc & 7u, mn = f >> 6;
            const int sh = 4 * (grp & 1);     // low nibbles: elements 0..15, high: 16..31
            const uint4 ch = pf.ch[k];
            const uint32_t q0 = (ch.x >> sh) & 0x0F0F0F0Fu, q1 = (ch.y >> sh) & 0x0F0F0F0Fu;
            const uint32_t q2 = (ch.z >> sh) & 0x0F0F0F0Fu, q3 = (ch.w >> sh) & 0x0F0F0F0Fu;
            const int slot = (r * 4 + p) * 64 + lane;
            reinterpret_cast<uint4 *>(st + St::kBH)[slot] =
                make_uint4(bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi));
            reinterpret_cast<uint4 *>(st + St::kBL)[slot] =
                make_uint4(bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo));
            reinterpret_cast<uint32_t *>(st + St::kBO)[slot] = mn * 0x01010101u;
        }
        reinterpret_cast<uint4 *>(st + St::kA)[(ta * 4 + pa) * 64 + la] = pf.a;
        if (PRE) return;
        if (c == 0 && grp == 0) reinterpret_cast<uint32_t *>(st + St::kM)[trow] = pf.meta.x;
        if (tid < 16 * CW) {
            reinterpret_cast<double *>(st + St::kS)[tid] =
                __builtin_ldexp((double)((pf.scw >> 16) & 0xFFu), (int)(int16_t)(pf.scw & 0xFFFFu));
            reinterpret_cast<uint32_t *>(st + St::kW)[tid] = pf.scw;
        }
    };

    float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // the block's integer sums on the matrix cores, then its combine into the row sums; CLEAN:
    // every activation scale of the workgroup's columns has an exponent of at least kNoTinyExp
    auto compute = [&](const unsigned char *st, int b, bool CLEAN) __attribute__((always_inline)) {
        v4i acc_h = {0, 0, 0, 0}, acc_l = {0, 0, 0, 0}, acc_o = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const int slot = (r * 4 + p) * 64 + lane;
            const v4i A = reinterpret_cast<const v4i *>(st + St::kA)[(c * 4 + p) * 64 + lane];
            const v4i Bh = reinterpret_cast<const v4i *>(st + St::kBH)[slot];
            const v4i Bl = reinterpret_cast<const v4i *>(st + St::kBL)[slot];
            const int bo = reinterpret_cast<const int *>(st + St::kBO)[slot];
            const v4i Bo = {bo, bo, bo, bo};
            acc_h = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bh, acc_h, 0, 0, 0);
            acc_l = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bl, acc_l, 0, 0, 0);
            acc_o = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bo, acc_o, 0, 0, 0);
        }
        const uint32_t dd = PRE ? t_meta[(size_t)b * 64 + trow].x : reinterpret_cast<const uint32_t *>(st + St::kM)[trow];
        const float fd = f16_value(dd), fm = f16_value(dd >> 16);
        const bool near = q4k_near(fd, fm);
        const double Dd = (double)fd, Dm = (double)fm;
        const double *S = (PRE ? t_S + (size_t)b * 16 * CW : reinterpret_cast<const double *>(st + St::kS)) + 16 * c + 4 * grp;
        if (CLEAN && __all(near)) {
            // no piece is tiny: every nonzero one is normal, no partial sum is subnormal or -0,
            // and an exact zero adds as +0 would, so plain conversions and adds give the
            // flushed ones' bits
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int Cb = 8 * acc_h[i] + acc_l[i];
                const double X = __builtin_fma((double)Cb, Dd, -((double)acc_o[i] * Dm));
                y[i] = y[i] + (float)(X * S[i]);
            }
        } else if (__all(near)) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int Cb = 8 * acc_h[i] + acc_l[i];
                const double X = __builtin_fma((double)Cb, Dd, -((double)acc_o[i] * Dm));
                const float piece = ftz_c((float)(X * S[i] + 0.0));   // + 0.0: an exact zero is +0
                y[i] = ftz_c(y[i] + piece);
            }
        } else {
            const uint32_t *W = (PRE ? t_W + (size_t)b * 16 * CW : reinterpret_cast<const uint32_t *>(st + St::kW)) + 16 * c + 4 * grp;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int Cb = 8 * acc_h[i] + acc_l[i];
                float piece;
                if (near) {
                    piece = piece_q4k_perblock_near(Cb, acc_o[i], Dd, Dm, S[i]);
                } else {
                    const int m = (int)((W[i] >> 16) & 0xFFu);
                    const int e = (int)(int16_t)(W[i] & 0xFFFFu);
                    piece = piece_q4k_perblock(Cb, acc_o[i], dd, m, e);
                }
                y[i] = fadd_ftz(y[i], piece);
            }
        }
    };

    bool ok = true;
    for (int i = tid; i < 16 * CW * G; i += 256 * CW) {
        const int col = min(colbase + i % (16 * CW), ncol - 1);
        const uint32_t w = scw[(size_t)col * G + i / (16 * CW)];
        ok = ok && (int)(int16_t)(w & 0xFFFFu) >= kNoTinyExp;
        if constexpr (PRE) {
            t_S[i] = __builtin_ldexp((double)((w >> 16) & 0xFFu), (int)(int16_t)(w & 0xFFFFu));
            t_W[i] = w;
        }
    }
    if constexpr (PRE)
        for (int i = tid; i < 64 * G; i += 256 * CW)
            t_meta[i] = ld16(gbase + (size_t)(i / 64) * kTileBytesQ4K + 8192 + 16 * (i % 64));
    const bool clean = __syncthreads_and(ok);

    unsigned char *st0 = lds, *st1 = lds + St::kBytes;
    // The loads run unconditionally (past the last block they repeat it): with every path
    // issuing the same loads, the compiler's wait before a stage is written counts exactly
    // the younger loads still in flight instead of waiting for all of them.
    if constexpr (PRE) {
        // a block's loads are its code chunks and activation codes only: three register
        // buffers (block k in p[k % 3]); the buffer a step stages takes the loads of the block
        // three steps later
        Pref<CW> p0, p1, p2;
        load(p0, 0);
        load(p1, min(1, G - 1));
        load(p2, min(2, G - 1));
        stage_write(p0, st0, 0);
        load(p0, min(3, G - 1));
        __syncthreads();
        auto step = [&](int b, Pref<CW> &ps) __attribute__((always_inline)) {
            compute((b & 1) ? st1 : st0, b, clean);
            if (b + 1 < G) stage_write(ps, (b & 1) ? st0 : st1, b + 1);
            load(ps, min(b + 4, G - 1));
            __syncthreads();
        };
        auto three = [&](int b) __attribute__((always_inline)) {
            step(b, p1);
            if (b + 1 >= G) return false;
            step(b + 1, p2);
            if (b + 2 >= G) return false;
            step(b + 2, p0);
            return true;
        };
        if constexpr (GT > 0) {
            // straight-line code: the compiler's waits count the loads in flight exactly
#pragma unroll
            for (int b = 0; b < GT; b += 3)
                if (!three(b)) break;
        } else {
            for (int b = 0; b < G; b += 3)
                if (!three(b)) break;
        }
    } else {
    Pref<CW> p0, p1;
    load(p0, 0);
    load(p1, min(1, G - 1));
    stage_write(p0, st0, 0);
    __syncthreads();
    for (int b = 0; b < G; b += 2) {
        // block b is in stage 0; block b+1's loads are in flight in p1
        load(p0, min(b + 2, G - 1));
        compute(st0, b, clean);
        if (b + 1 < G) stage_write(p1, st1, b + 1);
        __syncthreads();
        if (b + 1 >= G) break;
        load(p1, min(b + 3, G - 1));
        compute(st1, b + 1, clean);
        if (b + 2 < G) stage_write(p0, st0, b + 2);
        __syncthreads();
    }
    }

    const int64_t row = (int64_t)g * 64 + trow;
    if (row < rows) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int col = colbase + 16 * c + 4 * grp + i;
            if (col < ncol) out[(int64_t)col * rows + row] = canon_nan(y[i]);
        }
    }
}

// the LDS a kernel has beside its dynamic share (its own static LDS: the workgroup vote)
template <int CW, bool PRE, int GT = 0>
size_t cw_static_lds()
{
    static const size_t fixed = [] {
        hipFuncAttributes a{};
        return hipFuncGetAttributes(&a, reinterpret_cast<const void *>(gemm_mfma_q4k<CW, PRE, GT>)) == hipSuccess
                   ? a.sharedSizeBytes
                   : (size_t)kMaxLds;
    }();
    return fixed;
}

template <int CW, bool PRE, int GT = 0>
int launch_cw_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                    const qg_act_scale *scales, float *out, hipStream_t s, size_t lds)
{
    const int64_t groups = (rows + 63) / 64;
    const dim3 grid((unsigned)groups, (unsigned)((ncol + 16 * CW - 1) / (16 * CW)));
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_mfma_q4k<CW, PRE, GT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kMaxLds - cw_static_lds<CW, PRE, GT>()));
    (void)attr;   // a refusal shows up as a launch error below
    const uint32_t *w = reinterpret_cast<const uint32_t *>(scales);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemm_mfma_q4k<CW, PRE, GT>), grid, dim3(256 * CW), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, out);
    else
        hipLaunchKernelGGL((gemm_mfma_q4k<CW, PRE, GT>), grid, dim3(256 * CW), lds, s, static_cast<const uint8_t *>(image),
                           (int)rows, G, codes, w, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

// two operand stages (above 64 KiB: gfx950 gives a workgroup up to 160 KiB), with the
// per-block tables after them where those fit
template <int CW>
int launch_cw(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes, const qg_act_scale *scales,
              float *out, hipStream_t s)
{
    const size_t stages = 2 * (size_t)Stage<CW>::kBytes;
    const size_t tables = (size_t)G * (64 * 16 + 16 * CW * (8 + 4));
    if (tuning().mfma_pre_off == 0 && stages + tables + cw_static_lds<CW, true>() <= (size_t)kMaxLds) {
        if (G == 16) return launch_cw_typed<CW, true, 16>(rows, G, ncol, image, codes, scales, out, s, stages + tables);
        return launch_cw_typed<CW, true>(rows, G, ncol, image, codes, scales, out, s, stages + tables);
    }
    return launch_cw_typed<CW, false>(rows, G, ncol, image, codes, scales, out, s, stages);
}

template <int I>
__device__ __forceinline__ uint32_t field_s(uint32_t y, uint32_t z, uint32_t w)
{
    if constexpr (I < 5) return (uint32_t)(((uint64_t)y | ((uint64_t)z << 32)) >> (12 * I)) & 0xFFFu;
    else return (uint32_t)(((uint64_t)z | ((uint64_t)w << 32)) >> (12 * I - 32)) & 0xFFFu;
}

// The per-wave form, for fewer columns: each wave computes 16 rows x 16*CT columns over all
// blocks from its own registers (weights and activation operands loaded per wave, two
// register stages).  grid: x = 64-row group, y = batch of 16*CT activation columns; 4 waves,
// wave w = rows 16w..16w+15
template <int CT>
__global__ __launch_bounds__(256) void gemm_mfma_wave(const uint8_t *__restrict__ image, int rows, int G,
                                                     const int8_t *__restrict__ codes,
                                                     const qg_act_scale *__restrict__ scales, int ncol,
                                                     float *__restrict__ out)
{
    // LDS: [G][16*CT] activation scales as exact doubles m*2^e, then the same as
    // qg_act_scale words (for the general combine)
    extern __shared__ __align__(16) double s_S[];
    constexpr int NCOLS = 16 * CT;
    uint32_t *s_sc = reinterpret_cast<uint32_t *>(s_S + (size_t)G * NCOLS);
    const int C = G * 256;
    const int g = blockIdx.x;
    const int colbase = blockIdx.y * NCOLS;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;             // weight row within the wave's 16 rows
    const int grp = lane >> 4;           // K group (16 of each 64-element step)
    const int trow = 16 * wid + n;       // row within the 64-row tile
    const int64_t row = (int64_t)g * 64 + trow;

    const uint32_t *scw = reinterpret_cast<const uint32_t *>(scales);
    for (int i = threadIdx.x; i < G * NCOLS; i += 256) {
        const int b = i / NCOLS, j = i % NCOLS;
        const int col = colbase + j;
        const uint32_t w = col < ncol ? scw[(size_t)col * G + b] : 0u;
        s_sc[i] = w;
        s_S[i] = __builtin_ldexp((double)((w >> 16) & 0xFFu), (int)(int16_t)(w & 0xFFFFu));
    }
    __syncthreads();

    float y[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
        for (int i = 0; i < 4; i++) y[ct][i] = 0.0f;

    // one block's loads: this lane's row meta, its four 16-byte code chunks, and 16 bytes of
    // activation codes per column tile and 64-element step
    struct Stage {
        uint4 meta;
        uint4 ch[4];
        v4i A[CT][4];
    };
    // per-lane bases; a block adds a uniform offset
    const uint8_t *wbase = image + (size_t)g * G * kTileBytesQ4K + 16 * trow;
    const uint8_t *mbase = wbase + 8192;
    const uint8_t *cbase = wbase + 1024 * (grp >> 1);
    const int8_t *abase[CT];
    bool acol[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ct++) {
        const int col = colbase + 16 * ct + n;
        acol[ct] = col < ncol;
        abase[ct] = codes + (size_t)(acol[ct] ? col : 0) * C + 16 * grp;
    }
    auto load = [&](Stage &st, int b) {
        const size_t toff = (size_t)b * kTileBytesQ4K;
        st.meta = *reinterpret_cast<const uint4 *>(mbase + toff);
#pragma unroll
        for (int p = 0; p < 4; p++) st.ch[p] = *reinterpret_cast<const uint4 *>(cbase + toff + 2048 * p);
#pragma unroll
        for (int ct = 0; ct < CT; ct++) {
#pragma unroll
            for (int p = 0; p < 4; p++) {
                const v4i v = *reinterpret_cast<const v4i *>(abase[ct] + (size_t)b * 256 + 64 * p);
                st.A[ct][p] = acol[ct] ? v : v4i{0, 0, 0, 0};
            }
        }
    };
    auto compute = [&](const Stage &st, int b) {
        const uint4 meta = st.meta;
        uint32_t f[8];
        f[0] = field_s<0>(meta.y, meta.z, meta.w);
        f[1] = field_s<1>(meta.y, meta.z, meta.w);
        f[2] = field_s<2>(meta.y, meta.z, meta.w);
        f[3] = field_s<3>(meta.y, meta.z, meta.w);
        f[4] = field_s<4>(meta.y, meta.z, meta.w);
        f[5] = field_s<5>(meta.y, meta.z, meta.w);
        f[6] = field_s<6>(meta.y, meta.z, meta.w);
        f[7] = field_s<7>(meta.y, meta.z, meta.w);

        v4i acc_h[CT], acc_l[CT], acc_o[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ct++) acc_h[ct] = acc_l[ct] = acc_o[ct] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; p++) {
            // this lane's K group lies in sub-block 2p + grp/2, in the low or high nibbles
            const uint32_t fsel = 0u - (uint32_t)(grp >> 1);            // all ones for the odd sub-block
            const uint32_t fj = f[2 * p] ^ ((f[2 * p] ^ f[2 * p + 1]) & fsel);
            const uint32_t sc = fj & 63u, hi = sc >> 3, lo = sc & 7u, mn = fj >> 6;
            const int sh = 4 * (grp & 1);
            const uint32_t q0 = (st.ch[p].x >> sh) & 0x0F0F0F0Fu, q1 = (st.ch[p].y >> sh) & 0x0F0F0F0Fu;
            const uint32_t q2 = (st.ch[p].z >> sh) & 0x0F0F0F0Fu, q3 = (st.ch[p].w >> sh) & 0x0F0F0F0Fu;
            const v4i Bh = {bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi)};
            const v4i Bl = {bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo)};
            const int mrep = (int)(mn * 0x01010101u);
            const v4i Bo = {mrep, mrep, mrep, mrep};
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                acc_h[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.A[ct][p], Bh, acc_h[ct], 0, 0, 0);
                acc_l[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.A[ct][p], Bl, acc_l[ct], 0, 0, 0);
                acc_o[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.A[ct][p], Bo, acc_o[ct], 0, 0, 0);
            }
        }

        // combine each (row, column) of this block once, then add it into the row's sum
        const F16Scale d = f16_scale(meta.x & 0xFFFFu);
        const F16Scale dm = f16_scale(meta.x >> 16);
        const int gap = d.ex > dm.ex ? d.ex - dm.ex : dm.ex - d.ex;
        const bool near = gap <= 8;
        const double Dd = __builtin_ldexp((double)d.sig, d.ex);
        const double Dm = __builtin_ldexp((double)dm.sig, dm.ex);
        if (__all(near)) {
            // every row of the wave takes the near-exponent combine: no per-lane branch
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                const double *S = s_S + b * NCOLS + 16 * ct + 4 * grp;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int Cb = 8 * acc_h[ct][i] + acc_l[ct][i];
                    y[ct][i] = fadd_ftz(y[ct][i], piece_q4k_perblock_near(Cb, acc_o[ct][i], Dd, Dm, S[i]));
                }
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                const uint32_t *sv = s_sc + b * NCOLS + 16 * ct + 4 * grp;
                const double *S = s_S + b * NCOLS + 16 * ct + 4 * grp;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int Cb = 8 * acc_h[ct][i] + acc_l[ct][i];
                    const int Ob = acc_o[ct][i];
                    float piece;
                    if (near) {
                        piece = piece_q4k_perblock_near(Cb, Ob, Dd, Dm, S[i]);
                    } else {
                        const int m = (int)((sv[i] >> 16) & 0xFFu);
                        const int e = (int)(int16_t)(sv[i] & 0xFFFFu);
                        piece = piece_q4k_perblock(Cb, Ob, meta.x, m, e);
                    }
                    y[ct][i] = fadd_ftz(y[ct][i], piece);
                }
            }
        }
    };

    // two register sets, no copies: the next block's loads are in flight during this block's work
    Stage s0, s1;
    load(s0, 0);
    for (int b = 0; b < G; b += 2) {
        if (b + 1 < G) load(s1, b + 1);
        compute(s0, b);
        if (b + 1 >= G) break;
        if (b + 2 < G) load(s0, b + 2);
        compute(s1, b + 1);
    }

    if (row < rows) {
#pragma unroll
        for (int ct = 0; ct < CT; ct++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = colbase + 16 * ct + 4 * grp + i;
                if (col < ncol) out[(int64_t)col * rows + row] = canon_nan(y[ct][i]);
            }
    }
}

template <int CT>
int launch_wave(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes, const qg_act_scale *scales,
              float *out, hipStream_t s)
{
    const int64_t groups = (rows + 63) / 64;
    const dim3 grid((unsigned)groups, (unsigned)((ncol + 16 * CT - 1) / (16 * CT)));
    const size_t lds = (size_t)G * 16 * CT * (8 + 4);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL(gemm_mfma_wave<CT>, grid, dim3(256), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, scales, (int)ncol, out);
    else
        hipLaunchKernelGGL(gemm_mfma_wave<CT>, grid, dim3(256), lds, s, static_cast<const uint8_t *>(image), (int)rows,
                           G, codes, scales, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

// ---------------------------------------------------------------------------------------
// The ring form.  A workgroup owns one 64-row group and 16*CT columns; with WH waves per row
// quarter, wave w computes rows 16(w%4)..+15 against column tiles (w/4)*CT/WH .. +CT/WH-1,
// from an LDS ring of D+1 slots.  Each slot holds one block:
// the weight tile as it lies in the image, then the activation operands already in the order
// the matrix cores read them (operand (ct, p) = 1 KiB: lane l <- column 16ct + l%16, bytes
// 64p + 16(l/16) of the block).  The slots are filled by LDS-DMA loads (global_load_lds:
// lane l's bytes land at the wave-uniform LDS base + size * l) issued D blocks ahead, so the
// weight stream stays in flight without holding registers.  They are issued from inline
// asm: the compiler would otherwise wait for every outstanding one before each LDS read.
// The kernel waits for its own (s_waitcnt vmcnt with the exact count of younger loads) and
// a barrier then covers every wave's.
//
// The epilogue adds each block's pieces into the row sums with plain binary32 adds while no
// piece of the wave's rows is tiny (tiny_piece); a lane that meets one takes the exact
// combine and the flushed add from then on, and with it its wave.

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from global memory to LDS (base + 16 * lane, base wave-uniform); M0 is
// saved and restored, and the load waits one instruction after M0 is written
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base)
{
    uint32_t t;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(t)
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int CT, int D, int WH>
struct Ring {
    static constexpr int kWaves = 4 * WH;
    static constexpr int kA = kTileBytesQ4K;                // activation operands after the tile
    static constexpr int kSlot = kTileBytesQ4K + CT * 4 * 1024;
    static constexpr int kSlots = D + 1;                   // the block being computed + D in flight
    static constexpr int kRing = kSlots * kSlot;
    // DMA loads per block: the tile's 9 chunks and 4*CT activation operands, dealt out to the
    // waves in turn; every wave issues kDma (the last ones repeat chunk 8, so that every wave
    // issues the same count and can wait for an exact one)
    static constexpr int kLoads = 9 + 4 * CT;
    static constexpr int kDma = (kLoads + kWaves - 1) / kWaves;
};

// PerBlock Q4_K-style piece from the activation scale as the exact double S = m*2^e:
// R32(S * (d*C - dmin*O)), the same value as piece_q4k_perblock
__device__ __forceinline__ float piece_q4k_perblock_s(int C, int O, uint32_t d_dmin, double S)
{
    const F16Scale d = f16_scale(d_dmin & 0xFFFFu);
    const F16Scale dm = f16_scale(d_dmin >> 16);
    const double a = __builtin_ldexp((double)C * (double)d.sig * S, d.ex);
    const double b = __builtin_ldexp(-(double)O * (double)dm.sig * S, dm.ex);
    return r32_sum2(a, b);
}

// grid: x = 64-row group, y = batch of 16*CT activation columns; 4*WH waves
template <int CT, int D, int WH>
__global__ __launch_bounds__(256 * WH) void gemm_ring_q4k(const uint8_t *__restrict__ image, int rows, int G,
                                                          const int8_t *__restrict__ codes,
                                                          const uint32_t *__restrict__ scw, int ncol,
                                                          float *__restrict__ out)
{
    static_assert(D >= 2 && D <= 4, "ring depth");
    static_assert(CT % WH == 0, "whole column tiles per wave");
    using Rg = Ring<CT, D, WH>;
    constexpr int NC = 16 * CT;
    constexpr int NW = Rg::kWaves;
    constexpr int CTW = CT / WH;                       // column tiles per wave
    constexpr int K = Rg::kDma;
    extern __shared__ __align__(16) unsigned char lds[];
    double *s_S = reinterpret_cast<double *>(lds + Rg::kRing);     // [G][NC] activation scales m*2^e
    const int C = G * 256;
    const int g = blockIdx.x;
    const int colbase = blockIdx.y * NC;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int trow = 16 * (wid & 3) + n;               // row within the 64-row group
    const int ct0 = (wid >> 2) * CTW;                  // this wave's first column tile
    const uint8_t *gbase = image + (size_t)g * G * kTileBytesQ4K;

    // the scale table first: its loads are waited for by the compiler, which would also wait
    // for any DMA issued before them
    for (int i = threadIdx.x; i < G * NC; i += 64 * NW) {
        const int b = i / NC, col = colbase + i % NC;
        const uint32_t w = col < ncol ? scw[(size_t)col * G + b] : 0u;
        s_S[i] = __builtin_ldexp((double)((w >> 16) & 0xFFu), (int)(int16_t)(w & 0xFFFFu));
    }

    auto issue = [&](int b) {
        unsigned char *slot = lds + (b % Rg::kSlots) * Rg::kSlot;
        const uint8_t *tile = gbase + (size_t)b * kTileBytesQ4K;
#pragma unroll
        for (int j = 0; j < K; j++) {
            const int i = wid + NW * j;                 // this wave's j-th load of the block
            if (i < 9 || i >= Rg::kLoads) {
                const int ch = min(i, 8);
                dma16(tile + 1024 * ch + 16 * lane, lds_offset(slot + 1024 * ch));
            } else {
                const int k = i - 9;                    // operand (ct, p) = (k / 4, k % 4)
                const int col = min(colbase + 16 * (k >> 2) + n, ncol - 1);
                dma16(codes + (size_t)col * C + (size_t)b * 256 + 64 * (k & 3) + 16 * grp,
                      lds_offset(slot + Rg::kA + 1024 * k));
            }
        }
    };
    // own loads of the block after the one waited for still outstanding: nb blocks' worth
    // (nb < D; an exact count, so that the wait ends as soon as that block has landed)
    auto wait_blocks_after = [&](int nb) {
        if (nb >= 3) wait_vm<3 * K>();
        else if (nb == 2) wait_vm<2 * K>();
        else if (nb == 1) wait_vm<K>();
        else wait_vm<0>();
    };

    const int pre = min(D, G);
    for (int b = 0; b < pre; b++) issue(b);
    wait_blocks_after(pre - 1);
    __syncthreads();

    float y[CTW][4];
#pragma unroll
    for (int ct = 0; ct < CTW; ct++)
#pragma unroll
        for (int i = 0; i < 4; i++) y[ct][i] = 0.0f;
    bool tainted = false;     // this lane's row has met a tiny piece

    for (int b = 0; b < G; b++) {
        if (b + D < G) issue(b + D);
        const unsigned char *slot = lds + (b % Rg::kSlots) * Rg::kSlot;
        const uint4 meta = *reinterpret_cast<const uint4 *>(slot + 8192 + 16 * trow);
        uint32_t f[8];
        f[0] = field_s<0>(meta.y, meta.z, meta.w);
        f[1] = field_s<1>(meta.y, meta.z, meta.w);
        f[2] = field_s<2>(meta.y, meta.z, meta.w);
        f[3] = field_s<3>(meta.y, meta.z, meta.w);
        f[4] = field_s<4>(meta.y, meta.z, meta.w);
        f[5] = field_s<5>(meta.y, meta.z, meta.w);
        f[6] = field_s<6>(meta.y, meta.z, meta.w);
        f[7] = field_s<7>(meta.y, meta.z, meta.w);

        v4i acc_h[CTW], acc_l[CTW], acc_o[CTW];
#pragma unroll
        for (int ct = 0; ct < CTW; ct++) acc_h[ct] = acc_l[ct] = acc_o[ct] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; p++) {
            // this lane's K group lies in sub-block 2p + grp/2, in the low or high nibbles
            const uint32_t fsel = 0u - (uint32_t)(grp >> 1);
            const uint32_t fj = f[2 * p] ^ ((f[2 * p] ^ f[2 * p + 1]) & fsel);
            const uint32_t sc = fj & 63u, hi = sc >> 3, lo = sc & 7u, mn = fj >> 6;
            const uint4 ch = *reinterpret_cast<const uint4 *>(slot + 1024 * (2 * p + (grp >> 1)) + 16 * trow);
            const int sh = 4 * (grp & 1);
            const uint32_t q0 = (ch.x >> sh) & 0x0F0F0F0Fu, q1 = (ch.y >> sh) & 0x0F0F0F0Fu;
            const uint32_t q2 = (ch.z >> sh) & 0x0F0F0F0Fu, q3 = (ch.w >> sh) & 0x0F0F0F0Fu;
            const v4i Bh = {bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi)};
            const v4i Bl = {bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo)};
            const int mrep = (int)(mn * 0x01010101u);
            const v4i Bo = {mrep, mrep, mrep, mrep};
#pragma unroll
            for (int ct = 0; ct < CTW; ct++) {
                const v4i A = *reinterpret_cast<const v4i *>(slot + Rg::kA + 1024 * (4 * (ct0 + ct) + p) + 16 * lane);
                acc_h[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bh, acc_h[ct], 0, 0, 0);
                acc_l[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bl, acc_l[ct], 0, 0, 0);
                acc_o[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bo, acc_o[ct], 0, 0, 0);
            }
        }

        // combine each (row, column) of the block once, then add it into the row's sum
        const float fd = f16_value(meta.x), fm = f16_value(meta.x >> 16);
        const bool near = q4k_near(fd, fm);
        const double Dd = (double)fd, Dm = (double)fm;
        const double *S = s_S + (size_t)b * NC + 16 * ct0 + 4 * grp;
        bool fast = false;
        if (__all(near) && !__any(tainted)) {
            float pc[CTW][4];
            int lo = 0;
#pragma unroll
            for (int ct = 0; ct < CTW; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int Cb = 8 * acc_h[ct][i] + acc_l[ct][i];
                    const double X = __builtin_fma((double)Cb, Dd, -((double)acc_o[ct][i] * Dm));
                    pc[ct][i] = (float)(X * S[16 * ct + i]);
                    lo = min(lo, __builtin_amdgcn_frexp_expf(pc[ct][i]));
                }
            if (!__any(lo <= -102)) {
                // no tiny piece: every piece is zero or normal, and no partial sum can be
                // subnormal (nor -0), so plain adds give the flushed adds' bits
                fast = true;
#pragma unroll
                for (int ct = 0; ct < CTW; ct++)
#pragma unroll
                    for (int i = 0; i < 4; i++) y[ct][i] = y[ct][i] + pc[ct][i];
            }
        }
        if (!fast) {
#pragma unroll
            for (int ct = 0; ct < CTW; ct++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int Cb = 8 * acc_h[ct][i] + acc_l[ct][i];
                    const int Ob = acc_o[ct][i];
                    const float piece = near ? piece_q4k_perblock_near(Cb, Ob, Dd, Dm, S[16 * ct + i])
                                             : piece_q4k_perblock_s(Cb, Ob, meta.x, S[16 * ct + i]);
                    tainted |= tiny_piece(piece);
                    y[ct][i] = fadd_ftz(y[ct][i], piece);
                }
        }

        if (b + 1 < G) wait_blocks_after(min(b + D, G - 1) - (b + 1));
        __syncthreads();
    }

    const int64_t row = (int64_t)g * 64 + trow;
    if (row < rows) {
#pragma unroll
        for (int ct = 0; ct < CTW; ct++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = colbase + 16 * (ct0 + ct) + 4 * grp + i;
                if (col < ncol) out[(int64_t)col * rows + row] = canon_nan(y[ct][i]);
            }
    }
}

template <int CT, int D>
size_t ring_lds(int G)
{
    return (size_t)Ring<CT, D, 1>::kRing + (size_t)G * 16 * CT * sizeof(double);
}

template <int CT, int D, int WH>
int launch_ring_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                      const qg_act_scale *scales, float *out, hipStream_t s)
{
    const int64_t groups = (rows + 63) / 64;
    const dim3 grid((unsigned)groups, (unsigned)((ncol + 16 * CT - 1) / (16 * CT)));
    const size_t lds = ring_lds<CT, D>(G);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_ring_q4k<CT, D, WH>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    (void)attr;   // a refusal shows up as a launch error below
    const uint32_t *w = reinterpret_cast<const uint32_t *>(scales);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemm_ring_q4k<CT, D, WH>), grid, dim3(256 * WH), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, out);
    else
        hipLaunchKernelGGL((gemm_ring_q4k<CT, D, WH>), grid, dim3(256 * WH), lds, s, static_cast<const uint8_t *>(image),
                           (int)rows, G, codes, w, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores, ring) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

// the deepest ring that fits the LDS of a workgroup, or QG_E_UNSUPPORTED
template <int CT, int WH>
int launch_ring_d(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                  const qg_act_scale *scales, float *out, hipStream_t s)
{
    if (ring_lds<CT, 4>(G) <= (size_t)kMaxLds)
        return launch_ring_typed<CT, 4, WH>(rows, G, ncol, image, codes, scales, out, s);
    if (ring_lds<CT, 3>(G) <= (size_t)kMaxLds)
        return launch_ring_typed<CT, 3, WH>(rows, G, ncol, image, codes, scales, out, s);
    if (ring_lds<CT, 2>(G) <= (size_t)kMaxLds)
        return launch_ring_typed<CT, 2, WH>(rows, G, ncol, image, codes, scales, out, s);
    return QG_E_UNSUPPORTED;
}

// waves per row quarter: the tuning knob's value where it divides the column tiles, else 1
template <int CT>
int launch_ring(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                const qg_act_scale *scales, float *out, hipStream_t s)
{
    const int wh = tuning().mfma_ring_waves;
    if constexpr (CT >= 4)
        if (wh == 4) return launch_ring_d<CT, 4>(rows, G, ncol, image, codes, scales, out, s);
    if constexpr (CT >= 2)
        if (wh == 2) return launch_ring_d<CT, 2>(rows, G, ncol, image, codes, scales, out, s);
    return launch_ring_d<CT, 1>(rows, G, ncol, image, codes, scales, out, s);
}

}  // namespace

int launch_gemm_mfma(int64_t rows, int64_t cols, int64_t ncol, const void *image, const int8_t *codes,
                     const qg_act_scale *scales, float *out, hipStream_t s)
{
    const int G = (int)(cols / 256);
    const int form = tuning().mfma_form;
    int tiles = tuning().mfma_col_tiles;
    // derived (measured on the 14336 x 4096 matrix): up to 16 columns the ring with one column
    // tile, up to 32 the shared-operand form with two, beyond that the shared-operand form
    // with four
    if (form == 1 || (form == 0 && ncol <= 16)) {
        const int ct = tiles > 0 ? tiles : form == 0 ? 1 : ncol >= 48 ? 4 : ncol >= 24 ? 2 : 1;
        int st = QG_E_UNSUPPORTED;
        if (ct == 4) st = launch_ring<4>(rows, G, ncol, image, codes, scales, out, s);
        else if (ct == 2) st = launch_ring<2>(rows, G, ncol, image, codes, scales, out, s);
        else st = launch_ring<1>(rows, G, ncol, image, codes, scales, out, s);
        if (st != QG_E_UNSUPPORTED) return st;
        if (form == 1) return fail(QG_E_UNSUPPORTED, "gemm: rows of %d blocks do not fit the ring's LDS", G);
    }
    if (form == 2 || (form == 0 && ncol > 16)) {
        // shared operands: 2 column tiles up to 32 columns, else 4, unless asked otherwise
        if (tiles == 1) return launch_cw<1>(rows, G, ncol, image, codes, scales, out, s);
        if (tiles == 2 || (tiles == 0 && ncol <= 32)) return launch_cw<2>(rows, G, ncol, image, codes, scales, out, s);
        return launch_cw<4>(rows, G, ncol, image, codes, scales, out, s);
    }
    if (tiles == 2 || (tiles == 0 && ncol >= 32)) return launch_wave<2>(rows, G, ncol, image, codes, scales, out, s);
    return launch_wave<1>(rows, G, ncol, image, codes, scales, out, s);
}

}  // namespace qg
