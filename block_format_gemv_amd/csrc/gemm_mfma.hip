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
// Three forms, chosen by the shape (launch_gemm_mfma):
//   - staged (at most 16 columns, rows of at most 16 blocks): the one-column GEMV's structure,
//     every wave one block of a 16-, 32- or 64-row strip with all its loads issued at once,
//     the activation codes brought into LDS by LDS-DMA, pieces folded after one barrier;
//   - split (more columns on fewer rows, or longer rows): the same structure with the
//     activation operands loaded per wave and rounds of 16 blocks;
//   - shared operands (more columns on many rows): a workgroup owns one 64-row group and
//     16*CW columns, wave (r, c) computes rows 16r..16r+15 against columns 16c..16c+15; per
//     block the workgroup builds, once, the weight operands of its 64 rows (wave (r, c)
//     prepares the 64-element steps c, c+CW, .. of row quarter r) and the activation operands
//     of its columns in an LDS stage; every wave reads what it needs from there.  Two stages
//     alternate, and each thread's global loads run two blocks ahead.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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

// ---------------------------------------------------------------------------------------
// LDS-DMA: global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight into
// LDS (at a wave-uniform base + 16 * lane) without passing through registers.  It is issued from
// inline asm (the compiler would otherwise wait for every outstanding one before each LDS
// read); the kernel waits for its own (s_waitcnt vmcnt with the exact count of younger loads).

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

// ---------------------------------------------------------------------------------------
// The split form: the one-column GEMV's structure on the matrix cores.  A workgroup of 16
// waves owns a strip of 16*RTT rows (inside one 64-row image group) and 16*CT activation
// columns; wave w takes blocks w, w+16, ... (one round of 16 blocks at a time).  Every wave
// issues all the loads of its block at once (its rows' code chunks and block fields in the
// matrix cores' operand order, its columns' activation codes and scale words), so a launch
// keeps the whole weight stream in flight as the GEMV does, with no barrier between loads
// and use.  Per block the wave forms the three products per (16-row, 16-column) tile, combines
// each (row, column) once and parks the piece in LDS; after the round's barrier the first
// RTT*CT waves add each output's pieces in block order, four outputs per lane.
//
// grid: strips x column batches, laid out so that the batches of one strip go to the same
// XCD (workgroups are dealt to the 8 XCDs in turn): x = (s/8 * nbatch + cb) * 8 + s%8, strips
// padded to a multiple of 8 (the padding workgroups exit at once).

template <int RTT, int CT>
struct SplitLds {
    static constexpr int kW = 16;                                // waves
    static constexpr int kSlot = kW * RTT * CT * 1024;           // pieces of a round: [w][rt][ct][lane] x 4 floats
    static constexpr int kScale = 16 * CT * 12;                  // per wave: doubles m*2^e, then the words
    static constexpr int kFlags = 2 * kW;                        // per slot and wave: a tiny piece may occur
    static size_t bytes(int rounds) { return (size_t)(rounds > 1 ? 2 : 1) * kSlot + (size_t)kW * kScale + kFlags; }
};

template <int RTT, int CT>
__global__ __launch_bounds__(1024) void gemm_split_q4k(const uint8_t *image, int rows, int G,
                                                       const int8_t *__restrict__ codes,
                                                       const uint32_t *__restrict__ scw, int ncol, int strips,
                                                       int nbatch, float *__restrict__ out)
{
    using L = SplitLds<RTT, CT>;
    constexpr int W = L::kW;
    constexpr int NC = 16 * CT;
    extern __shared__ __align__(16) unsigned char lds[];
    const int x = (int)blockIdx.x;
    const int qx = x >> 3;
    const int cb = qx % nbatch;
    const int s = (qx / nbatch) * 8 + (x & 7);
    if (s >= strips) return;                   // padding workgroup: the whole group leaves at once
    constexpr int SPG = 4 / RTT;               // strips per 64-row group
    const int g = s / SPG;
    const int qr0 = (s % SPG) * RTT;           // first 16-row quarter of the strip within the group
    const int colbase = cb * NC;
    const int C = G * 256;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int rounds = (G + W - 1) / W;
    unsigned char *slots = lds;
    unsigned char *wscale = lds + (size_t)(rounds > 1 ? 2 : 1) * L::kSlot + (size_t)wid * L::kScale;
    double *sS = reinterpret_cast<double *>(wscale);
    uint32_t *sW = reinterpret_cast<uint32_t *>(wscale + NC * 8);
    unsigned char *flags = lds + (size_t)(rounds > 1 ? 2 : 1) * L::kSlot + (size_t)W * L::kScale;

    // the folding threads: RTT*CT waves, lane l of fold wave u = (rt, ct) owns the four outputs
    // (row 16(qr0+rt) + l%16, columns 16ct + 4(l/16) .. +3)
    const bool folder = wid < RTT * CT;
    float4 y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    const uint8_t *gbase = image + (size_t)g * G * kTileBytesQ4K;
    for (int r = 0; r < rounds; r++) {
        const int b = r * W + wid;
        unsigned char *slot = slots + (size_t)(rounds > 1 ? (r & 1) : 0) * L::kSlot;
        if (b < G) {
            // ---- loads: all of the block's, issued before any is used
            const uint8_t *tile = gbase + (size_t)b * kTileBytesQ4K;
            uint4 ch[RTT][4], meta[RTT];
#pragma unroll
            for (int rt = 0; rt < RTT; rt++) {
                const int trow = 16 * (qr0 + rt) + n;
                meta[rt] = ld16(tile + 8192 + 16 * trow);
#pragma unroll
                for (int st = 0; st < 4; st++) ch[rt][st] = ld16(tile + 1024 * (2 * st + (grp >> 1)) + 16 * trow);
            }
            v4i A[CT][4];
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                const int col = min(colbase + 16 * ct + n, ncol - 1);
                const int8_t *ab = codes + (size_t)col * C + (size_t)b * 256 + 16 * grp;
#pragma unroll
                for (int st = 0; st < 4; st++) A[ct][st] = *reinterpret_cast<const v4i *>(ab + 64 * st);
            }
            // this block's activation scales: lane j < NC loads column colbase + j's word
            const uint32_t w = scw[(size_t)min(colbase + min(lane, NC - 1), ncol - 1) * G + b];
            if (lane < NC) {
                sW[lane] = w;
                sS[lane] = __builtin_ldexp((double)((w >> 16) & 0xFFu), (int)(int16_t)(w & 0xFFFFu));
            }
            const bool tiny_col = lane < NC && (int)(int16_t)(w & 0xFFFFu) < kNoTinyExp;
            const bool tiny = __any(tiny_col);   // a piece of this block may be tiny: flushed combine and fold

            // ---- per row tile: weight operands, products, combine
#pragma unroll
            for (int rt = 0; rt < RTT; rt++) {
                // the lane's four sub-block fields: sub-block 2st + grp/2, 12 bits at 12(2st + grp/2)
                // of the 96-bit string; shifting the string by 12(grp/2) puts them at 24st
                const uint32_t sh = 12u * (uint32_t)(grp >> 1);
                const uint64_t lo64 = ((uint64_t)meta[rt].z << 32 | meta[rt].y) >> sh;
                const uint32_t y0 = (uint32_t)lo64;
                const uint32_t y1 = (uint32_t)(((uint64_t)meta[rt].w << 32 | meta[rt].z) >> sh);
                const uint32_t y2 = meta[rt].w >> sh;
                const uint32_t fs[4] = {y0 & 0xFFFu, (uint32_t)(lo64 >> 24) & 0xFFFu, (y1 >> 16) & 0xFFFu,
                                        (y2 >> 8) & 0xFFFu};
                v4i acc_h[CT], acc_l[CT], acc_o[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ct++) acc_h[ct] = acc_l[ct] = acc_o[ct] = v4i{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    const uint32_t f = fs[st];
                    const uint32_t hi = (f >> 3) & 7u, lo = f & 7u, mn = f >> 6;
                    const int shq = 4 * (grp & 1);   // low nibbles: elements 0..15, high: 16..31
                    const uint4 c4 = ch[rt][st];
                    const uint32_t q0 = (c4.x >> shq) & 0x0F0F0F0Fu, q1 = (c4.y >> shq) & 0x0F0F0F0Fu;
                    const uint32_t q2 = (c4.z >> shq) & 0x0F0F0F0Fu, q3 = (c4.w >> shq) & 0x0F0F0F0Fu;
                    const v4i Bh = {bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi)};
                    const v4i Bl = {bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo)};
                    const int mrep = (int)(mn * 0x01010101u);
                    const v4i Bo = {mrep, mrep, mrep, mrep};
#pragma unroll
                    for (int ct = 0; ct < CT; ct++) {
                        acc_h[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[ct][st], Bh, acc_h[ct], 0, 0, 0);
                        acc_l[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[ct][st], Bl, acc_l[ct], 0, 0, 0);
                        acc_o[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[ct][st], Bo, acc_o[ct], 0, 0, 0);
                    }
                }
                // combine each (row, column) once ("Module numerics", module description: the
                // block's terms summed exactly and rounded once)
                const uint32_t dd = meta[rt].x;
                const float fd = f16_value(dd), fm = f16_value(dd >> 16);
                const bool near = q4k_near(fd, fm);
                const double Dd = (double)fd, Dm = (double)fm;
#pragma unroll
                for (int ct = 0; ct < CT; ct++) {
                    const double *S = sS + 16 * ct + 4 * grp;
                    float p[4];
                    if (__all(near) && !tiny) {
                        // no piece is tiny: the conversion needs no flush, + 0 turns an exact -0 into +0
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int Cb = 8 * acc_h[ct][i] + acc_l[ct][i];
                            const double X = __builtin_fma((double)Cb, Dd, -((double)acc_o[ct][i] * Dm));
                            p[i] = (float)(X * S[i]) + 0.0f;
                        }
                    } else {
                        const uint32_t *Wd = sW + 16 * ct + 4 * grp;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int Cb = 8 * acc_h[ct][i] + acc_l[ct][i];
                            const int Ob = acc_o[ct][i];
                            if (near) {
                                p[i] = piece_q4k_perblock_near(Cb, Ob, Dd, Dm, S[i]);
                            } else {
                                const int m = (int)((Wd[i] >> 16) & 0xFFu);
                                const int e = (int)(int16_t)(Wd[i] & 0xFFFFu);
                                p[i] = piece_q4k_perblock(Cb, Ob, dd, m, e);
                            }
                        }
                    }
                    reinterpret_cast<float4 *>(slot)[((wid * RTT + rt) * CT + ct) * 64 + lane] =
                        make_float4(p[0], p[1], p[2], p[3]);
                }
            }
            if (lane == 0) flags[(r & 1) * W + wid] = tiny ? 1 : 0;
        }
        __syncthreads();
        if (folder) {
            // add the round's pieces in block order, plain adds unless one of them may be tiny
            const int nb = min(W, G - r * W);
            bool flush = false;
            for (int k = 0; k < nb; k++) flush |= flags[(r & 1) * W + k] != 0;
            const float4 *pc = reinterpret_cast<const float4 *>(slot) + (size_t)wid * 64 + lane;
            const size_t stride = (size_t)RTT * CT * 64;
            if (flush) {
                for (int k = 0; k < nb; k++) {
                    const float4 q = pc[k * stride];
                    y.x = fadd_ftz(y.x, q.x);
                    y.y = fadd_ftz(y.y, q.y);
                    y.z = fadd_ftz(y.z, q.z);
                    y.w = fadd_ftz(y.w, q.w);
                }
            } else if (nb == W) {
                float4 q[W];
#pragma unroll
                for (int k = 0; k < W; k++) q[k] = pc[k * stride];
#pragma unroll
                for (int k = 0; k < W; k++) {
                    y.x = y.x + q[k].x;
                    y.y = y.y + q[k].y;
                    y.z = y.z + q[k].z;
                    y.w = y.w + q[k].w;
                }
            } else {
                for (int k = 0; k < nb; k++) {
                    const float4 q = pc[k * stride];
                    y.x = y.x + q.x;
                    y.y = y.y + q.y;
                    y.z = y.z + q.z;
                    y.w = y.w + q.w;
                }
            }
        }
    }

    if (folder) {
        const int rt = wid / CT, ct = wid % CT;
        const int64_t row = (int64_t)g * 64 + 16 * (qr0 + rt) + n;
        if (row < rows) {
            const float v[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = colbase + 16 * ct + 4 * grp + i;
                if (col < ncol) out[(int64_t)col * rows + row] = canon_nan(v[i]);
            }
        }
    }
}

template <int RTT, int CT>
int launch_split_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                       const qg_act_scale *scales, float *out, hipStream_t s)
{
    using L = SplitLds<RTT, CT>;
    const int64_t groups = (rows + 63) / 64;
    const int64_t strips = groups * (4 / RTT);
    const int64_t nbatch = (ncol + 16 * CT - 1) / (16 * CT);
    const int64_t grid = (strips + 7) / 8 * 8 * nbatch;
    if (grid > 0x7fffffff) return fail(QG_E_SHAPE, "gemm: %lld rows x %lld columns is too many", (long long)rows,
                                       (long long)ncol);
    const int rounds = (G + L::kW - 1) / L::kW;
    const size_t lds = L::bytes(rounds);
    if (lds > (size_t)kMaxLds) return QG_E_UNSUPPORTED;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_split_q4k<RTT, CT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    (void)attr;   // a refusal shows up as a launch error below
    const uint32_t *w = reinterpret_cast<const uint32_t *>(scales);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemm_split_q4k<RTT, CT>), dim3((unsigned)grid), dim3(1024), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, (int)strips,
                              (int)nbatch, out);
    else
        hipLaunchKernelGGL((gemm_split_q4k<RTT, CT>), dim3((unsigned)grid), dim3(1024), lds, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, (int)strips,
                           (int)nbatch, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores, split) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

// ---------------------------------------------------------------------------------------
// The staged form (at most 16 columns, rows of at most 16 blocks): the split form's workgroup
// (16 waves, wave w takes block w for the strip's 16*RTT rows) with the activation codes of its
// columns staged in LDS.  A column's codes of four consecutive blocks are 1 KiB contiguous, so
// each wave brings those of its own block's group of four with one LDS-DMA instruction per
// column (each column's row padded by 16 bytes in LDS, so that the 16 lanes of an operand read,
// one per column, fall in different banks), issued before its weights, and waits for its own
// loads only: the four waves of a group write the same bytes to the same place.  Weights load
// straight into registers, each lane 8 bytes of one code chunk per 64-element step (the K
// order of the tile form).
//
// LDS: the codes [nc][C + 16] (nc = the columns, at most 16), the pieces [16 waves][RTT][64
// lanes] x 4 floats, the waves' scale tables, the tiny-piece flags.

template <int RTT>
struct StagedLds {
    // nc = the columns staged (at most 16)
    __host__ __device__ static size_t codes(int C, int nc) { return (size_t)nc * (C + 16); }
    static constexpr int kPieces = 16 * RTT * 1024;
    static constexpr int kScale = 16 * 12;
    __host__ __device__ static size_t bytes(int C, int nc) { return codes(C, nc) + kPieces + 16 * (size_t)kScale + 16; }
};

template <int RTT>
__global__ __launch_bounds__(1024) void gemm_staged_q4k(const uint8_t *image, int rows, int G,
                                                        const int8_t *__restrict__ codes,
                                                        const uint32_t *__restrict__ scw, int ncol, int strips,
                                                        float *__restrict__ out)
{
    using L = StagedLds<RTT>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int s = (int)blockIdx.x;
    constexpr int SPG = 4 / RTT;               // strips per 64-row group
    const int g = s / SPG;
    const int qr0 = (s % SPG) * RTT;
    const int C = G * 256, cs = C + 16;
    const int nc = min(ncol, 16);
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, grp = lane >> 4, h = grp & 1, jo = grp >> 1;
    const int b = min(wid, G - 1);             // a wave past the last block works on a copy and parks nothing
    const bool live = wid < G;
    unsigned char *acodes = lds;
    float *pieces = reinterpret_cast<float *>(lds + L::codes(C, nc));
    unsigned char *wscale = lds + L::codes(C, nc) + L::kPieces + (size_t)wid * L::kScale;
    double *sS = reinterpret_cast<double *>(wscale);
    uint32_t *sW = reinterpret_cast<uint32_t *>(wscale + 16 * 8);
    unsigned char *flags = lds + L::codes(C, nc) + L::kPieces + 16 * (size_t)L::kScale;

    // the columns' codes of this wave's group of four blocks (gq = b / 4) into LDS: one DMA
    // instruction per column, 16 bytes per lane (lane l: block 4gq + l/16).  The four waves of
    // a group bring the same bytes to the same place, so each wave only waits for its own loads.
    const int gq = b >> 2;
    for (int c = 0; c < nc; c++) {
        if (4 * gq + (lane >> 4) < G)
            dma16(codes + (size_t)c * C + 1024 * gq + 16 * lane, lds_offset(acodes + (size_t)c * cs + 1024 * gq));
    }
    // the block's weights: lane (n, grp) reads row 16(qr0 + rt) + n, 8 bytes at 8h of code chunk
    // 2st + jo for each step st, and the row's block fields
    const uint8_t *tile = image + ((size_t)g * G + b) * kTileBytesQ4K;
    uint2 ch[RTT][4];
    uint4 meta[RTT];
#pragma unroll
    for (int rt = 0; rt < RTT; rt++) {
        const int trow = 16 * (qr0 + rt) + n;
        meta[rt] = ld16(tile + 8192 + 16 * trow);
#pragma unroll
        for (int st = 0; st < 4; st++)
            ch[rt][st] = *reinterpret_cast<const uint2 *>(tile + 1024 * (2 * st + jo) + 16 * trow + 8 * h);
    }
    const uint32_t w = scw[(size_t)min(lane & 15, ncol - 1) * G + b];
    // the DMA loads were issued first: waiting for at most 5*RTT + 1 younger loads leaves them done
    wait_vm<5 * RTT + 1>();

    if (lane < 16) {
        sW[lane] = w;
        sS[lane] = __builtin_ldexp((double)((w >> 16) & 0xFFu), (int)(int16_t)(w & 0xFFFFu));
    }
    const bool tiny = __any(lane < 16 && (int)(int16_t)(w & 0xFFFFu) < kNoTinyExp);
    // this lane's activation operand of step st: codes of column n (past the last column, a
    // copy of it: computed and dropped), elements 32(2st + jo) + 8h .. +7 and +16 .. +23 of block b
    const unsigned char *arow = acodes + (size_t)min(n, nc - 1) * cs + (size_t)b * 256 + 32 * jo + 8 * h;
#pragma unroll
    for (int rt = 0; rt < RTT; rt++) {
        const uint32_t sh = 12u * (uint32_t)jo;
        const uint64_t lo64 = ((uint64_t)meta[rt].z << 32 | meta[rt].y) >> sh;
        const uint32_t y1 = (uint32_t)(((uint64_t)meta[rt].w << 32 | meta[rt].z) >> sh);
        const uint32_t y2 = meta[rt].w >> sh;
        const uint32_t fs[4] = {(uint32_t)lo64 & 0xFFFu, (uint32_t)(lo64 >> 24) & 0xFFFu, (y1 >> 16) & 0xFFFu,
                                (y2 >> 8) & 0xFFFu};
        v4i ah = {0, 0, 0, 0}, al = {0, 0, 0, 0}, ao = {0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < 4; st++) {
            const uint2 lo8 = *reinterpret_cast<const uint2 *>(arow + 64 * st);
            const uint2 hi8 = *reinterpret_cast<const uint2 *>(arow + 64 * st + 16);
            const v4i A = {(int)lo8.x, (int)lo8.y, (int)hi8.x, (int)hi8.y};
            const uint32_t f = fs[st];
            const uint32_t hi = (f >> 3) & 7u, lo = f & 7u;
            const int mr = (int)__builtin_amdgcn_perm(0u, f >> 6, 0x00000000u);   // mn (< 64) in every byte
            const uint2 c2 = ch[rt][st];
            const uint32_t q0 = c2.x & 0x0F0F0F0Fu, q1 = c2.y & 0x0F0F0F0Fu;
            const uint32_t q2 = (c2.x >> 4) & 0x0F0F0F0Fu, q3 = (c2.y >> 4) & 0x0F0F0F0Fu;
            const v4i Bh = {bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi)};
            const v4i Bl = {bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo)};
            const v4i Bo = {mr, mr, mr, mr};
            ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bh, ah, 0, 0, 0);
            al = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bl, al, 0, 0, 0);
            ao = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bo, ao, 0, 0, 0);
        }
        const uint32_t dd = meta[rt].x;
        const float fd = f16_value(dd), fm = f16_value(dd >> 16);
        const bool near = q4k_near(fd, fm);
        const double Dd = (double)fd, Dm = (double)fm;
        const double *S = sS + 4 * grp;
        float p[4];
        if (__all(near) && !tiny) {
            // no piece is tiny: the conversion needs no flush; an exact -0 is added to +0 or to
            // a nonzero partial sum by the fold, which gives what +0 would
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int Cb = 8 * ah[i] + al[i];
                const double X = __builtin_fma((double)Cb, Dd, -((double)ao[i] * Dm));
                p[i] = (float)(X * S[i]);
            }
        } else {
            const uint32_t *Wd = sW + 4 * grp;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int Cb = 8 * ah[i] + al[i];
                if (near) {
                    p[i] = piece_q4k_perblock_near(Cb, ao[i], Dd, Dm, S[i]);
                } else {
                    const int m = (int)((Wd[i] >> 16) & 0xFFu);
                    const int e = (int)(int16_t)(Wd[i] & 0xFFFFu);
                    p[i] = piece_q4k_perblock(Cb, ao[i], dd, m, e);
                }
            }
        }
        if (live) reinterpret_cast<float4 *>(pieces)[(wid * RTT + rt) * 64 + lane] = make_float4(p[0], p[1], p[2], p[3]);
    }
    if (lane == 0) flags[wid] = live && tiny ? 1 : 0;
    __syncthreads();

    // fold: thread t takes row tile t/256 and output o = t%256 of it (o = 4 lane' + i: row
    // lane' % 16, column 4 (lane' / 16) + i); block k's piece of it is float (k*RTT + rt)*256 + o
    const int t = (int)threadIdx.x;
    if (t < 256 * RTT) {
        const int frt = t >> 8, o = t & 255;
        const uint4 fw = *reinterpret_cast<const uint4 *>(flags);
        const uint32_t fm4[4] = {fw.x, fw.y, fw.z, fw.w};
        uint32_t any = 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int keep = min(max(G - 4 * q, 0), 4);
            any |= keep == 4 ? fm4[q] : fm4[q] & ((1u << (8 * keep)) - 1u);
        }
        const float *pc = pieces + frt * 256 + o;
        const size_t stride = (size_t)RTT * 256;
        float y = 0.0f;
        if (any != 0) {
            for (int k = 0; k < G; k++) y = fadd_ftz(y, pc[k * stride]);
        } else if (G == 16) {
            float q[16];
#pragma unroll
            for (int k = 0; k < 16; k++) q[k] = pc[k * stride];
#pragma unroll
            for (int k = 0; k < 16; k++) y = y + q[k];
        } else {
            for (int k = 0; k < G; k++) y = y + pc[k * stride];
        }
        const int lp = o >> 2, i = o & 3;
        const int64_t row = (int64_t)g * 64 + 16 * (qr0 + frt) + (lp & 15);
        const int col = 4 * (lp >> 4) + i;
        if (row < rows && col < ncol) out[(int64_t)col * rows + row] = canon_nan(y);
    }
}

template <int RTT>
int launch_staged_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                        const qg_act_scale *scales, float *out, hipStream_t s)
{
    using L = StagedLds<RTT>;
    const int64_t strips = (rows + 63) / 64 * (4 / RTT);
    if (strips > 0x7fffffff) return fail(QG_E_SHAPE, "gemm: %lld rows is too many", (long long)rows);
    const size_t lds = L::bytes(G * 256, (int)std::min<int64_t>(ncol, 16));
    if (lds > (size_t)kMaxLds) return QG_E_UNSUPPORTED;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_staged_q4k<RTT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    (void)attr;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(scales);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemm_staged_q4k<RTT>), dim3((unsigned)strips), dim3(1024), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, (int)strips, out);
    else
        hipLaunchKernelGGL((gemm_staged_q4k<RTT>), dim3((unsigned)strips), dim3(1024), lds, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, (int)strips, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores, staged) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

// ---------------------------------------------------------------------------------------
// The column-resident form (rows of at most 16 blocks with two column tiles, at most 32 with
// one): a workgroup of W <= 8 waves owns W row tiles of 16 rows (tile t: rows 16t .. 16t+15, quarter
// t%4 of 64-row image group t/4) and 16*CT activation columns.  At the start it brings every
// block's codes of its columns into LDS by LDS-DMA (the staged form's layout: column rows
// padded by 16 bytes) and its columns' activation scales per block into tables; one barrier.
// After it each wave walks its tile's blocks alone, with no further barrier: its rows' code
// chunks and block fields loaded six blocks ahead into a register ring, blocks taken two at a
// time (the three products per column tile of both, from LDS operands in the staged form's K
// order, formed step by step together), each (row, column) combined once and added in block
// order to the lane's running sums in registers.  The waves of a SIMD
// drift apart, so the matrix unit and the vector ALU serve different waves at once.
//
// grid: row chunks x column batches, the batches of one chunk on one XCD (x = (chunk/8 *
// nbatch + cb) * 8 + chunk%8, chunks padded to a multiple of 8), so that L2 serves the weight
// tiles to both.

#ifndef QG_RESIDENT_RING
#define QG_RESIDENT_RING 6
#endif
constexpr int kResidentRing = QG_RESIDENT_RING;   // blocks of weight loads in flight per wave

template <int CT>
struct ResidentLds {
    __host__ __device__ static size_t codes(int C) { return (size_t)16 * CT * (C + 16); }
    // the activation scales per (block, column): m*2^e as a double, then the word
    __host__ __device__ static size_t bytes(int C, int G) { return codes(C) + (size_t)G * 16 * CT * 12; }
};

// one block's loads of a row tile: the row's block fields and, per 64-element step st, the 8
// bytes at 8h of code chunk 2st + jo (the staged form's K order)
__device__ __forceinline__ void resident_load(const uint8_t *tile, int trow, int jo, int h, uint4 &meta, uint2 (&ch)[4])
{
    meta = ld16(tile + 8192 + 16 * trow);
#pragma unroll
    for (int st = 0; st < 4; st++) ch[st] = *reinterpret_cast<const uint2 *>(tile + 1024 * (2 * st + jo) + 16 * trow + 8 * h);
}

// one block of a wave's row tile against its CT column tiles, added to y (TINY: some piece of
// the workgroup may be tiny, so every piece is combined with the flush and added flushed)
template <int CT, bool TINY>
__device__ __forceinline__ void resident_block(const uint4 &meta, const uint2 (&ch)[4], const unsigned char *acodes,
                                               int cs, int b, const double *sSb, const uint32_t *sWb, int lane,
                                               float (&y)[CT][4])
{
    const int n = lane & 15, grp = lane >> 4, h = grp & 1, jo = grp >> 1;
    const uint32_t sh = 12u * (uint32_t)jo;
    const uint64_t lo64 = ((uint64_t)meta.z << 32 | meta.y) >> sh;
    const uint32_t y1 = (uint32_t)(((uint64_t)meta.w << 32 | meta.z) >> sh);
    const uint32_t y2 = meta.w >> sh;
    const uint32_t fs[4] = {(uint32_t)lo64 & 0xFFFu, (uint32_t)(lo64 >> 24) & 0xFFFu, (y1 >> 16) & 0xFFFu,
                            (y2 >> 8) & 0xFFFu};
    v4i ah[CT], al[CT], ao[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ct++) ah[ct] = al[ct] = ao[ct] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const uint32_t f = fs[st];
        const uint32_t hi = (f >> 3) & 7u, lo = f & 7u;
        const int mr = (int)__builtin_amdgcn_perm(0u, f >> 6, 0x00000000u);   // mn (< 64) in every byte
        const uint2 c2 = ch[st];
        const uint32_t q0 = c2.x & 0x0F0F0F0Fu, q1 = c2.y & 0x0F0F0F0Fu;
        const uint32_t q2 = (c2.x >> 4) & 0x0F0F0F0Fu, q3 = (c2.y >> 4) & 0x0F0F0F0Fu;
        const v4i Bh = {bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi)};
        const v4i Bl = {bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo)};
        const v4i Bo = {mr, mr, mr, mr};
#pragma unroll
        for (int ct = 0; ct < CT; ct++) {
            // column 16ct + n, elements 32(2st + jo) + 8h .. +7 and +16 .. +23 of block b
            const unsigned char *arow = acodes + (size_t)(16 * ct + n) * cs + (size_t)b * 256 + 32 * jo + 8 * h + 64 * st;
            const uint2 lo8 = *reinterpret_cast<const uint2 *>(arow);
            const uint2 hi8 = *reinterpret_cast<const uint2 *>(arow + 16);
            const v4i A = {(int)lo8.x, (int)lo8.y, (int)hi8.x, (int)hi8.y};
            ah[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bh, ah[ct], 0, 0, 0);
            al[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bl, al[ct], 0, 0, 0);
            ao[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bo, ao[ct], 0, 0, 0);
        }
    }
    // combine each (row, column) once ("Module numerics", module description) and add it
    const uint32_t dd = meta.x;
    const float fd = f16_value(dd), fm = f16_value(dd >> 16);
    const bool near = q4k_near(fd, fm);
    const double Dd = (double)fd, Dm = (double)fm;
    if (!TINY && __all(near)) {
        // no piece is tiny: the conversion needs no flush; an exact -0 added to +0 or to a
        // nonzero partial sum gives what +0 would.  One straight run for the whole block, so
        // the scale reads are issued together.
#pragma unroll
        for (int ct = 0; ct < CT; ct++) {
            const double *S = sSb + 16 * ct + 4 * grp;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int Cb = 8 * ah[ct][i] + al[ct][i];
                const double X = __builtin_fma((double)Cb, Dd, -((double)ao[ct][i] * Dm));
                y[ct][i] = y[ct][i] + (float)(X * S[i]);
            }
        }
        return;
    }
#pragma unroll
    for (int ct = 0; ct < CT; ct++) {
        const double *S = sSb + 16 * ct + 4 * grp;
        const uint32_t *Wd = sWb + 16 * ct + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int Cb = 8 * ah[ct][i] + al[ct][i];
            float pc;
            if (near) {
                pc = piece_q4k_perblock_near(Cb, ao[ct][i], Dd, Dm, S[i]);
            } else {
                const int m = (int)((Wd[i] >> 16) & 0xFFu);
                const int e = (int)(int16_t)(Wd[i] & 0xFFFFu);
                pc = piece_q4k_perblock(Cb, ao[ct][i], dd, m, e);
            }
            y[ct][i] = TINY ? fadd_ftz(y[ct][i], pc) : y[ct][i] + pc;
        }
    }
}

// two consecutive blocks of a wave's row tile: the products of both formed step by step
// together (twice the independent matrix and vector work between waits), then each block
// combined and added to y in block order, as resident_block does
template <int CT, bool TINY>
__device__ __forceinline__ void resident_pair(const uint4 &m0, const uint2 (&c0)[4], const uint4 &m1,
                                              const uint2 (&c1)[4], const unsigned char *acodes, int cs, int b,
                                              const double *sSb, const uint32_t *sWb, int lane, float (&y)[CT][4])
{
    constexpr int NC = 16 * CT;
    const int n = lane & 15, grp = lane >> 4, h = grp & 1, jo = grp >> 1;
    const uint32_t sh = 12u * (uint32_t)jo;
    uint32_t fs[2][4];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const uint4 &meta = u ? m1 : m0;
        const uint64_t lo64 = ((uint64_t)meta.z << 32 | meta.y) >> sh;
        const uint32_t y1 = (uint32_t)(((uint64_t)meta.w << 32 | meta.z) >> sh);
        const uint32_t y2 = meta.w >> sh;
        fs[u][0] = (uint32_t)lo64 & 0xFFFu;
        fs[u][1] = (uint32_t)(lo64 >> 24) & 0xFFFu;
        fs[u][2] = (y1 >> 16) & 0xFFFu;
        fs[u][3] = (y2 >> 8) & 0xFFFu;
    }
    v4i ah[2][CT], al[2][CT], ao[2][CT];
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
        for (int ct = 0; ct < CT; ct++) ah[u][ct] = al[u][ct] = ao[u][ct] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < 4; st++) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const uint32_t f = fs[u][st];
            const uint32_t hi = (f >> 3) & 7u, lo = f & 7u;
            const int mr = (int)__builtin_amdgcn_perm(0u, f >> 6, 0x00000000u);
            const uint2 c2 = u ? c1[st] : c0[st];
            const uint32_t q0 = c2.x & 0x0F0F0F0Fu, q1 = c2.y & 0x0F0F0F0Fu;
            const uint32_t q2 = (c2.x >> 4) & 0x0F0F0F0Fu, q3 = (c2.y >> 4) & 0x0F0F0F0Fu;
            const v4i Bh = {bytes_times(q0, hi), bytes_times(q1, hi), bytes_times(q2, hi), bytes_times(q3, hi)};
            const v4i Bl = {bytes_times(q0, lo), bytes_times(q1, lo), bytes_times(q2, lo), bytes_times(q3, lo)};
            const v4i Bo = {mr, mr, mr, mr};
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                const unsigned char *arow =
                    acodes + (size_t)(16 * ct + n) * cs + (size_t)(b + u) * 256 + 32 * jo + 8 * h + 64 * st;
                const uint2 lo8 = *reinterpret_cast<const uint2 *>(arow);
                const uint2 hi8 = *reinterpret_cast<const uint2 *>(arow + 16);
                const v4i A = {(int)lo8.x, (int)lo8.y, (int)hi8.x, (int)hi8.y};
                ah[u][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bh, ah[u][ct], 0, 0, 0);
                al[u][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bl, al[u][ct], 0, 0, 0);
                ao[u][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bo, ao[u][ct], 0, 0, 0);
            }
        }
    }
    // combine each (row, column) once ("Module numerics", module description) and add it
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const uint32_t dd = u ? m1.x : m0.x;
        const double *S0 = sSb + (size_t)u * NC;
        const uint32_t *W0 = sWb + (size_t)u * NC;
        const float fd = f16_value(dd), fm = f16_value(dd >> 16);
        const bool near = q4k_near(fd, fm);
        const double Dd = (double)fd, Dm = (double)fm;
        if (!TINY && __all(near)) {
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                const double *S = S0 + 16 * ct + 4 * grp;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int Cb = 8 * ah[u][ct][i] + al[u][ct][i];
                    const double X = __builtin_fma((double)Cb, Dd, -((double)ao[u][ct][i] * Dm));
                    y[ct][i] = y[ct][i] + (float)(X * S[i]);
                }
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ct++) {
                const double *S = S0 + 16 * ct + 4 * grp;
                const uint32_t *Wd = W0 + 16 * ct + 4 * grp;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int Cb = 8 * ah[u][ct][i] + al[u][ct][i];
                    float pc;
                    if (near) {
                        pc = piece_q4k_perblock_near(Cb, ao[u][ct][i], Dd, Dm, S[i]);
                    } else {
                        const int m = (int)((Wd[i] >> 16) & 0xFFu);
                        const int e = (int)(int16_t)(Wd[i] & 0xFFFFu);
                        pc = piece_q4k_perblock(Cb, ao[u][ct][i], dd, m, e);
                    }
                    y[ct][i] = TINY ? fadd_ftz(y[ct][i], pc) : y[ct][i] + pc;
                }
            }
        }
    }
}

template <int CT, bool TINY, int D>
__device__ __forceinline__ void resident_walk(const uint8_t *gbase, int G, int trow, const unsigned char *acodes,
                                              int cs, const double *sS, const uint32_t *sW, int lane, float (&y)[CT][4])
{
    constexpr int NC = 16 * CT;
    const int grp = lane >> 4, h = grp & 1, jo = grp >> 1;
    // a ring of D register sets, set k holding blocks k, k+D, ...: each is used and then
    // refilled in place with the block D ahead (past the last block: the last again, unused),
    // so no register with a load in flight is ever copied and the compiler's wait before a use
    // counts the younger loads exactly, across the loop's back edge too
    uint4 m[D];
    uint2 c[D][4];
#pragma unroll
    for (int k = 0; k < D; k++) resident_load(gbase + (size_t)min(k, G - 1) * kTileBytesQ4K, trow, jo, h, m[k], c[k]);
    int b = 0;
#pragma unroll 1
    for (; b + D <= G; b += D) {             // whole rounds: a straight-line body
#pragma unroll
        for (int k = 0; k < D; k += 2) {
            resident_pair<CT, TINY>(m[k], c[k], m[k + 1], c[k + 1], acodes, cs, b + k, sS + (size_t)(b + k) * NC,
                                    sW + (size_t)(b + k) * NC, lane, y);
            resident_load(gbase + (size_t)min(b + k + D, G - 1) * kTileBytesQ4K, trow, jo, h, m[k], c[k]);
            resident_load(gbase + (size_t)min(b + k + 1 + D, G - 1) * kTileBytesQ4K, trow, jo, h, m[k + 1], c[k + 1]);
        }
    }
    // the last blocks, fewer than D
#pragma unroll
    for (int k = 0; k < D - 1; k += 2) {
        if (b + k + 1 < G)
            resident_pair<CT, TINY>(m[k], c[k], m[k + 1], c[k + 1], acodes, cs, b + k, sS + (size_t)(b + k) * NC,
                                    sW + (size_t)(b + k) * NC, lane, y);
        else if (b + k < G)
            resident_block<CT, TINY>(m[k], c[k], acodes, cs, b + k, sS + (size_t)(b + k) * NC, sW + (size_t)(b + k) * NC,
                                     lane, y);
    }
}

template <int CT, int GT>
__global__ __launch_bounds__(512) void gemm_resident_q4k(const uint8_t *image, int rows, int G_arg,
                                                          const int8_t *__restrict__ codes,
                                                          const uint32_t *__restrict__ scw, int ncol, int tiles,
                                                          int chunks, int nbatch, float *__restrict__ out)
{
    using L = ResidentLds<CT>;
    constexpr int NC = 16 * CT;
    const int G = GT ? GT : G_arg;
    extern __shared__ __align__(16) unsigned char lds[];
    const int x = (int)blockIdx.x;
    const int qx = x >> 3;
    const int cb = qx % nbatch;
    const int chunk = (qx / nbatch) * 8 + (x & 7);
    if (chunk >= chunks) return;               // padding workgroup: the whole group leaves at once
    const int W = (int)(blockDim.x >> 6);
    const int C = G * 256, cs = C + 16;
    const int colbase = cb * NC;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned char *acodes = lds;
    double *sS = reinterpret_cast<double *>(lds + L::codes(C));
    uint32_t *sW = reinterpret_cast<uint32_t *>(sS + (size_t)G * NC);

    // the columns' codes: DMA instruction k moves 1 KiB (piece k % P of column k / P, P = the
    // 1 KiB pieces of a row, the last possibly partial: its lanes past the row load nothing);
    // wave w issues k = w, w + W, ...  A column past the last is a copy of the last (dropped).
    const int P = (C + 1023) / 1024;
    for (int k = wid; k < NC * P; k += W) {
        const int j = k / P, pk = k % P;
        if (1024 * pk + 16 * lane < C)
            dma16(codes + (size_t)min(colbase + j, ncol - 1) * C + 1024 * pk + 16 * lane,
                  lds_offset(acodes + (size_t)j * cs + 1024 * pk));
    }
    // the activation scales, [block][column]
    for (int i = threadIdx.x; i < NC * G; i += (int)blockDim.x) {
        const int b = i / NC, j = i % NC;
        const uint32_t w = scw[(size_t)min(colbase + j, ncol - 1) * G + b];
        sW[i] = w;
        sS[i] = __builtin_ldexp((double)((w >> 16) & 0xFFu), (int)(int16_t)(w & 0xFFFFu));
    }
    wait_vm<0>();                              // this wave's DMA and table loads have landed
    __syncthreads();

    const int t = chunk * W + wid;             // this wave's row tile
    if (t >= tiles) return;                    // no barrier follows
    // whether any piece of the workgroup may be tiny: an activation exponent below the bound
    bool tiny = false;
    for (int i = lane; i < NC * G; i += 64) tiny |= (int)(int16_t)(sW[i] & 0xFFFFu) < kNoTinyExp;
    tiny = __any(tiny);

    const int g = t >> 2, trow = 16 * (t & 3) + (lane & 15);
    const uint8_t *gbase = image + (size_t)g * G * kTileBytesQ4K;
    float y[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ct++) y[ct][0] = y[ct][1] = y[ct][2] = y[ct][3] = 0.0f;
    if (tiny) resident_walk<CT, true, kResidentRing>(gbase, G, trow, acodes, cs, sS, sW, lane, y);
    else resident_walk<CT, false, kResidentRing>(gbase, G, trow, acodes, cs, sS, sW, lane, y);

    const int64_t row = (int64_t)g * 64 + trow;
    if (row < rows) {
#pragma unroll
        for (int ct = 0; ct < CT; ct++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = colbase + 16 * ct + 4 * (lane >> 4) + i;
                if (col < ncol) out[(int64_t)col * rows + row] = canon_nan(y[ct][i]);
            }
    }
}

template <int CT, int GT>
int launch_resident_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                          const qg_act_scale *scales, float *out, hipStream_t s)
{
    using L = ResidentLds<CT>;
    const size_t lds = L::bytes(G * 256, G);
    if (lds > (size_t)kMaxLds) return QG_E_UNSUPPORTED;
    const int64_t tiles = (rows + 63) / 64 * 4;
    const int64_t nbatch = (ncol + 16 * CT - 1) / (16 * CT);
    // waves per workgroup: the tuning knob if set, else enough to spread every (tile, batch)
    // over the CUs one workgroup each
    int W = tuning().gemm_row_tiles;
    if (W <= 0) {
        const int64_t cus = device_cu_count();
        W = (int)std::min<int64_t>(8, std::max<int64_t>(1, (tiles * nbatch + cus - 1) / cus));
    }
    if (W > 8) W = 8;                          // 512 threads: 256 registers a lane
    const int64_t chunks = (tiles + W - 1) / W;
    const int64_t grid = (chunks + 7) / 8 * 8 * nbatch;
    if (grid > 0x7fffffff) return fail(QG_E_SHAPE, "gemm: %lld rows x %lld columns is too many", (long long)rows,
                                       (long long)ncol);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_resident_q4k<CT, GT>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    (void)attr;   // a refusal shows up as a launch error below
    const uint32_t *w = reinterpret_cast<const uint32_t *>(scales);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemm_resident_q4k<CT, GT>), dim3((unsigned)grid), dim3(64 * W), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, (int)tiles,
                              (int)chunks, (int)nbatch, out);
    else
        hipLaunchKernelGGL((gemm_resident_q4k<CT, GT>), dim3((unsigned)grid), dim3(64 * W), lds, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, codes, w, (int)ncol, (int)tiles,
                           (int)chunks, (int)nbatch, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores, column-resident) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

// two column tiles per workgroup where the rows' codes fit (at most 16 blocks), else one
int launch_resident(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                    const qg_act_scale *scales, float *out, hipStream_t s)
{
    int ct = tuning().mfma_col_tiles;
    if (ct == 0) ct = G <= 16 && ncol > 16 ? 2 : 1;
    int st = QG_E_UNSUPPORTED;
    if (ct == 2) st = G == 16 ? launch_resident_typed<2, 16>(rows, G, ncol, image, codes, scales, out, s)
                              : launch_resident_typed<2, 0>(rows, G, ncol, image, codes, scales, out, s);
    else if (ct == 1) st = G == 16 ? launch_resident_typed<1, 16>(rows, G, ncol, image, codes, scales, out, s)
                                   : launch_resident_typed<1, 0>(rows, G, ncol, image, codes, scales, out, s);
    if (st == QG_E_UNSUPPORTED)
        return fail(QG_E_UNSUPPORTED, "gemm: the column-resident form's LDS does not fit %d blocks of %d column tiles",
                    G, ct);
    return st;
}

// row tiles and column tiles per workgroup: the tuning knobs if set, else derived from the
// shape (enough workgroups to fill the CUs, and the widest column batch whose pieces fit)
int launch_split(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes, const qg_act_scale *scales,
                 float *out, hipStream_t s)
{
    int rtt = tuning().gemm_row_tiles;
    int ct = tuning().mfma_col_tiles;
    // derived: two row tiles of one column tile (two of each need more registers than 16 waves
    // have and spill to scratch; one row tile of two column tiles measured slower)
    if (ct == 0) ct = 1;
    if (rtt == 0) rtt = 2;
    const bool multi = G > 16;
    if (multi && rtt * ct > 4) {   // two slots of pieces: at most 64 KiB each
        if (rtt > 1) rtt = 4 / ct > 0 ? 4 / ct : 1;
        if (rtt * ct > 4) ct = 4 / rtt;
    }
    int st = QG_E_UNSUPPORTED;
    if (rtt == 1 && ct == 1) st = launch_split_typed<1, 1>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 1 && ct == 2) st = launch_split_typed<1, 2>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 1 && ct == 4) st = launch_split_typed<1, 4>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 2 && ct == 1) st = launch_split_typed<2, 1>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 2 && ct == 2) st = launch_split_typed<2, 2>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 2 && ct == 4) st = launch_split_typed<2, 4>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 4 && ct == 1) st = launch_split_typed<4, 1>(rows, G, ncol, image, codes, scales, out, s);
    else if (rtt == 4 && ct == 2) st = launch_split_typed<4, 2>(rows, G, ncol, image, codes, scales, out, s);
    if (st == QG_E_UNSUPPORTED) return fail(QG_E_UNSUPPORTED, "gemm: %d row tiles x %d column tiles do not fit", rtt, ct);
    return st;
}

}  // namespace

int launch_gemm_mfma(int64_t rows, int64_t cols, int64_t ncol, const void *image, const int8_t *codes,
                     const qg_act_scale *scales, float *out, hipStream_t s)
{
    const int G = (int)(cols / 256);
    int form = tuning().mfma_form;
    // derived (measured on the 4096- and 14336-row matrices): up to 16 columns of rows of up to
    // 16 blocks the staged form; more columns on fewer than 8192 rows the split form (enough
    // workgroups to fill the chip); more on larger matrices of rows of up to 16 blocks the
    // column-resident form (29.4 against 31.0 us at 64 columns on 14336 rows); otherwise the
    // shared-operand form
    if (form == 0) form = (G <= 16 && ncol <= 16) ? 1 : rows < 8192 ? 3 : G <= 16 ? 4 : 2;
    if (form == 1) {
        if (G > 16 || ncol > 16)
            return fail(QG_E_UNSUPPORTED, "gemm: the staged form takes at most 16 columns of at most 16 blocks");
        int rtt = tuning().gemm_row_tiles;
        if (rtt == 0) rtt = rows < 8192 ? 1 : ncol > 8 ? 4 : 2;
        int st = QG_E_UNSUPPORTED;
        if (rtt == 4) st = launch_staged_typed<4>(rows, G, ncol, image, codes, scales, out, s);
        else if (rtt == 2) st = launch_staged_typed<2>(rows, G, ncol, image, codes, scales, out, s);
        else st = launch_staged_typed<1>(rows, G, ncol, image, codes, scales, out, s);
        if (st == QG_E_UNSUPPORTED) return fail(QG_E_UNSUPPORTED, "gemm: the staged form's LDS does not fit");
        return st;
    }
    if (form == 3) return launch_split(rows, G, ncol, image, codes, scales, out, s);
    if (form == 4) return launch_resident(rows, G, ncol, image, codes, scales, out, s);
    // shared operands: 2 column tiles up to 32 columns, else 4, unless asked otherwise
    const int tiles = tuning().mfma_col_tiles;
    if (tiles == 1) return launch_cw<1>(rows, G, ncol, image, codes, scales, out, s);
    if (tiles == 2 || (tiles == 0 && ncol <= 32)) return launch_cw<2>(rows, G, ncol, image, codes, scales, out, s);
    return launch_cw<4>(rows, G, ncol, image, codes, scales, out, s);
}

}  // namespace qg
