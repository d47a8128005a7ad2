// gemm_mfma.hip -- batched-column GEMM of a Q4_K-style image under PerBlock scaling on the
// int8 matrix cores (v_mfma_i32_16x16x64_i8), for 16 or more activation columns.
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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// each byte of q (at most 15) times k (at most 7): the products stay below 128, so the two
// 16-bit halves multiply without carries between bytes
__device__ __forceinline__ int bytes_times(uint32_t q, uint32_t k)
{
    const us2 a = __builtin_bit_cast(us2, q);
    const us2 b = {(unsigned short)k, (unsigned short)k};
    return __builtin_bit_cast(int, a * b);
}

template <int I>
__device__ __forceinline__ uint32_t field(uint32_t y, uint32_t z, uint32_t w)
{
    if constexpr (I < 5) return (uint32_t)(((uint64_t)y | ((uint64_t)z << 32)) >> (12 * I)) & 0xFFFu;
    else return (uint32_t)(((uint64_t)z | ((uint64_t)w << 32)) >> (12 * I - 32)) & 0xFFFu;
}

// grid: x = 64-row group, y = batch of 16*CT activation columns; 4 waves, wave w = rows 16w..16w+15
template <int CT>
__global__ __launch_bounds__(256) void gemm_mfma_q4k(const uint8_t *__restrict__ image, int rows, int G,
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
        f[0] = field<0>(meta.y, meta.z, meta.w);
        f[1] = field<1>(meta.y, meta.z, meta.w);
        f[2] = field<2>(meta.y, meta.z, meta.w);
        f[3] = field<3>(meta.y, meta.z, meta.w);
        f[4] = field<4>(meta.y, meta.z, meta.w);
        f[5] = field<5>(meta.y, meta.z, meta.w);
        f[6] = field<6>(meta.y, meta.z, meta.w);
        f[7] = field<7>(meta.y, meta.z, meta.w);

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
int launch_ct(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes, const qg_act_scale *scales,
              float *out, hipStream_t s)
{
    const int64_t groups = (rows + 63) / 64;
    const dim3 grid((unsigned)groups, (unsigned)((ncol + 16 * CT - 1) / (16 * CT)));
    const size_t lds = (size_t)G * 16 * CT * (8 + 4);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL(gemm_mfma_q4k<CT>, grid, dim3(256), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, scales, (int)ncol, out);
    else
        hipLaunchKernelGGL(gemm_mfma_q4k<CT>, grid, dim3(256), lds, s, static_cast<const uint8_t *>(image), (int)rows,
                           G, codes, scales, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemm (matrix cores) launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace

int launch_gemm_mfma(int64_t rows, int64_t cols, int64_t ncol, const void *image, const int8_t *codes,
                     const qg_act_scale *scales, float *out, hipStream_t s)
{
    const int G = (int)(cols / 256);
    int ct = tuning().mfma_col_tiles;
    if (ct <= 0) ct = ncol >= 64 ? 2 : 1;
    if (ct >= 4) return launch_ct<4>(rows, G, ncol, image, codes, scales, out, s);
    if (ct >= 2) return launch_ct<2>(rows, G, ncol, image, codes, scales, out, s);
    return launch_ct<1>(rows, G, ncol, image, codes, scales, out, s);
}

}  // namespace qg
