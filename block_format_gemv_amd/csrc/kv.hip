// kv.hip -- attention over an int8 KV cache on the same exact machinery as the GEMV
// ("Module numerics" of logicaffeine_compile::spatial::decode_engine: Functions cache_row,
// int8_codes, quantize_head, int8_score, weighted_int8, attend_int8; Constants INV_127,
// VALUE_BLOCK).  The softmax between the scores and the weighted sum is the caller's.
//
//   cache rows      one wave per row: absmax, the binary16 of amax * (1/127) in binary32, the
//                   codes of x times the scale's binary32 reciprocal, nearest even, within 127.
//   query heads     the activation quantizer's per-lane code (quantize_lane): a whole head one
//                   PerBlock block (8-bit m), or 32-element Sub32 blocks (4-bit m).
//   scores          lane = cached position: the integer dots of its key row with the query's
//                   codes (the query in scalar registers), the query blocks' terms times the
//                   key scale summed exactly and rounded once.
//   weighted sum    one workgroup per head; per block of 32 positions the binary32 products
//                   p_j * d_j are coded under the least power of two 2^E with 127 * 2^E above
//                   their absmax, each value element's exact integer sum is rounded once
//                   (R32(2^E * T)), and the blocks are added in order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kValueBlock = 32;

__device__ __forceinline__ uint32_t wave_umax(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// binary16 bits -> binary32 (exact; inf and NaN kept)
__device__ __forceinline__ float half_bits_value(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// ---------------------------------------------------------------------------------------
// cache rows: grid = rows / 4 (4 waves), hd <= 256, lane l holds elements l, l + 64, ...

__global__ __launch_bounds__(256) void kv_cache_rows_kernel(int64_t n, int hd, const float *__restrict__ x,
                                                            uint16_t *__restrict__ scales, int8_t *__restrict__ codes)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n) return;
    const int lane = threadIdx.x & 63;
    const float *xr = x + r * hd;
    float v[4];
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int i = lane + 64 * k;
        v[k] = i < hd ? xr[i] : 0.0f;
        const uint32_t a = __float_as_uint(ftz(v[k])) & 0x7FFFFFFFu;   // a denormal reads as 0
        if (a <= 0x7F800000u && a > amax) amax = a;                      // NaN passed over
    }
    amax = wave_umax(amax);
    float prod = __uint_as_float(amax) * (1.0f / 127.0f);                // binary32
    // the product is rounded to binary32 first: kept opaque, the multiply and the conversion
    // cannot fuse into one mixed-precision FMA that rounds the exact product to binary16 once
    asm("" : "+v"(prod));
    const _Float16 h = (_Float16)prod;                                   // nearest even, subnormals kept
    const uint32_t hb = (uint32_t)__builtin_bit_cast(unsigned short, h);
    if (lane == 0) scales[r] = (uint16_t)hb;
    const float inv = 1.0f / (float)h;                                   // binary32 division
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int i = lane + 64 * k;
        if (i >= hd) break;
        int c = 0;
        if (!__builtin_isinf(inv)) {
            const float p = v[k] * inv;
            if (p == p) c = (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(p), -127.0f), 127.0f);
        }
        codes[r * hd + i] = (int8_t)c;
    }
}

// ---------------------------------------------------------------------------------------
// query heads: one wave per 256 elements, four per lane; GL lanes per activation block

template <int BITS, int GL>
__global__ __launch_bounds__(256) void kv_quantize_heads_kernel(int64_t total, const float *__restrict__ q,
                                                                int8_t *__restrict__ codes,
                                                                qg_act_scale *__restrict__ scales,
                                                                int32_t *__restrict__ err_flag)
{
    const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256;
    if (base >= total) return;
    const int lane = threadIdx.x & 63;
    const int64_t i0 = base + 4 * lane;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 < total) v = *reinterpret_cast<const float4 *>(q + i0);     // total is a multiple of 32
    const QuantLane ql = quantize_lane<BITS, GL>(v);
    if (i0 < total) {
        reinterpret_cast<uint32_t *>(codes + i0)[0] = ql.packed;
        if ((lane & (GL - 1)) == 0) {
            qg_act_scale s;
            s.e = (int16_t)ql.e;
            s.m = (uint8_t)ql.m;
            s.pad = 0;
            scales[i0 / (4 * GL)] = s;
            if (ql.inf && err_flag) *err_flag = 1;
        }
    }
}

// ---------------------------------------------------------------------------------------
// scores: grid = (position groups of 256, heads); lane = position

template <int MODE, int HD>
__global__ __launch_bounds__(256) void kv_scores_kernel(int nh, int grp, int64_t npos,
                                                        const int8_t *__restrict__ qcodes,
                                                        const uint32_t *__restrict__ qscales,
                                                        const uint16_t *__restrict__ kscales,
                                                        const int8_t *__restrict__ kcodes, float *__restrict__ out)
{
    constexpr int NB = MODE == QG_PERBLOCK ? 1 : HD / 32;     // query blocks
    constexpr int BW = HD / NB / 4;                           // code dwords per block
    const int h = blockIdx.y;
    const int kv = h / grp;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool have = j < npos;
    const int64_t jj = have ? j : npos - 1;
    // the query: uniform over the workgroup, read through scalar loads
    const uint32_t *qc = reinterpret_cast<const uint32_t *>(qcodes + (size_t)h * HD);
    const int8_t *krow = kcodes + ((size_t)kv * npos + jj) * HD;
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    uint32_t kw[HD / 4];
#pragma unroll
    for (int c = 0; c < HD / 16; c++) {
        const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(krow + 16 * c));
        kw[4 * c] = t.x;
        kw[4 * c + 1] = t.y;
        kw[4 * c + 2] = t.z;
        kw[4 * c + 3] = t.w;
    }
    const uint32_t ks = kscales[(size_t)kv * npos + jj];
    int P[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) {
        int acc = 0;
#pragma unroll
        for (int t = 0; t < BW; t++) acc = __builtin_amdgcn_sdot4((int)qc[b * BW + t], (int)kw[b * BW + t], acc, false);
        P[b] = acc;
    }
    float y;
    if (((ks >> 10) & 31u) == 31u) {
        y = __uint_as_float(0x7FC00000u);                     // a key scale that is not finite
    } else {
        const F16Scale d = f16_scale(ks);
        if constexpr (NB == 1) {
            const uint32_t w = qscales[h];
            const int m = (int)((w >> 16) & 0xFFu), e = (int)(int16_t)(w & 0xFFFFu);
            y = r32_exact_double(__builtin_ldexp((double)P[0] * (double)(d.sig * m), d.ex + e));
        } else {
            long long v[NB];
            int ex[NB];
#pragma unroll
            for (int b = 0; b < NB; b++) {
                const uint32_t w = qscales[(size_t)h * NB + b];
                const int m = (int)((w >> 16) & 0xFFu), e = (int)(int16_t)(w & 0xFFFFu);
                v[b] = (long long)(d.sig * m) * P[b];
                ex[b] = e + d.ex;
            }
            y = exact_sum<NB>(v, ex);
        }
    }
    if (have) out[(size_t)h * npos + j] = canon_nan(y);
}

// ---------------------------------------------------------------------------------------
// weighted sum: one workgroup of W waves per (head, group of EG value elements).  A wave
// covers BPW = 256 / EG blocks of 32 positions at a time, EG / 4 lanes per block, each lane
// four consecutive value elements; a round of W * BPW blocks (a 4096-position context at
// EG = 16 and W = 8: every block in one round, all its loads in flight together).  The
// round's pieces go to LDS ([block of the round][EG]) and after the round's barrier the
// first EG lanes add them in block order, one element per lane.

template <int HD, int EG, int W>
__global__ __launch_bounds__(64 * W) void kv_weighted_kernel(int grp, int64_t npos, const float *__restrict__ probs,
                                                             const uint16_t *__restrict__ vscales,
                                                             const int8_t *__restrict__ vcodes,
                                                             float *__restrict__ out)
{
    static_assert(EG % 4 == 0 && EG <= HD && HD % EG == 0 && EG <= 64, "element groups");
    constexpr int LPB = EG / 4;                // lanes per block
    constexpr int BPW = 64 / LPB;              // blocks per wave
    constexpr int RB = W * BPW;                // blocks per round
    __shared__ float s_piece[RB * EG];
    const int h = blockIdx.x;
    const int kv = h / grp;
    const int eg0 = (int)blockIdx.y * EG;      // this workgroup's first value element
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int sub = lane / LPB;                // this lane's block within the wave
    const int el = eg0 + 4 * (lane % LPB);     // its first value element
    const int64_t nblk = (npos + kValueBlock - 1) / kValueBlock;
    const float *ph = probs + (size_t)h * npos;
    const uint16_t *vs = vscales + (size_t)kv * npos;
    const int8_t *vc = vcodes + (size_t)kv * npos * HD;
    float y = 0.0f;                            // folding lanes: element threadIdx.x's running sum
    const int64_t rounds = (nblk + RB - 1) / RB;
    for (int64_t r = 0; r < rounds; r++) {
        const int kb = wid * BPW + sub;                    // block within the round
        const int64_t blk = r * RB + kb;
        float piece[4] = {0.f, 0.f, 0.f, 0.f};
        if (blk < nblk) {
            const int64_t j0 = blk * kValueBlock;
            const int nj = (int)(npos - j0 < kValueBlock ? npos - j0 : kValueBlock);
            // the block's codes, each of its LPB lanes coding PPL = 32 / LPB consecutive positions:
            // absmax and the flags reduced over the block's lanes, the packed codes (four
            // positions a dword) handed to every lane of the block
            constexpr int PPL = kValueBlock / LPB;
            const int q = lane % LPB;
            uint32_t amax = 0;
            int bad = 0;
            float w[PPL];
#pragma unroll
            for (int i = 0; i < PPL; i++) {
                const int j = q * PPL + i;
                w[i] = 0.0f;
                if (j < nj) {
                    const uint32_t sb = vs[j0 + j];
                    bad |= ((sb >> 10) & 31u) == 31u;
                    w[i] = ph[j0 + j] * half_bits_value(sb);            // binary32 product
                    const uint32_t a = __float_as_uint(ftz(w[i])) & 0x7FFFFFFFu;
                    if (a <= 0x7F800000u && a > amax) amax = a;
                }
            }
            static_assert(LPB == 4, "the block's lanes are one quad");
            amax = max(amax, (uint32_t)dpp<kDppQuadSwap1>((int)amax));
            amax = max(amax, (uint32_t)dpp<kDppQuadSwap2>((int)amax));
            bad |= dpp<kDppQuadSwap1>(bad);
            bad |= dpp<kDppQuadSwap2>(bad);
            const bool badb = bad != 0 || amax == 0x7F800000u;
            int E = 0, m1 = 1;
            if (!badb && amax != 0) least_scale<1>(__uint_as_float(amax), m1, E);
            uint32_t mine[PPL / 4];
#pragma unroll
            for (int k = 0; k < PPL / 4; k++) {
                uint32_t word = 0;
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const float f = ftz(w[4 * k + t]);
                    const int u = (badb || f != f) ? 0 : (int)__builtin_rint(__builtin_ldexp((double)f, -E));
                    word |= ((uint32_t)u & 255u) << (8 * t);
                }
                mine[k] = word;
            }
            // dword d (positions 4d .. 4d+3) is held by the block's lane d / (PPL / 4)
            uint32_t codes4[kValueBlock / 4];
#pragma unroll
            for (int d = 0; d < kValueBlock / 4; d++) {
                constexpr int K = PPL / 4;
                const int src = d / K;
                const int ctrl = src | (src << 2) | (src << 4) | (src << 6);   // quad_perm [src x4]
                const uint32_t v = mine[d % K];
                codes4[d] = (uint32_t)(ctrl == 0x00 ? dpp<0x00>((int)v)
                                     : ctrl == 0x55 ? dpp<0x55>((int)v)
                                     : ctrl == 0xAA ? dpp<0xAA>((int)v) : dpp<0xFF>((int)v));
            }
            // value element sums: rows j..j+3 of the lane's four elements, transposed to per
            // element dwords of four positions, against four codes at a time
            int T[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < kValueBlock; j += 4) {
                uint32_t r4[4];
#pragma unroll
                for (int t = 0; t < 4; t++)
                    r4[t] = j + t < nj ? *reinterpret_cast<const uint32_t *>(vc + (size_t)(j0 + j + t) * HD + el) : 0u;
                const uint32_t uu = codes4[j / 4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t col = ((r4[0] >> (8 * e)) & 255u) | (((r4[1] >> (8 * e)) & 255u) << 8) |
                                         (((r4[2] >> (8 * e)) & 255u) << 16) | (((r4[3] >> (8 * e)) & 255u) << 24);
                    T[e] = __builtin_amdgcn_sdot4((int)col, (int)uu, T[e], false);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; e++)
                piece[e] = badb ? __uint_as_float(0x7FC00000u)
                               : r32_exact_double(__builtin_ldexp((double)T[e], E));
        }
#pragma unroll
        for (int e = 0; e < 4; e++) s_piece[kb * EG + (el - eg0) + e] = piece[e];
        __syncthreads();
        if (threadIdx.x < EG) {
            const int64_t nb = nblk - r * RB < RB ? nblk - r * RB : RB;
            y = fold_ftz(y, s_piece + threadIdx.x, (int)nb, EG);
        }
        __syncthreads();
    }
    if (threadIdx.x < EG) out[(size_t)h * HD + eg0 + threadIdx.x] = canon_nan(y);
}

}  // namespace

int launch_kv_cache_rows(int64_t n, int64_t hd, const float *x, uint16_t *scales, int8_t *codes, hipStream_t s)
{
    if (n == 0) return QG_OK;
    const int64_t wgs = (n + 3) / 4;
    hipLaunchKernelGGL(kv_cache_rows_kernel, dim3((unsigned)wgs), dim3(256), 0, s, n, (int)hd, x, scales, codes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "kv cache rows launch: %s", hipGetErrorString(e));
    return QG_OK;
}

int launch_kv_quantize_heads(int mode, int64_t nh, int64_t hd, const float *q, int8_t *codes, qg_act_scale *scales,
                             int32_t *err_flag, hipStream_t s)
{
    const int64_t total = nh * hd;
    if (total == 0) return QG_OK;
    const int64_t wgs = (total + 1023) / 1024;
    const dim3 grid((unsigned)wgs), threads(256);
    if (mode == QG_SUB32)
        hipLaunchKernelGGL((kv_quantize_heads_kernel<4, 8>), grid, threads, 0, s, total, q, codes, scales, err_flag);
    else if (hd == 32)
        hipLaunchKernelGGL((kv_quantize_heads_kernel<8, 8>), grid, threads, 0, s, total, q, codes, scales, err_flag);
    else if (hd == 64)
        hipLaunchKernelGGL((kv_quantize_heads_kernel<8, 16>), grid, threads, 0, s, total, q, codes, scales, err_flag);
    else if (hd == 128)
        hipLaunchKernelGGL((kv_quantize_heads_kernel<8, 32>), grid, threads, 0, s, total, q, codes, scales, err_flag);
    else
        hipLaunchKernelGGL((kv_quantize_heads_kernel<8, 64>), grid, threads, 0, s, total, q, codes, scales, err_flag);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "kv quantize heads launch: %s", hipGetErrorString(e));
    return QG_OK;
}

namespace {
template <int MODE, int HD>
void scores_typed(int nh, int grp, int64_t npos, const int8_t *qc, const qg_act_scale *qs, const uint16_t *ks,
                  const int8_t *kc, float *out, hipStream_t s)
{
    const dim3 grid((unsigned)((npos + 255) / 256), (unsigned)nh);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    const uint32_t *qw = reinterpret_cast<const uint32_t *>(qs);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((kv_scores_kernel<MODE, HD>), grid, dim3(256), 0, s, ev0, ev1, 0, nh, grp, npos, qc, qw,
                              ks, kc, out);
    else
        hipLaunchKernelGGL((kv_scores_kernel<MODE, HD>), grid, dim3(256), 0, s, nh, grp, npos, qc, qw, ks, kc, out);
}

template <int HD>
void weighted_typed(int nh, int grp, int64_t npos, const float *p, const uint16_t *vs, const int8_t *vc, float *out,
                    hipStream_t s)
{
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    constexpr int EG = 16, W = 8;
    const dim3 grid((unsigned)nh, (unsigned)(HD / EG));
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((kv_weighted_kernel<HD, EG, W>), grid, dim3(64 * W), 0, s, ev0, ev1, 0, grp, npos, p,
                              vs, vc, out);
    else
        hipLaunchKernelGGL((kv_weighted_kernel<HD, EG, W>), grid, dim3(64 * W), 0, s, grp, npos, p, vs, vc, out);
}
}  // namespace

int launch_kv_scores(int mode, int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const int8_t *qcodes,
                     const qg_act_scale *qscales, const uint16_t *kscales, const int8_t *kcodes, float *out,
                     hipStream_t s)
{
    if (nh == 0 || npos == 0) return QG_OK;
    const int grp = (int)(nh / nkv);
    const int h = (int)nh;
    if (mode == QG_PERBLOCK) {
        if (hd == 32) scores_typed<QG_PERBLOCK, 32>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
        else if (hd == 64) scores_typed<QG_PERBLOCK, 64>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
        else if (hd == 128) scores_typed<QG_PERBLOCK, 128>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
        else scores_typed<QG_PERBLOCK, 256>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
    } else {
        if (hd == 32) scores_typed<QG_SUB32, 32>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
        else if (hd == 64) scores_typed<QG_SUB32, 64>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
        else if (hd == 128) scores_typed<QG_SUB32, 128>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
        else scores_typed<QG_SUB32, 256>(h, grp, npos, qcodes, qscales, kscales, kcodes, out, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "kv scores launch: %s", hipGetErrorString(e));
    return QG_OK;
}

int launch_kv_weighted(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs, const uint16_t *vscales,
                       const int8_t *vcodes, float *out, hipStream_t s)
{
    if (nh == 0) return QG_OK;
    const int grp = (int)(nh / nkv);
    if (hd == 32) weighted_typed<32>((int)nh, grp, npos, probs, vscales, vcodes, out, s);
    else if (hd == 64) weighted_typed<64>((int)nh, grp, npos, probs, vscales, vcodes, out, s);
    else if (hd == 128) weighted_typed<128>((int)nh, grp, npos, probs, vscales, vcodes, out, s);
    else weighted_typed<256>((int)nh, grp, npos, probs, vscales, vcodes, out, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "kv weighted launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace qg
