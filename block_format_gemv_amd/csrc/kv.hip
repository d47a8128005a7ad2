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

#include <mutex>

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

// Lane quad k's share of one block of a query head (eight positions a lane): the weights p_j
// and the value scales' bits.  Every load is issued, from position min(j, nj - 1) (nj >= 1), so
// that none waits on a branch; the coding ignores positions past nj.
__device__ __forceinline__ void load_weights(const float *ph, const uint16_t *vs, int64_t j0, int nj, int qq,
                                             float (&p)[8], uint32_t (&sb)[8])
{
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int j = min(qq * 8 + i, nj - 1);
        p[i] = ph[j0 + j];
        sb[i] = vs[j0 + j];
    }
}

// A lane quad's coding of one block: w_j = p_j * d_j in binary32, absmax and the flags reduced
// over the quad (quad_perm DPP), E from the absmax, and the codes rne(w_j / 2^E) of the lane's
// eight positions, four to a word.  No branches around it, so that the loads feeding it stay
// where they are issued.  The quotient is formed in binary32: when it is 0.5 or more in
// magnitude it is a normal number and exact, and below that the hardware's result, however
// rounded or flushed, is below 0.5 too, so the code is 0 as for the exact quotient.
__device__ __forceinline__ void code_quad(const float (&p)[8], const uint32_t (&sb)[8], int nj, int qq,
                                          uint32_t (&word)[2], int &E, bool &badb)
{
    uint32_t amax = 0;
    int bad = 0;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const bool in = qq * 8 + i < nj;
        bad |= (in && ((sb[i] >> 10) & 31u) == 31u) ? 1 : 0;
        w[i] = in ? p[i] * half_bits_value(sb[i]) : 0.0f;              // binary32 product
        const uint32_t a = __float_as_uint(ftz(w[i])) & 0x7FFFFFFFu;
        amax = (a <= 0x7F800000u && a > amax) ? a : amax;                // NaN passed over
    }
    amax = max(amax, (uint32_t)dpp<kDppQuadSwap1>((int)amax));
    amax = max(amax, (uint32_t)dpp<kDppQuadSwap2>((int)amax));
    bad |= dpp<kDppQuadSwap1>(bad);
    bad |= dpp<kDppQuadSwap2>(bad);
    badb = bad != 0 || amax == 0x7F800000u;
    E = 0;
    int m1 = 1;
    if (!badb && amax != 0) least_scale<1>(__uint_as_float(amax), m1, E);
#pragma unroll
    for (int kw = 0; kw < 2; kw++) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const float f = ftz(w[4 * kw + t]);
            const int u = (badb || f != f) ? 0 : (int)__builtin_rintf(__builtin_ldexpf(f, -E));
            v |= ((uint32_t)u & 255u) << (8 * t);
        }
        word[kw] = v;
    }
}

// The block's 32 value rows, four bytes of each (elements el .. el+3), rows past nj read from
// row nj - 1 and then zeroed: every load unconditional.
__device__ __forceinline__ void load_rows(const int8_t *vc, int hd, int64_t j0, int nj, int el,
                                          uint32_t (&rows)[kValueBlock])
{
#pragma unroll
    for (int t = 0; t < kValueBlock; t++)
        rows[t] = *reinterpret_cast<const uint32_t *>(vc + (size_t)(j0 + min(t, nj - 1)) * hd + el);
#pragma unroll
    for (int t = 0; t < kValueBlock; t++) rows[t] = t < nj ? rows[t] : 0u;
}

// The rows transposed by byte permutes (v_perm: selector bytes 0..3 take the second operand's
// bytes, 4..7 the first's): col[e][g] holds element e of positions 4g .. 4g+3, one byte each.
__device__ __forceinline__ void transpose_rows(const uint32_t (&rows)[kValueBlock], uint32_t (&col)[4][kValueBlock / 4])
{
#pragma unroll
    for (int g = 0; g < kValueBlock / 4; g++) {
        const uint32_t *r4 = rows + 4 * g;
        // interleave rows pairwise: (a0 b0 a1 b1) and (a2 b2 a3 b3), then pair the pairs
        const uint32_t p01l = __builtin_amdgcn_perm(r4[1], r4[0], 0x05010400u);
        const uint32_t p01h = __builtin_amdgcn_perm(r4[1], r4[0], 0x07030602u);
        const uint32_t p23l = __builtin_amdgcn_perm(r4[3], r4[2], 0x05010400u);
        const uint32_t p23h = __builtin_amdgcn_perm(r4[3], r4[2], 0x07030602u);
        col[0][g] = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
        col[1][g] = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
        col[2][g] = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
        col[3][g] = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
    }
}

// A piece R32(T * 2^E) (flushed) for |T| < 2^24 and E >= -132, the least exponent a normal
// absmax's scale has: (float)T is exact, and T * 2^E, a multiple of 2^-132 with at most 24
// significant bits, lies on the binary32 grid (normal or subnormal) wherever it is below
// 2^128, so ldexp is exact there and the flush is R32's; beyond, both are infinite.
__device__ __forceinline__ float value_piece(int T, int E) { return ftz(__builtin_ldexpf((float)T, E)); }

// The four elements' exact sums over the block, their dot chains interleaved, and the pieces
// (NaN for a bad block), selected without a branch.
__device__ __forceinline__ void block_pieces(const uint32_t (&col)[4][kValueBlock / 4], const uint32_t (&cw)[8], int E,
                                             bool bad, float (&pc)[4])
{
    int T[4] = {0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < kValueBlock / 4; g++)
#pragma unroll
        for (int e = 0; e < 4; e++) T[e] = __builtin_amdgcn_sdot4((int)col[e][g], (int)cw[g], T[e], false);
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const float v = value_piece(T[e], E);
        pc[e] = bad ? __uint_as_float(0x7FC00000u) : v;
    }
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
    // workgroups go to the eight XCDs in turn (linear id mod 8); with the head count a multiple
    // of 8 (then the linear id mod 8 is blockIdx.x mod 8), XCD x takes the consecutive heads
    // x * nh / 8 .. (x + 1) * nh / 8 - 1, so heads that share a KV head share that XCD's L2
    // and its value rows come from HBM once
    const int nh = (int)gridDim.x, bx = (int)blockIdx.x;
    const int h = (nh & 7) == 0 ? (bx & 7) * (nh >> 3) + (bx >> 3) : bx;
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
    static_assert(LPB == 4, "the block's lanes are one quad");
    const int q = lane % LPB;
    for (int64_t r = 0; r < rounds; r++) {
        const int kb = wid * BPW + sub;                    // block within the round
        const int64_t blk = r * RB + kb;
        // a lane past the last block reads the last block again and its pieces go unread
        const int64_t j0 = (blk < nblk ? blk : nblk - 1) * kValueBlock;
        const int nj = (int)(npos - j0 < kValueBlock ? npos - j0 : kValueBlock);
        // the quad's weights, then the block's rows, all in flight together; lane q of the
        // quad codes positions 8q .. 8q+7
        float p[8];
        uint32_t sb[8];
        load_weights(ph, vs, j0, nj, q, p, sb);
        uint32_t rows[kValueBlock];
        load_rows(vc, HD, j0, nj, el, rows);
        uint32_t mine[2];
        int E;
        bool badb;
        code_quad(p, sb, nj, q, mine, E, badb);
        // code word d (positions 4d .. 4d+3) is word d % 2 of the quad's lane d / 2
        uint32_t codes4[kValueBlock / 4];
#pragma unroll
        for (int d = 0; d < kValueBlock / 4; d++) {
            const uint32_t v = mine[d % 2];
            const int src = d / 2;
            codes4[d] = (uint32_t)(src == 0 ? dpp<0x00>((int)v)
                                 : src == 1 ? dpp<0x55>((int)v)
                                 : src == 2 ? dpp<0xAA>((int)v) : dpp<0xFF>((int)v));   // quad_perm [src x4]
        }
        uint32_t col[4][kValueBlock / 4];
        transpose_rows(rows, col);
        float piece[4];
        block_pieces(col, codes4, E, badb, piece);
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

// ---------------------------------------------------------------------------------------
// weighted sum in two passes over a caller's workspace of pieces, f32 [nh][nblk][HD]:
//
//   pieces  grid = (ceil(nblk / 4), nkv), four waves; wave w takes block 4x + w of KV head y for
//           every query head that shares it, so each cached value row is read once.  The
//           weights and scales of the first 16 heads are loaded first, then the block's rows
//           (every load unconditional, from clamped positions, all in flight together)
//           (lane: four consecutive elements, EL = HD / 4 lanes a row, HS = 64 / EL head
//           slots); lane quad k codes head k while the rows arrive and parks its eight code
//           words, E and the bad flag in the wave's LDS record k; the rows are transposed to
//           per-element words of four positions, and head slot s forms heads s, s + HS, ...
//           from the records: per element 8 v_dot4 (the four elements' chains interleaved) and
//           one rounding, four pieces a lane, stored as one 16-byte write.  No barrier: a wave's LDS operations run in order.
//   fold    kv_fold.hip: one lane per (head, element) adds the pieces in block order.

constexpr int kRec = 12;   // LDS words per head record: eight code words, E, the bad flag, padding

// Lane quad k's coding of its query head over the block, parked in the head's record r
// (eight code words, E, the bad flag) when `keep`.
__device__ __forceinline__ void park_record(const float (&p)[8], const uint32_t (&sb)[8], int nj, int qq, bool keep,
                                            uint32_t *r)
{
    uint32_t word[2];
    int E;
    bool badb;
    code_quad(p, sb, nj, qq, word, E, badb);
    if (keep) {
        r[2 * qq] = word[0];                    // code words 2qq, 2qq+1: positions 8qq .. 8qq+7
        r[2 * qq + 1] = word[1];
        if (qq == 0) {
            r[8] = (uint32_t)E;
            r[9] = badb ? 1u : 0u;
        }
    }
}

// Head slot `slot` forms N of its heads slot + (it0 + it) * HS of a batch of nh_batch heads:
// every record read issued before the dots; a head past the batch reads the batch's last
// record and stores nothing.  Head k2's pieces go to dst + k2 * head_stride.
template <int HS, int N>
__device__ __forceinline__ void form_heads(const uint32_t *rec, const uint32_t (&col)[4][kValueBlock / 4], int slot,
                                           int nh_batch, int it0, float *dst, size_t head_stride)
{
    uint4 c0[N], c1[N], eb[N];
#pragma unroll
    for (int it = 0; it < N; it++) {
        const uint32_t *r = rec + min(slot + (it0 + it) * HS, nh_batch - 1) * kRec;
        c0[it] = *reinterpret_cast<const uint4 *>(r);
        c1[it] = *reinterpret_cast<const uint4 *>(r + 4);
        eb[it] = *reinterpret_cast<const uint4 *>(r + 8);
    }
#pragma unroll
    for (int it = 0; it < N; it++) {
        const int k2 = slot + (it0 + it) * HS;
        const uint32_t cw[8] = {c0[it].x, c0[it].y, c0[it].z, c0[it].w, c1[it].x, c1[it].y, c1[it].z, c1[it].w};
        float pc[4];
        block_pieces(col, cw, (int)eb[it].x, eb[it].y != 0, pc);
        if (k2 < nh_batch) *reinterpret_cast<float4 *>(dst + k2 * head_stride) = make_float4(pc[0], pc[1], pc[2], pc[3]);
    }
}

template <int HS>
__device__ __forceinline__ void form_batch(const uint32_t *rec, const uint32_t (&col)[4][kValueBlock / 4], int slot,
                                           int nh_batch, float *dst, size_t head_stride)
{
    const int iters = (nh_batch + HS - 1) / HS;
    if (iters == 1) form_heads<HS, 1>(rec, col, slot, nh_batch, 0, dst, head_stride);
    else if (iters == 2) form_heads<HS, 2>(rec, col, slot, nh_batch, 0, dst, head_stride);
    else
        for (int it0 = 0; it0 < iters; it0 += 4) form_heads<HS, 4>(rec, col, slot, nh_batch, it0, dst, head_stride);
}

template <int HD>
__global__ __launch_bounds__(256) void kv_weighted_pieces_kernel(int nkv, int grp, int64_t npos, int64_t nblk,
                                                                 const float *__restrict__ probs,
                                                                 const uint16_t *__restrict__ vscales,
                                                                 const int8_t *__restrict__ vcodes,
                                                                 float *__restrict__ pieces)
{
    constexpr int EL = HD / 4;                 // lanes per value row
    constexpr int HS = 64 / EL;                // head slots per wave
    __shared__ __align__(16) uint32_t s_rec[4][16 * kRec];
    // workgroup i takes KV head i % nkv and blocks 4(i / nkv) ..: workgroups are dealt to the 8
    // XCDs in turn, so with nkv a multiple of 8 every piece of a KV head is written from one XCD
    const int kv = (int)(blockIdx.x % (unsigned)nkv);
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int64_t blk = (int64_t)(blockIdx.x / (unsigned)nkv) * 4 + wid;
    if (blk >= nblk) return;                   // nothing waits for this wave
    const int64_t j0 = blk * kValueBlock;
    const int nj = (int)(npos - j0 < kValueBlock ? npos - j0 : kValueBlock);
    const uint16_t *vs = vscales + (size_t)kv * npos;
    const int8_t *vc = vcodes + (size_t)kv * npos * HD;
    const float *pk = probs + (size_t)kv * grp * npos;   // the first query head of this KV head
    uint32_t *rec = s_rec[wid];
    const int q = lane % EL, slot = lane / EL;
    const int k = lane >> 2, qq = lane & 3;
    const size_t head_stride = (size_t)nblk * HD;
    float *dst = pieces + ((size_t)kv * grp * nblk + blk) * HD + 4 * q;   // head 0 of the batch

    // the first batch's weights, then the block's rows, all in flight together; lane quad k
    // codes query head k of the batch into record k
    int nheads = grp < 16 ? grp : 16;
    float p[8];
    uint32_t sb[8];
    load_weights(pk + (size_t)min(k, nheads - 1) * npos, vs, j0, nj, qq, p, sb);
    uint32_t rows[kValueBlock];
    load_rows(vc, HD, j0, nj, 4 * q, rows);
    park_record(p, sb, nj, qq, k < nheads, rec + min(k, 15) * kRec);
    uint32_t col[4][kValueBlock / 4];
    transpose_rows(rows, col);
    form_batch<HS>(rec, col, slot, nheads, dst, head_stride);
    // more than 16 query heads per KV head: the next batches, the records reused (the reads
    // above come first in the wave's LDS order)
    for (int hbase = 16; hbase < grp; hbase += 16) {
        nheads = grp - hbase < 16 ? grp - hbase : 16;
        load_weights(pk + (size_t)(hbase + min(k, nheads - 1)) * npos, vs, j0, nj, qq, p, sb);
        park_record(p, sb, nj, qq, k < nheads, rec + min(k, 15) * kRec);
        form_batch<HS>(rec, col, slot, nheads, dst + hbase * head_stride, head_stride);
    }
}

template <int HD>
void weighted_pieces_typed(int nkv, int grp, int64_t npos, int64_t nblk, const float *p, const uint16_t *vs,
                           const int8_t *vc, float *ws, hipStream_t s)
{
    hipLaunchKernelGGL((kv_weighted_pieces_kernel<HD>), dim3((unsigned)((nblk + 3) / 4 * nkv)), dim3(256), 0,
                       s, nkv, grp, npos, nblk, p, vs, vc, ws);
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

// The fixed workspace of qg_kv_weighted_noalloc: one copy on every device the library runs
// on, held until the process ends.  Host code reaches it only through the device address
// hipGetSymbolAddress gives for the current device (the array's name is not that address).
static __device__ __align__(256) float scratch[QG_KV_NOALLOC_BYTES / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
void *g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
std::once_flag g_scratch_once[kScratchDevices];
}  // namespace

int launch_kv_weighted_noalloc(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                               const uint16_t *vscales, const int8_t *vcodes, float *out, hipStream_t s)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "kv weighted (no allocation): hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchDevices)
        return fail(QG_E_RUNTIME, "kv weighted (no allocation): device %d beyond the %d supported", dev, kScratchDevices);
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (g_scratch_err[dev] == hipSuccess) g_scratch_ptr[dev] = ptr;
    });
    if (g_scratch_ptr[dev] == nullptr)
        return fail(QG_E_RUNTIME, "kv weighted (no allocation): the workspace's address on device %d: %s", dev,
                    hipGetErrorString(g_scratch_err[dev]));
    return launch_kv_weighted_two_pass(nh, nkv, npos, hd, probs, vscales, vcodes,
                                       static_cast<float *>(g_scratch_ptr[dev]), out, s);
}

size_t kv_weighted_workspace_bytes(int64_t nh, int64_t npos, int64_t hd)
{
    return (size_t)nh * (size_t)((npos + kValueBlock - 1) / kValueBlock) * (size_t)hd * sizeof(float);
}

int launch_kv_weighted_two_pass(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs,
                                const uint16_t *vscales, const int8_t *vcodes, float *ws, float *out, hipStream_t s)
{
    if (nh == 0) return QG_OK;
    const int grp = (int)(nh / nkv), g = (int)nkv;
    const int64_t nblk = (npos + kValueBlock - 1) / kValueBlock;
    if ((nblk + 3) / 4 * nkv > 0x7fffffff)
        return fail(QG_E_SHAPE, "kv weighted: %lld positions x %lld KV heads is too many", (long long)npos,
                    (long long)nkv);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);   // the span of both passes
    if (ev0 && ev1 && hipEventRecord(ev0, s) != hipSuccess)
        return fail(QG_E_RUNTIME, "kv weighted: recording the start event failed");
    if (nblk > 0) {
        if (hd == 32) weighted_pieces_typed<32>(g, grp, npos, nblk, probs, vscales, vcodes, ws, s);
        else if (hd == 64) weighted_pieces_typed<64>(g, grp, npos, nblk, probs, vscales, vcodes, ws, s);
        else if (hd == 128) weighted_pieces_typed<128>(g, grp, npos, nblk, probs, vscales, vcodes, ws, s);
        else weighted_pieces_typed<256>(g, grp, npos, nblk, probs, vscales, vcodes, ws, s);
    }
    launch_kv_fold_pieces(nh * hd, (int)hd, nblk, nkv, ws, out, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "kv weighted (two passes) launch: %s", hipGetErrorString(e));
    if (ev0 && ev1 && hipEventRecord(ev1, s) != hipSuccess)
        return fail(QG_E_RUNTIME, "kv weighted: recording the stop event failed");
    return QG_OK;
}

}  // namespace qg
