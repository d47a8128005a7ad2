// gemv.hip -- decode GEMV and batched-column GEMM over packed Q4_K-/Q6_K-style images.
//
// One lane owns one (row, block) pair of a 64-pair image tile: its nine (Q4_K) or fourteen
// (Q6_K) 16-byte loads per tile are each a contiguous 1 KiB per wave.  The lane forms the
// pair's integer sub-block sums with v_dot4 on int8 activation codes staged in LDS
// ("Module lane", Functions block_sums), turns them into the block's piece with one
// binary32 rounding (Functions lane / group; "Module numerics", module description and
// Functions exact_sum, scaled_to_f32), and the row's pieces are then added in block order
// by the lane that owns the row (module description: pieces added in order).
//
// A wave walks "super-tiles": K consecutive tiles that hold RT whole rows (RT*G = 64*K), so
// the in-order fold of every row stays inside one wave.  Bits do not depend on the grid.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// LDS staging of NC activation rows: one record per (column, 256-element block) holding
// the block's 256 codes, its code sums (Q4K: eight per-32 sums; Q6K: sixteen per-16 sums)
// and its scale(s) (PerBlock: one; Sub32: eight).  The record stride is an odd multiple of
// 16 bytes, so the 16-byte reads of 16 lanes on 16 different blocks fall in different banks.
template <int FMT, int MODE>
struct ActRec {
    static constexpr int kSums = FMT == QG_Q4K ? 8 : 16;
    static constexpr int kScales = MODE == QG_PERBLOCK ? 1 : 8;
    static constexpr int kSumOff = 256;
    static constexpr int kScOff = 256 + 4 * kSums;
    static constexpr int kRaw = kScOff + 4 * kScales;
    static constexpr int kStride = ((kRaw + 15) / 16) % 2 ? ((kRaw + 15) / 16) * 16 : ((kRaw + 15) / 16 + 1) * 16;
};
static_assert(ActRec<QG_Q4K, QG_PERBLOCK>::kStride == 304, "record stride");
static_assert(ActRec<QG_Q6K, QG_SUB32>::kStride == 368, "record stride");

struct ActView {
    const unsigned char *base;  // record of (column 0, block 0)
    int stride;                 // bytes between blocks
    int col_stride;             // bytes between columns (G records)
};

// 12-bit (sc | mn << 6) field of sub-block i from the 96-bit meta string (y, z, w)
template <int I>
__device__ __forceinline__ uint32_t q4k_field(uint32_t y, uint32_t z, uint32_t w)
{
    if constexpr (I < 5) {
        const uint64_t lo = (uint64_t)y | ((uint64_t)z << 32);
        return (uint32_t)(lo >> (12 * I)) & 0xFFFu;
    } else {
        const uint64_t hi = (uint64_t)z | ((uint64_t)w << 32);
        return (uint32_t)(hi >> (12 * I - 32)) & 0xFFFu;
    }
}

// Integer dot of one 32-element Q4_K sub-block (16 code bytes, nibble-split) with 32
// activation codes: low nibbles meet elements 0..15, high nibbles elements 16..31.
__device__ __forceinline__ int q4k_sub_dot(uint4 w, const int8_t *a)
{
    const uint4 a0 = *reinterpret_cast<const uint4 *>(a);
    const uint4 a1 = *reinterpret_cast<const uint4 *>(a + 16);
    int P = 0;
    P = sdot4(w.x & 0x0F0F0F0Fu, a0.x, P);
    P = sdot4((w.x >> 4) & 0x0F0F0F0Fu, a1.x, P);
    P = sdot4(w.y & 0x0F0F0F0Fu, a0.y, P);
    P = sdot4((w.y >> 4) & 0x0F0F0F0Fu, a1.y, P);
    P = sdot4(w.z & 0x0F0F0F0Fu, a0.z, P);
    P = sdot4((w.z >> 4) & 0x0F0F0F0Fu, a1.z, P);
    P = sdot4(w.w & 0x0F0F0F0Fu, a0.w, P);
    P = sdot4((w.w >> 4) & 0x0F0F0F0Fu, a1.w, P);
    return P;
}

// Integer dots of two 16-element Q6_K sub-blocks (2i, 2i+1): 4-bit low parts from ql, 2-bit
// high parts from the qh bit pairs 4s..4s+1 (sub-block 2i) and 4s+2..4s+3 (sub-block 2i+1).
template <int S>
__device__ __forceinline__ void q6k_sub_dots(uint4 L, uint4 H, const int8_t *a, int &P0, int &P1)
{
    const uint4 a0 = *reinterpret_cast<const uint4 *>(a);
    const uint4 a1 = *reinterpret_cast<const uint4 *>(a + 16);
    const uint32_t l[4] = {L.x, L.y, L.z, L.w};
    const uint32_t h[4] = {H.x, H.y, H.z, H.w};
    const uint32_t x0[4] = {a0.x, a0.y, a0.z, a0.w};
    const uint32_t x1[4] = {a1.x, a1.y, a1.z, a1.w};
    int p0 = 0, p1 = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t c0 = (l[k] & 0x0F0F0F0Fu) | (((h[k] >> (4 * S)) & 0x03030303u) << 4);
        const uint32_t c1 = ((l[k] >> 4) & 0x0F0F0F0Fu) | (((h[k] >> (4 * S + 2)) & 0x03030303u) << 4);
        p0 = sdot4(c0, x0[k], p0);
        p1 = sdot4(c1, x1[k], p1);
    }
    P0 = p0;
    P1 = p1;
}

// ---------------------------------------------------------------------------------------
// One lane's share of a tile, held in registers between its loads and its use.

template <int FMT>
struct TileRegs;

template <>
struct TileRegs<QG_Q4K> {
    static constexpr int kBytes = kTileBytesQ4K;
    uint4 w[8];     // code chunks (sub-blocks 0..7)
    uint4 meta;     // d | dmin << 16, then the 96-bit sc/mn field string
    __device__ __forceinline__ void load(const uint8_t *tile, int lane)
    {
#pragma unroll
        for (int i = 0; i < 8; i++) w[i] = *reinterpret_cast<const uint4 *>(tile + 1024 * i + 16 * lane);
        meta = *reinterpret_cast<const uint4 *>(tile + 8192 + 16 * lane);
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < 8; i++) w[i] = make_uint4(0, 0, 0, 0);
        meta = make_uint4(0, 0, 0, 0);
    }
};

template <>
struct TileRegs<QG_Q6K> {
    static constexpr int kBytes = kTileBytesQ6K;
    uint4 L[8];     // low 4 bits of the codes
    uint4 H[4];     // high 2 bits
    uint4 sc;       // sixteen int8 sub-block scales
    uint32_t d;     // binary16 bits of the block scale
    __device__ __forceinline__ void load(const uint8_t *tile, int lane)
    {
#pragma unroll
        for (int i = 0; i < 8; i++) L[i] = *reinterpret_cast<const uint4 *>(tile + 1024 * i + 16 * lane);
#pragma unroll
        for (int h = 0; h < 4; h++) H[h] = *reinterpret_cast<const uint4 *>(tile + 8192 + 1024 * h + 16 * lane);
        sc = *reinterpret_cast<const uint4 *>(tile + 12288 + 16 * lane);
        d = *reinterpret_cast<const uint16_t *>(tile + 13312 + 2 * lane);
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < 8; i++) L[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 4; h++) H[h] = make_uint4(0, 0, 0, 0);
        sc = make_uint4(0, 0, 0, 0);
        d = 0;
    }
};

// ---------------------------------------------------------------------------------------
// Pieces of one pair for NC activation columns.

template <int MODE, int NC>
__device__ __forceinline__ void pair_pieces(const TileRegs<QG_Q4K> &T, int b, int C, const ActView &av, int nsc,
                                            float (&piece)[NC])
{
    uint32_t f[8];
    f[0] = q4k_field<0>(T.meta.y, T.meta.z, T.meta.w);
    f[1] = q4k_field<1>(T.meta.y, T.meta.z, T.meta.w);
    f[2] = q4k_field<2>(T.meta.y, T.meta.z, T.meta.w);
    f[3] = q4k_field<3>(T.meta.y, T.meta.z, T.meta.w);
    f[4] = q4k_field<4>(T.meta.y, T.meta.z, T.meta.w);
    f[5] = q4k_field<5>(T.meta.y, T.meta.z, T.meta.w);
    f[6] = q4k_field<6>(T.meta.y, T.meta.z, T.meta.w);
    f[7] = q4k_field<7>(T.meta.y, T.meta.z, T.meta.w);
    using R = ActRec<QG_Q4K, MODE>;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const unsigned char *rec = av.base + (size_t)c * av.col_stride + (size_t)b * av.stride;
        const int8_t *a = reinterpret_cast<const int8_t *>(rec);
        const int32_t *S32 = reinterpret_cast<const int32_t *>(rec + R::kSumOff);
        const qg_act_scale *sc = reinterpret_cast<const qg_act_scale *>(rec + R::kScOff);
        if constexpr (MODE == QG_PERBLOCK) {
            int Cb = 0, Ob = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int P = q4k_sub_dot(T.w[i], a + 32 * i);
                Cb += __mul24((int)(f[i] & 63u), P);
                Ob += __mul24((int)(f[i] >> 6), S32[i]);
            }
            const qg_act_scale s = sc[0];
            piece[c] = piece_q4k_perblock(Cb, Ob, T.meta.x, s.m, s.e);
        } else {
            const F16Scale d = f16_scale(T.meta.x & 0xFFFFu);
            const F16Scale dm = f16_scale(T.meta.x >> 16);
            long long v[16];
            int e[16];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int P = q4k_sub_dot(T.w[i], a + 32 * i);
                const int Cj = __mul24((int)(f[i] & 63u), P);
                const int Oj = __mul24((int)(f[i] >> 6), S32[i]);
                const qg_act_scale s = sc[i];
                v[2 * i] = (long long)(d.sig * (int)s.m) * Cj;
                e[2 * i] = s.e + d.ex;
                v[2 * i + 1] = -(long long)(dm.sig * (int)s.m) * Oj;
                e[2 * i + 1] = s.e + dm.ex;
            }
            piece[c] = exact_sum<16>(v, e);
        }
    }
}

template <int MODE, int NC>
__device__ __forceinline__ void pair_pieces(const TileRegs<QG_Q6K> &T, int b, int C, const ActView &av, int nsc,
                                            float (&piece)[NC])
{
    using R = ActRec<QG_Q6K, MODE>;
    const uint32_t sw[4] = {T.sc.x, T.sc.y, T.sc.z, T.sc.w};
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const unsigned char *rec = av.base + (size_t)c * av.col_stride + (size_t)b * av.stride;
        const int8_t *a = reinterpret_cast<const int8_t *>(rec);
        const int32_t *S16 = reinterpret_cast<const int32_t *>(rec + R::kSumOff);
        const qg_act_scale *sc = reinterpret_cast<const qg_act_scale *>(rec + R::kScOff);
        int Ck[16];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            int P0, P1;
            if (i & 1) q6k_sub_dots<1>(T.L[i], T.H[i >> 1], a + 32 * i, P0, P1);
            else q6k_sub_dots<0>(T.L[i], T.H[i >> 1], a + 32 * i, P0, P1);
            // (q - 32) . a = q . a - 32 * sum(a)
            const int s0 = (int)(int8_t)(sw[(2 * i) >> 2] >> (8 * ((2 * i) & 3)));
            const int s1 = (int)(int8_t)(sw[(2 * i + 1) >> 2] >> (8 * ((2 * i + 1) & 3)));
            Ck[2 * i] = __mul24(s0, P0 - 32 * S16[2 * i]);
            Ck[2 * i + 1] = __mul24(s1, P1 - 32 * S16[2 * i + 1]);
        }
        if constexpr (MODE == QG_PERBLOCK) {
            int Cb = 0;
#pragma unroll
            for (int k = 0; k < 16; k++) Cb += Ck[k];
            const qg_act_scale s = sc[0];
            piece[c] = piece_q6k_perblock(Cb, T.d, s.m, s.e);
        } else {
            const F16Scale d = f16_scale(T.d);
            long long v[8];
            int e[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const qg_act_scale s = sc[j];
                v[j] = (long long)(d.sig * (int)s.m) * (long long)(Ck[2 * j] + Ck[2 * j + 1]);
                e[j] = s.e + d.ex;
            }
            piece[c] = exact_sum<8>(v, e);
        }
    }
}

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------------------
// The kernel.  blockIdx.y selects a batch of NC activation columns (col0 = NC*blockIdx.y).
// The first tile's loads are issued before the activations are staged, and with PIPE each
// tile's successor is loaded while the tile itself is being computed.

template <int FMT, int MODE, int NC, bool PIPE>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t *__restrict__ image, int64_t n_tiles,
                                                        int rows, int G, int K, int RT, int n_super,
                                                        const int8_t *__restrict__ codes,
                                                        const qg_act_scale *__restrict__ scales,
                                                        const int32_t *__restrict__ csums, int ncol,
                                                        float *__restrict__ out)
{
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int kTileBytes = TileRegs<FMT>::kBytes;
    const int C = G * 256;
    const int nsc = MODE == QG_PERBLOCK ? G : G * 8;
    const int col0 = blockIdx.y * NC;
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int nwaves = gridDim.x * kWaves;
    const int st0 = blockIdx.x * kWaves + wid;

    // the wave's first tile: loads in flight before anything else
    TileRegs<FMT> cur;
    {
        const int64_t t0 = (int64_t)st0 * K;
        if (st0 < n_super && t0 < n_tiles) cur.load(image + t0 * kTileBytes, lane);
        else cur.zero();
    }

    // stage NC activation columns as per-block records (codes, code sums, scales)
    using R = ActRec<FMT, MODE>;
    unsigned char *s_rec = lds;
    float *s_piece = reinterpret_cast<float *>(lds + (size_t)NC * G * R::kStride);
    for (int c = 0; c < NC; c++) {
        const int col = col0 + c;
        const bool have = col < ncol;
        unsigned char *rc = s_rec + (size_t)c * G * R::kStride;
        const uint4 *src = reinterpret_cast<const uint4 *>(codes + (size_t)col * C);
        for (int i = threadIdx.x; i < C / 16; i += kThreads)
            *reinterpret_cast<uint4 *>(rc + (size_t)(i >> 4) * R::kStride + 16 * (i & 15)) =
                have ? src[i] : make_uint4(0, 0, 0, 0);
        const int32_t *cs = csums + (size_t)col * (C / 16);
        for (int i = threadIdx.x; i < G * R::kSums; i += kThreads) {
            int32_t v = 0;
            if (have) v = R::kSums == 8 ? cs[2 * i] + cs[2 * i + 1] : cs[i];
            *reinterpret_cast<int32_t *>(rc + (size_t)(i / R::kSums) * R::kStride + R::kSumOff + 4 * (i % R::kSums)) = v;
        }
        // qg_act_scale is 4 bytes: copy it as one word
        const uint32_t *scw = reinterpret_cast<const uint32_t *>(scales) + (size_t)col * nsc;
        for (int i = threadIdx.x; i < nsc; i += kThreads)
            *reinterpret_cast<uint32_t *>(rc + (size_t)(i / R::kScales) * R::kStride + R::kScOff + 4 * (i % R::kScales)) =
                have ? scw[i] : 0u;
    }
    __syncthreads();

    const ActView av{s_rec, R::kStride, G * R::kStride};
    float *wp = s_piece + (size_t)wid * 64 * NC;

    for (int st = st0; st < n_super; st += nwaves) {
        float y[NC];
#pragma unroll
        for (int c = 0; c < NC; c++) y[c] = 0.0f;
        for (int k = 0; k < K; k++) {
            const int64_t t = (int64_t)st * K + k;
            if (!PIPE && (k > 0 || st != st0)) {
                if (t < n_tiles) cur.load(image + t * kTileBytes, lane);
                else cur.zero();
            }
            TileRegs<FMT> nxt;
            if constexpr (PIPE) {
                // successor in this wave's walk: next tile of the super-tile, else the next super-tile's first
                const int64_t tn = k + 1 < K ? t + 1 : (int64_t)(st + nwaves) * K;
                const bool more = k + 1 < K || st + nwaves < n_super;
                if (more && tn < n_tiles) nxt.load(image + tn * kTileBytes, lane);
                else nxt.zero();
            }
            const int lp = k * 64 + lane;            // pair within the super-tile
            const int rl = lp / G;
            const int b = lp - rl * G;
            float piece[NC];
            pair_pieces<MODE, NC>(cur, b, C, av, nsc, piece);
#pragma unroll
            for (int c = 0; c < NC; c++) wp[c * 64 + lane] = piece[c];
            wave_sync();
            // lane i < RT owns local row i: pairs [i*G, (i+1)*G); this tile has [64k, 64k+64)
            if (lane < RT) {
                if (K == 1 && (G & 3) == 0) {
                    // whole row in this tile, four pieces per LDS read
                    for (int q = lane * G; q < lane * G + G; q += 4) {
#pragma unroll
                        for (int c = 0; c < NC; c++) {
                            const float4 p4 = *reinterpret_cast<const float4 *>(wp + c * 64 + q);
                            y[c] = fadd_ftz(y[c], p4.x);
                            y[c] = fadd_ftz(y[c], p4.y);
                            y[c] = fadd_ftz(y[c], p4.z);
                            y[c] = fadd_ftz(y[c], p4.w);
                        }
                    }
                } else {
                    int q0 = lane * G, q1 = q0 + G;
                    q0 = q0 > k * 64 ? q0 : k * 64;
                    q1 = q1 < k * 64 + 64 ? q1 : k * 64 + 64;
                    for (int q = q0; q < q1; q++) {
#pragma unroll
                        for (int c = 0; c < NC; c++) y[c] = fadd_ftz(y[c], wp[c * 64 + q - k * 64]);
                    }
                }
            }
            wave_sync();
            if constexpr (PIPE) cur = nxt;
        }
        const int64_t row = (int64_t)st * RT + lane;
        if (lane < RT && row < rows) {
#pragma unroll
            for (int c = 0; c < NC; c++)
                if (col0 + c < ncol) out[(int64_t)(col0 + c) * rows + row] = canon_nan(y[c]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Integer sums per (row, sub-block) for one activation row (debug view of the integer stage)

template <int FMT>
__global__ __launch_bounds__(kThreads) void block_sums_kernel(const uint8_t *__restrict__ image, int64_t npairs,
                                                              int G, const int8_t *__restrict__ codes,
                                                              int32_t *__restrict__ csum_out,
                                                              int32_t *__restrict__ osum_out)
{
    const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= npairs) return;
    const int64_t t = p / 64;
    const int lane = (int)(p - t * 64);
    const int b = (int)(p % G);
    const int8_t *a = codes + (size_t)b * 256;
    if constexpr (FMT == QG_Q4K) {
        const uint8_t *tile = image + t * kTileBytesQ4K;
        const uint4 meta = *reinterpret_cast<const uint4 *>(tile + 8192 + 16 * lane);
        uint32_t f[8];
        f[0] = q4k_field<0>(meta.y, meta.z, meta.w);
        f[1] = q4k_field<1>(meta.y, meta.z, meta.w);
        f[2] = q4k_field<2>(meta.y, meta.z, meta.w);
        f[3] = q4k_field<3>(meta.y, meta.z, meta.w);
        f[4] = q4k_field<4>(meta.y, meta.z, meta.w);
        f[5] = q4k_field<5>(meta.y, meta.z, meta.w);
        f[6] = q4k_field<6>(meta.y, meta.z, meta.w);
        f[7] = q4k_field<7>(meta.y, meta.z, meta.w);
        for (int i = 0; i < 8; i++) {
            const uint4 w = *reinterpret_cast<const uint4 *>(tile + 1024 * i + 16 * lane);
            int S = 0;
            for (int k = 0; k < 32; k++) S += a[32 * i + k];
            csum_out[p * 8 + i] = (int)(f[i] & 63u) * q4k_sub_dot(w, a + 32 * i);
            osum_out[p * 8 + i] = (int)(f[i] >> 6) * S;
        }
    } else {
        const uint8_t *tile = image + t * kTileBytesQ6K;
        const uint4 scv = *reinterpret_cast<const uint4 *>(tile + 12288 + 16 * lane);
        const uint32_t sw[4] = {scv.x, scv.y, scv.z, scv.w};
        for (int i = 0; i < 8; i++) {
            const uint4 L = *reinterpret_cast<const uint4 *>(tile + 1024 * i + 16 * lane);
            const uint4 H = *reinterpret_cast<const uint4 *>(tile + 8192 + 1024 * (i >> 1) + 16 * lane);
            int P0, P1;
            if (i & 1) q6k_sub_dots<1>(L, H, a + 32 * i, P0, P1);
            else q6k_sub_dots<0>(L, H, a + 32 * i, P0, P1);
            int S0 = 0, S1 = 0;
            for (int k = 0; k < 16; k++) { S0 += a[32 * i + k]; S1 += a[32 * i + 16 + k]; }
            const int s0 = (int)(int8_t)(sw[(2 * i) >> 2] >> (8 * ((2 * i) & 3)));
            const int s1 = (int)(int8_t)(sw[(2 * i + 1) >> 2] >> (8 * ((2 * i + 1) & 3)));
            csum_out[p * 16 + 2 * i] = s0 * (P0 - 32 * S0);
            csum_out[p * 16 + 2 * i + 1] = s1 * (P1 - 32 * S1);
        }
    }
}

int gcd_int(int a, int b)
{
    while (b) { const int t = a % b; a = b; b = t; }
    return a;
}

template <int FMT, int MODE, int NC, bool PIPE>
int launch_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                 const qg_act_scale *scales, const int32_t *csums, float *out, hipStream_t s)
{
    const int g = gcd_int(G, 64);
    const int RT = 64 / g;                    // rows per super-tile
    const int K = G / g;                      // tiles per super-tile
    const int64_t n_super64 = (rows + RT - 1) / RT;
    const int64_t n_tiles = (rows * G + 63) / 64;
    if (n_super64 > 0x7fffffff) return fail(QG_E_SHAPE, "too many rows: %lld", (long long)rows);
    const int n_super = (int)n_super64;
    const size_t lds = (size_t)NC * G * ActRec<FMT, MODE>::kStride + (size_t)kWaves * 64 * NC * 4;
    const Tuning &tn = tuning();
    int64_t wgs;
    if (tn.grid_wgs > 0) {
        wgs = tn.grid_wgs;
    } else {
        const int wpc = tn.waves_per_cu > 0 ? tn.waves_per_cu : 16;
        const int64_t max_waves = (int64_t)device_cu_count() * wpc;
        const int64_t waves = n_super64 < max_waves ? n_super64 : max_waves;
        wgs = (waves + kWaves - 1) / kWaves;
    }
    if (wgs < 1) wgs = 1;
    if (wgs > 0x7fffffff) wgs = 0x7fffffff;
    const int64_t ybatches = (ncol + NC - 1) / NC;
    dim3 grid((unsigned)wgs, (unsigned)ybatches);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemv_kernel<FMT, MODE, NC, PIPE>), grid, dim3(kThreads), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), n_tiles, (int)rows, G, K, RT, n_super,
                              codes, scales, csums, (int)ncol, out);
    else
        hipLaunchKernelGGL((gemv_kernel<FMT, MODE, NC, PIPE>), grid, dim3(kThreads), lds, s,
                           static_cast<const uint8_t *>(image), n_tiles, (int)rows, G, K, RT, n_super, codes,
                           scales, csums, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemv launch: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int FMT, int MODE>
int launch_nc(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
              const qg_act_scale *scales, const int32_t *csums, float *out, hipStream_t s)
{
    // widest column batch whose staging fits 64 KiB of LDS
    auto fits = [&](int nc) {
        return (size_t)nc * G * ActRec<FMT, MODE>::kStride + (size_t)kWaves * 64 * nc * 4 <= 65536;
    };
    if (ncol >= 8 && fits(8)) return launch_typed<FMT, MODE, 8, false>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (ncol >= 4 && fits(4)) return launch_typed<FMT, MODE, 4, false>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (ncol >= 2 && fits(2)) return launch_typed<FMT, MODE, 2, false>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (tuning().pipeline) return launch_typed<FMT, MODE, 1, true>(rows, G, ncol, image, codes, scales, csums, out, s);
    return launch_typed<FMT, MODE, 1, false>(rows, G, ncol, image, codes, scales, csums, out, s);
}

}  // namespace

int launch_gemv(int fmt, int mode, int64_t rows, int64_t cols, int64_t ncol, const void *image,
                const int8_t *codes, const qg_act_scale *scales, const int32_t *csums, float *out,
                hipStream_t s)
{
    if (rows == 0 || ncol == 0) return QG_OK;
    const int G = (int)(cols / 256);
    if (fmt == QG_Q4K && mode == QG_PERBLOCK)
        return launch_nc<QG_Q4K, QG_PERBLOCK>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (fmt == QG_Q4K && mode == QG_SUB32)
        return launch_nc<QG_Q4K, QG_SUB32>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (fmt == QG_Q6K && mode == QG_PERBLOCK)
        return launch_nc<QG_Q6K, QG_PERBLOCK>(rows, G, ncol, image, codes, scales, csums, out, s);
    return launch_nc<QG_Q6K, QG_SUB32>(rows, G, ncol, image, codes, scales, csums, out, s);
}

int launch_block_sums(int fmt, int64_t rows, int64_t cols, const void *image, const int8_t *codes,
                      int32_t *csum_out, int32_t *osum_out, hipStream_t s)
{
    const int G = (int)(cols / 256);
    const int64_t npairs = rows * G;
    if (npairs == 0) return QG_OK;
    const int64_t wgs = (npairs + kThreads - 1) / kThreads;
    if (fmt == QG_Q4K)
        hipLaunchKernelGGL(block_sums_kernel<QG_Q4K>, dim3((unsigned)wgs), dim3(kThreads), 0, s,
                           static_cast<const uint8_t *>(image), npairs, G, codes, csum_out, osum_out);
    else
        hipLaunchKernelGGL(block_sums_kernel<QG_Q6K>, dim3((unsigned)wgs), dim3(kThreads), 0, s,
                           static_cast<const uint8_t *>(image), npairs, G, codes, csum_out, osum_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "block_sums launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace qg
