// gemv.hip -- decode GEMV and batched-column GEMM over packed Q4_K-/Q6_K-style images.
//
// A tile is 64 consecutive rows x one 256-element block; lane l of a wave owns row 64g + l
// of its tile.  Its nine (Q4_K) or fourteen (Q6_K) 16-byte loads are each a contiguous
// 1 KiB per wave.  Every lane of a wave works on the same block, so the block's activation
// codes, code sums and scale are wave-uniform.  With one activation column each wave
// brings its blocks' activations into its own registers (quantizing the f32 row itself,
// or loading the codes) and reads them out into scalar registers, the SGPR operands of the
// dot products; several columns share per-block records staged in LDS.
//
// Per pair the lane forms the integer sub-block sums ("Module lane", Functions block_sums),
// turns them into the block's piece with one binary32 rounding (Functions lane / group;
// "Module numerics", module description and Functions exact_sum, scaled_to_f32) and parks
// the piece in LDS.  A workgroup owns one 64-row group; after a barrier its first wave adds
// each row's pieces in ascending block order (module description: pieces added in order),
// one row per lane.  Bits do not depend on the launch configuration.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// a * b + c with a and b taken as signed 24-bit integers (exact when |a|, |b| < 2^23 and the
// result fits 32 bits): the target's 24-bit multiply, which reads the low 24 bits of each
// operand as they are (__mul24 would first mask b to 24 bits with two shifts).  A compiler
// intrinsic rather than inline assembly, so the instruction takes part in hazard checking.
extern "C" __device__ int qg_llvm_mul_i24(int, int) __asm("llvm.amdgcn.mul.i24");
__device__ __forceinline__ int mul_i24(int a, int b) { return qg_llvm_mul_i24(a, b); }
__device__ __forceinline__ int mad_i24(int a, int b, int c) { return qg_llvm_mul_i24(a, b) + c; }

// ---------------------------------------------------------------------------------------
// Activation sources.  Each hands out wave-uniform values: codes16(b, i) = codes 16i..16i+15
// of block b, sum32 / sum16 = code sums of a 32- / 16-element run, scale(b, j, per_block).

// NC columns staged in LDS, one record per (column, 256-element block) holding the block's
// 256 codes, its code sums (Q4K: eight per-32 sums; Q6K: sixteen per-16 sums) and its
// scale(s) (PerBlock: one; Sub32: eight).
template <int FMT, int MODE>
struct ActRec {
    static constexpr int kSums = FMT == QG_Q4K ? 8 : 16;
    static constexpr int kScales = MODE == QG_PERBLOCK ? 1 : 8;
    static constexpr int kSumOff = 256;
    static constexpr int kScOff = 256 + 4 * kSums;
    static constexpr int kStride = (kScOff + 4 * kScales + 15) / 16 * 16;
};

template <int FMT, int MODE>
struct ActLds {
    using R = ActRec<FMT, MODE>;
    const unsigned char *col;   // record of (this column, block 0)
    __device__ __forceinline__ const unsigned char *rec(int b) const { return col + (size_t)b * R::kStride; }
    __device__ __forceinline__ uint4 codes16(int b, int i) const
    {
        return *reinterpret_cast<const uint4 *>(rec(b) + 16 * i);
    }
    __device__ __forceinline__ int sum32(int b, int j) const
    {
        return reinterpret_cast<const int32_t *>(rec(b) + R::kSumOff)[j];
    }
    __device__ __forceinline__ int sum16(int b, int k) const
    {
        return reinterpret_cast<const int32_t *>(rec(b) + R::kSumOff)[k];
    }
    __device__ __forceinline__ qg_act_scale scale(int b, int j, int) const
    {
        return reinterpret_cast<const qg_act_scale *>(rec(b) + R::kScOff)[j];
    }
};

// One block of one activation row quantized by the wave itself, four codes per lane (lane
// l holds codes 4l..4l+3).  Every value the dot needs is read out of its lane with
// v_readlane, so it reaches the dot as a scalar (SGPR) operand like ActGlobal's.
struct ActWave {
    uint32_t packed;   // lane l: codes 4l..4l+3
    int s16;           // lane l: sum of the 16 codes of its quad
    int s32;           // lane l: sum of the 32 codes of its octet
    int m, e;          // lane l: the scale of its activation block
    uint32_t me;       // the same packed as a qg_act_scale (e in bits 0..15, m in 16..23)
    __device__ __forceinline__ uint4 codes16(int, int i) const
    {
        return make_uint4((uint32_t)__builtin_amdgcn_readlane((int)packed, 4 * i),
                          (uint32_t)__builtin_amdgcn_readlane((int)packed, 4 * i + 1),
                          (uint32_t)__builtin_amdgcn_readlane((int)packed, 4 * i + 2),
                          (uint32_t)__builtin_amdgcn_readlane((int)packed, 4 * i + 3));
    }
    __device__ __forceinline__ int sum32(int, int j) const { return __builtin_amdgcn_readlane(s32, 8 * j); }
    __device__ __forceinline__ int sum16(int, int k) const { return __builtin_amdgcn_readlane(s16, 4 * k); }
    __device__ __forceinline__ qg_act_scale scale(int, int j, int per_block) const
    {
        const int l = per_block == 1 ? 0 : 8 * j;
        const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)me, l);
        qg_act_scale s;
        s.e = (int16_t)(v & 0xFFFFu);
        s.m = (uint8_t)(v >> 16);
        s.pad = 0;
        return s;
    }
};

// The same with the block's 256 codes already read out into 64 scalar registers (done
// before the weight tile arrives, so the readouts stay off the tile's critical path).
struct ActWaveCodes {
    uint32_t c[64];
    ActWave w;
    __device__ __forceinline__ explicit ActWaveCodes(const ActWave &a) : w(a)
    {
#pragma unroll
        for (int i = 0; i < 64; i++) c[i] = (uint32_t)__builtin_amdgcn_readlane((int)a.packed, i);
    }
    __device__ __forceinline__ uint4 codes16(int, int i) const
    {
        return make_uint4(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
    }
    __device__ __forceinline__ int sum32(int b, int j) const { return w.sum32(b, j); }
    __device__ __forceinline__ int sum16(int b, int k) const { return w.sum16(b, k); }
    __device__ __forceinline__ qg_act_scale scale(int b, int j, int per_block) const { return w.scale(b, j, per_block); }
};

// The block's codes as two nibble planes for the 4-bit dot products of a Q4_K-style tile.
// A code is a = 16*ah + al with al = a & 15 (unsigned) and ah = a >> 4 (signed, -8..7).  A
// tile's code byte holds the codes of elements k (low nibble) and k + 16 (high nibble) of
// a 32-element sub-block, so plane dword (i, d) holds, nibble for nibble in the same order,
// the al (or ah) of elements 32i + 4d + t and 32i + 16 + 4d + t, t = 0..3.  Then with
// q' = q - 8 (the code nibble with its top bit flipped: a signed nibble),
//     sum q*a = 16 * (sum q'*ah + 8 * sum ah) + sum q*al,
// one signed and one unsigned v_dot8 per code dword.  kh[i] = 8 * (sum of ah over
// sub-block i).  Built once per block from the lanes' codes, before the tile is waited for.
struct ActPlanes {
    uint32_t al[32], ah[32];
    int kh[8];
    ActWave w;
    __device__ __forceinline__ explicit ActPlanes(const ActWave &a) : w(a)
    {
        const uint32_t lo = a.packed & 0x0F0F0F0Fu;
        const uint32_t hi = (a.packed >> 4) & 0x0F0F0F0Fu;
        // lane 8i + d (d < 4) pairs its codes with those of lane 8i + 4 + d (elements + 16)
        const uint32_t lo16 = (uint32_t)dpp<kDppRowShl4>((int)lo);
        const uint32_t hi16 = (uint32_t)dpp<kDppRowShl4>((int)hi);
        const uint32_t AL = lo | (lo16 << 4);
        const uint32_t AH = hi | (hi16 << 4);
        const int sh = quad_sum(__builtin_amdgcn_sdot8((int)AH, 0x11111111, 0, false));
#pragma unroll
        for (int i = 0; i < 8; i++) {
#pragma unroll
            for (int d = 0; d < 4; d++) {
                al[4 * i + d] = (uint32_t)__builtin_amdgcn_readlane((int)AL, 8 * i + d);
                ah[4 * i + d] = (uint32_t)__builtin_amdgcn_readlane((int)AH, 8 * i + d);
            }
            kh[i] = 8 * __builtin_amdgcn_readlane(sh, 8 * i);
        }
    }
    __device__ __forceinline__ int sum32(int b, int j) const { return w.sum32(b, j); }
    __device__ __forceinline__ int sum16(int b, int k) const { return w.sum16(b, k); }
    __device__ __forceinline__ qg_act_scale scale(int b, int j, int per_block) const { return w.scale(b, j, per_block); }
};

// The same values as ActPlanes and ActWaveCodes, handed out through a wave-private LDS area
// instead of v_readlane (one VALU instruction per value): every lane writes its share, then
// each lane reads the whole set back with broadcast ds_read_b128 (one address for the wave), so
// the values arrive as wave-uniform VGPRs.  A wave's LDS operations run in order, so its reads
// see its writes; a later block's writes come after this block's reads in program order.
constexpr int kActAreaWords = 160;   // per wave: 128 plane (or code) words, then 32 of sums

__device__ __forceinline__ uint4 lds_bcast16(const uint32_t *p) { return *reinterpret_cast<const uint4 *>(p); }

struct ActPlanesLds {
    uint32_t al[32], ah[32];
    int kh[8], s32[8];
    ActWave w;
    __device__ __forceinline__ ActPlanesLds(const ActWave &a, uint32_t *area, int lane) : w(a)
    {
        const uint32_t lo = a.packed & 0x0F0F0F0Fu;
        const uint32_t hi = (a.packed >> 4) & 0x0F0F0F0Fu;
        const uint32_t AL = lo | ((uint32_t)dpp<kDppRowShl4>((int)lo) << 4);
        const uint32_t AH = hi | ((uint32_t)dpp<kDppRowShl4>((int)hi) << 4);
        const int sh = quad_sum(__builtin_amdgcn_sdot8((int)AH, 0x11111111, 0, false));
        area[lane] = AL;
        area[64 + lane] = AH;
        if ((lane & 7) == 0) {
            area[128 + (lane >> 3)] = (uint32_t)(8 * sh);
            area[136 + (lane >> 3)] = (uint32_t)a.s32;
        }
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint4 l4 = lds_bcast16(area + 8 * i), h4 = lds_bcast16(area + 64 + 8 * i);
            al[4 * i] = l4.x; al[4 * i + 1] = l4.y; al[4 * i + 2] = l4.z; al[4 * i + 3] = l4.w;
            ah[4 * i] = h4.x; ah[4 * i + 1] = h4.y; ah[4 * i + 2] = h4.z; ah[4 * i + 3] = h4.w;
        }
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const uint4 a4 = lds_bcast16(area + 128 + 4 * k), s4 = lds_bcast16(area + 136 + 4 * k);
            kh[4 * k] = (int)a4.x; kh[4 * k + 1] = (int)a4.y; kh[4 * k + 2] = (int)a4.z; kh[4 * k + 3] = (int)a4.w;
            s32[4 * k] = (int)s4.x; s32[4 * k + 1] = (int)s4.y; s32[4 * k + 2] = (int)s4.z; s32[4 * k + 3] = (int)s4.w;
        }
    }
    __device__ __forceinline__ int sum32(int, int j) const { return s32[j]; }
    __device__ __forceinline__ int sum16(int b, int k) const { return w.sum16(b, k); }
    __device__ __forceinline__ qg_act_scale scale(int b, int j, int per_block) const { return w.scale(b, j, per_block); }
};

struct ActCodesLds {
    uint32_t c[64];
    int s16[16];
    ActWave w;
    __device__ __forceinline__ ActCodesLds(const ActWave &a, uint32_t *area, int lane) : w(a)
    {
        area[lane] = a.packed;
        if ((lane & 3) == 0) area[128 + (lane >> 2)] = (uint32_t)a.s16;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint4 v = lds_bcast16(area + 4 * i);
            c[4 * i] = v.x; c[4 * i + 1] = v.y; c[4 * i + 2] = v.z; c[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint4 v = lds_bcast16(area + 128 + 4 * k);
            s16[4 * k] = (int)v.x; s16[4 * k + 1] = (int)v.y; s16[4 * k + 2] = (int)v.z; s16[4 * k + 3] = (int)v.w;
        }
    }
    __device__ __forceinline__ uint4 codes16(int, int i) const
    {
        return make_uint4(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
    }
    __device__ __forceinline__ int sum32(int b, int j) const { return w.sum32(b, j); }
    __device__ __forceinline__ int sum16(int, int k) const { return s16[k]; }
    __device__ __forceinline__ qg_act_scale scale(int b, int j, int per_block) const { return w.scale(b, j, per_block); }
};

// ---------------------------------------------------------------------------------------
// Weight-side decoding

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
__device__ __forceinline__ int q4k_sub_dot(uint4 w, uint4 a0, uint4 a1)
{
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

// The integer dot of sub-block i of a Q4_K-style tile with the activation source.
template <class Act>
__device__ __forceinline__ int q4k_sub(const uint4 &w, int b, int i, const Act &act)
{
    return q4k_sub_dot(w, act.codes16(b, 2 * i), act.codes16(b, 2 * i + 1));
}

template <class Planes>
__device__ __forceinline__ int q4k_sub_planes(const uint4 &w, int i, const Planes &p)
{
    int X = p.kh[i];
    uint32_t Y = 0;
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        X = __builtin_amdgcn_sdot8((int)(q[d] ^ 0x88888888u), (int)p.ah[4 * i + d], X, false);
        Y = __builtin_amdgcn_udot8(q[d], p.al[4 * i + d], Y, false);
    }
    return 16 * X + (int)Y;
}

__device__ __forceinline__ int q4k_sub(const uint4 &w, int, int i, const ActPlanesLds &p)
{
    return q4k_sub_planes(w, i, p);
}

__device__ __forceinline__ int q4k_sub(const uint4 &w, int, int i, const ActPlanes &p)
{
    int X = p.kh[i];
    uint32_t Y = 0;
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; d++) {
        X = __builtin_amdgcn_sdot8((int)(q[d] ^ 0x88888888u), (int)p.ah[4 * i + d], X, false);
        Y = __builtin_amdgcn_udot8(q[d], p.al[4 * i + d], Y, false);
    }
    return 16 * X + (int)Y;
}

// Integer dots of two 16-element Q6_K sub-blocks (2i, 2i+1): 4-bit low parts from ql, 2-bit
// high parts from the qh bit pairs 4s..4s+1 (sub-block 2i) and 4s+2..4s+3 (sub-block 2i+1).
template <int S>
__device__ __forceinline__ void q6k_sub_dots(uint4 L, uint4 H, uint4 a0, uint4 a1, int &P0, int &P1)
{
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
// One lane's share of a tile, held in registers between its loads and its use.  The image is
// read once per call, so its loads are non-temporal (streamed past the caches).

__device__ __forceinline__ uint4 ld_stream(const uint8_t *p)
{
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int FMT>
struct TileRegs;

template <>
struct TileRegs<QG_Q4K> {
    static constexpr int kBytes = kTileBytesQ4K;
    uint4 w[8];     // code chunks (sub-blocks 0..7)
    uint4 meta;     // d | dmin << 16, then the 96-bit sc/mn field string
    // Issued in the order they are used (the meta chunk, then sub-blocks 0..7), each kept
    // in place, so a wave waits for one chunk at a time and starts on the first while the
    // rest are in flight.
    __device__ __forceinline__ void load(const uint8_t *tile, int lane)
    {
        meta = ld_stream(tile + 8192 + 16 * lane);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __builtin_amdgcn_sched_barrier(0);
            w[i] = ld_stream(tile + 1024 * i + 16 * lane);
        }
    }
};

template <>
struct TileRegs<QG_Q6K> {
    static constexpr int kBytes = kTileBytesQ6K;
    uint4 L[8];     // low 4 bits of the codes
    uint4 H[4];     // high 2 bits
    uint4 sc;       // sixteen int8 sub-block scales
    uint32_t d;     // binary16 bits of the block scale
    // the scales first, then each pair of sub-blocks' low and high bits in the order they are
    // used (L0 H0 L1 L2 H1 L3 ...), each kept in place so a pair waits for its own chunks only
    __device__ __forceinline__ void load(const uint8_t *tile, int lane)
    {
        d = *reinterpret_cast<const uint16_t *>(tile + 13312 + 2 * lane);
        sc = ld_stream(tile + 12288 + 16 * lane);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __builtin_amdgcn_sched_barrier(0);
            L[i] = ld_stream(tile + 1024 * i + 16 * lane);
            if ((i & 1) == 0) {
                __builtin_amdgcn_sched_barrier(0);
                H[i >> 1] = ld_stream(tile + 8192 + 1024 * (i >> 1) + 16 * lane);
            }
        }
    }
};

// The 32-element-block formats: eight blocks per tile, their eight binary16 scales in one
// 16-byte load per lane.
template <>
struct TileRegs<QG_Q8_0> {
    static constexpr int kBytes = kTileBytesQ8_0;
    uint4 w[16];    // int8 codes of elements 16i .. 16i+15
    uint4 d;        // binary16 bits of the eight blocks' scales
    // the scales first, then the code chunks in the order they are used (as the Q4_K tile)
    __device__ __forceinline__ void load(const uint8_t *tile, int lane)
    {
        d = ld_stream(tile + 16384 + 16 * lane);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            __builtin_amdgcn_sched_barrier(0);
            w[i] = ld_stream(tile + 1024 * i + 16 * lane);
        }
    }
};

template <>
struct TileRegs<QG_Q4_0> {
    static constexpr int kBytes = kTileBytesQ4_0;
    uint4 w[8];     // block i's 32 codes, nibble-split as in the Q4_K-style tile
    uint4 d;        // binary16 bits of the eight blocks' scales
    __device__ __forceinline__ void load(const uint8_t *tile, int lane)
    {
        d = ld_stream(tile + 8192 + 16 * lane);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __builtin_amdgcn_sched_barrier(0);
            w[i] = ld_stream(tile + 1024 * i + 16 * lane);
        }
    }
};

// ---------------------------------------------------------------------------------------
// The piece of one (row, block) pair for one activation column.

template <int MODE, class Act>
__device__ __forceinline__ float pair_piece(const TileRegs<QG_Q4K> &T, int b, const Act &act)
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
    if constexpr (MODE == QG_PERBLOCK) {
        // Everything that needs the meta chunk alone (it arrives first) is done before the
        // code chunks are waited for: the offset sum, the block scales and their product
        // with it (exact, as in piece_q4k_perblock_near).
        int Cb = 0, Ob = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) Ob = mad_i24((int)(f[i] >> 6), act.sum32(b, i), Ob);
        const qg_act_scale s = act.scale(b, 0, 1);
        const float fd = f16_value(T.meta.x), fm = f16_value(T.meta.x >> 16);
        const bool near = __all(q4k_near(fd, fm));
        const double Dd = (double)fd, S = __builtin_ldexp((double)s.m, s.e);
        const double nOD = -((double)Ob * (double)fm);
        // sub-block by sub-block in load order: each waits for its own chunk only
        // (|P| < 2^16, sc < 64: |Cb| < 2^25)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            __builtin_amdgcn_sched_barrier(0);
            const int P = q4k_sub(T.w[i], b, i, act);
            Cb = mad_i24((int)(f[i] & 63u), P, Cb);
        }
        if (near) {
            const double X = __builtin_fma((double)Cb, Dd, nOD) * S;
            // an activation exponent >= kNoTinyExp: X is 0 or at least 2^-102, so the
            // conversion needs no flush, and adding +0 turns an exact -0 into +0
            if (s.e >= kNoTinyExp) return (float)X + 0.0f;
            return r32_exact_double(X);
        }
        return piece_q4k_perblock(Cb, Ob, T.meta.x, s.m, s.e);
    } else {
        // the sub-block sums, then the activation side (the same for every row)
        int m[8], e[8], Cj[8], Oj[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            Cj[i] = mul_i24((int)(f[i] & 63u), q4k_sub(T.w[i], b, i, act));
            Oj[i] = mul_i24((int)(f[i] >> 6), act.sum32(b, i));
            const qg_act_scale s = act.scale(b, i, 8);
            m[i] = s.m;
            e[i] = s.e;
        }
        const Sub32Act g = sub32_act(m, e);
        float r;
        if (g.fast && sub32_first_route(Cj, Oj, g, T.meta.x, r)) return r;
        return piece_q4k_sub32(Cj, Oj, g, T.meta.x);
    }
}

template <int MODE, class Act>
__device__ __forceinline__ float pair_piece(const TileRegs<QG_Q6K> &T, int b, const Act &act)
{
    const uint32_t sw[4] = {T.sc.x, T.sc.y, T.sc.z, T.sc.w};
    int Ck[16];
    // sub-block pairs in load order, each waiting for its own chunks
#pragma unroll
    for (int i = 0; i < 8; i++) {
        __builtin_amdgcn_sched_barrier(0);
        int P0, P1;
        const uint4 a0 = act.codes16(b, 2 * i), a1 = act.codes16(b, 2 * i + 1);
        if (i & 1) q6k_sub_dots<1>(T.L[i], T.H[i >> 1], a0, a1, P0, P1);
        else q6k_sub_dots<0>(T.L[i], T.H[i >> 1], a0, a1, P0, P1);
        // (q - 32) . a = q . a - 32 * sum(a)
        const int s0 = (int)(int8_t)(sw[(2 * i) >> 2] >> (8 * ((2 * i) & 3)));
        const int s1 = (int)(int8_t)(sw[(2 * i + 1) >> 2] >> (8 * ((2 * i + 1) & 3)));
        // |P - 32 * sum| < 2^18, |s| <= 128
        Ck[2 * i] = mul_i24(s0, P0 - 32 * act.sum16(b, 2 * i));
        Ck[2 * i + 1] = mul_i24(s1, P1 - 32 * act.sum16(b, 2 * i + 1));
    }
    if constexpr (MODE == QG_PERBLOCK) {
        int Cb = 0;
#pragma unroll
        for (int k = 0; k < 16; k++) Cb += Ck[k];
        const qg_act_scale s = act.scale(b, 0, 1);
        return piece_q6k_perblock(Cb, T.d, s.m, s.e);
    } else {
        long long C[8];
        uint32_t db[8];
        int m[8], e[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const qg_act_scale s = act.scale(b, j, 8);
            C[j] = (long long)(Ck[2 * j] + Ck[2 * j + 1]);
            db[j] = T.d;
            m[j] = s.m;
            e[j] = s.e;
        }
        return piece_sub32_scaled(C, db, m, e);
    }
}

// The integer block sum C_j of block j of a 32-element-block tile (w = d*q for Q8_0,
// d*(q - 8) for Q4_0) against the activation block's codes.  |C_j| <= 32 * 128 * 127 < 2^19.
__device__ __forceinline__ int b32_sum(const TileRegs<QG_Q8_0> &T, const ActWaveCodes &act, int j)
{
    int P = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint4 w = T.w[2 * j + h];
        const int c = 8 * j + 4 * h;
        P = sdot4(w.x, act.c[c], P);
        P = sdot4(w.y, act.c[c + 1], P);
        P = sdot4(w.z, act.c[c + 2], P);
        P = sdot4(w.w, act.c[c + 3], P);
    }
    return P;
}

// (q - 8) . a = q . a - 8 * sum(a)
__device__ __forceinline__ int b32_sum(const TileRegs<QG_Q4_0> &T, const ActPlanes &act, int j)
{
    return q4k_sub(T.w[j], 0, j, act) - 8 * act.sum32(0, j);
}

// The pieces of one tile row: PerBlock, one per 32-element block, R32(m_j*2^e_j * d_j * C_j)
// (|C_j| < 2^19, d_j and m_j of 11 and 8 significant bits: the products are exact in f64 and
// the conversion is the one rounding); Sub32, one per tile, the eight terms summed exactly.
template <int MODE, int FMT, class Act>
__device__ __forceinline__ void b32_pieces(const TileRegs<FMT> &T, const Act &act,
                                           float (&p)[MODE == QG_PERBLOCK ? 8 : 1])
{
    int C[8];
    const uint32_t dw[4] = {T.d.x, T.d.y, T.d.z, T.d.w};
    if constexpr (MODE == QG_PERBLOCK) {
        // block by block in load order, each waiting for its own code chunks; with the block's
        // activation exponent >= kNoTinyExp the piece cannot be tiny (no flush, +0 for -0)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            __builtin_amdgcn_sched_barrier(0);
            C[j] = b32_sum(T, act, j);
            const qg_act_scale s = act.scale(0, j, 8);
            const double S = __builtin_ldexp((double)s.m, s.e);
            const double D = (double)f16_value(dw[j >> 1] >> (16 * (j & 1)));
            const double X = (double)C[j] * D * S;
            p[j] = s.e >= kNoTinyExp ? (float)X + 0.0f : r32_exact_double(X);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) C[j] = b32_sum(T, act, j);
        long long Cl[8];
        uint32_t db[8];
        int m[8], e[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const qg_act_scale s = act.scale(0, j, 8);
            Cl[j] = C[j];
            db[j] = (dw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            m[j] = s.m;
            e[j] = s.e;
        }
        p[0] = piece_sub32_scaled(Cl, db, m, e);
    }
}

// ---------------------------------------------------------------------------------------
// A workgroup's work on its 64-row group once the activations are in place.  W waves split
// the group's G blocks (wave w takes blocks w, w+W, ...); with DB (more blocks than waves)
// each wave loads its next tile while the current one is computed.  Pieces are parked in
// LDS; after a barrier the first wave adds each row's pieces in block order, one row per
// lane.  `act_of(c)` hands out column c's activation source.

template <int FMT, int MODE, int NC, int W, bool DB, class ActOf>
__device__ __forceinline__ void group_pieces_and_rows(const uint8_t *gbase, int G, int wid, int lane,
                                                      TileRegs<FMT> &t0, TileRegs<FMT> &t1,
                                                      const ActOf &act_of, float *s_piece, int64_t row0,
                                                      int rows, int col0, int ncol, float *__restrict__ out)
{
    using T = TileRegs<FMT>;
    auto compute = [&](const T &tile, int b) {
#pragma unroll
        for (int c = 0; c < NC; c++) s_piece[((size_t)c * G + b) * 64 + lane] = pair_piece<MODE>(tile, b, act_of(c));
    };
    if constexpr (DB) {
        // two register sets, no copies: t0 holds blocks wid, wid+2W, ...; t1 holds wid+W, ...
        for (int b = wid; b < G; b += 2 * W) {
            if (b + W < G) t1.load(gbase + (size_t)(b + W) * T::kBytes, lane);
            compute(t0, b);
            if (b + W >= G) break;
            if (b + 2 * W < G) t0.load(gbase + (size_t)(b + 2 * W) * T::kBytes, lane);
            compute(t1, b + W);
        }
    } else {
        // at most one block per wave
        if (wid < G) compute(t0, wid);
    }
    __syncthreads();

    if (wid == 0) {
        const int64_t row = row0 + lane;
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const float y = fold_ftz(0.0f, s_piece + (size_t)c * G * 64 + lane, G, 64);
            if (row < rows && col0 + c < ncol) out[(int64_t)(col0 + c) * rows + row] = canon_nan(y);
        }
    }
}

// Several columns.  blockIdx.x = 64-row group, blockIdx.y = batch of NC activation columns.

template <int FMT, int MODE, int NC, int W, bool DB>
__global__ __launch_bounds__(64 * W) void gemv_kernel(const uint8_t *__restrict__ image, int rows, int G,
                                                      const int8_t *__restrict__ codes,
                                                      const qg_act_scale *__restrict__ scales,
                                                      const int32_t *__restrict__ csums, int ncol,
                                                      float *__restrict__ out)
{
    extern __shared__ __align__(16) unsigned char lds[];
    using T = TileRegs<FMT>;
    using R = ActRec<FMT, MODE>;
    const int C = G * 256;
    const int nsc = MODE == QG_PERBLOCK ? G : G * 8;
    const int g = blockIdx.x;
    const int col0 = blockIdx.y * NC;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t *gbase = image + (size_t)g * G * T::kBytes;

    // the wave's first tile: loads in flight before anything else
    T t0;
    [[maybe_unused]] T t1;
    if (wid < G) t0.load(gbase + (size_t)wid * T::kBytes, lane);

    static_assert(NC > 1, "one column runs in gemv1_kernel");
    {
        // stage NC columns as per-block records (codes, code sums, scales)
        unsigned char *rec = lds;
        for (int c = 0; c < NC; c++) {
            const int col = col0 + c;
            const bool have = col < ncol;
            unsigned char *rc = rec + (size_t)c * G * R::kStride;
            const uint4 *src = reinterpret_cast<const uint4 *>(codes + (size_t)col * C);
            for (int i = threadIdx.x; i < C / 16; i += 64 * W)
                *reinterpret_cast<uint4 *>(rc + (size_t)(i >> 4) * R::kStride + 16 * (i & 15)) =
                    have ? src[i] : make_uint4(0, 0, 0, 0);
            const int32_t *cs = csums + (size_t)col * (C / 16);
            for (int i = threadIdx.x; i < G * R::kSums; i += 64 * W) {
                int32_t v = 0;
                if (have) v = R::kSums == 8 ? cs[2 * i] + cs[2 * i + 1] : cs[i];
                *reinterpret_cast<int32_t *>(rc + (size_t)(i / R::kSums) * R::kStride + R::kSumOff +
                                             4 * (i % R::kSums)) = v;
            }
            // qg_act_scale is 4 bytes: copy it as one word
            const uint32_t *scw = reinterpret_cast<const uint32_t *>(scales) + (size_t)col * nsc;
            for (int i = threadIdx.x; i < nsc; i += 64 * W)
                *reinterpret_cast<uint32_t *>(rc + (size_t)(i / R::kScales) * R::kStride + R::kScOff +
                                              4 * (i % R::kScales)) = have ? scw[i] : 0u;
        }
        __syncthreads();
        float *s_piece = reinterpret_cast<float *>(lds + (size_t)NC * G * R::kStride);
        auto act_of = [&](int c) { return ActLds<FMT, MODE>{lds + (size_t)c * G * R::kStride}; };
        group_pieces_and_rows<FMT, MODE, NC, W, DB>(gbase, G, wid, lane, t0, t1, act_of, s_piece, (int64_t)g * 64,
                                                    rows, col0, ncol, out);
    }
}

// ---------------------------------------------------------------------------------------
// One activation column.  Each wave brings the activation blocks it multiplies (wave w:
// blocks w, w+W, ...) into its own registers, four codes per lane: SRC_F32 quantizes the
// f32 row itself (the one-launch quantize + GEMV), SRC_CODES loads the quantized row.  A
// block's activation load is issued ahead of its weight tile, so getting the codes ready
// (quantizing, summing, reading them out into scalar registers) waits for that load alone
// and overlaps the weight stream.  With SRC_F32 workgroup 0 also writes the quantized row
// out exactly as qg_quantize_act does; the per-lane arithmetic is the same function.

enum { SRC_F32 = 0, SRC_CODES = 1 };

struct ActIO {
    const float *x;               // SRC_F32: the f32 row
    const int8_t *codes_in;       // SRC_CODES: the quantized row
    const uint32_t *scales_in;    //   and its qg_act_scale words
    int8_t *codes_out;            // SRC_F32: where workgroup 0 writes the quantized row
    qg_act_scale *scales_out;
    int32_t *csums_out;
    int32_t *err_flag;            // may be null
    unsigned long long *argmax;   // may be null: the row's argmax key is folded in here
};

// argmax of the output row ("Module numerics", Functions argmax) as one 64-bit key per row:
// the value's bits mapped so that unsigned order is numeric order (+0 and -0 both map to +0's
// key) in the high word, and ~row in the low word, so the larger key is the larger value and,
// among equals, the lower row.  A NaN, or a padding row, gives 0: "none".
__device__ __forceinline__ unsigned long long argmax_key(float y, int64_t row, bool valid)
{
    if (!valid || y != y) return 0ull;
    uint32_t u = __float_as_uint(y);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;                       // -0 equals +0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)row);
}

// Keeps the loads issued above here: a compiler-only barrier (no instruction, no wait) that
// neither the IR passes nor the scheduler move memory operations across.  (Loads through a
// const __restrict__ kernel argument count as invariant and would still move, so the
// kernel's image pointer is a plain one.)
__device__ __forceinline__ void load_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int SRC>
struct ActRaw;
template <>
struct ActRaw<SRC_F32> {
    float4 v;                     // elements 4l .. 4l+3 of the block
};
template <>
struct ActRaw<SRC_CODES> {
    uint32_t packed;              // codes 4l .. 4l+3 of the block
    uint32_t scale;               // the qg_act_scale word of the lane's activation block
};

// GL = lanes per activation block (64: one scale per 256 elements; 8: one per 32)
template <int SRC, int GL>
__device__ __forceinline__ ActRaw<SRC> load_act(const ActIO &io, int b, int lane)
{
    ActRaw<SRC> r;
    if constexpr (SRC == SRC_F32) {
        r.v = *reinterpret_cast<const float4 *>(io.x + (size_t)b * 256 + 4 * lane);
    } else {
        r.packed = reinterpret_cast<const uint32_t *>(io.codes_in + (size_t)b * 256)[lane];
        r.scale = io.scales_in[GL == 64 ? (size_t)b : (size_t)b * 8 + (lane >> 3)];
    }
    return r;
}

// Quantizes one block; workgroup 0 (emit) writes block b < G out.
template <int BITS, int GROUP_LANES>
__device__ __forceinline__ ActWave quantize_block_in_wave(float4 v, int b, int G, int lane, bool emit,
                                                          const ActIO &io)
{
    const QuantLane q = quantize_lane<BITS, GROUP_LANES>(v);
    ActWave a;
    a.packed = q.packed;
    a.s16 = quad_sum(q.sum4);                  // sums of 16 consecutive codes = 4 lanes
    a.s32 = octet_sum_of_quads(a.s16);
    a.m = q.m;
    a.e = q.e;
    a.me = ((uint32_t)q.e & 0xFFFFu) | ((uint32_t)q.m << 16);
    if (b < G) {
        const bool leader = (lane & (GROUP_LANES - 1)) == 0;
        if (emit) {
            reinterpret_cast<uint32_t *>(io.codes_out + (size_t)b * 256)[lane] = q.packed;
            if ((lane & 3) == 0) io.csums_out[(size_t)b * 16 + (lane >> 2)] = a.s16;
            if (leader) {
                qg_act_scale sc;
                sc.e = (int16_t)q.e;
                sc.m = (uint8_t)q.m;
                sc.pad = 0;
                io.scales_out[(size_t)b * (64 / GROUP_LANES) + lane / GROUP_LANES] = sc;
            }
        }
        if (q.inf && leader && io.err_flag) *io.err_flag = 1;
    }
    return a;
}

template <int SRC, int BITS, int GL>
__device__ __forceinline__ ActWave ready_act(const ActRaw<SRC> &r, int b, int G, int lane, bool emit, const ActIO &io)
{
    if constexpr (SRC == SRC_F32) {
        return quantize_block_in_wave<BITS, GL>(r.v, b, G, lane, emit, io);
    } else {
        ActWave a;
        a.packed = r.packed;
        a.s16 = quad_sum(__builtin_amdgcn_sdot4((int)r.packed, 0x01010101, 0, false));
        a.s32 = octet_sum_of_quads(a.s16);
        a.m = (int)((r.scale >> 16) & 0xFFu);
        a.e = (int)(int16_t)(r.scale & 0xFFFFu);
        a.me = r.scale;
        return a;
    }
}

// The block's piece: its codes go to scalar registers (as nibble planes for Q4_K-style
// tiles) before the tile's data is waited for.
template <int FMT, int MODE>
__device__ __forceinline__ float piece_one_lds(const TileRegs<FMT> &t, int b, const ActWave &a, uint32_t *area, int lane)
{
    if constexpr (FMT == QG_Q4K) {
        const ActPlanesLds p(a, area, lane);
        __builtin_amdgcn_sched_barrier(0);
        return pair_piece<MODE>(t, b, p);
    } else {
        const ActCodesLds c(a, area, lane);
        __builtin_amdgcn_sched_barrier(0);
        return pair_piece<MODE>(t, b, c);
    }
}

template <int FMT, int MODE>
__device__ __forceinline__ float piece_one(const TileRegs<FMT> &t, int b, const ActWave &a)
{
    if constexpr (FMT == QG_Q4K) {
        const ActPlanes p(a);
        __builtin_amdgcn_sched_barrier(0);
        return pair_piece<MODE>(t, b, p);
    } else {
        const ActWaveCodes c(a);
        __builtin_amdgcn_sched_barrier(0);
        return pair_piece<MODE>(t, b, c);
    }
}

// The matrices of one launch, all multiplied by the same activation row: workgroups
// gstart[m] .. gstart[m+1]-1 are the 64-row groups of matrix m.
struct Targets {
    int nmat;
    int gstart[QG_MAX_MATRICES + 1];
    int rows[QG_MAX_MATRICES];
    const uint8_t *image[QG_MAX_MATRICES];
    float *out[QG_MAX_MATRICES];
};

// This workgroup's matrix: the last one whose first group is at or before blockIdx.x (an
// empty matrix starts where the next one does; past nmat the starts equal the total).  Every
// index is a compile-time constant, so the descriptor's fields come in one batch of scalar
// loads rather than through loads that wait on each other.
struct Picked {
    const uint8_t *image;
    float *out;
    int rows, g;
};

// A value as an opaque scalar register: the selects below then choose between values, and the
// compiler cannot turn them back into one load through a computed index.
template <class V>
__device__ __forceinline__ V opaque_sgpr(V v)
{
    asm("" : "+s"(v));
    return v;
}

// The same for a pointer into global memory; it comes back as a global-address-space pointer
// seen through a generic one, so accesses through it stay global (not flat) loads and stores.
template <class P>
__device__ __forceinline__ P *opaque_global(P *p)
{
    uint64_t v = opaque_sgpr((uint64_t)(uintptr_t)p);
    auto *g = (__attribute__((address_space(1))) P *)(uintptr_t)v;
    return (P *)g;
}

__device__ __forceinline__ Picked pick_matrix(const Targets &tg, int bx)
{
    Picked p{opaque_global(tg.image[0]), opaque_global(tg.out[0]), opaque_sgpr(tg.rows[0]), bx};
    if (tg.nmat == 1) return p;
#pragma unroll
    for (int k = 1; k < QG_MAX_MATRICES; k++) {
        const int start = opaque_sgpr(tg.gstart[k]);
        const uint8_t *image = opaque_global(tg.image[k]);
        float *out = opaque_global(tg.out[k]);
        const int rows = opaque_sgpr(tg.rows[k]);
        const bool here = bx >= start;
        p.image = here ? image : p.image;
        p.out = here ? out : p.out;
        p.rows = here ? rows : p.rows;
        p.g = here ? bx - start : p.g;
    }
    return p;
}

// whether any of the W flag bytes is set (wave-uniform)
template <int W>
__device__ __forceinline__ bool any_flag(const unsigned char *f)
{
    uint32_t v;
    if constexpr (W == 16) {
        const uint4 q = *reinterpret_cast<const uint4 *>(f);
        v = q.x | q.y | q.z | q.w;
    } else if constexpr (W == 8) {
        const uint2 q = *reinterpret_cast<const uint2 *>(f);
        v = q.x | q.y;
    } else {
        v = *reinterpret_cast<const uint32_t *>(f);
    }
    return __builtin_amdgcn_readfirstlane((int)v) != 0;
}

// +0 plus the N pieces p[0], p[stride], ... in order with plain binary32 adds (all reads
// issued first).  Equal to the flushed fold when no piece is tiny: see fold_chain.
template <int N>
__device__ __forceinline__ float fold_fixed(const float *p, int stride)
{
    float a[N];
#pragma unroll
    for (int k = 0; k < N; k++) a[k] = p[(size_t)k * stride];
    float y = 0.0f;
#pragma unroll
    for (int k = 0; k < N; k++) y = y + a[k];
    return y;
}

template <int FMT, int MODE, int SRC, int W, bool DB>
__global__ __launch_bounds__(64 * W) void gemv1_kernel(const Targets tg, int G, ActIO io)
{
    extern __shared__ __align__(16) float s_piece[];
    using T = TileRegs<FMT>;
    constexpr int BITS = ActKind<FMT, MODE>::kBits, GL = ActKind<FMT, MODE>::kLanes;
    // pieces: G per row with DB, else W (one per wave); then one flag byte per wave (16 bytes);
    // then each wave's activation area
    unsigned char *s_small = reinterpret_cast<unsigned char *>(s_piece + (size_t)(DB ? G : W) * 64);
    [[maybe_unused]] uint32_t *area = reinterpret_cast<uint32_t *>(s_small + 16) + (threadIdx.x >> 6) * kActAreaWords;
    bool small = false;                          // a block of this wave may give a tiny piece
    const Picked pm = pick_matrix(tg, (int)blockIdx.x);   // this workgroup's matrix (wave-uniform)
    const int g = pm.g;
    const int rows = pm.rows;
    float *out = pm.out;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool emit = blockIdx.x == 0;           // the first workgroup writes the quantized row out
    const uint8_t *gbase = pm.image + (size_t)g * G * T::kBytes;

    // the first block's activations, then its tile: both loads unconditional (a wave past
    // the last block works on a copy of it and stores nothing), kept in this order
    const int bf = min(wid, G - 1);
    ActRaw<SRC> r0 = load_act<SRC, GL>(io, bf, lane);
    // Quantizing in the wave: every wave's activation load is issued before any wave's tile
    // loads (a barrier that waits for no memory), so the quantizing work starts ahead of the
    // weight stream (measured: 0.2 us of a 7.2 us launch; without quantizing it costs more
    // than it gains).
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SRC == SRC_F32) __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    T t0;
    [[maybe_unused]] T t1;
    t0.load(gbase + (size_t)bf * T::kBytes, lane);
    load_fence();
    ActWave a0 = ready_act<SRC, BITS, GL>(r0, wid, G, lane, emit, io);

    // Every use of the first tile is unconditional too, so the compiler cannot sink its loads
    // below the wait for the activation load.
    if constexpr (DB) {
        // blocks wid, wid + W, ...: t0 / t1 alternate, the next block's loads in flight
        // while this one is computed.  DB means G > W, so every wave has a first block.
        int b = wid;
        do {
            const int b1 = b + W;
            ActRaw<SRC> r1;
            if (b1 < G) {
                r1 = load_act<SRC, GL>(io, b1, lane);
                __builtin_amdgcn_sched_barrier(0);
                t1.load(gbase + (size_t)b1 * T::kBytes, lane);
                load_fence();
            }
            s_piece[(size_t)b * 64 + lane] = piece_one<FMT, MODE>(t0, b, a0);
            small |= __ballot(a0.e < kNoTinyExp) != 0;
            if (b1 >= G) break;
            const ActWave a1 = ready_act<SRC, BITS, GL>(r1, b1, G, lane, emit, io);
            const int b2 = b + 2 * W;
            if (b2 < G) {
                r0 = load_act<SRC, GL>(io, b2, lane);
                __builtin_amdgcn_sched_barrier(0);
                t0.load(gbase + (size_t)b2 * T::kBytes, lane);
                load_fence();
            }
            s_piece[(size_t)b1 * 64 + lane] = piece_one<FMT, MODE>(t1, b1, a1);
            small |= __ballot(a1.e < kNoTinyExp) != 0;
            if (b2 >= G) break;
            a0 = ready_act<SRC, BITS, GL>(r0, b2, G, lane, emit, io);
            b = b2;
        } while (true);
    } else {
        // at most one block per wave; a wave past the last block computes a copy and parks +0
        // Q4_K-style: the activation planes through LDS (the code words of a Q6_K-style block
        // would not fit the registers of 16 waves beside its tile)
        float p;
        if constexpr (FMT == QG_Q4K) p = piece_one_lds<FMT, MODE>(t0, bf, a0, area, lane);
        else p = piece_one<FMT, MODE>(t0, bf, a0);
        s_piece[(size_t)wid * 64 + lane] = wid < G ? p : 0.0f;
        small |= __ballot(a0.e < kNoTinyExp) != 0;
    }
    if (lane == 0) s_small[wid] = small ? 1 : 0;
    __syncthreads();

    // the first wave adds each row's pieces in block order, one row per lane: plain adds
    // unless a block's activation exponent allows a tiny piece (then the flushed chain)
    if (wid == 0) {
        const int64_t row = (int64_t)g * 64 + lane;
        float y;
        if (any_flag<W>(s_small)) y = fold_flushed(0.0f, s_piece + lane, G, 64);
        else if constexpr (DB) y = fold_chain_plain(0.0f, s_piece + lane, G, 64);
        else y = fold_fixed<W>(s_piece + lane, 64);   // G <= W; the pieces past G are +0
        y = canon_nan(y);
        if (row < rows) out[row] = y;
        if (io.argmax) {
            // the largest key of the group's 64 rows, then one atomic max per workgroup
            unsigned long long k = argmax_key(y, row, row < rows);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const unsigned long long o = __shfl_xor(k, off, 64);
                k = o > k ? o : k;
            }
            if (lane == 0 && k != 0ull) atomicMax(io.argmax, k);
        }
    }
}

// ---------------------------------------------------------------------------------------
// One activation column, Q4_K-style, PerBlock, rows of at most 16 blocks, on small matrices: a
// workgroup owns a quarter of a 64-row group (16 rows), so a matrix of few row groups still
// spreads over every compute unit.  Wave w takes block w as in gemv1_kernel; lane (r, kk) = (l %
// 16, l / 16) takes row r of the quarter and sub-blocks 2kk, 2kk+1 of the block (two 16-byte
// code chunks and the row's block fields).  The block's activation codes are quantized or
// loaded by the wave as in gemv1_kernel (lane l: codes 4l .. 4l+3) and split into nibble
// planes; the planes of sub-blocks 2kk, 2kk+1 sit in lanes 16kk .. 16kk+15, the lane group of
// kk, and reach its lanes by DPP row broadcasts.  Each lane's two integer sub-block sums and
// offset sums are added over the four lane groups (exact integers), then lanes kk = 0 form the
// pieces; the first wave adds each row's pieces in block order.

// v summed over the four 16-lane rows of the wave, in every lane: each swap with a copy of
// itself leaves the two halves (rows) to be added side by side in every lane
__device__ __forceinline__ int sum_over_rows(int v)
{
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // lanes l, l ^ 32
    const int s = (int)h[0] + (int)h[1];
    const auto r = __builtin_amdgcn_permlane16_swap(s, s, false, false);   // rows 2k, 2k + 1
    return (int)r[0] + (int)r[1];
}

template <int CTRL>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v)   // lane n of the lane's row of 16 (CTRL = 0x150 + n)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int SRC>
__global__ __launch_bounds__(1024) void gemv1_quarter_kernel(const Targets tg, int G, ActIO io)
{
    __shared__ __align__(16) float s_piece[16 * 16];     // [wave = block][row of the quarter]
    __shared__ __align__(16) unsigned char s_small[16];
    const int bx = (int)blockIdx.x;
    // the workgroup's matrix and 64-row group (the Targets count 64-row groups)
    const Picked pm = pick_matrix(tg, bx >> 2);
    const int qr = bx & 3;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, kk = lane >> 4;
    const bool emit = bx == 0;
    const int b = min(wid, G - 1);             // a wave past the last block works on a copy and parks nothing
    const int trow = 16 * qr + r;
    const uint8_t *tile = pm.image + ((size_t)pm.g * G + b) * kTileBytesQ4K;

    ActRaw<SRC> raw = load_act<SRC, 64>(io, b, lane);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SRC == SRC_F32) __builtin_amdgcn_s_barrier();   // every wave's activation load first
    __builtin_amdgcn_sched_barrier(0);
    const uint4 meta = ld_stream(tile + 8192 + 16 * trow);
    const uint4 w0 = ld_stream(tile + 1024 * (2 * kk) + 16 * trow);
    const uint4 w1 = ld_stream(tile + 1024 * (2 * kk + 1) + 16 * trow);
    load_fence();
    const ActWave a = ready_act<SRC, 8, 64>(raw, wid, G, lane, emit, io);

    // nibble planes of the codes (as ActPlanes): lane 8i + d (d < 4) holds dword d of sub-block
    // i's planes, so the lane group of kk holds those of sub-blocks 2kk (row lanes 0..3) and
    // 2kk + 1 (row lanes 8..11)
    const uint32_t lo = a.packed & 0x0F0F0F0Fu;
    const uint32_t hi = (a.packed >> 4) & 0x0F0F0F0Fu;
    const uint32_t AL = lo | ((uint32_t)dpp<kDppRowShl4>((int)lo) << 4);
    const uint32_t AH = hi | ((uint32_t)dpp<kDppRowShl4>((int)hi) << 4);
    const uint32_t sh = (uint32_t)quad_sum(__builtin_amdgcn_sdot8((int)AH, 0x11111111, 0, false));
    const uint32_t al[8] = {row_bcast<0x150>(AL), row_bcast<0x151>(AL), row_bcast<0x152>(AL), row_bcast<0x153>(AL),
                            row_bcast<0x158>(AL), row_bcast<0x159>(AL), row_bcast<0x15A>(AL), row_bcast<0x15B>(AL)};
    const uint32_t ah[8] = {row_bcast<0x150>(AH), row_bcast<0x151>(AH), row_bcast<0x152>(AH), row_bcast<0x153>(AH),
                            row_bcast<0x158>(AH), row_bcast<0x159>(AH), row_bcast<0x15A>(AH), row_bcast<0x15B>(AH)};
    const int kh0 = 8 * (int)row_bcast<0x150>(sh), kh1 = 8 * (int)row_bcast<0x158>(sh);
    const int s0 = (int)row_bcast<0x150>((uint32_t)a.s32), s1 = (int)row_bcast<0x158>((uint32_t)a.s32);

    // the fields of sub-blocks 2kk and 2kk + 1: bits 24kk .. 24kk + 23 of the 96-bit string
    const uint64_t pair = kk < 2 ? ((uint64_t)meta.z << 32 | meta.y) : ((uint64_t)meta.w << 32 | meta.z);
    const uint32_t f24 = (uint32_t)(pair >> (kk < 2 ? 24 * kk : 24 * kk - 32)) & 0xFFFFFFu;
    const int sc0 = (int)(f24 & 63u), mn0 = (int)((f24 >> 6) & 63u);
    const int sc1 = (int)((f24 >> 12) & 63u), mn1 = (int)((f24 >> 18) & 63u);

    // sum q*a = 16 * (sum (q-8)*ah + 8 * sum ah) + sum q*al, per sub-block (as q4k_sub)
    const uint32_t q0[4] = {w0.x, w0.y, w0.z, w0.w};
    const uint32_t q1[4] = {w1.x, w1.y, w1.z, w1.w};
    int X0 = kh0, X1 = kh1;
    uint32_t Y0 = 0, Y1 = 0;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        X0 = __builtin_amdgcn_sdot8((int)(q0[d] ^ 0x88888888u), (int)ah[d], X0, false);
        Y0 = __builtin_amdgcn_udot8(q0[d], al[d], Y0, false);
        X1 = __builtin_amdgcn_sdot8((int)(q1[d] ^ 0x88888888u), (int)ah[4 + d], X1, false);
        Y1 = __builtin_amdgcn_udot8(q1[d], al[4 + d], Y1, false);
    }
    int Cp = mad_i24(sc0, 16 * X0 + (int)Y0, mul_i24(sc1, 16 * X1 + (int)Y1));
    int Op = mad_i24(mn0, s0, mul_i24(mn1, s1));
    // the four lane groups' partial sums (exact integers), every lane getting the total
    Cp = sum_over_rows(Cp);
    Op = sum_over_rows(Op);

    const qg_act_scale sa = a.scale(b, 0, 1);
    const float fd = f16_value(meta.x), fm = f16_value(meta.x >> 16);
    float piece;
    if (q4k_near(fd, fm)) {
        const double X = __builtin_fma((double)Cp, (double)fd, -((double)Op * (double)fm)) * __builtin_ldexp((double)sa.m, sa.e);
        // an activation exponent >= kNoTinyExp: X is 0 or at least 2^-102, no flush needed, and
        // adding +0 turns an exact -0 into +0
        piece = sa.e >= kNoTinyExp ? (float)X + 0.0f : r32_exact_double(X);
    } else {
        piece = piece_q4k_perblock(Cp, Op, meta.x, sa.m, sa.e);
    }
    if (kk == 0 && wid < G) s_piece[wid * 16 + r] = piece;
    if (lane == 0) s_small[wid] = (wid < G && sa.e < kNoTinyExp) ? 1 : 0;
    __syncthreads();

    if (wid == 0 && lane < 16) {
        const int64_t row = (int64_t)pm.g * 64 + trow;
        float y;
        if (any_flag<16>(s_small)) y = fold_flushed(0.0f, s_piece + r, G, 16);
        else y = fold_chain_plain(0.0f, s_piece + r, G, 16);
        if (row < pm.rows) pm.out[row] = canon_nan(y);
    }
}

// Several activation columns on the one-column machinery (a quantized activation matrix, at
// most 16 blocks per row): each wave keeps its tile in registers and forms its block's piece
// for NC columns in turn, each column's codes read out into scalar registers as in the
// one-column kernel; the columns' activation loads are issued ahead of the tile.  Column c0 +
// c of the launch is blockIdx.y * NC + c; columns past ncol are worked on as copies of the
// last and dropped.  The first wave adds each row's pieces in block order per column.
struct ActCols {
    const int8_t *codes;          // column c's codes at codes + c * cstride
    const uint32_t *scales;       // its qg_act_scale words at scales + c * sstride
    int64_t cstride, sstride;
};

template <int FMT, int MODE, int NC>
__global__ __launch_bounds__(64 * 16) void gemv1_cols_kernel(const uint8_t *image, int rows, int G, ActCols ac,
                                                            int ncol, float *__restrict__ out)
{
    constexpr int W = 16;
    extern __shared__ __align__(16) float s_piece[];   // [NC][W][64] pieces, then W flag bytes
    unsigned char *s_small = reinterpret_cast<unsigned char *>(s_piece + (size_t)NC * W * 64);
    using T = TileRegs<FMT>;
    constexpr int BITS = ActKind<FMT, MODE>::kBits, GL = ActKind<FMT, MODE>::kLanes;
    const int g = (int)blockIdx.x;
    const int c0 = (int)blockIdx.y * NC;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bf = min(wid, G - 1);
    const uint8_t *gbase = image + (size_t)g * G * T::kBytes;
    const ActIO none{};

    ActRaw<SRC_CODES> r[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int64_t cc = min(c0 + c, ncol - 1);
        ActIO io{};
        io.codes_in = ac.codes + cc * ac.cstride;
        io.scales_in = ac.scales + cc * ac.sstride;
        r[c] = load_act<SRC_CODES, GL>(io, bf, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    T t0;
    t0.load(gbase + (size_t)bf * T::kBytes, lane);
    load_fence();
    bool small = false;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        __builtin_amdgcn_sched_barrier(0);
        const ActWave a = ready_act<SRC_CODES, BITS, GL>(r[c], bf, G, lane, false, none);
        const float p = piece_one<FMT, MODE>(t0, bf, a);
        s_piece[((size_t)c * W + wid) * 64 + lane] = wid < G ? p : 0.0f;
        small |= __ballot(a.e < kNoTinyExp) != 0;
    }
    if (lane == 0) s_small[wid] = small ? 1 : 0;
    __syncthreads();

    if (wid == 0) {
        const int64_t row = (int64_t)g * 64 + lane;
        const bool flushed = any_flag<W>(s_small);
#pragma unroll
        for (int c = 0; c < NC; c++) {
            if (c0 + c >= ncol) break;
            const float *pc = s_piece + (size_t)c * W * 64 + lane;
            const float y = flushed ? fold_flushed(0.0f, pc, G, 64) : fold_fixed<W>(pc, 64);
            if (row < rows) out[(int64_t)(c0 + c) * rows + row] = canon_nan(y);
        }
    }
}

// One activation column over a 32-element-block format.  A row has up to eight pieces per
// tile (PerBlock), too many to park all of a long row's in LDS, so the workgroup goes through
// its blocks in rounds of W (wave w takes block rW + w of round r): each round's pieces go to
// one of two LDS slots, and after the round's barrier the first wave adds them to its rows'
// running sums, in block order, while the others start the next round.  The next barrier
// falls after that fold, so a slot is written again only once it has been read.  Without DB
// there is one round (G <= W) and one slot.  Beside its pieces each wave parks a flag byte:
// whether an activation exponent of its tile allows a tiny piece (kNoTinyExp); a round
// without one is added with plain adds.
template <int FMT, int MODE, int SRC, int W, bool DB>
__global__ __launch_bounds__(64 * W) void gemv1_b32_kernel(const Targets tg, int G, ActIO io)
{
    constexpr int PPT = MODE == QG_PERBLOCK ? 8 : 1;      // pieces per tile row
    constexpr int SLOT = W * PPT * 64 + W * 64;           // words per slot: pieces, then tiny flags
    constexpr int BITS = ActKind<FMT, MODE>::kBits, GL = ActKind<FMT, MODE>::kLanes;
    extern __shared__ __align__(16) float s_ring[];
    using T = TileRegs<FMT>;
    using A = typename std::conditional<FMT == QG_Q4_0, ActPlanes, ActWaveCodes>::type;
    const Picked pm = pick_matrix(tg, (int)blockIdx.x);
    const int g = pm.g;
    const int rows = pm.rows;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool emit = blockIdx.x == 0;
    const uint8_t *gbase = pm.image + (size_t)g * G * T::kBytes;
    const int R = (G + W - 1) / W;                         // rounds; every wave goes through all

    float y = 0.0f;                                        // first wave: its row's running sum
    auto round = [&](const T &t, const ActWave &a, int r, int b) {
        float p[PPT];
        {
            const A act(a);
            __builtin_amdgcn_sched_barrier(0);
            b32_pieces<MODE>(t, act, p);
        }
        float *slot = s_ring + (DB ? (r & 1) * SLOT : 0);
        unsigned char *small = reinterpret_cast<unsigned char *>(slot + W * PPT * 64);
        const bool sm = __ballot(a.e < kNoTinyExp) != 0;   // a block of the tile may give a tiny piece
        if (b < G) {
#pragma unroll
            for (int j = 0; j < PPT; j++) slot[(wid * PPT + j) * 64 + lane] = p[j];
        }
        if (lane == 0) small[wid] = b < G && sm ? 1 : 0;
        __syncthreads();
        if (wid == 0) {
            const int nb = min(W, G - r * W);
            y = fold_flagged(y, slot + lane, nb * PPT, 64, any_flag<W>(small));
        }
    };

    // a block past the end (last round) is worked on as a copy of the last block and dropped
    int b = wid;
    ActRaw<SRC> r0 = load_act<SRC, GL>(io, min(b, G - 1), lane);
    __builtin_amdgcn_sched_barrier(0);
    T t0;
    [[maybe_unused]] T t1;
    t0.load(gbase + (size_t)min(b, G - 1) * T::kBytes, lane);
    load_fence();
    ActWave a0 = ready_act<SRC, BITS, GL>(r0, b, G, lane, emit, io);
    int r = 0;
    if constexpr (!DB) {
        round(t0, a0, 0, b);
    } else do {
        const int b1 = b + W;
        ActRaw<SRC> r1;
        if (r + 1 < R) {
            r1 = load_act<SRC, GL>(io, min(b1, G - 1), lane);
            __builtin_amdgcn_sched_barrier(0);
            t1.load(gbase + (size_t)min(b1, G - 1) * T::kBytes, lane);
            load_fence();
        }
        round(t0, a0, r, b);
        if (++r >= R) break;
        const ActWave a1 = ready_act<SRC, BITS, GL>(r1, b1, G, lane, emit, io);
        const int b2 = b1 + W;
        if (r + 1 < R) {
            r0 = load_act<SRC, GL>(io, min(b2, G - 1), lane);
            __builtin_amdgcn_sched_barrier(0);
            t0.load(gbase + (size_t)min(b2, G - 1) * T::kBytes, lane);
            load_fence();
        }
        round(t1, a1, r, b1);
        if (++r >= R) break;
        a0 = ready_act<SRC, BITS, GL>(r0, b2, G, lane, emit, io);
        b = b2;
    } while (true);

    if (wid == 0) {
        const int64_t row = (int64_t)g * 64 + lane;
        y = canon_nan(y);
        if (row < rows) pm.out[row] = y;
        if (io.argmax) {
            unsigned long long k = argmax_key(y, row, row < rows);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const unsigned long long o = __shfl_xor(k, off, 64);
                k = o > k ? o : k;
            }
            if (lane == 0 && k != 0ull) atomicMax(io.argmax, k);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Integer sums per (row, sub-block) for one activation row (debug view of the integer
// stage).  One wave per tile.

template <int FMT>
__global__ __launch_bounds__(256) void block_sums_kernel(const uint8_t *__restrict__ image, int rows, int G,
                                                         int64_t ntiles, const int8_t *__restrict__ codes,
                                                         int32_t *__restrict__ csum_out,
                                                         int32_t *__restrict__ osum_out)
{
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= ntiles) return;
    const int lane = threadIdx.x & 63;
    const int64_t g = t / G;
    const int b = (int)(t - g * G);
    const int64_t r = g * 64 + lane;
    const int8_t *a = codes + (size_t)b * 256;
    if constexpr (FMT == QG_Q4K) {
        TileRegs<QG_Q4K> T;
        T.load(image + t * kTileBytesQ4K, lane);
        if (r >= rows) return;
        uint32_t f[8];
        f[0] = q4k_field<0>(T.meta.y, T.meta.z, T.meta.w);
        f[1] = q4k_field<1>(T.meta.y, T.meta.z, T.meta.w);
        f[2] = q4k_field<2>(T.meta.y, T.meta.z, T.meta.w);
        f[3] = q4k_field<3>(T.meta.y, T.meta.z, T.meta.w);
        f[4] = q4k_field<4>(T.meta.y, T.meta.z, T.meta.w);
        f[5] = q4k_field<5>(T.meta.y, T.meta.z, T.meta.w);
        f[6] = q4k_field<6>(T.meta.y, T.meta.z, T.meta.w);
        f[7] = q4k_field<7>(T.meta.y, T.meta.z, T.meta.w);
        for (int i = 0; i < 8; i++) {
            int S = 0;
            for (int k = 0; k < 32; k++) S += a[32 * i + k];
            const uint4 a0 = *reinterpret_cast<const uint4 *>(a + 32 * i);
            const uint4 a1 = *reinterpret_cast<const uint4 *>(a + 32 * i + 16);
            csum_out[(r * G + b) * 8 + i] = (int)(f[i] & 63u) * q4k_sub_dot(T.w[i], a0, a1);
            osum_out[(r * G + b) * 8 + i] = (int)(f[i] >> 6) * S;
        }
    } else {
        TileRegs<QG_Q6K> T;
        T.load(image + t * kTileBytesQ6K, lane);
        if (r >= rows) return;
        const uint32_t sw[4] = {T.sc.x, T.sc.y, T.sc.z, T.sc.w};
        for (int i = 0; i < 8; i++) {
            int P0, P1;
            const uint4 a0 = *reinterpret_cast<const uint4 *>(a + 32 * i);
            const uint4 a1 = *reinterpret_cast<const uint4 *>(a + 32 * i + 16);
            if (i & 1) q6k_sub_dots<1>(T.L[i], T.H[i >> 1], a0, a1, P0, P1);
            else q6k_sub_dots<0>(T.L[i], T.H[i >> 1], a0, a1, P0, P1);
            int S0 = 0, S1 = 0;
            for (int k = 0; k < 16; k++) { S0 += a[32 * i + k]; S1 += a[32 * i + 16 + k]; }
            const int s0 = (int)(int8_t)(sw[(2 * i) >> 2] >> (8 * ((2 * i) & 3)));
            const int s1 = (int)(int8_t)(sw[(2 * i + 1) >> 2] >> (8 * ((2 * i + 1) & 3)));
            csum_out[(r * G + b) * 16 + 2 * i] = s0 * (P0 - 32 * S0);
            csum_out[(r * G + b) * 16 + 2 * i + 1] = s1 * (P1 - 32 * S1);
        }
    }
}

template <int FMT, int MODE, int SRC, int W, bool DB>
int launch_one_typed(const Targets &tg, int G, const ActIO &io, hipStream_t s)
{
    const int64_t groups = tg.gstart[tg.nmat];
    if (groups == 0) return QG_OK;
    if (!DB && G > W) return fail(QG_E_RUNTIME, "gemv: %d blocks do not fit %d waves", G, W);
    const size_t area = FMT == QG_Q4K && !DB ? (size_t)W * kActAreaWords * sizeof(uint32_t) : 0;
    const size_t lds = (size_t)(DB ? G : W) * 64 * sizeof(float) + 16 + area;
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemv1_kernel<FMT, MODE, SRC, W, DB>), dim3((unsigned)groups), dim3(64 * W), lds, s,
                              ev0, ev1, 0, tg, G, io);
    else
        hipLaunchKernelGGL((gemv1_kernel<FMT, MODE, SRC, W, DB>), dim3((unsigned)groups), dim3(64 * W), lds, s, tg, G,
                           io);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemv launch: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int FMT, int MODE, int SRC>
int launch_one(const Targets &tg, int G, const ActIO &io, hipStream_t s)
{
    // waves per workgroup: the tuning knob if set, else one wave per block up to 16; with
    // more blocks than 16 two tiles per wave (double-buffered), which takes 8-wave groups
    int w = tuning().waves_per_wg;
    if (w <= 0) w = G >= 16 ? 16 : G >= 8 ? 8 : 4;
    if (w > 8 && G > 16) w = 8;
    if (w >= 16) return launch_one_typed<FMT, MODE, SRC, 16, false>(tg, G, io, s);
    if (w >= 8) {
        if (G > 8) return launch_one_typed<FMT, MODE, SRC, 8, true>(tg, G, io, s);
        return launch_one_typed<FMT, MODE, SRC, 8, false>(tg, G, io, s);
    }
    if (G > 4) return launch_one_typed<FMT, MODE, SRC, 4, true>(tg, G, io, s);
    return launch_one_typed<FMT, MODE, SRC, 4, false>(tg, G, io, s);
}

template <int FMT, int MODE, int SRC, int W, bool DB>
int launch_b32_typed(const Targets &tg, int G, const ActIO &io, hipStream_t s)
{
    const int64_t groups = tg.gstart[tg.nmat];
    if (groups == 0) return QG_OK;
    if (!DB && G > W) return fail(QG_E_RUNTIME, "gemv: %d blocks do not fit one round of %d waves", G, W);
    const size_t lds = (DB ? 2 : 1) * (size_t)W * ((MODE == QG_PERBLOCK ? 8 : 1) + 1) * 64 * sizeof(float);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemv1_b32_kernel<FMT, MODE, SRC, W, DB>), dim3((unsigned)groups), dim3(64 * W), lds, s,
                              ev0, ev1, 0, tg, G, io);
    else
        hipLaunchKernelGGL((gemv1_b32_kernel<FMT, MODE, SRC, W, DB>), dim3((unsigned)groups), dim3(64 * W), lds, s,
                           tg, G, io);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemv launch: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int FMT, int MODE, int SRC>
int launch_b32(const Targets &tg, int G, const ActIO &io, hipStream_t s)
{
    // waves per workgroup: the tuning knob if set, else one wave per block up to 16; more
    // blocks than waves go in rounds of 8 (or 4) with the next round's tiles in flight
    int w = tuning().waves_per_wg;
    if (w <= 0) w = G <= 4 ? 4 : G <= 8 ? 8 : G <= 16 ? 16 : 8;
    if (w >= 16 && G <= 16) return launch_b32_typed<FMT, MODE, SRC, 16, false>(tg, G, io, s);
    if (w >= 8) {
        if (G <= 8) return launch_b32_typed<FMT, MODE, SRC, 8, false>(tg, G, io, s);
        return launch_b32_typed<FMT, MODE, SRC, 8, true>(tg, G, io, s);
    }
    if (G <= 4) return launch_b32_typed<FMT, MODE, SRC, 4, false>(tg, G, io, s);
    return launch_b32_typed<FMT, MODE, SRC, 4, true>(tg, G, io, s);
}

template <int SRC>
int launch_quarter(const Targets &tg, int G, const ActIO &io, hipStream_t s)
{
    const int64_t wgs = 4 * (int64_t)tg.gstart[tg.nmat];
    if (wgs == 0) return QG_OK;
    if (G > 16) return fail(QG_E_RUNTIME, "gemv: %d blocks do not fit 16 waves", G);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemv1_quarter_kernel<SRC>), dim3((unsigned)wgs), dim3(1024), 0, s, ev0, ev1, 0, tg, G,
                              io);
    else
        hipLaunchKernelGGL((gemv1_quarter_kernel<SRC>), dim3((unsigned)wgs), dim3(1024), 0, s, tg, G, io);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemv launch: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int SRC>
int launch_one_any(int fmt, int mode, const Targets &tg, int G, const ActIO &io, hipStream_t s)
{
    if (fmt == QG_Q4K && mode == QG_PERBLOCK && G <= 16 && !io.argmax && tuning().waves_per_wg == 0) {
        // 16-row workgroups where 64-row ones leave compute units idle
        const int q = tuning().gemv_quarter;
        if (q == 1 || (q == 0 && tg.gstart[tg.nmat] < 128)) return launch_quarter<SRC>(tg, G, io, s);
    }
    if (fmt == QG_Q8_0 && mode == QG_PERBLOCK) return launch_b32<QG_Q8_0, QG_PERBLOCK, SRC>(tg, G, io, s);
    if (fmt == QG_Q8_0 && mode == QG_SUB32) return launch_b32<QG_Q8_0, QG_SUB32, SRC>(tg, G, io, s);
    if (fmt == QG_Q4_0 && mode == QG_PERBLOCK) return launch_b32<QG_Q4_0, QG_PERBLOCK, SRC>(tg, G, io, s);
    if (fmt == QG_Q4_0 && mode == QG_SUB32) return launch_b32<QG_Q4_0, QG_SUB32, SRC>(tg, G, io, s);
    if (fmt == QG_Q4K && mode == QG_PERBLOCK) return launch_one<QG_Q4K, QG_PERBLOCK, SRC>(tg, G, io, s);
    if (fmt == QG_Q4K && mode == QG_SUB32) return launch_one<QG_Q4K, QG_SUB32, SRC>(tg, G, io, s);
    if (fmt == QG_Q6K && mode == QG_PERBLOCK) return launch_one<QG_Q6K, QG_PERBLOCK, SRC>(tg, G, io, s);
    return launch_one<QG_Q6K, QG_SUB32, SRC>(tg, G, io, s);
}

// the descriptor of nmat matrices (rows[m] rows each); QG_E_SHAPE if the row groups overflow
int make_targets(int nmat, const int64_t *rows, const void *const *images, float *const *outs, Targets &tg)
{
    tg.nmat = nmat;
    int64_t groups = 0;
    for (int m = 0; m < nmat; m++) {
        tg.gstart[m] = (int)groups;
        tg.rows[m] = (int)rows[m];
        tg.image[m] = static_cast<const uint8_t *>(images[m]);
        tg.out[m] = outs[m];
        groups += (rows[m] + 63) / 64;
        if (groups > 0x7fffffff) return fail(QG_E_SHAPE, "too many row groups in one launch");
    }
    for (int m = nmat; m <= QG_MAX_MATRICES; m++) tg.gstart[m] = (int)groups;
    for (int m = nmat; m < QG_MAX_MATRICES; m++) {
        tg.rows[m] = 0;
        tg.image[m] = nullptr;
        tg.out[m] = nullptr;
    }
    return QG_OK;
}

// LDS bytes the kernel needs for NC columns
template <int FMT, int MODE>
size_t gemv_lds(int G, int nc)
{
    const size_t pieces = (size_t)nc * G * 64 * 4;
    return nc > 1 ? (size_t)nc * G * ActRec<FMT, MODE>::kStride + pieces : pieces;
}

template <int FMT, int MODE, int NC, int W, bool DB>
int launch_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                 const qg_act_scale *scales, const int32_t *csums, float *out, hipStream_t s)
{
    const int64_t groups = (rows + 63) / 64;
    if (groups > 0x7fffffff) return fail(QG_E_SHAPE, "too many rows: %lld", (long long)rows);
    const size_t lds = gemv_lds<FMT, MODE>(G, NC);
    const dim3 grid((unsigned)groups, (unsigned)((ncol + NC - 1) / NC));
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemv_kernel<FMT, MODE, NC, W, DB>), grid, dim3(64 * W), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, codes, scales, csums, (int)ncol, out);
    else
        hipLaunchKernelGGL((gemv_kernel<FMT, MODE, NC, W, DB>), grid, dim3(64 * W), lds, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, codes, scales, csums, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemv launch: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int FMT, int MODE, int NC, int W>
int launch_db(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
              const qg_act_scale *scales, const int32_t *csums, float *out, hipStream_t s)
{
    if (G > W) return launch_typed<FMT, MODE, NC, W, true>(rows, G, ncol, image, codes, scales, csums, out, s);
    return launch_typed<FMT, MODE, NC, W, false>(rows, G, ncol, image, codes, scales, csums, out, s);
}

template <int FMT, int MODE, int NC>
int launch_w(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
             const qg_act_scale *scales, const int32_t *csums, float *out, hipStream_t s)
{
    // waves per workgroup: the tuning knob if set (16 is taken as 8: several columns'
    // registers do not fit 16 waves), else 8
    int w = tuning().waves_per_wg;
    if (w <= 0 || w > 8) w = 8;
    if (w >= 8) return launch_db<FMT, MODE, NC, 8>(rows, G, ncol, image, codes, scales, csums, out, s);
    return launch_db<FMT, MODE, NC, 4>(rows, G, ncol, image, codes, scales, csums, out, s);
}

template <int FMT, int MODE>
int launch_nc(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
              const qg_act_scale *scales, const int32_t *csums, float *out, hipStream_t s)
{
    // widest column batch whose LDS fits 64 KiB
    auto fits = [&](int nc) { return gemv_lds<FMT, MODE>(G, nc) <= 65536; };
    if (ncol >= 8 && fits(8)) return launch_w<FMT, MODE, 8>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (ncol >= 4 && fits(4)) return launch_w<FMT, MODE, 4>(rows, G, ncol, image, codes, scales, csums, out, s);
    if (fits(2)) return launch_w<FMT, MODE, 2>(rows, G, ncol, image, codes, scales, csums, out, s);
    // rows too wide for two columns' records: one launch per column
    const int64_t C = (int64_t)G * 256, nsc = MODE == QG_PERBLOCK ? G : (int64_t)G * 8;
    for (int64_t c = 0; c < ncol; c++) {
        const ActIO io{nullptr, codes + c * C, reinterpret_cast<const uint32_t *>(scales + c * nsc), nullptr, nullptr,
                       nullptr, nullptr, nullptr};
        Targets tg;
        float *oc = out + c * rows;
        int st = make_targets(1, &rows, &image, &oc, tg);
        if (st == QG_OK) st = launch_one<FMT, MODE, SRC_CODES>(tg, G, io, s);
        if (st != QG_OK) return st;
    }
    return QG_OK;
}

}  // namespace

int launch_gemv_fused(int fmt, int mode, int64_t rows, int64_t cols, const void *image, const float *x,
                      int8_t *codes, qg_act_scale *scales, int32_t *csums, int32_t *err_flag, float *out,
                      unsigned long long *argmax, hipStream_t s)
{
    if (rows == 0) return QG_OK;
    const ActIO io{x, nullptr, nullptr, codes, scales, csums, err_flag, argmax};
    Targets tg;
    const int st = make_targets(1, &rows, &image, &out, tg);
    if (st != QG_OK) return st;
    return launch_one_any<SRC_F32>(fmt, mode, tg, (int)(cols / 256), io, s);
}

int launch_gemv_multi(int fmt, int mode, int nmat, const int64_t *rows, int64_t cols, const void *const *images,
                      const float *x, const int8_t *codes_in, const qg_act_scale *scales_in, int8_t *codes_out,
                      qg_act_scale *scales_out, int32_t *csums_out, int32_t *err_flag, float *const *outs,
                      hipStream_t s)
{
    Targets tg;
    const int st = make_targets(nmat, rows, images, outs, tg);
    if (st != QG_OK) return st;
    const int G = (int)(cols / 256);
    if (x) {
        const ActIO io{x, nullptr, nullptr, codes_out, scales_out, csums_out, err_flag, nullptr};
        return launch_one_any<SRC_F32>(fmt, mode, tg, G, io, s);
    }
    const ActIO io{nullptr, codes_in, reinterpret_cast<const uint32_t *>(scales_in), nullptr, nullptr, nullptr, nullptr,
                   nullptr};
    return launch_one_any<SRC_CODES>(fmt, mode, tg, G, io, s);
}

template <int FMT, int MODE, int NC>
int launch_cols_typed(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                      const qg_act_scale *scales, float *out, hipStream_t s)
{
    const int64_t groups = (rows + 63) / 64;
    const int64_t batches = (ncol + NC - 1) / NC;
    const int64_t nsc = act_block(FMT, MODE) == 256 ? G : (int64_t)G * 8;
    const ActCols ac{codes, reinterpret_cast<const uint32_t *>(scales), (int64_t)G * 256, nsc};
    const size_t lds = (size_t)NC * 16 * 64 * sizeof(float) + 16;
    const dim3 grid((unsigned)groups, (unsigned)batches);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((gemv1_cols_kernel<FMT, MODE, NC>), grid, dim3(1024), lds, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(image), (int)rows, G, ac, (int)ncol, out);
    else
        hipLaunchKernelGGL((gemv1_cols_kernel<FMT, MODE, NC>), grid, dim3(1024), lds, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, ac, (int)ncol, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "gemv launch: %s", hipGetErrorString(e));
    return QG_OK;
}

template <int FMT, int MODE>
int launch_cols(int64_t rows, int G, int64_t ncol, const void *image, const int8_t *codes,
                const qg_act_scale *scales, float *out, hipStream_t s)
{
    if (ncol <= 2) return launch_cols_typed<FMT, MODE, 2>(rows, G, ncol, image, codes, scales, out, s);
    if (ncol <= 4) return launch_cols_typed<FMT, MODE, 4>(rows, G, ncol, image, codes, scales, out, s);
    return launch_cols_typed<FMT, MODE, 8>(rows, G, ncol, image, codes, scales, out, s);
}

int launch_gemv(int fmt, int mode, int64_t rows, int64_t cols, int64_t ncol, const void *image,
                const int8_t *codes, const qg_act_scale *scales, const int32_t *csums, float *out,
                hipStream_t s)
{
    if (rows == 0 || ncol == 0) return QG_OK;
    const int G = (int)(cols / 256);
    if (ncol > 1 && !is_b32(fmt) && G <= 16 && tuning().cols_off == 0) {
        // several columns, at most 16 blocks per row: the one-column machinery, NC columns a wave
        if (fmt == QG_Q4K && mode == QG_PERBLOCK)
            return launch_cols<QG_Q4K, QG_PERBLOCK>(rows, G, ncol, image, codes, scales, out, s);
        if (fmt == QG_Q4K && mode == QG_SUB32)
            return launch_cols<QG_Q4K, QG_SUB32>(rows, G, ncol, image, codes, scales, out, s);
        if (fmt == QG_Q6K && mode == QG_PERBLOCK)
            return launch_cols<QG_Q6K, QG_PERBLOCK>(rows, G, ncol, image, codes, scales, out, s);
        return launch_cols<QG_Q6K, QG_SUB32>(rows, G, ncol, image, codes, scales, out, s);
    }
    if (ncol == 1 || is_b32(fmt)) {
        // one launch per column (the 32-element-block formats have no several-column kernel)
        const int64_t nsc = act_block(fmt, mode) == 256 ? G : (int64_t)G * 8;
        for (int64_t c = 0; c < ncol; c++) {
            const ActIO io{nullptr, codes + c * cols, reinterpret_cast<const uint32_t *>(scales + c * nsc), nullptr,
                           nullptr, nullptr, nullptr, nullptr};
            Targets tg;
            float *oc = out + c * rows;
            int st = make_targets(1, &rows, &image, &oc, tg);
            if (st == QG_OK) st = launch_one_any<SRC_CODES>(fmt, mode, tg, G, io, s);
            if (st != QG_OK) return st;
        }
        return QG_OK;
    }
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
    const int64_t ntiles = (rows + 63) / 64 * G;
    if (ntiles == 0) return QG_OK;
    const int64_t wgs = (ntiles + 3) / 4;
    if (fmt == QG_Q4K)
        hipLaunchKernelGGL(block_sums_kernel<QG_Q4K>, dim3((unsigned)wgs), dim3(256), 0, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, ntiles, codes, csum_out, osum_out);
    else
        hipLaunchKernelGGL(block_sums_kernel<QG_Q6K>, dim3((unsigned)wgs), dim3(256), 0, s,
                           static_cast<const uint8_t *>(image), (int)rows, G, ntiles, codes, csum_out, osum_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "block_sums launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace qg
