// qg_device.hpp -- device-side exact arithmetic of the block combine and the row sum.
//
// Everything here is exact integer or exact f64 work followed by one binary32 rounding,
// as the method prescribes (rustdoc "Module numerics" of
// logicaffeine_compile::spatial::decode_engine: module description, the two ActScaling
// modes and the f32 model; Functions exact_sum, scaled_to_f32, ftz, fadd; "Module lane":
// module description and Functions lane, group).
//
// The code is compiled with -ffp-contract=off and IEEE f32/f64 denormal handling (the
// kernel descriptor's default), so every f64 operation below rounds exactly once, to
// nearest even, and binary32 conversions round on the gradual-underflow grid before the
// explicit flush.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

constexpr int kSumWindow = 64;   // places an exact sum keeps below its largest term's exponent

// ---------------------------------------------------------------------------------------
// binary16 block scale -> signed integer significand and exponent (value sig * 2^ex).
// The packer refuses inf/NaN scales, so the exponent field is 0..30 here.
struct F16Scale {
    int sig;
    int ex;
};

__device__ __forceinline__ F16Scale f16_scale(uint32_t h)
{
    const int E = (h >> 10) & 31;
    const int M = h & 1023;
    F16Scale s;
    s.sig = E ? (M | 1024) : M;
    s.ex = E ? E - 25 : -24;
    if (h & 0x8000u) s.sig = -s.sig;
    return s;
}

// ---------------------------------------------------------------------------------------
// binary32 helpers

__device__ __forceinline__ float ftz(float x)
{
    uint32_t u = __float_as_uint(x);
    return (u & 0x7F800000u) ? x : __uint_as_float(u & 0x80000000u);
}

// in-order row accumulation: binary32 add (nearest even), result flushed
__device__ __forceinline__ float fadd_ftz(float acc, float piece) { return ftz(acc + piece); }

// acc plus n pieces p[0], p[stride], ... in that order, each add flushed as fadd_ftz.  The
// pieces and the running sum are zero or normal, and such a sum lands in the subnormal range
// only when it is exact, so plain adds give the same partial sums unless one of them is
// subnormal.  The pieces are read in batches of eight, the next batch's reads issued before
// this batch's adds, so the dependent chain is one add per piece.  CHECK keeps the least
// binary exponent of the partial sums beside the chain (frexp: a subnormal has exponent
// <= -126, a zero 0) so that a lane where one was subnormal can run again with the flush.
__device__ __forceinline__ void fold_read8(float (&a)[8], const float *p, int k, int stride)
{
#pragma unroll
    for (int j = 0; j < 8; j++) a[j] = p[(size_t)(k + j) * stride];
}

template <bool CHECK>
__device__ __forceinline__ void fold_add8(float &y, int &lo, const float (&a)[8])
{
#pragma unroll
    for (int j = 0; j < 8; j++) {
        y = y + a[j];
        if constexpr (CHECK) lo = min(lo, __builtin_amdgcn_frexp_expf(y));
    }
}

template <bool CHECK>
__device__ __forceinline__ float fold_chain(float y, int &lo, const float *p, int n, int stride)
{
    const int n8 = n & ~7;
    int k = 0;
    if (n8 > 0) {
        // batches k (in a) and k + 8 (in b) alternate
        float a[8], b[8];
        fold_read8(a, p, 0, stride);
        do {
            const bool b_next = k + 8 < n8;
            if (b_next) fold_read8(b, p, k + 8, stride);
            fold_add8<CHECK>(y, lo, a);
            k += 8;
            if (!b_next) break;
            const bool a_next = k + 8 < n8;
            if (a_next) fold_read8(a, p, k + 8, stride);
            fold_add8<CHECK>(y, lo, b);
            k += 8;
            if (!a_next) break;
        } while (true);
    }
    for (; k < n; k++) {
        y = y + p[(size_t)k * stride];
        if constexpr (CHECK) lo = min(lo, __builtin_amdgcn_frexp_expf(y));
    }
    return y;
}

// acc plus the pieces with plain adds, for a row none of whose pieces is tiny
__device__ __forceinline__ float fold_chain_plain(float acc, const float *p, int n, int stride)
{
    int lo = 0;
    return fold_chain<false>(acc, lo, p, n, stride);
}

__device__ __forceinline__ float fold_flushed(float y, const float *p, int n, int stride)
{
    for (int i = 0; i < n; i++) y = fadd_ftz(y, p[(size_t)i * stride]);
    return y;
}

__device__ __forceinline__ float fold_ftz(float acc, const float *p, int n, int stride)
{
    int lo = 0;
    const float y = fold_chain<true>(acc, lo, p, n, stride);
    return lo <= -126 ? fold_flushed(acc, p, n, stride) : y;
}

// A piece is R32 of an exact value X that is an integer multiple of 2^(e + eps): e an
// activation scale exponent of its block and eps >= -24 the exponent of the least place of a
// binary16 block scale.  With every such e >= -78 a nonzero X is at least 2^-102, and so is
// its rounding: no piece of the block is tiny (tiny_piece), whatever the weights.
constexpr int kNoTinyExp = -78;

// Whether a piece may let a partial sum of the row become subnormal: nonzero and below 2^-102
// in magnitude.  A nonzero piece of at least 2^-102 has an ulp of at least 2^-125; when every
// nonzero piece of a row is one, every partial sum is a multiple of the least such ulp (an add
// rounds to a grid at least that coarse or is exact), so a nonzero partial sum is at least
// 2^-125 and the row's adds need no flush at all.
__device__ __forceinline__ bool tiny_piece(float p)
{
    const uint32_t u = __float_as_uint(p) & 0x7FFFFFFFu;
    return u - 1u < 0x0C7FFFFFu;
}

// acc plus the pieces as fold_ftz, for a row whose producers have flagged whether any of its
// pieces is tiny (tiny_piece): plain adds unless one is.
__device__ __forceinline__ float fold_flagged(float acc, const float *p, int n, int stride, bool tiny)
{
    if (tiny) return fold_flushed(acc, p, n, stride);
    int lo = 0;
    return fold_chain<false>(acc, lo, p, n, stride);
}

__device__ __forceinline__ float canon_nan(float y)
{
    return (y != y) ? __uint_as_float(0x7FC00000u) : y;
}

// ---------------------------------------------------------------------------------------
// One binary32 rounding of a value held exactly in one double (|significand| <= 53 bits).
// An exact zero is +0 whatever the signs of the factors that made it.
__device__ __forceinline__ float r32_exact_double(double x) { return x == 0.0 ? 0.0f : ftz((float)x); }

// One binary32 rounding of a + b for doubles a, b (each exact).  TwoSum gives the rounded
// sum s and its exact error t; nudging s to the odd neighbour when t != 0 (round to odd at
// 53 bits) makes the later rounding to <= 24 bits equal the rounding of a + b itself.
__device__ __forceinline__ float r32_sum2(double a, double b)
{
    double s = a + b;
    double bv = s - a;
    double av = s - bv;
    double t = (a - av) + (b - bv);
    if (s == 0.0) return 0.0f;              // exact cancellation (or two zeros): +0
    if (t != 0.0) {
        unsigned long long u = (unsigned long long)__double_as_longlong(s);
        if ((u & 1ull) == 0ull) {
            const bool away = (t > 0.0) == (s > 0.0);
            u = away ? u + 1ull : u - 1ull;
            s = __longlong_as_double((long long)u);
        }
    }
    return ftz((float)s);
}

// ---------------------------------------------------------------------------------------
// 128-bit exact sums (Sub32 groups)

typedef __int128 i128;
typedef unsigned __int128 u128;

__device__ __forceinline__ int bitlen64(uint64_t v) { return v ? 64 - __clzll((long long)v) : 0; }

// v * 2^exp rounded once to binary32: nearest even on the gradual-underflow grid, past the
// top infinite, then a subnormal result flushed to a zero of its sign; 0 -> +0.
__device__ inline float r32_i128(i128 v, int exp)
{
    if (v == 0) return 0.0f;
    const uint32_t sign = v < 0 ? 0x80000000u : 0u;
    const u128 M = v < 0 ? (u128)0 - (u128)v : (u128)v;
    const uint64_t hi = (uint64_t)(M >> 64), lo = (uint64_t)M;
    const int n = hi ? 64 + bitlen64(hi) : bitlen64(lo);
    int q = exp + n - 24;                   // exponent of the last kept place
    if (q < -149) q = -149;
    const int shift = q - exp;
    uint64_t R;
    if (shift <= 0) {
        R = (uint64_t)(M << (-shift));      // fewer than 24 significant bits: exact
    } else if (shift >= 127) {
        R = 0;
    } else {
        R = (uint64_t)(M >> shift);
        const u128 rem = M & (((u128)1 << shift) - 1);
        const u128 half = (u128)1 << (shift - 1);
        if (rem > half || (rem == half && (R & 1ull))) R += 1;
    }
    if (R == (1ull << 24)) { R >>= 1; q += 1; }
    if (R < (1ull << 23)) return __uint_as_float(sign);          // subnormal or zero: flushed
    const int biased = q + 150;
    if (biased > 254) return __uint_as_float(sign | 0x7F800000u);
    return __uint_as_float(sign | ((uint32_t)biased << 23) | (uint32_t)(R & 0x7FFFFFull));
}

// |a| * 2^ea > |b| * 2^eb ?
__device__ inline bool mag_greater(long long a, int ea, long long b, int eb)
{
    uint64_t A = a < 0 ? 0ull - (uint64_t)a : (uint64_t)a;
    uint64_t B = b < 0 ? 0ull - (uint64_t)b : (uint64_t)b;
    if (A == 0) return false;
    if (B == 0) return true;
    const int ta = ea + bitlen64(A), tb = eb + bitlen64(B);
    if (ta != tb) return ta > tb;
    if (ea > eb) A <<= (ea - eb); else B <<= (eb - ea);   // same leading place: no overflow
    return A > B;
}

// Sum of v[i] * 2^e[i] rounded once ("Module numerics", Functions exact_sum).  Terms are
// below 2^45 in magnitude here.  When every exponent is within kSumWindow of every other,
// no term can lie past the window and the aligned sum fits 128 bits.  Otherwise the
// largest-magnitude term (first of equals) fixes L, and a term whose exponent is below
// L - kSumWindow is floored to a multiple of 2^(L - kSumWindow) first.  Every index is a
// compile-time constant, so the terms stay in registers.
template <int N>
__device__ __forceinline__ float exact_sum(const long long (&v)[N], const int (&e)[N])
{
    int emin = e[0], emax = e[0];
#pragma unroll
    for (int i = 1; i < N; i++) {
        emin = e[i] < emin ? e[i] : emin;
        emax = e[i] > emax ? e[i] : emax;
    }
    if (emax - emin <= kSumWindow) {
        u128 s = 0;
#pragma unroll
        for (int i = 0; i < N; i++) s += (u128)(i128)v[i] << (e[i] - emin);
        return r32_i128((i128)s, emin);
    }
    // the window is engaged: rare, never at the shipped workloads
    long long vL = v[0];
    int eL = e[0];
#pragma unroll
    for (int i = 1; i < N; i++)
        if (mag_greater(v[i], e[i], vL, eL)) { vL = v[i]; eL = e[i]; }
    const int fe = eL - kSumWindow;
    int emin2 = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const int ei = e[i] < fe ? fe : e[i];
        emin2 = ei < emin2 ? ei : emin2;
    }
    u128 s = 0;
#pragma unroll
    for (int i = 0; i < N; i++) {
        long long vi = v[i];
        int ei = e[i];
        if (ei < fe) {
            const int sh = fe - ei;
            vi = sh >= 63 ? (vi < 0 ? -1 : 0) : (vi >> sh);   // arithmetic shift = floor
            ei = fe;
        }
        if (vi != 0) s += (u128)(i128)vi << (ei - emin2);
    }
    return r32_i128((i128)s, emin2);
}

// ---------------------------------------------------------------------------------------
// Activation quantization of 256 consecutive elements by one wave, four per lane (lane l
// holds elements 4l..4l+3) ("Module numerics": Functions absmax, wide_scale, block_scale,
// rne_div, quantize, quantize_blocks).  A block of 256 elements spans the wave, one of 32
// spans eight lanes: BITS significant bits (8 PerBlock, 4 Sub32) over GL lanes (64 or 8).
//
// The scale: exact integer arithmetic on amax's significand (least_scale).
//
// The codes: q = x/s has |q| <= 127.5, and a q that is not a half-integer lies more than
// 2^-26 from every half-integer (x = X*2^k with |X| < 2^24, s = m*2^e: near a half-integer
// the gap is a nonzero multiple of 1/(2m*2^(e-k)) with 2m*2^(e-k) < 4|X|).  In binary32,
// t = (x*2^-e) * rcp(m) is within 2^-15 of q (x*2^-e exact or below 2^-100; v_rcp_f32 within
// one ulp, 2^-23 relative, and one rounding of 2^-24), so rint(t) is q rounded to nearest
// unless t lies within 2^-13 of a half-integer.  Such elements (a few per ten thousand) are
// coded from the correctly rounded f64 quotient instead: an f64 quotient that is not a
// half-integer cannot round onto one, so its ties are exactly the true ties and go to even.

// least m*2^e (m with BITS significant bits) not below amax/127, amax a normal binary32 > 0
// (finite).  With amax = A*2^(E-150), A the 24-bit significand: scales m*2^(E-150+j) with
// 127*m*2^j >= A.  At j = J0 every admissible grid point lies above every grid point of a
// lower exponent (127*(2^BITS - 1)*2^(J0-1) < 2^23 <= A), so m = ceil(A / (127*2^J0)) is
// the least one when it has BITS bits; otherwise no grid point of exponent J0 is admissible
// and m = ceil(A / (127*2^(J0+1))) (at least 2^(BITS-1)) at J0 + 1 is.  Integer arithmetic
// only (uniform operands stay scalar).
template <int BITS>
__device__ __forceinline__ void least_scale(float amax, int &m, int &e)
{
    constexpr int J0 = BITS == 1 ? 17 : 17 - BITS;
    constexpr uint32_t D0 = 127u << J0, D1 = 127u << (J0 + 1);
    const uint32_t u = __float_as_uint(amax);
    const uint32_t A = (u & 0x7FFFFFu) | 0x800000u;
    const int E = (int)(u >> 23);
    uint32_t mm = (A + D0 - 1) / D0;
    int j = J0;
    if (mm >= (1u << BITS)) { mm = (A + D1 - 1) / D1; j = J0 + 1; }
    m = (int)mm;
    e = E - 150 + j;
}

// Lane exchanges within rows of 16 lanes through DPP (every source lane is valid)
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowMirror = 0x140;    // lane i of a row <- lane 15 - i
constexpr int kDppHalfMirror = 0x141;   // lane i of a half-row <- lane 7 - i
constexpr int kDppRowShl4 = 0x104;      // lane i of a row <- lane i + 4 (none for i >= 12: 0)

template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// sum over each group of 4 lanes (4l..4l+3), in every lane of the group
__device__ __forceinline__ int quad_sum(int v)
{
    v += dpp<kDppQuadSwap1>(v);
    return v + dpp<kDppQuadSwap2>(v);
}

// given quad sums, the sum over each group of 8 lanes
__device__ __forceinline__ int octet_sum_of_quads(int v) { return v + dpp<kDppHalfMirror>(v); }

struct QuantLane {
    uint32_t packed;   // the lane's four int8 codes, element 4l in the low byte
    int sum4;          // their sum
    int m, e;          // scale m*2^e of the lane's activation block (m = 0: block holds an inf)
    int inf;           // the lane's activation block holds an infinity
};

// significand bits and lanes per activation block of a (format, scaling)
template <int FMT, int MODE>
struct ActKind {
    static constexpr int kBits = MODE == QG_PERBLOCK ? 8 : 4;
    static constexpr int kLanes = (MODE == QG_SUB32 || FMT == QG_Q8_0 || FMT == QG_Q4_0) ? 8 : 64;
};

template <int BITS, int GL>
__device__ __forceinline__ QuantLane quantize_lane(float4 v4)
{
    static_assert(GL == 8 || GL == 16 || GL == 32 || GL == 64, "activation blocks of 32 to 256 elements");
    // a denormal reads as 0 and so does a NaN (passed over by absmax, code 0): one class test
    // (quiet and signalling NaN, negative and positive denormal)
    const float raw[4] = {v4.x, v4.y, v4.z, v4.w};
    float v[4];
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[i] = __builtin_amdgcn_classf(raw[i], 0x93) ? 0.0f : raw[i];
        const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;   // non-negative floats order as integers
        amax_bits = a > amax_bits ? a : amax_bits;
    }
    auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    amax_bits = umax(amax_bits, (uint32_t)dpp<kDppQuadSwap1>((int)amax_bits));
    amax_bits = umax(amax_bits, (uint32_t)dpp<kDppQuadSwap2>((int)amax_bits));
    amax_bits = umax(amax_bits, (uint32_t)dpp<kDppHalfMirror>((int)amax_bits));   // 8 lanes: 32 elements
    if constexpr (GL >= 16)
        amax_bits = umax(amax_bits, (uint32_t)dpp<kDppRowMirror>((int)amax_bits));  // 16 lanes: 64 elements
    if constexpr (GL >= 32) {
        const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)amax_bits, 0);
        const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)amax_bits, 16);
        const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)amax_bits, 32);
        const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)amax_bits, 48);
        if constexpr (GL == 64)
            amax_bits = umax(umax(r0, r1), umax(r2, r3));                          // the wave
        else
            amax_bits = (threadIdx.x & 32) ? umax(r2, r3) : umax(r0, r1);          // half waves
    }
    QuantLane q;
    q.inf = amax_bits == 0x7F800000u;
    if (q.inf) {
        q.m = 0; q.e = 0;
    } else if (amax_bits == 0) {
        q.m = 1 << (BITS - 1); q.e = 0;                   // all-zero block
    } else {
        least_scale<BITS>(__uint_as_float(amax_bits), q.m, q.e);
    }
    q.packed = 0;
    q.sum4 = 0;
    if (q.m != 0) {
        // t = (x * 2^-e) * rcp(m); v_rcp_f32 is within one ulp of 1/m (see the comment above)
        const float rm = __builtin_amdgcn_rcpf((float)q.m);
        float t[4], r[4];
        bool near = false;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            t[i] = __builtin_ldexpf(v[i], -q.e) * rm;
            r[i] = __builtin_rintf(t[i]);
            // t - r is exact (|t - r| <= 1/2 and r is 0 or within a factor 2 of t)
            near |= __builtin_fabsf(__builtin_fabsf(t[i] - r[i]) - 0.5f) < 0x1p-13f;
        }
        int c[4];
#pragma unroll
        for (int i = 0; i < 4; i++) c[i] = (int)r[i];
        if (near) {
            const double s = __builtin_ldexp((double)q.m, q.e);
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (__builtin_fabsf(__builtin_fabsf(t[i] - r[i]) - 0.5f) < 0x1p-13f)
                    c[i] = (int)__builtin_rint((double)v[i] / s);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            q.sum4 += c[i];
            q.packed |= ((uint32_t)c[i] & 0xFFu) << (8 * i);
        }
    }
    return q;
}

// ---------------------------------------------------------------------------------------
// Block pieces

// PerBlock, Q4_K-style: R32(m*2^e * (d*C - dmin*O)).  With sig_d*m < 2^19 and |C| < 2^25 each
// product is below 2^44 and exact in f64; ldexp by the combined exponent is exact too.
__device__ __forceinline__ float piece_q4k_perblock(int C, int O, uint32_t d_dmin, int m, int e)
{
    const F16Scale d = f16_scale(d_dmin & 0xFFFFu);
    const F16Scale dm = f16_scale(d_dmin >> 16);
    const double a = __builtin_ldexp((double)C * (double)(d.sig * m), d.ex + e);
    const double b = __builtin_ldexp(-(double)O * (double)(dm.sig * m), dm.ex + e);
    return r32_sum2(a, b);
}

// binary16 bits -> the value as a binary32 (exact: every binary16 is one)
__device__ __forceinline__ float f16_value(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// PerBlock, Q4_K-style, when X = C*Dd - O*Dm fits 45 significant bits: one fma forms it
// exactly, times S = m*2^e (8 significant bits) it stays exact in f64, and the conversion
// is the one rounding.  Gives the same bits as piece_q4k_perblock.
__device__ __forceinline__ float piece_q4k_perblock_near(int C, int O, double Dd, double Dm, double S)
{
    const double X = __builtin_fma((double)C, Dd, -((double)O * Dm));
    return r32_exact_double(X * S);
}

// Whether piece_q4k_perblock_near applies, from the binary exponents of the two block scales
// (frexp: value = f * 2^k, f in [0.5, 1)).  A binary16 value with exponent k has its last
// significant place at 2^(k-11) or above; |C| < 2^25 and |O| < 2^21 (8 sub-blocks of 32
// codes of at most 127 times 6-bit sub-scales and 4-bit codes, or times 6-bit offsets).  So
// X spans at most 37 + (kd - km) places when kd >= km and at most max(37, 33 + km - kd)
// otherwise: 45 or fewer when -12 <= kd - km <= 8.  A zero scale (k = 0) may fail the test;
// the general combine is exact for every input.
__device__ __forceinline__ bool q4k_near(float fd, float fm)
{
    const int gap = __builtin_amdgcn_frexp_expf(fd) - __builtin_amdgcn_frexp_expf(fm);
    return gap >= -12 && gap <= 8;
}

// PerBlock, Q6_K-style: one term R32(m*2^e * d*C); |C| < 2^27 so the product is < 2^46.
__device__ __forceinline__ float piece_q6k_perblock(int C, uint32_t dbits, int m, int e)
{
    const F16Scale d = f16_scale(dbits);
    const double X = __builtin_ldexp((double)C * (double)(d.sig * m), d.ex + e);
    // e >= kNoTinyExp: X is 0 or at least 2^-102, so the conversion needs no flush, and adding
    // +0 turns an exact -0 into +0
    if (e >= kNoTinyExp) return (float)X + 0.0f;
    return r32_exact_double(X);
}

// The exact sum of eight doubles T[j] (each exact, every one a multiple of 2^low) rounded once
// to binary32, as hi + lo: hi the rounded running sum, lo the sum of TwoSum's exact errors.
// Each error is a multiple of 2^low below 2^(top - 53), top bounding every partial sum
// (2^top > 8 * max |T|), so lo is exact while top - low <= 103, and then hi + lo is the sum and
// r32_sum2 rounds it once.  Returns false (out untouched) when the bound does not hold.
__device__ __forceinline__ bool sum8_pair(const double (&T)[8], int low, float &out)
{
    double hi = 0.0, lo = 0.0, amax = 0.0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const double a = hi, b = T[j];
        hi = a + b;
        const double bv = hi - a;
        lo += (a - (hi - bv)) + (b - bv);
        amax = __builtin_fmax(amax, __builtin_fabs(b));
    }
    int k;
    (void)__builtin_frexp(amax, &k);                // amax < 2^k
    if (amax != 0.0 && k + 3 - low > 103) return false;
    out = r32_sum2(hi, lo);
    return true;
}

// R32 of y = 2^emin * V when y is V's binary64 rounding scaled by a power of two (no underflow):
// the two roundings give V's own binary32 rounding unless y lies on a binary32 rounding boundary
// (bit 28 of the binary64 significand set, bits 0..27 clear: the midpoint of two binary32
// neighbours) or below the least binary32 normal.  True, with out set, when neither holds or
// y is zero (+0 then, whatever the sign).
__device__ __forceinline__ bool r32_of_rounded(double y, float &out)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, y);
    const uint32_t hi = (uint32_t)(b >> 32), lo = (uint32_t)b;
    const bool ok = ((hi & 0x7FF00000u) >= ((1023u - 126u) << 20) && (lo & 0x1FFFFFFFu) != 0x10000000u) || y == 0.0;
    out = (float)y + 0.0f;
    return ok;
}

// The activation side of a Q4_K-style Sub32 group, the same on every lane of a tile: the scales,
// their exponent extremes, whether the first route below applies (every significand in 8..15, as
// the quantizer gives them, and the exponents within 16 places) and then F_j = m_j * 2^(e_j -
// emin), else F_j = 0.  F_j is built from its bits in scalar registers: with m = 8 + r (r < 8),
// m * 2^d has the binary64 exponent 3 + d and the top three fraction bits r, all in the high word.
struct Sub32Act {
    int m[8], e[8];
    int emin, emax;
    bool fast;
    double F[8];
};

__device__ __forceinline__ Sub32Act sub32_act(const int (&m)[8], const int (&e)[8])
{
    Sub32Act g;
    // the extremes, and (m ^ 8) or-ed together (below 8 exactly when every m is in 8..15), in
    // scalar registers: a read of the first lane after each step keeps them there
    int emin = e[0], emax = e[0];
    uint32_t mo = (uint32_t)m[0] ^ 8u;
#pragma unroll
    for (int j = 1; j < 8; j++) {
        emin = __builtin_amdgcn_readfirstlane(e[j] < emin ? e[j] : emin);
        emax = __builtin_amdgcn_readfirstlane(e[j] > emax ? e[j] : emax);
        mo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(mo | ((uint32_t)m[j] ^ 8u)));
    }
    g.emin = emin;
    g.emax = emax;
    g.fast = emax - emin <= 16 && mo < 8u;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        g.m[j] = m[j];
        g.e[j] = e[j];
        const uint32_t hi = ((uint32_t)(1026 + e[j] - emin) << 20) | (((uint32_t)m[j] & 7u) << 17);
        g.F[j] = __builtin_bit_cast(double, (uint64_t)(g.fast ? hi : 0u) << 32);
    }
    return g;
}

// Sub32, Q4_K-style: R32(sum_j m_j 2^e_j (d*C_j - dmin*O_j)), the sixteen terms of exact_sum.
//
// First route (g.fast; all sixteen term exponents then lie within 16 + 29 places, so the sum
// window cannot engage; F_j < 2^20): IC = sum F_j C_j (< 2^45) and IO = sum F_j O_j (< 2^41) are exact f64
// sums and the group is 2^emin * (d*IC - dmin*IO).  dmin*IO is exact (< 2^52), so one fma
// gives V = d*IC - dmin*IO rounded once to binary64, and r32_of_rounded turns 2^emin times that
// into the piece.  False (out untouched) when it sits on a binary32 rounding boundary or below
// the normal range: then piece_q4k_sub32.
__device__ __forceinline__ bool sub32_first_route(const int (&C)[8], const int (&O)[8], const Sub32Act &g,
                                                  uint32_t d_dmin, float &out)
{
    double IC = 0.0, IO = 0.0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        IC = __builtin_fma(g.F[j], (double)C[j], IC);
        IO = __builtin_fma(g.F[j], (double)O[j], IO);
    }
    const float fd = f16_value(d_dmin), fm = f16_value(d_dmin >> 16);
    const double V = __builtin_fma(IC, (double)fd, -(IO * (double)fm));
    return r32_of_rounded(__builtin_ldexp(V, g.emin), out);
}

// The other groups (and the first route's boundary cases): when the block scales are near
// (q4k_near), X_j = d*C_j - dmin*O_j is exact in one fma (|C_j| < 2^22, |O_j| < 2^18) and T_j =
// X_j * m_j 2^e_j too; with the sum window not engaged the eight T_j are summed by sum8_pair.
// Failing that, the 128-bit sum of the sixteen terms.
__device__ __forceinline__ float piece_q4k_sub32(const int (&C)[8], const int (&O)[8], const Sub32Act &g,
                                                 uint32_t d_dmin)
{
    const float fd = f16_value(d_dmin), fm = f16_value(d_dmin >> 16);
    const F16Scale d = f16_scale(d_dmin & 0xFFFFu);
    const F16Scale dm = f16_scale(d_dmin >> 16);
    const int dlo = d.ex < dm.ex ? d.ex : dm.ex, dhi = d.ex < dm.ex ? dm.ex : d.ex;
    if (q4k_near(fd, fm) && (g.emax - g.emin) + (dhi - dlo) <= kSumWindow) {
        double T[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const double X = __builtin_fma((double)C[j], (double)fd, -((double)O[j] * (double)fm));
            T[j] = X * __builtin_ldexp((double)g.m[j], g.e[j]);
        }
        float r;
        if (sum8_pair(T, g.emin + dlo, r)) return r;
    }
    long long v[16];
    int ex[16];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        v[2 * j] = (long long)(d.sig * g.m[j]) * C[j];
        ex[2 * j] = g.e[j] + d.ex;
        v[2 * j + 1] = -(long long)(dm.sig * g.m[j]) * O[j];
        ex[2 * j + 1] = g.e[j] + dm.ex;
    }
    return exact_sum<16>(v, ex);
}

// Sub32 with one weight scale per term (Q6_K-style: d shared, C_j the pair of 16-element sums
// of sub-block j; the 32-element-block formats: d_j per block): R32(sum_j m_j 2^e_j d_j C_j),
// eight terms of at most 2^11 * 2^4 * 2^28 in magnitude, each exact as a double; summed by
// sum8_pair when the window is not engaged, else by the 128-bit sum.
__device__ __forceinline__ float piece_sub32_scaled(const long long (&C)[8], const uint32_t (&dbits)[8],
                                                    const int (&m)[8], const int (&e)[8])
{
    long long v[8];
    int ex[8];
    int emin, emax;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const F16Scale d = f16_scale(dbits[j]);
        v[j] = (long long)(d.sig * m[j]) * C[j];
        ex[j] = e[j] + d.ex;
        emin = j == 0 || ex[j] < emin ? ex[j] : emin;
        emax = j == 0 || ex[j] > emax ? ex[j] : emax;
    }
    if (emax - emin <= kSumWindow) {
        double T[8];
#pragma unroll
        for (int j = 0; j < 8; j++) T[j] = __builtin_ldexp((double)v[j], ex[j]);
        float r;
        if (sum8_pair(T, emin, r)) return r;
    }
    return exact_sum<8>(v, ex);
}

}  // namespace qg
