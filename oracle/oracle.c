/*
 * oracle.c -- CPU oracle of the exact block-quantized dot product (decode GEMV and its
 * batched-column form).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load this library.  It shares no source, header, table or helper with the GPU path,
 * and it reads a matrix only through its logical fields (codes, sub-block scales and
 * offsets, binary16 block scales), never through the packed GPU image.
 *
 * What it follows (page title, then the item on that page):
 *   [N]  rustdoc page "Module numerics" of logicaffeine_compile::spatial::decode_engine:
 *        the module description (the two activation scalings, in-order row sums, the f32
 *        model), Structs ActRow / ActScale / CodedRow / Scale / Segment / Unreadable,
 *        Constants COEF_BOUND / SUM_WINDOW / NAN / WIDE_BITS / ACT_BLOCK / GROUP, Functions
 *        absmax / block_scale / wide_scale / rne / rne_div / quantize / quantize_blocks /
 *        exact_sum / scaled_to_f32 / ftz / fadd / dot.
 *   [L]  rustdoc page "Module lane" of the same crate: the module description (a block's
 *        coefficient sum and offset sum, times the block scales and the activation scale,
 *        summed exactly, rounded once, added into the row) and Functions block_sums / group /
 *        lane.
 *
 * Readings taken where the pages leave a step open (each is also listed in the design notes):
 *   R1  Q4_K-style weight w = d*sc*q - dmin*mn; the second scale multiplies the offset term
 *       with a minus sign.  Q6_K-style w = d*sc*(q-32), no offset term.
 *   R2  binary16 block scales are read exactly, subnormals and zeros included; an exponent
 *       field of 31 (inf/NaN) makes the block Unreadable.
 *   R3  every activation element is read through ftz before the absmax and before coding;
 *       a NaN element is passed over by the absmax and gets code 0; +-inf is an error.
 *   R4  an all-zero activation block (absmax +0) takes the scale m = lo (128 or 8), e = 0,
 *       with every code 0.
 *   R5  "rounded once to f32, denormal flushed" = IEEE binary32 round-to-nearest-even on the
 *       gradual-underflow grid, then a subnormal result becomes a zero of its sign;
 *       a result past the largest finite value is infinite; an exact zero is +0.
 *   R6  a row's sum starts at +0 and adds the pieces in ascending block (group) order with
 *       binary32 adds, each result flushed; any NaN output is 0x7FC00000.
 *   R7  SUM_WINDOW (its value is not printed) is taken as 64.  A term's "least place" is the
 *       exponent it is formed with; the largest term is the one of largest magnitude, the
 *       lowest index among equals; a term below the window is floored (toward -inf) to a
 *       multiple of 2^(L - 64).  The window never engages at the shipped workloads.
 *   R8  PerBlock activation blocks are the weight format's own 256-element block; Sub32
 *       blocks are 32 elements and a 256-element group is one weight block.
 *
 * Build: plain C11 + GCC's __int128, -O2 -ffp-contract=off, no fast-math (SSE binary32
 * adds with the default MXCSR: no FTZ/DAZ).  Rows may be spread over OpenMP threads; the
 * arithmetic of each row is the same sequential loop whatever the thread count.
 *
 * argmax follows "Module numerics", Functions argmax.  The 32-element-block formats (Q8_0- and
 * Q4_0-style, b32_row) follow the module description's "the matrix format's own block, 32 or
 * 256 elements" under PerBlock, and its 256-element groups under Sub32.
 *
 * OR_MUTANT (0 = none) plants one deliberate mistake; only the oracle's own pin tests build
 * such variants, to show that some pin fails for each.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef OR_MUTANT
#define OR_MUTANT 0
#endif

typedef __int128 i128;
typedef unsigned __int128 u128;

#define OR_SUM_WINDOW 64
#define OR_COEF_BOUND 4096
#define OR_BLOCK 256

enum {
    OR_OK = 0,
    OR_E_NONFINITE = 1,   /* an activation block holds +-inf */
    OR_E_SHAPE = 2,       /* columns not a whole number of 256-element blocks, bad mode */
    OR_E_UNREADABLE = 3,  /* a block scale is inf or NaN (Unreadable) */
    OR_E_RANGE = 4,       /* a code, sub-scale or offset outside its field */
    OR_E_INTERNAL = 5     /* an exactness assertion failed */
};

static int g_threads = 1;

void or_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int or_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------------------------- */
/* binary32 bits                                                                           */

static uint32_t bits_of(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float float_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* [N] ftz: a denormal becomes a zero of the same sign. */
float or_ftz(float x)
{
    uint32_t u = bits_of(x);
    if ((u & 0x7F800000u) == 0) u &= 0x80000000u;
    return float_of(u);
}

/* A finite nonzero binary32 as X * 2^ex with X a signed integer of at most 24 bits. */
static void f32_split(float x, int64_t *X, int *ex)
{
    uint32_t u = bits_of(x);
    int E = (int)((u >> 23) & 255u);
    int64_t M = (int64_t)(u & 0x7FFFFFu);
    if (E == 0) { *X = M; *ex = -149; }
    else { *X = M | 0x800000; *ex = E - 150; }
    if (u >> 31) *X = -*X;
}

static int bitlen_u128(u128 v)
{
    int n = 0;
    while (v) { v >>= 1; n++; }
    return n;
}

/* [N] scaled_to_f32 (reading R5): v * 2^exp rounded once to binary32, nearest with ties to
 * even on the gradual-underflow grid, past the top infinite, then a subnormal result
 * flushed to a zero of its sign. */
float or_r32(i128 v, int exp)
{
    if (v == 0) return 0.0f;
    uint32_t sign = v < 0 ? 0x80000000u : 0u;
    u128 M = v < 0 ? (u128)(-v) : (u128)v;
    int n = bitlen_u128(M);
    int top = exp + n - 1;                          /* place of the leading bit */
    int q = top - 23;                               /* place of the last kept bit ... */
    if (q < -149) q = -149;                         /* ... never finer than the subnormal grid */
    u128 R;
    int shift = q - exp;
    if (shift <= 0) {
        R = M << (-shift);                          /* exact, fewer than 24 bits */
    } else if (shift >= 128) {
        R = 0;                                      /* below half the quantum: rounds to 0 */
    } else {
        R = M >> shift;
        u128 rem = M - (R << shift);
        u128 half = (u128)1 << (shift - 1);
#if OR_MUTANT == 3
        if (rem >= half) R += 1;                    /* MUTANT: ties away from zero */
#else
        if (rem > half || (rem == half && (R & 1))) R += 1;
#endif
    }
    if (R == ((u128)1 << 24)) { R >>= 1; q += 1; }  /* rounding carried into a new binade */
#if OR_MUTANT == 4
    /* MUTANT: decide the flush before rounding (24-bit significand, then flush) */
    if (top < -126) return float_of(sign);
#endif
    if (R < ((u128)1 << 23)) return float_of(sign);   /* subnormal or zero: flushed */
    int biased = q + 23 + 127;
    if (biased > 254) return float_of(sign | 0x7F800000u);
    return float_of(sign | ((uint32_t)biased << 23) | (uint32_t)(R - ((u128)1 << 23)));
}

float or_scaled_to_f32(int64_t v, int exp) { return or_r32((i128)v, exp); }

/* ------------------------------------------------------------------------------------- */
/* [N] exact_sum, reading R7                                                                */

typedef struct { i128 v; int e; } term_t;

/* -1, 0, 1 as |a.v|*2^a.e is below, equal to, above |b.v|*2^b.e */
static int mag_cmp(term_t a, term_t b)
{
    u128 A = a.v < 0 ? (u128)(-a.v) : (u128)a.v;
    u128 B = b.v < 0 ? (u128)(-b.v) : (u128)b.v;
    if (A == 0 || B == 0) return (A != 0) - (B != 0);
    int ta = a.e + bitlen_u128(A), tb = b.e + bitlen_u128(B);
    if (ta != tb) return ta > tb ? 1 : -1;
    /* same leading place: bring both to the smaller exponent (no overflow: same bit length) */
    if (a.e > b.e) A <<= (a.e - b.e); else B <<= (b.e - a.e);
    return (A > B) - (A < B);
}

static i128 floor_shift(i128 v, int s)
{
    if (s >= 127) return v < 0 ? -1 : 0;
    return v >> s;                                  /* GCC: arithmetic shift = floor */
}

/* Sum of v*2^e over the terms, rounded once: exact while every term's exponent is at least
 * SUM_WINDOW below the largest term's exponent; a term further down is floored there. */
static int exact_sum(const term_t *t, int n, float *out)
{
    if (n == 0) { *out = 0.0f; return OR_OK; }
    int L = 0;
    for (int i = 1; i < n; i++)
        if (mag_cmp(t[i], t[L]) > 0) L = i;         /* strict: the first of equals stays */
    int floor_e = t[L].e - OR_SUM_WINDOW;
    term_t u[32];
    if (n > 32) return OR_E_INTERNAL;
    int emin = 0;
    for (int i = 0; i < n; i++) {
        u[i] = t[i];
        if (u[i].e < floor_e) { u[i].v = floor_shift(u[i].v, floor_e - u[i].e); u[i].e = floor_e; }
        if (i == 0 || u[i].e < emin) emin = u[i].e;
    }
    i128 s = 0;
    const i128 lim = (i128)1 << 120;
    for (int i = 0; i < n; i++) {
        int sh = u[i].e - emin;
        if (u[i].v == 0) continue;
        if (sh > 118) return OR_E_INTERNAL;
        i128 w = u[i].v * ((i128)1 << sh);
        if (w > lim || w < -lim) return OR_E_INTERNAL;
        s += w;
    }
    *out = or_r32(s, emin);
    return OR_OK;
}

int or_exact_sum_i64(int n, const int64_t *v, const int32_t *e, float *out)
{
    term_t t[32];
    if (n < 0 || n > 32) return OR_E_SHAPE;
    for (int i = 0; i < n; i++) { t[i].v = v[i]; t[i].e = e[i]; }
    return exact_sum(t, n, out);
}

/* ------------------------------------------------------------------------------------- */
/* [N] Scale / Unreadable (reading R2): a binary16 block scale as sig * 2^exp, exactly.      */

static int f16_scale(uint16_t h, int64_t *sig, int *ex)
{
    int s = h >> 15, E = (h >> 10) & 31, M = h & 1023;
    if (E == 31) return OR_E_UNREADABLE;
    if (E == 0) { *sig = M; *ex = -24; }
    else { *sig = 1024 + M; *ex = E - 25; }
    if (s) *sig = -*sig;
    return OR_OK;
}

int or_f16_scale(uint16_t h, int64_t *sig, int32_t *ex)
{
    int e = 0;
    int r = f16_scale(h, sig, &e);
    *ex = e;
    return r;
}

/* ------------------------------------------------------------------------------------- */
/* Activation quantization                                                                 */

/* ceil(A * 2^a / (127 * 2^e)), A > 0, exact; a - e stays within a few dozen places here. */
static i128 ceil_ratio(int64_t A, int a, int e)
{
    int k = a - e;
    if (k >= 0) {
        i128 num = (i128)A << k;
        return (num + 126) / 127;
    }
    k = -k;
    if (k > 100) return 1;
    i128 den = (i128)127 << k;
    return ((i128)A + den - 1) / den;
}

/* [N] wide_scale (lo = 128, an 8-bit significand) and block_scale (lo = 8, a 4-bit one):
 * the least m * 2^e with lo <= m < 2*lo and 127 * m * 2^e >= amax, amax finite and > 0.
 * Walk the exponent down from a grid so coarse that m = lo is already enough, for as long
 * as a finer grid still has an admissible significand; the least value sits at the last
 * such exponent, with the least m there that reaches amax. */
static void least_scale(float amax, int lo, int *m, int *e)
{
    int64_t A; int a;
    f32_split(amax, &A, &a);
    int ee = a + 26;                                /* 127 * 2^ee > A * 2^a: one grid step covers amax */
#if OR_MUTANT == 8
    while (ceil_ratio(A, a, ee - 1) <= 2 * lo - 2) ee--;   /* MUTANT: admits one m too few */
#else
    while (ceil_ratio(A, a, ee - 1) <= 2 * lo - 1) ee--;
#endif
    i128 mm = ceil_ratio(A, a, ee);
    if (mm < lo) mm = lo;
    *m = (int)mm;
    *e = ee;
}

int or_least_scale(int lo, float amax, int32_t *m, int32_t *e)
{
    if (!(amax > 0.0f) || isinf(amax)) return OR_E_NONFINITE;
    int mm, ee;
    least_scale(amax, lo, &mm, &ee);
    *m = mm; *e = ee;
    return OR_OK;
}

/* [N] rne_div / rne: the nearest integer to x / (m * 2^e), ties to even, exactly. */
static int64_t rne_div(float x, int m, int e)
{
    if (x == 0.0f) return 0;
    int64_t X; int ex;
    f32_split(x, &X, &ex);
    int k = ex - e;                                 /* x / s = X * 2^k / m */
    u128 num = X < 0 ? (u128)(-X) : (u128)X;
    u128 den = (u128)m;
    if (k >= 0) {
        if (k > 60) return X < 0 ? -(1LL << 40) : (1LL << 40);   /* never: |x/s| <= 127 */
        num <<= k;
    } else {
        if (-k > 100) return 0;
        den <<= -k;
    }
    u128 q = num / den, r = num - q * den;
#if OR_MUTANT == 5
    if (2 * r >= den) q++;                          /* MUTANT: ties away from zero */
#else
    if (2 * r > den || (2 * r == den && (q & 1))) q++;
#endif
    return X < 0 ? -(int64_t)q : (int64_t)q;
}

int64_t or_rne_div(float x, int m, int e) { return rne_div(or_ftz(x), m, e); }

/* [N] Functions absmax.  Scans for the greatest |x| starting from +0: each element is flushed
 * first (a subnormal counts as zero) and NaNs are skipped, so an all-NaN block gives +0. */
static float absmax(const float *x, int64_t n)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; i++) {
#if OR_MUTANT == 6
        float v = x[i];                             /* MUTANT: no flush of denormal operands */
#else
        float v = or_ftz(x[i]);
#endif
        if (isnan(v)) continue;
        v = fabsf(v);
        if (v > a) a = v;
    }
    return a;
}

/* [N] quantize_blocks (mode 0: PerBlock, one scale per `block` elements, 8-bit significand)
 * and quantize (mode 1: Sub32, one scale per 32 elements, 4-bit significand).
 * x: f32 [n][cols]; codes: int8 [n][cols]; sm, se: the scale's m and e per activation
 * block, [n][cols/ablk]; sums16: int32 [n][cols/16], the sum of the codes of each run of
 * 16 elements (the activation side's per-unit code sums of the lane page). */
int or_quantize(int mode, int block, int64_t n, int64_t cols, const float *x, int8_t *codes,
                uint8_t *sm, int16_t *se, int32_t *sums16)
{
    if (mode != 0 && mode != 1) return OR_E_SHAPE;
    if (cols < 0 || n < 0 || cols % OR_BLOCK) return OR_E_SHAPE;
    int ablk = mode == 0 ? block : 32;
    int lo = mode == 0 ? 128 : 8;
    if (ablk <= 0 || cols % ablk || ablk % 16) return OR_E_SHAPE;
    int64_t nb = cols / ablk;
    int status = OR_OK;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *xb = x + r * cols + b * ablk;
            float amax = absmax(xb, ablk);
            int m, e;
            if (isinf(amax)) { status = OR_E_NONFINITE; m = 0; e = 0; }
            else if (amax == 0.0f) { m = lo; e = 0; }
            else least_scale(amax, lo, &m, &e);
            sm[r * nb + b] = (uint8_t)m;
            se[r * nb + b] = (int16_t)e;
            for (int i = 0; i < ablk; i++) {
                float v = or_ftz(xb[i]);
                int64_t c = 0;
                if (m != 0 && !isnan(v)) c = rne_div(v, m, e);
                if (c > 127 || c < -127) return OR_E_INTERNAL;   /* 127*m*2^e >= amax bounds it */
                codes[r * cols + b * ablk + i] = (int8_t)c;
            }
        }
        for (int64_t u = 0; u < cols / 16; u++) {
            int32_t s = 0;
            for (int i = 0; i < 16; i++) s += codes[r * cols + u * 16 + i];
            sums16[r * (cols / 16) + u] = s;
        }
    }
    return status;
}

/* ------------------------------------------------------------------------------------- */
/* The dot: one row of a block-format matrix against one quantized activation row          */

/* [N] fadd + ftz, f32 model of the module description: binary32 add, nearest-even, result
 * flushed.  Operands here are already normal or zero. */
static float fadd(float a, float b) { return or_ftz(a + b); }

static float canon_nan(float y)
{
    return isnan(y) ? float_of(0x7FC00000u) : y;    /* [N] NAN: quiet, no payload, no sign */
}

/* Integer sums of one 32-element sub-block of a Q4_K-style block, element by element
 * ([L] block_sums): coefficient sum sum(sc*q*c) and offset sum sum(mn*c). */
static void q4k_sub_sums(const uint8_t *q, int sc, int mn, const int8_t *c, int64_t *Cs, int64_t *Os)
{
    int64_t C = 0, O = 0;
    for (int i = 0; i < 32; i++) {
        int64_t coef = (int64_t)sc * q[i];
        int64_t offs = mn;
        C += coef * c[i];
        O += offs * c[i];
    }
    *Cs = C; *Os = O;
}

/* Integer coefficient sum of one 16-element sub-block of a Q6_K-style block. */
static int64_t q6k_sub_sum(const uint8_t *q, int sc, const int8_t *c)
{
    int64_t C = 0;
    for (int i = 0; i < 16; i++) {
        int64_t coef = (int64_t)sc * ((int64_t)q[i] - 32);
        C += coef * c[i];
    }
    return C;
}

static int check_q4k_row(const uint8_t *q, const uint8_t *sc, const uint8_t *mn, int64_t cols)
{
    for (int64_t i = 0; i < cols; i++) if (q[i] > 15) return OR_E_RANGE;
    for (int64_t j = 0; j < cols / 32; j++) if (sc[j] > 63 || mn[j] > 63) return OR_E_RANGE;
    return OR_OK;
}

/* One Q4_K-style row.  mode 0: per block the two terms m*2^e * d * C_b and
 * -m*2^e * dmin * O_b, summed exactly and rounded once ([N] module description, PerBlock;
 * [L] lane).  mode 1: per 256-element group the 16 terms of its eight 32-element
 * sub-blocks, each under its own activation scale, summed exactly and rounded once ([N]
 * module description, Sub32; [L] group).  The pieces are then added in order. */
static int q4k_row(int mode, int64_t cols, const uint8_t *q, const uint8_t *sc, const uint8_t *mn,
                   const uint16_t *d, const uint16_t *dmin, const int8_t *c, const uint8_t *sm,
                   const int16_t *se, float *out)
{
    int st = check_q4k_row(q, sc, mn, cols);
    if (st) return st;
    int64_t G = cols / OR_BLOCK;
    float y = 0.0f;
    float piece[4096];
    if (G > 4096) return OR_E_SHAPE;
    for (int64_t b = 0; b < G; b++) {
        int64_t sd, sm2; int ed, em;
        if (f16_scale(d[b], &sd, &ed) || f16_scale(dmin[b], &sm2, &em)) return OR_E_UNREADABLE;
        term_t t[16];
        int nt = 0;
        if (mode == 0) {
            int64_t Cb = 0, Ob = 0;
            for (int j = 0; j < 8; j++) {
                int64_t Cj, Oj;
#if OR_MUTANT == 7
                int jj = (j * 32) / 16 % 8;         /* MUTANT: sub-scale indexed per 16 elements */
                q4k_sub_sums(q + b * 256 + j * 32, sc[b * 8 + jj], mn[b * 8 + jj], c + b * 256 + j * 32, &Cj, &Oj);
#else
                q4k_sub_sums(q + b * 256 + j * 32, sc[b * 8 + j], mn[b * 8 + j], c + b * 256 + j * 32, &Cj, &Oj);
#endif
                Cb += Cj; Ob += Oj;
            }
            int m = sm[b], e = se[b];
            t[nt].v = (i128)m * sd * Cb; t[nt].e = e + ed; nt++;
#if OR_MUTANT == 1
            (void)em; (void)sm2;                    /* MUTANT: offset term dropped */
#elif OR_MUTANT == 2
            t[nt].v = (i128)m * sm2 * Ob; t[nt].e = e + em; nt++;     /* MUTANT: sign of offset term */
#else
            t[nt].v = -(i128)m * sm2 * Ob; t[nt].e = e + em; nt++;
#endif
        } else {
            for (int j = 0; j < 8; j++) {
                int64_t Cj, Oj;
                q4k_sub_sums(q + b * 256 + j * 32, sc[b * 8 + j], mn[b * 8 + j], c + b * 256 + j * 32, &Cj, &Oj);
                int m = sm[b * 8 + j], e = se[b * 8 + j];
                t[nt].v = (i128)m * sd * Cj; t[nt].e = e + ed; nt++;
                t[nt].v = -(i128)m * sm2 * Oj; t[nt].e = e + em; nt++;
            }
        }
        st = exact_sum(t, nt, &piece[b]);
        if (st) return st;
    }
#if OR_MUTANT == 9
    /* MUTANT: pieces folded by a balanced pairwise tree instead of in order */
    for (int64_t w = 1; w < G; w *= 2)
        for (int64_t i = 0; i + w < G; i += 2 * w) piece[i] = fadd(piece[i], piece[i + w]);
    y = G ? fadd(0.0f, piece[0]) : 0.0f;
#else
    for (int64_t b = 0; b < G; b++) y = fadd(y, piece[b]);
#endif
    *out = canon_nan(y);
    return OR_OK;
}

static int q6k_row(int mode, int64_t cols, const uint8_t *q, const int8_t *sc, const uint16_t *d,
                   const int8_t *c, const uint8_t *sm, const int16_t *se, float *out)
{
    for (int64_t i = 0; i < cols; i++) if (q[i] > 63) return OR_E_RANGE;
    int64_t G = cols / OR_BLOCK;
    float y = 0.0f;
    for (int64_t b = 0; b < G; b++) {
        int64_t sd; int ed;
        if (f16_scale(d[b], &sd, &ed)) return OR_E_UNREADABLE;
        term_t t[8];
        int nt = 0;
        if (mode == 0) {
            int64_t Cb = 0;
            for (int k = 0; k < 16; k++) Cb += q6k_sub_sum(q + b * 256 + k * 16, sc[b * 16 + k], c + b * 256 + k * 16);
            t[nt].v = (i128)sm[b] * sd * Cb; t[nt].e = se[b] + ed; nt++;
        } else {
            /* a 32-element activation block covers two 16-element weight sub-blocks */
            for (int j = 0; j < 8; j++) {
                int64_t Cj = q6k_sub_sum(q + b * 256 + j * 32, sc[b * 16 + 2 * j], c + b * 256 + j * 32)
                           + q6k_sub_sum(q + b * 256 + j * 32 + 16, sc[b * 16 + 2 * j + 1], c + b * 256 + j * 32 + 16);
                t[nt].v = (i128)sm[b * 8 + j] * sd * Cj; t[nt].e = se[b * 8 + j] + ed; nt++;
            }
        }
        float p;
        int st = exact_sum(t, nt, &p);
        if (st) return st;
        y = fadd(y, p);
    }
    *out = canon_nan(y);
    return OR_OK;
}

/* Formats with 32-element weight blocks and one binary16 scale per block ([N] module
 * description: "the matrix format's own block, 32 or 256 elements"): Q8_0-style (fmt 3), an
 * int8 code per weight, w = d*q; Q4_0-style (fmt 4), a 4-bit code, w = d*(q - 8).  q holds
 * the stored bytes: int8 two's complement for Q8_0, 0..15 for Q4_0.  The integer sum of one
 * 32-element block against 32 activation codes, element by element. */
static int64_t b32_sum(int fmt, const uint8_t *q, const int8_t *c)
{
    int64_t C = 0;
    for (int i = 0; i < 32; i++) {
#if OR_MUTANT == 12
        int64_t w = fmt == 3 ? (int64_t)q[i] : (int64_t)q[i] - 8;          /* MUTANT: Q8_0 read unsigned */
#elif OR_MUTANT == 13
        int64_t w = fmt == 3 ? (int64_t)(int8_t)q[i] : (int64_t)q[i];      /* MUTANT: Q4_0 offset dropped */
#else
        int64_t w = fmt == 3 ? (int64_t)(int8_t)q[i] : (int64_t)q[i] - 8;
#endif
        C += w * c[i];
    }
    return C;
}

/* One row of a 32-element-block matrix.  mode 0 (PerBlock over the format's own 32-element
 * block, 8-bit significand): per block the single term m*2^e * d * C_b, rounded once.  mode 1
 * (Sub32, 4-bit significand): per 256-element group the eight terms of its blocks, each
 * under its own activation and weight scale, summed exactly and rounded once.  The pieces
 * are then added in order. */
static int b32_row(int fmt, int mode, int64_t cols, const uint8_t *q, const uint16_t *d, const int8_t *c,
                   const uint8_t *sm, const int16_t *se, float *out)
{
    if (fmt == 4)
        for (int64_t i = 0; i < cols; i++) if (q[i] > 15) return OR_E_RANGE;
    int64_t nb = cols / 32;
    float y = 0.0f;
    const int per = mode == 0 ? 1 : 8;        /* blocks per piece */
    for (int64_t b0 = 0; b0 < nb; b0 += per) {
        term_t t[8];
        for (int j = 0; j < per; j++) {
            int64_t b = b0 + j;
            int64_t sd; int ed;
            if (f16_scale(d[b], &sd, &ed)) return OR_E_UNREADABLE;
            t[j].v = (i128)sm[b] * sd * b32_sum(fmt, q + b * 32, c + b * 32);
            t[j].e = se[b] + ed;
        }
        float p;
        int st = exact_sum(t, per, &p);
        if (st) return st;
        y = fadd(y, p);
    }
    *out = canon_nan(y);
    return OR_OK;
}

/* [N] dot, batched, for the 32-element-block formats: q [rows][cols], d [rows][cols/32],
 * activation scales [ncol][cols/32] (PerBlock over 32 elements, or Sub32). */
int or_gemm_b32(int fmt, int mode, int64_t rows, int64_t cols, int64_t ncol, const uint8_t *q, const uint16_t *d,
                const int8_t *codes, const uint8_t *sm, const int16_t *se, float *out)
{
    if ((fmt != 3 && fmt != 4) || (mode != 0 && mode != 1) || cols % OR_BLOCK) return OR_E_SHAPE;
    int status = OR_OK;
    const int64_t nsc = cols / 32;
#pragma omp parallel for schedule(dynamic, 16) num_threads(g_threads) if (g_threads > 1)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < ncol; k++) {
            int st = b32_row(fmt, mode, cols, q + r * cols, d + r * (cols / 32), codes + k * cols, sm + k * nsc,
                             se + k * nsc, &out[k * rows + r]);
            if (st) {
#pragma omp critical
                status = st;
            }
        }
    }
    return status;
}

/* [N] dot, batched: out[col * rows + r] = dot(row r, activation row col).
 * A single column (ncol = 1) is the decode GEMV. */
int or_gemm_q4k(int mode, int64_t rows, int64_t cols, int64_t ncol, const uint8_t *q, const uint8_t *sc,
                const uint8_t *mn, const uint16_t *d, const uint16_t *dmin, const int8_t *codes,
                const uint8_t *sm, const int16_t *se, float *out)
{
    if ((mode != 0 && mode != 1) || cols % OR_BLOCK || rows < 0 || ncol < 0) return OR_E_SHAPE;
    int64_t G = cols / OR_BLOCK, nsc = mode == 0 ? G : cols / 32;
    int status = OR_OK;
#pragma omp parallel for schedule(dynamic, 16) num_threads(g_threads) if (g_threads > 1)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < ncol; k++) {
            int st = q4k_row(mode, cols, q + r * cols, sc + r * (cols / 32), mn + r * (cols / 32),
                             d + r * G, dmin + r * G, codes + k * cols, sm + k * nsc, se + k * nsc,
                             &out[k * rows + r]);
            if (st) {
#pragma omp critical
                status = st;
            }
        }
    }
    return status;
}

int or_gemm_q6k(int mode, int64_t rows, int64_t cols, int64_t ncol, const uint8_t *q, const int8_t *sc,
                const uint16_t *d, const int8_t *codes, const uint8_t *sm, const int16_t *se, float *out)
{
    if ((mode != 0 && mode != 1) || cols % OR_BLOCK || rows < 0 || ncol < 0) return OR_E_SHAPE;
    int64_t G = cols / OR_BLOCK, nsc = mode == 0 ? G : cols / 32;
    int status = OR_OK;
#pragma omp parallel for schedule(dynamic, 16) num_threads(g_threads) if (g_threads > 1)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t k = 0; k < ncol; k++) {
            int st = q6k_row(mode, cols, q + r * cols, sc + r * (cols / 16), d + r * G,
                             codes + k * cols, sm + k * nsc, se + k * nsc, &out[k * rows + r]);
            if (st) {
#pragma omp critical
                status = st;
            }
        }
    }
    return status;
}

/* Integer sums per (row, 32-element sub-block) of a Q4_K-style matrix against one code row:
 * Cs = sum sc*q*c and Os = sum mn*c ([L] block_sums, before any scale). [rows][cols/32]. */
int or_sub_sums_q4k(int64_t rows, int64_t cols, const uint8_t *q, const uint8_t *sc, const uint8_t *mn,
                    const int8_t *codes, int64_t *Cs, int64_t *Os)
{
    if (cols % OR_BLOCK) return OR_E_SHAPE;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < cols / 32; j++)
            q4k_sub_sums(q + r * cols + j * 32, sc[r * (cols / 32) + j], mn[r * (cols / 32) + j],
                         codes + j * 32, &Cs[r * (cols / 32) + j], &Os[r * (cols / 32) + j]);
    return OR_OK;
}

/* Coefficient sums per (row, 16-element sub-block) of a Q6_K-style matrix: sum sc*(q-32)*c. */
int or_sub_sums_q6k(int64_t rows, int64_t cols, const uint8_t *q, const int8_t *sc, const int8_t *codes,
                    int64_t *Cs)
{
    if (cols % OR_BLOCK) return OR_E_SHAPE;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < cols / 16; k++)
            Cs[r * (cols / 16) + k] = q6k_sub_sum(q + r * cols + k * 16, sc[r * (cols / 16) + k], codes + k * 16);
    return OR_OK;
}

/* [N] Functions argmax.  A left-to-right scan with binary32 comparisons that replaces the best
 * position only on a strictly greater value, so the earliest of equal values wins (and +0
 * ties with -0); NaNs are skipped; the result is 0 when nothing but NaNs (or nothing) is
 * seen. */
int64_t or_argmax(const float *x, int64_t n)
{
    int64_t best = -1;
    for (int64_t i = 0; i < n; i++) {
        if (x[i] != x[i]) continue;                 /* NaN */
#if OR_MUTANT == 10
        if (best < 0 || x[i] >= x[best]) best = i;  /* planted: the last of equals */
#elif OR_MUTANT == 11
        if (best < 0 || bits_of(x[i]) > bits_of(x[best])) best = i;   /* planted: compares bit patterns */
#else
        if (best < 0 || x[i] > x[best]) best = i;
#endif
    }
    return best < 0 ? 0 : best;
}

/* ------------------------------------------------------------------------------------- */
/* int8 KV cache ([N] Functions cache_row, int8_codes, quantize_head, int8_score,           */
/* weighted_int8, attend_int8; Constants INV_127, VALUE_BLOCK).                            */
/*                                                                                         */
/* Readings (the pages leave these open):                                                  */
/*   K1 cache_row's scale is the binary16 (nearest even, subnormals kept, past the top       */
/*      infinite) of amax * INV_127 formed in binary32, INV_127 = 1/127 rounded to binary32, */
/*      amax as absmax (a denormal read as 0, a NaN passed over).                           */
/*   K2 int8_codes: inv = 1 / (the scale as binary32), a binary32 division; a code is the   */
/*      binary32 product x * inv to the nearest integer (ties to even), clamped to           */
/*      [-127, 127]; a NaN product gives 0; an infinite inv (a zero scale) gives all zeros.  */
/*   K3 quantize_head: PerBlock, the whole head one block under the 8-bit wide scale;       */
/*      Sub32, per 32 elements under the 4-bit block scale.  The head is a whole number of  */
/*      32-element groups.                                                                  */
/*   K4 int8_score: over the query's blocks b, m_b 2^e_b * (sum of c_i k_i) * d_k summed     */
/*      exactly (exact_sum, window included) and rounded once; a key whose scale is not     */
/*      finite scores the canonical NaN.                                                    */
/*   K5 weighted_int8: w_j = p_j * d_j in binary32 (d_j the value row's scale); per block   */
/*      of VALUE_BLOCK = 32 positions (the last one possibly shorter) the least power of two */
/*      2^E with 127 * 2^E >= absmax of the w_j (E = 0 for an all-zero block); codes        */
/*      u_j = rne(w_j / 2^E), exact (a NaN gives 0); per value element the piece            */
/*      R32(2^E * sum_j u_j v_j), the pieces added in block order (fadd).  A block holding   */
/*      an infinite w_j, or a value row whose scale is not finite, gives NaN pieces.         */
/*      The page does not print VALUE_BLOCK's value: 32 is a reading, and parity of the      */
/*      weighted sum's block length is unpinned by the pages.                               */
/* -------------------------------------------------------------------------------------- */

#define OR_VALUE_BLOCK 32

static int bitlen_u64(uint64_t v)
{
    int n = 0;
    while (v) { v >>= 1; n++; }
    return n;
}

/* [K1] binary32 -> binary16 bits: nearest even on the binary16 grid (subnormals kept: a
 * spacing of 2^-24 below 2^-14), past the largest finite value infinite, NaN -> 0x7E00. */
uint16_t or_f16_rne(float x)
{
    uint32_t u = bits_of(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return 0x7E00;
    if (isinf(x)) return sign | 0x7C00;
    if (x == 0.0f) return sign;
    int64_t X; int a;
    f32_split(fabsf(x), &X, &a);                        /* |x| = X * 2^a */
    int L = bitlen_u64((uint64_t)X) - 1 + a;            /* 2^L <= |x| < 2^(L+1) */
    int s = L - 10;                                     /* the grid spacing there */
    if (s < -24) s = -24;
    int k = a - s;
    uint64_t q;
    if (k >= 0) {
        q = (uint64_t)X << k;                           /* exact: |x| on the grid already */
    } else {
        int sh = -k;
        if (sh > 62) q = 0;
        else {
            uint64_t num = (uint64_t)X;
            q = num >> sh;
            uint64_t rem = num - (q << sh), half = 1ull << (sh - 1);
#if OR_MUTANT == 14
            if (rem >= half) q++;                       /* MUTANT: ties away from zero */
#else
            if (rem > half || (rem == half && (q & 1))) q++;
#endif
        }
    }
    if (q == 2048) { q = 1024; s += 1; }                /* rounded up to the next binade */
    if (s == -24 && q < 1024) return sign | (uint16_t)q;   /* subnormal (or zero) */
    int Eb = s + 25;                                    /* value (q / 1024) * 2^(s + 10) */
    if (Eb >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(Eb << 10) | (uint16_t)(q - 1024);
}

/* binary16 bits -> binary32 value (exact) */
static float f16_to_f32(uint16_t h)
{
    int s = h >> 15, E = (h >> 10) & 31, M = h & 1023;
    float v;
    if (E == 31) v = M ? NAN : INFINITY;
    else if (E == 0) v = ldexpf((float)M, -24);
    else v = ldexpf((float)(M | 1024), E - 25);
    return s ? -v : v;
}

/* [N] cache_row, K1, K2: n rows of hd elements -> scales (binary16 bits) [n], codes [n][hd]. */
int or_kv_cache_rows(int64_t n, int64_t hd, const float *x, uint16_t *scales, int8_t *codes)
{
    if (n < 0 || hd <= 0) return OR_E_SHAPE;
    const float inv127 = 1.0f / 127.0f;
    for (int64_t r = 0; r < n; r++) {
        const float *xr = x + r * hd;
        float amax = absmax(xr, hd);
        uint16_t h = or_f16_rne(amax * inv127);
        scales[r] = h;
        float inv = 1.0f / f16_to_f32(h);
        for (int64_t i = 0; i < hd; i++) {
            int c = 0;
            if (!isinf(inv)) {
                float p = xr[i] * inv;
                if (!isnan(p)) {
#if OR_MUTANT == 15
                    float rr = truncf(p);               /* MUTANT: toward zero */
#else
                    float rr = rintf(p);                /* nearest integer, ties to even */
#endif
                    if (rr > 127.0f) rr = 127.0f;
                    if (rr < -127.0f) rr = -127.0f;
                    c = (int)rr;
                }
            }
            codes[r * hd + i] = (int8_t)c;
        }
    }
    return OR_OK;
}

/* [N] quantize_head, K3: nh heads of hd elements -> codes [nh][hd], m, e [nh][hd / B]
 * (B = hd under PerBlock, 32 under Sub32).  OR_E_NONFINITE when a block holds +-inf (its
 * m = 0 and codes 0, as the activation quantizer). */
int or_kv_quantize_heads(int mode, int64_t nh, int64_t hd, const float *q, int8_t *codes, uint8_t *sm, int16_t *se)
{
    if ((mode != 0 && mode != 1) || nh < 0 || hd <= 0 || hd % 32) return OR_E_SHAPE;
    const int64_t B = mode == 0 ? hd : 32;
    const int lo = mode == 0 ? 128 : 8;
    const int64_t nb = hd / B;
    int status = OR_OK;
    for (int64_t h = 0; h < nh; h++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *xb = q + h * hd + b * B;
            float amax = absmax(xb, B);
            int m, e;
            if (isinf(amax)) { status = OR_E_NONFINITE; m = 0; e = 0; }
            else if (amax == 0.0f) { m = lo; e = 0; }
            else least_scale(amax, lo, &m, &e);
            sm[h * nb + b] = (uint8_t)m;
            se[h * nb + b] = (int16_t)e;
            for (int64_t i = 0; i < B; i++) {
                float v = or_ftz(xb[i]);
                int64_t c = 0;
                if (m != 0 && !isnan(v)) c = rne_div(v, m, e);
                if (c > 127 || c < -127) return OR_E_INTERNAL;
                codes[h * hd + b * B + i] = (int8_t)c;
            }
        }
    }
    return status;
}

/* [N] int8_score, K4, for every query head h against every cached key row j of its KV head
 * (h / (nh / nkv)): out[h * npos + j].  Keys: scales [nkv][npos], codes [nkv][npos][hd]. */
int or_kv_scores(int mode, int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const int8_t *qc, const uint8_t *qm,
                 const int16_t *qe, const uint16_t *ks, const int8_t *kc, float *out)
{
    if ((mode != 0 && mode != 1) || hd <= 0 || hd % 32 || nkv <= 0 || nh % nkv) return OR_E_SHAPE;
    const int64_t B = mode == 0 ? hd : 32, nb = hd / B, grp = nh / nkv;
    if (nb > 32) return OR_E_SHAPE;
    int status = OR_OK;
#pragma omp parallel for schedule(static) num_threads(g_threads) if (g_threads > 1)
    for (int64_t h = 0; h < nh; h++) {
        const int64_t kv = h / grp;
        for (int64_t j = 0; j < npos; j++) {
            const int8_t *k = kc + (kv * npos + j) * hd;
            int64_t sig; int ex;
            if (f16_scale(ks[kv * npos + j], &sig, &ex)) { out[h * npos + j] = canon_nan(NAN); continue; }
            term_t t[32];
            for (int64_t b = 0; b < nb; b++) {
                int64_t P = 0;
                for (int64_t i = 0; i < B; i++) P += (int64_t)qc[h * hd + b * B + i] * k[b * B + i];
                t[b].v = (i128)qm[h * nb + b] * sig * P;
                t[b].e = qe[h * nb + b] + ex;
            }
            float y;
            int st = exact_sum(t, (int)nb, &y);
            if (st) {
#pragma omp critical
                status = st;
            }
            out[h * npos + j] = canon_nan(y);
        }
    }
    return status;
}

/* [N] weighted_int8, K5, for every head h over its KV head's cached value rows:
 * out[h * hd + e] from probs [nh][npos], values: scales [nkv][npos], codes [nkv][npos][hd]. */
int or_kv_weighted(int64_t nh, int64_t nkv, int64_t npos, int64_t hd, const float *probs, const uint16_t *vs,
                   const int8_t *vc, float *out)
{
    if (hd <= 0 || nkv <= 0 || nh % nkv || npos < 0) return OR_E_SHAPE;
    const int64_t grp = nh / nkv;
#pragma omp parallel for schedule(static) num_threads(g_threads) if (g_threads > 1)
    for (int64_t h = 0; h < nh; h++) {
        const int64_t kv = h / grp;
        float *y = out + h * hd;
        for (int64_t e = 0; e < hd; e++) y[e] = 0.0f;
#if OR_MUTANT == 17
        for (int64_t j0 = (npos - 1) / OR_VALUE_BLOCK * OR_VALUE_BLOCK; j0 >= 0; j0 -= OR_VALUE_BLOCK) {   /* MUTANT: last block first */
#else
        for (int64_t j0 = 0; j0 < npos; j0 += OR_VALUE_BLOCK) {
#endif
            const int64_t nj = npos - j0 < OR_VALUE_BLOCK ? npos - j0 : OR_VALUE_BLOCK;
            float w[OR_VALUE_BLOCK];
            int bad = 0;
            for (int64_t j = 0; j < nj; j++) {
                const uint16_t s = vs[kv * npos + j0 + j];
                if (((s >> 10) & 31) == 31) bad = 1;
                w[j] = probs[h * npos + j0 + j] * f16_to_f32(s);
            }
            float amax = absmax(w, nj);
            if (isinf(amax)) bad = 1;
            int E = 0, m = 1;
            if (!bad && amax > 0.0f) least_scale(amax, 1, &m, &E);   /* m = 1: a power of two */
#if OR_MUTANT == 16
            E += 1;                                     /* MUTANT: not the least power of two */
#endif
            int64_t u[OR_VALUE_BLOCK];
            for (int64_t j = 0; j < nj; j++) {
                const float v = or_ftz(w[j]);
                u[j] = (bad || isnan(v)) ? 0 : rne_div(v, 1, E);
            }
            for (int64_t e = 0; e < hd; e++) {
                float piece;
                if (bad) piece = NAN;
                else {
                    int64_t T = 0;
                    for (int64_t j = 0; j < nj; j++) T += u[j] * vc[(kv * npos + j0 + j) * hd + e];
                    piece = or_r32((i128)T, E);
                }
                y[e] = fadd(y[e], piece);
            }
        }
        for (int64_t e = 0; e < hd; e++) y[e] = canon_nan(y[e]);
    }
    return OR_OK;
}

int or_mutant(void) { return OR_MUTANT; }
int or_coef_bound(void) { return OR_COEF_BOUND; }
int or_sum_window(void) { return OR_SUM_WINDOW; }
