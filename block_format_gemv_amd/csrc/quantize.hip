// quantize.hip -- activation quantizer: per activation block the least scale m*2^e with
// 127*m*2^e >= the block's largest magnitude, the exact nearest-even codes, and the code
// sums of every run of 16 elements ("Module numerics" of
// logicaffeine_compile::spatial::decode_engine: Functions absmax, wide_scale, block_scale,
// rne_div, quantize, quantize_blocks; the activation side's unit sums of "Module lane").
//
// One wave covers 256 consecutive elements (one PerBlock block, or eight Sub32 blocks),
// four per lane.  The scale comes from amax/127 in f64: the quotient is within 2^-53 of
// amax/127, and the nearest grid point of `bits` significant bits lies at least 2^-25 of
// it away unless it equals it, so rounding the f64 quotient up to `bits` significant bits
// gives the least admissible scale.  Codes are rint(x / s) in f64: |x/s| <= 127, and an
// f64 quotient that is not a half-integer cannot round onto one, so ties are exactly the
// true ties and go to even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kThreads = 256;

// least m*2^e (m with `bits` significant bits) not below amax/127, amax finite and > 0
template <int BITS>
__device__ __forceinline__ void least_scale(float amax, int &m, int &e)
{
    const double t = (double)amax / 127.0;
    int k;
    const double f = __builtin_frexp(t, &k);           // t = f * 2^k, f in [0.5, 1)
    double mm = __builtin_ceil(__builtin_ldexp(f, BITS));   // in [2^(BITS-1), 2^BITS]
    int ee = k - BITS;
    if (mm == (double)(1 << BITS)) { mm = (double)(1 << (BITS - 1)); ee += 1; }
    m = (int)mm;
    e = ee;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const float *__restrict__ x, int64_t nchunks,
                                                            int8_t *__restrict__ codes,
                                                            qg_act_scale *__restrict__ scales,
                                                            int32_t *__restrict__ csums,
                                                            int32_t *__restrict__ err_flag)
{
    constexpr int BITS = MODE == QG_PERBLOCK ? 8 : 4;
    constexpr int GROUP_LANES = MODE == QG_PERBLOCK ? 64 : 8;   // lanes sharing one scale
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (chunk >= nchunks) return;                         // wave-uniform
    const int64_t base = chunk * 256 + 4 * lane;
    const float4 v4 = *reinterpret_cast<const float4 *>(x + base);
    float v[4] = {ftz(v4.x), ftz(v4.y), ftz(v4.z), ftz(v4.w)};
    uint32_t amax_bits = 0;
    int inf = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
        if (a > 0x7F800000u) continue;                    // NaN: passed over
        if (a == 0x7F800000u) inf = 1;
        amax_bits = a > amax_bits ? a : amax_bits;        // non-negative floats order as integers
    }
#pragma unroll
    for (int off = 1; off < GROUP_LANES; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)amax_bits, off, 64);
        amax_bits = o > amax_bits ? o : amax_bits;
        inf |= __shfl_xor(inf, off, 64);
    }
    int m, e;
    if (inf) {
        m = 0; e = 0;
    } else if (amax_bits == 0) {
        m = 1 << (BITS - 1); e = 0;                       // all-zero block
    } else {
        least_scale<BITS>(__uint_as_float(amax_bits), m, e);
    }
    uint32_t packed = 0;
    int csum = 0;
    if (m != 0) {
        const double s = __builtin_ldexp((double)m, e);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int c = 0;
            if (v[i] == v[i]) c = (int)__builtin_rint((double)v[i] / s);
            csum += c;
            packed |= ((uint32_t)c & 0xFFu) << (8 * i);
        }
    }
    *reinterpret_cast<uint32_t *>(codes + base) = packed;
    // sums of 16 consecutive codes = 4 lanes
    csum += __shfl_xor(csum, 1, 64);
    csum += __shfl_xor(csum, 2, 64);
    if ((lane & 3) == 0) csums[base / 16] = csum;
    if ((lane & (GROUP_LANES - 1)) == 0) {
        qg_act_scale sc;
        sc.e = (int16_t)e;
        sc.m = (uint8_t)m;
        sc.pad = 0;
        scales[base / (GROUP_LANES * 4)] = sc;
        if (inf && err_flag) *err_flag = 1;
    }
}

}  // namespace

int launch_quantize(int mode, int block, int64_t n, int64_t cols, const float *x, int8_t *codes,
                    qg_act_scale *scales, int32_t *csums, int32_t *err_flag, hipStream_t s)
{
    (void)block;
    const int64_t nchunks = n * cols / 256;
    if (nchunks == 0) return QG_OK;
    const int64_t wgs = (nchunks + 3) / 4;
    if (mode == QG_PERBLOCK)
        hipLaunchKernelGGL(quantize_kernel<QG_PERBLOCK>, dim3((unsigned)wgs), dim3(kThreads), 0, s, x, nchunks,
                           codes, scales, csums, err_flag);
    else
        hipLaunchKernelGGL(quantize_kernel<QG_SUB32>, dim3((unsigned)wgs), dim3(kThreads), 0, s, x, nchunks,
                           codes, scales, csums, err_flag);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "quantize launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace qg
