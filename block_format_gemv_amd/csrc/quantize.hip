// quantize.hip -- activation quantizer: per activation block the least scale m*2^e with
// 127*m*2^e >= the block's largest magnitude, the exact nearest-even codes, and the code
// sums of every run of 16 elements ("Module numerics" of
// logicaffeine_compile::spatial::decode_engine: Functions absmax, wide_scale, block_scale,
// rne_div, quantize, quantize_blocks; the activation side's unit sums of "Module lane").
//
// One wave covers 256 consecutive elements (one block of 256, or eight blocks of 32), four
// per lane; the per-lane arithmetic (quantize_lane) is shared with the fused
// quantize + GEMV kernel so both give the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kThreads = 256;

template <int BITS, int GROUP_LANES>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const float *__restrict__ x, int64_t nchunks,
                                                            int8_t *__restrict__ codes,
                                                            qg_act_scale *__restrict__ scales,
                                                            int32_t *__restrict__ csums,
                                                            int32_t *__restrict__ err_flag)
{
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (chunk >= nchunks) return;                         // wave-uniform
    const int64_t base = chunk * 256 + 4 * lane;
    const QuantLane q = quantize_lane<BITS, GROUP_LANES>(*reinterpret_cast<const float4 *>(x + base));
    *reinterpret_cast<uint32_t *>(codes + base) = q.packed;
    // sums of 16 consecutive codes = 4 lanes
    const int csum = quad_sum(q.sum4);
    if ((lane & 3) == 0) csums[base / 16] = csum;
    if ((lane & (GROUP_LANES - 1)) == 0) {
        qg_act_scale sc;
        sc.e = (int16_t)q.e;
        sc.m = (uint8_t)q.m;
        sc.pad = 0;
        scales[base / (GROUP_LANES * 4)] = sc;
        if (q.inf && err_flag) *err_flag = 1;
    }
}

}  // namespace

int launch_quantize(int mode, int block, int64_t n, int64_t cols, const float *x, int8_t *codes,
                    qg_act_scale *scales, int32_t *csums, int32_t *err_flag, hipStream_t s)
{
    const int64_t nchunks = n * cols / 256;
    if (nchunks == 0) return QG_OK;
    const int64_t wgs = (nchunks + 3) / 4;
    const dim3 grid((unsigned)wgs), threads(kThreads);
    if (mode == QG_PERBLOCK && block == 256)
        hipLaunchKernelGGL((quantize_kernel<8, 64>), grid, threads, 0, s, x, nchunks, codes, scales, csums, err_flag);
    else if (mode == QG_PERBLOCK)
        hipLaunchKernelGGL((quantize_kernel<8, 8>), grid, threads, 0, s, x, nchunks, codes, scales, csums, err_flag);
    else
        hipLaunchKernelGGL((quantize_kernel<4, 8>), grid, threads, 0, s, x, nchunks, codes, scales, csums, err_flag);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "quantize launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace qg
