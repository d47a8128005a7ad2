// stream.hip -- plain streaming reads, to measure what the hardware delivers to one launch.
// No arithmetic of the method runs here; they are the ceilings the GEMV is compared against.
//
// stream_read_kernel reads with the GEMV's memory access pattern: every wave reads nine
// contiguous 1 KiB chunks (the size of one Q4_K-style tile) with non-temporal 16-byte loads
// and folds them by XOR.  stream_read_shape_kernel reads in a chosen launch geometry (waves
// per workgroup, KiB per wave per pass, one pass or a grid-stride loop over a given number of
// workgroups, non-temporal or ordinary loads), for a sweep of launch shapes.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kChunk = 1024;
constexpr int kChunksPerWave = 9;
constexpr int kWaves = 16;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64 * kWaves) void stream_read_kernel(const uint8_t *buf, int64_t nchunks, uint32_t magic,
                                                                  uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t c0 = wave * kChunksPerWave;
    v4u r[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; i++) {
        const int64_t c = c0 + i < nchunks ? c0 + i : nchunks - 1;     // clamped into the buffer
        r[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(buf + c * kChunk + 16 * lane));
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kChunksPerWave; i++)
        if (c0 + i < nchunks) x ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    // written only when a lane's fold meets the caller's value, so the loads cannot be dropped
    if (x == magic) sink[0] = x;
}

// K chunks of 1 KiB per wave per pass, all K loads issued before any is used; wave v of the
// launch reads chunks v*K .. v*K+K-1, then (grid-stride) those `stride` waves further on
template <int K, bool NT>
__global__ __launch_bounds__(1024) void stream_read_shape_kernel(const uint8_t *buf, int64_t nchunks, int64_t stride,
                                                                 uint32_t magic, uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    uint32_t x = 0;
    for (int64_t c0 = wave * K; c0 < nchunks; c0 += stride * K) {
        v4u r[K];
#pragma unroll
        for (int i = 0; i < K; i++) {
            const int64_t c = c0 + i < nchunks ? c0 + i : nchunks - 1;
            const v4u *p = reinterpret_cast<const v4u *>(buf + c * kChunk + 16 * lane);
            r[i] = NT ? __builtin_nontemporal_load(p) : *p;
        }
#pragma unroll
        for (int i = 0; i < K; i++)
            if (c0 + i < nchunks) x ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    }
    if (x == magic) sink[0] = x;
}

template <int K, bool NT>
void launch_shape_typed(dim3 grid, dim3 block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const uint8_t *buf,
                        int64_t nchunks, int64_t stride, uint32_t magic, uint32_t *sink)
{
    if (ev0 && ev1)
        hipExtLaunchKernelGGL((stream_read_shape_kernel<K, NT>), grid, block, 0, s, ev0, ev1, 0, buf, nchunks, stride,
                              magic, sink);
    else
        hipLaunchKernelGGL((stream_read_shape_kernel<K, NT>), grid, block, 0, s, buf, nchunks, stride, magic, sink);
}

template <bool NT>
int launch_shape_k(int k, dim3 grid, dim3 block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const uint8_t *buf,
                   int64_t nchunks, int64_t stride, uint32_t magic, uint32_t *sink)
{
    switch (k) {
    case 1: launch_shape_typed<1, NT>(grid, block, s, ev0, ev1, buf, nchunks, stride, magic, sink); break;
    case 2: launch_shape_typed<2, NT>(grid, block, s, ev0, ev1, buf, nchunks, stride, magic, sink); break;
    case 4: launch_shape_typed<4, NT>(grid, block, s, ev0, ev1, buf, nchunks, stride, magic, sink); break;
    case 8: launch_shape_typed<8, NT>(grid, block, s, ev0, ev1, buf, nchunks, stride, magic, sink); break;
    case 9: launch_shape_typed<9, NT>(grid, block, s, ev0, ev1, buf, nchunks, stride, magic, sink); break;
    case 16: launch_shape_typed<16, NT>(grid, block, s, ev0, ev1, buf, nchunks, stride, magic, sink); break;
    default: return fail(QG_E_INVALID, "qg_stream_read_shape: %d KiB per wave is not one of 1, 2, 4, 8, 9, 16", k);
    }
    return QG_OK;
}

}  // namespace

int launch_stream_read(const void *buf, size_t bytes, uint32_t magic, uint32_t *sink, hipStream_t s)
{
    const int64_t nchunks = (int64_t)(bytes / kChunk);
    if (nchunks == 0) return QG_OK;
    const int64_t waves = (nchunks + kChunksPerWave - 1) / kChunksPerWave;
    const int64_t wgs = (waves + kWaves - 1) / kWaves;
    if (wgs > 0x7fffffff) return fail(QG_E_SHAPE, "qg_stream_read: %zu bytes is too many", bytes);
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    if (ev0 && ev1)
        hipExtLaunchKernelGGL(stream_read_kernel, dim3((unsigned)wgs), dim3(64 * kWaves), 0, s, ev0, ev1, 0,
                              static_cast<const uint8_t *>(buf), nchunks, magic, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)wgs), dim3(64 * kWaves), 0, s,
                           static_cast<const uint8_t *>(buf), nchunks, magic, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "stream read launch: %s", hipGetErrorString(e));
    return QG_OK;
}

int launch_stream_read_shape(const void *buf, size_t bytes, int waves_per_wg, int kib_per_wave, int64_t wgs,
                             int flags, uint32_t magic, uint32_t *sink, hipStream_t s)
{
    const int64_t nchunks = (int64_t)(bytes / kChunk);
    if (nchunks == 0) return QG_OK;
    const int64_t k = kib_per_wave;
    const int64_t waves_needed = (nchunks + k - 1) / k;
    const int64_t grid = wgs > 0 ? wgs : (waves_needed + waves_per_wg - 1) / waves_per_wg;
    if (grid > 0x7fffffff) return fail(QG_E_SHAPE, "qg_stream_read_shape: %lld workgroups is too many", (long long)grid);
    const int64_t stride = grid * waves_per_wg;    // waves in the launch
    hipEvent_t ev0, ev1;
    take_timing_events(&ev0, &ev1);
    const dim3 g((unsigned)grid), b((unsigned)(64 * waves_per_wg));
    const uint8_t *p = static_cast<const uint8_t *>(buf);
    const int st = (flags & 1) ? launch_shape_k<false>(kib_per_wave, g, b, s, ev0, ev1, p, nchunks, stride, magic, sink)
                               : launch_shape_k<true>(kib_per_wave, g, b, s, ev0, ev1, p, nchunks, stride, magic, sink);
    if (st != QG_OK) return st;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_E_RUNTIME, "stream read launch: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace qg
