// stream.hip -- a plain streaming read with the GEMV's memory access pattern, to measure
// what the hardware delivers to one launch: every wave reads nine contiguous 1 KiB chunks
// (the size of one Q4_K-style tile) with non-temporal 16-byte loads and folds them by XOR.
// No arithmetic of the method runs here; it is the ceiling the GEMV is compared against.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kChunk = 1024;
constexpr int kChunksPerWave = 9;
constexpr int kWaves = 16;

__global__ __launch_bounds__(64 * kWaves) void stream_read_kernel(const uint8_t *buf, int64_t nchunks, uint32_t magic,
                                                                  uint32_t *__restrict__ sink)
{
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
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

}  // namespace qg
