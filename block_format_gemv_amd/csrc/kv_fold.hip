// kv_fold.hip -- the second pass of the KV-cache weighted sum ("Module numerics" of
// logicaffeine_compile::spatial::decode_engine: Functions weighted_int8): out[h][e] is the
// pieces (h, 0, e), (h, 1, e), ... added in block order, each binary32 sum flushed.
//
// This file is built with binary32 subnormals flushed (preserve-sign: the kernel's FP mode
// flushes the results and operands of its f32 arithmetic to zeros of their sign).  The pieces
// and the running sums are zero or normal, so flushing operands changes nothing, and a sum of
// two such values that lands below 2^-126 is exact there, so the flush of the result is the
// flushed add of the sum's definition: one v_add_f32 per piece, nothing beside the chain.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int kFoldLanes = 64;    // (head, element) sums a workgroup
constexpr int kFoldRound = 128;   // blocks a round
constexpr int kFoldPer = kFoldRound * kFoldLanes / 256;   // pieces a thread loads per round

// grid = ceil(total / 64) workgroups of 256 threads; workgroup x folds the sums t = 64x + i
// (i < 64; head t / hd, element t % hd) over the workspace f32 [nh][nblk][hd].  Per round of up
// to 128 blocks every thread loads 32 pieces (a wave's load: one block's 64 sums), all in
// flight together, into LDS [block][i]; after the barrier wave 0 adds them in block order.
__global__ __launch_bounds__(256) void kv_weighted_fold_kernel(int64_t total, int hd, int64_t nblk,
                                                               const float *__restrict__ pieces,
                                                               float *__restrict__ out)
{
    __shared__ float s_p[kFoldRound * kFoldLanes];
    const int tid = threadIdx.x;
    const int i = tid & (kFoldLanes - 1);
    const int64_t t = (int64_t)blockIdx.x * kFoldLanes + i;
    const bool live = t < total;
    const int64_t h = live ? t / hd : 0;
    const float *p = pieces + ((size_t)h * nblk * hd + (size_t)(live ? t - h * hd : 0));
    float y = 0.0f;
    for (int64_t r0 = 0; r0 < nblk; r0 += kFoldRound) {
        const int nb = (int)(nblk - r0 < kFoldRound ? nblk - r0 : kFoldRound);
        float v[kFoldPer];
#pragma unroll
        for (int j = 0; j < kFoldPer; j++) {
            const int b = (tid >> 6) + 4 * j;                  // block within the round
            v[j] = (live && b < nb) ? p[(size_t)(r0 + b) * hd] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kFoldPer; j++) s_p[((tid >> 6) + 4 * j) * kFoldLanes + i] = v[j];
        __syncthreads();
        if (tid < kFoldLanes && nb == kFoldRound) {
            // a whole round: every LDS read issued ahead of the adds it feeds
            float a[kFoldRound];
#pragma unroll
            for (int k = 0; k < kFoldRound; k++) a[k] = s_p[k * kFoldLanes + i];
#pragma unroll
            for (int k = 0; k < kFoldRound; k++) y = y + a[k];
        } else if (tid < kFoldLanes) {
            int b = 0;
            for (; b + 8 <= nb; b += 8) {
                float a[8];
#pragma unroll
                for (int k = 0; k < 8; k++) a[k] = s_p[(b + k) * kFoldLanes + i];
#pragma unroll
                for (int k = 0; k < 8; k++) y = y + a[k];
            }
            for (; b < nb; b++) y = y + s_p[b * kFoldLanes + i];
        }
        __syncthreads();
    }
    if (tid < kFoldLanes && live) out[t] = (y != y) ? __uint_as_float(0x7FC00000u) : y;
}

}  // namespace

void launch_kv_fold_pieces(int64_t total, int hd, int64_t nblk, const float *pieces, float *out, hipStream_t s)
{
    if (total == 0) return;
    hipLaunchKernelGGL(kv_weighted_fold_kernel, dim3((unsigned)((total + kFoldLanes - 1) / kFoldLanes)), dim3(256), 0, s,
                       total, hd, nblk, pieces, out);
}

}  // namespace qg
