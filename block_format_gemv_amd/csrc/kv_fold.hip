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

constexpr int kFoldChunk = 128;   // pieces a lane has in flight

// grid = ceil(total / 64) one-wave workgroups; lane t = h * HD + e folds the pieces of head h,
// element e from the workspace f32 [nh][nblk][HD] in chunks of 128 blocks: every load of a
// chunk issued first (a short last chunk reads block min(b, last) again, so that none waits on
// a branch), then the adds, each waiting only for its own piece (loads return in order).
// With per_kv > 0 (the workgroups of one KV head's query heads), workgroup i takes the
// elements of workgroup (i % nkv) * per_kv + i / nkv: the heads of KV head k then run on the XCD
// that wrote their pieces (the pieces kernel deals KV head k's workgroups to XCD k mod 8).
template <int HD>
__global__ __launch_bounds__(64) void kv_weighted_fold_kernel(int64_t total, int nblk, int nkv, int per_kv,
                                                              const float *__restrict__ pieces, float *__restrict__ out)
{
    const unsigned i = blockIdx.x;
    const int64_t w = per_kv > 0 ? (int64_t)(i % (unsigned)nkv) * per_kv + i / (unsigned)nkv : (int64_t)i;
    const int64_t t = w * 64 + threadIdx.x;
    if (t >= total) return;
    const int64_t h = t / HD;
    const float *p = pieces + ((size_t)h * (size_t)nblk * HD + (size_t)(t - h * HD));
    float y = 0.0f;
    // block counts in 32 bits (below 2^26): uniform compares and selects stay scalar
    for (int c0 = 0; c0 < nblk; c0 += kFoldChunk) {
        const int nb = min(nblk - c0, kFoldChunk);
        const float *pc = p + (size_t)c0 * HD;
        float a[kFoldChunk];
        if (nb == kFoldChunk) {
#pragma unroll
            for (int k = 0; k < kFoldChunk; k++) a[k] = pc[k * HD];
#pragma unroll
            for (int k = 0; k < kFoldChunk; k++) y = y + a[k];
        } else {
#pragma unroll
            for (int k = 0; k < kFoldChunk; k++) a[k] = pc[(size_t)min(k, nb - 1) * HD];
#pragma unroll
            for (int k = 0; k < kFoldChunk; k++) {
                const float z = y + a[k];
                y = k < nb ? z : y;
            }
        }
    }
    out[t] = (y != y) ? __uint_as_float(0x7FC00000u) : y;
}

}  // namespace

void launch_kv_fold_pieces(int64_t total, int hd, int64_t nblk, int64_t nkv, const float *pieces, float *out,
                           hipStream_t s)
{
    if (total == 0) return;
    const dim3 grid((unsigned)((total + 63) / 64)), block(64);
    // the workgroups per KV head: whole ones from head size 64 (total = nkv * grp * hd)
    const int per_kv = hd >= 64 ? (int)(total / nkv / 64) : 0;
    const int n = (int)nblk, g = (int)nkv;
    if (hd == 32) hipLaunchKernelGGL((kv_weighted_fold_kernel<32>), grid, block, 0, s, total, n, g, per_kv, pieces, out);
    else if (hd == 64) hipLaunchKernelGGL((kv_weighted_fold_kernel<64>), grid, block, 0, s, total, n, g, per_kv, pieces, out);
    else if (hd == 128) hipLaunchKernelGGL((kv_weighted_fold_kernel<128>), grid, block, 0, s, total, n, g, per_kv, pieces, out);
    else hipLaunchKernelGGL((kv_weighted_fold_kernel<256>), grid, block, 0, s, total, n, g, per_kv, pieces, out);
}

}  // namespace qg
