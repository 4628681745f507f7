// pa_cache_write.hip -- the slot write: new tokens' K/V into their physical
// slots of the block-paged cache.
//
// Follows "PagedAttention实现" (write_kv: block = position / block_size,
// offset = position % block_size, copy the token's head_dim values into the
// block at that offset) with the slot of "04 - Paged Attention 实现进度"
// section A.2 / B.2 (slot = physical block * block_size + offset, one entry
// per new token).
//
// Layout: one thread moves one 16-byte chunk of one (token, KV head) row, for
// K and for V.  Consecutive threads take consecutive chunks of the source
// row, so both the read of k/v and the write into the (block, head, offset)
// row of the cache are fully coalesced 16-byte accesses; the row of a token
// is head_dim * elem_bytes contiguous bytes on both sides.  The copy is a
// plain bit copy (no conversion).  HBM-bound: it moves 2 * 2 * num_tokens *
// num_kv_heads * head_dim * elem_bytes bytes.
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4 *__restrict__ k, const uint4 *__restrict__ v, uint4 *__restrict__ k_cache,
    uint4 *__restrict__ v_cache, const int64_t *__restrict__ slot_mapping, int64_t total_chunks,
    int num_kv_heads, int log2_chunks_per_row, int log2_block, int64_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_chunks) return;
    const int chunk = (int)(i & ((1 << log2_chunks_per_row) - 1));
    const int64_t row = i >> log2_chunks_per_row;           // token * num_kv_heads + head
    const int64_t token = row / num_kv_heads;
    const int head = (int)(row - token * num_kv_heads);
    const int64_t slot = slot_mapping[token];
    if (slot < 0 || slot >= num_slots) return;              // padding token / out of range
    const int64_t block = slot >> log2_block;
    const int64_t offset = slot & ((1 << log2_block) - 1);
    const int64_t dst_row = ((block * num_kv_heads + head) << log2_block) + offset;
    const int64_t dst = (dst_row << log2_chunks_per_row) + chunk;
    k_cache[dst] = k[i];
    v_cache[dst] = v[i];
}

static int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) r++;
    return r;
}

hipError_t launch_cache_write(const void *k, const void *v, void *k_cache, void *v_cache,
                              const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                              int head_dim, int num_blocks, int log2_block, int elem_bytes,
                              hipStream_t stream) {
    const int chunks_per_row = head_dim * elem_bytes / 16;   // a power of two >= 2
    const int64_t row_bytes = (int64_t)head_dim * elem_bytes;
    const int threads = 256;
    // keep one launch's grid well inside the 32-bit work-item limit
    const int64_t max_tokens = ((int64_t)1 << 30) / ((int64_t)num_kv_heads * chunks_per_row);
    for (int64_t t0 = 0; t0 < num_tokens; t0 += max_tokens) {
        const int64_t n = num_tokens - t0 < max_tokens ? num_tokens - t0 : max_tokens;
        const int64_t total = n * num_kv_heads * chunks_per_row;
        const int64_t blocks = (total + threads - 1) / threads;
        const int64_t src_off = t0 * num_kv_heads * row_bytes;
        hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           (const uint4 *)((const char *)k + src_off),
                           (const uint4 *)((const char *)v + src_off), (uint4 *)k_cache,
                           (uint4 *)v_cache, slot_mapping + t0, total, num_kv_heads,
                           ilog2(chunks_per_row), log2_block, (int64_t)num_blocks << log2_block);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pa
