// pa_internal.h -- shared declarations of the paged-decode library's
// kernels and launchers (not installed; the public ABI is include/pa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Work-balanced split (matrix-core path): head slots reserved per partial
// (the largest supported group).
constexpr int kMaxGroup = 16;

// Everything a decode kernel needs, passed by value as one kernel argument.
struct DecodeParams {
    void *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float *ws_m;              // [B][Hq][NP]       (split mode only;
    float *ws_l;              // [B][Hq][NP]        balanced mode: [W][2][16],
    float *ws_acc;            // [B][Hq][NP][D]     [W][2][16], [W][2][16][D])
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;                // num_q_heads / num_kv_heads
    int num_blocks;
    int log2_block;           // block_size = 1 << log2_block
    int max_blocks_per_seq;
    int max_context_len;
    int partition_size;       // tokens per work unit (single pass: >= max_context_len)
    int num_partitions;       // NP
    float scale_log2;         // scale * log2(e): scores are kept in base-2 log domain
    int num_units;            // wavefronts: NP * Hkv * B (grid), or W (persistent)
    int persistent;           // matrix-core path: num_units persistent wavefronts share
                              // the tile stream; partition_size 0 = free cuts
};

struct ReduceParams {
    void *out;
    const int32_t *context_lens;
    const float *ws_m;
    const float *ws_l;
    const float *ws_acc;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int head_dim;
    int max_context_len;
    int partition_size;
    int num_partitions;
    int num_waves;            // balanced mode: wavefronts of the decode kernel
};

// Shared-prefix decode (matrix-core path): packs of `pack` consecutive
// sequences share one wavefront's 32 columns (two groups of 16).
struct SharedParams {
    void *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_blocks;
    int log2_block;
    int max_blocks_per_seq;
    int max_context_len;
    float scale_log2;
    int pack;                 // sequences per pack
    int num_packs;            // ceil(num_seqs / pack)
    int max_tiles;            // ceil(max_context_len / 16)
    int num_waves;            // persistent wavefronts
    int *ws_cost;             // [num_packs] items (distinct tiles) per pack
    int *ws_items;            // [num_packs][pack * max_tiles] item records, 4 ints each
    float *ws_m;              // [W][2][32]
    float *ws_l;              // [W][2][32]
    float *ws_acc;            // [W][2][32][128]
};

struct PrefillParams {
    void *out;                 // [total_q][Hq][D]
    const void *q;             // [total_q][Hq][D]
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *cu_seqlens_q;   // [B + 1]
    const int32_t *context_lens;   // [B], after the chunk's write
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_blocks;
    int log2_block;
    int max_blocks_per_seq;
    int max_context_len;
    int units_per_seq;         // wavefronts per (sequence, KV head): ceil(max_q_len / rows per wavefront)
    float scale_log2;
};

// Query-head columns of one shared-prefix wavefront: two groups of 16.
constexpr int kMaxCols = 32;

// Work-unit numbering shared by the decode kernels.  Workgroups are handed
// to the 8 XCDs round-robin (workgroup w runs on XCD w % 8); this remaps the
// workgroup id so that consecutive logical units run on the same XCD at about
// the same time.  Units are numbered with the sequence fastest, so the
// samples of one prompt (adjacent sequences sharing prefix blocks) reading
// the same (KV head, partition) meet in one XCD's L2.
//
// The persistent kernels do not remap: their shares of the tile stream (KV
// head slowest) would then put one KV head's slices of every block on one
// XCD, and an XCD reading a single head's slices drew unevenly on the HBM
// channels -- one XCD ran 5% behind the rest and set the kernel's end.  In
// launch order the eight XCDs take shares from all heads alike.
__device__ __forceinline__ int xcd_remap(int w, int n) {
    const int q = n / kNumXcd, r = n % kNumXcd;
    const int x = w % kNumXcd, slot = w / kNumXcd;
    return x * q + (x < r ? x : r) + slot;
}

struct Unit {
    int b, g, part;
};

__device__ __forceinline__ Unit unit_of(int u, int num_seqs, int num_kv_heads) {
    Unit t;
    t.b = u % num_seqs;
    const int rest = u / num_seqs;
    t.g = rest % num_kv_heads;
    t.part = rest / num_kv_heads;
    return t;
}

__device__ __forceinline__ int clamp_ctx(int n, int max_context_len) {
    return n < 0 ? 0 : (n > max_context_len ? max_context_len : n);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Launchers: validate nothing (pa_api.cpp does), enqueue, return hipError_t.
hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream);
// query-head columns one matrix-core prefill wavefront serves (the 32
// columns of the 32x32x16 product)
constexpr int kPrefillColumns = 32;
// Prefill on the vector ALUs (every dtype / head_dim / block size): chunk rows
// per wavefront for a group size, and the launch.
int prefill_vector_rows(int group, int dtype);
hipError_t launch_prefill_vector(const PrefillParams &p, int head_dim, int dtype,
                                 hipStream_t stream);
hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int num_pairs,
                              int num_blocks, int64_t block_bytes, hipStream_t stream);
hipError_t launch_cache_write(const void *k, const void *v, void *k_cache, void *v_cache,
                              const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                              int head_dim, int num_blocks, int log2_block, int elem_bytes,
                              hipStream_t stream);

hipError_t launch_decode_vector(const DecodeParams &p, int head_dim, int dtype,
                                hipStream_t stream);
// Work-balanced split on the vector ALUs (same stream, slots and merge as the
// matrix-core balanced split); for block_size >= 16 and head dims whose
// 16-token tile covers whole 64-lane load passes.
bool vector_balanced_supported(int head_dim, int dtype, int block_size);
hipError_t launch_decode_vector_balanced(const DecodeParams &p, int head_dim, int dtype,
                                         hipStream_t stream);

hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t stream);

hipError_t launch_reduce(const ReduceParams &p, int dtype, hipStream_t stream);

hipError_t launch_reduce_balanced(const ReduceParams &p, int dtype, hipStream_t stream);

// phase bit 1: plan + decode kernels; bit 2: merge kernel.
hipError_t launch_decode_shared(const SharedParams &p, int phase, hipStream_t stream);

// Most partitions a fixed-partition split may have (their merge weights sit
// in the merge kernel's LDS).
constexpr int kMaxPartitions = 8192;

}  // namespace pa
