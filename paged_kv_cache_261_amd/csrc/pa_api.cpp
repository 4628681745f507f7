// pa_api.cpp -- the C ABI of include/pa.h: host-side validation, choice of
// kernel and partitioning, and kernel launches on the caller's stream.
// Nothing here allocates device memory or synchronises.
#include "pa.h"

#include <atomic>
#include <initializer_list>
#include <math.h>
#include <mutex>

#include "pa_internal.h"

// Scratch of pa_decode_noalloc: one file-scope device array, so every GPU
// the library runs on holds its own copy (PA_NOALLOC_SCRATCH_BYTES) until
// the process ends.  In host code `scratch` is only a stand-in for the
// symbol: its device address on each GPU comes from hipGetSymbolAddress
// (scratch_on below) and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) r++;
    return r;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

bool block_size_ok(int bs) { return is_pow2(bs) && bs <= 256; }

bool dtype_ok(int dtype) { return dtype == PA_F32 || dtype == PA_BF16; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Wavefronts of the work-balanced split: one per SIMD of an MI355X (256 CUs x
// 4 SIMDs), all resident at once.  Measured on the bf16 GQA workloads, 1024
// long streams beat 2048 or more shorter ones.
#ifndef PA_BALANCED_WAVES
#define PA_BALANCED_WAVES 1024
#endif
constexpr int kBalancedWaves = PA_BALANCED_WAVES;
#ifndef PA_SHARED_WAVES
#define PA_SHARED_WAVES 1024
#endif
constexpr int kSharedWaves = PA_SHARED_WAVES;

// Sequences per pack in shared-prefix mode: the largest power of two, at
// most 8, whose query heads fit the 32 columns of a wavefront.
int pack_of(int group) {
    int k = 8;
    while (k > 1 && k * group > pa::kMaxCols) k >>= 1;
    return k;
}

bool is_split_mode(int partition) {
    return partition == PA_PARTITION_BALANCED || partition == PA_PARTITION_SHARED;
}

bool balanced_applies(int dtype, int head_dim, int block_size, int num_q_heads,
                      int num_kv_heads) {
    return dtype == PA_BF16 && head_dim == 128 && block_size >= 16 && num_kv_heads > 0 &&
           num_q_heads % num_kv_heads == 0 && num_q_heads / num_kv_heads <= 16;
}

// The work-balanced split on the vector ALUs (any dtype; block_size >= 16;
// head dims whose 16-token tile covers whole 64-lane load passes).
bool vector_balanced_applies(int dtype, int head_dim, int block_size, int num_q_heads,
                             int num_kv_heads) {
    return head_dim_ok(head_dim) && dtype_ok(dtype) && block_size_ok(block_size) &&
           pa::vector_balanced_supported(head_dim, dtype == PA_BF16 ? 1 : 0, block_size) &&
           num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 &&
           num_q_heads / num_kv_heads <= 16;
}

// Either balanced split applies.
bool any_balanced_applies(int dtype, int head_dim, int block_size, int num_q_heads,
                          int num_kv_heads) {
    return balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads) ||
           vector_balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads);
}

// Partition size for the vector kernel (one wavefront per (sequence, KV
// head, partition)): small enough that about kVectorWaves wavefronts have
// work when every context is max_context_len long -- the kernel hides
// memory latency by occupancy -- but at least 64 tokens, at most 512, a
// power of two and a multiple of block_size.  Small problems run in one
// pass (the merge would cost more than it saves).
constexpr int64_t kVectorWaves = 8192;

int vector_partition(int num_seqs, int num_kv_heads, int block_size, int max_context_len) {
    const int64_t work = (int64_t)max_context_len * num_seqs * num_kv_heads;
    if (work <= 64 * 1024) return 0;
    int p = 64;
    while (p < 512 && (int64_t)p * kVectorWaves < work) p <<= 1;
    if (p < block_size) p = block_size;
    return max_context_len > p ? p : 0;
}

// Resolve the partition size: 0 = single pass, PA_PARTITION_BALANCED, or a
// multiple of block_size.
int resolve_partition(int partition_size, int num_seqs, int num_q_heads, int num_kv_heads,
                      int head_dim, int block_size, int max_context_len, int dtype, int algo) {
    if (partition_size != PA_PARTITION_AUTO) return partition_size;
    const int p = pa_decode_auto_partition(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           block_size, max_context_len, dtype);
    if (p == PA_PARTITION_BALANCED && algo == PA_ALGO_VECTOR &&
        !vector_balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads))
        return vector_partition(num_seqs, num_kv_heads, block_size, max_context_len);
    return p;
}

struct WorkspaceLayout {
    size_t m_off, l_off, acc_off, total;
    size_t cost_off, pos_off;            // shared-prefix mode
    int num_partitions;
    int pack, num_packs, max_tiles;      // shared-prefix mode
};

WorkspaceLayout layout(int num_seqs, int num_q_heads, int head_dim, int max_context_len,
                       int partition, int group = 1) {
    WorkspaceLayout w{};
    if (partition == PA_PARTITION_SHARED) {
        // cost [P] | items [P][pack * max_tiles][4] | m, l [W][2][32] |
        // acc [W][2][32][head_dim]
        const size_t slots = (size_t)kSharedWaves * 2 * pa::kMaxCols;
        w.pack = pack_of(group);
        w.num_packs = (num_seqs + w.pack - 1) / w.pack;
        w.max_tiles = (max_context_len + 15) / 16;
        w.cost_off = 0;
        w.pos_off = round256((size_t)w.num_packs * sizeof(int32_t));
        w.m_off = w.pos_off + round256((size_t)w.num_packs * w.pack * w.max_tiles * 4 *
                                       sizeof(int32_t));
        w.l_off = w.m_off + round256(slots * sizeof(float));
        w.acc_off = w.l_off + round256(slots * sizeof(float));
        w.total = w.acc_off + round256(slots * head_dim * sizeof(float));
        return w;
    }
    if (partition == PA_PARTITION_BALANCED) {
        // m [W][2][16] | l [W][2][16] | acc [W][2][16][head_dim]
        const size_t slots = (size_t)kBalancedWaves * 2 * pa::kMaxGroup;
        w.num_partitions = 0;
        w.m_off = 0;
        w.l_off = w.m_off + round256(slots * sizeof(float));
        w.acc_off = w.l_off + round256(slots * sizeof(float));
        w.total = w.acc_off + round256(slots * head_dim * sizeof(float));
        return w;
    }
    w.num_partitions = max_context_len <= 0 ? 1 : (max_context_len + partition - 1) / partition;
    const size_t rows = (size_t)num_seqs * num_q_heads * w.num_partitions;
    w.m_off = 0;
    w.l_off = round256(rows * sizeof(float));
    w.acc_off = w.l_off + round256(rows * sizeof(float));
    w.total = w.acc_off + round256(rows * head_dim * sizeof(float));
    return w;
}

struct DecodeArgs {
    void *out;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_tables, *context_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size;
    int max_blocks_per_seq, max_context_len;
    float scale;
    int dtype, algo;
};

int validate_decode(const DecodeArgs &a) {
    if (a.num_seqs < 0 || a.num_q_heads <= 0 || a.num_kv_heads <= 0 || a.num_blocks <= 0 ||
        a.max_blocks_per_seq <= 0 || a.max_context_len < 0)
        return PA_ERR_SHAPE;
    if (!dtype_ok(a.dtype) || !head_dim_ok(a.head_dim) || !block_size_ok(a.block_size))
        return PA_ERR_UNSUPPORTED;
    if (a.num_q_heads % a.num_kv_heads != 0) return PA_ERR_SHAPE;
    if (a.num_q_heads / a.num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
    if ((int64_t)a.max_context_len > (int64_t)a.max_blocks_per_seq * a.block_size)
        return PA_ERR_SHAPE;
    if (a.algo != PA_ALGO_AUTO && a.algo != PA_ALGO_VECTOR && a.algo != PA_ALGO_MFMA)
        return PA_ERR_ALGO;
    if (a.num_seqs == 0) return PA_OK;
    if (!a.out || !a.q || !a.k_cache || !a.v_cache || !a.block_tables || !a.context_lens)
        return PA_ERR_NULL;
    if (!aligned16(a.out) || !aligned16(a.q) || !aligned16(a.k_cache) || !aligned16(a.v_cache))
        return PA_ERR_ALIGN;
    return PA_OK;
}

bool mfma_applies(const DecodeArgs &a) {
    return a.dtype == PA_BF16 && a.head_dim == 128 && a.block_size >= 16 &&
           a.num_q_heads / a.num_kv_heads <= 16;
}

bool vector_balanced_applies(const DecodeArgs &a) {
    return vector_balanced_applies(a.dtype, a.head_dim, a.block_size, a.num_q_heads,
                                   a.num_kv_heads);
}

// Which kernel runs the work-balanced split: the matrix cores unless the
// caller asks for the vector ALUs (or the shape needs them).  -1: neither
// applies.
int balanced_kernel(const DecodeArgs &a) {
    if (a.algo != PA_ALGO_VECTOR && mfma_applies(a)) return PA_ALGO_MFMA;
    if (a.algo != PA_ALGO_MFMA && vector_balanced_applies(a)) return PA_ALGO_VECTOR;
    return -1;
}

// The kernels of a resolved split mode can run these arguments: PA_OK, or
// why not.
int check_split_mode(const DecodeArgs &a, int partition) {
    if (partition == PA_PARTITION_SHARED) {
        if (!mfma_applies(a) || a.algo == PA_ALGO_VECTOR) return PA_ERR_ALGO;
    } else if (partition == PA_PARTITION_BALANCED) {
        if (balanced_kernel(a) < 0) return PA_ERR_ALGO;
    } else if (partition <= 0 || partition % a.block_size) {
        return PA_ERR_SHAPE;
    }
    return PA_OK;
}

// Phase 1 (or the whole decode when num_partitions == 1).
int launch_units(const DecodeArgs &a, int partition, int num_partitions, float *ws_m,
                 float *ws_l, float *ws_acc, hipStream_t stream) {
    const bool balanced = partition == PA_PARTITION_BALANCED;
    bool use_mfma;
    if (balanced) {
        const int k = balanced_kernel(a);
        if (k < 0) return PA_ERR_ALGO;
        use_mfma = k == PA_ALGO_MFMA;
    } else if (a.algo == PA_ALGO_MFMA) {
        if (!mfma_applies(a)) return PA_ERR_ALGO;
        use_mfma = true;
    } else {
        use_mfma = a.algo == PA_ALGO_AUTO && mfma_applies(a);
    }
    // Matrix-core path: single pass runs one wavefront per (sequence, KV
    // head); every split runs the persistent wavefronts.  Vector path: the
    // balanced split runs the persistent wavefronts, fixed partitions and
    // the single pass one wavefront per (sequence, KV head, partition).
    const bool persistent = (use_mfma && num_partitions != 1) || (!use_mfma && balanced);
    const int64_t units = persistent ? kBalancedWaves
                                     : (int64_t)num_partitions * a.num_kv_heads * a.num_seqs;
    if (units > 0x7fffffff) return PA_ERR_SHAPE;
    pa::DecodeParams p{};
    p.out = a.out;
    p.q = a.q;
    p.k_cache = a.k_cache;
    p.v_cache = a.v_cache;
    p.block_tables = a.block_tables;
    p.context_lens = a.context_lens;
    p.ws_m = ws_m;
    p.ws_l = ws_l;
    p.ws_acc = ws_acc;
    p.num_seqs = a.num_seqs;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.num_q_heads / a.num_kv_heads;
    p.num_blocks = a.num_blocks;
    p.log2_block = ilog2(a.block_size);
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.max_context_len = a.max_context_len;
    p.partition_size = balanced ? 0 : partition;
    p.num_partitions = num_partitions;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    p.num_units = (int)units;
    p.persistent = persistent ? 1 : 0;

    const hipError_t e =
        use_mfma ? pa::launch_decode_mfma(p, stream)
        : balanced ? pa::launch_decode_vector_balanced(p, a.head_dim, a.dtype, stream)
                   : pa::launch_decode_vector(p, a.head_dim, a.dtype, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa::SharedParams shared_params(const DecodeArgs &a, const WorkspaceLayout &w, char *ws) {
    pa::SharedParams p{};
    p.out = a.out;
    p.q = a.q;
    p.k_cache = a.k_cache;
    p.v_cache = a.v_cache;
    p.block_tables = a.block_tables;
    p.context_lens = a.context_lens;
    p.num_seqs = a.num_seqs;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.num_q_heads / a.num_kv_heads;
    p.num_blocks = a.num_blocks;
    p.log2_block = ilog2(a.block_size);
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.max_context_len = a.max_context_len;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    p.pack = w.pack;
    p.num_packs = w.num_packs;
    p.max_tiles = w.max_tiles;
    p.num_waves = kSharedWaves;
    p.ws_cost = (int *)(ws + w.cost_off);
    p.ws_items = (int *)(ws + w.pos_off);
    p.ws_m = (float *)(ws + w.m_off);
    p.ws_l = (float *)(ws + w.l_off);
    p.ws_acc = (float *)(ws + w.acc_off);
    return p;
}

// Device address of `scratch` on each device, looked up once per device
// with that device current.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

hipError_t scratch_on(int device, void **ptr) {
    void *p = g_scratch[device].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[device].load(std::memory_order_relaxed);
        if (!p) {
            int current = -1;
            hipError_t e = hipGetDevice(&current);
            if (e != hipSuccess) return e;
            if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (current != device) {
                const hipError_t back = hipSetDevice(current);
                if (e == hipSuccess) e = back;
            }
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[device].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *pa_status_string(int status) {
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes inconsistent or out of range";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype or group size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_ALGO: return "requested kernel variant does not support this shape";
    case PA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case PA_ERR_SCRATCH:
        return "the problem needs more workspace than the library's static scratch holds";
    default: return "unknown status";
    }
}

int pa_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                         const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int num_blocks, int block_size, int dtype, void *stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || !block_size_ok(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGN;
    const hipError_t e = pa::launch_cache_write(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                                num_kv_heads, head_dim, num_blocks,
                                                ilog2(block_size), dtype == PA_BF16 ? 2 : 4,
                                                (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_pairs, int num_pairs,
                   int num_blocks, int num_kv_heads, int block_size, int head_dim, int dtype,
                   void *stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || !block_size_ok(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !block_pairs) return PA_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
    const int64_t block_bytes =
        (int64_t)num_kv_heads * block_size * head_dim * (dtype == PA_BF16 ? 2 : 4);
    if (block_bytes % 16) return PA_ERR_UNSUPPORTED;
    const hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, block_pairs, num_pairs,
                                                num_blocks, block_bytes, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, const int32_t *cu_seqlens_q,
               const int32_t *context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
               int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
               int max_context_len, int max_q_len, float scale, int dtype, void *stream) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0 || max_context_len < 0 || max_q_len < 0 ||
        num_q_heads % num_kv_heads)
        return PA_ERR_SHAPE;
    if (!dtype_ok(dtype) || !head_dim_ok(head_dim) || !block_size_ok(block_size) ||
        num_q_heads / num_kv_heads > 16)
        return PA_ERR_UNSUPPORTED;
    // the matrix-core kernel where its tile applies (it folds a positive
    // scale into the exponent), the vector ALUs elsewhere
    const bool mfma = balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads) &&
                      scale > 0.f;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size ||
        max_q_len > max_context_len)
        return PA_ERR_SHAPE;
    if (num_seqs == 0 || max_q_len == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens_q || !context_lens)
        return PA_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGN;
    pa::PrefillParams p{};
    p.out = out;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.cu_seqlens_q = cu_seqlens_q;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.num_blocks = num_blocks;
    p.log2_block = ilog2(block_size);
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    const int rows_per_wave = mfma ? pa::kPrefillColumns / p.group
                                   : pa::prefill_vector_rows(p.group, dtype);
    p.units_per_seq = (max_q_len + rows_per_wave - 1) / rows_per_wave;
    p.scale_log2 = scale * 1.4426950408889634f;
    // the grid: (sequence, KV head) groups, rounded up to whole rounds of
    // XCDs on the matrix-core path, times the row blocks of a chunk
    const int64_t groups = (int64_t)num_seqs * num_kv_heads;
    const int64_t padded = mfma ? (groups + pa::kNumXcd - 1) / pa::kNumXcd * pa::kNumXcd : groups;
    if (padded * p.units_per_seq > 0x7fffffff) return PA_ERR_SHAPE;
    const hipError_t e = mfma ? pa::launch_prefill(p, (hipStream_t)stream)
                              : pa::launch_prefill_vector(p, head_dim, dtype, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode_auto_partition(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_context_len, int dtype) {
    if (!block_size_ok(block_size)) return 0;
    if (balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads))
        return PA_PARTITION_BALANCED;
    const int p = vector_partition(num_seqs, num_kv_heads, block_size, max_context_len);
    if (p > 0 && vector_balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads))
        return PA_PARTITION_BALANCED;
    return p;
}

size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_context_len, int partition_size,
                                int dtype) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || !block_size_ok(block_size))
        return 0;
    if (partition_size == PA_PARTITION_AUTO) {
        // enough for whichever mode pa_decode picks (it may depend on algo)
        size_t best = 0;
        const int p = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads,
                                        head_dim, block_size, max_context_len, dtype,
                                        PA_ALGO_AUTO);
        const int pv = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads,
                                         head_dim, block_size, max_context_len, dtype,
                                         PA_ALGO_VECTOR);
        for (int q : {p, pv})
            if (is_split_mode(q) || (q > 0 && q % block_size == 0)) {
                const size_t n = layout(num_seqs, num_q_heads, head_dim, max_context_len, q).total;
                best = n > best ? n : best;
            }
        return best;
    }
    const int partition = partition_size;
    if (partition == PA_PARTITION_SHARED) {
        if (!balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads)) return 0;
    } else if (partition == PA_PARTITION_BALANCED) {
        if (!any_balanced_applies(dtype, head_dim, block_size, num_q_heads, num_kv_heads))
            return 0;
    } else if (partition <= 0 || partition % block_size) {
        return 0;
    }
    return layout(num_seqs, num_q_heads, head_dim, max_context_len, partition,
                  num_q_heads / num_kv_heads)
        .total;
}

int pa_decode_partitions(void *out, const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int num_blocks, int block_size, int max_blocks_per_seq,
                         int max_context_len, float scale, int partition_size,
                         void *workspace, size_t workspace_bytes, int dtype, int algo,
                         void *stream) {
    const DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       max_blocks_per_seq, max_context_len, scale, dtype, algo};
    int rc = validate_decode(a);
    if (rc != PA_OK) return rc;
    const int partition = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads,
                                            head_dim, block_size, max_context_len, dtype, algo);
    rc = check_split_mode(a, partition);
    if (rc != PA_OK) return rc;
    if (num_seqs == 0) return PA_OK;
    const WorkspaceLayout w = layout(num_seqs, num_q_heads, head_dim, max_context_len, partition,
                                     num_q_heads / num_kv_heads);
    if (w.num_partitions > pa::kMaxPartitions) return PA_ERR_SHAPE;
    if (!workspace || workspace_bytes < w.total) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ALIGN;
    char *ws = (char *)workspace;
    if (partition == PA_PARTITION_SHARED) {
        const hipError_t e =
            pa::launch_decode_shared(shared_params(a, w, ws), 1, (hipStream_t)stream);
        return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    return launch_units(a, partition, w.num_partitions, (float *)(ws + w.m_off),
                        (float *)(ws + w.l_off), (float *)(ws + w.acc_off), (hipStream_t)stream);
}

int pa_decode_reduce(void *out, const int32_t *context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int max_context_len, int partition_size,
                     const void *workspace, size_t workspace_bytes, int dtype, void *stream) {
    const bool balanced = is_split_mode(partition_size);
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
        (partition_size <= 0 && !balanced) || num_q_heads % num_kv_heads)
        return PA_ERR_SHAPE;
    if (!dtype_ok(dtype) || !head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
    if (balanced && num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
    if (partition_size == PA_PARTITION_SHARED && (head_dim != 128 || dtype != PA_BF16))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!out || !context_lens) return PA_ERR_NULL;
    const WorkspaceLayout w = layout(num_seqs, num_q_heads, head_dim, max_context_len,
                                     partition_size, num_q_heads / num_kv_heads);
    if (w.num_partitions > pa::kMaxPartitions) return PA_ERR_SHAPE;
    if (!workspace || workspace_bytes < w.total) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace) || !aligned16(out)) return PA_ERR_ALIGN;
    const char *ws = (const char *)workspace;
    if (partition_size == PA_PARTITION_SHARED) {
        DecodeArgs a{};
        a.out = out;
        a.context_lens = context_lens;
        a.num_seqs = num_seqs;
        a.num_q_heads = num_q_heads;
        a.num_kv_heads = num_kv_heads;
        a.head_dim = head_dim;
        a.block_size = 16;
        a.max_context_len = max_context_len;
        const hipError_t e = pa::launch_decode_shared(shared_params(a, w, (char *)ws), 2,
                                                      (hipStream_t)stream);
        return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    pa::ReduceParams p{};
    p.out = out;
    p.context_lens = context_lens;
    p.ws_m = (const float *)(ws + w.m_off);
    p.ws_l = (const float *)(ws + w.l_off);
    p.ws_acc = (const float *)(ws + w.acc_off);
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.head_dim = head_dim;
    p.max_context_len = max_context_len;
    p.partition_size = partition_size;
    p.num_partitions = w.num_partitions;
    p.num_waves = kBalancedWaves;
    const hipError_t e = balanced ? pa::launch_reduce_balanced(p, dtype, (hipStream_t)stream)
                                  : pa::launch_reduce(p, dtype, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
              int num_q_heads, int num_kv_heads, int head_dim, int num_blocks, int block_size,
              int max_blocks_per_seq, int max_context_len, float scale, int partition_size,
              void *workspace, size_t workspace_bytes, int dtype, int algo, void *stream) {
    const DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       max_blocks_per_seq, max_context_len, scale, dtype, algo};
    int rc = validate_decode(a);
    if (rc != PA_OK) return rc;
    const int partition = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads,
                                            head_dim, block_size, max_context_len, dtype, algo);
    if (!is_split_mode(partition) && (partition < 0 || (partition > 0 && partition % block_size)))
        return PA_ERR_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (partition == 0) {
        // single pass: one unit per (sequence, KV head) covering the whole context
        const int whole = max_context_len > 0 ? max_context_len : 1;
        return launch_units(a, whole, 1, nullptr, nullptr, nullptr, (hipStream_t)stream);
    }
    rc = pa_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                              max_blocks_per_seq, max_context_len, scale, partition, workspace,
                              workspace_bytes, dtype, algo, stream);
    if (rc != PA_OK) return rc;
    return pa_decode_reduce(out, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            max_context_len, partition, workspace, workspace_bytes, dtype, stream);
}

int pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                      int block_size, int max_blocks_per_seq, int max_context_len, float scale,
                      int partition_size, int dtype, int algo, void *stream) {
    const DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                       max_blocks_per_seq, max_context_len, scale, dtype, algo};
    const int rc = validate_decode(a);
    if (rc != PA_OK) return rc;
    const int partition = resolve_partition(partition_size, num_seqs, num_q_heads, num_kv_heads,
                                            head_dim, block_size, max_context_len, dtype, algo);
    if (!is_split_mode(partition) && (partition < 0 || (partition > 0 && partition % block_size)))
        return PA_ERR_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (partition == 0)   // single pass: no workspace at all
        return pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                         num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                         max_blocks_per_seq, max_context_len, scale, 0, nullptr, 0, dtype, algo,
                         stream);
    const int mode = check_split_mode(a, partition);
    if (mode != PA_OK) return mode;
    const WorkspaceLayout w = layout(num_seqs, num_q_heads, head_dim, max_context_len, partition,
                                     num_q_heads / num_kv_heads);
    if (w.total > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
    if (w.num_partitions > pa::kMaxPartitions) return PA_ERR_SHAPE;
    int device = -1;
    const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &device)
                                : hipGetDevice(&device);
    if (e != hipSuccess || device < 0 || device >= kMaxDevices) return PA_ERR_LAUNCH;
    void *ws = nullptr;
    if (scratch_on(device, &ws) != hipSuccess) return PA_ERR_LAUNCH;
    // every kernel writes each workspace piece before anything reads it, so
    // the scratch needs no clearing between calls
    return pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, block_size, max_blocks_per_seq,
                     max_context_len, scale, partition, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES,
                     dtype, algo, stream);
}

}  // extern "C"
