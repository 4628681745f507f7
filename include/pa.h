/*
 * pa.h -- paged KV-cache decode for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  It does two things:
 *
 *   1. the slot write: append new tokens' K/V into their physical slots of a
 *      block-paged cache (pa_reshape_and_cache);
 *   2. PagedAttention decode: each query head attends over its sequence's
 *      cached K/V, which is scattered over fixed-size physical blocks and
 *      reached through a per-sequence block table (pa_decode, and its two
 *      split-context phases pa_decode_partitions / pa_decode_reduce).
 *
 * Sources (cited by page title and the named part of the page):
 *   "PagedAttention实现" (ainanfeng.cn project page): KVBlock (a block holds
 *       block_size token slots of K and of V), PageTable (logical block ->
 *       physical block), PagedKVManager::write_kv (a token at position pos is
 *       in logical block pos / block_size at offset pos % block_size).
 *   "CS349E 第 7 讲 01_paged_attention.py" (lecture 7 script): demo 2, paper
 *       eq. 4 -- scores block by block, one softmax over the whole context,
 *       V multiplied in block by block; paged and contiguous KV give the same
 *       result.
 *   "04 - Paged Attention 实现进度": section A.2 (block_tables is
 *       [batch, max_blocks_per_seq], slot_mapping is [total_tokens]),
 *       section B.2 (Context: slot_mapping maps token -> physical slot, i.e.
 *       block id and offset; context_lens is each sequence's current length;
 *       block_tables records each sequence's blocks in order), section B.3
 *       (block size 16).
 *
 * Conventions (all entry points):
 *   - Every pointer argument named as a tensor is a DEVICE pointer to a
 *     contiguous, row-major buffer that the caller allocated and owns.  The
 *     library keeps no reference after the call returns.
 *   - pa_reshape_and_cache, pa_decode, pa_decode_partitions and
 *     pa_decode_reduce never allocate device memory and never synchronise:
 *     they validate their arguments on the host, enqueue kernels on `stream`
 *     (a hipStream_t; NULL = the default stream) and return.  Results are
 *     ready when the stream reaches that point.
 *   - Return value: PA_OK (0) or a negative PA_ERR_* status; nothing is
 *     enqueued when a status other than PA_OK is returned for an argument
 *     error.  The library never prints and never aborts.
 *   - Every tensor pointer (and the workspace) must be 16-byte aligned.
 *   - dtype: PA_F32 (float) or PA_BF16 (bfloat16 bit patterns).  q, out,
 *     new K/V and both caches share one dtype.  Arithmetic is float32.
 *   - Cache layout, for K and for V separately:
 *         cache[num_blocks][num_kv_heads][block_size][head_dim]
 *     so one (block, KV head) tile is block_size*head_dim contiguous
 *     elements.
 *   - Device-side integer data (slots, block ids, context lengths) is
 *     trusted for correctness but bounded for safety: a slot outside
 *     [0, num_blocks*block_size) is not written, a block-table entry outside
 *     [0, num_blocks) is not read (the tokens it would hold are left out),
 *     and a context length is clamped to [0, max_context_len].  Such inputs
 *     give unspecified results but no access outside the caller's buffers.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,         /* a required pointer is NULL                      */
    PA_ERR_SHAPE = -2,        /* sizes inconsistent or out of range              */
    PA_ERR_UNSUPPORTED = -3,  /* head_dim / block_size / dtype / group size      */
    PA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required      */
    PA_ERR_LAUNCH = -5,       /* the HIP runtime refused a kernel launch         */
    PA_ERR_ALGO = -6,         /* requested kernel variant cannot run this shape  */
    PA_ERR_ALIGN = -7,        /* a tensor pointer is not 16-byte aligned          */
    PA_ERR_SCRATCH = -8       /* pa_decode_noalloc: the problem's workspace is
                                 larger than the static scratch                  */
};

/* Special partition_size values for pa_decode / pa_decode_partitions /
 * pa_decode_reduce / pa_decode_workspace_size. */
#define PA_PARTITION_AUTO (-1)      /* the library chooses                     */
#define PA_PARTITION_BALANCED (-2)  /* work-balanced split                     */
#define PA_PARTITION_SHARED (-3)    /* balanced split that reads blocks shared
                                       by neighbouring sequences once
                                       (matrix-core path)                      */

/* Kernel variants for pa_decode / pa_decode_partitions. */
enum {
    PA_ALGO_AUTO = 0,   /* matrix-core kernel where it applies, else vector    */
    PA_ALGO_VECTOR = 1, /* vector-ALU kernel (any supported shape)             */
    PA_ALGO_MFMA = 2    /* matrix-core kernel: bf16, head_dim 128,
                           block_size >= 16, group size <= 16                  */
};

/*
 * Slot write ("PagedAttention实现", write_kv; "04 - Paged Attention 实现进度",
 * section A.2 slot_mapping).  For every token t with s = slot_mapping[t] >= 0:
 *     block = s / block_size,  offset = s % block_size,
 *     k_cache[block][g][offset][:] = k[t][g][:]   for every KV head g,
 * and the same for V.  The copy is bit-exact (no conversion).  Negative
 * slots mark padding tokens and are skipped.
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim]             (in)
 *   k_cache,
 *   v_cache       [num_blocks][num_kv_heads][block_size][head_dim] (in/out)
 *   slot_mapping  [num_tokens] int64                               (in)
 *
 * Slots within one call must be distinct (two tokens writing one slot race).
 * Supported: head_dim in {16, 32, 64, 128, 256}; block_size a power of two
 * in [1, 256]; dtype PA_F32 or PA_BF16.  num_tokens == 0 is a no-op.
 */
int pa_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                         const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int num_blocks, int block_size, int dtype,
                         void *stream);

/*
 * Copy-on-write block copies ("PagedAttention实现", cow_write: a block shared
 * by several sequences is copied whole into a fresh block before one of them
 * writes into it; "CS349E 第 7 讲 01_paged_attention.py", demo 3).  For every
 * pair i with (src, dst) = (block_pairs[2 i], block_pairs[2 i + 1]):
 *     k_cache[dst][:][:][:] = k_cache[src][:][:][:]   (all heads, all slots)
 * and the same for V, bit-exact.  A pair with an id outside [0, num_blocks)
 * or with src == dst is skipped.
 *
 *   k_cache,
 *   v_cache      [num_blocks][num_kv_heads][block_size][head_dim] (in/out)
 *   block_pairs  [num_pairs][2] int32, device memory               (in)
 *
 * The destinations must be distinct and none may be the source of another
 * pair in the same call (the pairs are copied concurrently); a fresh block
 * from the allocator always satisfies this.  Supported shapes and dtypes as
 * for pa_reshape_and_cache.  num_pairs == 0 is a no-op.
 */
int pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_pairs, int num_pairs,
                   int num_blocks, int num_kv_heads, int block_size, int head_dim, int dtype,
                   void *stream);

/*
 * Paged prefill ("04 - Paged Attention 实现进度", section B.2: a prefill batch
 * is packed by cu_seqlens_q; "CS349E 第 7 讲 01_paged_attention.py", demo 1
 * prefills a prompt before decoding, demo 2 / paper eq. 4 for the softmax over
 * the paged cache).  Sequence b contributes a chunk of n_b = cu_seqlens_q[b+1]
 * - cu_seqlens_q[b] query rows: the last n_b positions of its
 * context_lens[b] tokens, whose K/V must already be in the cache (write them
 * with pa_reshape_and_cache first).  Row r of the chunk, at position
 * p = context_lens[b] - n_b + r, attends causally over positions 0..p:
 *     out[row][h][:] = sum_{j<=p} softmax_j(scale * q[row][h] . k_j) v_j
 * with query head h reading KV head h / (num_q_heads / num_kv_heads).  A
 * chunk of one row is decode; a chunk that is the whole sequence is ordinary
 * causal prefill; anything between is chunked prefill over a cached prefix.
 *
 *   out, q         [total_q][num_q_heads][head_dim]  (total_q = cu_seqlens_q[num_seqs])
 *   cu_seqlens_q   [num_seqs + 1] int32, device, cu_seqlens_q[0] = 0, non-decreasing
 *   context_lens   [num_seqs] int32, device, n_b <= context_lens[b] <= max_context_len
 *   block_tables, k_cache, v_cache   as for pa_decode
 *   max_q_len      an upper bound of every n_b (sizes the grid)
 *
 * Supported: head_dim in {16, 32, 64, 128, 256}; block_size a power of two in
 * [1, 256]; group size at most 16; dtype PA_F32 or PA_BF16.  bfloat16 with
 * head_dim 128, block_size >= 16 and scale > 0 runs on the matrix cores,
 * everything else on the vector ALUs (float32 arithmetic either way).  Chunks with
 * n_b = 0 produce nothing.  Asynchronous on `stream`, no workspace.
 */
int pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, const int32_t *cu_seqlens_q,
               const int32_t *context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
               int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
               int max_context_len, int max_q_len, float scale, int dtype, void *stream);

/*
 * Split-context decode, the common source of the next four calls.  The one
 * softmax over a whole context of "CS349E 第 7 讲 01_paged_attention.py"
 * (demo 2, paper eq. 4: scores block by block, one softmax over all blocks,
 * V multiplied in block by block) does not depend on how the blocks are
 * grouped: a group of blocks keeps its own max m, its sum
 * l = sum 2^(s - m) and its weighted V sum acc, and groups combine by
 * rescaling each by 2^(m - M), M the largest m.  Splitting a long context
 * into such groups lets many wavefronts share one sequence.  The pages name
 * no split: "04 - Paged Attention 实现进度" (section A.3) names a second
 * generation of vLLM's kernel (v2) only by its tiling.
 */

/*
 * Partition mode the library uses when pa_decode / pa_decode_partitions get
 * partition_size == PA_PARTITION_AUTO for these sizes and PA_ALGO_AUTO:
 * 0 (single pass, no workspace), PA_PARTITION_BALANCED, or a multiple of
 * block_size.  A pure function of its arguments.  Where the vector kernel
 * runs (every shape the matrix-core kernels do not take, or PA_ALGO_VECTOR):
 * single pass for small problems (max_context_len * num_seqs *
 * num_kv_heads <= 65536, or a context that fits one partition below);
 * otherwise PA_PARTITION_BALANCED when block_size >= 16 and the head's
 * 16-token tile covers whole 64-lane load passes (every head_dim for
 * float32, head_dim >= 32 for bfloat16), else the power of two from 64 to
 * 512 tokens (at least block_size) that gives about 8192 wavefronts for
 * contexts of max_context_len.
 */
int pa_decode_auto_partition(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_context_len, int dtype);

/*
 * Bytes of device workspace pa_decode needs (0 in single-pass mode): the
 * (m, l, acc) states of the groups of a split context (above), plus, in the
 * balanced and shared modes, the plan that splits the work.  partition_size
 * as for pa_decode; for PA_PARTITION_AUTO the size is enough for every mode
 * the library may pick for these sizes.  dtype selects the kernel the mode
 * runs on (and so whether the mode applies); num_kv_heads and block_size
 * likewise.  A pure host function: no device call.  Returns 0 for invalid
 * sizes, and for modes the shape cannot run, as well.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_context_len, int partition_size,
                                int dtype);

/*
 * PagedAttention decode ("CS349E 第 7 讲 01_paged_attention.py", demo 2,
 * paper eq. 4).  One query token per sequence b, query head h, KV head
 * g = h / (num_q_heads / num_kv_heads), n = context_lens[b]:
 *     s_j = scale * dot(q[b][h], K_b[j]),   j < n
 *     out[b][h] = sum_j softmax(s)_j * V_b[j]
 * where K_b[j] is element g of the token at logical position j, found at
 * block block_tables[b][j / block_size], offset j % block_size.  One
 * softmax is taken over the whole context.  n == 0 gives zeros.
 *
 *   out           [num_seqs][num_q_heads][head_dim]                 (out)
 *   q             [num_seqs][num_q_heads][head_dim]                 (in)
 *   k_cache,
 *   v_cache       [num_blocks][num_kv_heads][block_size][head_dim]  (in)
 *   block_tables  [num_seqs][max_blocks_per_seq] int32              (in)
 *   context_lens  [num_seqs] int32, tokens visible to this step's query,
 *                 including the one appended by this step's slot write (in)
 *   max_context_len  an upper bound on context_lens (sizes the workspace)
 *   scale         softmax scale (usually 1/sqrt(head_dim))
 *   partition_size   0: single pass, one work unit per (sequence, KV head);
 *                 PA_PARTITION_AUTO: the library chooses
 *                 (pa_decode_auto_partition);
 *                 PA_PARTITION_BALANCED: work-balanced split: the 16-token
 *                 tiles of every (KV head, sequence) are laid end to end
 *                 and a fixed number of wavefronts take equal contiguous
 *                 shares; pieces of a context cut between wavefronts are
 *                 merged by log-sum-exp.  Needs block_size >= 16; runs on
 *                 the matrix cores where they apply (unless algo is
 *                 PA_ALGO_VECTOR), else on the vector ALUs, which take
 *                 float32 with any head_dim and bfloat16 with head_dim >= 32
 *                 (PA_ERR_ALGO otherwise);
 *                 PA_PARTITION_SHARED: like PA_PARTITION_BALANCED, but
 *                 consecutive sequences are taken in packs (8 when the
 *                 group size is at most 4, 4 up to 8, 2 up to 16) whose
 *                 query heads share one wavefront, and a physical block that
 *                 several members of a pack reference at the same logical
 *                 position (a shared prefix, e.g. forked samples) is read
 *                 once for all of them; a planning kernel counts the
 *                 distinct blocks first so the split stays balanced.  Put
 *                 sequences that share blocks next to each other;
 *                 otherwise a multiple of block_size: the context is split
 *                 into partitions of that many tokens, each reduced
 *                 separately, then merged by log-sum-exp (split-context
 *                 decode: pa_decode_partitions followed by pa_decode_reduce).
 *                 A fixed-partition split may have at most 8192 partitions.
 *   workspace     device scratch of at least pa_decode_workspace_size(...)
 *                 bytes in split mode (ignored in single-pass mode).  Calls
 *                 that share a workspace must be ordered on one stream.
 *   algo          PA_ALGO_AUTO, PA_ALGO_VECTOR or PA_ALGO_MFMA.
 *
 * Supported: head_dim in {16, 32, 64, 128, 256}; block_size a power of two in
 * [1, 256]; num_q_heads a multiple of num_kv_heads with a group size of at
 * most 16; dtype PA_F32 or PA_BF16.  Write this step's token with
 * pa_reshape_and_cache earlier on the same stream.
 */
int pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
              int num_q_heads, int num_kv_heads, int head_dim, int num_blocks, int block_size,
              int max_blocks_per_seq, int max_context_len, float scale, int partition_size,
              void *workspace, size_t workspace_bytes, int dtype, int algo, void *stream);

/*
 * Phase 1 of split-context decode (the grouping above): per (sequence, query
 * head, partition p)
 * of partition_size tokens (a positive multiple of block_size), the running
 * max m_p (base-2 log domain: scores times scale*log2(e)), the sum
 * l_p = sum_j 2^(s_j - m_p) and the unnormalised acc_p = sum_j 2^(s_j - m_p)
 * V[j] go to the workspace.  A sequence with a single partition has its
 * final output written to `out` directly.  Same arguments as pa_decode.
 *
 * Workspace layout (float32), NP = ceil(max_context_len / partition_size):
 *     m   [num_seqs][num_q_heads][NP]
 *     l   [num_seqs][num_q_heads][NP]
 *     acc [num_seqs][num_q_heads][NP][head_dim]
 * each array starting at a 256-byte aligned offset, in that order.  This is
 * the exchange format for splitting one sequence's context across devices.
 * With PA_PARTITION_BALANCED or PA_PARTITION_SHARED the workspace layout is
 * internal to the library (a plan and per-wavefront partial states).
 */
int pa_decode_partitions(void *out, const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int num_blocks, int block_size, int max_blocks_per_seq,
                         int max_context_len, float scale, int partition_size,
                         void *workspace, size_t workspace_bytes, int dtype, int algo,
                         void *stream);

/*
 * Phase 2 of split-context decode (the combination rule above): for every
 * sequence with more than one partition, merge the partitions in ascending
 * order:
 *     M = max_p m_p,  w_p = 2^(m_p - M),
 *     out = (sum_p w_p acc_p) / (sum_p w_p l_p).
 * Sequences with one partition are left alone (phase 1 wrote them);
 * empty contexts get zeros here.  partition_size must be the value phase 1
 * resolved (not PA_PARTITION_AUTO; see pa_decode_auto_partition); with
 * PA_PARTITION_BALANCED or PA_PARTITION_SHARED the pieces of each
 * (sequence, KV head) are merged the same way, and empty contexts get zeros
 * too.
 */
int pa_decode_reduce(void *out, const int32_t *context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int max_context_len, int partition_size,
                     const void *workspace, size_t workspace_bytes, int dtype, void *stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Arguments and results are those of pa_decode without
 * the workspace.  Split modes use scratch the library holds instead: a
 * file-scope device array of PA_NOALLOC_SCRATCH_BYTES on every GPU the
 * library runs on, kept until the process ends.  Its device address is
 * looked up on the first call on each device (the device of `stream`, or
 * the current device for the default stream); no call allocates or frees
 * device memory.
 *
 * A problem whose workspace (pa_decode_workspace_size for the partition
 * mode the call resolves to) is larger than the scratch returns
 * PA_ERR_SCRATCH with nothing enqueued; a failed address lookup returns
 * PA_ERR_LAUNCH.  Single-pass decode (partition_size 0, or the library's
 * choice of it) uses no scratch.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (nothing in it needs clearing: each call writes every
 * piece before reading it).  Calls that may overlap on one GPU -- on
 * different streams, or from host threads without ordering -- race on it
 * and give wrong results: order them on one stream.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
int pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                      int block_size, int max_blocks_per_seq, int max_context_len, float scale,
                      int partition_size, int dtype, int algo, void *stream);

/*
 * A static, human-readable name for a status code.  Every entry point
 * reports failure by its return value instead of aborting, as
 * "PagedAttention实现" (PagedKVManager::allocate_block) returns false when
 * no free block is left; this turns the code into text.  Never NULL;
 * unknown codes give "unknown status".
 */
const char *pa_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
