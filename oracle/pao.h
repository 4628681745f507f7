/*
 * pao.h -- CPU oracle for paged KV-cache decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * helper with the GPU library (include/pa.h and its sources).
 *
 * It is plain, slow and obviously correct on purpose:
 *   - a host block pool with a LIFO free stack, reference counts, fork,
 *     copy-on-write and free;
 *   - the slot write that places one token's K/V at its physical slot;
 *   - decode attention in float64, in three forms (concatenate-then-attend,
 *     blockwise with one global softmax, partitioned with a log-sum-exp merge);
 *   - prefill attention in float64: a chunk of new tokens per sequence, each
 *     attending causally over the cache up to its own position.
 *
 * Sources (cited by page title and the named part of the page):
 *   [P1] "PagedAttention实现" (ainanfeng.cn project page): KVBlock, PageTable,
 *        PagedKVManager::{allocate_block, write_kv, cow_write, free_sequence,
 *        print_status} and its main() demo.
 *   [P2] "CS349E 第 7 讲 01_paged_attention.py -- PagedAttention: block table,
 *        blockwise attention, sharing and copy-on-write" (lecture script):
 *        demo 1 (block-table growth), demo 2 (paged = contiguous; paper eq. 4
 *        blockwise attention), demo 3 (parallel sampling, copy-on-write),
 *        demo 4 (beam search); demo 1's prefill of a 7-token prompt.
 *   [P3] "04 - Paged Attention 实现进度": section A.2 (five components,
 *        block_tables / slot_mapping shapes), section B.2 (Context fields,
 *        cu_seqlens_q / cu_seqlens_k of a prefill batch), section B.3 (block
 *        size 16).
 *
 * Every function returns a status: 0 on success, a negative PAO_E* code on
 * error.  The oracle never aborts on bad input.
 */
#ifndef PAO_H
#define PAO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PAO_OK = 0,
    PAO_E_OOM = -1,      /* free stack empty                                */
    PAO_E_SEQ = -2,      /* unknown or freed sequence id                    */
    PAO_E_POS = -3,      /* token position outside the sequence's table     */
    PAO_E_ARG = -4,      /* bad size / dtype / null pointer                 */
    PAO_E_SLOT = -5,     /* slot out of range or repeated within one call   */
    PAO_E_BLOCK = -6,    /* block id out of range or not held               */
    PAO_E_TABLE = -7     /* block table entry invalid for a visible token   */
};

enum { PAO_F32 = 0, PAO_BF16 = 1 };

/* ------------------------------------------------------------------------ */
/* Host block pool                                                           */
/* ------------------------------------------------------------------------ */
typedef struct pao_pool pao_pool;

/* free_order: the initial free stack, bottom first, so the first block handed
 * out is free_order[num_blocks-1].  NULL means 0..num_blocks-1 as in [P1]'s
 * constructor (so the first allocation returns num_blocks-1). */
pao_pool *pao_pool_create(int num_blocks, int block_size, const int32_t *free_order);
void pao_pool_destroy(pao_pool *p);

/* Pool-level block ops ([P2] BlockPool.alloc / BlockPool.decref). */
int pao_block_alloc(pao_pool *p);               /* >=0 block id, or PAO_E_OOM */
int pao_block_decref(pao_pool *p, int block);   /* pushes the block at ref 0  */
int pao_block_ref(const pao_pool *p, int block);/* ref count, or PAO_E_BLOCK  */

/* Sequence ops. */
int pao_seq_new(pao_pool *p);                    /* new empty sequence id      */
int pao_seq_alloc_block(pao_pool *p, int seq);   /* [P1] allocate_block        */
int pao_seq_slot(const pao_pool *p, int seq, int pos, int64_t *slot); /* [P1] write_kv addressing */
int pao_seq_fork(pao_pool *p, int seq);          /* share every block, ref++   */
int pao_seq_append(pao_pool *p, int seq, int64_t *slot,
                   int32_t *cow_src, int32_t *cow_dst); /* write position len  */
int pao_seq_free(pao_pool *p, int seq);          /* [P1] free_sequence         */
int pao_seq_len(const pao_pool *p, int seq);
int pao_seq_num_blocks(const pao_pool *p, int seq);
int pao_seq_table(const pao_pool *p, int seq, int32_t *row, int max_blocks);

/* out[0..5] = total blocks, free blocks, used blocks, peak used blocks,
 * copy-on-write copies so far, live sequences. */
void pao_pool_stats(const pao_pool *p, int64_t *out);

/* ------------------------------------------------------------------------ */
/* KV storage: raw element bytes, layout [num_blocks][num_kv_heads]          */
/* [block_size][head_dim] for K and for V.                                    */
/* ------------------------------------------------------------------------ */

/* Copy token t's K/V ([num_tokens][num_kv_heads][head_dim]) to the physical
 * slot slot_mapping[t]; negative slots are skipped.  Slots must be in range
 * and distinct within the call (PAO_E_SLOT otherwise, nothing written). */
int pao_slot_write(void *k_cache, void *v_cache, const void *k, const void *v,
                   const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                   int head_dim, int num_blocks, int block_size, int elem_bytes);

/* Whole-block copy src -> dst for K and V (every slot, every KV head). */
int pao_copy_block(void *k_cache, void *v_cache, int src, int dst, int num_blocks,
                   int num_kv_heads, int head_dim, int block_size, int elem_bytes);

/* ------------------------------------------------------------------------ */
/* Decode attention in float64.                                               */
/*   out  [num_seqs][num_q_heads][head_dim] float64                          */
/*   q    [num_seqs][num_q_heads][head_dim] in dtype                         */
/*   caches [num_blocks][num_kv_heads][block_size][head_dim] in dtype        */
/*   block_tables [num_seqs][max_blocks_per_seq] int32                       */
/*   context_lens [num_seqs] int32 (tokens visible to this step's query)     */
/* Query head h reads KV head h / (num_q_heads / num_kv_heads).              */
/* nthreads <= 0 means the OpenMP default.                                   */
/* ------------------------------------------------------------------------ */
int pao_decode_concat_f64(double *out, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_dim, int num_blocks, int block_size,
                          int max_blocks_per_seq, double scale, int dtype, int nthreads);

int pao_decode_blockwise_f64(double *out, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int num_blocks, int block_size,
                             int max_blocks_per_seq, double scale, int dtype, int nthreads);

int pao_decode_partitioned_f64(double *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int num_blocks,
                               int block_size, int max_blocks_per_seq, double scale,
                               int dtype, int partition_size, int nthreads);

/* ------------------------------------------------------------------------ */
/* Prefill attention over the paged cache in float64 (a chunk of new tokens  */
/* per sequence, causal).                                                      */
/*   out  [total_q][num_q_heads][head_dim] float64                           */
/*   q    [total_q][num_q_heads][head_dim] in dtype: the chunk of sequence b  */
/*        is rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1                     */
/*   context_lens [num_seqs]: tokens in the cache after the chunk's write     */
/* The chunk's n_b tokens are the last n_b positions of the sequence: row r  */
/* of the chunk sits at position p = context_lens[b] - n_b + r and attends   */
/* over positions 0 .. p (its own included).  n_b == 1 is decode.            */
/* ------------------------------------------------------------------------ */
int pao_prefill_concat_f64(double *out, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *block_tables,
                           const int32_t *cu_seqlens_q, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int num_blocks, int block_size, int max_blocks_per_seq,
                           double scale, int dtype, int nthreads);

#ifdef __cplusplus
}
#endif
#endif /* PAO_H */
