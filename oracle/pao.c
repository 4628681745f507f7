/*
 * pao.c -- CPU oracle for paged KV-cache decode (TEST INFRASTRUCTURE ONLY).
 *
 * Read pao.h first: it names the pages this file follows ([P1], [P2], [P3])
 * and says who may use it.  Everything here is written for a reader checking
 * it against the pages by eye: plain loops, float64, no blocking, no fusion.
 */
#include "pao.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================== */
/* Host block pool                                                           */
/* ======================================================================== */

typedef struct {
    int alive;
    int len;         /* tokens written so far                 */
    int n_blocks;    /* entries used in table                  */
    int cap;
    int32_t *table;  /* logical block -> physical block ([P1] PageTable) */
} pao_seq;

struct pao_pool {
    int num_blocks;
    int block_size;
    int32_t *ref;        /* ref count per physical block ([P1] KVBlock.ref_count) */
    int32_t *stack;      /* free blocks; top of stack = stack[n_free-1]           */
    int n_free;
    int64_t peak_used;
    int64_t n_copies;
    int n_seqs, seqs_cap;
    pao_seq *seqs;
};

pao_pool *pao_pool_create(int num_blocks, int block_size, const int32_t *free_order)
{
    if (num_blocks <= 0 || block_size <= 0) return NULL;
    pao_pool *p = (pao_pool *)calloc(1, sizeof(pao_pool));
    if (!p) return NULL;
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->ref = (int32_t *)calloc((size_t)num_blocks, sizeof(int32_t));
    p->stack = (int32_t *)malloc((size_t)num_blocks * sizeof(int32_t));
    if (!p->ref || !p->stack) { pao_pool_destroy(p); return NULL; }
    /* [P1] PagedKVManager constructor: every block id is pushed in order, so
     * the free list starts as 0..n-1 and pop_back hands out n-1 first. */
    for (int i = 0; i < num_blocks; i++) {
        int b = free_order ? free_order[i] : i;
        if (b < 0 || b >= num_blocks) { pao_pool_destroy(p); return NULL; }
        p->stack[i] = b;
    }
    /* a free order must be a permutation */
    for (int i = 0; i < num_blocks; i++) p->ref[p->stack[i]]++;
    for (int i = 0; i < num_blocks; i++)
        if (p->ref[i] != 1) { pao_pool_destroy(p); return NULL; }
    memset(p->ref, 0, (size_t)num_blocks * sizeof(int32_t));
    p->n_free = num_blocks;
    return p;
}

void pao_pool_destroy(pao_pool *p)
{
    if (!p) return;
    for (int s = 0; s < p->n_seqs; s++) free(p->seqs[s].table);
    free(p->seqs);
    free(p->ref);
    free(p->stack);
    free(p);
}

/* [P1] allocate_block: fail (no block) when the free list is empty,
 * otherwise take the back of the list and give it reference count 1. */
int pao_block_alloc(pao_pool *p)
{
    if (p->n_free == 0) return PAO_E_OOM;
    int b = p->stack[--p->n_free];
    p->ref[b] = 1;
    int64_t used = p->num_blocks - p->n_free;
    if (used > p->peak_used) p->peak_used = used;
    return b;
}

/* [P1] free_sequence, per block: drop one reference; a block whose count
 * reaches zero goes back on the free list. */
int pao_block_decref(pao_pool *p, int block)
{
    if (block < 0 || block >= p->num_blocks || p->ref[block] <= 0) return PAO_E_BLOCK;
    p->ref[block]--;
    if (p->ref[block] == 0) p->stack[p->n_free++] = block;
    return PAO_OK;
}

int pao_block_ref(const pao_pool *p, int block)
{
    if (block < 0 || block >= p->num_blocks) return PAO_E_BLOCK;
    return p->ref[block];
}

static pao_seq *get_seq(const pao_pool *p, int seq)
{
    if (seq < 0 || seq >= p->n_seqs || !p->seqs[seq].alive) return NULL;
    return &p->seqs[seq];
}

static int table_push(pao_seq *s, int32_t b)
{
    if (s->n_blocks == s->cap) {
        int ncap = s->cap ? 2 * s->cap : 8;
        int32_t *t = (int32_t *)realloc(s->table, (size_t)ncap * sizeof(int32_t));
        if (!t) return PAO_E_ARG;
        s->table = t;
        s->cap = ncap;
    }
    s->table[s->n_blocks++] = b;
    return PAO_OK;
}

int pao_seq_new(pao_pool *p)
{
    if (p->n_seqs == p->seqs_cap) {
        int ncap = p->seqs_cap ? 2 * p->seqs_cap : 16;
        pao_seq *t = (pao_seq *)realloc(p->seqs, (size_t)ncap * sizeof(pao_seq));
        if (!t) return PAO_E_ARG;
        p->seqs = t;
        p->seqs_cap = ncap;
    }
    pao_seq *s = &p->seqs[p->n_seqs];
    memset(s, 0, sizeof(*s));
    s->alive = 1;
    return p->n_seqs++;
}

/* [P1] allocate_block(seq_id): append a fresh block to the sequence's page
 * table.  Returns the block id. */
int pao_seq_alloc_block(pao_pool *p, int seq)
{
    pao_seq *s = get_seq(p, seq);
    if (!s) return PAO_E_SEQ;
    int b = pao_block_alloc(p);
    if (b < 0) return b;
    if (table_push(s, b) != PAO_OK) { pao_block_decref(p, b); return PAO_E_ARG; }
    return b;
}

/* [P1] write_kv addressing: a token at position pos lives in logical block
 * pos / block_size at offset pos % block_size; the page table gives the
 * physical block.  [P3] section B.2: the slot is that block's id combined
 * with the offset, i.e. physical_block * block_size + offset. */
int pao_seq_slot(const pao_pool *p, int seq, int pos, int64_t *slot)
{
    const pao_seq *s = get_seq(p, seq);
    if (!s) return PAO_E_SEQ;
    if (pos < 0) return PAO_E_POS;
    int page_idx = pos / p->block_size;
    int offset = pos % p->block_size;
    if (page_idx >= s->n_blocks) return PAO_E_POS;  /* [P1] leaves this unchecked */
    int physical = s->table[page_idx];
    *slot = (int64_t)physical * p->block_size + offset;
    return PAO_OK;
}

/* Fork: the child starts with the parent's table and length, and every
 * shared block gains one reference.  [P1] has no such operation (nothing
 * there raises a count above one); [P2] demo 3 and demo 4 need it: n samples
 * or beam candidates share the prompt's blocks. */
int pao_seq_fork(pao_pool *p, int seq)
{
    if (!get_seq(p, seq)) return PAO_E_SEQ;
    int child = pao_seq_new(p);   /* may move p->seqs */
    if (child < 0) return child;
    pao_seq *s = &p->seqs[seq];
    pao_seq *c = &p->seqs[child];
    for (int i = 0; i < s->n_blocks; i++) {
        if (table_push(c, s->table[i]) != PAO_OK) return PAO_E_ARG;
        p->ref[s->table[i]]++;
    }
    c->len = s->len;
    return child;
}

/* Reserve the slot for the token at position len, then len++.
 *  - [P2] demo 1: a new block is taken only when the last one is full (or
 *    the table does not yet reach this position).
 *  - [P1] cow_write: if the block that holds the position is shared
 *    (ref > 1), take a new block, copy the whole old block into it, point the
 *    table at the copy and drop one reference on the old block, then write.
 *    Here the copy itself is left to whoever holds the KV bytes: the pair
 *    (cow_src, cow_dst) is reported, and both are -1 when no copy happened.
 *    Unlike [P1], an empty free list is reported (PAO_E_OOM) instead of
 *    popping from an empty vector. */
int pao_seq_append(pao_pool *p, int seq, int64_t *slot, int32_t *cow_src, int32_t *cow_dst)
{
    pao_seq *s = get_seq(p, seq);
    if (!s) return PAO_E_SEQ;
    *cow_src = -1;
    *cow_dst = -1;
    int pos = s->len;
    int page_idx = pos / p->block_size;
    if (page_idx >= s->n_blocks) {
        int b = pao_seq_alloc_block(p, seq);
        if (b < 0) return b;
        s = &p->seqs[seq];
    } else {
        int old = s->table[page_idx];
        if (p->ref[old] > 1) {
            int nb = pao_block_alloc(p);
            if (nb < 0) return nb;
            p->ref[old]--;
            s->table[page_idx] = nb;
            p->n_copies++;
            *cow_src = old;
            *cow_dst = nb;
        }
    }
    int rc = pao_seq_slot(p, seq, pos, slot);
    if (rc != PAO_OK) return rc;
    s->len = pos + 1;
    return PAO_OK;
}

/* [P1] free_sequence: walk the table in order, dropping one reference per
 * entry; blocks reaching zero return to the free list. */
int pao_seq_free(pao_pool *p, int seq)
{
    pao_seq *s = get_seq(p, seq);
    if (!s) return PAO_E_SEQ;
    for (int i = 0; i < s->n_blocks; i++) {
        int rc = pao_block_decref(p, s->table[i]);
        if (rc != PAO_OK) return rc;
    }
    free(s->table);
    memset(s, 0, sizeof(*s));
    return PAO_OK;
}

int pao_seq_len(const pao_pool *p, int seq)
{
    const pao_seq *s = get_seq(p, seq);
    return s ? s->len : PAO_E_SEQ;
}

int pao_seq_num_blocks(const pao_pool *p, int seq)
{
    const pao_seq *s = get_seq(p, seq);
    return s ? s->n_blocks : PAO_E_SEQ;
}

/* [P3] section A.2: one row of block_tables [batch, max_blocks_per_seq];
 * entries past the sequence's blocks are -1. */
int pao_seq_table(const pao_pool *p, int seq, int32_t *row, int max_blocks)
{
    const pao_seq *s = get_seq(p, seq);
    if (!s) return PAO_E_SEQ;
    if (s->n_blocks > max_blocks) return PAO_E_ARG;
    for (int i = 0; i < max_blocks; i++) row[i] = i < s->n_blocks ? s->table[i] : -1;
    return s->n_blocks;
}

/* [P1] print_status reports total blocks, free blocks and live sequences;
 * [P2] demo 2-4 also read used blocks, peak used blocks and the number of
 * copy-on-write copies. */
void pao_pool_stats(const pao_pool *p, int64_t *out)
{
    int live = 0;
    for (int s = 0; s < p->n_seqs; s++) live += p->seqs[s].alive;
    out[0] = p->num_blocks;
    out[1] = p->n_free;
    out[2] = p->num_blocks - p->n_free;
    out[3] = p->peak_used;
    out[4] = p->n_copies;
    out[5] = live;
}

/* ======================================================================== */
/* KV storage                                                                */
/* ======================================================================== */

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* [P1] write_kv: copy the head_dim values of K and V into the block at the
 * token's offset.  Here one token carries every KV head, and its place is
 * given by its slot ([P3] section A.2 slot_mapping): block = slot /
 * block_size, offset = slot % block_size.  The copy is byte-for-byte. */
int pao_slot_write(void *k_cache, void *v_cache, const void *k, const void *v,
                   const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                   int head_dim, int num_blocks, int block_size, int elem_bytes)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
        block_size <= 0 || (elem_bytes != 2 && elem_bytes != 4))
        return PAO_E_ARG;
    if (num_tokens == 0) return PAO_OK;
    if (!k_cache || !v_cache || !k || !v || !slot_mapping) return PAO_E_ARG;

    /* check: every slot in range, no slot used twice */
    int64_t n_slots = (int64_t)num_blocks * block_size;
    int64_t *sorted = (int64_t *)malloc((size_t)num_tokens * sizeof(int64_t));
    if (!sorted) return PAO_E_ARG;
    int n = 0;
    for (int t = 0; t < num_tokens; t++) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        if (s >= n_slots) { free(sorted); return PAO_E_SLOT; }
        sorted[n++] = s;
    }
    qsort(sorted, (size_t)n, sizeof(int64_t), cmp_i64);
    for (int i = 1; i < n; i++)
        if (sorted[i] == sorted[i - 1]) { free(sorted); return PAO_E_SLOT; }
    free(sorted);

    size_t row = (size_t)head_dim * (size_t)elem_bytes;   /* one head of one token */
    for (int t = 0; t < num_tokens; t++) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        for (int g = 0; g < num_kv_heads; g++) {
            size_t src = ((size_t)t * num_kv_heads + g) * row;
            size_t dst = (((size_t)block * num_kv_heads + g) * block_size + offset) * row;
            memcpy((char *)k_cache + dst, (const char *)k + src, row);
            memcpy((char *)v_cache + dst, (const char *)v + src, row);
        }
    }
    return PAO_OK;
}

/* [P1] cow_write copies the whole block (every slot) before writing. */
int pao_copy_block(void *k_cache, void *v_cache, int src, int dst, int num_blocks,
                   int num_kv_heads, int head_dim, int block_size, int elem_bytes)
{
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return PAO_E_BLOCK;
    if (!k_cache || !v_cache || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        (elem_bytes != 2 && elem_bytes != 4))
        return PAO_E_ARG;
    size_t bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes;
    memmove((char *)k_cache + (size_t)dst * bytes, (char *)k_cache + (size_t)src * bytes, bytes);
    memmove((char *)v_cache + (size_t)dst * bytes, (char *)v_cache + (size_t)src * bytes, bytes);
    return PAO_OK;
}

/* ======================================================================== */
/* Decode attention in float64                                               */
/* ======================================================================== */

/* Exact widening of one stored element to double: float32 directly; bfloat16
 * is the upper half of a float32 bit pattern. */
static double load_elem(const void *base, size_t idx, int dtype)
{
    if (dtype == PAO_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k_cache, *v_cache;
    const int32_t *block_tables, *context_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size;
    int max_blocks_per_seq, dtype;
    double scale;
} decode_args;

static int check_args(const decode_args *a, double *out)
{
    if (a->num_seqs < 0) return PAO_E_ARG;
    if (a->num_seqs == 0) return PAO_OK;
    if (!out || !a->q || !a->k_cache || !a->v_cache || !a->block_tables || !a->context_lens)
        return PAO_E_ARG;
    if (a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->num_q_heads % a->num_kv_heads)
        return PAO_E_ARG;
    if (a->head_dim <= 0 || a->block_size <= 0 || a->num_blocks <= 0 ||
        a->max_blocks_per_seq <= 0)
        return PAO_E_ARG;
    if (a->dtype != PAO_F32 && a->dtype != PAO_BF16) return PAO_E_ARG;
    /* every visible token must map to a valid block */
    for (int b = 0; b < a->num_seqs; b++) {
        int n = a->context_lens[b];
        if (n < 0 || n > a->max_blocks_per_seq * a->block_size) return PAO_E_ARG;
        int nblk = (n + a->block_size - 1) / a->block_size;
        for (int i = 0; i < nblk; i++) {
            int32_t phys = a->block_tables[(size_t)b * a->max_blocks_per_seq + i];
            if (phys < 0 || phys >= a->num_blocks) return PAO_E_TABLE;
        }
    }
    return PAO_OK;
}

/* Element i of head g at logical token position j of sequence b, read
 * through the block table ([P1] write_kv addressing, read direction). */
static size_t pool_index(const decode_args *a, int b, int g, int j, int i)
{
    int32_t phys = a->block_tables[(size_t)b * a->max_blocks_per_seq + j / a->block_size];
    int off = j % a->block_size;
    return (((size_t)phys * a->num_kv_heads + g) * a->block_size + off) * a->head_dim + i;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* (1) Concatenate, then attend.  [P2] demo 2 reads a sequence's K/V back
 * into contiguous arrays and runs ordinary attention on them; [P3] (closing
 * summary) describes the same "gather to contiguous K/V, reuse attention"
 * path.  Per (sequence b, KV head g):
 *   K[j][i], V[j][i]  for j < n = context_lens[b]   (gather, exact upcast)
 * and for every query head h with h / G == g:
 *   s_j = scale * sum_i q[h][i] K[j][i]
 *   m   = max_j s_j,  w_j = exp(s_j - m),  L = sum_j w_j
 *   o[h][i] = (sum_j w_j V[j][i]) / L
 * n == 0 gives zeros. */
int pao_decode_concat_f64(double *out, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_dim, int num_blocks, int block_size,
                          int max_blocks_per_seq, double scale, int dtype, int nthreads)
{
    decode_args a = {q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, dtype, scale};
    int rc = check_args(&a, out);
    if (rc != PAO_OK || num_seqs == 0) return rc;
    set_threads(nthreads);
    const int G = num_q_heads / num_kv_heads;
    const int d = head_dim;
    const long n_pairs = (long)num_seqs * num_kv_heads;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long pair = 0; pair < n_pairs; pair++) {
        int b = (int)(pair / num_kv_heads);
        int g = (int)(pair % num_kv_heads);
        int n = context_lens[b];
        if (n == 0) {
            for (int h = g * G; h < (g + 1) * G; h++)
                for (int i = 0; i < d; i++) out[((size_t)b * num_q_heads + h) * d + i] = 0.0;
            continue;
        }
        double *K = (double *)malloc((size_t)n * d * sizeof(double));
        double *V = (double *)malloc((size_t)n * d * sizeof(double));
        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!K || !V || !s) {
            free(K); free(V); free(s);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int j = 0; j < n; j++)
            for (int i = 0; i < d; i++) {
                K[(size_t)j * d + i] = load_elem(k_cache, pool_index(&a, b, g, j, i), dtype);
                V[(size_t)j * d + i] = load_elem(v_cache, pool_index(&a, b, g, j, i), dtype);
            }
        for (int h = g * G; h < (g + 1) * G; h++) {
            size_t qo = ((size_t)b * num_q_heads + h) * d;
            double m = -INFINITY;
            for (int j = 0; j < n; j++) {
                double acc = 0.0;
                for (int i = 0; i < d; i++) acc += load_elem(q, qo + i, dtype) * K[(size_t)j * d + i];
                s[j] = scale * acc;
                if (s[j] > m) m = s[j];
            }
            double L = 0.0;
            for (int j = 0; j < n; j++) {
                s[j] = exp(s[j] - m);   /* s now holds the weights w_j */
                L += s[j];
            }
            for (int i = 0; i < d; i++) {
                double acc = 0.0;
                for (int j = 0; j < n; j++) acc += s[j] * V[(size_t)j * d + i];
                out[qo + i] = acc / L;
            }
        }
        free(K); free(V); free(s);
    }
    return failed ? PAO_E_ARG : PAO_OK;
}

/* (2) Blockwise, [P2] demo 2's "paper eq. 4" form: scores are computed block
 * by block straight from the physical blocks (no gather), one softmax is
 * taken over all blocks together, and V is multiplied in block by block. */
int pao_decode_blockwise_f64(double *out, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int num_blocks, int block_size,
                             int max_blocks_per_seq, double scale, int dtype, int nthreads)
{
    decode_args a = {q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, dtype, scale};
    int rc = check_args(&a, out);
    if (rc != PAO_OK || num_seqs == 0) return rc;
    set_threads(nthreads);
    const int G = num_q_heads / num_kv_heads;
    const int d = head_dim, bs = block_size;
    const long n_rows = (long)num_seqs * num_q_heads;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long row = 0; row < n_rows; row++) {
        int b = (int)(row / num_q_heads);
        int h = (int)(row % num_q_heads);
        int g = h / G;
        int n = context_lens[b];
        size_t qo = (size_t)row * d;
        if (n == 0) {
            for (int i = 0; i < d; i++) out[qo + i] = 0.0;
            continue;
        }
        int nblk = (n + bs - 1) / bs;
        double *s = (double *)malloc((size_t)nblk * bs * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const int32_t *table = block_tables + (size_t)b * max_blocks_per_seq;
        /* scores, block by block */
        for (int blk = 0; blk < nblk; blk++) {
            int valid = n - blk * bs < bs ? n - blk * bs : bs;
            size_t base = ((size_t)table[blk] * num_kv_heads + g) * bs * d;
            for (int t = 0; t < valid; t++) {
                double acc = 0.0;
                for (int i = 0; i < d; i++)
                    acc += load_elem(q, qo + i, dtype) * load_elem(k_cache, base + (size_t)t * d + i, dtype);
                s[blk * bs + t] = scale * acc;
            }
        }
        /* one softmax over the whole context */
        double m = -INFINITY;
        for (int j = 0; j < n; j++) if (s[j] > m) m = s[j];
        double L = 0.0;
        for (int j = 0; j < n; j++) { s[j] = exp(s[j] - m); L += s[j]; }
        /* weighted V, block by block */
        for (int i = 0; i < d; i++) out[qo + i] = 0.0;
        for (int blk = 0; blk < nblk; blk++) {
            int valid = n - blk * bs < bs ? n - blk * bs : bs;
            size_t base = ((size_t)table[blk] * num_kv_heads + g) * bs * d;
            for (int t = 0; t < valid; t++)
                for (int i = 0; i < d; i++)
                    out[qo + i] += s[blk * bs + t] * load_elem(v_cache, base + (size_t)t * d + i, dtype);
        }
        for (int i = 0; i < d; i++) out[qo + i] /= L;
        free(s);
    }
    return failed ? PAO_E_ARG : PAO_OK;
}

/* (3) Partitioned.  The context is cut into partitions of partition_size
 * tokens (a multiple of block_size).  Inside a partition the softmax is kept
 * online, token by token: a running max m, a running sum l and an
 * unnormalised accumulator acc, all rescaled by exp(m_old - m_new) whenever
 * the max grows.  The partitions are then merged by log-sum-exp:
 *   M = max_p m_p,  w_p = exp(m_p - M),
 *   o = (sum_p w_p acc_p) / (sum_p w_p l_p).
 * This is the split-context decode the spec path adds on top of the
 * pages' one-softmax-over-the-whole-context rule; in exact arithmetic it
 * equals forms (1) and (2). */
int pao_decode_partitioned_f64(double *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int num_blocks,
                               int block_size, int max_blocks_per_seq, double scale,
                               int dtype, int partition_size, int nthreads)
{
    decode_args a = {q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, dtype, scale};
    if (partition_size <= 0 || block_size <= 0 || partition_size % block_size) return PAO_E_ARG;
    int rc = check_args(&a, out);
    if (rc != PAO_OK || num_seqs == 0) return rc;
    set_threads(nthreads);
    const int G = num_q_heads / num_kv_heads;
    const int d = head_dim;
    const long n_rows = (long)num_seqs * num_q_heads;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long row = 0; row < n_rows; row++) {
        int b = (int)(row / num_q_heads);
        int h = (int)(row % num_q_heads);
        int g = h / G;
        int n = context_lens[b];
        size_t qo = (size_t)row * d;
        if (n == 0) {
            for (int i = 0; i < d; i++) out[qo + i] = 0.0;
            continue;
        }
        int np = (n + partition_size - 1) / partition_size;
        double *m_p = (double *)malloc((size_t)np * sizeof(double));
        double *l_p = (double *)malloc((size_t)np * sizeof(double));
        double *acc_p = (double *)calloc((size_t)np * d, sizeof(double));
        if (!m_p || !l_p || !acc_p) {
            free(m_p); free(l_p); free(acc_p);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int p = 0; p < np; p++) {
            int j0 = p * partition_size;
            int j1 = j0 + partition_size < n ? j0 + partition_size : n;
            double m = -INFINITY, l = 0.0;
            double *acc = acc_p + (size_t)p * d;
            for (int j = j0; j < j1; j++) {
                double dot = 0.0;
                for (int i = 0; i < d; i++)
                    dot += load_elem(q, qo + i, dtype) * load_elem(k_cache, pool_index(&a, b, g, j, i), dtype);
                double sj = scale * dot;
                double m_new = sj > m ? sj : m;
                double alpha = exp(m - m_new);   /* exp(-inf) = 0 on the first token */
                double w = exp(sj - m_new);
                l = l * alpha + w;
                for (int i = 0; i < d; i++)
                    acc[i] = acc[i] * alpha + w * load_elem(v_cache, pool_index(&a, b, g, j, i), dtype);
                m = m_new;
            }
            m_p[p] = m;
            l_p[p] = l;
        }
        double M = -INFINITY;
        for (int p = 0; p < np; p++) if (m_p[p] > M) M = m_p[p];
        double den = 0.0;
        for (int i = 0; i < d; i++) out[qo + i] = 0.0;
        for (int p = 0; p < np; p++) {
            double w = exp(m_p[p] - M);
            den += w * l_p[p];
            for (int i = 0; i < d; i++) out[qo + i] += w * acc_p[(size_t)p * d + i];
        }
        for (int i = 0; i < d; i++) out[qo + i] /= den;
        free(m_p); free(l_p); free(acc_p);
    }
    return failed ? PAO_E_ARG : PAO_OK;
}

/* (4) Prefill: for sequence b the chunk's n_b = cu[b+1] - cu[b] query rows
 * are the last n_b positions of a sequence of n = context_lens[b] tokens
 * whose K/V (the chunk's included) are already in the cache ([P3] section
 * B.2: a prefill batch is packed by cu_seqlens_q; [P2] demo 1 prefills a
 * prompt, then decodes).  Row r of the chunk, at position p = n - n_b + r,
 * attends causally over positions 0..p:
 *   s_j = scale * sum_i q[r][h][i] K[j][i],   j <= p
 *   o[r][h][i] = (sum_{j<=p} exp(s_j - m) V[j][i]) / sum_{j<=p} exp(s_j - m),
 * m = max_{j<=p} s_j.  The gather is the same as in (1). */
int pao_prefill_concat_f64(double *out, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *block_tables,
                           const int32_t *cu_seqlens_q, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int num_blocks, int block_size, int max_blocks_per_seq,
                           double scale, int dtype, int nthreads)
{
    decode_args a = {q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, dtype, scale};
    int rc = check_args(&a, out);
    if (rc != PAO_OK || num_seqs == 0) return rc;
    if (!cu_seqlens_q || cu_seqlens_q[0] != 0) return PAO_E_ARG;
    for (int b = 0; b < num_seqs; b++) {
        int nq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        if (nq < 0 || nq > context_lens[b]) return PAO_E_ARG;
    }
    set_threads(nthreads);
    const int G = num_q_heads / num_kv_heads;
    const int d = head_dim;
    const long n_pairs = (long)num_seqs * num_kv_heads;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long pair = 0; pair < n_pairs; pair++) {
        int b = (int)(pair / num_kv_heads);
        int g = (int)(pair % num_kv_heads);
        int n = context_lens[b];
        int q0 = cu_seqlens_q[b], nq = cu_seqlens_q[b + 1] - q0;
        if (nq == 0) continue;
        double *K = (double *)malloc((size_t)n * d * sizeof(double));
        double *V = (double *)malloc((size_t)n * d * sizeof(double));
        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (!K || !V || !s) {
            free(K); free(V); free(s);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int j = 0; j < n; j++)
            for (int i = 0; i < d; i++) {
                K[(size_t)j * d + i] = load_elem(k_cache, pool_index(&a, b, g, j, i), dtype);
                V[(size_t)j * d + i] = load_elem(v_cache, pool_index(&a, b, g, j, i), dtype);
            }
        for (int r = 0; r < nq; r++) {
            int p = n - nq + r;               /* position of chunk row r */
            for (int h = g * G; h < (g + 1) * G; h++) {
                size_t qo = ((size_t)(q0 + r) * num_q_heads + h) * d;
                double m = -INFINITY;
                for (int j = 0; j <= p; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < d; i++)
                        acc += load_elem(q, qo + i, dtype) * K[(size_t)j * d + i];
                    s[j] = scale * acc;
                    if (s[j] > m) m = s[j];
                }
                double L = 0.0;
                for (int j = 0; j <= p; j++) {
                    s[j] = exp(s[j] - m);
                    L += s[j];
                }
                for (int i = 0; i < d; i++) {
                    double acc = 0.0;
                    for (int j = 0; j <= p; j++) acc += s[j] * V[(size_t)j * d + i];
                    out[qo + i] = acc / L;
                }
            }
        }
        free(K); free(V); free(s);
    }
    return failed ? PAO_E_ARG : PAO_OK;
}
