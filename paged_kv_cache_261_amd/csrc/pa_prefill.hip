// pa_prefill.hip -- paged prefill: a chunk of new tokens per sequence, each
// attending causally over the paged cache up to its own position.
//
// What it computes ("04 - Paged Attention 实现进度", section B.2: a prefill
// batch is packed by cu_seqlens_q; "CS349E 第 7 讲 01_paged_attention.py",
// demo 1 prefills a prompt before decoding; demo 2 / paper eq. 4 for the
// per-query softmax over the paged cache): the chunk of sequence b is q rows
// cu[b] .. cu[b+1]-1, the last n_b positions of its context_lens[b] tokens
// (already written through slot_mapping); row r at position
// p = context_lens[b] - n_b + r attends over positions 0..p.
//
// How (matrix cores; bf16, head_dim 128, block_size >= 16, group size
// G <= 16): one wavefront serves 32 query-head columns of one KV head -- the
// G heads of TPU = 32 / G consecutive chunk rows (two 16-column groups that
// share every K/V load) -- and walks the keys 0 .. (its last row's position)
// in 16-token tiles with the tile step of pa_mfma_tile.h; a column's causal
// limit is its row's position, so the last tiles are partly masked per
// column.  Wavefronts of one (sequence, KV head) stream the same K/V tiles
// close together in time, so the repeats are served by L2.
//
// Order of the wavefronts: a unit's work grows with its sequence's context
// and its rows' positions, and the grid is many times larger than what is
// resident, so the dispatch order sets the end.  The (sequence, KV head)
// groups are ranked by context length, longest first, and dealt to the
// eight XCDs round-robin (group i to XCD i % 8: every XCD gets a share of
// long and short contexts); within a group the units run from the last
// rows (most keys) to the first.  All units of a group stay on one XCD and
// run back to back, which keeps its K/V tiles in that XCD's L2.
#include "pa_mfma_tile.h"

namespace pa {

// The sequence of rank r when sequences are ordered by context length,
// longest first (ties by index).  Each lane holds one sequence's length;
// with more sequences than lanes the order is the plain one.
__device__ __forceinline__ int seq_of_rank(const PrefillParams &p, const int32_t *ctx_lens,
                                           int r) {
    const int B = p.num_seqs;
    if (B > kWave) return r;
    const int lane = threadIdx.x;
    const int key = lane < B ? clamp_ctx(ctx_lens[lane], p.max_context_len) : -1;
    int rank = 0;
    for (int m = 0; m < B; m++) {
        const int km = __builtin_amdgcn_readlane(key, m);
        rank += (km > key || (km == key && m < lane)) ? 1 : 0;
    }
    // the ranks of lanes 0 .. B-1 are a permutation of 0 .. B-1
    return __builtin_ctzll(__ballot(lane < B && rank == r));
}

constexpr int kPrefillCols = kPrefillColumns;

#ifndef PA_PREFILL_WAVES_PER_EU
#define PA_PREFILL_WAVES_PER_EU 2
#endif

__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
void prefill_mfma_kernel(const PrefillParams args, const int32_t *__restrict__ tables,
                         const int32_t *__restrict__ cu_q, const int32_t *__restrict__ ctx_lens,
                         void *__restrict__ out) {
    const PrefillParams &p = args;
    const int lane = threadIdx.x;
    const Lane ln{lane & 15, lane >> 4};
    const int G = p.group;
    const int TPU = kPrefillCols / G;                       // chunk rows per wavefront
    // workgroup -> (XCD, slot on it) -> group i = (rank, KV head), unit u
    const int xcd = blockIdx.x % kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    const int i = (slot / p.units_per_seq) * kNumXcd + xcd;
    if (i >= p.num_seqs * p.num_kv_heads) return;
    const int u = p.units_per_seq - 1 - slot % p.units_per_seq;
    const int g = i % p.num_kv_heads;
    const int b = __builtin_amdgcn_readfirstlane(seq_of_rank(p, ctx_lens, i / p.num_kv_heads));
    const int q0 = __builtin_amdgcn_readfirstlane(cu_q[b]);
    const int nq = __builtin_amdgcn_readfirstlane(cu_q[b + 1]) - q0;
    const int r0 = u * TPU;                                 // first chunk row of the unit
    if (r0 >= nq) return;
    const int n = __builtin_amdgcn_readfirstlane(clamp_ctx(ctx_lens[b], p.max_context_len));
    const int first_pos = n - nq;                           // position of chunk row 0
    const int r_end = min(nq, r0 + TPU);
    const int kmax = first_pos + r_end;                     // keys 0 .. kmax-1
    if (kmax <= 0) return;

    // this lane's columns: column cg * 16 + row16 = head hj of chunk row r
    int ncol[kPrefillGroups], rowid[kPrefillGroups], head[kPrefillGroups];
    bool ok[kPrefillGroups];
    bf16x8 qv[kPrefillGroups][4];
    Acc a[kPrefillGroups];
#pragma unroll
    for (int cg = 0; cg < kPrefillGroups; cg++) {
        const int col = cg * 16 + ln.row16;
        const int r = r0 + col / G;
        head[cg] = g * G + col % G;
        ok[cg] = col / G < TPU && r < r_end;
        rowid[cg] = q0 + r;
        ncol[cg] = ok[cg] ? first_pos + r + 1 : 0;           // keys 0 .. its position
        const char *qrow = (const char *)p.q +
                           (((size_t)(ok[cg] ? rowid[cg] : q0) * p.num_q_heads +
                             (ok[cg] ? head[cg] : 0)) * kD + 8 * ln.grp) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            u32x4 raw = *(const u32x4 *)(qrow + 64 * kk);
            if (!ok[cg]) raw = (u32x4){0u, 0u, 0u, 0u};
            qv[cg][kk] = __builtin_bit_cast(bf16x8, raw);
        }
        acc_init(a[cg]);
    }

    const char *kbase = (const char *)p.k_cache;
    const char *vbase = (const char *)p.v_cache;
    const int32_t *table = tables + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.log2_block;
    const int bs_mask = (1 << log2bs) - 1;
    const int ntiles = (kmax + kTile - 1) / kTile;
    auto phys_of = [&](int t) -> int { return table[(min(t, ntiles - 1) * kTile) >> log2bs]; };
    auto issue = [&](int t, int phys, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
        const bool in = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
        const int rows = in ? min(kTile, kmax - t * kTile) : 0;
        const size_t off = ((((size_t)(in ? phys : 0) * p.num_kv_heads + g) << log2bs) +
                            ((t * kTile) & bs_mask)) * (size_t)kRowBytes;
        // default cache policy: the wavefronts of one (sequence, KV head)
        // read the same tiles in turn (with the non-temporal hint the
        // prefill took 0.61 ms instead of 0.48)
        load_tile_rows<kReuseAux>(kbase, vbase, off, rows, ln, kr, vr);
    };
    // phys[j]: block id of the tile in buffer j (kept, not re-read, so no
    // table read sits between a tile's compute and the next load)
    u32x4 kr[2][4], vr[2][4];
    int phys[2];
    phys[0] = phys_of(0);
    issue(0, phys[0], kr[0], vr[0]);
    int phys_next = phys_of(1);
    for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int t = t0 + j;
            if (t >= ntiles) break;
            phys[j ^ 1] = phys_next;
            issue(t + 1, phys_next, kr[j ^ 1], vr[j ^ 1]);
            phys_next = phys_of(t + 2);
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the wait
            if ((unsigned)phys[j] < (unsigned)p.num_blocks) {
#pragma unroll
                for (int cg = 0; cg < kPrefillGroups; cg++)
                    tile_update<true>(kr[j], vr[j], qv[cg], ncol[cg] - t * kTile, p.scale_log2,
                                      a[cg], ln);
            }
        }
    }
#pragma unroll
    for (int cg = 0; cg < kPrefillGroups; cg++) {
        acc_finish(a[cg]);
        if (ok[cg])
            store_row((char *)out + ((size_t)rowid[cg] * p.num_q_heads + head[cg]) * kD * 2,
                      a[cg], ln);
    }
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
    // groups dealt to the XCDs round-robin: kNumXcd * ceil(groups / kNumXcd)
    // slots of units_per_seq workgroups (the surplus ones return at once)
    const int64_t groups = (int64_t)p.num_seqs * p.num_kv_heads;
    const int64_t units = (groups + kNumXcd - 1) / kNumXcd * kNumXcd * p.units_per_seq;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_mfma_kernel, dim3((unsigned)units), dim3(kWave), 0, stream, p,
                       p.block_tables, p.cu_seqlens_q, p.context_lens, p.out);
    return hipGetLastError();
}

}  // namespace pa
