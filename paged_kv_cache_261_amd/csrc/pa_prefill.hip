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
// G <= 16): one wavefront serves 16 query-head columns of one KV head (16 x
// kPrefillGroups with the compile-time knob) -- the G heads of TPU = 16 / G
// consecutive chunk rows -- and walks the keys 0 .. (the last row's
// position) two 16-token tiles at a time: both score products (the decode
// tile step's layouts), one online-softmax update over the 32 keys, and P.V
// on the 16x16x32 matrix-core product; a column's causal limit is its row's
// position, so the last tiles are partly masked per column.  A workgroup of
// kWgWaves such wavefronts (consecutive units of one (sequence, KV head))
// reads each K/V tile from memory once and shares it through LDS.
//
// Order of the workgroups: a unit's work grows with its sequence's context
// and its rows' positions, and the grid is many times larger than what is
// resident, so the dispatch order sets the end.  The (sequence, KV head)
// groups are ranked by context length, longest first, and dealt to the
// eight XCDs round-robin (group i to XCD i % 8: every XCD gets a share of
// long and short contexts); within a group the unit blocks run from the
// last rows (most keys) to the first.  All blocks of a group stay on one XCD
// and run back to back, which keeps its K/V tiles in that XCD's L2.
#include "pa_mfma_tile.h"

namespace pa {

// The sequence of rank r when sequences are ordered by context length,
// longest first (ties by index).  Each lane holds one sequence's length;
// with more sequences than lanes the order is the plain one.
__device__ __forceinline__ int seq_of_rank(const PrefillParams &p, const int32_t *ctx_lens,
                                           int r) {
    const int B = p.num_seqs;
    if (B > kWave) return r;
    const int lane = threadIdx.x & (kWave - 1);
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
#define PA_PREFILL_WAVES_PER_EU 4
#endif

// ---------------------------------------------------------------------------
// Each tile (16 rows of K and of V, 8 KiB) is read from memory once per
// workgroup in 16-byte pieces, so every request covers whole 128-byte
// lines; the wavefronts then read their operands out of LDS: K in the
// register layout of the decode tile step, V through the transposing LDS
// read.  LDS rows are padded (below), so the 16 lanes that read one column
// of 16 K rows do not all fall in the same banks.  Four stages form a ring:
// while tiles 2p and 2p+1 are read and computed out of two of them, tiles
// 2p+2 and 2p+3 (loaded during the step before) are written into the other
// two and tiles 2p+4 and 2p+5 are loaded; one LDS-only barrier per step (no
// wait on the loads in flight).
// ---------------------------------------------------------------------------
#ifndef PA_PREFILL_WG_WAVES
#define PA_PREFILL_WG_WAVES 8
#endif
constexpr int kWgWaves = PA_PREFILL_WG_WAVES;
constexpr int kWgThreads = kWave * kWgWaves;
// 16-byte pieces of one tile: 256 of K, then 256 of V
constexpr int kPieces = 2 * kTile * kRowBytes / 16;
static_assert(kPieces % kWgThreads == 0, "tile pieces must divide over the workgroup");
constexpr int kPiecesPerThread = kPieces / kWgThreads;
// LDS row padding in bytes, measured: 32 for K and V (288-byte rows) is
// best; 16 or 64 run 6% slower, and unpadded V rows nearly halve the speed
// (the transposing reads of four rows then fall in the same banks)
#ifndef PA_PREFILL_KPAD
#define PA_PREFILL_KPAD 32
#endif
#ifndef PA_PREFILL_VPAD
#define PA_PREFILL_VPAD 32
#endif
constexpr int kLdsRowK = kRowBytes + PA_PREFILL_KPAD;   // LDS row strides (padded)
constexpr int kLdsRowV = kRowBytes + PA_PREFILL_VPAD;
constexpr int kVBase = kTile * kLdsRowK;                 // V rows follow the K rows
constexpr int kStage = kVBase + kTile * kLdsRowV;

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two consecutive tiles A and B in one step: both score products, one
// softmax update over their 32 keys, and P.V as one
// v_mfma_f32_16x16x32_bf16 per product whose k slots 8 grp .. 8 grp + 3
// hold tile A's tokens 4 grp .. 4 grp + 3 and 8 grp + 4 .. 8 grp + 7 tile
// B's -- the order in which the lane holds P.  okA / okB: the tile's block
// id is valid (a tile with an invalid id contributes nothing).
// The operands come straight out of the two stages, K of A, then K of B,
// then V, with scheduling fences between the score products, so no more
// than one tile's K is in registers at a time (the step fits four
// wavefronts per SIMD).
__device__ __forceinline__ void read_k(const char *stage, Lane ln, u32x4 (&kr)[4]) {
#pragma unroll
    for (int j = 0; j < 4; j++)
        kr[j] = *(const u32x4 *)(stage + ln.row16 * kLdsRowK + ln.grp * 16 + 64 * j);
}
__device__ __forceinline__ s16x4 read_vt(const char *stage, Lane ln, int nn) {
    const char *vrow =
        stage + kVBase + (4 * ln.grp + (ln.row16 >> 2)) * kLdsRowV + (ln.row16 & 3) * 8;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(vrow + 32 * nn));
}
// scheduling fences in the pair step: bit 0 after tile A's scores, bit 1
// after tile B's, bit 2 before the V reads (measured: 3 best, 0.2% over 7)
#ifndef PA_PAIR_FENCES
#define PA_PAIR_FENCES 3
#endif
__device__ __forceinline__ void pair_update(const char *stA, const char *stB,
                                            const bf16x8 (&qv)[4], int nv, bool okA, bool okB,
                                            float scale_log2, Acc &a, Lane ln) {
    f32x4 SA = {0.f, 0.f, 0.f, 0.f}, SB = {0.f, 0.f, 0.f, 0.f};
    {
        u32x4 kr[4];
        read_k(stA, ln, kr);
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]),
                                                         qv[kk], SA, 0, 0, 0);
    }
    if (PA_PAIR_FENCES & 1) __builtin_amdgcn_sched_barrier(0);
    {
        u32x4 kr[4];
        read_k(stB, ln, kr);
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]),
                                                         qv[kk], SB, 0, 0, 0);
    }
    if (PA_PAIR_FENCES & 2) __builtin_amdgcn_sched_barrier(0);
    // visible rows of each tile for this column (none when its block id is invalid)
    const int limA = okA ? nv : 0;
    const int limB = okB ? nv - kTile : 0;
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        s[i] = 4 * ln.grp + i < limA ? SA[i] * scale_log2 : -INFINITY;
        s[4 + i] = 4 * ln.grp + i < limB ? SB[i] * scale_log2 : -INFINITY;
    }
    const float lmax = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                             fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    const float tmax = xor32_max(xor16_max(lmax));
#if PA_RESCALE_SLACK > 0
    const float m_new = tmax > a.m + (float)PA_RESCALE_SLACK ? tmax : a.m;
#else
    const float m_new = fmaxf(a.m, tmax);
#endif
    const float shift = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(a.m - shift);
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; i++) pr[i] = fast_exp2(s[i] - shift);
    a.lsum = a.lsum * alpha +
             (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7])));
    a.m = m_new;
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int nn = 0; nn < 8; nn++) a.o[nn] *= alpha;
    }
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, (u32x4){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                        pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])});
    if (PA_PAIR_FENCES & 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nn = 0; nn < 8; nn++) {
        const uint2 x = __builtin_bit_cast(uint2, read_vt(stA, ln, nn));
        const uint2 y = __builtin_bit_cast(uint2, read_vt(stB, ln, nn));
        a.o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, (u32x4){x.x, x.y, y.x, y.y}), pb, a.o[nn], 0, 0, 0);
    }
}
constexpr int kStages = 4;

__global__ __launch_bounds__(kWgThreads)
__attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
void prefill_mfma_kernel(const PrefillParams args, const int32_t *__restrict__ tables,
                         const int32_t *__restrict__ cu_q, const int32_t *__restrict__ ctx_lens,
                         void *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) char lds[kStages * kStage];
    const PrefillParams &p = args;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Lane ln{lane & 15, lane >> 4};
    const int G = p.group;
    const int TPU = kPrefillCols / G;
    const int ubs = (p.units_per_seq + kWgWaves - 1) / kWgWaves;   // unit blocks per group
    // workgroup -> (XCD, slot on it) -> group i = (rank, KV head), unit block
    const int xcd = blockIdx.x % kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    const int i = (slot / ubs) * kNumXcd + xcd;
    if (i >= p.num_seqs * p.num_kv_heads) return;             // whole workgroup
    const int ub = ubs - 1 - slot % ubs;
    const int g = i % p.num_kv_heads;
    const int b = __builtin_amdgcn_readfirstlane(seq_of_rank(p, ctx_lens, i / p.num_kv_heads));
    const int q0 = __builtin_amdgcn_readfirstlane(cu_q[b]);
    const int nq = __builtin_amdgcn_readfirstlane(cu_q[b + 1]) - q0;
    const int wg_r0 = ub * kWgWaves * TPU;                    // first chunk row of the block
    if (wg_r0 >= nq) return;                                  // whole workgroup
    const int n = __builtin_amdgcn_readfirstlane(clamp_ctx(ctx_lens[b], p.max_context_len));
    const int first_pos = n - nq;
    const int wg_r_end = min(nq, wg_r0 + kWgWaves * TPU);
    const int kmax = first_pos + wg_r_end;                    // keys 0 .. kmax-1 for the block
    if (kmax <= 0) return;                                    // whole workgroup
    const int r0 = wg_r0 + wave * TPU;                        // this wavefront's first row
    const int r_end = min(nq, r0 + TPU);                      // r_end <= r0: no rows

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
        ncol[cg] = ok[cg] ? first_pos + r + 1 : 0;
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
    // thread tid moves pieces tid, tid + kWgThreads, ...: piece c is bytes
    // 16 (c % 16) .. of row (c / 16) % 16 of K (c < 256) or of V
    auto issue = [&](int t, int phys, u32x4 (&gr)[kPiecesPerThread]) {
        const bool in = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
        const int rows = in ? min(kTile, kmax - t * kTile) : 0;
        const size_t off = ((((size_t)(in ? phys : 0) * p.num_kv_heads + g) << log2bs) +
                            ((t * kTile) & bs_mask)) * (size_t)kRowBytes;
#pragma unroll
        for (int j = 0; j < kPiecesPerThread; j++) {
            const int c = tid + j * kWgThreads;
            const int goff = ((c >> 4) & (kTile - 1)) * kRowBytes + (c & 15) * 16;
            // K or V is the same for the whole wavefront (256 is a multiple of
            // 64), so only that pool's descriptor is built
            const bool of_k = wave * kWave + j * kWgThreads < kPieces / 2;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((of_k ? kbase : vbase) + off), (short)0, rows * kRowBytes, kRsrcWord3);
            gr[j] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, goff, 0, kReuseAux));
        }
    };
    auto stage_write = [&](int st, const u32x4 (&gr)[kPiecesPerThread]) {
        char *base = lds + st * kStage;
#pragma unroll
        for (int j = 0; j < kPiecesPerThread; j++) {
            const int c = tid + j * kWgThreads;
            const int row = c >> 4;   // 0..15: K row, 16..31: V row
            const int lo = row < kTile ? row * kLdsRowK : kVBase + (row - kTile) * kLdsRowV;
            *(u32x4 *)(base + lo + (c & 15) * 16) = gr[j];
        }
    };
    // O / l of column row16 in bfloat16: a.o[nn][i] holds dim 16 nn + 4 grp + i
    auto store_out_row = [&](char *out_row, const Acc &acc) {
        const float inv = acc.lsum > 0.f ? 1.f / acc.lsum : 0.f;
        char *dst = out_row + 8 * ln.grp;
#pragma unroll
        for (int nn = 0; nn < 8; nn++)
            *(uint2 *)(dst + 32 * nn) =
                (uint2){pack_bf16x2(acc.o[nn][0] * inv, acc.o[nn][1] * inv),
                        pack_bf16x2(acc.o[nn][2] * inv, acc.o[nn][3] * inv)};
    };

    // tiles 2p and 2p+1 are computed in step p out of stages (2p) % 4 and
    // (2p+1) % 4; tiles 2p+2, 2p+3 (loaded during step p-1) are written into
    // the stages step p-1 read, and tiles 2p+4, 2p+5 are loaded.  Tiles past
    // the last are written too (as zeros: their loads read nothing), so no
    // stale LDS bits meet a zero probability.
    const int ntiles2 = (ntiles + 1) & ~1;
    u32x4 gr[2][kPiecesPerThread];
    int phA = phys_of(0), phB = phys_of(1);
    issue(0, phA, gr[0]);
    issue(1, phB, gr[1]);
    stage_write(0, gr[0]);
    stage_write(1, gr[1]);
    int phC = phys_of(2), phD = phys_of(3);
    issue(2, phC, gr[0]);
    issue(3, phD, gr[1]);
    lds_barrier();
    for (int t = 0; t < ntiles; t += 2) {
        const int sa = t & 3;
        const bool okA = (unsigned)phA < (unsigned)p.num_blocks;
        const bool okB = (unsigned)phB < (unsigned)p.num_blocks;
#pragma unroll
        for (int cg = 0; cg < kPrefillGroups; cg++)
            pair_update(lds + sa * kStage, lds + (sa + 1) * kStage, qv[cg], ncol[cg] - t * kTile,
                        okA, okB, p.scale_log2, a[cg], ln);
        if (t + 2 < ntiles2) {
            stage_write((t + 2) & 3, gr[0]);
            stage_write((t + 3) & 3, gr[1]);
        }
        phA = phC;
        phB = phD;
        phC = phys_of(t + 4);
        phD = phys_of(t + 5);
        issue(t + 4, phC, gr[0]);
        issue(t + 5, phD, gr[1]);
        lds_barrier();
    }
#pragma unroll
    for (int cg = 0; cg < kPrefillGroups; cg++) {
        acc_finish(a[cg]);
        if (ok[cg])
            store_out_row((char *)out + ((size_t)rowid[cg] * p.num_q_heads + head[cg]) * kD * 2,
                          a[cg]);
    }
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
    const int64_t groups = (int64_t)p.num_seqs * p.num_kv_heads;
    const int64_t ubs = (p.units_per_seq + kWgWaves - 1) / kWgWaves;
    const int64_t wgs = (groups + kNumXcd - 1) / kNumXcd * kNumXcd * ubs;
    if (wgs == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_mfma_kernel, dim3((unsigned)wgs), dim3(kWgThreads), 0,
                       stream, p, p.block_tables, p.cu_seqlens_q, p.context_lens, p.out);
    return hipGetLastError();
}
}  // namespace pa
