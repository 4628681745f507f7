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
// G <= 16, scale > 0): one wavefront serves 32 query-head columns of one KV
// head -- the G heads of 32 / G consecutive chunk rows -- on the
// 32x32x16 bf16 product, and walks the keys 0 .. (the last row's position)
// two 16-token tiles at a time: 8 score products S[32 keys x 32 columns],
// one online-softmax update over the 32 keys, and 8 P.V products; a
// column's causal limit is its row's position, applied only on the steps
// that reach past some column's row (or hold a tile with an invalid block
// id).  A workgroup of kWgWaves such wavefronts (consecutive units of one
// (sequence, KV head)) reads each K/V tile from memory once and shares it
// through LDS.
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
#define PA_PREFILL_WAVES_PER_EU 3
#endif

// ---------------------------------------------------------------------------
// Each tile (16 rows of K and of V, 8 KiB) is read from memory once per
// workgroup in 16-byte pieces, so every request covers whole 128-byte
// lines; the wavefronts then read their operands out of LDS: K as the
// score product's first operand (lane l: key l % 32 of the pair, 8 dims
// from 8 (l / 32) per 16-dim step), V through the transposing LDS read.
// LDS rows are padded (below), so the lanes that read one dim range of
// 32 K rows do not all fall in the same banks.  Four stages form a ring:
// while tiles 2p and 2p+1 are read and computed out of two of them, tiles
// 2p+2 and 2p+3 (loaded during the step before) are written into the other
// two and tiles 2p+4 and 2p+5 are loaded; one LDS-only barrier per step (no
// wait on the loads in flight).
// ---------------------------------------------------------------------------
#ifndef PA_PREFILL_WG_WAVES
#define PA_PREFILL_WG_WAVES 4
#endif
constexpr int kWgWaves = PA_PREFILL_WG_WAVES;
constexpr int kWgThreads = kWave * kWgWaves;
// 16-byte pieces of one tile: 256 of K, then 256 of V
constexpr int kPieces = 2 * kTile * kRowBytes / 16;
static_assert(kPieces % kWgThreads == 0, "tile pieces must divide over the workgroup");
constexpr int kPiecesPerThread = kPieces / kWgThreads;
// LDS row padding in bytes.  K rows of 272 bytes (68 banks of 4 bytes):
// the 16 rows that one K read spans start 4 banks apart and cover all 64.
// V rows of 320 bytes (80 banks): the four rows of one transposing read
// start 16 banks apart, and with the two 32-byte column halves the 32
// lanes of a pass cover all 64 banks.  Measured: no bank conflicts, where
// 288-byte rows for both had 17 M conflict cycles per launch of the
// chunked-prefill workload and ran 1.5% slower; unpadded V rows nearly
// halve the speed.
#ifndef PA_PREFILL_KPAD
#define PA_PREFILL_KPAD 16
#endif
#ifndef PA_PREFILL_VPAD
#define PA_PREFILL_VPAD 64
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

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Softmax state of one wavefront for its 32 columns (32x32x16 products):
// O^T block mb (dims 32 mb .. 32 mb + 31): lane holds column lane % 32 at
// dims 32 mb + 8 i + 4 (lane / 32) + j in o[mb][4 i + j].
struct Acc32 {
    f32x16 o[4];
    float m;
    float lsum;      // this lane's share (the other 16 keys sit in lane ^ 32)
};

// One step over a pair of 16-key tiles (32 keys) for the 32 columns.
//  scores: S[32 keys x 32 columns] = K_pair . Q^T, 8 x v_mfma_f32_32x32x16_bf16;
//          the lane holds column lane % 32 at keys 8 i + 4 (lane / 32) + j;
//  softmax: per column over its 16 keys and the partner lane's 16;
//  P.V:    O^T[32 mb + .., col] += V^T[dims, 16 keys] . P[16 keys, cols],
//          2 key blocks x 4 dim blocks; key block kb's k slot 8 h + 4 i' + j
//          is key 16 kb + 8 i' + 4 h + j (h = lane / 32) -- the order in
//          which the lane holds P -- and V arrives through the transposing
//          LDS read in the same order.
__device__ __forceinline__ void pair_update32(const char *stA, const char *stB,
                                              const bf16x8 (&qv)[8], int nv, bool okA, bool okB,
                                              float scale_log2, Acc32 &a, int lane) {
    const int col = lane & 31, half = lane >> 5;
    const char *krow = (col < 16 ? stA : stB) + (col & 15) * kLdsRowK + half * 16;
    f32x16 S = {};
#pragma unroll
    for (int kk = 0; kk < 8; kk++) {
        const u32x4 kr = *(const u32x4 *)(krow + 32 * kk);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr), qv[kk], S, 0,
                                                    0, 0);
    }
    float s[16];
    // a valid column sees every key of the pair unless the pair reaches past
    // its row or holds a tile with an invalid block id: then mask
    const bool need_mask = __ballot(nv < 32) != 0 || !okA || !okB;
    if (need_mask) {
        const int limA = okA ? nv : 0;
        const int limB = okB ? nv : 0;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int key = 8 * i + 4 * half + j;
                const int lim = i < 2 ? limA : limB;
                s[4 * i + j] = key < lim ? S[4 * i + j] : -INFINITY;
            }
    } else {
#pragma unroll
        for (int e = 0; e < 16; e++) s[e] = S[e];
    }
    float lmax = s[0];
#pragma unroll
    for (int e = 1; e < 16; e++) lmax = fmaxf(lmax, s[e]);
    const float tmax = xor32_max(lmax) * scale_log2;
#if PA_RESCALE_SLACK > 0
    const float m_new = tmax > a.m + (float)PA_RESCALE_SLACK ? tmax : a.m;
#else
    const float m_new = fmaxf(a.m, tmax);
#endif
    const float shift = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(a.m - shift);
    float pr[16];
#pragma unroll
    for (int e = 0; e < 16; e++) pr[e] = fast_exp2(fmaf(s[e], scale_log2, -shift));
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e++) ls += pr[e];
    a.lsum = a.lsum * alpha + ls;
    a.m = m_new;
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int mb = 0; mb < 4; mb++) a.o[mb] *= alpha;
    }
    bf16x8 pk[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
        pk[kb] = __builtin_bit_cast(
            bf16x8, (u32x4){pack_bf16x2(pr[8 * kb + 0], pr[8 * kb + 1]),
                            pack_bf16x2(pr[8 * kb + 2], pr[8 * kb + 3]),
                            pack_bf16x2(pr[8 * kb + 4], pr[8 * kb + 5]),
                            pack_bf16x2(pr[8 * kb + 6], pr[8 * kb + 7])});
    // transposing V reads: lane q of each 16-lane group reads 4 dims of key
    // row 8 i' + 4 half + q / 4 of the tile; lane i of the group receives
    // one dim (dbase + i) of the 4 keys
    const int q = lane & 15, g16 = lane >> 4;
    const int vrow0 = 4 * half + (q >> 2);
    const int vcol = (16 * (g16 & 1) + 4 * (q & 3)) * 2;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        const char *vt = (kb == 0 ? stA : stB) + kVBase + vcol;
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            const uint2 x = __builtin_bit_cast(
                uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) s16x4 *)(vt + vrow0 * kLdsRowV +
                                                                        64 * mb)));
            const uint2 y = __builtin_bit_cast(
                uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) s16x4 *)(vt + (vrow0 + 8) *
                                                                                 kLdsRowV +
                                                                        64 * mb)));
            a.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, (u32x4){x.x, x.y, y.x, y.y}), pk[kb], a.o[mb], 0, 0,
                0);
        }
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
    const int G = p.group;
    const int TPU = kPrefillCols / G;
    const int ubs = (p.units_per_seq + kWgWaves - 1) / kWgWaves;   // unit blocks per group
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

    // column lane % 32 = (row r0 + col / G, head g G + col % G)
    const int col = lane & 31, half = lane >> 5;
    const int r = r0 + col / G;
    const int head = g * G + col % G;
    const bool ok = col / G < TPU && r < r_end;
    const int rowid = q0 + r;
    const int ncol = ok ? first_pos + r + 1 : (1 << 30);
    bf16x8 qv[8];
    {
        const char *qrow = (const char *)p.q +
                           (((size_t)(ok ? rowid : q0) * p.num_q_heads + (ok ? head : 0)) * kD) * 2 +
                           16 * half;
#pragma unroll
        for (int kk = 0; kk < 8; kk++) {
            u32x4 raw = *(const u32x4 *)(qrow + 32 * kk);
            if (!ok) raw = (u32x4){0u, 0u, 0u, 0u};
            qv[kk] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    Acc32 a;
#pragma unroll
    for (int mb = 0; mb < 4; mb++) a.o[mb] = (f32x16){};
    a.m = -INFINITY;
    a.lsum = 0.f;

    const char *kbase = (const char *)p.k_cache;
    const char *vbase = (const char *)p.v_cache;
    const int32_t *table = tables + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.log2_block;
    const int bs_mask = (1 << log2bs) - 1;
    const int ntiles = (kmax + kTile - 1) / kTile;
    auto phys_of = [&](int t) -> int { return table[(min(t, ntiles - 1) * kTile) >> log2bs]; };
    auto issue = [&](int t, int phys, u32x4 (&gr)[kPiecesPerThread]) {
        const bool in = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
        const int rows = in ? min(kTile, kmax - t * kTile) : 0;
        const size_t off = ((((size_t)(in ? phys : 0) * p.num_kv_heads + g) << log2bs) +
                            ((t * kTile) & bs_mask)) * (size_t)kRowBytes;
#pragma unroll
        for (int j = 0; j < kPiecesPerThread; j++) {
            const int c = tid + j * kWgThreads;
            const int goff = ((c >> 4) & (kTile - 1)) * kRowBytes + (c & 15) * 16;
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
            const int row = c >> 4;
            const int lo = row < kTile ? row * kLdsRowK : kVBase + (row - kTile) * kLdsRowV;
            *(u32x4 *)(base + lo + (c & 15) * 16) = gr[j];
        }
    };

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
        pair_update32(lds + sa * kStage, lds + (sa + 1) * kStage, qv, ncol - t * kTile, okA, okB,
                      p.scale_log2, a, lane);
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
    const float lsum = xor32_sum(a.lsum);
    if (ok) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        char *orow = (char *)out + ((size_t)rowid * p.num_q_heads + head) * kD * 2;
#pragma unroll
        for (int mb = 0; mb < 4; mb++)
#pragma unroll
            for (int ii = 0; ii < 4; ii++)
                *(uint2 *)(orow + (32 * mb + 8 * ii + 4 * half) * 2) =
                    (uint2){pack_bf16x2(a.o[mb][4 * ii + 0] * inv, a.o[mb][4 * ii + 1] * inv),
                            pack_bf16x2(a.o[mb][4 * ii + 2] * inv, a.o[mb][4 * ii + 3] * inv)};
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
