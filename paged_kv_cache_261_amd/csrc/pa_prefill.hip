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
// consecutive chunk rows -- and walks the keys 0 .. (the last row's position)
// in 16-token tiles with the tile step of pa_mfma_tile.h; a column's causal
// limit is its row's position, so the last tiles are partly masked per
// column.  A workgroup of kWgWaves such wavefronts (consecutive units of one
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
#define PA_PREFILL_WAVES_PER_EU 4
#endif

// ---------------------------------------------------------------------------
// Each tile (16 rows of K and of V, 8 KiB) is read from memory once per
// workgroup in 16-byte pieces, so every request covers whole 128-byte
// lines; the wavefronts then read the tile out of LDS in exactly the
// register layout of the tile step, so the arithmetic -- and every output
// bit -- is that of a wavefront loading the tile itself.  LDS rows are
// padded (below), so the 16 lanes that read one column of 16 K rows do not
// all fall in the same banks.  Two stages alternate: while tile t is read
// and computed out of one, tile t+1 is written into the other and tile t+3
// is loaded (two register sets hold the tiles in flight, so a load has two
// iterations to arrive); one LDS-only barrier per tile (no wait on the
// loads in flight).
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
// LDS row padding in bytes, measured: 32 for K and V (288-byte rows) ran
// 1-2% faster than 16 (the unpadded 256-byte stride puts every K row of a
// column read in the same banks)
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

__global__ __launch_bounds__(kWgThreads)
__attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
void prefill_mfma_kernel(const PrefillParams args, const int32_t *__restrict__ tables,
                         const int32_t *__restrict__ cu_q, const int32_t *__restrict__ ctx_lens,
                         void *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kStage];
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
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + off), (short)0, rows * kRowBytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + off), (short)0, rows * kRowBytes, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < kPiecesPerThread; j++) {
            const int c = tid + j * kWgThreads;
            const int goff = ((c >> 4) & (kTile - 1)) * kRowBytes + (c & 15) * 16;
            // K or V is the same for the whole wavefront (256 is a multiple of 64)
            const bool of_k = wave * kWave + j * kWgThreads < kPieces / 2;
            gr[j] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(of_k ? krs : vrs, goff, 0, kReuseAux));
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
    // The tile step's operands out of a stage.  K: the layout load_tile_rows
    // gives.  V: P.V product nn covers dims 16 nn .. 16 nn + 15 (not
    // 8 m + nn as in the decode kernels); lane L = row16 of group grp reads
    // the 8 bytes of row 4 grp + L / 4 at dims 16 nn + 4 (L % 4), and the
    // transposing LDS read (within each 16 lanes, lane i takes element i % 4
    // of the reads of lanes i / 4 + 4 k, k = 0..3) hands lane (m, grp) dim
    // 16 nn + m of tokens 4 grp .. 4 grp + 3: the operand the product takes,
    // with no byte permutes.
    auto stage_read = [&](int st, u32x4 (&kr)[4], s16x4 (&vt)[8]) {
        const char *base = lds + st * kStage;
#pragma unroll
        for (int j = 0; j < 4; j++)
            kr[j] = *(const u32x4 *)(base + ln.row16 * kLdsRowK + ln.grp * 16 + 64 * j);
        const char *vrow =
            base + kVBase + (4 * ln.grp + (ln.row16 >> 2)) * kLdsRowV + (ln.row16 & 3) * 8;
#pragma unroll
        for (int nn = 0; nn < 8; nn++)
            vt[nn] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(vrow + 32 * nn));
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

    // tile x is loaded into register set x % 2 three iterations ahead and
    // written to its stage at the end of the iteration before its own
    u32x4 gr[2][kPiecesPerThread];
    int ph0 = phys_of(0), ph1 = phys_of(1), ph2 = phys_of(2), ph3 = phys_of(3);
    issue(0, ph0, gr[0]);
    stage_write(0, gr[0]);
    issue(1, ph1, gr[1]);
    issue(2, ph2, gr[0]);
    lds_barrier();
    for (int t0 = 0; t0 < ntiles; t0 += 2) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int t = t0 + j;
            if (t >= ntiles) break;
            u32x4 kr[4];
            s16x4 vt[8];
            stage_read(j, kr, vt);
            if ((unsigned)ph0 < (unsigned)p.num_blocks) {
#pragma unroll
                for (int cg = 0; cg < kPrefillGroups; cg++)
                    tile_update_v<true>(kr, [&](int nn) { return vt[nn]; }, qv[cg],
                                        ncol[cg] - t * kTile, p.scale_log2, a[cg], ln);
            }
            if (t + 1 < ntiles) stage_write(j ^ 1, gr[j ^ 1]);
            issue(t + 3, ph3, gr[j ^ 1]);
            ph0 = ph1;
            ph1 = ph2;
            ph2 = ph3;
            ph3 = phys_of(t + 4);
            lds_barrier();
        }
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
