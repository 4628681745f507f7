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
// workgroup, straight into an LDS stage by buffer loads with an LDS
// destination: one such load moves 1 KiB (64 lanes x 16 bytes, four rows),
// and each of the four wavefronts moves two of a tile's eight (K rows 0-15
// by wavefronts 0 and 1, V rows by 2 and 3).  The wavefronts then read their
// operands out of LDS: K as the score product's first operand (lane l: key
// l % 32 of the pair, 8 dims from 8 (l / 32) per 16-dim step), V through the
// transposing LDS read.
//
// A load writes its 64 lanes' bytes contiguously, so rows cannot be padded;
// instead the 16 16-byte pieces of a row are permuted (the permutation is
// applied to the global addresses the lanes load from): K row r holds
// piece c at slot c ^ r, so the 16 rows that one K read spans sit in 16
// different slots and cover all 64 banks; V row r holds piece c at slot
// c ^ 4 (r & 3), so the four rows of one transposing read start 16 banks
// apart.  No bank conflicts either way.
//
// Six stages (three pairs) form a ring: step p computes pair p out of two
// of them while pair p+1 (issued the step before) lands, and first issues
// pair p+2 into the two that pair p-1 used; before its barrier each
// wavefront waits for its own loads of pair p+1 (the four it issued most
// recently, pair p+2's, stay in flight).  Loads past a descriptor's size
// write zeros, so rows past the context and tiles past the last arrive as
// zeros, and no stale LDS bits meet a zero probability.
// ---------------------------------------------------------------------------
#ifndef PA_PREFILL_WG_WAVES
#define PA_PREFILL_WG_WAVES 4
#endif
constexpr int kWgWaves = PA_PREFILL_WG_WAVES;
static_assert(kWgWaves == 4, "each wavefront moves two 1 KiB quarters of K or of V per tile");
constexpr int kWgThreads = kWave * kWgWaves;
constexpr int kLdsRow = kRowBytes;                 // unpadded rows (pieces permuted)
constexpr int kVBase = kTile * kLdsRow;            // V rows follow the K rows
constexpr int kStage = kVBase + kTile * kLdsRow;   // 8 KiB
constexpr int kStages = 6;

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

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// P.V operand of dim block mb out of the tile whose V rows start at LDS byte
// vrow (row vrow0 of the stage, column vcol applied): two transposing reads,
// rows vrow0 and vrow0 + 8 -- the lane's 8 k slots.  The piece at byte
// column vcol of row r sits at slot ^ 4 (r & 3), i.e. 64 (q >> 2) bytes on,
// which the caller folds into vcol; dim block mb flips bits 6-7.
__device__ __forceinline__ u32x4 read_v_operand(unsigned vrow, int mb) {
    const unsigned va = vrow ^ (64u * mb);
    const uint2 x =
        __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(size_t)va));
    const uint2 y = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(size_t)(va + 8 * kLdsRow)));
    return (u32x4){x.x, x.y, y.x, y.y};
}

// One step over a pair of 16-key tiles (32 keys) for the 32 columns.
//  scores: S[32 keys x 32 columns] = K_pair . Q^T, 8 x v_mfma_f32_32x32x16_bf16;
//          the lane holds column lane % 32 at keys 8 i + 4 (lane / 32) + j;
//  softmax: per column over its 16 keys and the partner lane's 16;
//  P.V:    O^T[32 mb + .., col] += V^T[dims, 16 keys] . P[16 keys, cols],
//          2 key blocks x 4 dim blocks; key block kb's k slot 8 h + 4 i' + j
//          is key 16 kb + 8 i' + 4 h + j (h = lane / 32) -- the order in
//          which the lane holds P -- and V arrives through the transposing
//          LDS read in the same order.
// stA / stB: LDS byte offsets of the pair's two stages.
__device__ __forceinline__ void pair_update32(unsigned stA, unsigned stB,
                                              const bf16x8 (&qv)[8], int nv, bool okA, bool okB,
                                              float scale_log2, Acc32 &a, int lane) {
    const int col = lane & 31, half = lane >> 5;
    // piece 2 kk + half of row krw sits at slot (2 kk + half) ^ krw
    //   = 2 kk ^ (half ^ krw): the row's address with slot half ^ krw, xor 32 kk
    const int krw = col & 15;
    const unsigned kaddr = (col < 16 ? stA : stB) + (unsigned)(krw * kLdsRow) +
                           (unsigned)(((half ^ krw) & 15) << 4);
    f32x16 S = {};
#pragma unroll
    for (int kk = 0; kk < 8; kk++) {
        const u32x4 kr = *(const lds_u32x4 *)(size_t)(kaddr ^ (32u * kk));
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr), qv[kk], S, 0,
                                                    0, 0);
    }
    // transposing V reads: lane q of each 16-lane group reads 4 dims of key
    // row 8 i' + 4 half + q / 4 of the tile; lane i of the group receives
    // one dim (dbase + i) of the 4 keys.  Tile A's operands are read here,
    // so they arrive while the softmax runs; tile B's after it (registers).
    const int q = lane & 15, g16 = lane >> 4;
    const int vrow0 = 4 * half + (q >> 2);
    const unsigned vcol = (unsigned)((16 * (g16 & 1) + 4 * (q & 3)) * 2 + 64 * (q >> 2));
    const unsigned vrowA = stA + (unsigned)(kVBase + vrow0 * kLdsRow) + vcol;
    const unsigned vrowB = stB + (unsigned)(kVBase + vrow0 * kLdsRow) + vcol;
    u32x4 vA[4];
#pragma unroll
    for (int mb = 0; mb < 4; mb++) vA[mb] = read_v_operand(vrowA, mb);
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
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
        a.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vA[mb]), pk[0],
                                                          a.o[mb], 0, 0, 0);
#pragma unroll
    for (int mb = 0; mb < 4; mb++)
        a.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, read_v_operand(vrowB, mb)), pk[1], a.o[mb], 0, 0, 0);
}
// s_waitcnt operand that waits until at most n vector memory operations of
// this wavefront are outstanding (the other counters untouched)
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__global__ __launch_bounds__(kWgThreads)
__attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
void prefill_mfma_kernel(const PrefillParams args, const int32_t *__restrict__ tables,
                         const int32_t *__restrict__ cu_q, const int32_t *__restrict__ ctx_lens,
                         void *__restrict__ out) {
    __shared__ __attribute__((aligned(1024))) char lds[kStages * kStage];
    const unsigned lds0 = (unsigned)(size_t)(__attribute__((address_space(3))) char *)lds;
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
    // this wavefront's two 1 KiB quarters of every tile: quarter c = 2 wave + jj
    // (0-3: K rows 4c .. 4c+3; 4-7: V rows 4(c-4) ..); lane l writes LDS bytes
    // 16 l of the quarter: row 4 (c & 3) + l / 16, slot l % 16, which holds
    // piece (l % 16) ^ r (K) or (l % 16) ^ 4 (r & 3) (V) of that row
    const bool moves_k = wave < 2;
    unsigned voff[2];
#pragma unroll
    for (int jj = 0; jj < 2; jj++) {
        const int row = 4 * ((2 * wave + jj) & 3) + (lane >> 4);
        const int sl = lane & 15;
        const int piece = moves_k ? (sl ^ row) : (sl ^ (4 * (row & 3)));
        voff[jj] = (unsigned)(row * kRowBytes + piece * 16);
    }
    // Buffer load of tile t (block id phys) into stage st.  Issued from an
    // asm statement: a buffer-to-LDS load from the builtin makes the compiler
    // wait for every such load in flight before any later LDS read (it
    // cannot tell the stages apart, even as separate LDS arrays addressed
    // through their own pointers), which would void the two-pair lead.
    // The statement has no register outputs (the data goes to LDS); its
    // completion is awaited explicitly before the barrier that publishes the
    // stage.
    auto load_tile = [&](int t, int st) {
        const int phys = phys_of(t);
        const bool in = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
        const int rows = in ? min(kTile, kmax - t * kTile) : 0;
        const size_t off = ((((size_t)(in ? phys : 0) * p.num_kv_heads + g) << log2bs) +
                            ((t * kTile) & bs_mask)) * (size_t)kRowBytes;
        const uint64_t base = (uint64_t)(size_t)((moves_k ? kbase : vbase) + off);
        typedef int i32x4v __attribute__((ext_vector_type(4)));
        const i32x4v rs = {(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu),
                           rows * kRowBytes, kRsrcWord3};
        const unsigned m0base = lds0 + (unsigned)(st * kStage + 2 * wave * 1024);
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const unsigned m0v = __builtin_amdgcn_readfirstlane(m0base + jj * 1024);
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :
                         : "s"(m0v), "v"(voff[jj]), "s"(rs)
                         : "memory", "m0");
        }
    };
    const int npairs = (ntiles + 1) >> 1;
    load_tile(0, 0);
    load_tile(1, 1);
    load_tile(2, 2);
    load_tile(3, 3);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(4));
    lds_barrier();
    int sp = 0;   // stage pair (0, 1, 2) of pair p
    for (int pp = 0; pp < npairs; pp++) {
        const int t = 2 * pp;
        const int sw = sp == 0 ? 2 : sp - 1;   // pair p+2 goes where pair p-1 was
        load_tile(t + 4, 2 * sw);
        load_tile(t + 5, 2 * sw + 1);
        const bool okA = (unsigned)phys_of(t) < (unsigned)p.num_blocks;
        const bool okB = (unsigned)phys_of(t + 1) < (unsigned)p.num_blocks;
        pair_update32(lds0 + (unsigned)(2 * sp * kStage), lds0 + (unsigned)((2 * sp + 1) * kStage),
                      qv, ncol - t * kTile, okA, okB, p.scale_log2, a, lane);
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(4));
        lds_barrier();
        sp = sp == 2 ? 0 : sp + 1;
    }
    // The last four loads (tiles past the last pair, zero-sized) may still be
    // in flight; the compiler does not count loads issued from asm, so drain
    // them here, before the workgroup's LDS can be handed to another.
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
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
