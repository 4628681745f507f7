// pa_decode_vector.hip -- PagedAttention decode on the vector ALUs.
//
// What it computes ("CS349E 第 7 讲 01_paged_attention.py", demo 2, paper
// eq. 4): for each sequence b and query head h (KV head g = h / G), the
// scores of h against every cached token, block by block through the block
// table ("PagedAttention实现": a position's logical block is position /
// block_size, its offset position % block_size, the page table gives the
// physical block), one softmax over the whole context, and the
// probability-weighted sum of V.
//
// How (one wavefront per work unit = (sequence, KV head, partition)):
//  - a token's head_dim row is split into 16-byte chunks; LPT = head_dim /
//    (16 / elem_bytes) lanes hold one token, so one wavefront pass covers
//    TPW = 64 / LPT tokens with one 16-byte load per lane for K and one for
//    V (the TPW rows of a pass are contiguous in memory whenever
//    block_size >= TPW);
//  - every lane keeps the q chunk of all G query heads of its KV head, so
//    each K/V load serves the whole group;
//  - dot products are completed with a butterfly over the LPT lanes of a
//    token (cross-lane shuffles);
//  - each token slot r of the pass runs its own online softmax (running max
//    m, running sum l, accumulator acc rescaled by 2^(m_old - m_new)); the
//    TPW slot states are merged at the end by the log-sum-exp rule;
//  - scores live in base-2 log domain (scale * log2 e folded in), so the
//    exponentials are single v_exp_f32 instructions;
//  - the loads of the next pass are issued before the current pass is
//    computed.
// Tokens at or beyond the context length are selected out (score -inf,
// never multiplied in), so whatever the unused slots hold never reaches the
// output.
#include "pa_internal.h"
#include "pa_vector_chunk.h"

#include <math.h>

namespace pa {

// T: storage type (float, or uint16_t holding bfloat16 bits).  D: head_dim.
// GP: query heads handled per KV head, a power of two >= group (extra heads
// are computed on zeros and never stored).
template <typename T, int D, int GP>
__global__ __launch_bounds__(kWave) void decode_vector_kernel(const DecodeParams p) {
    constexpr int kVec = Chunk<T>::kVec;
    constexpr int LPT = D / kVec;              // lanes per token row
    constexpr int TPW = kWave / LPT;           // tokens per wavefront pass
    static_assert(LPT >= 1 && LPT <= kWave && kWave % LPT == 0, "head_dim");

    const int lane = threadIdx.x;
    const int r = lane / LPT;                  // token slot within a pass
    const int c = lane % LPT;                  // 16-byte chunk of head_dim

    const int u = xcd_remap(blockIdx.x, p.num_units);
    const Unit w = unit_of(u, p.num_seqs, p.num_kv_heads);
    const int n = clamp_ctx(p.context_lens[w.b], p.max_context_len);
    const int P = p.partition_size;
    const int t0 = w.part * P;
    const int n_parts = n == 0 ? 1 : (n + P - 1) / P;
    if (w.part >= n_parts) return;             // nothing in this partition
    const int t1 = min(n, t0 + P);

    const int G = p.group;
    const int bs_mask = (1 << p.log2_block) - 1;
    const T *kc = (const T *)p.k_cache;
    const T *vc = (const T *)p.v_cache;
    const int32_t *table = p.block_tables + (size_t)w.b * p.max_blocks_per_seq;

    // q chunk c of every head in the group
    float q[GP][kVec];
#pragma unroll
    for (int j = 0; j < GP; j++) {
        if (j < G) {
            const int h = w.g * G + j;
            const uint4 raw =
                *(const uint4 *)((const T *)p.q + ((size_t)w.b * p.num_q_heads + h) * D + c * kVec);
            Chunk<T>::unpack(raw, q[j]);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; e++) q[j][e] = 0.f;
        }
    }

    float m[GP], l[GP], acc[GP][kVec];
#pragma unroll
    for (int j = 0; j < GP; j++) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < kVec; e++) acc[j][e] = 0.f;
    }

    // Address of this lane's chunk of token tok (or -1 if the token is not
    // visible or its block id is out of range).
    auto chunk_offset = [&](int tok) -> int64_t {
        if (tok >= t1) return -1;
        const int phys = table[tok >> p.log2_block];
        if ((unsigned)phys >= (unsigned)p.num_blocks) return -1;
        return ((((int64_t)phys * p.num_kv_heads + w.g) << p.log2_block) + (tok & bs_mask)) * D +
               c * kVec;
    };
    const uint4 zero = {0u, 0u, 0u, 0u};
    int64_t off = chunk_offset(t0 + r);
    uint4 kraw = off >= 0 ? *(const uint4 *)(kc + off) : zero;
    uint4 vraw = off >= 0 ? *(const uint4 *)(vc + off) : zero;

    for (int base = t0; base < t1; base += TPW) {
        // issue the next pass's loads before working on this one
        const int64_t off_n = chunk_offset(base + TPW + r);
        const uint4 kraw_n = off_n >= 0 ? *(const uint4 *)(kc + off_n) : zero;
        const uint4 vraw_n = off_n >= 0 ? *(const uint4 *)(vc + off_n) : zero;

        const bool valid = off >= 0;
        float kf[kVec], vf[kVec];
        Chunk<T>::unpack(kraw, kf);
        Chunk<T>::unpack(vraw, vf);
#pragma unroll
        for (int j = 0; j < GP; j++) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; e++) dot = fmaf(q[j][e], kf[e], dot);
#pragma unroll
            for (int o = LPT / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
            const float s = valid ? dot * p.scale_log2 : -INFINITY;
            const float m_new = fmaxf(m[j], s);
            if (m_new != -INFINITY) {          // nothing seen yet: state stays empty
                const float alpha = fast_exp2(m[j] - m_new);
                const float pw = fast_exp2(s - m_new);
                l[j] = l[j] * alpha + pw;
#pragma unroll
                for (int e = 0; e < kVec; e++) acc[j][e] = fmaf(acc[j][e], alpha, pw * vf[e]);
                m[j] = m_new;
            }
        }
        off = off_n;
        kraw = kraw_n;
        vraw = vraw_n;
    }

    // merge the TPW token-slot states (lanes with the same chunk c)
#pragma unroll
    for (int o = LPT; o < kWave; o <<= 1) {
#pragma unroll
        for (int j = 0; j < GP; j++) {
            const float m_o = __shfl_xor(m[j], o);
            const float l_o = __shfl_xor(l[j], o);
            const float mm = fmaxf(m[j], m_o);
            const float fa = m[j] == -INFINITY ? 0.f : fast_exp2(m[j] - mm);
            const float fb = m_o == -INFINITY ? 0.f : fast_exp2(m_o - mm);
            l[j] = l[j] * fa + l_o * fb;
#pragma unroll
            for (int e = 0; e < kVec; e++) {
                const float a_o = __shfl_xor(acc[j][e], o);
                acc[j][e] = acc[j][e] * fa + a_o * fb;
            }
            m[j] = mm;
        }
    }

    if (r != 0) return;
#pragma unroll
    for (int j = 0; j < GP; j++) {
        if (j >= G) continue;
        const int h = w.g * G + j;
        const size_t row = (size_t)w.b * p.num_q_heads + h;
        if (n_parts == 1) {
            const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
            float o[kVec];
#pragma unroll
            for (int e = 0; e < kVec; e++) o[e] = acc[j][e] * inv;
            Chunk<T>::pack_store((T *)p.out + row * D + c * kVec, o);
        } else {
            const size_t prow = row * p.num_partitions + w.part;
            float *dst = p.ws_acc + prow * D + c * kVec;
#pragma unroll
            for (int e = 0; e < kVec; e++) dst[e] = acc[j][e];
            if (c == 0) {
                p.ws_m[prow] = m[j];
                p.ws_l[prow] = l[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Work-balanced split on the vector ALUs (block_size >= 16).
//
// W persistent wavefronts split the stream of 16-token tiles (KV head
// slowest, then sequence, then tile; a sequence of n tokens has ceil(n/16)
// tiles per KV head) into equal contiguous shares, exactly as the
// matrix-core balanced split does, so the same merge kernel combines the
// pieces: a wavefront finishes the units it covers whole in place and
// leaves its first and last unit, if partial, in its partial slots 0 and 1.
//
// A tile of one (block, KV head) is 16 contiguous rows of head_dim values.
// Lane (r, c) = (lane / LPT, lane % LPT) loads 16-byte chunk c of row
// i * TPW + r in pass i, through a buffer descriptor that covers only the
// tile's visible rows (the rest read as zero), so the tile loop has no
// branches and the loads of the next tiles are in flight while one is
// computed.  The block-table entry of a tile is
// read with a scalar load one tile ahead.  Dot products are completed over
// the LPT lanes of a row with DPP adds (quad permutes, half-row and row
// mirrors) and row-swap permutes; each token slot r keeps its own online
// softmax state, folded in once per tile, and the TPW slot states are
// merged by log-sum-exp at the end of a unit.
// ---------------------------------------------------------------------------
constexpr int kTileTok = 16;

// Sum over aligned groups of LPT lanes (LPT a power of two <= 64).
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false);
    return v + __int_as_float(moved);
}

template <int LPT>
__device__ __forceinline__ float lane_group_sum(float x) {
    if (LPT >= 2) x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    if (LPT >= 4) x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    if (LPT >= 8) x = dpp_add<0x141>(x);   // row_half_mirror: the other quad of 8
    if (LPT >= 16) x = dpp_add<0x140>(x);  // row_mirror: the other half of the row
    if (LPT >= 32) {                        // the other row of 16 (lane ^ 16)
        const uint32_t u = __float_as_uint(x);
        const auto rr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        x = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
    }
    if (LPT >= 64) {                        // the other half of the wave (lane ^ 32)
        const uint32_t u = __float_as_uint(x);
        const auto rr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        x = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
    }
    return x;
}

template <typename T, int D, int GP>
struct VecShape {
    static constexpr int kVec = Chunk<T>::kVec;
    static constexpr int LPT = D / kVec;            // lanes per token row
    static constexpr int TPW = kWave / LPT;         // rows per load instruction
    static constexpr int PASSES = kTileTok / TPW;   // loads per lane per tile, K or V
    static constexpr int kRow = D * (int)sizeof(T);
    // tiles in flight while one is computed: as many as the registers allow
    // (a tile buffer is 2 * PASSES * 4 VGPRs, the state of the heads
    // GP * (2 kVec + 2))
    static constexpr int kBuf = 2 * PASSES * 4, kState = GP * (2 * kVec + 2);
    static constexpr int DEPTH = PASSES >= 8                      ? 1
                                 : 4 * kBuf + kState <= 320 ? 3
                                 : 3 * kBuf + kState <= 360 ? 2
                                                            : 1;
    static constexpr int BUFS = DEPTH + 1;
    static constexpr bool kOk = TPW <= kTileTok;
};

template <typename T, int D, int GP>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(1)))
void decode_vector_balanced_kernel(const DecodeParams args, const int32_t *__restrict__ tables,
                                   const int32_t *__restrict__ ctx_lens, void *__restrict__ out,
                                   float *__restrict__ ws_m, float *__restrict__ ws_l,
                                   float *__restrict__ ws_acc) {
    using S = VecShape<T, D, GP>;
    constexpr int kVec = S::kVec, LPT = S::LPT, TPW = S::TPW, PASSES = S::PASSES;
    constexpr int kRow = S::kRow, DEPTH = S::DEPTH, BUFS = S::BUFS;
    static_assert(S::kOk, "a tile of 16 rows must cover whole load passes");
    // restrict arguments: the stores cannot alias the block tables, so the
    // per-tile table reads stay on the scalar unit
    DecodeParams p = args;
    p.block_tables = tables;
    p.context_lens = ctx_lens;
    const int lane = threadIdx.x;
    const int r = lane / LPT;                  // token slot within a pass
    const int c = lane % LPT;                  // 16-byte chunk of head_dim
    const int W = p.num_units;
    const int w = blockIdx.x;       // launch order: see xcd_remap
    const int B = p.num_seqs;
    const int G = p.group;

    // tile prefix over sequences: lane i owns sequences [i K, i K + K)
    const int K = (B + kWave - 1) / kWave;
    auto tiles_of = [&](int b) {
        return (clamp_ctx(p.context_lens[b], p.max_context_len) + kTileTok - 1) / kTileTok;
    };
    int local = 0;
    for (int j = 0; j < K; j++) {
        const int b = lane * K + j;
        if (b < B) local += tiles_of(b);
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    const int excl = incl - local;
    const int TT = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1));
    const int total = TT * p.num_kv_heads;
    const int C = (total + W - 1) / W;

    const char *kbase = (const char *)p.k_cache;
    const char *vbase = (const char *)p.v_cache;
    const int log2bs = p.log2_block;
    const int bs_mask = (1 << log2bs) - 1;
    const int x1 = min(w * C + C, total);
    int x = w * C;
    int slot = 0;
    while (x < x1) {
        const int g = x / TT;
        const int rr = x - g * TT;
        // the sequence holding stream position rr: find its lane, then walk
        const unsigned long long own = __ballot(rr >= excl && rr < incl);
        const int jl = __builtin_ctzll(own);
        int base = __builtin_amdgcn_readfirstlane(__shfl(excl, jl));
        int b = jl * K;
        int Tb;
        if (K == 1) {
            Tb = __builtin_amdgcn_readfirstlane(__shfl(local, jl));
        } else {
            Tb = __builtin_amdgcn_readfirstlane(tiles_of(b));
            while (rr >= base + Tb) {
                base += Tb;
                b++;
                Tb = __builtin_amdgcn_readfirstlane(tiles_of(b));
            }
        }
        const int t_begin = rr - base;                 // tiles [t_begin, t_end) of unit (g, b)
        const int t_end = min(Tb, t_begin + (x1 - x));
        x += t_end - t_begin;
        const int n = __builtin_amdgcn_readfirstlane(clamp_ctx(p.context_lens[b], p.max_context_len));

        // q chunk c of every head of the group (zeros past G)
        float q[GP][kVec];
#pragma unroll
        for (int j = 0; j < GP; j++) {
            if (j < G) {
                const uint4 raw = *(const uint4 *)((const T *)p.q +
                                                   ((size_t)b * p.num_q_heads + g * G + j) * D +
                                                   c * kVec);
                Chunk<T>::unpack(raw, q[j]);
            } else {
#pragma unroll
                for (int e = 0; e < kVec; e++) q[j][e] = 0.f;
            }
        }
        float m[GP], l[GP], acc[GP][kVec];
#pragma unroll
        for (int j = 0; j < GP; j++) {
            m[j] = -INFINITY;
            l[j] = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; e++) acc[j][e] = 0.f;
        }

        const int32_t *__restrict__ table = p.block_tables + (size_t)b * p.max_blocks_per_seq;
        const int ntiles = t_end - t_begin;
        auto phys_of = [&](int t) -> int {             // t clamped into the range
            const int tt = t_begin + (t < ntiles ? t : ntiles - 1);
            return table[(tt * kTileTok) >> log2bs];
        };
        auto load_tile = [&](int t, int phys, uint4 (&kr)[PASSES], uint4 (&vr)[PASSES]) -> int {
            const int tok = (t_begin + t) * kTileTok;
            const bool ok = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
            const int rows = ok ? min(kTileTok, n - tok) : 0;
            const size_t off = ((((size_t)(ok ? phys : 0) * p.num_kv_heads + g) << log2bs) +
                                (tok & bs_mask)) * (size_t)kRow;
            const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + off), (short)0, rows * kRow, 0x00020000);
            const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vbase + off), (short)0, rows * kRow, 0x00020000);
#pragma unroll
            for (int i = 0; i < PASSES; i++) {
                const int lo = (i * TPW + r) * kRow + c * 16;
                // non-temporal: each tile is read once (evict-first lines)
                kr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, lo, 0, 2));
                vr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, lo, 0, 2));
            }
            return rows;
        };
        // fold one tile (rows visible) into the slot states
        auto update = [&](const uint4 (&kr)[PASSES], const uint4 (&vr)[PASSES], int rows) {
#pragma unroll
            for (int j = 0; j < GP; j++) {
                if (j >= G) continue;
                float s[PASSES];
                float tmax = -INFINITY;
#pragma unroll
                for (int i = 0; i < PASSES; i++) {
                    float kf[kVec];
                    Chunk<T>::unpack(kr[i], kf);
                    float dot = 0.f;
#pragma unroll
                    for (int e = 0; e < kVec; e++) dot = fmaf(q[j][e], kf[e], dot);
                    dot = lane_group_sum<LPT>(dot);
                    s[i] = i * TPW + r < rows ? dot * p.scale_log2 : -INFINITY;
                    tmax = fmaxf(tmax, s[i]);
                }
                const float m_new = fmaxf(m[j], tmax);
                // a slot that has seen nothing keeps m = -inf: shift by 0,
                // which makes alpha and every weight exactly 0
                const float shift = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = fast_exp2(m[j] - shift);
                m[j] = m_new;
                float lsum = 0.f, pv[kVec];
#pragma unroll
                for (int e = 0; e < kVec; e++) pv[e] = 0.f;
#pragma unroll
                for (int i = 0; i < PASSES; i++) {
                    const float pw = fast_exp2(s[i] - shift);
                    lsum += pw;
                    float vf[kVec];
                    Chunk<T>::unpack(vr[i], vf);
#pragma unroll
                    for (int e = 0; e < kVec; e++) pv[e] = fmaf(pw, vf[e], pv[e]);
                }
                l[j] = fmaf(l[j], alpha, lsum);
#pragma unroll
                for (int e = 0; e < kVec; e++) acc[j][e] = fmaf(acc[j][e], alpha, pv[e]);
            }
        };

        uint4 kr[BUFS][PASSES], vr[BUFS][PASSES];
        int rows[BUFS];
        int phys_next = phys_of(0);
#pragma unroll
        for (int j = 0; j < DEPTH; j++) {
            rows[j] = load_tile(j, phys_next, kr[j], vr[j]);
            phys_next = phys_of(j + 1);
        }
        for (int tb = 0; tb < ntiles; tb += BUFS) {
#pragma unroll
            for (int j = 0; j < BUFS; j++) {
                const int t = tb + j;
                if (t >= ntiles) break;
                const int jn = (j + DEPTH) % BUFS;
                rows[jn] = load_tile(t + DEPTH, phys_next, kr[jn], vr[jn]);
                phys_next = phys_of(t + DEPTH + 1);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the wait
                update(kr[j], vr[j], rows[j]);
            }
        }

        // merge the TPW token-slot states (lanes with the same chunk c)
#pragma unroll
        for (int o = LPT; o < kWave; o <<= 1) {
#pragma unroll
            for (int j = 0; j < GP; j++) {
                if (j >= G) continue;
                const float m_o = __shfl_xor(m[j], o);
                const float l_o = __shfl_xor(l[j], o);
                const float mm = fmaxf(m[j], m_o);
                const float fa = m[j] == -INFINITY ? 0.f : fast_exp2(m[j] - mm);
                const float fb = m_o == -INFINITY ? 0.f : fast_exp2(m_o - mm);
                l[j] = l[j] * fa + l_o * fb;
#pragma unroll
                for (int e = 0; e < kVec; e++) {
                    const float a_o = __shfl_xor(acc[j][e], o);
                    acc[j][e] = acc[j][e] * fa + a_o * fb;
                }
                m[j] = mm;
            }
        }
        const bool whole = t_begin == 0 && t_end == Tb;
        if (r == 0) {
#pragma unroll
            for (int j = 0; j < GP; j++) {
                if (j >= G) continue;
                if (whole) {
                    const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
                    float o[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; e++) o[e] = acc[j][e] * inv;
                    Chunk<T>::pack_store((T *)out + ((size_t)b * p.num_q_heads + g * G + j) * D +
                                             c * kVec,
                                         o);
                } else {
                    const size_t prow = ((size_t)w * 2 + slot) * kMaxGroup + j;
                    float *dst = ws_acc + prow * D + c * kVec;
#pragma unroll
                    for (int e = 0; e < kVec; e++) dst[e] = acc[j][e];
                    if (c == 0) {
                        ws_m[prow] = m[j];
                        ws_l[prow] = l[j];
                    }
                }
            }
        }
        // the merge kernel expects a unit that begins inside a share in
        // slot 1, whatever the wavefront's earlier units were
        slot = 1;
    }
}

template <typename T, int D, int GP>
static void launch_balanced_g(const DecodeParams &p, hipStream_t stream) {
    if constexpr (VecShape<T, D, GP>::kOk)
        hipLaunchKernelGGL((decode_vector_balanced_kernel<T, D, GP>), dim3(p.num_units),
                           dim3(kWave), 0, stream, p, p.block_tables, p.context_lens, p.out,
                           p.ws_m, p.ws_l, p.ws_acc);
}

template <typename T, int D>
static hipError_t launch_balanced_d(const DecodeParams &p, hipStream_t stream) {
    switch (p.group <= 1 ? 1 : p.group <= 2 ? 2 : p.group <= 4 ? 4 : p.group <= 8 ? 8 : 16) {
    case 1: launch_balanced_g<T, D, 1>(p, stream); break;
    case 2: launch_balanced_g<T, D, 2>(p, stream); break;
    case 4: launch_balanced_g<T, D, 4>(p, stream); break;
    case 8: launch_balanced_g<T, D, 8>(p, stream); break;
    default: launch_balanced_g<T, D, 16>(p, stream); break;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_balanced_t(const DecodeParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
    case 16: return launch_balanced_d<T, 16>(p, stream);
    case 32: return launch_balanced_d<T, 32>(p, stream);
    case 64: return launch_balanced_d<T, 64>(p, stream);
    case 128: return launch_balanced_d<T, 128>(p, stream);
    default: return launch_balanced_d<T, 256>(p, stream);
    }
}

bool vector_balanced_supported(int head_dim, int dtype, int block_size) {
    const int vec = dtype == 0 ? 4 : 8;
    return block_size >= kTileTok && kWave / (head_dim / vec) <= kTileTok;
}

hipError_t launch_decode_vector_balanced(const DecodeParams &p, int head_dim, int dtype,
                                         hipStream_t stream) {
    if (p.num_units == 0) return hipSuccess;
    return dtype == 0 ? launch_balanced_t<float>(p, head_dim, stream)
                      : launch_balanced_t<uint16_t>(p, head_dim, stream);
}

template <typename T, int D>
static hipError_t launch_d(const DecodeParams &p, hipStream_t stream) {
    const dim3 grid(p.num_units), block(kWave);
    switch (p.group <= 1 ? 1 : p.group <= 2 ? 2 : p.group <= 4 ? 4 : p.group <= 8 ? 8 : 16) {
    case 1: hipLaunchKernelGGL((decode_vector_kernel<T, D, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_vector_kernel<T, D, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_vector_kernel<T, D, 4>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_vector_kernel<T, D, 8>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_vector_kernel<T, D, 16>), grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(const DecodeParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
    case 16: return launch_d<T, 16>(p, stream);
    case 32: return launch_d<T, 32>(p, stream);
    case 64: return launch_d<T, 64>(p, stream);
    case 128: return launch_d<T, 128>(p, stream);
    default: return launch_d<T, 256>(p, stream);
    }
}

hipError_t launch_decode_vector(const DecodeParams &p, int head_dim, int dtype,
                                hipStream_t stream) {
    if (p.num_units == 0) return hipSuccess;
    return dtype == 0 ? launch_t<float>(p, head_dim, stream)
                      : launch_t<uint16_t>(p, head_dim, stream);
}

}  // namespace pa
