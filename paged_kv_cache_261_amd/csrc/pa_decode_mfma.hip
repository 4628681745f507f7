// pa_decode_mfma.hip -- PagedAttention decode for bfloat16 caches with the
// grouped query heads of one KV head on the CDNA4 matrix cores.
//
// Same result as the vector kernel ("CS349E 第 7 讲 01_paged_attention.py",
// demo 2, paper eq. 4: scores block by block through the block table, one
// softmax over the whole context, probability-weighted sum of V), computed
// one 16-token tile at a time by one wavefront:
//
//   scores   S[16 tokens x 16 heads] = K_tile[16 x 128] . Q^T[128 x 16]
//            4 x v_mfma_f32_16x16x32_bf16; the G query heads of the KV head
//            fill G of the 16 columns (the rest are zero queries);
//   softmax  online, per head, in base-2 log domain; the tile max is
//            reduced across the 4 lane groups with two row-swap permutes;
//   P.V      O^T[128 x 16] += V_tile^T[128 x 16 tokens] . P^T[16 x 16]
//            8 x v_mfma_f32_16x16x16_bf16 (P rounded to bfloat16, fp32
//            accumulation).
//
// Register layouts (lane = 16 * grp + row16):
//  - S: lane holds S[token 4*grp + i][head row16], i = 0..3.  That is
//    exactly the B operand of the P.V product (k = token 4*grp + i,
//    column = head row16), so P never leaves the lane.
//  - K operand (A of the score MFMA, row = token): for MFMA kk the lane
//    holds dims [32*kk + 8*grp, +8) of token row16, so each of the four
//    16-byte loads of a tile reads 64 contiguous bytes of every row; the
//    query (B, column = head) is loaded with the same dim order, so the
//    products pair matching dims whatever the hardware's k order is.
//  - V operand (A of the P.V MFMA, row = dim, k = token): lane loads the 16
//    contiguous bytes of dims [8*row16, 8*row16 + 8) of tokens 4*grp + i
//    (each load reads 4 whole rows); MFMA n uses dim 8*row16 + n of those 4
//    tokens (one byte-permute per register to transpose).
//  - O^T accumulator: lane holds head row16 at dims 32*grp + 8*i + n, i.e.
//    32 contiguous dims, written back as 16-byte stores.
//
// Memory: a (block, KV head) tile of 16 tokens x 128 dims is 4 KiB
// contiguous.  Tiles are read through buffer descriptors whose byte range
// covers only the tile's visible rows, so rows past the context read as
// zero without a memory access and the tile loop has no branches: the
// loads of the next tile are issued before the current one is computed and
// the compiler counts the outstanding loads exactly.  The block-table
// entry of a tile is read with a scalar load one tile ahead.
//
// Two ways to cut the work into wavefronts:
//  - decode_mfma_kernel: single pass, one wavefront per (sequence, KV head);
//  - decode_mfma_balanced_kernel: a fixed number W of persistent wavefronts;
//    the tiles of all (KV head, sequence) units are laid end to end and
//    every wavefront takes an equal contiguous share of that stream, so the
//    load is even whatever the mix of context lengths.  Either the shares
//    are cut at any tile (work-balanced split; pieces merged by
//    reduce_balanced_kernel) or at partition boundaries (fixed-partition
//    split; partitions merged by reduce_kernel).
#include "pa_internal.h"

#include <math.h>

namespace pa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head_dim handled by these kernels
constexpr int kTile = 16;        // tokens per tile
constexpr int kRowBytes = kD * 2;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, CDNA

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum with the lane 16 (resp. 32) positions away, on the VALU: the
// gfx950 row-swap permutes exchange rows of 16 lanes (resp. halves of the
// wave) between two registers, so swapping a value with itself pairs every
// lane with lane ^ 16 (resp. lane ^ 32).
__device__ __forceinline__ float xor16_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));   // RNE
}

}  // namespace

// Prefetch depth: tiles whose loads are in flight while a tile is computed.
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 1
#endif
// Occupancy hint: waves per SIMD the register allocation must allow (0: none).
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 3
#endif

constexpr int kDepth = PA_MFMA_DEPTH;
constexpr int kBufs = kDepth + 1;

// Softmax state of one wavefront for the (up to 16) query heads of a unit.
struct Acc {
    f32x4 o[8];     // O^T: head row16, dims 32*grp + 8*i + n  ->  o[n][i]
    float m;        // running max of head row16 (base-2 log domain)
    float lsum;     // this lane's share of the running sum
};

struct Lane {
    int row16, grp;
};

__device__ __forceinline__ void acc_init(Acc &a) {
#pragma unroll
    for (int nn = 0; nn < 8; nn++) a.o[nn] = (f32x4){0.f, 0.f, 0.f, 0.f};
    a.m = -INFINITY;
    a.lsum = 0.f;
}

// Query operand of unit (b, g): head row16 of the group, dims
// [32*kk + 8*grp, +8) for MFMA kk; zero for the padding heads row16 >= G.
__device__ __forceinline__ void load_q(const DecodeParams &p, int b, int g, Lane ln,
                                       bf16x8 (&qv)[4]) {
    const bool real = ln.row16 < p.group;
    const char *qrow = (const char *)p.q +
                       (((size_t)b * p.num_q_heads + g * p.group + (real ? ln.row16 : 0)) * kD +
                        8 * ln.grp) * 2;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
        u32x4 raw = *(const u32x4 *)(qrow + 64 * kk);
        if (!real) raw = (u32x4){0u, 0u, 0u, 0u};
        qv[kk] = __builtin_bit_cast(bf16x8, raw);
    }
}

// Tiles [tile_begin, tile_end) of unit (b, g); tile t holds tokens
// [16 t, 16 t + 16), of which the first n of the sequence are visible.
// With emit_every > 0, emit(t) runs after every tile t that ends a run of
// emit_every tiles (counted from tile 0 of the sequence) and after the last
// tile; it takes the state of that run and must leave `a` reset.  The loads
// of the following tiles stay in flight across it.
template <typename Emit>
__device__ __forceinline__ void run_tiles(const DecodeParams &p, int b, int g, int tile_begin,
                                          int tile_end, int n, const bf16x8 (&qv)[4], Acc &a,
                                          Lane ln, int emit_every, Emit &&emit) {
    const int ntiles = tile_end - tile_begin;
    if (ntiles <= 0) return;
    const char *kbase = (const char *)p.k_cache;
    const char *vbase = (const char *)p.v_cache;
    const int32_t *__restrict__ table = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.log2_block;
    const int bs_mask = (1 << log2bs) - 1;
    const int k_lane_off = ln.row16 * kRowBytes + ln.grp * 16;        // + 64 * kk
    const int v_lane_off = (4 * ln.grp) * kRowBytes + ln.row16 * 16;  // + i * kRowBytes

    // Physical block of tile t (t clamped into the range, so the table entry
    // read always belongs to a visible token).
    auto phys_of = [&](int t) -> int {
        const int tt = tile_begin + (t < ntiles ? t : ntiles - 1);
        return table[(tt * kTile) >> log2bs];
    };
    // Issue the loads of tile t; returns its visible row count (0 when the
    // tile is past the range or its block id is out of range).
    auto load_tile = [&](int t, int phys, u32x4 (&kr)[4], u32x4 (&vr)[4]) -> int {
        const int tok = (tile_begin + t) * kTile;
        const bool ok = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
        const int rows = ok ? min(kTile, n - tok) : 0;
        const size_t tile = ((((size_t)(ok ? phys : 0) * p.num_kv_heads + g) << log2bs) +
                             (tok & bs_mask)) * (size_t)kRowBytes;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + tile), (short)0, rows * kRowBytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + tile), (short)0, rows * kRowBytes, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < 4; i++)   // the 64*i step stays inside the lane's row
            kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  krs, k_lane_off, 64 * i, 0));
#pragma unroll
        for (int i = 0; i < 4; i++)
            vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  vrs, v_lane_off + i * kRowBytes, 0, 0));
        return rows;
    };

    auto compute_tile = [&](int nv, const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]), qv[kk],
                                                        S, 0, 0, 0);
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; i++) s[i] = 4 * ln.grp + i < nv ? S[i] * p.scale_log2 : -INFINITY;
        const float tmax = xor32_max(xor16_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))));
        const float m_new = fmaxf(a.m, tmax);       // finite: the tile has a visible row
        const float alpha = fast_exp2(a.m - m_new); // 0 on the first tile (m = -inf)
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; i++) pr[i] = fast_exp2(s[i] - m_new);
        a.lsum = a.lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        a.m = m_new;
#pragma unroll
        for (int nn = 0; nn < 8; nn++) a.o[nn] *= alpha;
        const s16x4 pb = __builtin_bit_cast(
            s16x4, (uint2){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
#pragma unroll
        for (int nn = 0; nn < 8; nn++) {
            // dim 8*row16 + nn of tokens 4*grp + 0..3: word nn/2 of each row,
            // low half for even nn, high half for odd nn
            const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t d0 = __builtin_amdgcn_perm(vr[1][nn >> 1], vr[0][nn >> 1], sel);
            const uint32_t d1 = __builtin_amdgcn_perm(vr[3][nn >> 1], vr[2][nn >> 1], sel);
            const s16x4 av = __builtin_bit_cast(s16x4, (uint2){d0, d1});
            a.o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, a.o[nn], 0, 0, 0);
        }
    };

    u32x4 kr[kBufs][4], vr[kBufs][4];
    int rows[kBufs];
    int phys_next = phys_of(0);
#pragma unroll
    for (int j = 0; j < kDepth; j++) {         // prologue: tiles 0 .. depth-1
        rows[j] = load_tile(j, phys_next, kr[j], vr[j]);
        phys_next = phys_of(j + 1);
    }
    for (int tb = 0; tb < ntiles; tb += kBufs) {
#pragma unroll
        for (int j = 0; j < kBufs; j++) {
            const int t = tb + j;
            if (t >= ntiles) break;
            const int jn = (j + kDepth) % kBufs;
            rows[jn] = load_tile(t + kDepth, phys_next, kr[jn], vr[jn]);
            phys_next = phys_of(t + kDepth + 1);
            // keep the prefetch ahead of the wait for tile t
            __builtin_amdgcn_sched_barrier(0);
            if (rows[j] > 0) compute_tile(rows[j], kr[j], vr[j]);
            if (emit_every > 0 &&
                ((tile_begin + t + 1) % emit_every == 0 || t == ntiles - 1))
                emit(tile_begin + t);
        }
    }
}

struct NoEmit {
    __device__ void operator()(int) const {}
};

// Sum the lane shares of l over the 4 lane groups (after the last tile).
__device__ __forceinline__ void acc_finish(Acc &a) { a.lsum = xor32_sum(xor16_sum(a.lsum)); }

// out[b][g*G + row16] = O / l, in bfloat16.
__device__ __forceinline__ void store_final(const DecodeParams &p, int b, int g, const Acc &a,
                                            Lane ln) {
    if (ln.row16 >= p.group) return;
    const size_t row = (size_t)b * p.num_q_heads + g * p.group + ln.row16;
    const float inv = a.lsum > 0.f ? 1.f / a.lsum : 0.f;
    char *dst = (char *)p.out + (row * kD + 32 * ln.grp) * 2;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        u32x4 wv;
#pragma unroll
        for (int j = 0; j < 4; j++)
            wv[j] = pack_bf16x2(a.o[2 * j][i] * inv, a.o[2 * j + 1][i] * inv);
        *(u32x4 *)(dst + 16 * i) = wv;
    }
}

// Unnormalised partial state of head row16: m and l to m_dst/l_dst, the
// head's accumulator (head_dim floats) to acc_dst.
__device__ __forceinline__ void store_partial(float *m_dst, float *l_dst, float *acc_dst,
                                              const Acc &a, Lane ln) {
    float *dst = acc_dst + 32 * ln.grp;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const f32x4 lo = {a.o[0][i], a.o[1][i], a.o[2][i], a.o[3][i]};
        const f32x4 hi = {a.o[4][i], a.o[5][i], a.o[6][i], a.o[7][i]};
        *(f32x4 *)(dst + 8 * i) = lo;
        *(f32x4 *)(dst + 8 * i + 4) = hi;
    }
    if (ln.grp == 0) {
        *m_dst = a.m;
        *l_dst = a.lsum;
    }
}

// ---------------------------------------------------------------------------
// Single pass: one wavefront per (sequence, KV head), the whole context.
// Wavefronts of consecutive sequences with the same KV head run side by
// side on one XCD, so samples that share prefix blocks read them through
// the same L2 at about the same time.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWave)
#if PA_MFMA_WAVES > 0
__attribute__((amdgpu_waves_per_eu(PA_MFMA_WAVES)))
#endif
void decode_mfma_kernel(const DecodeParams p) {
    const Lane ln{(int)threadIdx.x & 15, (int)threadIdx.x >> 4};
    const int u = xcd_remap(blockIdx.x, p.num_units);
    const Unit w = unit_of(u, p.num_seqs, p.num_kv_heads);
    const int n = clamp_ctx(p.context_lens[w.b], p.max_context_len);
    bf16x8 qv[4];
    load_q(p, w.b, w.g, ln, qv);
    Acc a;
    acc_init(a);
    run_tiles(p, w.b, w.g, 0, (n + kTile - 1) / kTile, n, qv, a, ln, 0, NoEmit{});
    acc_finish(a);
    store_final(p, w.b, w.g, a, ln);
}

// ---------------------------------------------------------------------------
// Persistent split: W wavefronts share the tile stream evenly.
//
// Stream order: KV head g slowest, then sequence b, then tile; sequence b
// contributes T_b = ceil(n_b / 16) tiles per KV head, so unit (g, b) starts
// at g * TT + S_b with S_b = sum_{b' < b} T_b' and TT = S_B.  Wavefront w
// owns [w C, w C + C) with C = ceil(Hkv TT / W).
//
//  - free cuts (part_tiles == 0, the work-balanced split): the wavefront
//    computes exactly the tiles it owns.  Its pieces are whole units
//    (finished in place) except possibly its first and its last, which go
//    to partial slots 0 and 1 of the wavefront.
//  - partition cuts (part_tiles == P / 16, fixed partitions of P tokens):
//    the wavefront computes every partition whose first tile it owns, whole
//    (so it may run up to one partition past its share), emitting each
//    partition's state into the [B][Hq][NP] workspace -- or the final output
//    when the context has one partition.  Consecutive partitions of a unit
//    keep the tile pipeline running across their boundary.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tiles_of(const DecodeParams &p, int b) {
    return (clamp_ctx(p.context_lens[b], p.max_context_len) + kTile - 1) / kTile;
}
// The same for a sequence index every lane agrees on, as a scalar.
__device__ __forceinline__ int tiles_of_uniform(const DecodeParams &p, int b) {
    return __builtin_amdgcn_readfirstlane(tiles_of(p, b));
}

__global__ __launch_bounds__(kWave)
#if PA_MFMA_WAVES > 0
__attribute__((amdgpu_waves_per_eu(PA_MFMA_WAVES)))
#endif
void decode_mfma_balanced_kernel(const DecodeParams args, const int32_t *__restrict__ tables,
                                 const int32_t *__restrict__ ctx_lens, void *__restrict__ out,
                                 float *__restrict__ ws_m, float *__restrict__ ws_l,
                                 float *__restrict__ ws_acc) {
    // The pointers the kernel reads tables through and writes results
    // through arrive as separate restrict arguments, so the compiler knows
    // the stores never touch the block tables and keeps the per-tile table
    // reads on the scalar unit.
    DecodeParams p = args;
    p.block_tables = tables;
    p.context_lens = ctx_lens;
    p.out = out;
    p.ws_m = ws_m;
    p.ws_l = ws_l;
    p.ws_acc = ws_acc;
    const int lane = threadIdx.x;
    const Lane ln{lane & 15, lane >> 4};
    const int W = p.num_units;
    const int w = xcd_remap(blockIdx.x, W);
    const int B = p.num_seqs;
    const int PT = p.partition_size / kTile;   // tiles per partition; 0: free cuts

    // tile prefix over sequences: lane i owns sequences [i K, i K + K)
    const int K = (B + kWave - 1) / kWave;
    int local = 0;
    for (int j = 0; j < K; j++) {
        const int b = lane * K + j;
        if (b < B) local += tiles_of(p, b);
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    const int excl = incl - local;
    // values every lane agrees on are moved to scalar registers, so the
    // compiler treats the unit's addresses as uniform
    const int TT = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1));
    const int total = TT * p.num_kv_heads;
    const int C = (total + W - 1) / W;

    const int x1 = min(w * C + C, total);
    int x = w * C;
    int slot = 0;
    while (x < x1) {
        const int g = x / TT;
        const int r = x - g * TT;
        // the sequence holding stream position r: find its lane, then walk
        const unsigned long long own = __ballot(r >= excl && r < incl);
        const int jl = __builtin_ctzll(own);
        int base = __builtin_amdgcn_readfirstlane(__shfl(excl, jl));
        int b = jl * K;
        int Tb = tiles_of_uniform(p, b);
        while (r >= base + Tb) {
            base += Tb;
            b++;
            Tb = tiles_of_uniform(p, b);
        }
        const int t_in = r - base;                     // first owned tile of the unit
        const int t_lim = min(Tb, t_in + (x1 - x));    // end of the owned tiles
        x += t_lim - t_in;
        int t_begin = t_in, t_end = t_lim;
        if (PT > 0) {   // the partitions that start inside [t_in, t_lim)
            t_begin = (t_in + PT - 1) / PT * PT;
            if (t_begin >= t_lim) continue;
            t_end = min(Tb, (t_lim - 1) / PT * PT + PT);
        }
        const int n = __builtin_amdgcn_readfirstlane(clamp_ctx(p.context_lens[b], p.max_context_len));

        bf16x8 qv[4];
        load_q(p, b, g, ln, qv);
        Acc a;
        acc_init(a);
        if (PT > 0) {
            const int n_parts = (Tb + PT - 1) / PT;
            run_tiles(p, b, g, t_begin, t_end, n, qv, a, ln, PT, [&](int t) {
                acc_finish(a);
                if (n_parts == 1) {
                    store_final(p, b, g, a, ln);
                } else if (ln.row16 < p.group) {
                    const size_t prow =
                        ((size_t)b * p.num_q_heads + g * p.group + ln.row16) * p.num_partitions +
                        t / PT;
                    store_partial(p.ws_m + prow, p.ws_l + prow, p.ws_acc + prow * kD, a, ln);
                }
                acc_init(a);
            });
        } else {
            run_tiles(p, b, g, t_begin, t_end, n, qv, a, ln, 0, NoEmit{});
            acc_finish(a);
            if (t_begin == 0 && t_end == Tb) {
                store_final(p, b, g, a, ln);
            } else if (ln.row16 < p.group) {
                const size_t prow = ((size_t)w * 2 + slot) * kMaxGroup + ln.row16;
                store_partial(p.ws_m + prow, p.ws_l + prow, p.ws_acc + prow * kD, a, ln);
            }
            slot = 1;
        }
    }
}

hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t stream) {
    if (p.num_units == 0) return hipSuccess;
    if (p.persistent)
        hipLaunchKernelGGL(decode_mfma_balanced_kernel, dim3(p.num_units), dim3(kWave), 0, stream,
                           p, p.block_tables, p.context_lens, p.out, p.ws_m, p.ws_l, p.ws_acc);
    else
        hipLaunchKernelGGL(decode_mfma_kernel, dim3(p.num_units), dim3(kWave), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
