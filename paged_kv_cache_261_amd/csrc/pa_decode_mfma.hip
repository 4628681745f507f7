// pa_decode_mfma.hip -- PagedAttention decode for bfloat16 caches with the
// grouped query heads of one KV head on the CDNA4 matrix cores.
//
// Same result as the vector kernel ("CS349E 第 7 讲 01_paged_attention.py",
// demo 2, paper eq. 4: scores block by block through the block table, one
// softmax over the whole context, probability-weighted sum of V), computed
// one 16-token tile at a time by one wavefront whose 16 MFMA columns hold the
// G query heads of one KV head (the rest are zero queries); the per-tile step
// and its register layouts are in pa_mfma_tile.h.
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
#include "pa_mfma_tile.h"

#include <math.h>

namespace pa {

// Prefetch depth: tiles whose loads are in flight while a tile is computed.
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 3
#endif
// Occupancy hint: waves per SIMD the register allocation must allow (0: none).
#ifndef PA_SPLIT_WAVES_PER_EU
#define PA_SPLIT_WAVES_PER_EU 1
#endif
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 2
#endif

constexpr int kDepth = PA_MFMA_DEPTH;
constexpr int kBufs = kDepth + 1;

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
        load_tile_rows(kbase, vbase, tile, rows, ln, kr, vr);
        return rows;
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
            if (rows[j] > 0) tile_update<false>(kr[j], vr[j], qv, rows[j], p.scale_log2, a, ln);
            if (emit_every > 0 &&
                ((tile_begin + t + 1) % emit_every == 0 || t == ntiles - 1))
                emit(tile_begin + t);
        }
    }
}

struct NoEmit {
    __device__ void operator()(int) const {}
};


// out[b][g*G + row16] = O / l, in bfloat16.
__device__ __forceinline__ void store_final(const DecodeParams &p, int b, int g, const Acc &a,
                                            Lane ln) {
    if (ln.row16 >= p.group) return;
    store_row((char *)p.out + ((size_t)b * p.num_q_heads + g * p.group + ln.row16) * kD * 2, a,
              ln);
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
#if PA_SPLIT_WAVES_PER_EU > 0
__attribute__((amdgpu_waves_per_eu(PA_SPLIT_WAVES_PER_EU)))
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
    const int w = blockIdx.x;       // launch order: see xcd_remap
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
            // Each partition's softmax state (m, l, acc over its own tokens)
            // is merged into the run's state by the log-sum-exp rule as soon
            // as the partition ends; the run -- this wavefront's consecutive
            // partitions of the unit -- then leaves one merged state, in the
            // row of its first partition, and marks its other partitions
            // empty (m = -inf, l = 0) for the merge kernel.  Writing every
            // partition's accumulator instead would put a burst of stores at
            // the end of the run, which costs more than the whole merge.
            const int n_parts = (Tb + PT - 1) / PT;
            const int G = p.group;
            Acc run;
            acc_init(run);
            run_tiles(p, b, g, t_begin, t_end, n, qv, a, ln, PT, [&](int) {
                acc_finish(a);
                acc_merge(run, a);
                acc_init(a);
            });
            if (n_parts == 1) {
                store_final(p, b, g, run, ln);
            } else if (ln.row16 < G) {
                const size_t prow =
                    ((size_t)b * p.num_q_heads + g * G + ln.row16) * p.num_partitions +
                    t_begin / PT;
                store_partial(p.ws_m + prow, p.ws_l + prow, p.ws_acc + prow * kD, run, ln);
                if (ln.grp == 0) {
                    const int k_end = (t_end + PT - 1) / PT - t_begin / PT;
                    for (int k = 1; k < k_end; k++) {
                        p.ws_m[prow + k] = -INFINITY;
                        p.ws_l[prow + k] = 0.f;
                    }
                }
            }
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
