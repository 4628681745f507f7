// pa_decode_shared.hip -- PagedAttention decode that reads a KV tile once for
// every sequence of a pack that shares it.
//
// Sharing comes from forks: samples of one prompt point their block tables
// at the prompt's physical blocks ("PagedAttention实现", cow_write and the
// reference counts of KVBlock; "CS349E 第 7 讲 01_paged_attention.py",
// demo 3: n samples share the prompt's blocks).  Decode then reads the same
// shared block once per sample.  Here NPK consecutive sequences form a pack
// whose query heads fill NPK*G of the 32 columns of one wavefront (two
// 16-column matrix-core groups that share every K/V load; NPK is the largest
// power of two up to 8 that fits), and each distinct physical block among
// the pack's block-table entries at a tile index is loaded once and folded
// into the columns of the sequences that reference it (pa_mfma_tile.h).  The
// result per sequence is the plain decode result: sharing changes no value
// (demo 3 observations).
//
// Three kernels:
//  1. plan_shared_kernel, one workgroup per pack: lists the pack's items.
//     At tile index t, member i owns an item when it is the first member (in
//     order) that reaches t with its block id; the item is (block id, t, the
//     members with that id, the most rows any of them sees).  Items are
//     stored in tile-index order; U_k = the pack's item count.
//  2. decode_shared_kernel: W persistent wavefronts split the stream of
//     items (KV head slowest, then pack, then item) into equal shares; each
//     item is one tile load and one update of the columns of its members, so
//     a share may start or end anywhere.  A pack a wavefront covers whole is
//     finished in place; otherwise its state goes to one of the wavefront's
//     two partial slots: slot 0 for the first unit of its share, slot 1 for
//     the last (only those two can be partial).
//  3. reduce_shared_kernel: per (KV head, pack, column), merge the pieces
//     by log-sum-exp; which wavefronts and slots hold them follows from the
//     split alone.
#include "pa_mfma_tile.h"

namespace pa {

// ---------------------------------------------------------------------------
// 1. Plan: the item list of each pack.
// ---------------------------------------------------------------------------
// Item record (16 bytes): block id (0 when out of range, with rows 0), tile
// index, rows | member mask << 8, unused.  One workgroup per pack, one
// thread per tile index (in chunks of blockDim.x): each thread counts its
// tile's items, a workgroup-wide prefix places them.
constexpr int kPlanMaxThreads = 1024;

template <int NPK>
__global__ __launch_bounds__(kPlanMaxThreads) void plan_shared_kernel(const SharedParams p) {
    __shared__ int wave_sum[kPlanMaxThreads / kWave];
    const int k = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int nw = blockDim.x / kWave;
    int n[NPK];
    int maxT = 0;
#pragma unroll
    for (int i = 0; i < NPK; i++) {
        const int b = k * NPK + i;
        n[i] = b < p.num_seqs ? clamp_ctx(p.context_lens[b], p.max_context_len) : 0;
        maxT = max(maxT, (n[i] + kTile - 1) / kTile);
    }
    // the block ids of the first chunk of tile indices, read alongside the
    // context lengths rather than after them (one memory round trip, not
    // two): every index below max_tiles is inside the table row
    int id0[NPK];
#pragma unroll
    for (int i = 0; i < NPK; i++) {
        const int b = k * NPK + i;
        id0[i] = b < p.num_seqs && tid < p.max_tiles
                     ? p.block_tables[(size_t)b * p.max_blocks_per_seq +
                                      ((tid * kTile) >> p.log2_block)]
                     : -1;
    }
    int4 *items = (int4 *)p.ws_items + (size_t)k * NPK * p.max_tiles;
    int running = 0;
    for (int t0 = 0; t0 < maxT; t0 += blockDim.x) {
        const int t = t0 + tid;
        int id[NPK];
        bool v[NPK];
#pragma unroll
        for (int i = 0; i < NPK; i++) {
            v[i] = t * kTile < n[i];          // then t < max_tiles
            id[i] = !v[i] ? -1
                    : t0 == 0 ? id0[i]
                              : p.block_tables[(size_t)(k * NPK + i) * p.max_blocks_per_seq +
                                               ((t * kTile) >> p.log2_block)];
        }
        int cost = 0;
#pragma unroll
        for (int i = 0; i < NPK; i++) {
            bool dup = false;
#pragma unroll
            for (int j = 0; j < i; j++) dup |= v[j] && id[j] == id[i];
            cost += (v[i] && !dup) ? 1 : 0;
        }
        int incl = cost;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == kWave - 1) wave_sum[wv] = incl;
        __syncthreads();
        int before = 0, chunk = 0;
        for (int j = 0; j < nw; j++) {
            const int sj = wave_sum[j];
            before += j < wv ? sj : 0;
            chunk += sj;
        }
        // this tile index's items go to [running + before + incl - cost, ... + cost)
        int q = running + before + incl - cost;
#pragma unroll
        for (int i = 0; i < NPK; i++) {
            bool dup = false;
#pragma unroll
            for (int j = 0; j < i; j++) dup |= v[j] && id[j] == id[i];
            if (v[i] && !dup) {
                int mask = 0, maxn = 0;
#pragma unroll
                for (int m = 0; m < NPK; m++)
                    if (v[m] && id[m] == id[i]) {
                        mask |= 1 << m;
                        maxn = max(maxn, n[m]);
                    }
                const bool ok = (unsigned)id[i] < (unsigned)p.num_blocks;
                const int rows = ok ? min(kTile, maxn - t * kTile) : 0;
                items[q++] = make_int4(ok ? id[i] : 0, t, rows | (mask << 8), 0);
            }
        }
        running += chunk;
        __syncthreads();                 // wave_sum is rewritten by the next chunk
    }
    if (tid == 0) p.ws_cost[k] = running;
}

// ---------------------------------------------------------------------------
// 2. Decode over packs.
// ---------------------------------------------------------------------------
#ifndef PA_SHARED_WAVES_PER_EU
#define PA_SHARED_WAVES_PER_EU 1
#endif
// Items whose loads are in flight while one is computed.
#ifndef PA_SHARED_DEPTH
#define PA_SHARED_DEPTH 1
#endif
constexpr int kSD = PA_SHARED_DEPTH;
constexpr int kSB = kSD + 1;

template <int NPK, int NCG>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(PA_SHARED_WAVES_PER_EU)))
void decode_shared_kernel(const SharedParams args, const int32_t *__restrict__ ctx_lens,
                          void *__restrict__ out, float *__restrict__ ws_m,
                          float *__restrict__ ws_l, float *__restrict__ ws_acc,
                          const int *__restrict__ ws_cost,
                          const int4 *__restrict__ ws_items) {
    // restrict arguments: the stores cannot alias the item lists, so the
    // per-item reads stay on the scalar unit
    SharedParams p = args;
    p.context_lens = ctx_lens;
    p.out = out;
    const int lane = threadIdx.x;
    const Lane ln{lane & 15, lane >> 4};
    const int W = p.num_waves;
    const int w = blockIdx.x;       // launch order: see xcd_remap
    const int G = p.group;
    const int NPACK = p.num_packs;

    // item-count prefix over packs: lane i owns packs [i K, i K + K)
    const int K = (NPACK + kWave - 1) / kWave;
    int local = 0;
    for (int j = 0; j < K; j++) {
        const int k = lane * K + j;
        if (k < NPACK) local += ws_cost[k];
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

    // this lane's columns, one per column group of 16: column
    // cg * 16 + row16 is head hj of member im of the pack; group_members[cg]:
    // the members with a column in group cg (an item none of them references
    // leaves the group untouched and is skipped for it)
    int im[NCG], hj[NCG], group_members[NCG];
    bool col_real[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; cg++) {
        const int col = cg * 16 + ln.row16;
        im[cg] = col / G;
        hj[cg] = col - im[cg] * G;
        col_real[cg] = im[cg] < NPK;
        const int lo = (cg * 16) / G, hi = min(NPK - 1, (cg * 16 + 15) / G);
        group_members[cg] = lo > hi ? 0 : ((1 << (hi + 1)) - 1) & ~((1 << lo) - 1);
    }

    const char *kbase = (const char *)p.k_cache;
    const char *vbase = (const char *)p.v_cache;
    const int bs_mask = (1 << p.log2_block) - 1;
    const int x1 = min(w * C + C, total);
    int x = w * C;

    // A finished pack's state is written out late: a store counts in the
    // same in-order counter as the loads, so a store issued between two
    // tile loads holds up the wait for the later one.  The state of the
    // wave's first pack waits in `pend` until the next pack's first loads
    // are in flight, or, if that pack is the wave's last, until the end.
    // Partial states go to the wave's two slots: slot 0 holds the share's
    // first unit, slot 1 its last (only those two can be partial).
    Acc pend[NCG];
    bool have_pend = false, pend_whole = false;
    int pend_g = 0, pend_k = 0, pend_slot = 0;
    int slot = 0;
    auto emit = [&](const Acc (&st)[NCG], bool whole, int g, int k, int sl) {
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) {
            if (whole) {
                const int b = k * NPK + (col_real[cg] ? im[cg] : 0);
                if (col_real[cg] && b < p.num_seqs)
                    store_row((char *)out + ((size_t)b * p.num_q_heads + g * G + hj[cg]) * kD * 2,
                              st[cg], ln);
            } else {
                const size_t prow = ((size_t)w * 2 + sl) * kMaxCols + cg * 16 + ln.row16;
                store_partial(ws_m + prow, ws_l + prow, ws_acc + prow * kD, st[cg], ln);
            }
        }
    };
    while (x < x1) {
        const int g = x / TT;
        const int r = x - g * TT;
        // the pack holding stream position r: find its lane, then walk
        const unsigned long long own = __ballot(r >= excl && r < incl);
        const int jl = __builtin_ctzll(own);
        int base = __builtin_amdgcn_readfirstlane(__shfl(excl, jl));
        int k = jl * K;
        int Uk;
        if (K == 1) {
            Uk = __builtin_amdgcn_readfirstlane(__shfl(local, jl));
        } else {
            Uk = __builtin_amdgcn_readfirstlane(ws_cost[k]);
            while (r >= base + Uk) {
                base += Uk;
                k++;
                Uk = __builtin_amdgcn_readfirstlane(ws_cost[k]);
            }
        }
        const int q_begin = r - base;                  // items [q_begin, q_end) of pack k
        const int q_end = min(Uk, q_begin + (x1 - x));
        x += q_end - q_begin;
        const bool last_pack = x >= x1;

        // this lane's columns within the pack
        int b_col[NCG], n_col[NCG];
        bool col_ok[NCG];
        bf16x8 qv[NCG][4];
        Acc a[NCG];
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) {
            b_col[cg] = k * NPK + (col_real[cg] ? im[cg] : 0);
            col_ok[cg] = col_real[cg] && b_col[cg] < p.num_seqs;
            n_col[cg] = col_ok[cg] ? clamp_ctx(p.context_lens[b_col[cg]], p.max_context_len) : 0;
            const char *qrow = (const char *)p.q +
                               (((size_t)(col_ok[cg] ? b_col[cg] : 0) * p.num_q_heads + g * G +
                                 (col_ok[cg] ? hj[cg] : 0)) * kD + 8 * ln.grp) * 2;
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                u32x4 raw = *(const u32x4 *)(qrow + 64 * kk);
                if (!col_ok[cg]) raw = (u32x4){0u, 0u, 0u, 0u};
                qv[cg][kk] = __builtin_bit_cast(bf16x8, raw);
            }
            acc_init(a[cg]);
        }

        // items q_begin .. q_end-1; the loads of items q+1 .. q+kSD are in
        // flight while item q is computed.  Item records are held in two
        // VGPR windows of 64 (lane i: record base + i) and read out with lane
        // reads; the window just left is reloaded with the one after next,
        // a whole window ahead of its use, so no memory round trip sits
        // between computing one item and issuing the next.  The two windows
        // alternate instead of being copied: a copy of a freshly loaded
        // register would wait for its load.
        const int4 *list = ws_items + (size_t)k * NPK * p.max_tiles;
        const int last = q_end - 1;
        int wb = q_begin;                            // first record of the current window
        bool in_b = false;                           // current window: wB (else wA)
        const u32x4 *rlist = (const u32x4 *)list;
        const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)list, (short)0, q_end * 16, kRsrcWord3);
        u32x4 wA = rlist[min(wb + lane, last)];
        u32x4 wB = rlist[min(wb + kWave + lane, last)];
        auto record = [&](int q) -> int4 {           // q in [wb, wb + 64), uniform
            const int i = q - wb;
            int4 r;
            if (in_b) {
                r = make_int4(__builtin_amdgcn_readlane(wB[0], i), __builtin_amdgcn_readlane(wB[1], i),
                              __builtin_amdgcn_readlane(wB[2], i), 0);
            } else {
                r = make_int4(__builtin_amdgcn_readlane(wA[0], i), __builtin_amdgcn_readlane(wA[1], i),
                              __builtin_amdgcn_readlane(wA[2], i), 0);
            }
            return r;
        };
        auto issue = [&](const int4 &it, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
            const size_t off = ((((size_t)it.x * p.num_kv_heads + g) << p.log2_block) +
                                ((it.y * kTile) & bs_mask)) * (size_t)kRowBytes;
            load_tile_rows(kbase, vbase, off, it.z & 0xff, ln, kr, vr);
        };
        const int4 none = make_int4(0, 0, 0, 0);
        u32x4 kr[kSB][4], vr[kSB][4];
        int4 rec[kSB];
#pragma unroll
        for (int j = 0; j < kSD; j++) {
            rec[j] = q_begin + j < q_end ? record(q_begin + j) : none;
            issue(rec[j], kr[j], vr[j]);
        }
        if (have_pend && !last_pack) {
            emit(pend, pend_whole, pend_g, pend_k, pend_slot);
            have_pend = false;
        }
        for (int q0 = q_begin; q0 < q_end; q0 += kSB) {
#pragma unroll
            for (int j = 0; j < kSB; j++) {
                const int q = q0 + j;
                if (q >= q_end) break;
                const int jn = (j + kSD) % kSB;
                if (q + kSD == wb + kWave) {           // into the next window
                    // the two branches load through different instructions
                    // (a pointer read, a buffer read) so that the compiler
                    // keeps each load in its branch, writing straight into
                    // the window it refills
                    const int idx = min(wb + 2 * kWave + lane, last);
                    if (in_b)
                        wB = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           lrs, idx * 16, 0, 0));
                    else
                        wA = rlist[idx];
                    wb += kWave;
                    in_b = !in_b;
                }
                rec[jn] = q + kSD < q_end ? record(q + kSD) : none;
                issue(rec[jn], kr[jn], vr[jn]);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the wait
                const int4 it = rec[j];
                if ((it.z & 0xff) > 0) {
                    const int mask = it.z >> 8;
#pragma unroll
                    for (int cg = 0; cg < NCG; cg++) {
                        if ((mask & group_members[cg]) == 0) continue;   // none of its columns
                        const bool in_mask = col_ok[cg] && ((mask >> im[cg]) & 1);
                        const int nv = in_mask ? n_col[cg] - it.y * kTile : 0;
                        tile_update<true>(kr[j], vr[j], qv[cg], nv, p.scale_log2, a[cg], ln);
                    }
                }
            }
        }

        const bool whole = q_begin == 0 && q_end == Uk;
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) acc_finish(a[cg]);
        const int sl = slot;             // 0 for the share's first unit, then 1
        slot = 1;
        if (have_pend) {                 // this is the wave's last pack
            emit(pend, pend_whole, pend_g, pend_k, pend_slot);
            have_pend = false;
            emit(a, whole, g, k, sl);
        } else {
#pragma unroll
            for (int cg = 0; cg < NCG; cg++) pend[cg] = a[cg];
            have_pend = true;
            pend_whole = whole;
            pend_g = g;
            pend_k = k;
            pend_slot = sl;
        }
    }
    if (have_pend) emit(pend, pend_whole, pend_g, pend_k, pend_slot);
}

// ---------------------------------------------------------------------------
// 3. Merge.
// ---------------------------------------------------------------------------
// One workgroup of 4 wavefronts per (KV head, pack) unit.  The unit's
// position in the item stream gives its pieces without a lookup: with C
// items per share, the unit's items [start, start + U) lie in the shares of
// wavefronts first = start / C .. last = (start + U - 1) / C.  One share
// (first == last) finished it in place.  Otherwise wavefront `first` holds
// a piece in slot 0 if its share starts exactly at the unit (the unit is
// its first) and in slot 1 if not (the unit is its last), and every later
// wavefront up to `last` in slot 0 (its share starts inside the unit).
// All 32 columns are merged at once, 8 threads per column and 16 dims per
// thread, pieces summed in ascending wavefront order; up to kDirect pieces
// are loaded in one round and merged in registers.
constexpr int kReduceThreads = 256;
constexpr int kDirect = 6;

template <int NPK, int NCG>
__global__ __launch_bounds__(kReduceThreads) void reduce_shared_kernel(
    const SharedParams p, const int *__restrict__ ws_cost) {
    const int unit = blockIdx.x;                   // g * NPACK + k
    const int NPACK = p.num_packs;
    const int k = unit % NPACK, g = unit / NPACK;
    const int G = p.group;
    const int tid = threadIdx.x, lane = tid % kWave;

    // position of the unit in the item stream (as the decode kernel split it)
    const int U = __builtin_amdgcn_readfirstlane(ws_cost[k]);
    int before = 0, all = 0;
    for (int kk = lane; kk < NPACK; kk += kWave) {
        const int u = ws_cost[kk];
        all += u;
        if (kk < k) before += u;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
        before += __shfl_xor(before, o);
        all += __shfl_xor(all, o);
    }
    const int S = before, TT = all;
    int first = 0, last = 0, first_slot = 0;
    if (U > 0) {
        const int C = (TT * p.num_kv_heads + p.num_waves - 1) / p.num_waves;
        const int start = g * TT + S;
        first = start / C;
        last = (start + U - 1) / C;
        first_slot = start == first * C ? 0 : 1;
    }
    const int npieces = last - first + 1;
    // piece q: wavefront first + q, slot (q == 0 ? first_slot : 0)
    auto piece_row = [&](int q, int c) -> size_t {
        return ((size_t)(first + q) * 2 + (q == 0 ? first_slot : 0)) * kMaxCols + c;
    };

    // 8 lanes per column, 16 dims per lane: the 32 columns at once
    const int c = tid / 8, sub = tid % 8;
    const int im = c / G;
    const int b = k * NPK + im;
    if (c >= NCG * 16 || im >= NPK || b >= p.num_seqs) return;
    uint16_t *o = (uint16_t *)p.out +
                  ((size_t)b * p.num_q_heads + (size_t)g * G + (c - im * G)) * kD + 16 * sub;
    if (U == 0) {                                   // empty context
        *(uint4 *)o = make_uint4(0u, 0u, 0u, 0u);
        *(uint4 *)(o + 8) = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    if (npieces == 1) return;                       // finished by one wavefront
    float num[16], den = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e++) num[e] = 0.f;
    if (npieces <= kDirect) {
        // every piece's m, l and 16 accumulator values in one round of loads
        float mq[kDirect], lq[kDirect];
        float4 aq[kDirect][4];
#pragma unroll
        for (int q = 0; q < kDirect; q++) {
            if (q < npieces) {
                const size_t prow = piece_row(q, c);
                mq[q] = p.ws_m[prow];
                lq[q] = p.ws_l[prow];
                const float4 *src = (const float4 *)(p.ws_acc + prow * kD + 16 * sub);
#pragma unroll
                for (int v = 0; v < 4; v++) aq[q][v] = src[v];
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kDirect; q++)
            if (q < npieces) M = fmaxf(M, mq[q]);
        if (M != -INFINITY) {
#pragma unroll
            for (int q = 0; q < kDirect; q++) {
                if (q < npieces && mq[q] != -INFINITY) {   // empty piece: weight 0
                    const float wq = __builtin_amdgcn_exp2f(mq[q] - M);
                    den = fmaf(wq, lq[q], den);
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        num[4 * v + 0] = fmaf(wq, aq[q][v].x, num[4 * v + 0]);
                        num[4 * v + 1] = fmaf(wq, aq[q][v].y, num[4 * v + 1]);
                        num[4 * v + 2] = fmaf(wq, aq[q][v].z, num[4 * v + 2]);
                        num[4 * v + 3] = fmaf(wq, aq[q][v].w, num[4 * v + 3]);
                    }
                }
            }
        }
    } else {
        float M = -INFINITY;
        for (int q = 0; q < npieces; q++) M = fmaxf(M, p.ws_m[piece_row(q, c)]);
        if (M != -INFINITY) {
            for (int q = 0; q < npieces; q++) {
                const size_t prow = piece_row(q, c);
                const float mq = p.ws_m[prow];
                const float wq = mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq - M);
                den = fmaf(wq, p.ws_l[prow], den);
                const float4 *src = (const float4 *)(p.ws_acc + prow * kD + 16 * sub);
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const float4 a4 = src[v];
                    num[4 * v + 0] = fmaf(wq, a4.x, num[4 * v + 0]);
                    num[4 * v + 1] = fmaf(wq, a4.y, num[4 * v + 1]);
                    num[4 * v + 2] = fmaf(wq, a4.z, num[4 * v + 2]);
                    num[4 * v + 3] = fmaf(wq, a4.w, num[4 * v + 3]);
                }
            }
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint32_t wv[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
        wv[e] = (uint32_t)f32_to_bf16(num[2 * e] * inv) |
                ((uint32_t)f32_to_bf16(num[2 * e + 1] * inv) << 16);
    *(uint4 *)o = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    *(uint4 *)(o + 8) = make_uint4(wv[4], wv[5], wv[6], wv[7]);
}

// ---------------------------------------------------------------------------
template <int NPK, int NCG>
static hipError_t launch_shared_t(const SharedParams &p, int phase, hipStream_t stream) {
    if (phase & 1) {
        // one thread per tile index, up to kPlanMaxThreads (then chunks)
        const int plan_threads =
            std::min(kPlanMaxThreads, std::max(kWave, (p.max_tiles + kWave - 1) / kWave * kWave));
        hipLaunchKernelGGL(plan_shared_kernel<NPK>, dim3(p.num_packs), dim3(plan_threads), 0,
                           stream, p);
        hipLaunchKernelGGL((decode_shared_kernel<NPK, NCG>), dim3(p.num_waves), dim3(kWave), 0,
                           stream, p, p.context_lens, p.out, p.ws_m, p.ws_l, p.ws_acc, p.ws_cost,
                           (const int4 *)p.ws_items);
    }
    if (phase & 2)
        hipLaunchKernelGGL((reduce_shared_kernel<NPK, NCG>),
                           dim3((unsigned)p.num_kv_heads * p.num_packs), dim3(kReduceThreads), 0,
                           stream, p, p.ws_cost);
    return hipGetLastError();
}

hipError_t launch_decode_shared(const SharedParams &p, int phase, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    // columns used: pack * group <= 32, in one or two groups of 16
    const bool two = p.pack * p.group > 16;
    switch (p.pack) {
    case 8: return two ? launch_shared_t<8, 2>(p, phase, stream)
                       : launch_shared_t<8, 1>(p, phase, stream);
    case 4: return two ? launch_shared_t<4, 2>(p, phase, stream)
                       : launch_shared_t<4, 1>(p, phase, stream);
    case 2: return two ? launch_shared_t<2, 2>(p, phase, stream)
                       : launch_shared_t<2, 1>(p, phase, stream);
    default: return launch_shared_t<1, 1>(p, phase, stream);
    }
}

}  // namespace pa
