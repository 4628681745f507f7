// pa_decode_shared.hip -- PagedAttention decode that reads a KV tile once for
// every sequence of a pack that shares it.
//
// Sharing comes from forks: samples of one prompt point their block tables
// at the prompt's physical blocks ("PagedAttention实现", cow_write and the
// reference counts of KVBlock; "CS349E 第 7 讲 01_paged_attention.py",
// demo 3: n samples share the prompt's blocks).  Decode then reads the same
// shared block once per sample.  Here NPK consecutive sequences form a pack
// whose G query heads each fill NPK*G of the 16 matrix-core columns of one
// wavefront, so for every tile index t the wavefront loads each distinct
// physical block among the pack's block-table entries once and folds it into
// the columns of the sequences that reference it (pa_mfma_tile.h).  The
// result per sequence is the plain decode result: sharing changes no value
// (demo 3 observations).
//
// Three kernels:
//  1. plan_shared_kernel, one wavefront per pack: the cost of tile index t is
//     the number of distinct block ids among the members that reach it;
//     pos_k[t] = sum of costs before t, U_k = pos_k[T_k].
//  2. decode_shared_kernel: W persistent wavefronts split the stream of
//     costs (KV head slowest, then pack, then tile index) into equal shares;
//     a wavefront computes every tile index whose position lies in its
//     share.  A pack it covers whole is finished in place; otherwise its
//     state goes to one of the wavefront's two partial slots (only its first
//     and last pack can be partial) and the slot is recorded in a small
//     directory.
//  3. reduce_shared_kernel: per (KV head, pack, column), merge the recorded
//     pieces by log-sum-exp.
#include "pa_mfma_tile.h"

namespace pa {

namespace {

__device__ __forceinline__ int shared_tiles_of(const SharedParams &p, int b) {
    if (b >= p.num_seqs) return 0;
    return (clamp_ctx(p.context_lens[b], p.max_context_len) + kTile - 1) / kTile;
}

// Index of the first entry >= v in the non-decreasing pos[0..n] (pos[n] >= v),
// found by the whole wavefront: each round probes 64 evenly spaced entries of
// the candidate range [lo, hi] (the last probe at hi) and keeps the stretch
// between the last probe below v and the first one at or above it.
__device__ __forceinline__ int wave_lower_bound(const int *pos, int n, int v) {
    const int lane = threadIdx.x;
    int lo = 0, hi = n;                                // answer in [lo, hi]
    while (hi - lo >= kWave) {
        const int step = (hi - lo + kWave - 2) / (kWave - 1);   // 63 step >= hi - lo
        const int idx = min(lo + lane * step, hi);
        const unsigned long long ge = __ballot(pos[idx] >= v);  // lane 63 probes hi
        const int f = __builtin_ctzll(ge);
        if (f == 0) return lo;
        const int nlo = lo + (f - 1) * step + 1;
        hi = min(lo + f * step, hi);
        lo = nlo;
    }
    const unsigned long long ge = __ballot(pos[min(lo + lane, hi)] >= v);
    return lo + __builtin_ctzll(ge);
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. Plan: distinct tiles per tile index of each pack.
// ---------------------------------------------------------------------------
template <int NPK>
__global__ __launch_bounds__(kWave) void plan_shared_kernel(const SharedParams p) {
    const int k = blockIdx.x;
    const int lane = threadIdx.x;
    int T[NPK];
    int maxT = 0;
#pragma unroll
    for (int i = 0; i < NPK; i++) {
        T[i] = shared_tiles_of(p, k * NPK + i);
        maxT = max(maxT, T[i]);
    }
    int *pos = p.ws_pos + (size_t)k * (p.max_tiles + 1);
    int running = 0;
    for (int t0 = 0; t0 < maxT; t0 += kWave) {
        const int t = t0 + lane;
        int cost = 0;
        if (t < maxT) {
            int id[NPK];
            bool v[NPK];
#pragma unroll
            for (int i = 0; i < NPK; i++) {
                v[i] = t < T[i];
                id[i] = v[i] ? p.block_tables[(size_t)(k * NPK + i) * p.max_blocks_per_seq +
                                              ((t * kTile) >> p.log2_block)]
                             : -1;
            }
#pragma unroll
            for (int i = 0; i < NPK; i++) {
                bool dup = false;
#pragma unroll
                for (int j = 0; j < i; j++) dup |= v[j] && id[j] == id[i];
                cost += (v[i] && !dup) ? 1 : 0;
            }
        }
        int incl = cost;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (t < maxT) pos[t + 1] = running + incl;
        running += __shfl(incl, kWave - 1);
    }
    if (lane == 0) {
        pos[0] = 0;
        p.ws_cost[k] = running;
    }
}

// ---------------------------------------------------------------------------
// 2. Decode over packs.
// ---------------------------------------------------------------------------
#ifndef PA_SHARED_WAVES_PER_EU
#define PA_SHARED_WAVES_PER_EU 2
#endif

// Per-tile-index view of the pack: block id, reach and visible rows of each
// member, all uniform (scalar).
template <int NPK>
struct PackTile {
    int id[NPK];
    bool valid[NPK];
    int nvis[NPK];
};

template <int NPK>
__device__ __forceinline__ void pack_tile_read(const SharedParams &p, const int32_t *const (&tab)[NPK],
                                               const int (&T)[NPK], const int (&n)[NPK], int t,
                                               PackTile<NPK> &pt) {
#pragma unroll
    for (int i = 0; i < NPK; i++) {
        pt.valid[i] = t < T[i];
        pt.id[i] = pt.valid[i] ? tab[i][(t * kTile) >> p.log2_block] : -1;
        pt.nvis[i] = min(kTile, n[i] - t * kTile);
    }
}

// Items of tile index t of a pack: member i owns an item when it is the first
// member (in order) that reaches t with its block id; the item loads that
// tile once for the members with the same id (mask), reading the most rows
// any of them can see (rows).  owners: bit i set when member i owns an item,
// so popcount(owners) is the plan's cost of t.  A block id outside the pool
// gives rows == 0: nothing is loaded or computed for it.
struct PackItem {
    int rows;
    int mask;
    int t;
    size_t tile_byte_off;
};

template <int NPK>
__device__ __forceinline__ void pack_items(const SharedParams &p, const PackTile<NPK> &pt, int t,
                                           int g, PackItem (&items)[NPK], int &owners) {
    const int bs_mask = (1 << p.log2_block) - 1;
    owners = 0;
#pragma unroll
    for (int i = 0; i < NPK; i++) {
        bool dup = false;
        int mask = 0, rows = 0;
#pragma unroll
        for (int m = 0; m < NPK; m++) {
            const bool same = pt.valid[i] && pt.valid[m] && pt.id[m] == pt.id[i];
            if (m < i) dup |= same;
            if (m >= i && same) {
                mask |= 1 << m;
                rows = max(rows, pt.nvis[m]);
            }
        }
        const bool own = pt.valid[i] && !dup;
        const bool ok = own && (unsigned)pt.id[i] < (unsigned)p.num_blocks;
        owners |= own ? 1 << i : 0;
        items[i].rows = ok ? rows : 0;
        items[i].mask = mask;
        items[i].t = t;
        items[i].tile_byte_off =
            ((((size_t)(ok ? pt.id[i] : 0) * p.num_kv_heads + g) << p.log2_block) +
             ((t * kTile) & bs_mask)) * (size_t)kRowBytes;
    }
}

template <int NPK>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(PA_SHARED_WAVES_PER_EU)))
void decode_shared_kernel(const SharedParams args, const int32_t *__restrict__ tables,
                          const int32_t *__restrict__ ctx_lens, void *__restrict__ out,
                          float *__restrict__ ws_m, float *__restrict__ ws_l,
                          float *__restrict__ ws_acc, int *__restrict__ ws_dir,
                          const int *__restrict__ ws_cost, const int *__restrict__ ws_pos) {
    // restrict arguments: the stores cannot alias the tables, so the
    // per-tile block-id reads stay on the scalar unit
    SharedParams p = args;
    p.block_tables = tables;
    p.context_lens = ctx_lens;
    p.out = out;
    const int lane = threadIdx.x;
    const Lane ln{lane & 15, lane >> 4};
    const int W = p.num_waves;
    const int w = xcd_remap(blockIdx.x, W);
    const int G = p.group;
    const int NPACK = p.num_packs;
    if (lane == 0) {
        ws_dir[2 * w] = -1;
        ws_dir[2 * w + 1] = -1;
    }

    // cost prefix over packs: lane i owns packs [i K, i K + K)
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

    // this lane's column: member im of the pack, head j of the group
    const int im = ln.row16 / G;
    const int hj = ln.row16 - im * G;
    const bool col_real = im < NPK;

    const int x1 = min(w * C + C, total);
    int x = w * C;
    int slot = 0;
    while (x < x1) {
        const int g = x / TT;
        const int r = x - g * TT;
        const unsigned long long own = __ballot(r >= excl && r < incl);
        const int jl = __builtin_ctzll(own);
        int base = __builtin_amdgcn_readfirstlane(__shfl(excl, jl));
        int k = jl * K;
        int Uk = __builtin_amdgcn_readfirstlane(ws_cost[k]);
        while (r >= base + Uk) {
            base += Uk;
            k++;
            Uk = __builtin_amdgcn_readfirstlane(ws_cost[k]);
        }
        const int off = r - base;
        const int lim = min(Uk, off + (x1 - x));
        x += lim - off;

        int T[NPK], n[NPK];
        const int32_t *tab[NPK];
        int maxT = 0;
#pragma unroll
        for (int i = 0; i < NPK; i++) {
            const int b = k * NPK + i;
            n[i] = b < p.num_seqs
                       ? __builtin_amdgcn_readfirstlane(
                             clamp_ctx(p.context_lens[b], p.max_context_len))
                       : 0;
            T[i] = (n[i] + kTile - 1) / kTile;
            maxT = max(maxT, T[i]);
            tab[i] = p.block_tables + (size_t)min(b, p.num_seqs - 1) * p.max_blocks_per_seq;
        }
        const int *pos = ws_pos + (size_t)k * (p.max_tiles + 1);
        const int t_begin = __builtin_amdgcn_readfirstlane(wave_lower_bound(pos, maxT, off));
        const int t_end = __builtin_amdgcn_readfirstlane(wave_lower_bound(pos, maxT, lim));
        if (t_begin >= t_end) continue;

        // this lane's column within the pack
        const int b_col = k * NPK + (col_real ? im : 0);
        const bool col_ok = col_real && b_col < p.num_seqs;
        int n_col = 0;
#pragma unroll
        for (int i = 0; i < NPK; i++)
            if (i == im) n_col = n[i];
        bf16x8 qv[4];
        {
            const char *qrow = (const char *)p.q +
                               (((size_t)(col_ok ? b_col : 0) * p.num_q_heads + g * G +
                                 (col_ok ? hj : 0)) * kD + 8 * ln.grp) * 2;
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                u32x4 raw = *(const u32x4 *)(qrow + 64 * kk);
                if (!col_ok) raw = (u32x4){0u, 0u, 0u, 0u};
                qv[kk] = __builtin_bit_cast(bf16x8, raw);
            }
        }
        Acc a;
        acc_init(a);

        // the items of tile indices t_begin..t_end-1 in order, owners in
        // member order within a tile index; the loads of the next item are
        // issued before the current one is computed.  A tile index's items
        // are worked out when the loop enters it, from the view read one
        // tile index ahead, and only then is the next view requested, so
        // waiting for a view never waits for the newest reads.
        const char *kbase = (const char *)p.k_cache;
        const char *vbase = (const char *)p.v_cache;
        const int nitems = __builtin_amdgcn_readfirstlane(pos[t_end] - pos[t_begin]);
        PackTile<NPK> view;
        // the owners' items of the current tile index, in member order, as a
        // queue that only ever moves by whole positions (every index below is
        // a constant, so the queue stays in scalar registers)
        PackItem queue[NPK];
        int left = 0;
        int t_cur = t_begin - 1;
        pack_tile_read(p, tab, T, n, t_begin, view);
        auto take = [&]() {
            if (left == 0) {   // enter the next tile index (each has an owner)
                t_cur++;
                PackItem items[NPK];
                int owners;
                pack_items(p, view, t_cur, g, items, owners);
                pack_tile_read(p, tab, T, n, min(t_cur + 1, t_end - 1), view);
#pragma unroll
                for (int m = NPK - 1; m >= 0; m--)
                    if ((owners >> m) & 1) {
#pragma unroll
                        for (int k = NPK - 1; k > 0; k--) queue[k] = queue[k - 1];
                        queue[0] = items[m];
                    }
                left = __builtin_popcount(owners);
            }
            PackItem r = queue[0];
#pragma unroll
            for (int k = 0; k + 1 < NPK; k++) queue[k] = queue[k + 1];
            left--;
            // uniform by construction; say so, or a buffer descriptor built
            // from it would be made lane by lane
            r.rows = __builtin_amdgcn_readfirstlane(r.rows);
            r.mask = __builtin_amdgcn_readfirstlane(r.mask);
            r.t = __builtin_amdgcn_readfirstlane(r.t);
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)r.tile_byte_off);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(r.tile_byte_off >> 32));
            r.tile_byte_off = ((size_t)hi << 32) | lo;
            return r;
        };
        u32x4 kr[2][4], vr[2][4];
        PackItem itm[2];
        itm[0] = take();
        load_tile_rows(kbase, vbase, itm[0].tile_byte_off, itm[0].rows, ln, kr[0], vr[0]);
        for (int q0 = 0; q0 < nitems; q0 += 2) {
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int q = q0 + j;
                if (q >= nitems) break;
                PackItem next{0, 0, t_cur, 0};
                if (q + 1 < nitems) next = take();
                itm[(j + 1) & 1] = next;
                load_tile_rows(kbase, vbase, next.tile_byte_off, next.rows, ln,
                               kr[(j + 1) & 1], vr[(j + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the wait
                const PackItem &it = itm[j];
                if (it.rows > 0) {
                    const bool in_mask = col_ok && ((it.mask >> im) & 1);
                    const int nv = in_mask ? n_col - it.t * kTile : 0;
                    tile_update<true>(kr[j], vr[j], qv, nv, p.scale_log2, a, ln);
                }
            }
        }
        acc_finish(a);
        if (t_begin == 0 && t_end == maxT) {
            if (col_ok)
                store_row((char *)out +
                              ((size_t)b_col * p.num_q_heads + g * G + hj) * kD * 2,
                          a, ln);
        } else {
            const size_t prow = ((size_t)w * 2 + slot) * kMaxGroup + ln.row16;
            store_partial(ws_m + prow, ws_l + prow, ws_acc + prow * kD, a, ln);
            if (lane == 0) ws_dir[2 * w + slot] = g * NPACK + k;
            slot = 1;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. Merge.
// ---------------------------------------------------------------------------
template <typename V>
__device__ __forceinline__ V block128_sum(V x, V *red) {
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
    __syncthreads();
    x = red[0] + red[1];
    __syncthreads();
    return x;
}

template <int NPK>
__global__ __launch_bounds__(kD) void reduce_shared_kernel(const SharedParams p,
                                                           const int *__restrict__ ws_dir,
                                                           const int *__restrict__ ws_cost) {
    __shared__ int red[2];
    const int c = blockIdx.x % kMaxGroup;
    const int unit = blockIdx.x / kMaxGroup;       // g * NPACK + k
    const int NPACK = p.num_packs;
    const int k = unit % NPACK, g = unit / NPACK;
    const int G = p.group;
    const int im = c / G;
    if (im >= NPK) return;
    const int b = k * NPK + im;
    if (b >= p.num_seqs) return;
    const int i = threadIdx.x;
    int before = 0, all = 0;
    for (int kk = i; kk < NPACK; kk += kD) {
        const int u = ws_cost[kk];
        all += u;
        if (kk < k) before += u;
    }
    const int S = block128_sum(before, red);
    const int TT = block128_sum(all, red);
    const int U = ws_cost[k];
    uint16_t *o = (uint16_t *)p.out + ((size_t)b * p.num_q_heads + (size_t)g * G + (c - im * G)) * kD;
    if (U == 0) {
        o[i] = 0;
        return;
    }
    const int C = (TT * p.num_kv_heads + p.num_waves - 1) / p.num_waves;
    const int start = g * TT + S;
    const int first = start / C, last = (start + U - 1) / C;
    float M = -INFINITY;
    int pieces = 0;
    for (int w = first; w <= last; w++)
        for (int s = 0; s < 2; s++)
            if (ws_dir[2 * w + s] == unit) {
                M = fmaxf(M, p.ws_m[((size_t)w * 2 + s) * kMaxGroup + c]);
                pieces++;
            }
    if (pieces == 0) return;                       // finished by one wavefront
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
        for (int w = first; w <= last; w++)
            for (int s = 0; s < 2; s++)
                if (ws_dir[2 * w + s] == unit) {
                    const size_t prow = ((size_t)w * 2 + s) * kMaxGroup + c;
                    const float mq = p.ws_m[prow];
                    if (mq == -INFINITY) continue;
                    const float wq = __builtin_amdgcn_exp2f(mq - M);
                    den = fmaf(wq, p.ws_l[prow], den);
                    num = fmaf(wq, p.ws_acc[prow * kD + i], num);
                }
    }
    o[i] = f32_to_bf16(den > 0.f ? num / den : 0.f);
}

// ---------------------------------------------------------------------------
template <int NPK>
static hipError_t launch_shared_t(const SharedParams &p, int phase, hipStream_t stream) {
    if (phase & 1) {
        hipLaunchKernelGGL(plan_shared_kernel<NPK>, dim3(p.num_packs), dim3(kWave), 0, stream, p);
        hipLaunchKernelGGL(decode_shared_kernel<NPK>, dim3(p.num_waves), dim3(kWave), 0, stream, p,
                           p.block_tables, p.context_lens, p.out, p.ws_m, p.ws_l, p.ws_acc,
                           p.ws_dir, p.ws_cost, p.ws_pos);
    }
    if (phase & 2)
        hipLaunchKernelGGL(reduce_shared_kernel<NPK>,
                           dim3((unsigned)p.num_kv_heads * p.num_packs * kMaxGroup), dim3(kD), 0,
                           stream, p, p.ws_dir, p.ws_cost);
    return hipGetLastError();
}

hipError_t launch_decode_shared(const SharedParams &p, int phase, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    switch (p.pack) {
    case 4: return launch_shared_t<4>(p, phase, stream);
    case 2: return launch_shared_t<2>(p, phase, stream);
    default: return launch_shared_t<1>(p, phase, stream);
    }
}

}  // namespace pa
