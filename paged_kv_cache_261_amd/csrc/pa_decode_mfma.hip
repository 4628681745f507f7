// pa_decode_mfma.hip -- PagedAttention decode for bfloat16 caches with the
// grouped query heads of one KV head on the CDNA4 matrix cores.
//
// Same result as the vector kernel ("CS349E 第 7 讲 01_paged_attention.py",
// demo 2, paper eq. 4: scores block by block through the block table, one
// softmax over the whole context, probability-weighted sum of V), computed
// one 16-token tile at a time by one wavefront per (sequence, KV head,
// partition):
//
//   scores   S[16 tokens x 16 heads] = K_tile[16 x 128] . Q^T[128 x 16]
//            4 x v_mfma_f32_16x16x32_bf16; the G query heads of the KV head
//            fill G of the 16 columns (the rest are zero queries);
//   softmax  online, per head, in base-2 log domain; the tile max is
//            reduced across the 4 lane groups with two cross-lane shuffles;
//   P.V      O^T[128 x 16] += V_tile^T[128 x 16 tokens] . P^T[16 x 16]
//            8 x v_mfma_f32_16x16x16_bf16 (P rounded to bfloat16, fp32
//            accumulation).
//
// Register layouts (lane = 16 * grp + row16):
//  - S: lane holds S[token 4*grp + i][head row16], i = 0..3.  That is
//    exactly the B operand of the P.V product (k = token 4*grp + i,
//    column = head row16), so P never leaves the lane.
//  - K operand (A of the score MFMA, row = token): lane loads the 64
//    contiguous bytes of token row16 at dims [32*grp, 32*grp + 32); the
//    query (B, column = head) is loaded with the same dim order, so the
//    products pair matching dims whatever the hardware's k order is.
//  - V operand (A of the P.V MFMA, row = dim, k = token): lane loads the 16
//    contiguous bytes of dims [8*row16, 8*row16 + 8) of tokens 4*grp + i;
//    MFMA n uses dim 8*row16 + n of those 4 tokens (one byte-permute per
//    register pair to transpose).
//  - O^T accumulator: lane holds head row16 at dims 32*grp + 8*i + n, i.e.
//    32 contiguous dims, written back as 16-byte stores.
//
// Memory: a (block, KV head) tile of 16 tokens x 128 dims is 4 KiB
// contiguous; each lane issues 4 + 4 sixteen-byte loads per tile, and the
// next tile's loads are issued before the current tile is computed.  The
// block table is read 64 entries at a time into one register per lane and
// each tile's physical block id is taken with a scalar lane read, so the
// tile base address is computed in scalar registers.
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

constexpr int kD = 128;          // head_dim handled by this kernel
constexpr int kTile = 16;        // tokens per tile
constexpr int kRowBytes = kD * 2;

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
#define PA_MFMA_WAVES 0
#endif

constexpr int kDepth = PA_MFMA_DEPTH;
constexpr int kBufs = kDepth + 1;

__global__ __launch_bounds__(kWave)
#if PA_MFMA_WAVES > 0
__attribute__((amdgpu_waves_per_eu(PA_MFMA_WAVES)))
#endif
void decode_mfma_kernel(const DecodeParams p) {
    const int lane = threadIdx.x;
    const int row16 = lane & 15;
    const int grp = lane >> 4;

    const int u = xcd_remap(blockIdx.x, p.num_units);
    const Unit w = unit_of(u, p.num_seqs, p.num_kv_heads);
    const int n = clamp_ctx(p.context_lens[w.b], p.max_context_len);
    const int P = p.partition_size;
    const int t0 = w.part * P;
    const int n_parts = n == 0 ? 1 : (n + P - 1) / P;
    if (w.part >= n_parts) return;
    const int t1 = min(n, t0 + P);
    const int G = p.group;

    const char *kbase = (const char *)p.k_cache;
    const char *vbase = (const char *)p.v_cache;
    const int32_t *__restrict__ table = p.block_tables + (size_t)w.b * p.max_blocks_per_seq;
    const int log2bs = p.log2_block;
    const int bs_mask = (1 << log2bs) - 1;

    // query operand: head row16 of the group, dims [32*grp, 32*grp + 32)
    bf16x8 qv[4];
    {
        const bool real = row16 < G;
        const char *qrow = (const char *)p.q +
                           (((size_t)w.b * p.num_q_heads + w.g * G + (real ? row16 : 0)) * kD +
                            32 * grp) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            u32x4 raw = *(const u32x4 *)(qrow + 16 * kk);
            if (!real) raw = (u32x4){0u, 0u, 0u, 0u};
            qv[kk] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    const int k_lane_off = row16 * kRowBytes + grp * 64;       // + 16 * kk
    const int v_lane_off = (4 * grp) * kRowBytes + row16 * 16; // + i * kRowBytes

    f32x4 o[8];
#pragma unroll
    for (int nn = 0; nn < 8; nn++) o[nn] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;     // running max of head row16 (base-2 log domain)
    float lsum = 0.f;        // this lane's share of the running sum

    const int ntiles = (t1 - t0 + kTile - 1) / kTile;

    // Physical block of tile t (index clamped into the unit, so always a
    // valid table entry for t >= 0).
    auto phys_of = [&](int t) -> int {
        const int tt = t < ntiles ? t : ntiles - 1;
        return table[(t0 + tt * kTile) >> log2bs];
    };
    // Issue the loads of tile t through buffer descriptors whose byte range
    // covers only the tile's visible token rows: rows past the context (and
    // every row of a tile past the unit, or of a block id out of range) read
    // as zero without touching memory, so the loop needs no branches and the
    // compiler can count outstanding loads exactly.
    auto load_tile = [&](int t, int phys, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
        const int tok = t0 + t * kTile;
        const bool ok = t < ntiles && (unsigned)phys < (unsigned)p.num_blocks;
        const int rows = ok ? min(kTile, t1 - tok) : 0;
        const size_t tile = ((((size_t)(ok ? phys : 0) * p.num_kv_heads + w.g) << log2bs) +
                             (tok & bs_mask)) * (size_t)kRowBytes;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + tile), (short)0, rows * kRowBytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + tile), (short)0, rows * kRowBytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < 4; i++)   // the 16*i step stays inside the lane's row
            kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  krs, k_lane_off, 16 * i, 0));
#pragma unroll
        for (int i = 0; i < 4; i++)
            vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  vrs, v_lane_off + i * kRowBytes, 0, 0));
    };

    auto compute_tile = [&](int t, const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]), qv[kk],
                                                        S, 0, 0, 0);
        const int nv = t1 - (t0 + t * kTile);     // visible tokens in this tile (>= 1)
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; i++) s[i] = 4 * grp + i < nv ? S[i] * p.scale_log2 : -INFINITY;
        const float tmax = xor32_max(xor16_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))));
        const float m_new = fmaxf(m, tmax);       // finite: the tile has a visible token
        const float alpha = fast_exp2(m - m_new); // 0 on the first tile (m = -inf)
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; i++) pr[i] = fast_exp2(s[i] - m_new);
        lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m = m_new;
#pragma unroll
        for (int nn = 0; nn < 8; nn++) o[nn] *= alpha;
        const s16x4 pb = __builtin_bit_cast(
            s16x4, (uint2){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
#pragma unroll
        for (int nn = 0; nn < 8; nn++) {
            // dim 8*row16 + nn of tokens 4*grp + 0..3: word nn/2 of each row,
            // low half for even nn, high half for odd nn
            const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t d0 = __builtin_amdgcn_perm(vr[1][nn >> 1], vr[0][nn >> 1], sel);
            const uint32_t d1 = __builtin_amdgcn_perm(vr[3][nn >> 1], vr[2][nn >> 1], sel);
            const s16x4 a = __builtin_bit_cast(s16x4, (uint2){d0, d1});
            o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[nn], 0, 0, 0);
        }
    };

    if (ntiles > 0) {
        u32x4 kr[kBufs][4], vr[kBufs][4];
        int phys_next = phys_of(0);
#pragma unroll
        for (int j = 0; j < kDepth; j++) {         // prologue: tiles 0 .. depth-1
            load_tile(j, phys_next, kr[j], vr[j]);
            phys_next = phys_of(j + 1);
        }
        for (int tb = 0; tb < ntiles; tb += kBufs) {
#pragma unroll
            for (int j = 0; j < kBufs; j++) {
                const int t = tb + j;
                if (t >= ntiles) break;
                load_tile(t + kDepth, phys_next, kr[(j + kDepth) % kBufs], vr[(j + kDepth) % kBufs]);
                phys_next = phys_of(t + kDepth + 1);
                // keep the prefetch ahead of the wait for tile t
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, kr[j], vr[j]);
            }
        }
    }

    lsum = xor32_sum(xor16_sum(lsum));
    if (row16 >= G) return;
    const size_t row = (size_t)w.b * p.num_q_heads + w.g * G + row16;
    if (n_parts == 1) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        char *dst = (char *)p.out + (row * kD + 32 * grp) * 2;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            u32x4 wv;
#pragma unroll
            for (int j = 0; j < 4; j++)
                wv[j] = pack_bf16x2(o[2 * j][i] * inv, o[2 * j + 1][i] * inv);
            *(u32x4 *)(dst + 16 * i) = wv;
        }
    } else {
        const size_t prow = row * p.num_partitions + w.part;
        float *dst = p.ws_acc + prow * kD + 32 * grp;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f32x4 lo = {o[0][i], o[1][i], o[2][i], o[3][i]};
            const f32x4 hi = {o[4][i], o[5][i], o[6][i], o[7][i]};
            *(f32x4 *)(dst + 8 * i) = lo;
            *(f32x4 *)(dst + 8 * i + 4) = hi;
        }
        if (grp == 0) {
            p.ws_m[prow] = m;
            p.ws_l[prow] = lsum;
        }
    }
}

hipError_t launch_decode_mfma(const DecodeParams &p, hipStream_t stream) {
    if (p.num_units == 0) return hipSuccess;
    hipLaunchKernelGGL(decode_mfma_kernel, dim3(p.num_units), dim3(kWave), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
