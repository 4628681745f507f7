// pa_mfma_tile.h -- the per-tile step of matrix-core PagedAttention decode,
// shared by the decode kernels of pa_decode_mfma.hip and pa_decode_shared.hip.
//
// One wavefront holds the softmax state of 16 query-head columns and folds in
// one 16-token tile of K and V at a time ("CS349E 第 7 讲
// 01_paged_attention.py", demo 2, paper eq. 4: scores block by block, one
// softmax over the whole context kept online, V multiplied in block by
// block):
//
//   scores   S[16 tokens x 16 columns] = K_tile[16 x 128] . Q^T[128 x 16]
//            4 x v_mfma_f32_16x16x32_bf16;
//   softmax  online per column in base-2 log domain; the tile max is reduced
//            across the 4 lane groups with two row-swap permutes, and the
//            reference max lags the running max by at most 8 (lazy rescale);
//   P.V      O^T[128 x 16] += V_tile^T[128 x 16 tokens] . P^T[16 x 16]
//            2 x 8 x v_mfma_f32_16x16x16_bf16: P as the sum of two bfloat16
//            parts (its high part and what rounding dropped), fp32
//            accumulation.
//
// Register layouts (lane = 16 * grp + row16; column = row16):
//  - S: lane holds S[token 4*grp + i][column row16], i = 0..3 -- exactly the
//    B operand of the P.V product (k = token 4*grp + i, column row16), so P
//    never leaves the lane.
//  - K operand (A of the score MFMA, row = token): for MFMA kk the lane holds
//    dims [32*kk + 8*grp, +8) of token row16, so each of a tile's four
//    16-byte loads reads 64 contiguous bytes of every row; the query (B,
//    column) uses the same dim order, so the products pair matching dims
//    whatever the hardware's k order is.
//  - V operand (A of the P.V MFMA, row = dim, k = token): lane loads the 16
//    contiguous bytes of dims [8*row16, +8) of tokens 4*grp + i (each load
//    reads 4 whole rows); MFMA n uses dim 8*row16 + n of those 4 tokens (one
//    byte-permute per register to transpose).
//  - O^T accumulator: lane holds column row16 at dims 32*grp + 8*i + n, i.e.
//    32 contiguous dims, written back as 16-byte stores.
#pragma once

#include <math.h>

#include "pa_internal.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // head_dim of the matrix-core kernels
constexpr int kTile = 16;        // tokens per tile
constexpr int kRowBytes = kD * 2;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer descriptor, CDNA
// Cache policy (buffer-load aux bits) of K/V tiles read once per launch: the
// non-temporal hint (bit 1) marks their lines evict-first, so a stream of
// tiles that will not be read again does not push other lines out of the
// caches.  On the decode workloads it raised the achieved HBM rate from
// 5.8 to 6.4-6.6 TB/s.
constexpr int kStreamAux = 2;
// Tiles read by many wavefronts in turn (prefill) keep the default policy.
constexpr int kReuseAux = 0;

// Lazy rescale: a column's reference max (the m the exponents are taken
// against) moves only when a tile's max exceeds it by more than this many
// log2 units.  Any reference gives the same softmax -- l and the accumulator
// are both taken against it and the final O / l cancels it -- and a lag of
// at most 8 keeps every p <= 2^8, far from the fp32 and bf16 ranges.  Once
// the reference settles, alpha is exactly 1 for every column and the
// rescale below is skipped.  0 gives the plain running max.
#ifndef PA_RESCALE_SLACK
#define PA_RESCALE_SLACK 8
#endif

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

// Softmax state of one wavefront for its 16 columns.
struct Acc {
    f32x4 o[8];     // O^T: column row16, dims 32*grp + 8*i + n  ->  o[n][i]
    float m;        // running max of column row16 (base-2 log domain)
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

// Sum the lane shares of l over the 4 lane groups (after the last tile).
__device__ __forceinline__ void acc_finish(Acc &a) { a.lsum = xor32_sum(xor16_sum(a.lsum)); }

// dst <- the log-sum-exp merge of two finished states (each lane holds its
// column's full l): M = max(m1, m2), weights 2^(m - M), an empty state
// (m = -inf) weighing 0.
__device__ __forceinline__ void acc_merge(Acc &dst, const Acc &src) {
    const float M = fmaxf(dst.m, src.m);
    const float wd = dst.m == -INFINITY ? 0.f : fast_exp2(dst.m - M);
    const float ws = src.m == -INFINITY ? 0.f : fast_exp2(src.m - M);
#pragma unroll
    for (int nn = 0; nn < 8; nn++) dst.o[nn] = dst.o[nn] * wd + src.o[nn] * ws;
    dst.lsum = dst.lsum * wd + src.lsum * ws;
    dst.m = M;
}

// Fold one tile into the state.  kr / vr: the tile's K and V operands as
// loaded; nv: rows of the tile visible to this lane's column (tokens at or
// past nv are selected out).  With kMaybeEmpty a column may see no visible
// row in this tile nor before it; the update then leaves it untouched.
// v_op(nn) gives the A operand of P.V product nn (4 bf16: one dim, tokens
// 4*grp .. 4*grp+3 of the lane's group).
template <bool kMaybeEmpty, typename VOp>
__device__ __forceinline__ void tile_update_v(const u32x4 (&kr)[4], VOp &&v_op,
                                              const bf16x8 (&qv)[4], int nv, float scale_log2,
                                              Acc &a, Lane ln) {
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]), qv[kk], S,
                                                    0, 0, 0);
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; i++) s[i] = 4 * ln.grp + i < nv ? S[i] * scale_log2 : -INFINITY;
    const float tmax = xor32_max(xor16_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))));
#if PA_RESCALE_SLACK > 0
    float m_new = tmax > a.m + (float)PA_RESCALE_SLACK ? tmax : a.m;
#else
    float m_new = fmaxf(a.m, tmax);
#endif
    // Without kMaybeEmpty m_new is finite (the tile has a visible row for
    // every column) and alpha is 0 on a column's first tile (m = -inf).
    // With it, a column that has seen nothing keeps m = -inf: shift by 0
    // instead, which makes alpha and every p exactly 0.
    const float shift = (kMaybeEmpty && m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(a.m - shift);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; i++) pr[i] = fast_exp2(s[i] - shift);
    a.lsum = a.lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    a.m = m_new;
    // once the running max settles, alpha is 1 for every column and the
    // rescale would multiply by one: skip it (same bits, fewer VALU ops)
#ifndef PA_NO_RESCALE_SKIP
    if (__ballot(alpha != 1.f) != 0)
#endif
    {
#pragma unroll
        for (int nn = 0; nn < 8; nn++) a.o[nn] *= alpha;
    }
    // P enters the product as two bfloat16 parts, hi = bf16(p) and
    // lo = bf16(p - hi), so its rounding costs 2^-17 of a weight instead of
    // 2^-9; the second product is free here, where the tile loads set the
    // pace
    const uint32_t h01 = pack_bf16x2(pr[0], pr[1]), h23 = pack_bf16x2(pr[2], pr[3]);
    const s16x4 pb = __builtin_bit_cast(s16x4, (uint2){h01, h23});
    const s16x4 pl = __builtin_bit_cast(
        s16x4, (uint2){pack_bf16x2(pr[0] - bf16_lo(h01), pr[1] - bf16_hi(h01)),
                       pack_bf16x2(pr[2] - bf16_lo(h23), pr[3] - bf16_hi(h23))});
#pragma unroll
    for (int nn = 0; nn < 8; nn++) {
        const s16x4 vo = v_op(nn);
        a.o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo, pb, a.o[nn], 0, 0, 0);
        a.o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo, pl, a.o[nn], 0, 0, 0);
    }
}

// The tile step on V as loaded by load_tile_rows: product nn takes dim
// 8*row16 + nn of the lane group's 4 tokens, transposed in registers.
template <bool kMaybeEmpty>
__device__ __forceinline__ void tile_update(const u32x4 (&kr)[4], const u32x4 (&vr)[4],
                                            const bf16x8 (&qv)[4], int nv, float scale_log2,
                                            Acc &a, Lane ln) {
    tile_update_v<kMaybeEmpty>(
        kr,
        [&](int nn) {
            // word nn/2 of each row, low half for even nn, high half for odd nn
            const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t d0 = __builtin_amdgcn_perm(vr[1][nn >> 1], vr[0][nn >> 1], sel);
            const uint32_t d1 = __builtin_amdgcn_perm(vr[3][nn >> 1], vr[2][nn >> 1], sel);
            return __builtin_bit_cast(s16x4, (uint2){d0, d1});
        },
        qv, nv, scale_log2, a, ln);
}

// Issue the 8 sixteen-byte loads of one (block, KV head) tile through buffer
// descriptors covering only its first `rows` token rows: rows past it (and
// the whole tile when rows == 0) read as zero without a memory access.
// tile_byte_off: byte offset of the tile's first row in the caches.
template <int kAux = kStreamAux>
__device__ __forceinline__ void load_tile_rows(const char *kbase, const char *vbase,
                                               size_t tile_byte_off, int rows, Lane ln,
                                               u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    const int k_lane_off = ln.row16 * kRowBytes + ln.grp * 16;        // + 64 * kk
    const int v_lane_off = (4 * ln.grp) * kRowBytes + ln.row16 * 16;  // + i * kRowBytes
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(kbase + tile_byte_off), (short)0, rows * kRowBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(vbase + tile_byte_off), (short)0, rows * kRowBytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 4; i++)   // the 64*i step stays inside the lane's row
        kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              krs, k_lane_off, 64 * i, kAux));
#pragma unroll
    for (int i = 0; i < 4; i++)
        vr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              vrs, v_lane_off + i * kRowBytes, 0, kAux));
}

// Unnormalised state of column row16 to a partial slot: m and l to
// m_dst / l_dst (one lane group writes them), the accumulator (head_dim
// floats) to acc_dst.
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

// O / l of column row16, in bfloat16, to one head_dim row of the output.
__device__ __forceinline__ void store_row(void *out_row, const Acc &a, Lane ln) {
    const float inv = a.lsum > 0.f ? 1.f / a.lsum : 0.f;
    char *dst = (char *)out_row + 32 * ln.grp * 2;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        u32x4 wv;
#pragma unroll
        for (int j = 0; j < 4; j++)
            wv[j] = pack_bf16x2(a.o[2 * j][i] * inv, a.o[2 * j + 1][i] * inv);
        *(u32x4 *)(dst + 16 * i) = wv;
    }
}

}  // namespace pa
