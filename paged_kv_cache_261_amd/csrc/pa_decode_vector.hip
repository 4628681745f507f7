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

#include <math.h>

namespace pa {

namespace {

template <typename T>
struct Chunk;

// 16 bytes of float32: 4 values.
template <>
struct Chunk<float> {
    static constexpr int kVec = 4;
    __device__ static void unpack(const uint4 &w, float (&x)[4]) {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z);
        x[3] = __uint_as_float(w.w);
    }
    __device__ static void pack_store(void *dst, const float (&x)[4]) {
        uint4 w;
        w.x = __float_as_uint(x[0]);
        w.y = __float_as_uint(x[1]);
        w.z = __float_as_uint(x[2]);
        w.w = __float_as_uint(x[3]);
        *(uint4 *)dst = w;
    }
};

// 16 bytes of bfloat16: 8 values.
template <>
struct Chunk<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static void unpack(const uint4 &w, float (&x)[8]) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
        x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
    __device__ static void pack_store(void *dst, const float (&x)[8]) {
        uint4 w;
        w.x = f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        w.y = f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        w.z = f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
        w.w = f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
        *(uint4 *)dst = w;
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace

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
