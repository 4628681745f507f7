// pa_reduce.hip -- second phase of split-context decode: merge the partial
// softmax states of each (sequence, query head) by log-sum-exp.
//
// Each piece q of the context of sequence b, query head h left (m_q, l_q,
// acc_q) with m_q in base-2 log domain, l_q = sum 2^(s - m_q) and
// acc_q = sum 2^(s - m_q) V.  The whole-context softmax of
// "CS349E 第 7 讲 01_paged_attention.py" (demo 2, paper eq. 4) is recovered
// exactly (up to rounding):
//     M = max_q m_q,  w_q = 2^(m_q - M),  out = sum_q w_q acc_q / sum_q w_q l_q.
// Pieces are summed in ascending order: no atomics, deterministic.  A piece
// with nothing visible has m_q = -inf and weight 0, and its accumulator is
// not read (the matrix-core split leaves the accumulators of the partitions
// it merged in-wave unwritten).
//
// One workgroup per (sequence, query head) row, one thread per element of
// head_dim.  The piece weights are computed once, by the threads in turn,
// and kept in LDS; the accumulator sum then streams acc_q with coalesced
// loads, several pieces in flight per thread.  Workspace traffic is
// pieces * (head_dim + 2) * 4 bytes per row, small next to the KV bytes the
// first phase reads.
#include "pa_internal.h"

#include <math.h>

namespace pa {

template <typename T>
__device__ __forceinline__ void store_out(T *dst, float x);

template <>
__device__ __forceinline__ void store_out<float>(float *dst, float x) { *dst = x; }

template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *dst, float x) {
    *dst = f32_to_bf16(x);
}

// Reductions over a workgroup of D threads (D a power of two, 16..256).
template <int D>
__device__ __forceinline__ float block_max(float x, float *red) {
    constexpr int kW = D < kWave ? D : kWave;
#pragma unroll
    for (int o = kW / 2; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kW));
    if (D > kWave) {
        if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
        __syncthreads();
        x = red[0];
        for (int i = 1; i < D / kWave; i++) x = fmaxf(x, red[i]);
        __syncthreads();
    }
    return x;
}

template <int D, typename V>
__device__ __forceinline__ V block_sum(V x, V *red) {
    constexpr int kW = D < kWave ? D : kWave;
#pragma unroll
    for (int o = kW / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o, kW);
    if (D > kWave) {
        if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
        __syncthreads();
        x = red[0];
        for (int i = 1; i < D / kWave; i++) x += red[i];
        __syncthreads();
    }
    return x;
}

// Merge n pieces into one output row.  Piece q's state is m[q*ms], l[q*ms]
// and acc + q*as (head_dim floats); `weights` is LDS for n floats.
template <typename T, int D>
__device__ __forceinline__ void merge_row(T *out, int n, const float *m, const float *l,
                                          size_t ms, const float *acc, size_t as,
                                          float *weights, float *red) {
    const int i = threadIdx.x;
    float mx = -INFINITY;
    for (int q = i; q < n; q += D) mx = fmaxf(mx, m[(size_t)q * ms]);
    const float M = block_max<D>(mx, red);
    float dl = 0.f;
    for (int q = i; q < n; q += D) {
        const float mq = m[(size_t)q * ms];
        const float wq = (mq == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq - M);
        weights[q] = wq;
        dl = fmaf(wq, l[(size_t)q * ms], dl);
    }
    const float den = block_sum<D>(dl, red);   // its barrier also publishes weights[]
    if (D <= kWave) __syncthreads();
    float num = 0.f;
    if (M != -INFINITY) {
        // a piece of weight 0 is skipped, not multiplied: an empty piece's
        // accumulator is never written
        const float *a = acc + i;
#pragma unroll 8
        for (int q = 0; q < n; q++)
            if (weights[q] != 0.f) num = fmaf(weights[q], a[(size_t)q * as], num);
    }
    store_out(out + i, den > 0.f ? num / den : 0.f);
}

// Fixed partitions: row = (b, h); piece q is partition q of the row.
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_kernel(const ReduceParams p) {
    extern __shared__ float lds[];
    const int row = blockIdx.x;                 // b * num_q_heads + h
    const int b = row / p.num_q_heads;
    const int n = clamp_ctx(p.context_lens[b], p.max_context_len);
    const int n_parts = (n + p.partition_size - 1) / p.partition_size;
    if (n_parts <= 1) return;                   // phase 1 wrote the output itself
    const size_t prow = (size_t)row * p.num_partitions;
    merge_row<T, D>((T *)p.out + (size_t)row * D, n_parts, p.ws_m + prow, p.ws_l + prow, 1,
                    p.ws_acc + prow * D, D, lds + 8, lds);
}

// Units cut into at most this many pieces are merged in registers.
constexpr int kDirectPieces = 8;

// Work-balanced split: one workgroup per (sequence, KV head, head of the
// group).  The split is re-derived from the context lengths exactly as the
// decode kernel made it: sequence b contributes T_b = ceil(n_b / 16) tiles
// per KV head, S_b = sum_{b' < b} T_b', TT = sum_b T_b, and each of the W
// wavefronts owned C = ceil(Hkv TT / W) consecutive tiles of the stream
// (KV head slowest, then sequence, then tile).  Unit (g, b) spans
// [g TT + S_b, g TT + S_b + T_b); if one wavefront covered it whole, that
// wavefront wrote the output.  Otherwise wavefronts first..last each hold a
// piece: wavefront `first` in slot 1 when the unit began inside its share
// (slot 0 when exactly at its start), every later one in slot 0.  An empty
// context gives zeros.
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_balanced_kernel(const ReduceParams p) {
    extern __shared__ float lds[];
    const int j = blockIdx.x % p.group;
    const int unit = blockIdx.x / p.group;
    const int b = unit / p.num_kv_heads;
    const int g = unit % p.num_kv_heads;
    constexpr int kTileTokens = 16;
    // every wavefront of the workgroup sums the tile counts itself (no
    // barrier): lanes of width kW stride over the sequences
    constexpr int kW = D < kWave ? D : kWave;
    const int lane = threadIdx.x % kW;
    int before = 0, all = 0;
    for (int s = lane; s < p.num_seqs; s += kW) {
        const int t = (clamp_ctx(p.context_lens[s], p.max_context_len) + kTileTokens - 1) /
                      kTileTokens;
        all += t;
        if (s < b) before += t;
    }
#pragma unroll
    for (int o = kW / 2; o >= 1; o >>= 1) {
        before += __shfl_xor(before, o, kW);
        all += __shfl_xor(all, o, kW);
    }
    const int S = before, TT = all;
    const int Tb = (clamp_ctx(p.context_lens[b], p.max_context_len) + kTileTokens - 1) /
                   kTileTokens;
    const int C = (TT * p.num_kv_heads + p.num_waves - 1) / p.num_waves;
    T *out = (T *)p.out + ((size_t)b * p.num_q_heads + (size_t)g * p.group + j) * D;
    if (Tb == 0) {
        store_out(out + threadIdx.x, 0.f);
        return;
    }
    const int start = g * TT + S;
    const int first = start / C, last = (start + Tb - 1) / C;
    if (first == last) return;                  // finished by its wavefront
    // pieces are wavefronts first..last; wavefront first's piece sits in
    // slot 1 unless the unit began exactly at its share's start, the rest
    // in slot 0: piece 0 at row r0, piece q >= 1 at row r1 + 2*16*(q-1)
    const int slot0 = start != first * C ? 1 : 0;
    const size_t r0 = ((size_t)first * 2 + slot0) * kMaxGroup + j;
    const size_t r1 = ((size_t)(first + 1) * 2) * kMaxGroup + j;
    const int n = last - first + 1;
    const int i = threadIdx.x;
    auto row_of = [&](int q) -> size_t {
        return q == 0 ? r0 : r1 + (size_t)(q - 1) * 2 * kMaxGroup;
    };
    if (n <= kDirectPieces) {
        // every thread loads every piece's m and l (one broadcast address
        // per piece) with its own accumulator element, all at once, and
        // merges in registers: one round trip, no barrier
        float mq[kDirectPieces], lq[kDirectPieces], aq[kDirectPieces];
#pragma unroll
        for (int q = 0; q < kDirectPieces; q++) {
            if (q < n) {
                const size_t rq = row_of(q);
                mq[q] = p.ws_m[rq];
                lq[q] = p.ws_l[rq];
                aq[q] = p.ws_acc[rq * D + i];
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kDirectPieces; q++)
            if (q < n) M = fmaxf(M, mq[q]);
        float num = 0.f, den = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int q = 0; q < kDirectPieces; q++) {
                if (q < n && mq[q] != -INFINITY) {   // empty piece: weight 0, not read
                    const float wq = __builtin_amdgcn_exp2f(mq[q] - M);
                    den = fmaf(wq, lq[q], den);
                    num = fmaf(wq, aq[q], num);
                }
            }
        }
        store_out(out + i, den > 0.f ? num / den : 0.f);
        return;
    }
    if (slot0 == 0) {
        // uniform stride 2 * 16 rows between consecutive pieces
        merge_row<T, D>(out, n, p.ws_m + r0, p.ws_l + r0, 2 * kMaxGroup, p.ws_acc + r0 * D,
                        (size_t)2 * kMaxGroup * D, lds + 8, lds);
    } else {
        // the first piece is one slot further than the stride predicts
        float *red = lds, *weights = lds + 8;
        float mx = p.ws_m[r0];
        for (int q = 1 + i; q < n; q += D) mx = fmaxf(mx, p.ws_m[row_of(q)]);
        const float M = block_max<D>(mx, red);
        float dl = 0.f;
        for (int q = i; q < n; q += D) {
            const size_t rq = row_of(q);
            const float mq = p.ws_m[rq];
            const float wq = (mq == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq - M);
            weights[q] = wq;
            dl = fmaf(wq, p.ws_l[rq], dl);
        }
        const float den = block_sum<D>(dl, red);
        if (D <= kWave) __syncthreads();
        float num = 0.f;
        if (M != -INFINITY) {
            num = weights[0] * p.ws_acc[r0 * D + i];
            const float *a = p.ws_acc + r1 * D + i;
#pragma unroll 8
            for (int q = 1; q < n; q++)
                num = fmaf(weights[q], a[(size_t)(q - 1) * 2 * kMaxGroup * D], num);
        }
        store_out(out + i, den > 0.f ? num / den : 0.f);
    }
}

template <typename T>
static hipError_t launch_reduce_t(const ReduceParams &p, size_t lds, hipStream_t stream) {
    const unsigned rows = (unsigned)p.num_seqs * (unsigned)p.num_q_heads;
    switch (p.head_dim) {
    case 16: hipLaunchKernelGGL((reduce_kernel<T, 16>), dim3(rows), dim3(16), lds, stream, p); break;
    case 32: hipLaunchKernelGGL((reduce_kernel<T, 32>), dim3(rows), dim3(32), lds, stream, p); break;
    case 64: hipLaunchKernelGGL((reduce_kernel<T, 64>), dim3(rows), dim3(64), lds, stream, p); break;
    case 128: hipLaunchKernelGGL((reduce_kernel<T, 128>), dim3(rows), dim3(128), lds, stream, p); break;
    default: hipLaunchKernelGGL((reduce_kernel<T, 256>), dim3(rows), dim3(256), lds, stream, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams &p, int dtype, hipStream_t stream) {
    if (p.num_seqs == 0) return hipSuccess;
    const size_t lds = (8 + (size_t)p.num_partitions) * sizeof(float);
    return dtype == 0 ? launch_reduce_t<float>(p, lds, stream)
                      : launch_reduce_t<uint16_t>(p, lds, stream);
}

template <typename T>
static void launch_reduce_balanced_t(const ReduceParams &p, unsigned rows, size_t lds,
                                     hipStream_t stream) {
    switch (p.head_dim) {
    case 16: hipLaunchKernelGGL((reduce_balanced_kernel<T, 16>), dim3(rows), dim3(16), lds, stream, p); break;
    case 32: hipLaunchKernelGGL((reduce_balanced_kernel<T, 32>), dim3(rows), dim3(32), lds, stream, p); break;
    case 64: hipLaunchKernelGGL((reduce_balanced_kernel<T, 64>), dim3(rows), dim3(64), lds, stream, p); break;
    case 128: hipLaunchKernelGGL((reduce_balanced_kernel<T, 128>), dim3(rows), dim3(128), lds, stream, p); break;
    default: hipLaunchKernelGGL((reduce_balanced_kernel<T, 256>), dim3(rows), dim3(256), lds, stream, p); break;
    }
}

hipError_t launch_reduce_balanced(const ReduceParams &p, int dtype, hipStream_t stream) {
    const unsigned rows = (unsigned)p.num_seqs * (unsigned)p.num_kv_heads * (unsigned)p.group;
    if (rows == 0) return hipSuccess;
    const size_t lds = (8 + (size_t)p.num_waves) * sizeof(float);   // pieces <= wavefronts
    if (dtype == 0)
        launch_reduce_balanced_t<float>(p, rows, lds, stream);
    else
        launch_reduce_balanced_t<uint16_t>(p, rows, lds, stream);
    return hipGetLastError();
}

}  // namespace pa
