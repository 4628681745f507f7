// pa_reduce.hip -- second phase of split-context decode: merge the
// per-partition softmax states of a sequence by log-sum-exp.
//
// Each partition p of sequence b, query head h left (m_p, l_p, acc_p) with
// m_p in base-2 log domain, l_p = sum 2^(s - m_p), acc_p = sum 2^(s - m_p) V.
// The whole-context softmax of "CS349E 第 7 讲 01_paged_attention.py"
// (demo 2, paper eq. 4) is recovered exactly (up to rounding):
//     M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p.
// Partitions are visited in ascending order: no atomics, deterministic.
//
// One workgroup per (sequence, query head), one thread per output element;
// the partition maxima and sums are re-read by every thread (they stay in
// the cache).  The workspace traffic is NP * (head_dim + 2) * 4 bytes per
// (sequence, head) -- small next to the KV bytes of phase 1.
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

template <typename T>
__global__ __launch_bounds__(256) void reduce_kernel(const ReduceParams p) {
    const int row = blockIdx.x;                 // b * num_q_heads + h
    const int b = row / p.num_q_heads;
    const int i = threadIdx.x;                  // element of head_dim
    const int n = clamp_ctx(p.context_lens[b], p.max_context_len);
    const int n_parts = (n + p.partition_size - 1) / p.partition_size;
    if (n_parts <= 1) return;                   // phase 1 wrote the output itself

    const float *m = p.ws_m + (size_t)row * p.num_partitions;
    const float *l = p.ws_l + (size_t)row * p.num_partitions;
    const float *acc = p.ws_acc + (size_t)row * p.num_partitions * p.head_dim;
    float M = -INFINITY;
    for (int q = 0; q < n_parts; q++) M = fmaxf(M, m[q]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
        for (int q = 0; q < n_parts; q++) {
            if (m[q] == -INFINITY) continue;    // a partition with nothing visible
            const float wq = __builtin_amdgcn_exp2f(m[q] - M);
            den = fmaf(wq, l[q], den);
            num = fmaf(wq, acc[(size_t)q * p.head_dim + i], num);
        }
    }
    store_out((T *)p.out + (size_t)row * p.head_dim + i, den > 0.f ? num / den : 0.f);
}

hipError_t launch_reduce(const ReduceParams &p, int dtype, hipStream_t stream) {
    const unsigned rows = (unsigned)p.num_seqs * (unsigned)p.num_q_heads;
    if (rows == 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(reduce_kernel<float>, dim3(rows), dim3(p.head_dim), 0, stream, p);
    else
        hipLaunchKernelGGL(reduce_kernel<uint16_t>, dim3(rows), dim3(p.head_dim), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
