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

// The same merge for a row of n <= 64 pieces of which at most kSparse have
// a non-zero weight (the matrix-core split merges a wavefront's consecutive
// partitions itself and marks the others empty): every wavefront takes one
// piece per lane for the weights (no LDS, no barrier), then the non-empty
// pieces' accumulators are read in one round.  Returns false, having done
// nothing, when the row does not qualify.
constexpr int kSparse = 16;

template <typename T, int D>
__device__ __forceinline__ bool merge_row_sparse(T *out, int n, const float *m, const float *l,
                                                 const float *acc, size_t as) {
    constexpr int kW = D < kWave ? D : kWave;
    if (n > kW) return false;
    const int lane = threadIdx.x % kW;
    const float mq = lane < n ? m[lane] : -INFINITY;
    const float lq = lane < n ? l[lane] : 0.f;   // loaded beside m: one round trip
    float M = mq;
#pragma unroll
    for (int o = kW / 2; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, kW));
    const float wq = (mq == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mq - M);
    float dl = wq * lq;
#pragma unroll
    for (int o = kW / 2; o >= 1; o >>= 1) dl += __shfl_xor(dl, o, kW);
    unsigned long long nz = __ballot(wq != 0.f);
    if (__builtin_popcountll(nz) > kSparse) return false;
    // pieces in ascending order, as merge_row sums them, kChunk at a time
    // with all of a chunk's loads issued together; a slot past the last
    // non-empty piece re-reads the first one (written, so finite) with
    // weight 0, which leaves the sum unchanged
    constexpr int kChunk = 8;
    const int i = threadIdx.x;
    const int q_first = nz != 0 ? __builtin_ctzll(nz) : 0;
    float num = 0.f;
#pragma unroll 1
    for (int c = 0; c < kSparse && nz != 0; c += kChunk) {
        float w[kChunk], a[kChunk];
#pragma unroll
        for (int r = 0; r < kChunk; r++) {
            const bool has = nz != 0;
            const int q = has ? __builtin_ctzll(nz) : q_first;
            nz &= nz - 1;
            w[r] = has ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), q)) : 0.f;
            a[r] = acc[(size_t)q * as + i];
        }
#pragma unroll
        for (int r = 0; r < kChunk; r++) num = fmaf(w[r], a[r], num);
    }
    store_out(out + i, dl > 0.f ? num / dl : 0.f);
    return true;
}

// Fixed partitions: row = (b, h); piece q is partition q of the row.
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_kernel(const ReduceParams p) {
    extern __shared__ float lds[];
    const int row = blockIdx.x;                 // b * num_q_heads + h
    const int b = row / p.num_q_heads;
    const int n = clamp_ctx(p.context_lens[b], p.max_context_len);
    const int n_parts = (n + p.partition_size - 1) / p.partition_size;
    T *out = (T *)p.out + (size_t)row * D;
    if (n_parts == 0) {
        // an empty context has no tiles, so the matrix-core split never
        // visits it: its row is zeros, written here
        store_out(out + threadIdx.x, 0.f);
        return;
    }
    if (n_parts == 1) return;                   // phase 1 wrote the output itself
    const size_t prow = (size_t)row * p.num_partitions;
    if (merge_row_sparse<T, D>(out, n_parts, p.ws_m + prow, p.ws_l + prow, p.ws_acc + prow * D, D))
        return;
    merge_row<T, D>(out, n_parts, p.ws_m + prow, p.ws_l + prow, 1, p.ws_acc + prow * D, D,
                    lds + 8, lds);
}

// Units cut into at most this many pieces are merged in registers.
constexpr int kDirectPieces = 8;

// Work-balanced split.  The split is re-derived from the context lengths
// exactly as the decode kernels made it: sequence b contributes
// T_b = ceil(n_b / 16) tiles per KV head, S_b = sum_{b' < b} T_b',
// TT = sum_b T_b, and each of the W wavefronts owned C = ceil(Hkv TT / W)
// consecutive tiles of the stream (KV head slowest, then sequence, then
// tile).  Unit (g, b) spans [g TT + S_b, g TT + S_b + T_b); if one
// wavefront covered it whole, that wavefront wrote the output.  Otherwise
// wavefronts first..last each hold a piece: wavefront `first` in slot 1 when
// the unit began inside its share (slot 0 when exactly at its start), every
// later one in slot 0.  An empty context gives zeros.
constexpr int kTileTokens = 16;

// Merge the pieces of a unit that starts at stream position `start` and
// spans wavefronts first..last (first < last), for head j of the group,
// into out (head_dim values; thread i writes element i).
template <typename T, int D>
__device__ __forceinline__ void merge_unit_row(const ReduceParams &p, T *out, int start,
                                               int first, int last, int C, int j, float *lds) {
    const int slot0 = start != first * C ? 1 : 0;
    const size_t r0 = ((size_t)first * 2 + slot0) * kMaxGroup + j;
    const size_t r1 = ((size_t)(first + 1) * 2) * kMaxGroup + j;
    const int n = last - first + 1;
    const int i = threadIdx.x;
    auto row_of = [&](int q) -> size_t {   // piece 0 at r0, piece q >= 1 at r1 + 2*16*(q-1)
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
        return;
    }
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

// The register merge for JB heads j0 .. j0+JB-1 of a unit cut into
// n <= kDirectPieces pieces (heads past the group are skipped): all loads
// are issued before the first store.  out0: the output row of head j0.
template <typename T, int D, int JB>
__device__ __forceinline__ void merge_unit_rows_direct(const ReduceParams &p, T *out0, int start,
                                                       int first, int last, int C, int j0) {
    const int slot0 = start != first * C ? 1 : 0;
    const int n = last - first + 1;
    const int i = threadIdx.x;
    float mq[JB][kDirectPieces], lq[JB][kDirectPieces], aq[JB][kDirectPieces];
#pragma unroll
    for (int jj = 0; jj < JB; jj++) {
        const int j = j0 + jj;
#pragma unroll
        for (int q = 0; q < kDirectPieces; q++) {
            if (q < n && j < p.group) {
                const size_t rq =
                    (q == 0 ? ((size_t)first * 2 + slot0) : ((size_t)(first + q) * 2)) * kMaxGroup + j;
                mq[jj][q] = p.ws_m[rq];
                lq[jj][q] = p.ws_l[rq];
                aq[jj][q] = p.ws_acc[rq * D + i];
            }
        }
    }
#pragma unroll
    for (int jj = 0; jj < JB; jj++) {
        if (j0 + jj >= p.group) break;
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kDirectPieces; q++)
            if (q < n) M = fmaxf(M, mq[jj][q]);
        float num = 0.f, den = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int q = 0; q < kDirectPieces; q++) {
                if (q < n && mq[jj][q] != -INFINITY) {   // empty piece: weight 0, not read
                    const float wq = __builtin_amdgcn_exp2f(mq[jj][q] - M);
                    den = fmaf(wq, lq[jj][q], den);
                    num = fmaf(wq, aq[jj][q], num);
                }
            }
        }
        store_out(out0 + (size_t)jj * D + i, den > 0.f ? num / den : 0.f);
    }
}

__device__ __forceinline__ int tiles_of_seq(const ReduceParams &p, int s) {
    return (clamp_ctx(p.context_lens[s], p.max_context_len) + kTileTokens - 1) / kTileTokens;
}

// One workgroup per (sequence, KV head, head of the group) row.
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_balanced_kernel(const ReduceParams p) {
    extern __shared__ float lds[];
    const int j = blockIdx.x % p.group;
    const int unit = blockIdx.x / p.group;
    const int b = unit / p.num_kv_heads;
    const int g = unit % p.num_kv_heads;
    // every wavefront of the workgroup sums the tile counts itself (no
    // barrier): lanes of width kW stride over the sequences
    constexpr int kW = D < kWave ? D : kWave;
    const int lane = threadIdx.x % kW;
    int before = 0, all = 0;
    for (int s = lane; s < p.num_seqs; s += kW) {
        const int t = tiles_of_seq(p, s);
        all += t;
        if (s < b) before += t;
    }
#pragma unroll
    for (int o = kW / 2; o >= 1; o >>= 1) {
        before += __shfl_xor(before, o, kW);
        all += __shfl_xor(all, o, kW);
    }
    const int S = before, TT = all;
    const int Tb = tiles_of_seq(p, b);
    const int C = (TT * p.num_kv_heads + p.num_waves - 1) / p.num_waves;
    T *out = (T *)p.out + ((size_t)b * p.num_q_heads + (size_t)g * p.group + j) * D;
    if (Tb == 0) {
        store_out(out + threadIdx.x, 0.f);
        return;
    }
    const int start = g * TT + S;
    const int first = start / C, last = (start + Tb - 1) / C;
    if (first == last) return;                  // finished by its wavefront
    merge_unit_row<T, D>(p, out, start, first, last, C, j, lds);
}

// The same merge indexed by wavefront boundary, for batches with many more
// rows than wavefronts: only units that a boundary cuts need work, and each
// is handled by the workgroup of the first boundary inside it (boundary
// wb = 1..W-1 sits at stream position wb C), all heads of its group in
// turn.  The last ceil(B / 8) workgroups write zeros for empty contexts,
// 8 sequences each.
constexpr int kZeroSeqsPerGroup = 8;

template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_boundary_kernel(const ReduceParams p) {
    extern __shared__ float lds[];
    const int W = p.num_waves;
    const int B = p.num_seqs;
    const int tid = threadIdx.x;
    if ((int)blockIdx.x >= W - 1) {
        const int s0 = ((int)blockIdx.x - (W - 1)) * kZeroSeqsPerGroup;
        for (int s = s0; s < min(B, s0 + kZeroSeqsPerGroup); s++) {
            if (tiles_of_seq(p, s) != 0) continue;
            T *o = (T *)p.out + (size_t)s * p.num_q_heads * D;
            for (int e = tid; e < p.num_q_heads * D; e += D) store_out(o + e, 0.f);
        }
        return;
    }
    const int wb = blockIdx.x + 1;
    // tile prefix over sequences, per wavefront: lane i owns sequences
    // [i K, i K + K)
    constexpr int kW = D < kWave ? D : kWave;
    const int lane = tid % kW;
    const int K = (B + kW - 1) / kW;
    int local = 0;
    for (int k = 0; k < K; k++) {
        const int s = lane * K + k;
        if (s < B) local += tiles_of_seq(p, s);
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kW; off <<= 1) {
        const int y = __shfl_up(incl, off, kW);
        if (lane >= off) incl += y;
    }
    const int excl = incl - local;
    const int TT = __shfl(incl, kW - 1, kW);
    const int total = TT * p.num_kv_heads;
    const int C = (total + W - 1) / W;
    const int x = wb * C;
    if (x >= total) return;
    const int g = x / TT;
    const int r = x - g * TT;
    // the sequence holding position r: its lane, then a walk
    const unsigned long long own = __ballot(r >= excl && r < incl);
    const int jl = __builtin_ctzll(own) % kW;
    int base = __shfl(excl, jl, kW);
    int b = jl * K;
    int Tb = tiles_of_seq(p, b);
    while (r >= base + Tb) {
        base += Tb;
        b++;
        Tb = tiles_of_seq(p, b);
    }
    const int start = g * TT + base;
    // the unit starts here (not cut), or an earlier boundary cuts it
    if (start == x || start < (wb - 1) * C) return;
    const int first = wb - 1, last = (start + Tb - 1) / C;
    T *out = (T *)p.out + ((size_t)b * p.num_q_heads + (size_t)g * p.group) * D;
    if (last - first + 1 <= kDirectPieces) {
        constexpr int JB = 4;                     // heads merged per round of loads
        for (int j0 = 0; j0 < p.group; j0 += JB)
            merge_unit_rows_direct<T, D, JB>(p, out + (size_t)j0 * D, start, first, last, C, j0);
        return;
    }
    for (int j = 0; j < p.group; j++) {
        merge_unit_row<T, D>(p, out + (size_t)j * D, start, first, last, C, j, lds);
        __syncthreads();                          // lds is reused by the next head
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

template <typename T, int D>
static void launch_reduce_balanced_d(const ReduceParams &p, size_t lds, hipStream_t stream) {
    const unsigned rows = (unsigned)p.num_seqs * (unsigned)p.num_kv_heads * (unsigned)p.group;
    if (rows > (unsigned)p.num_waves) {
        // by boundary: W - 1 cut points plus the empty-context zeroing groups
        const unsigned groups = (unsigned)(p.num_waves - 1) +
                                (unsigned)((p.num_seqs + kZeroSeqsPerGroup - 1) / kZeroSeqsPerGroup);
        hipLaunchKernelGGL((reduce_boundary_kernel<T, D>), dim3(groups), dim3(D), lds, stream, p);
    } else {
        hipLaunchKernelGGL((reduce_balanced_kernel<T, D>), dim3(rows), dim3(D), lds, stream, p);
    }
}

template <typename T>
static void launch_reduce_balanced_t(const ReduceParams &p, size_t lds, hipStream_t stream) {
    switch (p.head_dim) {
    case 16: launch_reduce_balanced_d<T, 16>(p, lds, stream); break;
    case 32: launch_reduce_balanced_d<T, 32>(p, lds, stream); break;
    case 64: launch_reduce_balanced_d<T, 64>(p, lds, stream); break;
    case 128: launch_reduce_balanced_d<T, 128>(p, lds, stream); break;
    default: launch_reduce_balanced_d<T, 256>(p, lds, stream); break;
    }
}

hipError_t launch_reduce_balanced(const ReduceParams &p, int dtype, hipStream_t stream) {
    const unsigned rows = (unsigned)p.num_seqs * (unsigned)p.num_kv_heads * (unsigned)p.group;
    if (rows == 0) return hipSuccess;
    const size_t lds = (8 + (size_t)p.num_waves) * sizeof(float);   // pieces <= wavefronts
    if (dtype == 0)
        launch_reduce_balanced_t<float>(p, lds, stream);
    else
        launch_reduce_balanced_t<uint16_t>(p, lds, stream);
    return hipGetLastError();
}

}  // namespace pa
