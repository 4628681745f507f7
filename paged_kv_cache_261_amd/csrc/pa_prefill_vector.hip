// pa_prefill_vector.hip -- paged prefill on the vector ALUs, for every shape
// the matrix-core prefill does not take: float32, any head_dim from 16 to
// 256, block sizes from 1 to 256.
//
// What it computes is what pa_prefill.hip computes ("04 - Paged Attention
// 实现进度", section B.2: a prefill batch packed by cu_seqlens_q;
// "CS349E 第 7 讲 01_paged_attention.py", demo 1 prefills a prompt before
// decoding, demo 2 / paper eq. 4 for the softmax over the paged cache): the
// chunk of sequence b is q rows cu[b] .. cu[b+1]-1, the last n_b positions
// of its context_lens[b] tokens; row r at position p = context_lens[b] -
// n_b + r attends over positions 0..p.
//
// How: a chunk row is a decode query whose context ends at its own
// position, so the kernel is the vector decode kernel's loop with more
// columns.  One wavefront serves NC query-head columns of one KV head -- the
// G heads of R = NC / G consecutive chunk rows -- and walks the keys
// 0 .. (its last row's position): a key's 16-byte chunks spread over LPT =
// head_dim / (16 / elem_bytes) lanes, TPW = 64 / LPT keys per load pass,
// every lane holding its chunk of all NC queries, so each K/V load serves
// every column; a column takes a key only up to its row's position
// (causal limit), and keys in blocks outside the pool are left out.  Each
// key slot keeps its own online softmax per column; the TPW slot states are
// merged by log-sum-exp at the end.  Consecutive units (row blocks of one
// sequence and KV head, which read the same keys) run on one XCD at about
// the same time, so their K/V reads meet in its L2.
#include "pa_internal.h"
#include "pa_vector_chunk.h"

#include <math.h>

namespace pa {

template <typename T, int D, int NC>
__global__ __launch_bounds__(kWave) void prefill_vector_kernel(const PrefillParams p) {
    constexpr int kVec = Chunk<T>::kVec;
    constexpr int LPT = D / kVec;              // lanes per key row
    constexpr int TPW = kWave / LPT;           // keys per load pass
    static_assert(LPT >= 1 && LPT <= kWave && kWave % LPT == 0, "head_dim");

    const int lane = threadIdx.x;
    const int r = lane / LPT;                  // key slot within a pass
    const int c = lane % LPT;                  // 16-byte chunk of head_dim

    // unit -> (sequence b, KV head g, row block rb); consecutive units of one
    // (b, g) run side by side on one XCD
    const int u = xcd_remap(blockIdx.x, (int)gridDim.x);
    const int rb = u % p.units_per_seq;
    const int bg = u / p.units_per_seq;
    const int g = bg % p.num_kv_heads;
    const int b = bg / p.num_kv_heads;
    const int G = p.group;
    const int R = NC / G;                      // chunk rows per wavefront
    const int q0 = p.cu_seqlens_q[b];
    const int nq = p.cu_seqlens_q[b + 1] - q0;
    const int r0 = rb * R;
    if (r0 >= nq) return;
    const int n = clamp_ctx(p.context_lens[b], p.max_context_len);
    const int first_pos = n - nq;              // position of chunk row 0
    const int r_end = min(nq, r0 + R);
    const int kmax = max(0, first_pos + r_end);   // keys 0 .. kmax-1 serve the block

    // column j = (row r0 + j / G, head g G + j % G): its query chunk c and
    // its causal limit (keys below it are visible)
    float q[NC][kVec];
    int lim[NC];
#pragma unroll
    for (int j = 0; j < NC; j++) {
        const int rr = j / G;
        const bool ok = rr < R && r0 + rr < r_end;
        lim[j] = ok ? max(0, first_pos + r0 + rr + 1) : 0;
        if (ok) {
            const size_t row = (size_t)(q0 + r0 + rr) * p.num_q_heads + g * G + j % G;
            const uint4 raw = *(const uint4 *)((const T *)p.q + row * D + c * kVec);
            Chunk<T>::unpack(raw, q[j]);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; e++) q[j][e] = 0.f;
        }
    }
    float m[NC], l[NC], acc[NC][kVec];
#pragma unroll
    for (int j = 0; j < NC; j++) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < kVec; e++) acc[j][e] = 0.f;
    }

    const int bs_mask = (1 << p.log2_block) - 1;
    const T *kc = (const T *)p.k_cache;
    const T *vc = (const T *)p.v_cache;
    const int32_t *table = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    // this lane's chunk of key tok, or -1 (past the keys, or in a block
    // outside the pool)
    auto chunk_offset = [&](int tok) -> int64_t {
        if (tok >= kmax) return -1;
        const int phys = table[tok >> p.log2_block];
        if ((unsigned)phys >= (unsigned)p.num_blocks) return -1;
        return ((((int64_t)phys * p.num_kv_heads + g) << p.log2_block) + (tok & bs_mask)) * D +
               c * kVec;
    };
    const uint4 zero = {0u, 0u, 0u, 0u};
    int64_t off = chunk_offset(r);
    uint4 kraw = off >= 0 ? *(const uint4 *)(kc + off) : zero;
    uint4 vraw = off >= 0 ? *(const uint4 *)(vc + off) : zero;

    for (int base = 0; base < kmax; base += TPW) {
        // the next pass's loads go out before this pass is computed
        const int64_t off_n = chunk_offset(base + TPW + r);
        const uint4 kraw_n = off_n >= 0 ? *(const uint4 *)(kc + off_n) : zero;
        const uint4 vraw_n = off_n >= 0 ? *(const uint4 *)(vc + off_n) : zero;

        const int tok = base + r;
        const bool valid = off >= 0;
        float kf[kVec], vf[kVec];
        Chunk<T>::unpack(kraw, kf);
        Chunk<T>::unpack(vraw, vf);
#pragma unroll
        for (int j = 0; j < NC; j++) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; e++) dot = fmaf(q[j][e], kf[e], dot);
#pragma unroll
            for (int o = LPT / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
            const float s = (valid && tok < lim[j]) ? dot * p.scale_log2 : -INFINITY;
            const float m_new = fmaxf(m[j], s);
            if (m_new != -INFINITY) {          // nothing seen yet: the state stays empty
                const float alpha = __builtin_amdgcn_exp2f(m[j] - m_new);
                const float pw = __builtin_amdgcn_exp2f(s - m_new);
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

    // merge the TPW key-slot states (lanes holding the same chunk c)
#pragma unroll
    for (int o = LPT; o < kWave; o <<= 1) {
#pragma unroll
        for (int j = 0; j < NC; j++) {
            const float m_o = __shfl_xor(m[j], o);
            const float l_o = __shfl_xor(l[j], o);
            const float mm = fmaxf(m[j], m_o);
            const float fa = m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[j] - mm);
            const float fb = m_o == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_o - mm);
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
    for (int j = 0; j < NC; j++) {
        const int rr = j / G;
        if (rr >= R || r0 + rr >= r_end) continue;
        const size_t row = (size_t)(q0 + r0 + rr) * p.num_q_heads + g * G + j % G;
        const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;   // no visible key: zeros
        float o[kVec];
#pragma unroll
        for (int e = 0; e < kVec; e++) o[e] = acc[j][e] * inv;
        Chunk<T>::pack_store((T *)p.out + row * D + c * kVec, o);
    }
}

// Columns per wavefront: 16 for float32, 8 for bfloat16 (its 16-byte chunk
// holds twice the values, so the same registers hold half the columns),
// raised to the next power of two of the group size when that is larger.
static int prefill_vector_columns(int group, int dtype) {
    int nc = dtype == 1 ? 8 : 16;
    while (nc < group) nc <<= 1;
    return nc;
}

int prefill_vector_rows(int group, int dtype) { return prefill_vector_columns(group, dtype) / group; }

template <typename T, int D>
static void launch_d(const PrefillParams &p, int nc, unsigned grid, hipStream_t stream) {
    switch (nc) {
    case 8: hipLaunchKernelGGL((prefill_vector_kernel<T, D, 8>), dim3(grid), dim3(kWave), 0, stream, p); break;
    default: hipLaunchKernelGGL((prefill_vector_kernel<T, D, 16>), dim3(grid), dim3(kWave), 0, stream, p); break;
    }
}

template <typename T>
static void launch_t(const PrefillParams &p, int head_dim, int nc, unsigned grid,
                     hipStream_t stream) {
    switch (head_dim) {
    case 16: launch_d<T, 16>(p, nc, grid, stream); break;
    case 32: launch_d<T, 32>(p, nc, grid, stream); break;
    case 64: launch_d<T, 64>(p, nc, grid, stream); break;
    case 128: launch_d<T, 128>(p, nc, grid, stream); break;
    default: launch_d<T, 256>(p, nc, grid, stream); break;
    }
}

hipError_t launch_prefill_vector(const PrefillParams &p, int head_dim, int dtype,
                                 hipStream_t stream) {
    const int64_t units = (int64_t)p.num_seqs * p.num_kv_heads * p.units_per_seq;
    if (units == 0) return hipSuccess;
    const int nc = prefill_vector_columns(p.group, dtype);
    if (dtype == 1)
        launch_t<uint16_t>(p, head_dim, nc, (unsigned)units, stream);
    else
        launch_t<float>(p, head_dim, nc, (unsigned)units, stream);
    return hipGetLastError();
}

}  // namespace pa
