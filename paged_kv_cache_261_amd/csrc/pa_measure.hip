// pa_measure.hip -- a plain streaming read of one device buffer, the
// practical HBM read ceiling the decode kernels are set against (calibration
// for the benchmark; not part of the decode path).
//
// PA_MEASURE_SINK_WORDS workgroups of 256 threads take pieces of 32 KiB in
// turn (workgroup w reads pieces w, w + G, w + 2 G, ...): every thread
// issues its 8 sixteen-byte loads of a piece before using any, through a
// buffer descriptor that covers the piece, so the access has the shape of a
// decode kernel's tile loads.  The words read are XOR-folded and each
// workgroup stores one word, so no load can be optimised away and the host
// can check that every byte was read.
#include "pa_measure.h"

#include "pa_internal.h"

namespace pa {

constexpr int kReadThreads = 256;
constexpr int kReadLoads = 8;
constexpr int64_t kPieceBytes = (int64_t)kReadThreads * kReadLoads * 16;

typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

template <int kAux>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const char *__restrict__ buf,
                                                                   int64_t bytes,
                                                                   uint32_t *__restrict__ sink) {
    const int64_t pieces = (bytes + kPieceBytes - 1) / kPieceBytes;
    uint32_t x = 0;
    for (int64_t pc = blockIdx.x; pc < pieces; pc += gridDim.x) {
        const int64_t off = pc * kPieceBytes;
        const int64_t len = bytes - off < kPieceBytes ? bytes - off : kPieceBytes;
        // bytes past `len` read as zero, which leaves the XOR unchanged
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(buf + off), (short)0, (int)len, 0x00020000);
        u32x4m r[kReadLoads];
#pragma unroll
        for (int j = 0; j < kReadLoads; j++)
            r[j] = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs, (threadIdx.x + j * kReadThreads) * 16, 0,
                                                  kAux));
#pragma unroll
        for (int j = 0; j < kReadLoads; j++) x ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
    __shared__ uint32_t part[kReadThreads / kWave];
    if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int i = 0; i < kReadThreads / kWave; i++) y ^= part[i];
        sink[blockIdx.x] = y;
    }
}

// Paged tile reads: W persistent wavefronts (one per SIMD), wavefront w the
// tiles [w C, w C + C) of the list, each tile's 16-byte loads (L per lane
// per pool) issued kTileDepth tiles ahead of their use, as the decode
// kernels do.
constexpr int kTileWaves = PA_MEASURE_SINK_WORDS / 4;   // 1024
constexpr int kTileDepth = 3;

template <int L>
__global__ __launch_bounds__(kWave) void tile_read_kernel(const char *__restrict__ kp,
                                                          const char *__restrict__ vp,
                                                          const int32_t *__restrict__ tiles,
                                                          int num_tiles, int chunk,
                                                          uint32_t *__restrict__ sink) {
    constexpr int kBytes = L * kWave * 16;
    const int t0 = blockIdx.x * chunk;
    const int t1 = min(num_tiles, t0 + chunk);
    u32x4m kr[kTileDepth + 1][L], vr[kTileDepth + 1][L];
    auto issue = [&](int t, u32x4m (&k)[L], u32x4m (&v)[L]) {
        const bool ok = t < t1;
        // (index 0 when past the share, so even a hoisted load stays in the list)
        const size_t off = ok ? (size_t)tiles[ok ? t : 0] * kBytes : 0;
        const int len = ok ? kBytes : 0;   // past the share: nothing is read
        const __amdgpu_buffer_rsrc_t ks = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kp + off), (short)0, len, 0x00020000);
        const __amdgpu_buffer_rsrc_t vs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vp + off), (short)0, len, 0x00020000);
#pragma unroll
        for (int j = 0; j < L; j++) {
            k[j] = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(
                                                  ks, (threadIdx.x + j * kWave) * 16, 0, 2));
            v[j] = __builtin_bit_cast(u32x4m, __builtin_amdgcn_raw_buffer_load_b128(
                                                  vs, (threadIdx.x + j * kWave) * 16, 0, 2));
        }
    };
    uint32_t x = 0;
#pragma unroll
    for (int d = 0; d < kTileDepth; d++) issue(t0 + d, kr[d], vr[d]);
    for (int tb = t0; tb < t1; tb += kTileDepth + 1) {
#pragma unroll
        for (int j = 0; j <= kTileDepth; j++) {
            const int t = tb + j;
            if (t >= t1) break;
            issue(t + kTileDepth, kr[(j + kTileDepth) % (kTileDepth + 1)],
                  vr[(j + kTileDepth) % (kTileDepth + 1)]);
            __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the use
#pragma unroll
            for (int i = 0; i < L; i++)
                x ^= kr[j][i].x ^ kr[j][i].y ^ kr[j][i].z ^ kr[j][i].w ^ vr[j][i].x ^
                     vr[j][i].y ^ vr[j][i].z ^ vr[j][i].w;
        }
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
    // four words per wavefront, so every sink word is written
    if (threadIdx.x < 4) sink[blockIdx.x * 4 + threadIdx.x] = threadIdx.x == 0 ? x : 0u;
}

}  // namespace pa

extern "C" int pa_measure_tile_read(const void *k_pool, const void *v_pool,
                                    const int32_t *tiles, int num_tiles, int tile_bytes,
                                    uint32_t *sink, void *stream) {
    if (!sink || !k_pool || !v_pool || !tiles) return PA_ERR_NULL;
    if (num_tiles < 1) return PA_ERR_SHAPE;
    if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192)
        return PA_ERR_UNSUPPORTED;
    if (((uintptr_t)k_pool & 15u) || ((uintptr_t)v_pool & 15u) || ((uintptr_t)sink & 3u))
        return PA_ERR_ALIGN;
    const int chunk = (num_tiles + pa::kTileWaves - 1) / pa::kTileWaves;
    const dim3 grid(pa::kTileWaves), block(pa::kWave);
    const hipStream_t s = (hipStream_t)stream;
    const char *kp = (const char *)k_pool, *vp = (const char *)v_pool;
    switch (tile_bytes) {
    case 1024: hipLaunchKernelGGL(pa::tile_read_kernel<1>, grid, block, 0, s, kp, vp, tiles, num_tiles, chunk, sink); break;
    case 2048: hipLaunchKernelGGL(pa::tile_read_kernel<2>, grid, block, 0, s, kp, vp, tiles, num_tiles, chunk, sink); break;
    case 4096: hipLaunchKernelGGL(pa::tile_read_kernel<4>, grid, block, 0, s, kp, vp, tiles, num_tiles, chunk, sink); break;
    default: hipLaunchKernelGGL(pa::tile_read_kernel<8>, grid, block, 0, s, kp, vp, tiles, num_tiles, chunk, sink); break;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" int pa_measure_stream_read(const void *buf, size_t bytes, int nontemporal,
                                      uint32_t *sink, void *stream) {
    if (!sink || (bytes > 0 && !buf)) return PA_ERR_NULL;
    if (((uintptr_t)buf & 15u) || (bytes & 15u) || ((uintptr_t)sink & 3u)) return PA_ERR_ALIGN;
    const dim3 grid(PA_MEASURE_SINK_WORDS), block(pa::kReadThreads);
    if (nontemporal)
        hipLaunchKernelGGL(pa::stream_read_kernel<2>, grid, block, 0, (hipStream_t)stream,
                           (const char *)buf, (int64_t)bytes, sink);
    else
        hipLaunchKernelGGL(pa::stream_read_kernel<0>, grid, block, 0, (hipStream_t)stream,
                           (const char *)buf, (int64_t)bytes, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
