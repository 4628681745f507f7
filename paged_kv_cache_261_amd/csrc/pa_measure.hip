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

}  // namespace pa

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
