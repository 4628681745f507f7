// pa_vector_chunk.h -- 16-byte chunks of a K/V row for the vector-ALU
// kernels (decode and prefill): unpacking to float and packing back, for
// float32 and bfloat16 storage.
#pragma once

#include "pa_internal.h"

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
}  // namespace pa
