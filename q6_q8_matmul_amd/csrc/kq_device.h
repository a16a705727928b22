// kq_device.h -- device helpers and internal launcher declarations of libkq.
//
// Shared by the gfx950 kernels of this library only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// Byte sizes of the block formats.
constexpr int kQK = 256;        // values per superblock
constexpr int kQ4KBytes = 144;  // Q4_K superblock
constexpr int kQ6KBytes = 210;  // Q6_K superblock
constexpr int kQ81Bytes = 36;   // q8_1 block (32 values)

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Plain 16-byte load (global_load_dwordx4).
__device__ __forceinline__ uint4 load16(const void* p) {
    const u32x4_t v = *(const u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Sum over the 64 lanes of a wavefront with a fixed xor-butterfly order;
// every lane receives the same total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Launchers (return the launch status).
hipError_t launch_quantize_q8_1(const float* x, void* xq, int64_t rows, int64_t k,
                                hipStream_t stream);
hipError_t launch_gemv_q4k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream);
hipError_t launch_gemv_q6k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream);
hipError_t launch_mmq_q4k(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                          int64_t k, hipStream_t stream);

}  // namespace kq
