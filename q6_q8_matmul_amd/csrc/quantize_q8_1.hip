// quantize_q8_1.hip -- f32 activations -> q8_1 blocks on gfx950.
//
// One q8_1 block = 32 values -> {f16 d, f16 s, int8 code[32]} (leone-cuda
// "CUDA kernel design": q8_1 blocks of 32 signed codes, an f16 scale and an
// f16 source sum, produced by a separate kernel once per GEMV input).
//
// Mapping: eight lanes per block, each lane owns four consecutive values
// (one 16-byte load).  A wavefront therefore reads 1 KiB and writes 288
// contiguous bytes (8 blocks).  The block routine (quantize_block8) runs the
// max and the source-sum tree over the eight lanes with xor shuffles.
#include "kq_device.h"

namespace kq {
namespace {

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float4* __restrict__ x,
                                                            uint32_t* __restrict__ xq,
                                                            int64_t nblocks) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int j = threadIdx.x & 7;
    if (blk >= nblocks) return;  // whole 8-lane groups leave together

    quantize_block8(x[blk * 8 + j], j, xq + blk * 9);
}

}  // namespace

hipError_t launch_quantize_q8_1(const float* x, void* xq, int64_t rows, int64_t k,
                                hipStream_t stream) {
    const int64_t nblocks = rows * (k / 32);
    const int64_t threads = nblocks * 8;
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const float4*)x, (uint32_t*)xq, nblocks);
    return hipGetLastError();
}

}  // namespace kq
