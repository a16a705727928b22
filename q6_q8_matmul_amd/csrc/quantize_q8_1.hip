// quantize_q8_1.hip -- f32 activations -> q8_1 blocks on gfx950.
//
// One q8_1 block = 32 values -> {f16 d, f16 s, int8 code[32]} (leone-cuda
// "CUDA kernel design": q8_1 blocks of 32 signed codes, an f16 scale and an
// f16 source sum, produced by a separate kernel once per GEMV input).
//
// Mapping: eight lanes per block, each lane owns four consecutive values
// (one 16-byte load).  A wavefront therefore reads 1 KiB and writes 288
// contiguous bytes (8 blocks).  The max and the source-sum tree run over the
// eight lanes with xor shuffles; the tree adds a[i] + a[i+h] for
// h = 16, 8, 4, 2, 1 exactly as its definition states, so the sum is the
// same f32 value bit for bit (IEEE addition is commutative).
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

    float4 v = x[blk * 8 + j];

    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 4, 8));
    a = fmaxf(a, __shfl_xor(a, 2, 8));
    a = fmaxf(a, __shfl_xor(a, 1, 8));

    const float d = a / 127.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;

    auto code = [&](float t) -> uint32_t {
        float q = roundf(t * id);
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        return (uint32_t)((int)q) & 0xffu;
    };
    const uint32_t packed = code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);

    // Source-sum tree.  Lane L holds a[4L..4L+3]; h = 16, 8, 4 pair lanes
    // L and L^4, L^2, L^1; h = 2, 1 finish inside lane 0.
    float4 o;
    o.x = __shfl_xor(v.x, 4, 8); o.y = __shfl_xor(v.y, 4, 8);
    o.z = __shfl_xor(v.z, 4, 8); o.w = __shfl_xor(v.w, 4, 8);
    v.x = v.x + o.x; v.y = v.y + o.y; v.z = v.z + o.z; v.w = v.w + o.w;
    o.x = __shfl_xor(v.x, 2, 8); o.y = __shfl_xor(v.y, 2, 8);
    o.z = __shfl_xor(v.z, 2, 8); o.w = __shfl_xor(v.w, 2, 8);
    v.x = v.x + o.x; v.y = v.y + o.y; v.z = v.z + o.z; v.w = v.w + o.w;
    o.x = __shfl_xor(v.x, 1, 8); o.y = __shfl_xor(v.y, 1, 8);
    o.z = __shfl_xor(v.z, 1, 8); o.w = __shfl_xor(v.w, 1, 8);
    v.x = v.x + o.x; v.y = v.y + o.y; v.z = v.z + o.z; v.w = v.w + o.w;
    const float s = (v.x + v.z) + (v.y + v.w);

    uint32_t* out = xq + blk * 9;
    out[1 + j] = packed;
    if (j == 0) out[0] = float_to_half_bits(d) | (float_to_half_bits(s) << 16);
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
