// splitk_sum.hip -- the fixed-order sum of a K-split product's partial
// results (cajeta "One model, start to last token" 3.1: a split along the
// reduction dimension, then a fixup pass that combines the pieces).
//
// y holds the sums of K range 0; part holds ranges 1..nparts as
// [nparts][count] f32.  Every y[i] becomes ((y[i] + part[0][i]) + part[1][i])
// + ...: the same order on every run, no atomics.
#include "kq_device.h"

#include <algorithm>

namespace kq {
namespace {

// The float4 form when y is 16-byte aligned and count a multiple of 4.
__global__ __launch_bounds__(256) void splitk_sum_kernel(float* __restrict__ y,
                                                         const float* __restrict__ part,
                                                         int64_t count, int nparts) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    if (((uintptr_t)y & 15) == 0 && (count & 3) == 0) {
        float4* y4 = (float4*)y;
        const float4* p4 = (const float4*)part;
        const int64_t c4 = count >> 2;
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < c4; i += stride) {
            float4 v = y4[i];
            for (int z = 0; z < nparts; ++z) {
                const float4 q = p4[(int64_t)z * c4 + i];
                v.x += q.x;
                v.y += q.y;
                v.z += q.z;
                v.w += q.w;
            }
            y4[i] = v;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
            float v = y[i];
            for (int z = 0; z < nparts; ++z) v += part[(int64_t)z * count + i];
            y[i] = v;
        }
    }
}

}  // namespace

hipError_t launch_splitk_sum(float* y, const float* part, int64_t count, int nparts,
                             hipStream_t stream) {
    if (count <= 0 || nparts <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((count / 4 + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0,
                       stream, y, part, count, nparts);
    return hipGetLastError();
}

}  // namespace kq
