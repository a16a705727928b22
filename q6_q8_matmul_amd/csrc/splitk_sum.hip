// splitk_sum.hip -- the fixed-order sum of a K-split product's partial
// results (cajeta "One model, start to last token" 3.1: a split along the
// reduction dimension, then a fixup pass that combines the pieces).
//
// y holds the sums of K range 0 of a window of `rows` x `cols` outputs (row
// stride ldy); part holds ranges 1..nparts of the same window as
// [nparts][rows][cols] f32.  Every output becomes ((y + part[0]) + part[1])
// + ...: the same order on every run, no atomics.
#include "kq_device.h"

#include <algorithm>

namespace kq {
namespace {

// One thread per float4 of a row (the scalar form when a row's window is not
// 16-byte aligned or its width not a multiple of 4).
__global__ __launch_bounds__(256) void splitk_sum_kernel(float* __restrict__ y, int64_t ldy,
                                                         const float* __restrict__ part,
                                                         int64_t rows, int64_t cols, int nparts,
                                                         bool vec) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t plane = rows * cols;
    if (vec) {
        const int64_t c4 = cols >> 2, n4 = rows * c4;
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
            const int64_t r = i / c4, c = 4 * (i - r * c4);
            float4* yp = (float4*)(y + r * ldy + c);
            float4 v = *yp;
            for (int z = 0; z < nparts; ++z) {
                const float4 q = *(const float4*)(part + z * plane + r * cols + c);
                v.x += q.x;
                v.y += q.y;
                v.z += q.z;
                v.w += q.w;
            }
            *yp = v;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < plane; i += stride) {
            const int64_t r = i / cols, c = i - r * cols;
            float v = y[r * ldy + c];
            for (int z = 0; z < nparts; ++z) v += part[z * plane + i];
            y[r * ldy + c] = v;
        }
    }
}

}  // namespace

hipError_t launch_splitk_sum(float* y, int64_t ldy, const float* part, int64_t rows, int64_t cols,
                             int nparts, hipStream_t stream) {
    if (rows <= 0 || cols <= 0 || nparts <= 0) return hipSuccess;
    const bool vec = ((uintptr_t)y & 15) == 0 && (ldy & 3) == 0 && (cols & 3) == 0 &&
                     ((uintptr_t)part & 15) == 0;
    const int64_t items = vec ? rows * (cols >> 2) : rows * cols;
    const int64_t blocks = std::min<int64_t>((items + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, ldy, part,
                       rows, cols, nparts, vec);
    return hipGetLastError();
}

}  // namespace kq
