// read_probe.hip -- the device's streaming-read rate, for the benchmark.
//
// Not part of the k-quant path: the decode GEMVs are weight-streaming bound
// (minfer "The CUDA backend" 2.2), so their rate is reported beside what a
// plain read of the same bytes reaches on the same device.  One workgroup per
// 32 KiB chunk; thread t loads the 16-byte words base + 256u + t, u = 0..7,
// all eight issued before any is used; every wavefront xor-folds its lanes'
// words and lane 0 stores the result, so no load can be dropped and the
// written bytes are 1/2048 of the read ones.
#include "kq_device.h"

namespace kq {
namespace {

constexpr int kProbeWords = 8;   // 16-byte words per thread

__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * (256 * kProbeWords) + threadIdx.x;
    uint4 v[kProbeWords];
#pragma unroll
    for (int u = 0; u < kProbeWords; ++u) {
        const int64_t j = base + 256 * u;
        v[u] = j < n16 ? load16(p + 16 * j) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kProbeWords; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

int64_t read_probe_words(int64_t nbytes) {
    return (nbytes / 16 + 256 * kProbeWords - 1) / (256 * kProbeWords) * 4;
}

hipError_t launch_read_probe(const void* p, int64_t nbytes, uint32_t* out, hipStream_t stream) {
    const int64_t n16 = nbytes / 16;
    const int64_t grid = (n16 + 256 * kProbeWords - 1) / (256 * kProbeWords);
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t*)p, n16, out);
    return hipGetLastError();
}

}  // namespace kq
