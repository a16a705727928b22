// read_probe.hip -- the device's streaming-read rate, for the benchmark.
//
// Not part of the k-quant path: the decode GEMVs are weight-streaming bound
// (minfer "The CUDA backend" 2.2), so their rate is reported beside what a
// plain read of the same bytes reaches on the same device.  The buffer is
// cut into chunks of 256*U 16-byte words; thread t of a 256-thread workgroup
// loads the words 256u + t of its chunk, u = 0..U-1, all U issued before any
// is used.  Workgroup b takes chunks b, b + G, b + 2G, ... of a grid of G
// workgroups: G = the chunk count is the one-shot form, a few workgroups per
// CU the persistent form.  Every wavefront xor-folds its lanes' words and
// lane 0 stores the result, so no load can be dropped.
#include "kq_device.h"

namespace kq {
namespace {

template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ p, int64_t n16,
                                                         int64_t nchunks, uint32_t* __restrict__ out) {
    uint32_t acc = 0;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t base = c * (256 * U) + threadIdx.x;
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + 256 * u;
            v[u] = j < n16 ? load16(p + 16 * j) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

int64_t probe_grid(int64_t nbytes, int64_t grid, int loads) {
    const int64_t nchunks = (nbytes / 16 + 256 * loads - 1) / (256 * loads);
    return grid == 0 ? nchunks : (grid < nchunks ? grid : nchunks);
}

}  // namespace

int64_t read_probe_words(int64_t nbytes, int64_t grid, int loads) {
    return 4 * probe_grid(nbytes, grid, loads);
}

hipError_t launch_read_probe(const void* p, int64_t nbytes, uint32_t* out, int64_t grid, int loads,
                             hipStream_t stream) {
    const int64_t n16 = nbytes / 16;
    const int64_t nchunks = (n16 + 256 * loads - 1) / (256 * loads);
    const int64_t g = probe_grid(nbytes, grid, loads);
    const dim3 gd((unsigned)g), bd(256);
    const uint8_t* b = (const uint8_t*)p;
    switch (loads) {
        case 4: hipLaunchKernelGGL(read_probe_kernel<4>, gd, bd, 0, stream, b, n16, nchunks, out); break;
        case 8: hipLaunchKernelGGL(read_probe_kernel<8>, gd, bd, 0, stream, b, n16, nchunks, out); break;
        case 16: hipLaunchKernelGGL(read_probe_kernel<16>, gd, bd, 0, stream, b, n16, nchunks, out); break;
        case 32: hipLaunchKernelGGL(read_probe_kernel<32>, gd, bd, 0, stream, b, n16, nchunks, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kq
