// repack_q6k.hip -- raw Q6_K rows -> the split Q6_K layout, once at load.
//
// cajeta "One model, start to last token" 2 (residency): a Q6_K weight is
// split into a scale prefix and 208-byte bodies, so the kernels read it with
// aligned 16-byte loads.  Layout (g = row * S + s, S = k / 256):
//   bytes [2g, 2g+2)                 f16 d of superblock g
//   bytes [2G, P)                    zero, P = 2G rounded up to 16 (G = m*S)
//   bytes [P + 208g, P + 208g + 208) ql, qh and the 16 int8 scales of g
// The raw superblocks are 210 bytes, so every other one starts at 2 mod 4:
// one thread per (superblock, 16-byte chunk of bytes 0..207) reads with
// 4-byte-aligned loads and realigns by a 16-bit funnel shift (reading at most
// the two bytes before an odd superblock, never past the tensor); the chunk
// index 13 moves d.
#include "kq_device.h"

namespace kq {
namespace {

__global__ __launch_bounds__(256) void repack_q6k_kernel(const uint8_t* __restrict__ w,
                                                         uint8_t* __restrict__ wr, int64_t G,
                                                         int64_t prefix) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t g = t / 14;
    const int ch = (int)(t - g * 14);
    if (g >= G) return;
    const uint8_t* p = w + g * kQ6KBytes;
    if (ch == 13) {
        *(uint16_t*)(wr + 2 * g) = *(const uint16_t*)(p + 208);
        if (g == G - 1)   // the padding after the last d
            for (int64_t b = 2 * G; b < prefix; ++b) wr[b] = 0;
        return;
    }
    const int phase = (int)(g & 1) * 2;   // w is 16-byte aligned, 210 = 2 mod 4
    const uint8_t* base = p - phase + 16 * ch;
    const uint4 cur = load16(base);
    const uint32_t nxt = *(const uint32_t*)(base + (phase ? 16 : 12));
    uint4 v = cur;
    if (phase) {
        v.x = (cur.x >> 16) | (cur.y << 16);
        v.y = (cur.y >> 16) | (cur.z << 16);
        v.z = (cur.z >> 16) | (cur.w << 16);
        v.w = (cur.w >> 16) | (nxt << 16);
    }
    *(uint4*)(wr + prefix + g * 208 + 16 * ch) = v;
}

}  // namespace

hipError_t launch_repack_q6k(const void* w, void* wr, int64_t m, int64_t k, hipStream_t stream) {
    const int64_t G = m * (k / kQK);
    const int64_t prefix = (2 * G + 15) / 16 * 16;
    const int64_t threads = G * 14;
    hipLaunchKernelGGL(repack_q6k_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, (const uint8_t*)w, (uint8_t*)wr, G, prefix);
    return hipGetLastError();
}

}  // namespace kq
