// producers.hip -- RMSNorm and SwiGLU kernels that write q8_1 blocks
// themselves, so the GEMV after them needs no separate quantisation launch
// (leone-cuda "CUDA kernel design": RMSNorm and SwiGLU write their dense
// output and their q8_1 blocks; the backend keeps the q8_1 activation for the
// next GEMV; minfer "The CUDA backend" 2.2: fused producers removed most
// standalone decode quantise launches).
//
// Work split: the values of a row are written in 256-value segments (eight
// q8_1 blocks) by 64-lane wavefronts, lane t owning values 4t .. 4t+3 of the
// segment (16-byte loads); the eight lanes of each aligned group quantise one
// block with the library's q8_1 block routine.
//
// RMSNorm (n % 256 == 0).  One 256-thread workgroup per segment for few rows
// (each repeats the same fixed reduction over the whole row and writes a
// disjoint segment, as the pages describe), one per row for many rows.  The
// order: reduction lane l = 0..255 accumulates fmaf(h_i, h_i, acc) over
// i = l, l+256, ...; then a pairwise tree a[l] += a[l+h], h = 128, 64, ..., 1.
// Then r = 1 / sqrtf(ss/n + eps) (IEEE division and square root, no
// approximate reciprocal root) and y = (h * r) * g, with h = x + res
// recomputed when a residual is given.
//
// SwiGLU.  y = (t / (1 + e(-t))) * u, with e(a) evaluated by Cody and
// Waite's reduction by ln 2 (C1 = 0.693359375 exact in 9 bits, C2 = ln 2 - C1
// rounded to f32; k = rint(a log2 e)) and the degree-7 Taylor polynomial of
// exp at 0 in Horner form with fused multiply-adds, then ldexp; +inf above
// a = 100, +0 below -110.  Every step is one IEEE operation, so the values are
// reproducible bit for bit on any IEEE implementation of the same steps.
#include "kq_device.h"

namespace kq {
namespace {

__device__ __forceinline__ float exp_f32(float a) {
    if (a > 100.0f) return __builtin_inff();
    if (a < -110.0f) return 0.0f;
    const float k = __builtin_rintf(a * 1.44269504088896341f);
    float r = __builtin_fmaf(-k, 0.693359375f, a);
    r = __builtin_fmaf(-k, -2.12194440054690583e-4f, r);
    float p = 1.0f / 5040.0f;
    p = __builtin_fmaf(p, r, 1.0f / 720.0f);
    p = __builtin_fmaf(p, r, 1.0f / 120.0f);
    p = __builtin_fmaf(p, r, 1.0f / 24.0f);
    p = __builtin_fmaf(p, r, 1.0f / 6.0f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)k);
}

__device__ __forceinline__ float silu_f32(float t) { return t / (1.0f + exp_f32(-t)); }

__device__ __forceinline__ float4 load4(const float* p) { return *(const float4*)p; }

// RMSNorm, one 256-thread workgroup: thread l is reduction lane l (its fma
// chain over i = l, l+256, ... with the loads of several steps in flight);
// tree levels h = 128 and 64 through LDS, h = 32 ... 1 by shuffles in
// wavefront 0.  PER_SEGMENT: workgroup row*segs + seg writes segment seg of
// the row (wavefront 0; every workgroup of the row repeats the same
// reduction, whose row reads hit L2).  Otherwise workgroup `row` writes all
// segments of its row, wavefront w taking segments w, w+4, ...  STASH (one
// workgroup per row, the row in dynamic LDS): the reduction pass keeps each
// h = x (+ res) it forms, and the second pass reads them from LDS instead of
// reading the row from memory again; the values and their order are the
// same, so the outputs are too.
template <bool PER_SEGMENT, bool STASH>
__global__ __launch_bounds__(256) void rmsnorm_q8_1_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ res,
                                                           const float* __restrict__ g, float eps,
                                                           float* __restrict__ y,
                                                           uint32_t* __restrict__ xq, int n,
                                                           int segs) {
    __shared__ float part[256];
    extern __shared__ float hbuf[];   // STASH: the row's n values of h
    const int l = threadIdx.x;
    const int lane = l & 63, wave = l >> 6;
    const int64_t row = PER_SEGMENT ? blockIdx.x / segs : blockIdx.x;
    const float* xr = x + row * n;
    const float* rr = res ? res + row * n : nullptr;

    // PER_SEGMENT: wavefront 0 fetches its segment before the reduction
    int seg = PER_SEGMENT ? (int)(blockIdx.x - row * segs) : wave;
    float4 h0 = {}, q0 = {}, g0 = {};
    if (PER_SEGMENT && wave == 0) {
        const int i = seg * 256 + 4 * lane;
        h0 = load4(xr + i);
        if (rr) q0 = load4(rr + i);
        g0 = load4(g + i);
    }

    float acc = 0.0f;
#pragma unroll 16
    for (int i = l; i < n; i += 256) {
        const float h = rr ? xr[i] + rr[i] : xr[i];
        if (STASH) hbuf[i] = h;
        acc = __builtin_fmaf(h, h, acc);
    }
    part[l] = acc;
    __syncthreads();
    if (l < 128) part[l] = part[l] + part[l + 128];
    __syncthreads();
    if (l < 64) {
        float s = part[l] + part[l + 64];
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) s = s + __shfl_xor(s, h, 64);
        if (l == 0) part[0] = s;
    }
    __syncthreads();
    const float ss = part[0];
    const float r = 1.0f / sqrtf(ss / (float)n + eps);

    if (PER_SEGMENT && wave != 0) return;
    for (; seg < segs; seg += PER_SEGMENT ? segs : 4) {
        const int i = seg * 256 + 4 * lane;
        float4 h = PER_SEGMENT ? h0 : STASH ? *(const float4*)(hbuf + i) : load4(xr + i);
        if (rr && !STASH) {
            const float4 q = PER_SEGMENT ? q0 : load4(rr + i);
            h.x = h.x + q.x; h.y = h.y + q.y; h.z = h.z + q.z; h.w = h.w + q.w;
        }
        const float4 gg = PER_SEGMENT ? g0 : load4(g + i);
        float4 v;
        v.x = (h.x * r) * gg.x;
        v.y = (h.y * r) * gg.y;
        v.z = (h.z * r) * gg.z;
        v.w = (h.w * r) * gg.w;
        if (y) *(float4*)(y + row * n + i) = v;
        quantize_block8(v, lane & 7, xq + (row * (n / 32) + seg * 8 + (lane >> 3)) * 9);
    }
}

__global__ __launch_bounds__(64) void swiglu_q8_1_kernel(const float* __restrict__ gate,
                                                         const float* __restrict__ up,
                                                         float* __restrict__ y,
                                                         uint32_t* __restrict__ xq) {
    const int64_t i = (int64_t)blockIdx.x * 256 + 4 * threadIdx.x;
    const float4 a = load4(gate + i), u = load4(up + i);
    float4 v;
    v.x = silu_f32(a.x) * u.x;
    v.y = silu_f32(a.y) * u.y;
    v.z = silu_f32(a.z) * u.z;
    v.w = silu_f32(a.w) * u.w;
    if (y) *(float4*)(y + i) = v;
    quantize_block8(v, threadIdx.x & 7, xq + (i >> 5) * 9);
}

}  // namespace

hipError_t launch_rmsnorm_q8_1(const float* x, const float* res, const float* g, float eps,
                               float* y, void* xq, int64_t rows, int64_t n, hipStream_t stream) {
    const int segs = (int)(n / 256);
    // Few rows: one workgroup per segment keeps every q8_1 block of a decode
    // row in flight at once (the repeated row reads hit L2).  Many rows: one
    // workgroup per row reduces once; it keeps the row in LDS between its two
    // passes when the row fits 64 KB beside the 1 KB reduction buffer, and
    // reads it again otherwise.
    if (rows * segs <= 4096 || rows < 64)
        hipLaunchKernelGGL((rmsnorm_q8_1_kernel<true, false>), dim3((unsigned)(rows * segs)), dim3(256),
                           0, stream, x, res, g, eps, y, (uint32_t*)xq, (int)n, segs);
    else if (n * 4 + 1024 <= 65536)
        hipLaunchKernelGGL((rmsnorm_q8_1_kernel<false, true>), dim3((unsigned)rows), dim3(256),
                           (size_t)n * 4, stream, x, res, g, eps, y, (uint32_t*)xq, (int)n, segs);
    else
        hipLaunchKernelGGL((rmsnorm_q8_1_kernel<false, false>), dim3((unsigned)rows), dim3(256), 0,
                           stream, x, res, g, eps, y, (uint32_t*)xq, (int)n, segs);
    return hipGetLastError();
}

hipError_t launch_swiglu_q8_1(const float* gate, const float* up, float* y, void* xq,
                              int64_t rows, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(swiglu_q8_1_kernel, dim3((unsigned)(rows * (n / 256))), dim3(64), 0, stream,
                       gate, up, y, (uint32_t*)xq);
    return hipGetLastError();
}

}  // namespace kq
