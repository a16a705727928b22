// gemv_q4k.hip -- Q4_K x q8_1 matrix-vector product (decode, batch 1..4).
//
// The decode matmul reads every weight byte once, so the kernel is bound by
// HBM bandwidth (minfer "The CUDA backend" 2.2: decode is weight-streaming
// bound; cajeta "One model, start to last token" 4: bytes per second against
// the memory bus is a decode kernel's only figure of merit).
//
// Layout of the work:
//   * a workgroup of 4 wavefronts owns 4*RPW consecutive output rows, each
//     wavefront RPW rows that it streams concurrently;
//   * inside a wavefront, 8 groups of 8 lanes take 8 consecutive superblocks
//     of a row per pass, so one pass is a contiguous 1152-byte read;
//     lane k of a group loads the 16-byte slice k of the 128 code bytes
//     (both nibbles: 16 values of sub-block 2c and 16 of sub-block 2c+1,
//     c = k/2) plus the 16-byte superblock header (d, dmin, packed scales);
//   * the q8_1 activation is restaged once per workgroup into LDS as plain
//     int8 codes plus, per (32-block, 16-value half), the pair
//     {d8, d8 * sum of the half's codes}; chunks of superblocks are staged in
//     turn when the whole row does not fit the LDS budget;
//   * integer dots with v_dot4_i32_i8 (4-bit codes are non-negative bytes),
//     then per lane: d*(sc*A*d8) - dmin*(m*d8*Bq), accumulated in a private
//     f32 register over the whole row; the minimum term uses the q8 codes
//     (leone-cuda "CUDA kernel design": minimum correction formed from the
//     same lane-local codes);
//   * one fixed xor-butterfly over the 64 lanes per row and batch column,
//     then the optional residual is added when the row is written
//     (leone-cuda "CUDA kernel design": residual epilogue, same f32 addition
//     as the separate add it replaces).
// No atomics; the reduction order is fixed, so results are bitwise
// reproducible.
#include "kq_device.h"

namespace kq {
namespace {

constexpr int kWaves = 4;

struct HalfScale {  // per (q8_1 block, 16-value half)
    float d8;
    float d8_bq;    // d8 * (sum of the half's 16 codes), exact in f32
};

template <int BATCH>
__device__ __forceinline__ void stage_activation(const uint8_t* __restrict__ xq, int nb_row,
                                                 int j0, int nbc, int cap, int8_t* codes,
                                                 HalfScale* hs) {
    // blocks [j0, j0 + nbc) of every batch column; column stride = cap blocks
    for (int idx = threadIdx.x; idx < BATCH * nbc; idx += blockDim.x) {
        const int bb = idx / nbc;
        const int j = idx - bb * nbc;
        const uint32_t* blk =
            (const uint32_t*)(xq + ((int64_t)bb * nb_row + j0 + j) * kQ81Bytes);
        const uint32_t hdr = blk[0];
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = blk[1 + i];
        const float d8 = half_bits_to_float(hdr);
        int s0 = dot4(c[0], 0x01010101u, dot4(c[1], 0x01010101u, 0));
        s0 = dot4(c[2], 0x01010101u, dot4(c[3], 0x01010101u, s0));
        int s1 = dot4(c[4], 0x01010101u, dot4(c[5], 0x01010101u, 0));
        s1 = dot4(c[6], 0x01010101u, dot4(c[7], 0x01010101u, s1));
        uint4* dst = (uint4*)(codes + (bb * cap + j) * 32);
        dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
        dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
        HalfScale* h = hs + (bb * cap + j) * 2;
        h[0] = HalfScale{d8, d8 * (float)s0};
        h[1] = HalfScale{d8, d8 * (float)s1};
    }
}

template <int BATCH, int RPW>
__global__ __launch_bounds__(256) void gemv_q4k_kernel(const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ xq,
                                                       float* y, const float* residual,
                                                       int m, int S, int schunk) {
    extern __shared__ __align__(16) uint8_t smem[];
    int8_t* codes = (int8_t*)smem;                                  // [BATCH][schunk*256]
    HalfScale* hs = (HalfScale*)(smem + BATCH * schunk * kQK);       // [BATCH][schunk*8][2]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 3;      // superblock within a pass
    const int k8 = lane & 7;        // 16-byte code slice within the superblock
    const int c = k8 >> 1;          // 64-value chunk: sub-blocks 2c (low nibbles), 2c+1 (high)
    const int hh = k8 & 1;          // which 16 values of each sub-block
    const int row0 = (blockIdx.x * kWaves + wave) * RPW;
    const int64_t row_bytes = (int64_t)S * kQ4KBytes;
    const int nb_row = S * 8;

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    for (int kc = 0; kc < S; kc += schunk) {
        const int nsb = min(schunk, S - kc);
        if (kc > 0) __syncthreads();
        stage_activation<BATCH>(xq, nb_row, kc * 8, nsb * 8, schunk * 8, codes, hs);
        __syncthreads();

        for (int sl = grp; sl < nsb; sl += 8) {
            const int sb = kc + sl;
            uint4 hdr[RPW], qs[RPW];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int r = min(row0 + i, m - 1);  // clamped rows are computed, not stored
                const uint8_t* p = w + (int64_t)r * row_bytes + (int64_t)sb * kQ4KBytes;
                hdr[i] = *(const uint4*)p;
                qs[i] = *(const uint4*)(p + 16 + 16 * k8);
            }
            const int cbase = sl * 256 + 64 * c + 16 * hh;  // within the staged chunk
            const int jl = sl * 8 + 2 * c;                  // local 32-block index of sub-block 2c
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const float d = half_bits_to_float(hdr[i].x);
                const float dmin = half_bits_to_float(hdr[i].x >> 16);
                const uint32_t h1 = hdr[i].y, h2 = hdr[i].z, h3 = hdr[i].w;
                // six-bit scales/mins of sub-blocks 2c and 2c+1
                uint32_t S4, M4;
                if (c < 2) {
                    S4 = h1 & 0x3f3f3f3fu;
                    M4 = h2 & 0x3f3f3f3fu;
                } else {
                    S4 = (h3 & 0x0f0f0f0fu) | ((h1 >> 2) & 0x30303030u);
                    M4 = ((h3 >> 4) & 0x0f0f0f0fu) | ((h2 >> 2) & 0x30303030u);
                }
                const int sh = (c & 1) * 16;
                const int sc_a = (S4 >> sh) & 0xff, sc_b = (S4 >> (sh + 8)) & 0xff;
                const float m_a = (float)((M4 >> sh) & 0xff), m_b = (float)((M4 >> (sh + 8)) & 0xff);
                const uint32_t lo0 = qs[i].x & 0x0f0f0f0fu, lo1 = qs[i].y & 0x0f0f0f0fu;
                const uint32_t lo2 = qs[i].z & 0x0f0f0f0fu, lo3 = qs[i].w & 0x0f0f0f0fu;
                const uint32_t hi0 = (qs[i].x >> 4) & 0x0f0f0f0fu, hi1 = (qs[i].y >> 4) & 0x0f0f0f0fu;
                const uint32_t hi2 = (qs[i].z >> 4) & 0x0f0f0f0fu, hi3 = (qs[i].w >> 4) & 0x0f0f0f0fu;
#pragma unroll
                for (int b = 0; b < BATCH; ++b) {
                    const int8_t* cb = codes + b * (schunk * kQK) + cbase;
                    const uint4 alo = *(const uint4*)cb;
                    const uint4 ahi = *(const uint4*)(cb + 32);
                    int A_lo = dot4(lo0, alo.x, 0);
                    A_lo = dot4(lo1, alo.y, A_lo);
                    A_lo = dot4(lo2, alo.z, A_lo);
                    A_lo = dot4(lo3, alo.w, A_lo);
                    int A_hi = dot4(hi0, ahi.x, 0);
                    A_hi = dot4(hi1, ahi.y, A_hi);
                    A_hi = dot4(hi2, ahi.z, A_hi);
                    A_hi = dot4(hi3, ahi.w, A_hi);
                    const HalfScale sa = hs[(b * schunk * 8 + jl) * 2 + hh];
                    const HalfScale sb2 = hs[(b * schunk * 8 + jl + 1) * 2 + hh];
                    const float fa = (float)(A_lo * sc_a) * sa.d8 + (float)(A_hi * sc_b) * sb2.d8;
                    const float fm = m_a * sa.d8_bq + m_b * sb2.d8_bq;
                    acc[i][b] += d * fa - dmin * fm;
                }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = row0 + i;
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const float t = wave_sum(acc[i][b]);
            if (lane == 0 && r < m) {
                const int64_t o = (int64_t)b * m + r;
                y[o] = residual ? residual[o] + t : t;
            }
        }
    }
}

template <int BATCH>
hipError_t launch_batch(const void* w, const void* xq, float* y, const float* residual,
                        int64_t m, int64_t k, int lds_limit, hipStream_t stream) {
    constexpr int RPW = 2;
    const int S = (int)(k / kQK);
    // LDS per staged superblock and column: 256 code bytes + 8 blocks * 2 halves * 8 bytes
    const int per_sb = BATCH * (kQK + 8 * 2 * (int)sizeof(HalfScale));
    const int budget = lds_limit < 65536 ? lds_limit : 65536;
    int schunk = budget / per_sb;
    if (schunk > S) schunk = S;
    if (schunk < 1) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)schunk * per_sb;
    const int rows_per_block = kWaves * RPW;
    const int64_t grid = (m + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_q4k_kernel<BATCH, RPW>), dim3((unsigned)grid), dim3(64 * kWaves), lds,
                       stream, (const uint8_t*)w, (const uint8_t*)xq, y, residual, (int)m, S, schunk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_q4k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, hipStream_t stream) {
    switch (batch) {
        case 1: return launch_batch<1>(w, xq, y, residual, m, k, lds_limit, stream);
        case 2: return launch_batch<2>(w, xq, y, residual, m, k, lds_limit, stream);
        case 3: return launch_batch<3>(w, xq, y, residual, m, k, lds_limit, stream);
        case 4: return launch_batch<4>(w, xq, y, residual, m, k, lds_limit, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kq
