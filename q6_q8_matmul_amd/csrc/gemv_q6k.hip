// gemv_q6k.hip -- Q6_K x q8_1 matrix-vector product (output head, batch 1..4).
//
// Weight streaming bound like the Q4_K GEMV (minfer "The CUDA backend" 2.2).
// A Q6_K superblock is 210 bytes, so superblock starts are only 2-byte
// aligned; with byte loads the pages' first CUDA path was capped far below the
// memory bus (minfer "The CUDA backend" 3.2.2).  This kernel keeps the 210-byte
// layout and loads only whole aligned dwords: a lane that needs 8 bytes at a
// 2 (mod 4) address reads the three aligned dwords around them and funnel-
// shifts (v_alignbit_b32).  Every read stays inside the tensor: at most the
// two bytes before a superblock that starts at 2 (mod 4), which are the tail
// of the previous superblock.
//
// Work layout (as the Q4_K GEMV): 4 wavefronts x RPW rows per workgroup;
// 8 groups of 8 lanes take 8 consecutive superblocks of a row per pass.
// Lane (h, q) of a group, h = 0..1, q = 0..3, owns values
//   128h + 32g + 8q + i,   g = 0..3, i = 0..7,
// which come from ql[64h + 8q + i] (g = 0, 2: low / high nibble),
// ql[64h + 32 + 8q + i] (g = 1, 3) and qh[32h + 8q + i] (bits 2g, 2g+1), and
// use scale 8h + 2g + (q >= 2).  The lane forms 4*(q6 - 32) directly as an int8
// byte ((code XOR 32) << 2 is a sign-correct int8 because the code is 6 bits
// wide), so a v_dot4_i32_i8 chain over 8 values gives 4x the integer dot of
// the group; the factor 4 is folded back into d exactly.
//
// The activation is staged into LDS once per workgroup (int8 codes and the
// per-32-block d8), in chunks when it exceeds the LDS budget.  Per lane:
// sum_g float(A*sc)*d8 per superblock, times d/4, accumulated in a private f32
// register; then one fixed 64-lane xor-butterfly per row and column and the
// optional residual add on the row write (leone-cuda "CUDA kernel design":
// Q6_K GEMV with residual epilogue, fixed reduction order, no atomics).
#include "kq_device.h"

namespace kq {
namespace {

constexpr int kWaves = 4;

template <int BATCH>
__device__ __forceinline__ void stage_activation(const uint8_t* __restrict__ xq, int nb_row,
                                                 int j0, int nbc, int cap, int8_t* codes,
                                                 float* d8s) {
    for (int idx = threadIdx.x; idx < BATCH * nbc; idx += blockDim.x) {
        const int bb = idx / nbc;
        const int j = idx - bb * nbc;
        const uint32_t* blk =
            (const uint32_t*)(xq + ((int64_t)bb * nb_row + j0 + j) * kQ81Bytes);
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = blk[1 + i];
        uint4* dst = (uint4*)(codes + (bb * cap + j) * 32);
        dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
        dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
        d8s[bb * cap + j] = half_bits_to_float(blk[0]);
    }
}

// Eight bytes starting at byte offset `off` of a superblock that starts at
// `sb` (2-byte aligned, sb_par = sb & 3 in {0, 2}).  Reads the three aligned
// dwords [off - par, off - par + 12); for the offsets used here that range
// ends before byte 197 of the superblock and starts at most 2 bytes before it.
__device__ __forceinline__ uint2 load8_u(const uint8_t* sb, int sb_par, int off) {
    const uint32_t* p = (const uint32_t*)(sb + off - sb_par);
    const uint32_t a = p[0], b = p[1], c = p[2];
    const uint32_t sh = (uint32_t)sb_par * 8u;
    return make_uint2(__builtin_amdgcn_alignbit(b, a, sh), __builtin_amdgcn_alignbit(c, b, sh));
}

template <int BATCH, int RPW>
__global__ __launch_bounds__(256) void gemv_q6k_kernel(const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ xq,
                                                       float* y, const float* residual,
                                                       int m, int S, int schunk) {
    extern __shared__ __align__(16) uint8_t smem[];
    int8_t* codes = (int8_t*)smem;                             // [BATCH][schunk*256]
    float* d8s = (float*)(smem + BATCH * schunk * kQK);         // [BATCH][schunk*8]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 3;
    const int k8 = lane & 7;
    const int h = k8 >> 2;          // 128-value half of the superblock
    const int q = k8 & 3;           // 8-value slice within each 32-value group
    const int row0 = (blockIdx.x * kWaves + wave) * RPW;
    const int64_t row_bytes = (int64_t)S * kQ6KBytes;
    const int nb_row = S * 8;

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    for (int kc = 0; kc < S; kc += schunk) {
        const int nsb = min(schunk, S - kc);
        if (kc > 0) __syncthreads();
        stage_activation<BATCH>(xq, nb_row, kc * 8, nsb * 8, schunk * 8, codes, d8s);
        __syncthreads();

        for (int sl = grp; sl < nsb; sl += 8) {
            const int sbi = kc + sl;
            uint2 L[RPW], L2[RPW], H[RPW], SC[RPW];
            uint32_t DH[RPW];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int r = min(row0 + i, m - 1);
                const int64_t off = (int64_t)r * row_bytes + (int64_t)sbi * kQ6KBytes;
                const uint8_t* sb = w + off;
                const int par = (int)(off & 3);
                L[i] = load8_u(sb, par, 64 * h + 8 * q);
                L2[i] = load8_u(sb, par, 64 * h + 32 + 8 * q);
                H[i] = load8_u(sb, par, 128 + 32 * h + 8 * q);
                // the 8 scale bytes of this half: [192 + 8h, 200 + 8h)
                const uint32_t* ps = (const uint32_t*)(sb + 192 + 8 * h - par);
                const uint32_t s0 = ps[0], s1 = ps[1];
                const uint32_t s2 = par ? ps[2] : 0u;  // only when the bytes straddle
                SC[i] = make_uint2(__builtin_amdgcn_alignbit(s1, s0, (uint32_t)par * 8u),
                                   __builtin_amdgcn_alignbit(s2, s1, (uint32_t)par * 8u));
                DH[i] = *(const uint16_t*)(sb + 208);
            }
            const int cbase = sl * 256 + 128 * h + 8 * q;
            const int jl = sl * 8 + 4 * h;
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const float dq = half_bits_to_float(DH[i]) * 0.25f;
                // scale of group g: byte 2g + (q >> 1) of the half's 8 scale bytes
                const uint64_t s64 = (uint64_t)SC[i].x | ((uint64_t)SC[i].y << 32);
                int sc[4];
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    sc[g] = (int)(int8_t)(uint8_t)(s64 >> (8 * (2 * g + (q >> 1))));
                uint32_t v[4][2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint32_t l = t ? L[i].y : L[i].x;
                    const uint32_t l2 = t ? L2[i].y : L2[i].x;
                    const uint32_t hb = t ? H[i].y : H[i].x;
                    v[0][t] = (((l << 2) & 0x3c3c3c3cu) | ((hb << 6) & 0xc0c0c0c0u)) ^ 0x80808080u;
                    v[1][t] = (((l2 << 2) & 0x3c3c3c3cu) | ((hb << 4) & 0xc0c0c0c0u)) ^ 0x80808080u;
                    v[2][t] = (((l >> 2) & 0x3c3c3c3cu) | ((hb << 2) & 0xc0c0c0c0u)) ^ 0x80808080u;
                    v[3][t] = (((l2 >> 2) & 0x3c3c3c3cu) | (hb & 0xc0c0c0c0u)) ^ 0x80808080u;
                }
#pragma unroll
                for (int b = 0; b < BATCH; ++b) {
                    const int8_t* cb = codes + b * (schunk * kQK) + cbase;
                    const float* db = d8s + b * (schunk * 8) + jl;
                    float t = 0.0f;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint2 a = *(const uint2*)(cb + 32 * g);
                        const int A4 = dot4(v[g][1], a.y, dot4(v[g][0], a.x, 0));
                        t += (float)__mul24(A4, sc[g]) * db[g];
                    }
                    acc[i][b] += dq * t;
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
    const int per_sb = BATCH * (kQK + 8 * (int)sizeof(float));
    const int budget = lds_limit < 65536 ? lds_limit : 65536;
    int schunk = budget / per_sb;
    if (schunk > S) schunk = S;
    if (schunk < 1) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)schunk * per_sb;
    const int rows_per_block = kWaves * RPW;
    const int64_t grid = (m + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_q6k_kernel<BATCH, RPW>), dim3((unsigned)grid), dim3(64 * kWaves), lds,
                       stream, (const uint8_t*)w, (const uint8_t*)xq, y, residual, (int)m, S, schunk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_q6k(const void* w, const void* xq, float* y, const float* residual,
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
