// mmq_q4k.hip -- Q4_K x q8_1 matrix-matrix product on the int8 matrix cores.
//
// minfer "The CUDA backend" 2.3 describes the method: the weights are never
// dequantised -- their raw block bytes are staged in on-chip memory and
// decoded in registers where the integer matrix instruction needs them; the
// activations are quantised once per call by a prepass; the integer tile
// product accumulates exactly in int32; the float scales are applied after
// the integer loop.  On gfx950 one v_mfma_i32_32x32x32_i8 covers K = 32, i.e.
// exactly one q8_1 block, so every MFMA result is the integer dot A of one
// (weight row, token, 32-block) and receives its own scale:
//     T = d8 * (D * A - Mn * Bq),  D = d*sc, Mn = dmin*m, Bq = sum of q8 codes.
//
// Tiling: a workgroup (4 wavefronts, 2 x 2) computes 128 weight rows x BN =
// 64 NTW tokens; each wavefront a 64 x 32 NTW block of 2 x NTW 32 x 32 MFMA
// tiles (NTW = 2, or 1 where three smaller workgroups per CU take fewer
// rounds of the grid, see launch_mmq_q4k).  The K
// loop walks one superblock (256 values, 8 q8_1 blocks) at a time, every
// global load of a stage issued before the first LDS write:
//   * raw Q4_K superblocks of the 128 rows -> LDS (16-byte loads);
//     per row and sub-block D (f32), per row the eight m (bf16) and -dmin;
//   * q8_1 blocks of the BN tokens -> LDS as int8 codes (rows padded to
//     272 bytes against bank conflicts) plus per (token, block) d8 and
//     z = d8*Bq, the latter as three bf16 parts whose sum is exactly z;
//   * the minimum terms of the whole superblock: two bf16 MFMAs over the
//     8 blocks x 3 parts give sum_j m_j z_j (exact products, f32 sums),
//     times -dmin per row: the start of the superblock's partial;
//   * per pair of blocks (the low and high nibbles of the same 32 code
//     bytes): nibbles -> two int8 operands in registers, two int8 MFMAs
//     give the exact block dots; one f32 MFMA forms both blocks' scale outer
//     products D (x) d8; the VALU only converts the dots and applies the
//     scales (2 instructions per output and block).  Per-superblock partials
//     are added to the output accumulator once per superblock, so each
//     output sees about 11 + k/256 f32 roundings in sequence.
// Outputs beyond m or n are computed from clamped (valid) rows/tokens and not
// stored.  No atomics; results are bitwise reproducible.
#include "kq_device.h"

#include <algorithm>

namespace kq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 128;            // weight rows per workgroup
constexpr int kCodeStride = 272;   // LDS bytes per token row of codes (256 + 16 pad)
constexpr int kTokStride = 9;      // floats per token in the d8 plane (8 + 1 pad)
constexpr int kZStride = 40;       // bf16 per token in the z plane (4 x 8 + 8 pad)

template <int NTW>
struct Smem {
    static constexpr int BN = 64 * NTW;  // tokens per workgroup
    uint8_t wraw[BM * kQ4KBytes];        // raw superblocks, 144 bytes per row
    float dsc[8][BM];                    // D = d*sc    per (block, row)
    uint32_t mins[BM][4];                // m of blocks 0..7 per row, as bf16 (exact)
    float ndmin[BM];                     // -dmin per row
    int8_t codes[BN * kCodeStride];      // q8 codes per token
    float d8[BN * kTokStride];           // per (token, block)
    uint16_t zs[BN * kZStride];          // z = d8 * (sum of the block's codes) per
                                         // (token, block) as three bf16 parts
                                         // [hi x 8][mid x 8][lo x 8][0 x 8]
};

template <int NTW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NTW == 1 ? 3 : 2, NTW == 1 ? 3 : 2)))
void mmq_q4k_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq,
                    float* __restrict__ y, int M, int N, int S) {
    constexpr int BN = Smem<NTW>::BN;
    __shared__ __align__(16) Smem<NTW> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // wave position in the 2 x 2 grid
    const int l32 = lane & 31, h2 = lane >> 5;
    const int m0 = blockIdx.x * BM;
    const int n0 = blockIdx.y * BN;
    const int64_t row_bytes = (int64_t)S * kQ4KBytes;
    const int nb_row = S * 8;

    float acc[2][NTW][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    for (int sb = 0; sb < S; ++sb) {
        // ---- staging, every global load issued before the first LDS write.
        // Weights: two threads per row; thread (row, e) takes the 16-byte
        // chunks e, e+2, ... of the row's 144-byte superblock (9 chunks); the
        // even thread also decodes the header chunk into D per sub-block,
        // the eight m as bf16 and -dmin.  Activations: BN tokens x 8 q8_1
        // blocks, 2 NTW (token, block) pairs per thread, each also writing
        // the three bf16 parts of its z.
        {
            // recompute the staging addresses every superblock: kept live
            // across the MFMA loop they would cost registers it needs
            int ts = tid;
            asm volatile("" : "+v"(ts));
            const int rr = ts >> 1, e = ts & 1;
            const int gr = min(m0 + rr, M - 1);
            const uint8_t* p = w + (int64_t)gr * row_bytes + (int64_t)sb * kQ4KBytes;
            uint4 cw[5];
#pragma unroll
            for (int c = 0; c < 5; ++c) {
                const int ch = e + 2 * c;
                if (ch < 9) cw[c] = load16(p + 16 * ch);
            }
            uint4 c0[2 * NTW], c1[2 * NTW];
            uint32_t hd[2 * NTW];
#pragma unroll
            for (int i = 0; i < 2 * NTW; ++i) {
                const int idx = ts + 256 * i;
                const int t = idx >> 3, j = idx & 7;
                const int gt = min(n0 + t, N - 1);
                const uint8_t* blk = xq + ((int64_t)gt * nb_row + sb * 8 + j) * kQ81Bytes;
                hd[i] = *(const uint32_t*)blk;
                c0[i] = load16(blk + 4);
                c1[i] = load16(blk + 20);
            }
#pragma unroll
            for (int c = 0; c < 5; ++c) {
                const int ch = e + 2 * c;
                if (ch < 9) *(uint4*)(sm.wraw + rr * kQ4KBytes + 16 * ch) = cw[c];
            }
            if (e == 0) {   // (D, Mn) per sub-block from the header chunk
                const uint4 hdr = cw[0];
                const float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
                const uint32_t lowS = hdr.y & 0x3f3f3f3fu, lowM = hdr.z & 0x3f3f3f3fu;
                const uint32_t hiS = (hdr.w & 0x0f0f0f0fu) | ((hdr.y >> 2) & 0x30303030u);
                const uint32_t hiM = ((hdr.w >> 4) & 0x0f0f0f0fu) | ((hdr.z >> 2) & 0x30303030u);
                uint32_t mb[4];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t s4 = j < 4 ? lowS : hiS, m4 = j < 4 ? lowM : hiM;
                    const int sh = 8 * (j & 3);
                    sm.dsc[j][rr] = d * (float)((s4 >> sh) & 0xff);
                    // m < 64 has at most six significant bits: its bf16 is exact
                    const uint32_t mbits = __float_as_uint((float)((m4 >> sh) & 0xff)) >> 16;
                    if (j & 1) mb[j >> 1] |= mbits << 16;
                    else mb[j >> 1] = mbits;
                }
                *(uint4*)sm.mins[rr] = make_uint4(mb[0], mb[1], mb[2], mb[3]);
                sm.ndmin[rr] = -dmin;
            }
#pragma unroll
            for (int i = 0; i < 2 * NTW; ++i) {
                const int idx = tid + 256 * i;
                const int t = idx >> 3, j = idx & 7;
                const uint32_t cc[8] = {c0[i].x, c0[i].y, c0[i].z, c0[i].w,
                                        c1[i].x, c1[i].y, c1[i].z, c1[i].w};
                int sum = 0;
#pragma unroll
                for (int q = 0; q < 8; ++q) sum = dot4(cc[q], 0x01010101u, sum);
                const float d8 = half_bits_to_float(hd[i]);
                uint4* dst = (uint4*)(sm.codes + t * kCodeStride + 32 * j);
                dst[0] = c0[i];
                dst[1] = c1[i];
                sm.d8[t * kTokStride + j] = d8;
                // z in three bf16 parts, each the next eight significant bits
                // (truncation leaves an exact remainder; a finite z has 24)
                const float z = d8 * (float)sum;
                const uint32_t zh = __float_as_uint(z) & 0xffff0000u;
                const float r1 = z - __uint_as_float(zh);
                const uint32_t zm = __float_as_uint(r1) & 0xffff0000u;
                const float r2 = r1 - __uint_as_float(zm);
                const bool fin = __builtin_isfinite(z);
                uint16_t* zt = sm.zs + t * kZStride + j;
                zt[0] = (uint16_t)(zh >> 16);
                zt[8] = fin ? (uint16_t)(zm >> 16) : (uint16_t)0;
                zt[16] = fin ? (uint16_t)(__float_as_uint(r2) >> 16) : (uint16_t)0;
                zt[24] = 0;
            }
        }
        __syncthreads();

        // Per-superblock partial of every output, per 32 x 32 tile:
        //   part  = -dmin * sum_j m_j z_j      two bf16 MFMAs over the 8
        //           blocks x 3 parts of z (products exact, f32 sums), one
        //           f32 multiply per output;
        // then each pair of blocks (2p, 2p+1) -- the low and high nibbles of
        // the same code bytes -- adds
        //   S     = D (x) d8           f32 MFMA, two outer products
        //   part += float(A_2p) * S_2p + float(A_2p+1) * S_2p+1   (VALU)
        // with A the exact int32 block dots from the int8 MFMA.
        v16f part[2][NTW];
        {
            v8bf am[2], bz[NTW][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                am[mt] = __builtin_bit_cast(v8bf, *(const uint4*)sm.mins[wm * 64 + mt * 32 + l32]);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const uint16_t* zt = sm.zs + (wn * 32 * NTW + nt * 32 + l32) * kZStride + 8 * h2;
                bz[nt][0] = __builtin_bit_cast(v8bf, *(const uint4*)zt);
                bz[nt][1] = __builtin_bit_cast(v8bf, *(const uint4*)(zt + 16));
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                // -dmin of this lane's 16 output rows: 4 runs of 4
                float nd[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 v = *(const float4*)(sm.ndmin + wm * 64 + mt * 32 + 8 * g + 4 * h2);
                    nd[4 * g] = v.x; nd[4 * g + 1] = v.y; nd[4 * g + 2] = v.z; nd[4 * g + 3] = v.w;
                }
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const v16f zero = {};
                    v16f pm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[mt], bz[nt][0], zero, 0, 0, 0);
                    pm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[mt], bz[nt][1], pm, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) part[mt][nt][i] = nd[i] * pm[i];
                }
            }
        }

#pragma unroll 1
        for (int pp = 0; pp < 4; ++pp) {
            const int jl = 2 * pp + h2;   // this lane's block within the pair for the f32 MFMA
            v4i A[2][2];
            float Dp[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int r = wm * 64 + mt * 32 + l32;
                const uint4 q = *(const uint4*)(sm.wraw + r * kQ4KBytes + 16 + 32 * pp + 16 * h2);
                A[mt][0] = v4i{(int)(q.x & 0x0f0f0f0fu), (int)(q.y & 0x0f0f0f0fu),
                               (int)(q.z & 0x0f0f0f0fu), (int)(q.w & 0x0f0f0f0fu)};
                A[mt][1] = v4i{(int)((q.x >> 4) & 0x0f0f0f0fu), (int)((q.y >> 4) & 0x0f0f0f0fu),
                               (int)((q.z >> 4) & 0x0f0f0f0fu), (int)((q.w >> 4) & 0x0f0f0f0fu)};
                Dp[mt] = sm.dsc[jl][r];
            }
            v4i B[NTW][2];
            float dp[NTW];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int t = wn * 32 * NTW + nt * 32 + l32;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint4 a = *(const uint4*)(sm.codes + t * kCodeStride + 32 * (2 * pp + e) + 16 * h2);
                    B[nt][e] = v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
                }
                dp[nt] = sm.d8[t * kTokStride + jl];
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                    const v32f zf = {};
                    const v16i R0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mt][0], B[nt][0], zero, 0, 0, 0);
                    const v16i R1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mt][1], B[nt][1], zero, 0, 0, 0);
                    const v32f S = __builtin_amdgcn_mfma_f32_32x32x1f32(Dp[mt], dp[nt], zf, 0, 0, 0);
                    v16f pt = part[mt][nt];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        pt[i] += (float)R0[i] * S[i];
                        pt[i] += (float)R1[i] * S[16 + i];
                    }
                    part[mt][nt] = pt;
                }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < NTW; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] += part[a][b][i];
        __syncthreads();
    }

    // ---- store: lane holds token (l32) and 16 rows of each tile
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int n = n0 + wn * 32 * NTW + nt * 32 + l32;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm * 64 + mt * 32 + 8 * (i >> 2) + 4 * h2 + (i & 3);
                if (m < M) y[(int64_t)n * M + m] = acc[mt][nt][i];
            }
        }
}

}  // namespace

// Tokens per workgroup, 128 (NTW = 2: two workgroups per CU) or 64 (NTW =
// 1: 168 VGPRs and 49 KB of LDS, three per CU, whose staging then hides
// better behind the others' arithmetic).  Measured on one box at 2048
// tokens, a full round of the 64-token form takes ~0.75 of a round of the
// 128-token one, so the form with the fewer weighted rounds is launched:
// QKV 4608 rows (1152 small tiles in two rounds of 768 slots against 576
// large ones in two rounds of 512) takes 64 tokens, 206 -> 158 us; gate/up
// 18944 rows (seven small rounds against five large) and down 3584 rows
// (two small rounds against one large) take 128.
hipError_t launch_mmq_q4k(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                          int64_t k, int cus, hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int64_t mt = (m + BM - 1) / BM;
    const int64_t t2 = mt * ((n + 127) / 128), t1 = mt * ((n + 63) / 64);
    const int64_t s2 = (int64_t)cus * std::max(1, occupancy((const void*)mmq_q4k_kernel<2>, 256, 0));
    const int64_t s1 = (int64_t)cus * std::max(1, occupancy((const void*)mmq_q4k_kernel<1>, 256, 0));
    // the 64-token grid must also fit 65535 workgroups in y (n up to 65535*128
    // is accepted, which only the 128-token form covers)
    const bool small = (n + 63) / 64 <= 65535 && 3 * ((t1 + s1 - 1) / s1) < 4 * ((t2 + s2 - 1) / s2);
    const int bn = small ? 64 : 128;
    dim3 grid((unsigned)mt, (unsigned)((n + bn - 1) / bn));
    if (small)
        hipLaunchKernelGGL(mmq_q4k_kernel<1>, grid, dim3(256), 0, stream, (const uint8_t*)w,
                           (const uint8_t*)xq, y, (int)m, (int)n, S);
    else
        hipLaunchKernelGGL(mmq_q4k_kernel<2>, grid, dim3(256), 0, stream, (const uint8_t*)w,
                           (const uint8_t*)xq, y, (int)m, (int)n, S);
    return hipGetLastError();
}

}  // namespace kq
