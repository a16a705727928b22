// mmq_q6k.hip -- Q6_K x q8_1 matrix-matrix product on the int8 matrix cores.
//
// The prefill product for the Q6_K tensors of a mixed Q4_K/Q6_K model (cajeta
// "One model, start to last token" 3: the Q6_K value and down projections run
// on their own tensor-core tile; minfer "The CUDA backend" 2.3: raw block
// bytes staged on chip, integer tile products, float scales applied after the
// integer loop).
//
// A Q6_K weight is d * sc_g * (q - 32) with a signed 8-bit scale sc_g per 16
// values.  The scale cannot be applied after a 32-value integer dot (the two
// 16-value halves of a q8_1 block carry different scales), so it is folded
// into the integer operand instead: u = -sc_g * (q - 32) lies in
// [-4096, 4064] and splits exactly into two int8 operands,
//     u = 32 * a + b,   a = u >> 5 in [-128, 127],   b = u & 31 in [0, 31].
// Two v_mfma_i32_32x32x32_i8 per (32 x 32 tile, q8_1 block) give
// Ca = sum a*code and Cb = sum b*code, and the exact integer
//     t = 32 * Ca + Cb = -sum over the block of sc*(q-32)*code
// (|t| < 2^24, so it converts to f32 without rounding).  The VALU then needs
// one shift-add, one conversion and one fused multiply-add by d8 per output
// and block; d (and the sign) is applied once per superblock.
//
// Tiling: a workgroup (4 wavefronts) computes 128 weight rows x BN = 32 NT
// tokens; wavefront w owns rows 32w .. 32w+31 and all BN tokens (NT 32 x 32
// MFMA tiles), so every weight value is decoded by exactly one lane.  NT = 4
// (BN = 128) amortises the decode over the most tiles; a product whose
// 128 x 128 grid would leave compute units idle (the 512-row value
// projection: 64 workgroups for 256 CUs) takes NT = 2 or 1.  Per
// superblock (256 values = 8 q8_1 blocks), every global load of a stage
// issued before the first LDS write:
//   * the 210-byte superblocks of the 128 rows -> LDS, realigned to 4 bytes
//     (every other superblock starts at 2 mod 4; 4-byte-aligned 16-byte
//     loads plus a 16-bit funnel shift, never reading outside the weight
//     tensor); -d per row as f32;
//   * the q8_1 blocks of the BN tokens -> LDS as int8 codes (token rows
//     padded to 272 bytes) and f32 d8 per (token, block).
// Outputs beyond m or n are computed from clamped (valid) rows/tokens and not
// stored.  No atomics; results are bitwise reproducible.
#include "kq_device.h"

#include <algorithm>
#include <atomic>

namespace kq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;            // weight rows per workgroup
constexpr int kRawDw = 56;         // LDS dwords per row: 53 used (212 B), 16-byte aligned rows
constexpr int kCodeStride = 272;   // LDS bytes per token row of codes (256 + 16 pad)
constexpr int kTokStride = 9;      // floats per token in the d8 plane (8 + 1 pad)

template <int NT>
struct Smem {
    static constexpr int BN = 32 * NT;   // tokens per workgroup
    uint32_t wraw[BM * kRawDw];          // realigned Q6_K superblock per row
    float negd[BM];                      // -d per row
    int8_t codes[BN * kCodeStride];      // q8 codes per token
    float d8[BN * kTokStride];           // per (token, block)
};

// Four 6-bit codes (one per byte, 0..63) -> the int8 operand bytes a and b
// of u = -sc*(q-32) = 32a + b.  nsc = -sc and c32 = 32*sc in both 16-bit
// halves; the products are formed in 16-bit lanes (|u| < 2^15).
__device__ __forceinline__ void split4(uint32_t q, u16x2 nsc, u16x2 c32, uint32_t& a4,
                                       uint32_t& b4) {
    const uint32_t e = q & 0x00ff00ffu;          // codes 0 and 2
    const uint32_t o = (q >> 8) & 0x00ff00ffu;   // codes 1 and 3
    const u16x2 ue = __builtin_bit_cast(u16x2, e) * nsc + c32;
    const u16x2 uo = __builtin_bit_cast(u16x2, o) * nsc + c32;
    const uint32_t ae = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, ue) >> (short)5);
    const uint32_t ao = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, uo) >> (short)5);
    const uint32_t we = __builtin_bit_cast(uint32_t, ue), wo = __builtin_bit_cast(uint32_t, uo);
    a4 = (ae & 0x00ff00ffu) | ((ao & 0x00ff00ffu) << 8);
    b4 = ((we & 0x00ff00ffu) | ((wo & 0x00ff00ffu) << 8)) & 0x1f1f1f1fu;
}

// SPLIT: the weights are in the split layout (208-byte bodies at w, 16-byte
// aligned, and the f16 d of superblock row * S + s at wd[row * S + s]).
// K split: workgroup z of the grid's third dimension takes superblocks
// [z * sb_per, min(S, (z + 1) * sb_per)); z = 0 writes its sums to y, z > 0
// to part + (z - 1) * M * N (the same [token][row] layout), and a second
// launch adds the parts to y in the order z = 1, 2, ...
template <int NT, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mmq_q6k_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ wd,
                    const uint8_t* __restrict__ xq, float* y, float* part, int M, int N, int S,
                    int sb_per) {
    constexpr int BN = Smem<NT>::BN;
    __shared__ __align__(16) Smem<NT> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31, h2 = lane >> 5;
    const int m0 = blockIdx.x * BM;
    const int n0 = blockIdx.y * BN;
    const int64_t row_bytes = (int64_t)S * kQ6KBytes;
    const int nb_row = S * 8;
    const int r = wave * 32 + l32;   // this lane's weight row within the tile
    const int sb_beg = (int)blockIdx.z * sb_per, sb_end = min(S, sb_beg + sb_per);
    float* out = blockIdx.z == 0 ? y : part + (int64_t)(blockIdx.z - 1) * M * N;

    float acc[NT][16];
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;

    for (int sb = sb_beg; sb < sb_end; ++sb) {
        // ---- staging, every global load issued before the first LDS write.
        // Weights: two threads per row; thread (row, e) takes the 16-byte
        // chunks e, e+2, ... of the superblock's bytes 0..207 (13 chunks),
        // realigned to the superblock start; the odd thread also takes the
        // f16 d at bytes 208..209.  Activations: BN tokens x 8 q8_1 blocks,
        // NT (token, block) pairs per thread.
        {
            // recompute the staging addresses every superblock: kept live
            // across the MFMA loop they would cost registers it needs
            int ts = tid;
            asm volatile("" : "+v"(ts));
            const int rr = ts >> 1, e = ts & 1;
            const int gr = min(m0 + rr, M - 1);
            const int64_t g = (int64_t)gr * S + sb;
            const uint8_t* p = SPLIT ? w + g * 208 : w + (int64_t)gr * row_bytes + (int64_t)sb * kQ6KBytes;
            const int phase = SPLIT ? 0 : (int)((uintptr_t)p & 2);
            const uint8_t* base = p - phase;   // p - 2 lies in the previous superblock
            uint4 cur[7];
            uint32_t nxt[7];
#pragma unroll
            for (int c = 0; c < 7; ++c) {
                const int ch = e + 2 * c;
                if (ch < 13) {
                    cur[c] = load16(base + 16 * ch);
                    if (!SPLIT) nxt[c] = *(const uint32_t*)(base + 16 * ch + (phase ? 16 : 12));
                }
            }
            const uint32_t dbits = !e ? 0u : SPLIT ? (uint32_t)wd[g] : (uint32_t) * (const uint16_t*)(p + 208);
            uint4 c0[NT], c1[NT];
            uint32_t hd[NT];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int idx = ts + 256 * i;
                const int t = idx >> 3, j = idx & 7;
                const int gt = min(n0 + t, N - 1);
                const uint8_t* blk = xq + ((int64_t)gt * nb_row + sb * 8 + j) * kQ81Bytes;
                hd[i] = *(const uint32_t*)blk;
                c0[i] = load16(blk + 4);
                c1[i] = load16(blk + 20);
            }
#pragma unroll
            for (int c = 0; c < 7; ++c) {
                const int ch = e + 2 * c;
                if (ch < 13) {
                    uint4 v = cur[c];
                    if (!SPLIT && phase) {
                        v.x = (cur[c].x >> 16) | (cur[c].y << 16);
                        v.y = (cur[c].y >> 16) | (cur[c].z << 16);
                        v.z = (cur[c].z >> 16) | (cur[c].w << 16);
                        v.w = (cur[c].w >> 16) | (nxt[c] << 16);
                    }
                    *(uint4*)(sm.wraw + rr * kRawDw + 4 * ch) = v;
                }
            }
            if (e) {
                sm.wraw[rr * kRawDw + 52] = dbits;
                sm.negd[rr] = -half_bits_to_float(dbits);
            }
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int idx = tid + 256 * i;
                const int t = idx >> 3, j = idx & 7;
                uint4* dst = (uint4*)(sm.codes + t * kCodeStride + 32 * j);
                dst[0] = c0[i];
                dst[1] = c1[i];
                sm.d8[t * kTokStride + j] = half_bits_to_float(hd[i]);
            }
        }
        __syncthreads();

        float pt[NT][16];
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) pt[b][i] = 0.0f;

        const uint32_t* row = sm.wraw + r * kRawDw;
        const uint4 scv = *(const uint4*)(row + 48);   // 16 int8 scales at byte 192
        const uint32_t sc_dw[4] = {scv.x, scv.y, scv.z, scv.w};
#pragma unroll 1
        for (int n = 0; n < 2; ++n) {
            // this lane's 16 values of each block of half n: ql bytes
            // 64n + 32(c&1) + 16h2 .., qh bytes 128 + 32n + 16h2 ..
            const uint4 qla = *(const uint4*)(row + 16 * n + 4 * h2);
            const uint4 qlb = *(const uint4*)(row + 16 * n + 8 + 4 * h2);
            const uint4 qhv = *(const uint4*)(row + 32 + 8 * n + 4 * h2);
            const uint32_t QLa[4] = {qla.x, qla.y, qla.z, qla.w};
            const uint32_t QLb[4] = {qlb.x, qlb.y, qlb.z, qlb.w};
            const uint32_t QH[4] = {qhv.x, qhv.y, qhv.z, qhv.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * n + c;
                // scale of this lane's 16 values: index 8n + 2c + h2
                const int sidx = 2 * c + h2;   // within the half's 8 scales
                const uint32_t sdw = n ? sc_dw[2 + (sidx >> 2)] : sc_dw[sidx >> 2];
                const int sc = (int)(int8_t)(sdw >> (8 * (sidx & 3)));
                const uint32_t nsc16 = (uint32_t)(-sc) & 0xffffu, c16 = (uint32_t)(32 * sc) & 0xffffu;
                const u16x2 nsc = __builtin_bit_cast(u16x2, nsc16 | (nsc16 << 16));
                const u16x2 c32 = __builtin_bit_cast(u16x2, c16 | (c16 << 16));
                uint32_t av[4], bv[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t ql = (c & 1) ? QLb[d] : QLa[d];
                    const uint32_t lo4 = (c >> 1) ? (ql >> 4) & 0x0f0f0f0fu : ql & 0x0f0f0f0fu;
                    const uint32_t hi2 = ((QH[d] >> (2 * c)) & 0x03030303u) << 4;
                    split4(lo4 | hi2, nsc, c32, av[d], bv[d]);
                }
                const v4i A = v4i{(int)av[0], (int)av[1], (int)av[2], (int)av[3]};
                const v4i B = v4i{(int)bv[0], (int)bv[1], (int)bv[2], (int)bv[3]};
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int t = nt * 32 + l32;
                    const uint4 x = *(const uint4*)(sm.codes + t * kCodeStride + 32 * j + 16 * h2);
                    const v4i X = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
                    const float d8 = sm.d8[t * kTokStride + j];
                    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                    const v16i Ra = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, X, zero, 0, 0, 0);
                    const v16i Rb = __builtin_amdgcn_mfma_i32_32x32x32_i8(B, X, zero, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        pt[nt][i] = __builtin_fmaf((float)((Ra[i] << 5) + Rb[i]), d8, pt[nt][i]);
                }
            }
        }
        // ---- apply -d per row (the lane's 16 rows 8(i/4) + 4h2 + (i%4))
        float nd[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 v = *(const float4*)(sm.negd + wave * 32 + 8 * g + 4 * h2);
            nd[4 * g + 0] = v.x; nd[4 * g + 1] = v.y; nd[4 * g + 2] = v.z; nd[4 * g + 3] = v.w;
        }
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][i] = __builtin_fmaf(pt[b][i], nd[i], acc[b][i]);
        __syncthreads();
    }

    // ---- store: lane holds token (l32 of each tile) and 16 rows
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + nt * 32 + l32;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + wave * 32 + 8 * (i >> 2) + 4 * h2 + (i & 3);
            if (m < M) out[(int64_t)n * M + m] = acc[nt][i];
        }
    }
}

}  // namespace

// Tokens per workgroup: the largest of 128, 64, 32 whose grid still gives
// every compute unit a workgroup (a smaller tile repeats the weight decode
// for fewer tokens, but idle compute units cost more).
static int mmq_q6k_nt(int64_t m, int64_t n, int cus) {
    const int64_t mt = (m + BM - 1) / BM;
    for (int nt = 4; nt > 1; nt >>= 1)
        if (mt * ((n + 32 * nt - 1) / (32 * nt)) >= cus) return nt;
    return 1;
}

// K-split plan (measured on MI355X, Qwen2-7B prefill shapes at 2048 tokens
// and smaller token counts): when the 128-token grid has fewer than two
// workgroups per CU the K range is cut into 4 parts (at most S/2), with the
// widest token tile whose split grid still gives every CU two workgroups
// (else 32 tokens).  512 x 3584 x 2048: 56 -> 43 us; 3584 x 18944 x 2048:
// 757 -> 708 us (448 tiles are 1.75 rounds of two per CU, 1792 are 3.5).
// A split that needs more than max_ws bytes of workspace is not taken.
MmqPlan plan_mmq_q6k(int64_t m, int64_t n, int64_t k, int cus, int64_t max_ws) {
    const int S = (int)(k / kQK);
    const int64_t mt = (m + BM - 1) / BM;
    auto tiles = [&](int nt) { return mt * ((n + 32 * nt - 1) / (32 * nt)); };
    const MmqPlan whole{mmq_q6k_nt(m, n, cus), 1, S, 0};
    if (tiles(4) >= 2 * (int64_t)cus || S < 4) return whole;
    const int want = std::min(4, S / 2);
    const int sb_per = (S + want - 1) / want;
    const int parts = (S + sb_per - 1) / sb_per;
    int nt = 1;
    for (int c = 4; c > 1; c >>= 1)
        if (tiles(c) * parts >= 2 * (int64_t)cus) {
            nt = c;
            break;
        }
    const MmqPlan split{nt, parts, sb_per, (int64_t)(parts - 1) * m * n * 4};
    return split.ws_bytes <= max_ws ? split : whole;
}

template <bool SPLIT>
static hipError_t launch_mmq_q6k_any(const uint8_t* w, const uint16_t* wd, const void* xq, float* y,
                                     int64_t m, int64_t n, int S, const MmqPlan& p, float* part,
                                     hipStream_t stream) {
    const int nt = p.nt;
    dim3 grid((unsigned)((m + BM - 1) / BM), (unsigned)((n + 32 * nt - 1) / (32 * nt)), (unsigned)p.parts);
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, w, wd, (const uint8_t*)xq, y, part,
                           (int)m, (int)n, S, p.sb_per);
    };
    if (nt == 4) launch(mmq_q6k_kernel<4, SPLIT>);
    else if (nt == 2) launch(mmq_q6k_kernel<2, SPLIT>);
    else launch(mmq_q6k_kernel<1, SPLIT>);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.parts > 1) e = launch_splitk_sum(y, m, part, n, m, p.parts - 1, stream);
    return e;
}

hipError_t launch_mmq_q6k_plan(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                               int64_t k, const MmqPlan& plan, void* ws, hipStream_t stream) {
    return launch_mmq_q6k_any<false>((const uint8_t*)w, nullptr, xq, y, m, n, (int)(k / kQK), plan,
                                     (float*)ws, stream);
}

// Workspace of the allocation-free entry point: a static device array, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never uses the array's name as an address: hipGetSymbolAddress gives each
// device's copy, once per device, and that address is kept.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
std::atomic<void*> g_scratch_ptr[64];
}

hipError_t noalloc_scratch(int device, void** ptr) {
    if (device < 0 || device >= 64) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (!p) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_mmq_q6k(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                          int64_t k, int cus, hipStream_t stream) {
    return launch_mmq_q6k_plan(w, xq, y, m, n, k, plan_mmq_q6k(m, n, k, cus, 0), nullptr, stream);
}

hipError_t launch_mmq_q6k_split(const void* wr, const void* xq, float* y, int64_t m, int64_t n,
                                int64_t k, int cus, hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int64_t G = m * S;
    const uint8_t* bodies = (const uint8_t*)wr + (2 * G + 15) / 16 * 16;
    return launch_mmq_q6k_any<true>(bodies, (const uint16_t*)wr, xq, y, m, n, S,
                                    plan_mmq_q6k(m, n, k, cus, 0), nullptr, stream);
}

}  // namespace kq
