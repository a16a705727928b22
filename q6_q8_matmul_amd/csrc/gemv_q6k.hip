// gemv_q6k.hip -- Q6_K x q8_1 matrix-vector product (output head, batch 1..8),
// on the raw 210-byte layout or on the split layout (f16 d prefix, 208-byte
// bodies 16-byte aligned) made by kq_repack_q6k.
//
// Weight streaming bound like the Q4_K GEMV (minfer "The CUDA backend" 2.2).
// A Q6_K superblock is 210 bytes, so superblock starts are only 2-byte
// aligned; with byte loads the pages' first CUDA path was capped far below the
// memory bus (minfer "The CUDA backend" 3.2.2).  This kernel keeps the 210-byte
// layout and loads only whole aligned dwords: a lane that needs 8 bytes at a
// 2 (mod 4) address reads the three aligned dwords around them and funnel-
// shifts (v_alignbit_b32).  Every read stays inside the tensor: at most the
// two bytes before a superblock that starts at 2 (mod 4), which are the tail
// of the previous superblock.  On the split layout the same lanes read the
// same bytes with aligned 8-byte loads and no shift, and d from the prefix.
//
// Work layout (as the Q4_K GEMV): WAVES wavefronts x RPW rows per row group;
// 8 groups of 8 lanes take 8 consecutive superblocks of a row per pass; the
// raw loads of each pass are requested DEPTH passes ahead of their use.  When
// the activation fits in LDS the grid is persistent (a few workgroups per
// compute unit walk the row groups) and the load ring runs on across row
// groups.
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

#include <algorithm>
#include <type_traits>

namespace kq {
namespace gemv6 {

struct Raw {            // one lane's raw dwords of one superblock of one row
    uint32_t l[3];      // ql, values g = 0 / 2
    uint32_t l2[3];     // ql, values g = 1 / 3
    uint32_t h[3];      // qh
    uint32_t s[3];      // the half's 8 scale bytes (third dword only if misaligned)
    uint32_t dpar;      // f16 d in the low half, byte parity of the superblock in bit 16
};

struct RawS {           // the same share read from the split layout (aligned)
    uint2 l, l2, h, s;  // ql (g = 0 / 2), ql (g = 1 / 3), qh, the half's 8 scale bytes
    uint32_t d;         // f16 d in the low half
};

// LDS layout of one staged column (cap = 8 * schunk q8_1 blocks):
//   codes [schunk][256]  per superblock: lane k = 4h + q finds the 8-value
//                        pieces (block 4h+g, values 8q..8q+7) of g = 0, 1 in
//                        bytes [16k, 16k+16) and of g = 2, 3 in
//                        [128+16k, 128+16k+16), so the 8 lanes of a group read
//                        8 distinct 16-byte bank quads; the two 128-byte
//                        halves trade places in odd superblocks, so the two
//                        groups that one LDS cycle serves (superblocks sb and
//                        sb+1, 256 bytes apart) use different banks too;
//   d8    [cap]          per block.
constexpr int kLdsPerSb = 256 + 8 * 4;

__device__ __forceinline__ int swz(int sb) { return 8 * (sb & 1); }   // in 16-byte units

// Staging of blocks [j0, j0 + nbc) of every column (nbc a multiple of 8):
// one thread per (column, q8_1 block), U blocks per thread per round.  A
// round is split into the issue of its global loads and the LDS writes, so a
// kernel can issue the first round's loads before its weight loads (loads
// complete in issue order: activation loads issued after the weight ring
// would wait for the weights' HBM latency before the staging could finish).
template <int U>
struct StageRegs {
    uint32_t c[U][9];
};

template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_issue(StageRegs<U>& r, const uint8_t* __restrict__ xq,
                                            int nb_row, int j0, int nbc, int base) {
    const int total = BATCH * nbc;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int idx = base + i * NT + (int)threadIdx.x;
        if (idx < total) {
            const int bb = idx / nbc;
            const int j = idx - bb * nbc;
            const uint32_t* blk = (const uint32_t*)(xq + ((int64_t)bb * nb_row + j0 + j) * kQ81Bytes);
#pragma unroll
            for (int e = 0; e < 9; ++e) r.c[i][e] = blk[e];
        }
    }
}

template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_write(const StageRegs<U>& r, int nbc, int base, int schunk,
                                            uint8_t* lds) {
    const int cap = schunk * 8;
    uint8_t* codes = lds;
    float* d8s = (float*)(lds + BATCH * schunk * 256);
    const int total = BATCH * nbc;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int idx = base + i * NT + (int)threadIdx.x;
        if (idx < total) {
            const int bb = idx / nbc;
            const int j = idx - bb * nbc;
            const int sb = j >> 3, jj = j & 7, h = jj >> 2, g = jj & 3;
            uint8_t* cs = codes + (bb * schunk + sb) * 256 + 8 * (g & 1);
            const int u0 = ((g < 2) ? 0 : 8) ^ swz(sb);
#pragma unroll
            for (int q = 0; q < 4; ++q)   // 8-value piece q goes to lane 4h + q
                *(uint2*)(cs + 16 * (u0 + 4 * h + q)) = make_uint2(r.c[i][1 + 2 * q], r.c[i][2 + 2 * q]);
            d8s[bb * cap + j] = half_bits_to_float(r.c[i][0]);
        }
    }
}

// The rest of a staging whose first round was issued into r: its LDS writes,
// every later round, and the closing barrier.
template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_finish(StageRegs<U>& r, const uint8_t* __restrict__ xq,
                                             int nb_row, int j0, int nbc, int schunk,
                                             uint8_t* lds) {
    stage_write<BATCH, NT, U>(r, nbc, 0, schunk, lds);
    for (int base = NT * U; base < BATCH * nbc; base += NT * U) {
        stage_issue<BATCH, NT, U>(r, xq, nb_row, j0, nbc, base);
        stage_write<BATCH, NT, U>(r, nbc, base, schunk, lds);
    }
    __syncthreads();
}

// A whole staging (all loads of a round in flight before any is used).
template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_activation(const uint8_t* __restrict__ xq, int nb_row,
                                                 int j0, int nbc, int schunk, uint8_t* lds) {
    StageRegs<U> r;
    stage_issue<BATCH, NT, U>(r, xq, nb_row, j0, nbc, 0);
    stage_finish<BATCH, NT, U>(r, xq, nb_row, j0, nbc, schunk, lds);
}

// Three aligned dwords covering the 8 bytes at offset `off` of a superblock
// starting at `sb` with sb % 4 == par: [off - par, off - par + 12).  For the
// offsets used here the range starts at most 2 bytes before the superblock
// (the tail of the previous one) and ends before byte 197 of it.
__device__ __forceinline__ void load3(uint32_t (&d)[3], const uint8_t* sb, int par, int off) {
    const uint32_t* p = (const uint32_t*)(sb + off - par);
    d[0] = p[0];
    d[1] = p[1];
    d[2] = p[2];
}

template <int RPW>
__device__ __forceinline__ void load_pass(Raw (&r)[RPW], const uint8_t* __restrict__ w, int row0,
                                          int m, int64_t row_bytes, int sb, int S, int h, int q) {
    const int sbc = min(sb, S - 1);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int row = min(row0 + i, m - 1);
        const int64_t off = (int64_t)row * row_bytes + (int64_t)sbc * kQ6KBytes;
        const uint8_t* p = w + off;
        const int par = (int)(off & 3);
        load3(r[i].l, p, par, 64 * h + 8 * q);
        load3(r[i].l2, p, par, 64 * h + 32 + 8 * q);
        load3(r[i].h, p, par, 128 + 32 * h + 8 * q);
        const uint32_t* ps = (const uint32_t*)(p + 192 + 8 * h - par);
        r[i].s[0] = ps[0];
        r[i].s[1] = ps[1];
        r[i].s[2] = par ? ps[2] : 0u;  // only when the bytes straddle
        r[i].dpar = (uint32_t)*(const uint16_t*)(p + 208) | ((uint32_t)par << 15);
    }
}

// Split layout: superblock g = row * S + s has its 208-byte body at
// wb + 208 g (16-byte aligned) and its d at wd[g].
template <int RPW>
__device__ __forceinline__ void load_pass(RawS (&r)[RPW], const uint8_t* __restrict__ wb,
                                          const uint16_t* __restrict__ wd, int row0, int m, int S,
                                          int sb, int h, int q) {
    const int sbc = min(sb, S - 1);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int64_t g = (int64_t)min(row0 + i, m - 1) * S + sbc;
        const uint8_t* p = wb + g * 208;
        r[i].l = *(const uint2*)(p + 64 * h + 8 * q);
        r[i].l2 = *(const uint2*)(p + 64 * h + 32 + 8 * q);
        r[i].h = *(const uint2*)(p + 128 + 32 * h + 8 * q);
        r[i].s = *(const uint2*)(p + 192 + 8 * h);
        r[i].d = wd[g];
    }
}

// One row's share of one superblock: the 8 code dwords, the scale dwords and
// d, already aligned.
struct Share {
    uint32_t L0, L1, M0, M1, H0, H1, S0, S1;
    float dq;
};

__device__ __forceinline__ Share share_of(const Raw& r) {
    const uint32_t sh = (r.dpar >> 16) * 16u;   // 0 or 16 bits
    Share z;
    z.L0 = __builtin_amdgcn_alignbit(r.l[1], r.l[0], sh);
    z.L1 = __builtin_amdgcn_alignbit(r.l[2], r.l[1], sh);
    z.M0 = __builtin_amdgcn_alignbit(r.l2[1], r.l2[0], sh);
    z.M1 = __builtin_amdgcn_alignbit(r.l2[2], r.l2[1], sh);
    z.H0 = __builtin_amdgcn_alignbit(r.h[1], r.h[0], sh);
    z.H1 = __builtin_amdgcn_alignbit(r.h[2], r.h[1], sh);
    z.S0 = __builtin_amdgcn_alignbit(r.s[1], r.s[0], sh);
    z.S1 = __builtin_amdgcn_alignbit(r.s[2], r.s[1], sh);
    z.dq = half_bits_to_float(r.dpar) * 0.25f;
    return z;
}

__device__ __forceinline__ Share share_of(const RawS& r) {
    Share z;
    z.L0 = r.l.x; z.L1 = r.l.y;
    z.M0 = r.l2.x; z.M1 = r.l2.y;
    z.H0 = r.h.x; z.H1 = r.h.y;
    z.S0 = r.s.x; z.S1 = r.s.y;
    z.dq = half_bits_to_float(r.d) * 0.25f;
    return z;
}

template <int BATCH, int RPW, class R>
__device__ __forceinline__ void compute_pass(const R (&r)[RPW], float (&acc)[RPW][BATCH],
                                             const uint8_t* lds, int schunk, int sl, int h, int q) {
    const uint8_t* codes = lds;
    const float* d8s = (const float*)(lds + BATCH * schunk * 256);
    const int k = 4 * h + q;
    uint2 a[BATCH][4];
    float db[BATCH][4];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
        const uint8_t* cs = codes + (b * schunk + sl) * 256;
        const uint4 lo = *(const uint4*)(cs + 16 * (k ^ swz(sl)));
        const uint4 hi = *(const uint4*)(cs + 16 * ((8 + k) ^ swz(sl)));
        a[b][0] = make_uint2(lo.x, lo.y);
        a[b][1] = make_uint2(lo.z, lo.w);
        a[b][2] = make_uint2(hi.x, hi.y);
        a[b][3] = make_uint2(hi.z, hi.w);
        const float4 d4 = *(const float4*)(d8s + (b * schunk + sl) * 8 + 4 * h);
        db[b][0] = d4.x; db[b][1] = d4.y; db[b][2] = d4.z; db[b][3] = d4.w;
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const Share z = share_of(r[i]);
        const uint32_t L0 = z.L0, L1 = z.L1, M0 = z.M0, M1 = z.M1, H0 = z.H0, H1 = z.H1;
        const uint32_t S0 = z.S0, S1 = z.S1;
        const float dq = z.dq;
        // scale of group g: signed byte 2g + (q >> 1) of the half's 8 scale bytes
        const uint32_t so = 8u * (uint32_t)(q >> 1);
        int sc[4];
        sc[0] = __builtin_amdgcn_sbfe((int)S0, so, 8);
        sc[1] = __builtin_amdgcn_sbfe((int)S0, so + 16u, 8);
        sc[2] = __builtin_amdgcn_sbfe((int)S1, so, 8);
        sc[3] = __builtin_amdgcn_sbfe((int)S1, so + 16u, 8);
        // 4*(q6 - 32) per byte: ((low nibble | high bits << 4) << 2) ^ 0x80
        uint32_t v[4][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t l = t ? L1 : L0;
            const uint32_t l2 = t ? M1 : M0;
            const uint32_t hb = t ? H1 : H0;
            v[0][t] = (((l << 2) & 0x3c3c3c3cu) | ((hb << 6) & 0xc0c0c0c0u)) ^ 0x80808080u;
            v[1][t] = (((l2 << 2) & 0x3c3c3c3cu) | ((hb << 4) & 0xc0c0c0c0u)) ^ 0x80808080u;
            v[2][t] = (((l >> 2) & 0x3c3c3c3cu) | ((hb << 2) & 0xc0c0c0c0u)) ^ 0x80808080u;
            v[3][t] = (((l2 >> 2) & 0x3c3c3c3cu) | (hb & 0xc0c0c0c0u)) ^ 0x80808080u;
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            float t = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int A4 = dot4(v[g][1], a[b][g].y, dot4(v[g][0], a[b][g].x, 0));
                t += (float)__mul24(A4, sc[g]) * db[b][g];
            }
            acc[i][b] += dq * t;
        }
    }
}

// Sum of each (row, column) accumulator over the wavefront, residual add and
// store (lane 0).
template <int BATCH, int RPW>
__device__ __forceinline__ void finish_rows(float (&acc)[RPW][BATCH], float* y,
                                            const float* residual, int row0, int m, int lane) {
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
            acc[i][b] = 0.0f;
        }
    }
}

// PERSIST = false: one workgroup per WAVES*RPW rows; the activation is
// staged (in chunks if needed) by every workgroup.
// PERSIST = true (only when the whole activation fits in LDS): a grid of a
// few workgroups per compute unit stages the activation once and walks the
// row groups blockIdx.x, blockIdx.x + gridDim.x, ...; the load ring runs
// across group boundaries, so a wavefront's next rows are already in flight
// while it finishes the current ones.
// SPLIT: the weights are in the split layout, bodies at w and d at wd.
template <int BATCH, int RPW, int DEPTH, int WAVES, bool PERSIST, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES) void gemv_q6k_kernel(const uint8_t* __restrict__ w,
                                                              const uint16_t* __restrict__ wd,
                                                              const uint8_t* __restrict__ xq,
                                                              float* y, const float* residual,
                                                              int m, int S, int schunk) {
    extern __shared__ __align__(16) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 3;
    const int k8 = lane & 7;
    const int h = k8 >> 2;          // 128-value half of the superblock
    const int q = k8 & 3;           // 8-value slice within each 32-value group
    const int64_t row_bytes = (int64_t)S * kQ6KBytes;
    const int nb_row = S * 8;
    const int npass = (S + 7) >> 3;

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    using R = std::conditional_t<SPLIT, RawS, Raw>;
    R ring[DEPTH][RPW];
    auto load = [&](R (&slot)[RPW], int row0, int sb) {
        if constexpr (SPLIT)
            load_pass<RPW>(slot, w, wd, row0, m, S, sb, h, q);
        else
            load_pass<RPW>(slot, w, row0, m, row_bytes, sb, S, h, q);
    };
    if constexpr (PERSIST) {
        const int rows_per_group = WAVES * RPW;
        const int ngroups = (m + rows_per_group - 1) / rows_per_group;
        const int nitems = ((ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x) * npass;
        // (group, pass) of the next item to load and of the next to compute
        int gl = blockIdx.x, pl = 0;
        StageRegs<2> sr;   // the activation loads go first (see stage_issue)
        stage_issue<BATCH, 64 * WAVES, 2>(sr, xq, nb_row, 0, S * 8, 0);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (d == 0 || d < nitems) {   // nitems >= 1: at most one workgroup per group
                load(ring[d], (gl * WAVES + wave) * RPW, 8 * pl + grp);
                if (++pl == npass) { pl = 0; gl += gridDim.x; }
            }
        }
        stage_finish<BATCH, 64 * WAVES, 2>(sr, xq, nb_row, 0, S * 8, schunk, smem);
        int gc = blockIdx.x, pc = 0;
        for (int it0 = 0; it0 < nitems; it0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int it = it0 + d;
                if (it < nitems) {
                    if (8 * pc + grp < S) compute_pass<BATCH, RPW>(ring[d], acc, smem, schunk, 8 * pc + grp, h, q);
                    if (it + DEPTH < nitems) {
                        load(ring[d], (gl * WAVES + wave) * RPW, 8 * pl + grp);
                        if (++pl == npass) { pl = 0; gl += gridDim.x; }
                    }
                    if (++pc == npass) {
                        finish_rows<BATCH, RPW>(acc, y, residual, (gc * WAVES + wave) * RPW, m, lane);
                        pc = 0;
                        gc += gridDim.x;
                    }
                }
            }
        }
    } else {
        const int row0 = (blockIdx.x * WAVES + wave) * RPW;
        const int chunk_passes = schunk >> 3;
        constexpr int U = BATCH >= 2 && BATCH <= 4 ? 4 : 2;
        StageRegs<U> sr;   // the activation loads go first (see stage_issue)
        stage_issue<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, min(schunk, S) * 8, 0);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            load(ring[d], row0, 8 * d + grp);

        stage_finish<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, min(schunk, S) * 8, schunk, smem);

        for (int p0 = 0; p0 < npass; p0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int p = p0 + d;
                if (p < npass) {
                    const int chunk = p / chunk_passes;
                    const int pl = p - chunk * chunk_passes;
                    if (pl == 0 && p > 0) {
                        __syncthreads();
                        const int kc = chunk * schunk;
                        stage_activation<BATCH, 64 * WAVES, (BATCH >= 2 && BATCH <= 4 ? 4 : 2)>(xq, nb_row, kc * 8, min(schunk, S - kc) * 8,
                                                            schunk, smem);
                    }
                    if (8 * p + grp < S)
                        compute_pass<BATCH, RPW>(ring[d], acc, smem, schunk, 8 * pl + grp, h, q);
                    if (p + DEPTH < npass)
                        load(ring[d], row0, 8 * (p + DEPTH) + grp);
                }
            }
        }
        finish_rows<BATCH, RPW>(acc, y, residual, row0, m, lane);
    }
}

// Launch one variant.  `persist_per_cu` > 0 asks for the persistent form with
// that many workgroups per compute unit (capped by occupancy); it is used
// only when the whole activation fits in one LDS piece.
template <int BATCH, int RPW, int DEPTH, int WAVES, bool SPLIT = false>
hipError_t launch_variant(const void* w, const void* xq, float* y, const float* residual,
                          int64_t m, int64_t k, int lds_budget, int cus, int persist_per_cu,
                          hipStream_t stream, const uint16_t* wd = nullptr) {
    const int S = (int)(k / kQK);
    const int per_sb = BATCH * kLdsPerSb;
    int schunk = (lds_budget / per_sb) & ~7;
    const int s_round = (S + 7) & ~7;
    if (schunk > s_round) schunk = s_round;
    if (schunk < 8) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)schunk * per_sb;
    const int rows_per_block = WAVES * RPW;
    const int64_t ngroups = (m + rows_per_block - 1) / rows_per_block;
    if (persist_per_cu > 0 && schunk >= S) {
        auto kern = gemv_q6k_kernel<BATCH, RPW, DEPTH, WAVES, true, SPLIT>;
        const int o = occupancy((const void*)kern, 64 * WAVES, lds);
        const int64_t grid = std::min<int64_t>(ngroups, (int64_t)cus * std::min(o, persist_per_cu));
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WAVES), lds, stream,
                           (const uint8_t*)w, wd, (const uint8_t*)xq, y, residual, (int)m, S, schunk);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemv_q6k_kernel<BATCH, RPW, DEPTH, WAVES, false, SPLIT>), dim3((unsigned)ngroups),
                       dim3(64 * WAVES), lds, stream, (const uint8_t*)w, wd, (const uint8_t*)xq, y,
                       residual, (int)m, S, schunk);
    return hipGetLastError();
}

}  // namespace gemv6

namespace gemv6 {
template <bool SPLIT>
hipError_t dispatch(const void* w, const uint16_t* wd, const void* xq, float* y,
                    const float* residual, int64_t m, int64_t k, int batch, int cus,
                    hipStream_t stream) {
    // Launch shape measured on MI355X over the 128256 x 4096 output head
    // (back-to-back launches on two rotating weight copies): two rows per
    // wavefront, one pass ahead, persistent grid of up to six workgroups per
    // compute unit -- 85 us at batch 1 (94 us for one workgroup per row
    // group), 124 us at batch 4 (160 us).
    switch (batch) {
        case 1: return launch_variant<1, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 2: return launch_variant<2, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 3: return launch_variant<3, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 4: return launch_variant<4, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 5: return launch_variant<5, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 6: return launch_variant<6, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 7: return launch_variant<7, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 8: return launch_variant<8, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace gemv6

hipError_t launch_gemv_q6k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream) {
    (void)lds_limit;
    return gemv6::dispatch<false>(w, nullptr, xq, y, residual, m, k, batch, cus, stream);
}

hipError_t launch_gemv_q6k_split(const void* wr, const void* xq, float* y, const float* residual,
                                 int64_t m, int64_t k, int batch, int lds_limit, int cus,
                                 hipStream_t stream) {
    (void)lds_limit;
    const int64_t G = m * (k / kQK);
    const uint8_t* bodies = (const uint8_t*)wr + (2 * G + 15) / 16 * 16;
    return gemv6::dispatch<true>(bodies, (const uint16_t*)wr, xq, y, residual, m, k, batch, cus,
                                 stream);
}

}  // namespace kq
