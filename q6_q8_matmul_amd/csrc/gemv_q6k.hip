// gemv_q6k.hip -- Q6_K x q8_1 matrix-vector product (output head, batch 1..8),
// on the raw 210-byte layout or on the split layout (f16 d prefix, 208-byte
// bodies 16-byte aligned) made by kq_repack_q6k.
//
// Weight streaming bound like the Q4_K GEMV (minfer "The CUDA backend" 2.2).
// A Q6_K superblock is 210 bytes, so superblock starts are only 2-byte
// aligned; with byte loads the pages' first CUDA path was capped far below the
// memory bus (minfer "The CUDA backend" 3.2.2).  This kernel keeps the 210-byte
// layout and loads only whole aligned dwords: a lane that needs 32 bytes at a
// 2 (mod 4) address reads the nine aligned dwords around them and funnel-
// shifts (v_alignbit_b32).  Every read stays inside the tensor: at most the
// two bytes before a superblock that starts at 2 (mod 4), which are the tail
// of the previous superblock.  On the split layout the same lanes read the
// same bytes with aligned 16-byte loads and no shift, and d from the prefix.
//
// Work layout: WAVES wavefronts x RPW rows per row group, a whole wavefront
// per row; 16 groups of 4 lanes take 16 consecutive superblocks of a row per
// pass; the loads of each pass are requested DEPTH passes ahead of their use.
// When the activation fits in LDS the grid is persistent (a few workgroups
// per compute unit walk the row groups) and the load ring runs on across row
// groups.
// Lane t of a group (h = t / 2, c = t % 2) owns the 64 values of q8_1 blocks
// 4h + c and 4h + c + 2 of the superblock: both nibbles of ql bytes
// [64h + 32c, 64h + 32c + 32) (low: block 4h + c, high: block 4h + c + 2),
// their high bits from qh bytes [32h, 32h + 32) (bits 2c, 2c+1 and 2c+4,
// 2c+5), and the four 16-value scales 8h + 2c, 8h + 2c + 1, 8h + 2c + 4,
// 8h + 2c + 5.  The lane forms 4*(q6 - 32) directly as an int8 byte ((code
// << 2) with bit 7 inverted is sign-correct because the code is 6 bits wide),
// so a v_dot4_i32_i8 chain over 16 values gives 4x the integer dot of one
// scale group; the factor 4 is folded back into d exactly.  Per block the two
// scale groups combine in integers (A0*sc0 + A1*sc1), so each block costs one
// conversion and one multiply-add per column.
//
// The activation is staged into LDS once per workgroup (int8 codes and the
// per-32-block d8), in chunks when it exceeds the LDS budget.  Per lane:
// sum over its two blocks of d8 * float(A0*sc0 + A1*sc1) per superblock,
// times d/4, accumulated in a private f32 register; then one fixed 64-lane
// xor-butterfly per row and column and the optional residual add on the row
// write (leone-cuda "CUDA kernel design": Q6_K GEMV with residual epilogue,
// fixed reduction order, no atomics).
#include "kq_device.h"

#include <algorithm>
#include <type_traits>

namespace kq {
namespace gemv6 {

constexpr int kSbPerPass = 16;   // superblocks of a row per wavefront pass

struct Raw {            // one lane's raw dwords of one superblock of one row
    uint32_t l[9];      // ql bytes [64h + 32c, +32), 2 (mod 4) shifted
    uint32_t q[9];      // qh bytes [32h, +32)
    uint32_t s[3];      // the half's 8 scale bytes (third dword only if misaligned)
    uint32_t dpar;      // f16 d in the low half, byte parity of the superblock in bit 16
};

struct RawS {           // the same share read from the split layout (aligned)
    uint4 l0, l1;       // ql
    uint4 q0, q1;       // qh
    uint2 s;            // the half's 8 scale bytes
    uint32_t d;         // f16 d in the low half
};

// LDS layout of a staged activation (schunk superblocks, BATCH columns):
//   codes [schunk][BATCH][256]  every column's 256 q8 codes of a superblock;
//                               16-byte unit u (values 16u..16u+15) stored at
//                               unit u ^ swz(sb); lane t reads units
//                               8h + 2c + {0, 1, 4, 5};
//   dz    [BATCH][schunk][4]    float2 per (column, superblock, lane t): d8
//                               of blocks 4h + c and 4h + c + 2.
// The sixteen lanes that one LDS cycle serves are the four lanes of each of
// superblocks sb .. sb+3 (sb a multiple of 4).  Their units 8h + 2c + r0 for
// one read differ in bits 1 and 3, and swz(sb) = (sb & 1) | (sb & 2) << 1
// sets bits 0 and 2 by superblock, so the sixteen 16-byte reads hit distinct
// bank groups (the superblock stride is a multiple of 256 bytes).  The dz
// reads of 32 lanes are 256 contiguous bytes.
constexpr int lds_per_sb(int batch) { return batch * (256 + 4 * 8); }

__device__ __forceinline__ int swz(int sb) { return (sb & 1) | ((sb & 2) << 1); }

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

// Column of item `idx` (n items per column), without a division.
template <int BATCH>
__device__ __forceinline__ int column_of(int idx, int n) {
    int bb = 0;
#pragma unroll
    for (int c = 1; c < BATCH; ++c) bb += idx >= c * n ? 1 : 0;
    return bb;
}

template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_issue(StageRegs<U>& r, const uint8_t* __restrict__ xq,
                                            int nb_row, int j0, int nbc, int base) {
    const int total = BATCH * nbc;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int idx = base + i * NT + (int)threadIdx.x;
        if (idx < total) {
            const int bb = column_of<BATCH>(idx, nbc);
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
    float* dz = (float*)(lds + schunk * BATCH * 256);
    const int total = BATCH * nbc;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int idx = base + i * NT + (int)threadIdx.x;
        if (idx < total) {
            const int bb = column_of<BATCH>(idx, nbc);
            const int j = idx - bb * nbc;
            const int sb = j >> 3, jj = j & 7;
            uint8_t* cs = lds + (sb * BATCH + bb) * 256;
            const int x = swz(sb);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *(uint4*)(cs + 16 * ((2 * jj + hh) ^ x)) =
                    make_uint4(r.c[i][1 + 4 * hh], r.c[i][2 + 4 * hh], r.c[i][3 + 4 * hh], r.c[i][4 + 4 * hh]);
            // block jj = 4h + g is read by lane t = 2h + (g & 1), slot g >> 1
            const int h = jj >> 2, g = jj & 3;
            dz[((bb * schunk + sb) * 4 + 2 * h + (g & 1)) * 2 + (g >> 1)] = half_bits_to_float(r.c[i][0]);
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

// N + 1 aligned dwords covering the 4N bytes at offset `off` of a superblock
// starting at `sb` with sb % 4 == par: [off - par, off - par + 4N + 4).  For
// the offsets used here the range starts at most 2 bytes before the
// superblock (the tail of the previous one) and ends before byte 197 of it.
template <int N>
__device__ __forceinline__ void load_dwords(uint32_t (&d)[N + 1], const uint8_t* sb, int par, int off) {
    const uint32_t* p = (const uint32_t*)(sb + off - par);
#pragma unroll
    for (int e = 0; e <= N; ++e) d[e] = p[e];
}

template <int RPW>
__device__ __forceinline__ void load_pass(Raw (&r)[RPW], const uint8_t* __restrict__ w, int row0,
                                          int m, int64_t row_bytes, int sb, int S, int h, int c) {
    const int sbc = min(sb, S - 1);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int row = min(row0 + i, m - 1);
        const int64_t off = (int64_t)row * row_bytes + (int64_t)sbc * kQ6KBytes;
        const uint8_t* p = w + off;
        const int par = (int)(off & 3);
        load_dwords<8>(r[i].l, p, par, 64 * h + 32 * c);
        load_dwords<8>(r[i].q, p, par, 128 + 32 * h);
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
                                          int sb, int h, int c) {
    const int sbc = min(sb, S - 1);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int64_t g = (int64_t)min(row0 + i, m - 1) * S + sbc;
        const uint8_t* p = wb + g * 208;
        r[i].l0 = load16(p + 64 * h + 32 * c);
        r[i].l1 = load16(p + 64 * h + 32 * c + 16);
        r[i].q0 = load16(p + 128 + 32 * h);
        r[i].q1 = load16(p + 128 + 32 * h + 16);
        r[i].s = *(const uint2*)(p + 192 + 8 * h);
        r[i].d = wd[g];
    }
}

// One row's share of one superblock: the 8 ql and 8 qh dwords, the two scale
// dwords and d, already aligned.
struct Share {
    uint32_t L[8], Q[8];
    uint32_t S0, S1;
    float dq;
};

__device__ __forceinline__ Share share_of(const Raw& r) {
    const uint32_t sh = (r.dpar >> 16) * 16u;   // 0 or 16 bits
    Share z;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        z.L[e] = __builtin_amdgcn_alignbit(r.l[e + 1], r.l[e], sh);
        z.Q[e] = __builtin_amdgcn_alignbit(r.q[e + 1], r.q[e], sh);
    }
    z.S0 = __builtin_amdgcn_alignbit(r.s[1], r.s[0], sh);
    z.S1 = __builtin_amdgcn_alignbit(r.s[2], r.s[1], sh);
    z.dq = half_bits_to_float(r.dpar) * 0.25f;
    return z;
}

__device__ __forceinline__ Share share_of(const RawS& r) {
    Share z;
    z.L[0] = r.l0.x; z.L[1] = r.l0.y; z.L[2] = r.l0.z; z.L[3] = r.l0.w;
    z.L[4] = r.l1.x; z.L[5] = r.l1.y; z.L[6] = r.l1.z; z.L[7] = r.l1.w;
    z.Q[0] = r.q0.x; z.Q[1] = r.q0.y; z.Q[2] = r.q0.z; z.Q[3] = r.q0.w;
    z.Q[4] = r.q1.x; z.Q[5] = r.q1.y; z.Q[6] = r.q1.z; z.Q[7] = r.q1.w;
    z.S0 = r.s.x; z.S1 = r.s.y;
    z.dq = half_bits_to_float(r.d) * 0.25f;
    return z;
}

template <int BATCH, int RPW, class R>
__device__ __forceinline__ void compute_pass(const R (&r)[RPW], float (&acc)[RPW][BATCH],
                                             const uint8_t* lds, int schunk, int sl, int c) {
    // rows first: 4*(q6 - 32) bytes of blocks c (lo) and c + 2 (hi), the four
    // int8 scales, d/4.  Code byte = nibble | (qh bits << 4); (code << 2) with
    // bit 7 inverted: nibble into bits 2..5, the qh bit pair into bits 6, 7
    // (qh bits 2g, 2g+1 for block g, so shifts 6 - 2c and 2 - 2c), the odd qh
    // bits inverted up front.
    const uint32_t s_lo = 6u - 2u * (uint32_t)c, s_hi = 2u - 2u * (uint32_t)c;
    const uint32_t so = 16u * (uint32_t)c;   // scale bytes 2c, 2c+1 of each scale dword
    uint4 wl[RPW][2], wh[RPW][2];
    int sc[RPW][4];
    float dq[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const Share z = share_of(r[i]);
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t qn = z.Q[e] ^ 0xaaaaaaaau;
            lo[e] = ((z.L[e] & 0x0f0f0f0fu) << 2) | ((qn << s_lo) & 0xc0c0c0c0u);
            hi[e] = ((z.L[e] >> 2) & 0x3c3c3c3cu) | ((qn << s_hi) & 0xc0c0c0c0u);
        }
        wl[i][0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        wl[i][1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
        wh[i][0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        wh[i][1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        sc[i][0] = __builtin_amdgcn_sbfe((int)z.S0, so, 8);
        sc[i][1] = __builtin_amdgcn_sbfe((int)z.S0, so + 8u, 8);
        sc[i][2] = __builtin_amdgcn_sbfe((int)z.S1, so, 8);
        sc[i][3] = __builtin_amdgcn_sbfe((int)z.S1, so + 8u, 8);
        dq[i] = z.dq;
    }
    // then one column at a time: its activation slice of this lane, used by
    // every row
    const int t = threadIdx.x & 3;
    const int h = t >> 1;
    const uint8_t* cs = lds + sl * (BATCH * 256);
    const int x = swz(sl);
    const int u0 = 8 * h + 2 * c;
    const float2* dz = (const float2*)(lds + schunk * BATCH * 256) + sl * 4 + t;
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
        uint4 a[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            a[rr] = *(const uint4*)(cs + b * 256 + 16 * ((u0 + (rr & 1) + 4 * (rr >> 1)) ^ x));
        const float2 d8 = dz[b * schunk * 4];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int Tl = __mul24(dot16_z(wl[i][0], a[0]), sc[i][0]) + __mul24(dot16_z(wl[i][1], a[1]), sc[i][1]);
            const int Th = __mul24(dot16_z(wh[i][0], a[2]), sc[i][2]) + __mul24(dot16_z(wh[i][1], a[3]), sc[i][3]);
            const float v = fmaf(d8.y, (float)Th, d8.x * (float)Tl);
            acc[i][b] = fmaf(dq[i], v, acc[i][b]);
        }
    }
}

// Sum of each (row, column) accumulator over the wavefront (the columns of
// a row in one transposing butterfly: lane 64b/NB holds column b), residual
// add and store.
template <int BATCH, int RPW>
__device__ __forceinline__ void finish_rows(float (&acc)[RPW][BATCH], float* y,
                                            const float* residual, int row0, int m, int lane) {
    constexpr int NB = pow2_ceil(BATCH);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = row0 + i;
        float v[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) v[b] = b < BATCH ? acc[i][b] : 0.0f;
        const float t = lane_sums<NB, 64>(v, lane);
        const int b = lane / (64 / NB);
        if (lane % (64 / NB) == 0 && b < BATCH && r < m) {
            const int64_t o = (int64_t)b * m + r;
            y[o] = residual ? residual[o] + t : t;
        }
#pragma unroll
        for (int bb = 0; bb < BATCH; ++bb) acc[i][bb] = 0.0f;
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
    const int grp = lane >> 2;      // superblock of the pass
    const int t = lane & 3;
    const int h = t >> 1;           // 128-value half of the superblock
    const int c = t & 1;            // blocks 4h + c and 4h + c + 2 of the half
    const int64_t row_bytes = (int64_t)S * kQ6KBytes;
    const int nb_row = S * 8;
    const int npass = (S + kSbPerPass - 1) / kSbPerPass;

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    using R = std::conditional_t<SPLIT, RawS, Raw>;
    R ring[DEPTH][RPW];
    auto load = [&](R (&slot)[RPW], int row0, int sb) {
        if constexpr (SPLIT)
            load_pass<RPW>(slot, w, wd, row0, m, S, sb, h, c);
        else
            load_pass<RPW>(slot, w, row0, m, row_bytes, sb, S, h, c);
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
                load(ring[d], (gl * WAVES + wave) * RPW, kSbPerPass * pl + grp);
                if (++pl == npass) { pl = 0; gl += gridDim.x; }
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the staging arithmetic after the weight loads
        stage_finish<BATCH, 64 * WAVES, 2>(sr, xq, nb_row, 0, S * 8, schunk, smem);
        int gc = blockIdx.x, pc = 0;
        for (int it0 = 0; it0 < nitems; it0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int it = it0 + d;
                if (it < nitems) {
                    if (kSbPerPass * pc + grp < S)
                        compute_pass<BATCH, RPW>(ring[d], acc, smem, schunk, kSbPerPass * pc + grp, c);
                    __builtin_amdgcn_sched_barrier(0);   // the slot's next loads after its use
                    if (it + DEPTH < nitems) {
                        load(ring[d], (gl * WAVES + wave) * RPW, kSbPerPass * pl + grp);
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
        const int chunk_passes = schunk / kSbPerPass;
        constexpr int U = BATCH >= 2 && BATCH <= 4 ? 4 : 2;
        StageRegs<U> sr;   // the activation loads go first (see stage_issue)
        stage_issue<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, min(schunk, S) * 8, 0);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            load(ring[d], row0, kSbPerPass * d + grp);
        __builtin_amdgcn_sched_barrier(0);   // keep the staging arithmetic after the weight loads
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
                        stage_activation<BATCH, 64 * WAVES, U>(xq, nb_row, kc * 8, min(schunk, S - kc) * 8,
                                                               schunk, smem);
                    }
                    if (kSbPerPass * p + grp < S)
                        compute_pass<BATCH, RPW>(ring[d], acc, smem, schunk, kSbPerPass * pl + grp, c);
                    if (p + DEPTH < npass)
                        load(ring[d], row0, kSbPerPass * (p + DEPTH) + grp);
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
    const int per_sb = lds_per_sb(BATCH);
    int schunk = (lds_budget / per_sb) / kSbPerPass * kSbPerPass;   // whole passes
    const int s_round = (S + kSbPerPass - 1) / kSbPerPass * kSbPerPass;
    if (schunk > s_round) schunk = s_round;
    if (schunk < kSbPerPass) return hipErrorInvalidConfiguration;
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
    // Launch shapes measured on the 128256 x 4096 output head (two weight
    // copies rotating, 431 MB each): four wavefronts per workgroup and a
    // persistent grid.  Raw layout: one row per wavefront, one pass ahead,
    // four workgroups per CU at batch 1 (79 us; six: 81), six at batch 2..8
    // (batch 4: 97 us).  Split layout: two rows per wavefront at batch 1
    // (75 us), one row two passes ahead at batches 2..4 (batch 4: 88 us,
    // one pass ahead: 93).  A row's share per lane is 64 values, so two rows
    // per wavefront take 140-160 VGPRs on the raw layout, where they were
    // slower.
    if constexpr (SPLIT) {
        switch (batch) {
            case 1: return launch_variant<1, 2, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 4, stream, wd);
            case 2: return launch_variant<2, 1, 2, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 4, stream, wd);
            case 3: return launch_variant<3, 1, 2, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 4, stream, wd);
            case 4: return launch_variant<4, 1, 2, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 4, stream, wd);
            default: break;
        }
    } else if (batch == 1) {
        return launch_variant<1, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 4, stream, wd);
    }
    switch (batch) {
        case 1: return launch_variant<1, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 2: return launch_variant<2, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 3: return launch_variant<3, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 4: return launch_variant<4, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 5: return launch_variant<5, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 6: return launch_variant<6, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 7: return launch_variant<7, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
        case 8: return launch_variant<8, 1, 1, 4, SPLIT>(w, xq, y, residual, m, k, 65536, cus, 6, stream, wd);
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
