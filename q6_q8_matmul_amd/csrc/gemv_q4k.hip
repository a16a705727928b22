// gemv_q4k.hip -- Q4_K x q8_1 matrix-vector product (decode, batch 1..8),
// for one weight tensor or for up to 8 tensors that share one activation.
//
// The decode matmul reads every weight byte once, so the kernel is bound by
// HBM bandwidth (minfer "The CUDA backend" 2.2: decode is weight-streaming
// bound; cajeta "One model, start to last token" 4: bytes per second against
// the memory bus is a decode kernel's only figure of merit).  On gfx950 the
// vector ALU work per weight byte is the other limit, so the decode is laid
// out to keep the per-lane instruction count low.
//
// Layout of the work:
//   * a wavefront streams row pairs: lanes 0..31 one row, lanes 32..63 the
//     next; RPW pairs per wavefront, WAVES wavefronts per workgroup;
//   * in a half-wave, 8 groups of 4 lanes take 8 consecutive superblocks per
//     pass; lane t of a group loads the 16-byte header and the code bytes
//     [32t, 32t+32), whose low nibbles are sub-block 2t and high nibbles
//     sub-block 2t+1, so each lane owns two whole 32-value sub-blocks and
//     their two (scale, min) pairs; lanes 0, 1 take their six-bit fields
//     from the low bits of scale bytes 0..7 and lanes 2, 3 from the nibbles
//     of bytes 8..11 plus the top bits of bytes 0..7, both through the same
//     v_bfe_u32 sequence with lane-constant offsets and widths (a zero width
//     gives zero), so the code has no lane-dependent branches;
//   * the loads of the first DEPTH passes are issued before anything else and
//     every later pass is requested DEPTH passes ahead (a register ring), so
//     HBM latency overlaps the activation staging and the arithmetic;
//   * when the whole activation fits in LDS the grid is persistent: a few
//     workgroups per compute unit stage it once and walk the row groups
//     (blockIdx.x, blockIdx.x + gridDim.x, ...) of one tensor or of a table
//     of tensors (the segmented form), and the load ring runs on across row
//     groups, so the memory pipe never drains between them;
//   * the q8_1 activation is restaged once per workgroup into LDS: per
//     superblock its 256 codes in natural order, 16-byte units xor-swizzled
//     by superblock so a 16-lane read hits distinct banks, and per lane one
//     float4 (d8 of its two blocks, d8 * (sum of each block's codes)); when
//     the row does not fit the LDS budget it is staged in chunks of whole
//     passes;
//   * integer dots with v_dot4_i32_i8 (4-bit codes are non-negative bytes),
//     one 32-value dot A_j per sub-block and column, then per lane
//     acc += (d*sc_j) * (A_j*d8_j) - (dmin*m_j) * (d8_j*Bq_j) in f32, with
//     d*sc_j and dmin*m_j formed once per row (exact: f16 times a six-bit
//     integer); the minimum term uses the q8 codes (leone-cuda "CUDA kernel
//     design": minimum correction formed from the same lane-local codes);
//   * one fixed xor-butterfly over the 32 lanes of a row per batch column,
//     then the optional residual is added when the row is written
//     (leone-cuda "CUDA kernel design": residual epilogue, same f32 addition
//     as the separate add it replaces).
// No atomics; the reduction order is fixed, so results are bitwise
// reproducible.
#include "kq_device.h"

#include <algorithm>

namespace kq {
namespace gemv4 {

struct Slice {      // one lane's share of one superblock of one row
    uint4 hdr;      // d, dmin, 12 scale bytes
    uint4 qa;       // code bytes [32t, 32t+16)
    uint4 qb;       // code bytes [32t+16, 32t+32)
};

// LDS layout of a staged activation (schunk superblocks, BATCH columns): one
// block of lds_per_sb(BATCH) bytes per superblock sb, holding
//   codes [BATCH][256]    column b's 256 q8 codes; 16-byte unit u (values
//                         16u..16u+15) stored at unit u ^ (sb & 3); lane t
//                         reads units 4t .. 4t+3 (blocks 2t, 2t+1);
//   dz    [DZ][4]         float4 per (column, lane t): d8 of blocks 2t and
//                         2t+1, then d8 * (sum of the block's 32 codes) for
//                         each; DZ = BATCH rounded up to an odd count.
// Every column and dz offset is then a compile-time immediate from one base
// per lane and pass.  The sixteen lanes that one LDS cycle serves are four
// lanes t of each of superblocks sb .. sb+3 (sb a multiple of 4).  The block
// stride is an odd multiple of 64 bytes modulo 256, so for the codes the
// xor puts the four superblocks on different low unit bits and t on the
// high ones, and for dz the superblocks land on different 64-byte quarters:
// either way sixteen distinct 16-byte bank groups.
constexpr int lds_dz_cols(int batch) { return batch + ((batch & 1) ? 0 : 1); }
constexpr int lds_per_sb(int batch) { return batch * 256 + lds_dz_cols(batch) * 64; }

__device__ __forceinline__ int swz(int sb) { return sb & 3; }

// Staging of blocks [j0, j0 + nbc) of every column (j0, nbc multiples of 8),
// U items per thread per round, in one of two forms:
//   * BATCH >= 4: an item is a (column, run of 4 q8_1 blocks).  A run is 144
//     bytes and starts 16-byte aligned (xq is 16-byte aligned, a column is
//     288 * S bytes, j0 a multiple of 8), so it comes in nine 16-byte loads
//     whose dwords are its four blocks, and the lane's d8 values leave in
//     two float4 writes;
//   * fewer columns: an item is one (column, block), nine dword loads.  The
//     code words of a run's blocks sit at odd dword offsets of its load
//     registers and must be copied into aligned quads for the 16-byte LDS
//     writes; the small-batch kernels cannot spare those registers (batch 1:
//     59 -> 102 VGPRs), and a small batch has little to stage.
// A round is split into the issue of its global loads (into StageRegs) and
// the LDS writes, so a kernel can issue the first round's loads before its
// weight loads: loads complete in issue order, and activation loads issued
// after the weight ring would have to wait for the weights' HBM latency
// before the staging could finish.
template <int BATCH>
constexpr bool stage_runs() { return BATCH >= 4; }

template <int BATCH>
__device__ __forceinline__ int stage_items(int nbc) { return stage_runs<BATCH>() ? BATCH * (nbc >> 2) : BATCH * nbc; }

template <int BATCH, int U>
struct StageRegs {
    uint4 q[stage_runs<BATCH>() ? U : 1][9];    // runs
    uint32_t c[stage_runs<BATCH>() ? 1 : U][9];  // single blocks
};

// Column of item `idx` (n items per column), without a division.
template <int BATCH>
__device__ __forceinline__ int column_of(int idx, int n) {
    int bb = 0;
#pragma unroll
    for (int c = 1; c < BATCH; ++c) bb += idx >= c * n ? 1 : 0;
    return bb;
}

__device__ __forceinline__ uint32_t word_of(const uint4 (&c)[9], int w) {   // w a constant
    const uint4 v = c[w >> 2];
    return (w & 3) == 0 ? v.x : (w & 3) == 1 ? v.y : (w & 3) == 2 ? v.z : v.w;
}

template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_issue(StageRegs<BATCH, U>& r, const uint8_t* __restrict__ xq,
                                            int nb_row, int j0, int nbc, int base) {
    constexpr bool runs = stage_runs<BATCH>();
    const int per_col = runs ? nbc >> 2 : nbc;
    const int total = BATCH * per_col;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int idx = base + i * NT + (int)threadIdx.x;
        if (idx < total) {
            const int bb = column_of<BATCH>(idx, per_col);
            const int j = idx - bb * per_col;
            if constexpr (runs) {
                const uint8_t* run = xq + ((int64_t)bb * nb_row + j0 + 4 * j) * kQ81Bytes;
#pragma unroll
                for (int e = 0; e < 9; ++e) r.q[i][e] = load16(run + 16 * e);
            } else {
                const uint32_t* blk = (const uint32_t*)(xq + ((int64_t)bb * nb_row + j0 + j) * kQ81Bytes);
#pragma unroll
                for (int e = 0; e < 9; ++e) r.c[i][e] = blk[e];
            }
        }
    }
}

// Codes and d8 values of block jj (0..7) of superblock sb, column bb; the
// block's nine words come from `word(0..8)` (d|s word, then the 8 code words).
template <int BATCH, class Word>
__device__ __forceinline__ void stage_block(uint8_t* lds, int bb, int sb, int jj, Word word,
                                            float& d8, float& z) {
    uint8_t* cs = lds + sb * lds_per_sb(BATCH) + bb * 256;
    const int x = swz(sb);
    d8 = half_bits_to_float(word(0));
    int sq = 0;
#pragma unroll
    for (int u = 1; u <= 8; ++u) sq = dot4(word(u), 0x01010101u, sq);
    z = d8 * (float)sq;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        *(uint4*)(cs + 16 * ((2 * jj + h) ^ x)) =
            make_uint4(word(1 + 4 * h), word(2 + 4 * h), word(3 + 4 * h), word(4 + 4 * h));
}

template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_write(const StageRegs<BATCH, U>& r, int nbc, int base,
                                            uint8_t* lds) {
    constexpr bool runs = stage_runs<BATCH>();
    const int per_col = runs ? nbc >> 2 : nbc;
    const int total = BATCH * per_col;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int idx = base + i * NT + (int)threadIdx.x;
        if (idx < total) {
            const int bb = column_of<BATCH>(idx, per_col);
            const int j = idx - bb * per_col;
            if constexpr (runs) {
                const int sb = j >> 1, hq = j & 1;   // blocks 4hq .. 4hq+3 of superblock sb
                float v[2][4];                       // lanes 2hq, 2hq+1
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    stage_block<BATCH>(lds, bb, sb, 4 * hq + e,
                                       [&](int u) { return word_of(r.q[i], 9 * e + u); },
                                       v[e >> 1][e & 1], v[e >> 1][2 + (e & 1)]);
                float4* dp = (float4*)(lds + sb * lds_per_sb(BATCH) + BATCH * 256) + bb * 4 + 2 * hq;
                dp[0] = make_float4(v[0][0], v[0][1], v[0][2], v[0][3]);
                dp[1] = make_float4(v[1][0], v[1][1], v[1][2], v[1][3]);
            } else {
                const int sb = j >> 3, jj = j & 7;
                float d8, z;
                stage_block<BATCH>(lds, bb, sb, jj, [&](int u) { return r.c[i][u]; }, d8, z);
                float* dp = (float*)(lds + sb * lds_per_sb(BATCH) + BATCH * 256) + (bb * 4 + (jj >> 1)) * 4;
                dp[jj & 1] = d8;
                dp[2 + (jj & 1)] = z;
            }
        }
    }
}

// The rest of a staging whose first round was issued into r: its LDS writes,
// every later round, and the closing barrier.
template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_finish(StageRegs<BATCH, U>& r, const uint8_t* __restrict__ xq,
                                             int nb_row, int j0, int nbc, uint8_t* lds) {
    stage_write<BATCH, NT, U>(r, nbc, 0, lds);
    for (int base = NT * U; base < stage_items<BATCH>(nbc); base += NT * U) {
        stage_issue<BATCH, NT, U>(r, xq, nb_row, j0, nbc, base);
        stage_write<BATCH, NT, U>(r, nbc, base, lds);
    }
    __syncthreads();
}

// A whole staging (all loads of a round in flight before any is used).
template <int BATCH, int NT, int U>
__device__ __forceinline__ void stage_activation(const uint8_t* __restrict__ xq, int nb_row,
                                                 int j0, int nbc, uint8_t* lds) {
    StageRegs<BATCH, U> r;
    stage_issue<BATCH, NT, U>(r, xq, nb_row, j0, nbc, 0);
    stage_finish<BATCH, NT, U>(r, xq, nb_row, j0, nbc, lds);
}

template <int RPW>
__device__ __forceinline__ void load_pass(Slice (&s)[RPW], const uint8_t* const (&rowp)[RPW],
                                          int sb, int S, int t) {
    const int sbc = min(sb, S - 1);  // lanes past the row end reload a valid superblock
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const uint8_t* p = rowp[i] + sbc * kQ4KBytes;
        s[i].hdr = load16(p);
        s[i].qa = load16(p + 16 + 32 * t);
        s[i].qb = load16(p + 32 + 32 * t);
    }
}

__device__ __forceinline__ int dot16(uint4 w, uint4 a, int c) {
    return dot4(w.w, a.w, dot4(w.z, a.z, dot4(w.y, a.y, dot4(w.x, a.x, c))));
}

__device__ __forceinline__ uint4 lo_nibbles(uint4 q) {
    return make_uint4(q.x & 0x0f0f0f0fu, q.y & 0x0f0f0f0fu, q.z & 0x0f0f0f0fu, q.w & 0x0f0f0f0fu);
}

__device__ __forceinline__ uint4 hi_nibbles(uint4 q) {
    return make_uint4((q.x >> 4) & 0x0f0f0f0fu, (q.y >> 4) & 0x0f0f0f0fu, (q.z >> 4) & 0x0f0f0f0fu,
                      (q.w >> 4) & 0x0f0f0f0fu);
}

template <int BATCH, int RPW>
__device__ __forceinline__ void compute_pass(const Slice (&s)[RPW], float (&acc)[RPW][BATCH],
                                             const uint8_t* lds, int sl, int t) {
    // six-bit fields of sub-blocks j = 2t, 2t+1 (byte e = 2(t%2) + {0,1} of
    // a scale word): j < 4 -> scale = bits 0..5 of byte e of bytes 0..3, min
    // = the same of bytes 4..7; j >= 4 -> scale = low nibble of byte 8+e
    // with bits 6..7 of byte e above it, min = high nibble of byte 8+e with
    // bits 6..7 of byte 4+e
    const bool hi = t >= 2;
    const uint32_t p0 = 16u * (uint32_t)(t & 1);
    const uint32_t wl = hi ? 4u : 6u, wh = hi ? 2u : 0u, mo = hi ? 4u : 0u;
    float ds0[RPW], ds1[RPW], dm0[RPW], dm1[RPW];
    uint4 la[RPW], lb[RPW], ha[RPW], hb[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const uint4 hdr = s[i].hdr;
        const float d = half_bits_to_float(hdr.x);
        const float dmin = half_bits_to_float(hdr.x >> 16);
        const uint32_t ws = hi ? hdr.w : hdr.y, wm = hi ? hdr.w : hdr.z;
        const uint32_t sc0 = __builtin_amdgcn_ubfe(ws, p0, wl) | (__builtin_amdgcn_ubfe(hdr.y, p0 + 6, wh) << 4);
        const uint32_t sc1 = __builtin_amdgcn_ubfe(ws, p0 + 8, wl) | (__builtin_amdgcn_ubfe(hdr.y, p0 + 14, wh) << 4);
        const uint32_t m0 = __builtin_amdgcn_ubfe(wm, p0 + mo, wl) | (__builtin_amdgcn_ubfe(hdr.z, p0 + 6, wh) << 4);
        const uint32_t m1 = __builtin_amdgcn_ubfe(wm, p0 + 8 + mo, wl) | (__builtin_amdgcn_ubfe(hdr.z, p0 + 14, wh) << 4);
        ds0[i] = d * (float)sc0;
        ds1[i] = d * (float)sc1;
        dm0[i] = dmin * (float)m0;
        dm1[i] = dmin * (float)m1;
        la[i] = lo_nibbles(s[i].qa);
        lb[i] = lo_nibbles(s[i].qb);
        ha[i] = hi_nibbles(s[i].qa);
        hb[i] = hi_nibbles(s[i].qb);
    }
    // then one column at a time: its activation slice of this lane (units
    // 4t .. 4t+3 and the d8 float4), used by every row
    const uint8_t* cs = lds + sl * lds_per_sb(BATCH) + 64 * t;
    const float4* dz = (const float4*)(lds + sl * lds_per_sb(BATCH) + BATCH * 256) + t;
    const int x = swz(sl);
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
        uint4 a[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = *(const uint4*)(cs + 16 * (r ^ x) + b * 256);
        const float4 z = dz[4 * b];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int A0 = dot16(lb[i], a[1], dot16_z(la[i], a[0]));
            const int A1 = dot16(hb[i], a[3], dot16_z(ha[i], a[2]));
            float v = acc[i][b];
            v = fmaf(ds0[i], (float)A0 * z.x, v);
            v = fmaf(ds1[i], (float)A1 * z.y, v);
            v = fmaf(-dm0[i], z.z, v);
            v = fmaf(-dm1[i], z.w, v);
            acc[i][b] = v;
        }
    }
}

// Sum over the 32 lanes of a half-wavefront (fixed xor-butterfly order).
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Row pointers of row group g for this lane (rows past m are clamped: they
// are computed, not stored).
template <int RPW>
__device__ __forceinline__ void group_rows(const uint8_t* (&rowp)[RPW], const uint8_t* w, int g,
                                           int waves, int wave, int half, int m,
                                           int64_t row_bytes) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = min(2 * ((g * waves + wave) * RPW + i) + half, m - 1);
        rowp[i] = w + (int64_t)r * row_bytes;
    }
}

// Half-wavefront sums of the accumulators, residual add and store (lane 0 of
// each half), then reset.
template <int BATCH, int RPW>
__device__ __forceinline__ void finish_rows(float (&acc)[RPW][BATCH], float* y,
                                            const float* residual, int pair0, int half, int lane,
                                            int m) {
    // the columns of a row in one transposing butterfly over its half
    // wavefront: lane 32b/NB of the half holds column b
    constexpr int NB = pow2_ceil(BATCH);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = 2 * (pair0 + i) + half;
        float v[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) v[b] = b < BATCH ? acc[i][b] : 0.0f;
        const float t = lane_sums<NB, 32>(v, lane);
        const int l = lane & 31, b = l / (32 / NB);
        if (l % (32 / NB) == 0 && b < BATCH && r < m) {
            const int64_t o = (int64_t)b * m + r;
            y[o] = residual ? residual[o] + t : t;
        }
#pragma unroll
        for (int bb = 0; bb < BATCH; ++bb) acc[i][bb] = 0.0f;
    }
}

// Weight tensors of one persistent launch: segment s has m[s] rows, weights
// w[s], output y[s] and residual res[s] (or null); its row groups are
// g0[s] .. g0[s+1]-1 of the launch.  All segments share the q8_1 activation,
// k and the batch (leone-cuda "CUDA kernel design": QKV, and gate with up,
// share one quantisation; cajeta "One model, start to last token" 4: the
// paired q|k|v and gate|up launches).
struct Segs {
    int ngroups, n;
    int g0[kMaxSegs + 1];
    int m[kMaxSegs];
    const uint8_t* w[kMaxSegs];
    float* y[kMaxSegs];
    const float* res[kMaxSegs];
};

// The one-tensor launch: a table of one row, kept small so the kernel reads
// it with a few independent scalar loads.
struct Seg1 {
    const uint8_t* w;
    float* y;
    const float* res;
    int m, ngroups;
};

// Position in the segment table of a stream of increasing row groups; it
// advances only when a segment boundary is crossed, so the table is read once
// per segment, not once per group.
struct SegCursor {
    int s, g0, g1, m;
    const uint8_t* w;
    float* y;
    const float* res;
};

__device__ __forceinline__ void seg_seek(SegCursor& c, const Segs& sg, int g) {
    while (g >= c.g1 && c.s + 1 < sg.n) {
        ++c.s;
        c.g0 = sg.g0[c.s];
        c.g1 = sg.g0[c.s + 1];
        c.m = sg.m[c.s];
        c.w = sg.w[c.s];
        c.y = sg.y[c.s];
        c.res = sg.res[c.s];
    }
}
__device__ __forceinline__ void seg_seek(SegCursor&, const Seg1&, int) {}

__device__ __forceinline__ SegCursor seg_start(const Segs& sg, int g) {
    SegCursor c{0, sg.g0[0], sg.g0[1], sg.m[0], sg.w[0], sg.y[0], sg.res[0]};
    seg_seek(c, sg, g);
    return c;
}
__device__ __forceinline__ SegCursor seg_start(const Seg1& t, int) {
    return SegCursor{0, 0, t.ngroups, t.m, t.w, t.y, t.res};
}

// One workgroup per WAVES*RPW row pairs; every workgroup stages the
// activation (in chunks when it exceeds the LDS budget).
template <int BATCH, int RPW, int DEPTH, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_q4k_kernel(const uint8_t* __restrict__ w,
                                                              const uint8_t* __restrict__ xq,
                                                              float* y, const float* residual,
                                                              int m, int S, int schunk) {
    extern __shared__ __align__(16) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int grp = (lane >> 2) & 7;   // superblock within a pass
    const int t = lane & 3;            // slice pair within the superblock
    const int64_t row_bytes = (int64_t)S * kQ4KBytes;
    const int nb_row = S * 8;
    const int npass = (S + 7) >> 3;

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    Slice ring[DEPTH][RPW];
    const uint8_t* rowp[RPW];
    const int pair0 = (blockIdx.x * WAVES + wave) * RPW;   // first row pair of this wave
    const int chunk_passes = schunk >> 3;   // schunk is a multiple of 8 superblocks
    constexpr int U = stage_runs<BATCH>() ? 1 : (BATCH == 1 ? 2 : 4);
    StageRegs<BATCH, U> sr;   // the activation loads go first (see stage_issue)
    stage_issue<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, min(schunk, S) * 8, 0);
    group_rows<RPW>(rowp, w, blockIdx.x, WAVES, wave, half, m, row_bytes);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_pass<RPW>(ring[d], rowp, 8 * d + grp, S, t);
    __builtin_amdgcn_sched_barrier(0);   // keep the staging arithmetic after the weight loads
    stage_finish<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, min(schunk, S) * 8, smem);

    for (int p0 = 0; p0 < npass; p0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int p = p0 + d;
            if (p < npass) {
                const int chunk = p / chunk_passes;
                const int pl = p - chunk * chunk_passes;   // pass within the staged chunk
                if (pl == 0 && p > 0) {                    // uniform over the workgroup
                    __syncthreads();
                    const int kc = chunk * schunk;
                    stage_activation<BATCH, 64 * WAVES, U>(xq, nb_row, kc * 8,
                                                        min(schunk, S - kc) * 8, smem);
                }
                if (8 * p + grp < S)   // lanes past the row end add nothing
                    compute_pass<BATCH, RPW>(ring[d], acc, smem, 8 * pl + grp, t);
                if (p + DEPTH < npass)
                    load_pass<RPW>(ring[d], rowp, 8 * (p + DEPTH) + grp, S, t);
            }
        }
    }
    finish_rows<BATCH, RPW>(acc, y, residual, pair0, half, lane, m);
}

// K split over two wavefronts per row pair (the whole activation staged in
// one piece): wavefront w of the first WH takes passes [0, np2) of its row
// pair, wavefront WH + w the passes [np2, npass) of the same pair.  The second
// half's row sums go through LDS and are added to the first half's in that
// order, so results are deterministic.  With one activation piece per
// workgroup limited by LDS, this doubles the wavefronts streaming weights.
// One pass is in flight per wavefront: requesting all of a wavefront's
// passes together with the staging was slower (the staging and the barrier
// then finish behind the weight loads, and the passes run back to back).
template <int BATCH, int RPW, int WH>
__global__ __launch_bounds__(128 * WH) void gemv_q4k_ksplit(const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ xq,
                                                            float* y, const float* residual,
                                                            int m, int S, int schunk) {
    extern __shared__ __align__(16) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kh = wave / WH, wv = wave - kh * WH;   // K half, wavefront within the half
    const int half = lane >> 5;
    const int grp = (lane >> 2) & 7;
    const int t = lane & 3;
    const int64_t row_bytes = (int64_t)S * kQ4KBytes;
    const int nb_row = S * 8;
    const int npass = (S + 7) >> 3;
    const int np2 = (npass + 1) >> 1;
    const int pbeg = kh * np2, pend = min(npass, pbeg + np2);

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    const int pair0 = (blockIdx.x * WH + wv) * RPW;
    Slice ring[RPW];
    const uint8_t* rowp[RPW];
    constexpr int U = stage_runs<BATCH>() ? 1 : 2;
    StageRegs<BATCH, U> sr;   // the activation loads go first (see stage_issue)
    stage_issue<BATCH, 128 * WH, U>(sr, xq, nb_row, 0, S * 8, 0);
    group_rows<RPW>(rowp, w, blockIdx.x, WH, wv, half, m, row_bytes);
    load_pass<RPW>(ring, rowp, 8 * pbeg + grp, S, t);   // unconditional (clamped): no merge
    __builtin_amdgcn_sched_barrier(0);   // keep the staging arithmetic after the weight loads
    stage_finish<BATCH, 128 * WH, U>(sr, xq, nb_row, 0, S * 8, smem);

    for (int p = pbeg; p < pend; ++p) {
        if (8 * p + grp < S)   // lanes past the row end add nothing
            compute_pass<BATCH, RPW>(ring, acc, smem, 8 * p + grp, t);
        if (p + 1 < pend) load_pass<RPW>(ring, rowp, 8 * (p + 1) + grp, S, t);
    }

    float* red = (float*)(smem + (size_t)schunk * lds_per_sb(BATCH));   // [WH*RPW*2][BATCH]
    float v[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) v[i][b] = half_wave_sum(acc[i][b]);
    if (kh == 1 && (lane & 31) == 0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int b = 0; b < BATCH; ++b) red[((wv * RPW + i) * 2 + half) * BATCH + b] = v[i][b];
    }
    __syncthreads();
    if (kh == 0 && (lane & 31) == 0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = 2 * (pair0 + i) + half;
            if (r < m) {
#pragma unroll
                for (int b = 0; b < BATCH; ++b) {
                    const float sum = v[i][b] + red[((wv * RPW + i) * 2 + half) * BATCH + b];
                    const int64_t o = (int64_t)b * m + r;
                    y[o] = residual ? residual[o] + sum : sum;
                }
            }
        }
    }
}

// Persistent form (the whole activation fits in LDS): a grid of a few
// workgroups per compute unit stages the activation once and walks the row
// groups blockIdx.x, blockIdx.x + gridDim.x, ... of all segments; the load
// ring runs on across group (and segment) boundaries, so the memory pipe never
// drains between them.
template <int BATCH, int RPW, int DEPTH, int WAVES, class Tab>
__global__ __launch_bounds__(64 * WAVES) void gemv_q4k_persistent(const Tab sg,
                                                                  const uint8_t* __restrict__ xq,
                                                                  int S, int schunk) {
    extern __shared__ __align__(16) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int grp = (lane >> 2) & 7;
    const int t = lane & 3;
    const int64_t row_bytes = (int64_t)S * kQ4KBytes;
    const int nb_row = S * 8;
    const int npass = (S + 7) >> 3;
    const int ngroups = sg.ngroups;
    const int nitems = ((ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x) * npass;

    float acc[RPW][BATCH];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int b = 0; b < BATCH; ++b) acc[i][b] = 0.0f;

    Slice ring[DEPTH][RPW];
    const uint8_t* rowp[RPW];
    // (group, pass) of the next item to load and of the next to compute
    int gl = blockIdx.x, pl = 0;
    constexpr int U = stage_runs<BATCH>() ? 1 : 2;
    StageRegs<BATCH, U> sr;   // the activation loads go first (see stage_issue)
    stage_issue<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, S * 8, 0);
    SegCursor cl = seg_start(sg, gl);
    auto rows_of = [&](int g) {
        seg_seek(cl, sg, g);
        group_rows<RPW>(rowp, cl.w, g - cl.g0, WAVES, wave, half, cl.m, row_bytes);
    };
    rows_of(gl);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (d == 0 || d < nitems) {   // nitems >= 1: the grid has at most one workgroup per group
            load_pass<RPW>(ring[d], rowp, 8 * pl + grp, S, t);
            if (++pl == npass) {
                pl = 0;
                gl += gridDim.x;
                if (gl < ngroups) rows_of(gl);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the staging arithmetic after the weight loads
    stage_finish<BATCH, 64 * WAVES, U>(sr, xq, nb_row, 0, S * 8, smem);
    int gc = blockIdx.x, pc = 0;
    SegCursor cc = seg_start(sg, gc);
    for (int it0 = 0; it0 < nitems; it0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int it = it0 + d;
            if (it < nitems) {
                if (8 * pc + grp < S)   // lanes past the row end add nothing
                    compute_pass<BATCH, RPW>(ring[d], acc, smem, 8 * pc + grp, t);
                if (it + DEPTH < nitems) {
                    load_pass<RPW>(ring[d], rowp, 8 * pl + grp, S, t);
                    if (++pl == npass) {
                        pl = 0;
                        gl += gridDim.x;
                        if (gl < ngroups) rows_of(gl);
                    }
                }
                if (++pc == npass) {
                    seg_seek(cc, sg, gc);
                    finish_rows<BATCH, RPW>(acc, cc.y, cc.res, ((gc - cc.g0) * WAVES + wave) * RPW,
                                            half, lane, cc.m);
                    pc = 0;
                    gc += gridDim.x;
                }
            }
        }
    }
}

// Persistent launch over the row groups of table `tab` (one tensor or a
// segment table).
template <int BATCH, int RPW, int DEPTH, int WAVES, class Tab>
hipError_t launch_persistent(const Tab& tab, const void* xq, int64_t k, int schunk, size_t lds,
                             int cus, int per_cu, hipStream_t stream) {
    if (tab.ngroups == 0) return hipSuccess;
    auto kern = gemv_q4k_persistent<BATCH, RPW, DEPTH, WAVES, Tab>;
    const int o = occupancy((const void*)kern, 64 * WAVES, lds);
    const int grid = std::min(tab.ngroups, cus * std::min(o, per_cu));
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WAVES), lds, stream, tab,
                       (const uint8_t*)xq, (int)(k / kQK), schunk);
    return hipGetLastError();
}

// K-split launch (the whole activation in one piece of at most lds_limit).
template <int BATCH, int RPW, int WH>
size_t ksplit_lds(int64_t k) {
    const int S = (int)(k / kQK);
    return (size_t)((S + 7) & ~7) * lds_per_sb(BATCH) + (size_t)WH * RPW * 2 * BATCH * 4;
}

template <int BATCH, int RPW, int WH>
hipError_t launch_ksplit(const void* w, const void* xq, float* y, const float* residual,
                         int64_t m, int64_t k, int lds_limit, hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int schunk = (S + 7) & ~7;
    const size_t lds = ksplit_lds<BATCH, RPW, WH>(k);
    if (lds > (size_t)lds_limit) return hipErrorInvalidConfiguration;
    const int64_t ngroups = (m + WH * RPW * 2 - 1) / (WH * RPW * 2);
    hipLaunchKernelGGL((gemv_q4k_ksplit<BATCH, RPW, WH>), dim3((unsigned)ngroups), dim3(128 * WH),
                       lds, stream, (const uint8_t*)w, (const uint8_t*)xq, y, residual, (int)m, S,
                       schunk);
    return hipGetLastError();
}

// LDS chunk (superblocks per staged piece) of a batch under a budget; 0 if
// not even one pass fits.
template <int BATCH>
int chunk_for(int64_t k, int lds_budget) {
    const int S = (int)(k / kQK);
    int schunk = (lds_budget / lds_per_sb(BATCH)) & ~7;      // whole passes of 8 superblocks
    const int s_round = (S + 7) & ~7;
    if (schunk > s_round) schunk = s_round;
    return schunk < 8 ? 0 : schunk;
}

// Launch one variant on one weight tensor.  `persist_per_cu` > 0 asks for the
// persistent form with that many workgroups per compute unit (capped by
// occupancy); it is used only when the whole activation fits in one LDS
// piece.
template <int BATCH, int RPW, int DEPTH, int WAVES>
hipError_t launch_variant(const void* w, const void* xq, float* y, const float* residual,
                          int64_t m, int64_t k, int lds_budget, int cus, int persist_per_cu,
                          hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int schunk = chunk_for<BATCH>(k, lds_budget);
    if (schunk == 0) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)schunk * lds_per_sb(BATCH);
    if (persist_per_cu > 0 && schunk >= S) {
        const int rows_per_group = WAVES * RPW * 2;
        const Seg1 tab{(const uint8_t*)w, y, residual, (int)m,
                       (int)((m + rows_per_group - 1) / rows_per_group)};
        return launch_persistent<BATCH, RPW, DEPTH, WAVES>(tab, xq, k, schunk, lds, cus,
                                                           persist_per_cu, stream);
    }
    const int rows_per_block = WAVES * RPW * 2;
    const int64_t ngroups = (m + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_q4k_kernel<BATCH, RPW, DEPTH, WAVES>), dim3((unsigned)ngroups),
                       dim3(64 * WAVES), lds, stream, (const uint8_t*)w, (const uint8_t*)xq, y,
                       residual, (int)m, S, schunk);
    return hipGetLastError();
}

}  // namespace gemv4

namespace gemv4 {
// Batches 5..8 (decode of several sequences): the persistent four-wavefront
// form when the activation fits in 64 KB of LDS, else the chunked form with
// one pass in flight over eight wavefronts.
template <int B>
hipError_t wide(const void* w, const void* xq, float* y, const float* residual, int64_t m,
                int64_t k, int64_t whole, int one_piece, int cus, hipStream_t stream) {
    return whole > 65536 ? launch_variant<B, 1, 1, 8>(w, xq, y, residual, m, k, one_piece, cus, 0, stream)
                         : launch_variant<B, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
}
}  // namespace gemv4

hipError_t launch_gemv_q4k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream) {
    using namespace gemv4;
    // Launch shapes chosen by measurement on MI355X (back-to-back launches
    // over enough rotating weight copies that every launch streams from HBM,
    // Llama-3-8B decode shapes).  Batch 1: one row pair per wavefront, one
    // pass ahead, persistent grid -- eight wavefronts and three workgroups
    // per CU for tall or long rows (gate|up 28672x4096), else four
    // wavefronts and four workgroups (4096x4096); two or three passes ahead
    // were slower on all three.  Long rows with too few row pairs to occupy
    // that grid (down 4096x14336: 2048 pairs of 7 passes for 6144
    // wavefronts) take the K split instead, two wavefronts per row pair
    // (8.5 against 9.0 us; three or four per pair: 8.6-10.3 us).
    // Batches 2-4 use the four-wavefront persistent form (QKV 6144x4096 at
    // batch 4) unless the activation needs more than 64 KB of LDS: at batch 4
    // the K split when the whole activation still fits one workgroup's LDS
    // (down 4096x14336), else one pass in flight over eight wavefronts per
    // row group, staged in pieces.
    const int S = (int)(k / kQK);
    const int64_t s_round = (S + 7) & ~7;
    const int64_t whole = (int64_t)lds_per_sb(batch) * s_round;
    const int one_piece = whole <= lds_limit ? lds_limit : 65536;
    const bool big = m >= 16384 || S > 16;
    const bool split1 = S >= 32 && m < 48LL * cus && ksplit_lds<1, 1, 4>(k) <= (size_t)lds_limit;
    switch (batch) {
        case 1: if (split1) return launch_ksplit<1, 1, 4>(w, xq, y, residual, m, k, lds_limit, stream);
                return big ? launch_variant<1, 1, 1, 8>(w, xq, y, residual, m, k, 65536, cus, 3, stream)
                           : launch_variant<1, 1, 1, 4>(w, xq, y, residual, m, k, 65536, cus, 4, stream);
        case 2: return launch_variant<2, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
        case 3: return launch_variant<3, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
        case 4: return whole > 65536 ? (whole + 4096 <= lds_limit
                                            ? launch_ksplit<4, 1, 8>(w, xq, y, residual, m, k, lds_limit, stream)
                                            : launch_variant<4, 1, 1, 8>(w, xq, y, residual, m, k, one_piece, cus, 0, stream))
                                     : launch_variant<4, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
        case 5: return wide<5>(w, xq, y, residual, m, k, whole, one_piece, cus, stream);
        case 6: return wide<6>(w, xq, y, residual, m, k, whole, one_piece, cus, stream);
        case 7: return wide<7>(w, xq, y, residual, m, k, whole, one_piece, cus, stream);
        case 8: return wide<8>(w, xq, y, residual, m, k, whole, one_piece, cus, stream);
        default: return hipErrorInvalidValue;
    }
}

namespace gemv4 {
// Segments of one launch: persistent when the activation fits the budget,
// else one ordinary launch per segment.
template <int BATCH, int RPW, int DEPTH, int WAVES>
hipError_t launch_segs(const Segs& sg, const void* xq, int64_t k, int lds_budget, int cus,
                       int per_cu, int lds_limit, hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int schunk = chunk_for<BATCH>(k, lds_budget);
    if (schunk >= S && schunk > 0) {
        Segs tab = sg;   // row groups of each segment, in segment order
        const int rows_per_group = WAVES * RPW * 2;
        tab.g0[0] = 0;
        for (int s = 0; s < tab.n; ++s)
            tab.g0[s + 1] = tab.g0[s] + (tab.m[s] + rows_per_group - 1) / rows_per_group;
        tab.ngroups = tab.g0[tab.n];
        return launch_persistent<BATCH, RPW, DEPTH, WAVES>(
            tab, xq, k, schunk, (size_t)schunk * lds_per_sb(BATCH), cus, per_cu, stream);
    }
    for (int s = 0; s < sg.n; ++s) {
        if (sg.m[s] == 0) continue;
        const hipError_t e = launch_gemv_q4k(sg.w[s], xq, sg.y[s], sg.res[s], sg.m[s], k, BATCH,
                                             lds_limit, cus, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // namespace gemv4

hipError_t launch_gemv_q4k_seg(int nseg, const void* const* w, const int64_t* m, float* const* y,
                               const float* const* residual, const void* xq, int64_t k, int batch,
                               int lds_limit, int cus, hipStream_t stream) {
    using namespace gemv4;
    Segs sg = {};
    sg.n = nseg;
    int64_t total = 0;
    for (int s = 0; s < nseg; ++s) {   // zero-row segments get no row groups
        sg.w[s] = (const uint8_t*)w[s];
        sg.y[s] = y[s];
        sg.res[s] = residual ? residual[s] : nullptr;
        sg.m[s] = (int)m[s];
        total += m[s];
    }
    // the single-tensor launch shapes, chosen on the launch's total rows
    const int S = (int)(k / kQK);
    const int64_t whole = (int64_t)lds_per_sb(batch) * ((S + 7) & ~7);
    const bool big = total >= 16384 || S > 16;
    const int fit = whole > 65536 ? 0 : 65536;   // 0: one ordinary launch per segment
    switch (batch) {
        case 1: return big ? launch_segs<1, 1, 1, 8>(sg, xq, k, 65536, cus, 3, lds_limit, stream)
                           : launch_segs<1, 1, 1, 4>(sg, xq, k, 65536, cus, 4, lds_limit, stream);
        case 2: return launch_segs<2, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        case 3: return launch_segs<3, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        case 4: return launch_segs<4, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        case 5: return launch_segs<5, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        case 6: return launch_segs<6, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        case 7: return launch_segs<7, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        case 8: return launch_segs<8, 1, 1, 4>(sg, xq, k, fit, cus, 6, lds_limit, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kq
