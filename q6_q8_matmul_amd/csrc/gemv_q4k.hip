// gemv_q4k.hip -- Q4_K x q8_1 matrix-vector product (decode, batch 1..4).
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
//     pass; lane t of a group loads the 16-byte code slices [16t, 16t+16) and
//     [64+16t, 64+16t+16) plus the 16-byte header, i.e. 16 values of each of
//     sub-blocks 2c, 2c+1, 2c+4, 2c+5 (c = t/2, values 16h..16h+15, h = t%2),
//     so every lane decodes the same mix of low (j < 4) and high (j >= 4)
//     six-bit fields and the code has no lane-dependent branches;
//   * the loads of the first DEPTH passes are issued before anything else and
//     every later pass is requested DEPTH passes ahead (a register ring), so
//     HBM latency overlaps the activation staging and the arithmetic;
//   * when the whole activation fits in LDS the grid is persistent: a few
//     workgroups per compute unit stage it once and walk the row groups
//     (blockIdx.x, blockIdx.x + gridDim.x, ...), and the load ring runs on
//     across row groups, so the memory pipe never drains between them;
//   * the q8_1 activation is restaged once per workgroup into LDS: per
//     superblock the 16-byte slices in the order the lanes read them, and per
//     lane the four d8 values and the four d8 * (sum of the slice's codes);
//     when the row does not fit the LDS budget it is staged in chunks of whole
//     passes;
//   * integer dots with v_dot4_i32_i8 (4-bit codes are non-negative bytes),
//     then per lane sum_j d8_j*(sc_j*A_j) and sum_j m_j*(d8_j*Bq_j) in f32 and
//     acc += d*first - dmin*second; the minimum term uses the q8 codes
//     (leone-cuda "CUDA kernel design": minimum correction formed from the
//     same lane-local codes);
//   * one fixed xor-butterfly over the 32 lanes of a row per batch column,
//     then the optional residual is added when the row is written
//     (leone-cuda "CUDA kernel design": residual epilogue, same f32 addition
//     as the separate add it replaces).
// No atomics; the reduction order is fixed, so results are bitwise
// reproducible.
#include "kq_device.h"

#include <algorithm>
#include <atomic>

namespace kq {
namespace gemv4 {

struct Slice {      // one lane's share of one superblock of one row
    uint4 hdr;      // d, dmin, 12 scale bytes
    uint4 qa;       // code bytes [16t, 16t+16)
    uint4 qb;       // code bytes [64+16t, 64+16t+16)
};

// LDS layout of one staged column (schunk superblocks):
//   codes [schunk][256]   quad 4r + t (16 bytes) = the slice lane t reads as
//                         its r-th block: r = 0, 1, 2, 3 <-> blocks 2c, 2c+1,
//                         2c+4, 2c+5, values 16h..16h+15;
//   slot  [schunk][4][8]  per lane t: d8 of its four blocks, then
//                         d8 * (sum of the slice's 16 codes) for each.
constexpr int kLdsPerSb = 256 + 4 * 8 * 4;

__device__ __forceinline__ int quad_of(int jj) {   // slice r of lane 2c (h = 0) of block jj
    const int hiA = jj >> 2, c = (jj >> 1) & 1, e = jj & 1;
    return 4 * (2 * hiA + e) + 2 * c;
}

// Stage blocks [j0, j0 + nbc) of every column (nbc a multiple of 8): one
// thread per q8_1 block, the loads of U blocks in flight before any is used.
// Ends with a barrier.
template <int BATCH, int NT>
__device__ __forceinline__ void stage_activation(const uint8_t* __restrict__ xq, int nb_row,
                                                 int j0, int nbc, int schunk, uint8_t* lds) {
    constexpr int U = 2;
    uint8_t* codes = lds;
    float* slots = (float*)(lds + BATCH * schunk * 256);
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) {
        const uint32_t* col = (const uint32_t*)(xq + ((int64_t)bb * nb_row + j0) * kQ81Bytes);
        for (int base = 0; base < nbc; base += NT * U) {
            uint32_t c[U][9];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int j = base + i * NT + (int)threadIdx.x;
                if (j < nbc) {
#pragma unroll
                    for (int e = 0; e < 9; ++e) c[i][e] = col[j * 9 + e];
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int j = base + i * NT + (int)threadIdx.x;
                if (j < nbc) {
                    const int sb = j >> 3, jj = j & 7;
                    const float d8 = half_bits_to_float(c[i][0]);
                    const int s0 = dot4(c[i][1], 0x01010101u, dot4(c[i][2], 0x01010101u,
                                   dot4(c[i][3], 0x01010101u, dot4(c[i][4], 0x01010101u, 0))));
                    const int s1 = dot4(c[i][5], 0x01010101u, dot4(c[i][6], 0x01010101u,
                                   dot4(c[i][7], 0x01010101u, dot4(c[i][8], 0x01010101u, 0))));
                    const int q0 = quad_of(jj);
                    uint8_t* cs = codes + (bb * schunk + sb) * 256 + 16 * q0;
                    *(uint4*)cs = make_uint4(c[i][1], c[i][2], c[i][3], c[i][4]);
                    *(uint4*)(cs + 16) = make_uint4(c[i][5], c[i][6], c[i][7], c[i][8]);
                    const int r = q0 >> 2, t0 = q0 & 3;   // slice index and lane (h = 0)
                    float* sl = slots + ((bb * schunk + sb) * 4 + t0) * 8;
                    sl[r] = d8;
                    sl[4 + r] = d8 * (float)s0;
                    sl[8 + r] = d8;                       // lane t0 + 1 (h = 1)
                    sl[12 + r] = d8 * (float)s1;
                }
            }
        }
    }
    __syncthreads();
}

template <int RPW>
__device__ __forceinline__ void load_pass(Slice (&s)[RPW], const uint8_t* const (&rowp)[RPW],
                                          int sb, int S, int t) {
    const int sbc = min(sb, S - 1);  // lanes past the row end reload a valid superblock
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const uint8_t* p = rowp[i] + sbc * kQ4KBytes;
        s[i].hdr = load16(p);
        s[i].qa = load16(p + 16 + 16 * t);
        s[i].qb = load16(p + 80 + 16 * t);
    }
}

__device__ __forceinline__ int dot16(uint4 w, uint4 a) {
    return dot4(w.w, a.w, dot4(w.z, a.z, dot4(w.y, a.y, dot4(w.x, a.x, 0))));
}

template <int BATCH, int RPW>
__device__ __forceinline__ void compute_pass(const Slice (&s)[RPW], float (&acc)[RPW][BATCH],
                                             const uint8_t* lds, int schunk, int sl, int t) {
    // activation slices of this lane for every column: read once, used by all rows
    const uint8_t* codes = lds;
    const float* slots = (const float*)(lds + BATCH * schunk * 256);
    uint4 a[BATCH][4];
    float4 d8v[BATCH], dbq[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
        const uint8_t* cs = codes + (b * schunk + sl) * 256 + 16 * t;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[b][r] = *(const uint4*)(cs + 64 * r);
        const float4* sp = (const float4*)(slots + ((b * schunk + sl) * 4 + t) * 8);
        d8v[b] = sp[0];
        dbq[b] = sp[1];
    }
    const uint32_t sh = 16u * (uint32_t)(t >> 1);   // byte 2c of the scale words
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const uint4 hdr = s[i].hdr;
        const float d = half_bits_to_float(hdr.x);
        const float dmin = half_bits_to_float(hdr.x >> 16);
        // six-bit scales/mins: j = 2c, 2c+1 in the low six bits of bytes 0..3,
        // j = 2c+4, 2c+5 in the nibbles of bytes 8..11 plus the top two bits
        // of bytes 0..7
        const int sc0 = (int)__builtin_amdgcn_ubfe(hdr.y, sh, 6);
        const int sc1 = (int)__builtin_amdgcn_ubfe(hdr.y, sh + 8, 6);
        const int sc2 = (int)(__builtin_amdgcn_ubfe(hdr.w, sh, 4) | (__builtin_amdgcn_ubfe(hdr.y, sh + 6, 2) << 4));
        const int sc3 = (int)(__builtin_amdgcn_ubfe(hdr.w, sh + 8, 4) | (__builtin_amdgcn_ubfe(hdr.y, sh + 14, 2) << 4));
        const float m0 = (float)__builtin_amdgcn_ubfe(hdr.z, sh, 6);
        const float m1 = (float)__builtin_amdgcn_ubfe(hdr.z, sh + 8, 6);
        const float m2 = (float)(__builtin_amdgcn_ubfe(hdr.w, sh + 4, 4) | (__builtin_amdgcn_ubfe(hdr.z, sh + 6, 2) << 4));
        const float m3 = (float)(__builtin_amdgcn_ubfe(hdr.w, sh + 12, 4) | (__builtin_amdgcn_ubfe(hdr.z, sh + 14, 2) << 4));
        const uint4 qa = s[i].qa, qb = s[i].qb;
        const uint4 w0 = make_uint4(qa.x & 0x0f0f0f0fu, qa.y & 0x0f0f0f0fu, qa.z & 0x0f0f0f0fu, qa.w & 0x0f0f0f0fu);
        const uint4 w1 = make_uint4((qa.x >> 4) & 0x0f0f0f0fu, (qa.y >> 4) & 0x0f0f0f0fu,
                                    (qa.z >> 4) & 0x0f0f0f0fu, (qa.w >> 4) & 0x0f0f0f0fu);
        const uint4 w2 = make_uint4(qb.x & 0x0f0f0f0fu, qb.y & 0x0f0f0f0fu, qb.z & 0x0f0f0f0fu, qb.w & 0x0f0f0f0fu);
        const uint4 w3 = make_uint4((qb.x >> 4) & 0x0f0f0f0fu, (qb.y >> 4) & 0x0f0f0f0fu,
                                    (qb.z >> 4) & 0x0f0f0f0fu, (qb.w >> 4) & 0x0f0f0f0fu);
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int A0 = dot16(w0, a[b][0]), A1 = dot16(w1, a[b][1]);
            const int A2 = dot16(w2, a[b][2]), A3 = dot16(w3, a[b][3]);
            float f = (float)__mul24(A0, sc0) * d8v[b].x;
            f += (float)__mul24(A1, sc1) * d8v[b].y;
            f += (float)__mul24(A2, sc2) * d8v[b].z;
            f += (float)__mul24(A3, sc3) * d8v[b].w;
            float g = m0 * dbq[b].x;
            g += m1 * dbq[b].y;
            g += m2 * dbq[b].z;
            g += m3 * dbq[b].w;
            acc[i][b] += d * f - dmin * g;
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
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = 2 * (pair0 + i) + half;
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const float v = half_wave_sum(acc[i][b]);
            if ((lane & 31) == 0 && r < m) {
                const int64_t o = (int64_t)b * m + r;
                y[o] = residual ? residual[o] + v : v;
            }
            acc[i][b] = 0.0f;
        }
    }
}

// PERSIST = false: one workgroup per WAVES*RPW row pairs, every workgroup
// stages the activation (in chunks if needed).
// PERSIST = true (only when the whole activation fits in LDS): a grid of a
// few workgroups per compute unit stages it once and walks the row groups
// blockIdx.x, blockIdx.x + gridDim.x, ...; the load ring runs across group
// boundaries.
template <int BATCH, int RPW, int DEPTH, int WAVES, bool PERSIST>
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
    if constexpr (PERSIST) {
        const int pairs_per_group = WAVES * RPW;
        const int ngroups = (m + 2 * pairs_per_group - 1) / (2 * pairs_per_group);
        const int nitems = ((ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x) * npass;
        // (group, pass) of the next item to load and of the next to compute
        int gl = blockIdx.x, pl = 0;
        group_rows<RPW>(rowp, w, gl, WAVES, wave, half, m, row_bytes);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (d < nitems) {
                load_pass<RPW>(ring[d], rowp, 8 * pl + grp, S, t);
                if (++pl == npass) {
                    pl = 0;
                    gl += gridDim.x;
                    group_rows<RPW>(rowp, w, gl, WAVES, wave, half, m, row_bytes);
                }
            }
        }
        stage_activation<BATCH, 64 * WAVES>(xq, nb_row, 0, S * 8, schunk, smem);
        int gc = blockIdx.x, pc = 0;
        for (int it0 = 0; it0 < nitems; it0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int it = it0 + d;
                if (it < nitems) {
                    if (8 * pc + grp < S)   // lanes past the row end add nothing
                        compute_pass<BATCH, RPW>(ring[d], acc, smem, schunk, 8 * pc + grp, t);
                    if (it + DEPTH < nitems) {
                        load_pass<RPW>(ring[d], rowp, 8 * pl + grp, S, t);
                        if (++pl == npass) {
                            pl = 0;
                            gl += gridDim.x;
                            group_rows<RPW>(rowp, w, gl, WAVES, wave, half, m, row_bytes);
                        }
                    }
                    if (++pc == npass) {
                        finish_rows<BATCH, RPW>(acc, y, residual, (gc * WAVES + wave) * RPW, half,
                                                lane, m);
                        pc = 0;
                        gc += gridDim.x;
                    }
                }
            }
        }
    } else {
        const int pair0 = (blockIdx.x * WAVES + wave) * RPW;   // first row pair of this wave
        const int chunk_passes = schunk >> 3;   // schunk is a multiple of 8 superblocks
        group_rows<RPW>(rowp, w, blockIdx.x, WAVES, wave, half, m, row_bytes);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_pass<RPW>(ring[d], rowp, 8 * d + grp, S, t);

        stage_activation<BATCH, 64 * WAVES>(xq, nb_row, 0, min(schunk, S) * 8, schunk, smem);

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
                        stage_activation<BATCH, 64 * WAVES>(xq, nb_row, kc * 8,
                                                            min(schunk, S - kc) * 8, schunk, smem);
                    }
                    if (8 * p + grp < S)   // lanes past the row end add nothing
                        compute_pass<BATCH, RPW>(ring[d], acc, smem, schunk, 8 * pl + grp, t);
                    if (p + DEPTH < npass)
                        load_pass<RPW>(ring[d], rowp, 8 * (p + DEPTH) + grp, S, t);
                }
            }
        }
        finish_rows<BATCH, RPW>(acc, y, residual, pair0, half, lane, m);
    }
}

// Launch one variant.  `persist_per_cu` > 0 asks for the persistent form with
// that many workgroups per compute unit (capped by occupancy); it is used
// only when the whole activation fits in one LDS piece.
template <int BATCH, int RPW, int DEPTH, int WAVES>
hipError_t launch_variant(const void* w, const void* xq, float* y, const float* residual,
                          int64_t m, int64_t k, int lds_budget, int cus, int persist_per_cu,
                          hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int per_sb = BATCH * kLdsPerSb;
    int schunk = (lds_budget / per_sb) & ~7;      // whole passes of 8 superblocks
    const int s_round = (S + 7) & ~7;
    if (schunk > s_round) schunk = s_round;
    if (schunk < 8) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)schunk * per_sb;
    const int rows_per_block = WAVES * RPW * 2;
    const int64_t ngroups = (m + rows_per_block - 1) / rows_per_block;
    if (persist_per_cu > 0 && schunk >= S) {
        auto kern = gemv_q4k_kernel<BATCH, RPW, DEPTH, WAVES, true>;
        static std::atomic<int> occ{0};
        int o = occ.load(std::memory_order_relaxed);
        if (o == 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, 64 * WAVES, lds) != hipSuccess || o < 1)
                o = 1;
            occ.store(o, std::memory_order_relaxed);
        }
        const int64_t grid = std::min<int64_t>(ngroups, (int64_t)cus * std::min(o, persist_per_cu));
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WAVES), lds, stream,
                           (const uint8_t*)w, (const uint8_t*)xq, y, residual, (int)m, S, schunk);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemv_q4k_kernel<BATCH, RPW, DEPTH, WAVES, false>), dim3((unsigned)ngroups),
                       dim3(64 * WAVES), lds, stream, (const uint8_t*)w, (const uint8_t*)xq, y,
                       residual, (int)m, S, schunk);
    return hipGetLastError();
}

}  // namespace gemv4

hipError_t launch_gemv_q4k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream) {
    using namespace gemv4;
    // Launch shapes measured on MI355X (back-to-back launches over rotating
    // weight copies, Llama-3-8B decode shapes).  Batch 1: one row pair per
    // wavefront, one pass ahead, persistent grid -- eight wavefronts and three
    // workgroups per CU for tall or long rows (gate|up 28672x4096: 12.3 us,
    // down 4096x14336: 9.4 us), else four wavefronts and four workgroups
    // (4096x4096: 4.8 us).  Batches 2-4 use the four-wavefront persistent
    // form (QKV 6144x4096 at batch 4: 8.8 us) unless the activation only fits
    // in several LDS pieces or needs more than 64 KB, where three passes in
    // flight over eight wavefronts per row group work better.
    const int S = (int)(k / kQK);
    const int64_t s_round = (S + 7) & ~7;
    const int64_t whole = (int64_t)batch * kLdsPerSb * s_round;
    const int one_piece = whole <= lds_limit ? lds_limit : 65536;
    const bool big = m >= 16384 || S > 16;
    switch (batch) {
        case 1: return big ? launch_variant<1, 1, 1, 8>(w, xq, y, residual, m, k, 65536, cus, 3, stream)
                           : launch_variant<1, 1, 1, 4>(w, xq, y, residual, m, k, 65536, cus, 4, stream);
        case 2: return launch_variant<2, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
        case 3: return launch_variant<3, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
        case 4: return whole > 65536 ? launch_variant<4, 1, 3, 8>(w, xq, y, residual, m, k, one_piece, cus, 0, stream)
                                     : launch_variant<4, 1, 1, 4>(w, xq, y, residual, m, k, one_piece, cus, 6, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kq
