// mmq_q4k.hip -- Q4_K x q8_1 matrix-matrix product on the int8 matrix cores.
//
// minfer "The CUDA backend" 2.3 describes the method: the weights are never
// dequantised -- their raw block bytes are staged on chip and decoded in
// registers where the integer matrix instruction needs them; the activations
// are quantised once per call by a prepass; the integer tile product
// accumulates exactly in int32; the float scales are applied after the
// integer loop.  On gfx950 one v_mfma_i32_32x32x32_i8 covers K = 32, exactly
// one q8_1 block, so every MFMA result is the integer dot A of one (token,
// weight row, 32-block) and takes its own scales:
//     T = d8 * (D * A - Mn * Bq),  D = d*sc, Mn = dmin*m, Bq = sum of q8 codes.
//
// Epilogue without a conversion.  The MFMA accumulator starts at the bit
// pattern of 1.5*2^23, so its int32 result read as f32 is exactly
// 1.5*2^23 + A (|A| <= 15*127*32 < 2^22 keeps it in one binade).  One FMA
// with the per-row constants D and -1.5*2^23*D (exact: D has at most 17
// significant bits) gives round(D*A), and a second FMA adds its product with
// the token's d8.  Both are full-rate VALU instructions; the lane layout of
// the output (one weight row per lane, sixteen tokens per lane) makes D a
// per-lane value and d8 a per-element one, so no outer product of scales is
// formed on the matrix cores.
//
// Minimum term: sum_j m_j z_j with z = d8*Bq (exact in f32, 24 bits) split by
// truncation into three bf16 parts, so two v_mfma_f32_32x32x16_bf16 over
// 8 blocks x 3 parts give it with exact products; times -dmin it starts the
// superblock's partial.  Per-superblock partials are added to the output
// accumulator once per superblock: each output sees about 11 + k/256 f32
// roundings in sequence, whatever k is.
//
// Workgroup: 12 wavefronts (three per SIMD), 192 weight rows x 128 tokens;
// wavefront (wr, wt) owns rows 64wr..64wr+63 (two 32-row tiles) and tokens
// 32wt..32wt+31.  The K loop walks one superblock (256 values, 8 q8_1
// blocks) per step through two LDS stages:
//   * the raw bytes of step sb+1 -- 16-byte chunks of the Q4_K superblocks
//     of 192 rows, the 16-byte code halves and header dwords of 128 tokens x
//     8 q8_1 blocks -- are copied from memory straight into LDS
//     (global_load_lds) while step sb computes;
//   * a derive phase decodes each row's header once per workgroup (D and
//     -1.5*2^23*D per sub-block, m as bf16, -dmin) and each token block's
//     d8 (rewritten in place as f32) and z parts;
//   * the compute phase reads everything from LDS.
// The last tile of m or n is shifted inward to lie inside the tensor (its
// first rows or tokens repeat the previous tile's and are not stored); a
// problem smaller than one tile clamps its rows and tokens instead.  With a
// workspace, the tiles of the grid's last, partly filled round can run as
// several workgroups over K ranges (a K split), whose partial sums a second
// launch adds in a fixed order.  No atomics; results are bitwise
// reproducible.
#include "kq_device.h"

#include <algorithm>

namespace kq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int WR = 3, WT = 4;        // wavefront grid: row groups x token groups
constexpr int NWAVE = WR * WT;       // 12 wavefronts: three per SIMD
constexpr int BM = 64 * WR;          // 192 weight rows per workgroup
constexpr int BN = 32 * WT;          // 128 tokens per workgroup
constexpr int NTHR = 64 * NWAVE;     // 768 threads
constexpr int kZStride = 40;         // bf16 per token in the z plane (32 + 8 pad)
constexpr uint32_t kMagicBits = 0x4B400000u;   // 1.5 * 2^23
constexpr float kMagic = 12582912.0f;

// Raw bytes of one superblock step, written by global_load_lds, laid out so
// the compute phase's reads (32 consecutive rows or tokens, one 16-byte
// chunk each) hit distinct LDS banks and every per-block offset is an
// immediate of one per-lane base:
//   * weight code chunk c (bytes 16c..16c+15 of the 128 code bytes) of row
//     r at slot 128*(r/16) + 16*c + r%16 (sixteen rows side by side);
//   * weight headers (d, dmin, twelve scale bytes) at slot r;
//   * token code chunk c = 2j+h (q8_1 block j, half h) of token t at slot
//     17*t + c (one pad slot per token);
//   * token headers {f16 d8, f16 s} of (t, j) at dword 8*t + j.
constexpr int kXStride = 17;         // 16-byte slots per token in the code region
struct Stage {
    uint4 wc[BM * 8];
    uint4 wh[BM];
    uint4 xc[BN * kXStride];
    uint32_t xh[BN * 8];
};

struct Smem {
    Stage st[2];
    float2 dn[8][BM];        // per block j, row: D_j and -1.5*2^23*D_j
    float d8[8][BN];         // per block j, token: d8 as f32
    uint4 mb[BM];            // m_0..m_7 of the row as bf16 (exact: m < 64)
    float nd[BM];            // -dmin of the row
    uint16_t z[BN][kZStride];   // [hi x 8][mid x 8][lo x 8][0 x 8][pad]: bf16 parts of z
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
static_assert(NTHR == 4 * BM, "row headers are decoded by four threads per row");

// Copies from memory straight into LDS: lane i's bytes, read at sbase + voff,
// land at the (wavefront-uniform) LDS address + size*i.  Written as inline
// assembly so the compiler does not tie every later LDS read to these
// copies: it cannot tell the two stages apart and would wait for the next
// step's copies before reading the current step.  The kernel waits for
// them itself (vmcnt(0) and a barrier before a stage is read).  m0 is
// written by the copies and used by nothing else in this file.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)p);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, void* lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds_addr(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* sbase, uint32_t voff, void* lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds_addr(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

// The copy instructions of a step (64 lanes each): 24 for weight codes (16
// rows x 4 chunks; 16 lanes read one chunk of 16 consecutive rows), 3 for
// weight headers (64 rows), 34 for token code slots (consecutive lanes read
// consecutive 16-byte chunks of one token; a pad slot re-reads the token's
// last chunk), 16 for token headers (8 tokens x 8 dwords).  Wavefronts 0..3
// issue them, one kind each (0: weight codes, 1 and 2: halves of the token
// codes, 3: token and weight headers): on each SIMD the oldest wavefront,
// which the arbitration favours, takes the stalls of the memory pipeline
// while the SIMD's two other wavefronts compute.  Rows and tokens beyond the
// tensor are clamped to its last row / token.
__device__ __forceinline__ void issue_stage(Stage& st, int wave, int lane, const uint8_t* w,
                                            const uint8_t* xq, int sb, int m0, int n0, int M,
                                            int N, int S) {
    const uint32_t xrow = (uint32_t)S * 8 * kQ81Bytes, wrow = (uint32_t)S * kQ4KBytes;
    const uint8_t* wb = w + (int64_t)sb * kQ4KBytes;
    const uint8_t* xb = xq + (int64_t)sb * (8 * kQ81Bytes);
    if (wave == 0) {
#pragma unroll 4
        for (int u = 0; u < 24; ++u) {
            const int r = 16 * (u >> 1) + (lane & 15), c = 4 * (u & 1) + (lane >> 4);
            dma16(wb, (uint32_t)min(m0 + r, M - 1) * wrow + 16 + 16 * c, &st.wc[64 * u]);
        }
    } else if (wave < 3) {
#pragma unroll 1
        for (int u = 17 * (wave - 1); u < 17 * wave; ++u) {
            const int s = 64 * u + lane;
            const int t = s / kXStride;
            const int c = min(s - kXStride * t, 15);
            dma16(xb, (uint32_t)min(n0 + t, N - 1) * xrow + kQ81Bytes * (c >> 1) + 4 + 16 * (c & 1),
                  &st.xc[64 * u]);
        }
    } else if (wave == 3) {
#pragma unroll 4
        for (int u = 0; u < 16; ++u) {
            const int s = 64 * u + lane;
            dma4(xb, (uint32_t)min(n0 + (s >> 3), N - 1) * xrow + kQ81Bytes * (s & 7), &st.xh[64 * u]);
        }
#pragma unroll
        for (int u = 0; u < 3; ++u)
            dma16(wb, (uint32_t)min(m0 + 64 * u + lane, M - 1) * wrow, &st.wh[64 * u]);
    }
}

// One q8_1 block j of the superblock for this wavefront's two 32-row tiles.
template <int J>
__device__ __forceinline__ void block_step(v16f (&part)[2], const v16i& magic, const Stage& st,
                                           const Smem& sm, int xa, int wa, int dnrow, int d8tok) {
    // d8 of the sixteen tokens of this lane's outputs
    float d8v[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
        const float4 v = *(const float4*)((const char*)&sm.d8[J][0] + d8tok + 32 * g4);
        d8v[4 * g4] = v.x; d8v[4 * g4 + 1] = v.y; d8v[4 * g4 + 2] = v.z; d8v[4 * g4 + 3] = v.w;
    }
    const uint4 ca = *(const uint4*)((const char*)st.xc + xa + 32 * J);
    const v4i a = v4i{(int)ca.x, (int)ca.y, (int)ca.z, (int)ca.w};
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        // low nibbles of code pair J/2 for even J, high nibbles for odd J
        const uint4 q = *(const uint4*)((const char*)st.wc + wa + 4096 * rt + 512 * (J >> 1));
        const int sh = 4 * (J & 1);
        const v4i b = v4i{(int)((q.x >> sh) & 0x0f0f0f0fu), (int)((q.y >> sh) & 0x0f0f0f0fu),
                          (int)((q.z >> sh) & 0x0f0f0f0fu), (int)((q.w >> sh) & 0x0f0f0f0fu)};
        const float2 dnv = *(const float2*)((const char*)&sm.dn[J][0] + dnrow + 256 * rt);
        const v16f f = __builtin_bit_cast(v16f, __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, magic, 0, 0, 0));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float t = __builtin_fmaf(f[i], dnv.x, dnv.y);   // round(D*A)
            part[rt][i] = __builtin_fmaf(t, d8v[i], part[rt][i]);
        }
    }
}

// K split of the tail: the tiles of row blocks tail_rb.. run as `parts`
// workgroups each, workgroup z taking superblocks [z * sb_per, min(S, (z + 1)
// * sb_per)); z = 0 writes its sums to y, z > 0 to part + (z - 1) * N * Mt
// ([token][row - tail_rb * BM], Mt = M - tail_rb * BM), which a second launch
// adds to y in the order z = 1, 2, ...  The other tiles take the whole K
// range.  The grid holds the unsplit tiles, then `parts` copies of the tail.
template <bool CLAMP>
__global__ __launch_bounds__(NTHR, 1)
void mmq_q4k_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, float* y,
                    float* part, int M, int N, int S, int mtiles, int ntiles, int sb_per,
                    int tail_rb) {
    __shared__ __align__(16) Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int wr = wave / WT, wt = wave % WT;

    // Tile of this workgroup.  Consecutive workgroups go to different XCDs
    // (round robin); tiles are regrouped so each XCD walks a contiguous run
    // of tiles, the token tiles of one row block after another, and shares
    // those rows' weights in its L2.
    // The unsplit tiles are dispatched first and the split ones after them,
    // each set regrouped on its own, so every XCD gets an equal share of
    // both.
    int tm, tn, z;
    {
        const int64_t head = (int64_t)tail_rb * ntiles;              // unsplit tiles
        const int64_t tail = ((int64_t)mtiles - tail_rb) * ntiles;   // split tiles
        const int64_t lin = blockIdx.x;
        const bool in_head = lin < head;
        const int64_t total = in_head ? head : (int64_t)gridDim.x - head;
        const int64_t l = in_head ? lin : lin - head;
        const int64_t q = total / 8, r = total % 8;
        const int64_t xcd = l % 8, slot = l / 8;
        const int64_t t = xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
        int64_t tile = t;
        z = 0;
        if (!in_head) {
            z = (int)(t / tail);
            tile = head + t % tail;
        }
        tm = (int)(tile / ntiles);
        tn = (int)(tile % ntiles);
    }
    const bool split_tile = tm >= tail_rb && gridDim.x > (unsigned)(mtiles * ntiles);
    const int sb_beg = split_tile ? z * sb_per : 0;
    const int nsb = split_tile ? min(S, sb_beg + sb_per) - sb_beg : S;
    const int ldo = z == 0 ? M : M - tail_rb * BM;    // row stride of this workgroup's output
    const int roff = z == 0 ? 0 : tail_rb * BM;       // first row of that output
    float* out = z == 0 ? y : part + (int64_t)(z - 1) * N * ldo;
    // A tile at the end of m or n starts early enough to lie inside the
    // tensor (its first rows/tokens repeat the previous tile's and are not
    // stored); the CLAMP form (a problem smaller than one tile) clamps.
    const int m0 = CLAMP ? tm * BM : min(tm * BM, M - BM);
    const int n0 = CLAMP ? tn * BN : min(tn * BN, N - BN);
    const int mown = tm * BM, nown = tn * BN;   // first row / token this tile stores

    issue_stage(sm.st[0], wave, lane, w, xq, sb_beg, m0, n0, M, N, S);

    // the fourth bf16 part of z is zero and never rewritten
    for (int i = tid; i < BN * 8; i += NTHR) sm.z[i >> 3][24 + (i & 7)] = 0;

    v16i magic;
#pragma unroll
    for (int i = 0; i < 16; ++i) magic[i] = (int)kMagicBits;
    asm volatile("" : "+v"(magic));   // one register block, read by every MFMA

    v16f acc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rt][i] = 0.0f;

    // per-lane byte offsets of the compute phase's reads
    const int tk = 32 * wt;                       // token offset of this wavefront
    const int ta = tk + l32;                      // token of this lane's MFMA operand row
    const int rw = 64 * wr + l32;                 // this lane's row in the first tile
    const int xa = 16 * (kXStride * ta + h2);     // token codes: + 32*j
    const int wa = 16 * (128 * (rw >> 4) + (rw & 15)) + 256 * h2;   // weight codes: + 512*(j/2) + 4096*rt
    const int dnrow = 8 * rw;                     // (D, nc) of row rw in a block's row: + 256*rt
    const int d8tok = 4 * (tk + 4 * h2);          // d8 of tokens tk+8g+4h2.. in a block's row: + 32*g

    for (int s = 0; s < nsb; ++s) {
        Stage& st = sm.st[s & 1];
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's copies have landed
        __syncthreads();                      // everyone's copies; the previous step's reads done

        // ---- derive: token blocks (d8 as f32, z parts), then row headers
        for (int i = tid; i < BN * 8; i += NTHR) {
            const int j = i / BN, t = i % BN;   // consecutive lanes: consecutive tokens
            const uint4 c0 = st.xc[kXStride * t + 2 * j];
            const uint4 c1 = st.xc[kXStride * t + 2 * j + 1];
            int bq = dot4(c0.x, 0x01010101u, 0);
            bq = dot4(c0.y, 0x01010101u, bq);
            bq = dot4(c0.z, 0x01010101u, bq);
            bq = dot4(c0.w, 0x01010101u, bq);
            bq = dot4(c1.x, 0x01010101u, bq);
            bq = dot4(c1.y, 0x01010101u, bq);
            bq = dot4(c1.z, 0x01010101u, bq);
            bq = dot4(c1.w, 0x01010101u, bq);
            const float d8 = half_bits_to_float(st.xh[8 * t + j]);
            // z = d8*Bq is exact in f32; three bf16 parts by truncation,
            // each the next eight significant bits (the last remainder has
            // at most eight, so it is exact in bf16 too)
            const float zf = d8 * (float)bq;
            const uint32_t zh = __float_as_uint(zf) & 0xffff0000u;
            const float r1 = zf - __uint_as_float(zh);
            const uint32_t zm = __float_as_uint(r1) & 0xffff0000u;
            const float r2 = r1 - __uint_as_float(zm);
            const bool fin = __builtin_isfinite(zf);
            sm.z[t][j] = (uint16_t)(zh >> 16);
            sm.z[t][8 + j] = fin ? (uint16_t)(zm >> 16) : (uint16_t)0;
            sm.z[t][16 + j] = fin ? (uint16_t)(__float_as_uint(r2) >> 16) : (uint16_t)0;
            sm.d8[j][t] = d8;
        }
        // row headers: four threads per row (in four wavefront groups), two sub-blocks each
        {
            const int r = tid % BM, qb = tid / BM;    // 768 threads = 4 x 192 rows
            const uint4 hdr = st.wh[r];
            const float d = half_bits_to_float(hdr.x);
            // six-bit scales and mins: bytes 4..7 hold sc_0..3 (low six bits)
            // and the top bits of sc_4..7; bytes 8..11 the same for m; bytes
            // 12..15 the low nibbles of sc_4..7 and m_4..7
            const uint32_t sw = qb < 2 ? hdr.y & 0x3f3f3f3fu
                                       : (hdr.w & 0x0f0f0f0fu) | ((hdr.y >> 2) & 0x30303030u);
            const uint32_t mw = qb < 2 ? hdr.z & 0x3f3f3f3fu
                                       : ((hdr.w >> 4) & 0x0f0f0f0fu) | ((hdr.z >> 2) & 0x30303030u);
            const int sh = 16 * (qb & 1);               // bytes 2(qb&1), 2(qb&1)+1 of the word
            const float D0 = d * (float)((sw >> sh) & 0xffu), D1 = d * (float)((sw >> (sh + 8)) & 0xffu);
            sm.dn[2 * qb][r] = make_float2(D0, -kMagic * D0);
            sm.dn[2 * qb + 1][r] = make_float2(D1, -kMagic * D1);
            // m < 64 is exact in bf16: the top half of its f32 pattern
            const uint32_t m0b = __float_as_uint((float)((mw >> sh) & 0xffu)) >> 16;
            const uint32_t m1b = __float_as_uint((float)((mw >> (sh + 8)) & 0xffu)) >> 16;
            ((uint32_t*)&sm.mb[r])[qb] = m0b | (m1b << 16);
            if (qb == 0) sm.nd[r] = -half_bits_to_float(hdr.x >> 16);
        }
        __syncthreads();
        // the next step's copies, into the other stage (free since the first barrier)
        if (s + 1 < nsb)
            issue_stage(sm.st[(s + 1) & 1], wave, lane, w, xq, sb_beg + s + 1, m0, n0, M, N, S);

        // ---- compute: two 32-row tiles x 32 tokens per wavefront
        v16f part[2];
        {
            const v8bf za0 = __builtin_bit_cast(v8bf, *(const uint4*)&sm.z[ta][8 * h2]);
            const v8bf za1 = __builtin_bit_cast(v8bf, *(const uint4*)&sm.z[ta][16 + 8 * h2]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int r = rw + 32 * rt;
                const v8bf mbv = __builtin_bit_cast(v8bf, sm.mb[r]);
                const v16f zero = {};
                v16f pm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za0, mbv, zero, 0, 0, 0);
                pm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za1, mbv, pm, 0, 0, 0);
                const float nd = sm.nd[r];
#pragma unroll
                for (int i = 0; i < 16; ++i) part[rt][i] = nd * pm[i];
            }
        }
        // One block at a time: the scheduling fences keep the compiler from
        // hoisting later blocks' loads (and their registers) into this one.
        block_step<0>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<1>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<2>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<3>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<4>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<5>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<6>(part, magic, st, sm, xa, wa, dnrow, d8tok);
        __builtin_amdgcn_sched_barrier(0);
        block_step<7>(part, magic, st, sm, xa, wa, dnrow, d8tok);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[rt] += part[rt];
    }

    // ---- store: lane holds weight row l32 of each tile and 16 tokens
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int m = m0 + 64 * wr + 32 * rt + l32;
        if (m < mown || m >= M) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int n = n0 + 32 * wt + 8 * (i >> 2) + 4 * h2 + (i & 3);
            if (n >= nown && n < N) out[(int64_t)n * ldo + (m - roff)] = acc[rt][i];
        }
    }
}

}  // namespace

// K-split plan from a cost model fitted on MI355X (Qwen2-7B prefill shapes
// at 2048 tokens).  With one workgroup per CU a grid of G workgroups runs in
// ceil(G / cus) rounds; a workgroup of s superblocks takes about s + 2
// superblock steps (its first stage is not overlapped, nor are its stores),
// one step of a full round 4.66 us (gate 18944 x 3584 x 2048: 522 us for 7
// rounds of 16 steps).  Each extra K range adds one f32 plane over the split
// tiles' outputs, written and then read by the sum launch at about 5 TB/s.
// Only the row blocks that make up the last, partly filled round are split
// (the whole grid when it is less than one round), into P = 2..8 ranges of
// ceil(S/P) superblocks; the least estimated time wins, P = 1 (no split)
// included.  Measured in one run: down 3584 x 18944 (304 tiles, 1.2 rounds)
// 708 -> 482 us with 5 ranges over its last 512 rows, QKV 4608 x 3584 (384
// tiles) 155 -> 136 us with 2 over its last 1536, gate 18944 x 3584 541 ->
// 524 us.
MmqPlan plan_mmq_q4k(int64_t m, int64_t n, int64_t k, int cus, int64_t max_ws) {
    const int S = (int)(k / kQK);
    const int64_t mt = (m + BM - 1) / BM, nt = (n + BN - 1) / BN, tiles = mt * nt;
    const double step_us = 4.66;
    auto rounds = [&](int64_t g) { return (g + cus - 1) / cus; };
    MmqPlan best{4, 1, S, 0, 0};
    double best_us = (double)rounds(tiles) * (S + 2) * step_us;
    // row blocks whose tiles fill the whole rounds stay unsplit
    const int64_t full = tiles / cus * cus;
    const int64_t head_rb = tiles == full ? mt : full / nt;
    if (head_rb >= mt) return best;
    const int64_t tail_rows = m - head_rb * BM;
    const double plane_us = 8.0 * (double)n * (double)tail_rows / 5e12 * 1e6;
    for (int P = 2; P <= 8 && P <= S; ++P) {
        const int sb_per = (S + P - 1) / P;
        const int parts = (S + sb_per - 1) / sb_per;
        if (parts != P) continue;
        const int64_t ws = (int64_t)(parts - 1) * n * tail_rows * 4;
        if (ws > max_ws) break;
        const int64_t head = head_rb * nt, tail = tiles - head;
        const double us = (double)rounds(head) * (S + 2) * step_us +
                          (double)rounds(tail * parts) * (sb_per + 2) * step_us +
                          (parts - 1) * plane_us;
        if (us < best_us) {
            best = MmqPlan{4, parts, sb_per, ws, (int)head_rb};
            best_us = us;
        }
    }
    return best;
}

hipError_t launch_mmq_q4k_plan(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                               int64_t k, const MmqPlan& p, void* ws, hipStream_t stream) {
    const int S = (int)(k / kQK);
    const int64_t mt = (m + BM - 1) / BM, nt = (n + BN - 1) / BN;
    if (p.parts < 1 || p.tail_rb < 0 || p.tail_rb > mt) return hipErrorInvalidConfiguration;
    const int tail_rb = p.parts > 1 ? p.tail_rb : (int)mt;
    const int64_t grid = tail_rb * nt + (mt - tail_rb) * nt * p.parts;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    auto kern = (m < BM || n < BN) ? mmq_q4k_kernel<true> : mmq_q4k_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTHR), 0, stream, (const uint8_t*)w,
                       (const uint8_t*)xq, y, (float*)ws, (int)m, (int)n, S, (int)mt, (int)nt,
                       p.sb_per, tail_rb);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.parts > 1) {
        const int64_t r0 = (int64_t)tail_rb * BM;
        e = launch_splitk_sum(y + r0, m, (const float*)ws, n, m - r0, p.parts - 1, stream);
    }
    return e;
}

hipError_t launch_mmq_q4k(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                          int64_t k, int cus, hipStream_t stream) {
    return launch_mmq_q4k_plan(w, xq, y, m, n, k, plan_mmq_q4k(m, n, k, cus, 0), nullptr, stream);
}

}  // namespace kq
