// kq_device.h -- device helpers and internal launcher declarations of libkq.
//
// Shared by the gfx950 kernels of this library only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace kq {

// Byte sizes of the block formats.
constexpr int kQK = 256;        // values per superblock
constexpr int kQ4KBytes = 144;  // Q4_K superblock
constexpr int kQ6KBytes = 210;  // Q6_K superblock
constexpr int kQ81Bytes = 36;   // q8_1 block (32 values)
constexpr int kMaxSegs = 8;     // weight segments of one segmented GEMV launch

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Plain 16-byte load (global_load_dwordx4).
__device__ __forceinline__ uint4 load16(const void* p) {
    const u32x4_t v = *(const u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Byte-wise signed dot of four int8 pairs, from zero: the VOP3P form takes
// the zero as an inline constant (the accumulating VOP2 form that the
// compiler picks for the builtin needs a v_mov to clear its destination).
__device__ __forceinline__ int dot4_z(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Dot of 16 int8 pairs (one 16-byte slice each), from zero.
__device__ __forceinline__ int dot16_z(uint4 w, uint4 a) {
    return dot4(w.w, a.w, dot4(w.z, a.z, dot4(w.y, a.y, dot4_z(w.x, a.x))));
}

// Sum over the 64 lanes of a wavefront with a fixed xor-butterfly order;
// every lane receives the same total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// N lane sums at once (a transposing butterfly).  The values v[0..N) of the
// SPAN lanes of a span (SPAN = 32 or 64; N a power of two <= SPAN) are added
// over the span with the same pairs in the same order as N separate xor
// butterflies from lane bit log2(SPAN) - 1 down, so each sum is bitwise the
// one such a butterfly gives; but at each of the first log2 N steps a lane
// keeps only the half of its values that its lane bit selects and sends the
// other half to its partner, so the N sums take N - 1 + log2(SPAN / N)
// exchanges instead of N log2 SPAN.  Returns, in lane L, the sum of value
// (L mod SPAN) / (SPAN / N).  The halves are chosen with a bit mask: a
// conditional choice between array elements becomes an indexed access that
// the compiler expands over the whole array.
template <int N, int SPAN>
__device__ __forceinline__ float lane_sums(float (&v)[N], int lane) {
    static_assert((N & (N - 1)) == 0 && N <= SPAN && (SPAN == 32 || SPAN == 64), "shape");
    int m = SPAN / 2;
#pragma unroll
    for (int c = N; c > 1; c >>= 1, m >>= 1) {
        const uint32_t up = (lane & m) ? 0xffffffffu : 0u;
#pragma unroll
        for (int i = 0; i < c / 2; ++i) {
            const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + c / 2]);
            const float keep = __uint_as_float((hi & up) | (lo & ~up));
            const float send = __uint_as_float((lo & up) | (hi & ~up));
            v[i] = keep + __shfl_xor(send, m, 64);
        }
    }
    float s = v[0];
#pragma unroll
    for (; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    return s;
}

constexpr int pow2_ceil(int n) { return n <= 1 ? 1 : 2 * pow2_ceil((n + 1) / 2); }

// q8_1 quantisation of one 32-value block by eight consecutive lanes
// (j = lane & 7 of an aligned group of 8, all active); lane j owns values
// 4j .. 4j+3 in v and writes code dword j; lane 0 also writes the header
// dword {f16 d, f16 s}.  amax -> d = amax/127 -> id = 1/d -> roundf(x*id)
// clamped to +-127 (0 where x*id is NaN: a zero value in a block whose 1/d
// overflows); the source sum is the pairwise tree a[i] += a[i+h]
// (h = 16 ... 1), which the xor shuffles reproduce exactly because IEEE
// addition is commutative (leone-cuda "CUDA kernel design": q8_1 blocks of
// 32 signed codes, an f16 scale and an f16 source sum).
__device__ __forceinline__ void quantize_block8(float4 v, int j, uint32_t* __restrict__ blk) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 4, 8));
    a = fmaxf(a, __shfl_xor(a, 2, 8));
    a = fmaxf(a, __shfl_xor(a, 1, 8));

    const float d = a / 127.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;

    auto code = [&](float t) -> uint32_t {
        float q = roundf(t * id);
        q = (q != q) ? 0.0f : q;   // 0 * inf when 1/d overflows (d < 2^-128)
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        return (uint32_t)((int)q) & 0xffu;
    };
    const uint32_t packed = code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);

    // Source-sum tree.  Lane L holds a[4L..4L+3]; h = 16, 8, 4 pair lanes
    // L and L^4, L^2, L^1; h = 2, 1 finish inside lane 0.
    float4 o;
    o.x = __shfl_xor(v.x, 4, 8); o.y = __shfl_xor(v.y, 4, 8);
    o.z = __shfl_xor(v.z, 4, 8); o.w = __shfl_xor(v.w, 4, 8);
    v.x = v.x + o.x; v.y = v.y + o.y; v.z = v.z + o.z; v.w = v.w + o.w;
    o.x = __shfl_xor(v.x, 2, 8); o.y = __shfl_xor(v.y, 2, 8);
    o.z = __shfl_xor(v.z, 2, 8); o.w = __shfl_xor(v.w, 2, 8);
    v.x = v.x + o.x; v.y = v.y + o.y; v.z = v.z + o.z; v.w = v.w + o.w;
    o.x = __shfl_xor(v.x, 1, 8); o.y = __shfl_xor(v.y, 1, 8);
    o.z = __shfl_xor(v.z, 1, 8); o.w = __shfl_xor(v.w, 1, 8);
    v.x = v.x + o.x; v.y = v.y + o.y; v.z = v.z + o.z; v.w = v.w + o.w;
    const float s = (v.x + v.z) + (v.y + v.w);

    blk[1 + j] = packed;
    if (j == 0) blk[0] = float_to_half_bits(d) | (float_to_half_bits(s) << 16);
}

// Workgroups of kernel `kern` that fit on one compute unit with `threads`
// threads and `lds` bytes of dynamic LDS: asked once per (kernel, threads,
// LDS size) and kept for the process; 1 if the query fails.  Persistent
// launches size their grid with it (an over-full grid is still correct,
// its extra workgroups just wait for a slot).
inline int occupancy(const void* kern, int threads, size_t lds) {
    struct Entry {
        const void* kern;
        int threads;
        size_t lds;
        int occ;
    };
    static std::mutex mu;
    static Entry table[64];
    static int n = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; ++i)
        if (table[i].kern == kern && table[i].threads == threads && table[i].lds == lds)
            return table[i].occ;
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, threads, lds) != hipSuccess || o < 1)
        o = 1;
    if (n < 64) table[n++] = Entry{kern, threads, lds, o};
    return o;
}

// Launchers (return the launch status).
hipError_t launch_quantize_q8_1(const float* x, void* xq, int64_t rows, int64_t k,
                                hipStream_t stream);
hipError_t launch_gemv_q4k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream);
hipError_t launch_gemv_q4k_seg(int nseg, const void* const* w, const int64_t* m, float* const* y,
                               const float* const* residual, const void* xq, int64_t k, int batch,
                               int lds_limit, int cus, hipStream_t stream);
hipError_t launch_gemv_q6k(const void* w, const void* xq, float* y, const float* residual,
                           int64_t m, int64_t k, int batch, int lds_limit, int cus,
                           hipStream_t stream);
int64_t read_probe_words(int64_t nbytes, int64_t grid, int loads);
hipError_t launch_read_probe(const void* p, int64_t nbytes, uint32_t* out, int64_t grid, int loads,
                             hipStream_t stream);
hipError_t launch_mmq_q4k(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                          int64_t k, int cus, hipStream_t stream);
// Launch plan of a prefill product: NT 32-token tiles per workgroup (Q6_K),
// the K range cut into `parts` pieces of sb_per superblocks.  Q4_K: only the
// tiles of row blocks tail_rb.. (the last, partly filled round) are split;
// tail_rb = 0 splits every tile.  parts > 1 needs ws_bytes = (parts - 1) *
// n * (rows of the split row blocks) * 4 bytes.
struct MmqPlan {
    int nt, parts, sb_per;
    int64_t ws_bytes;
    int tail_rb = 0;
};
MmqPlan plan_mmq_q6k(int64_t m, int64_t n, int64_t k, int cus, int64_t max_ws);
MmqPlan plan_mmq_q4k(int64_t m, int64_t n, int64_t k, int cus, int64_t max_ws);
hipError_t launch_mmq_q4k_plan(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                               int64_t k, const MmqPlan& plan, void* ws, hipStream_t stream);
// y[r*ldy + c] = ((y + part[0][r][c]) + part[1][r][c]) + ... for r < rows,
// c < cols, over nparts planes [rows][cols].
hipError_t launch_splitk_sum(float* y, int64_t ldy, const float* part, int64_t rows, int64_t cols,
                             int nparts, hipStream_t stream);
// Static scratch of the allocation-free Q6_K product (bytes), and its
// address on `device` (which must be the current device).
constexpr int64_t kNoallocScratchBytes = 32LL << 20;
hipError_t noalloc_scratch(int device, void** ptr);
hipError_t launch_mmq_q6k_plan(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                               int64_t k, const MmqPlan& plan, void* ws, hipStream_t stream);
hipError_t launch_mmq_q6k(const void* w, const void* xq, float* y, int64_t m, int64_t n,
                          int64_t k, int cus, hipStream_t stream);
hipError_t launch_mmq_q6k_split(const void* wr, const void* xq, float* y, int64_t m, int64_t n,
                                int64_t k, int cus, hipStream_t stream);
hipError_t launch_gemv_q6k_split(const void* wr, const void* xq, float* y, const float* residual,
                                 int64_t m, int64_t k, int batch, int lds_limit, int cus,
                                 hipStream_t stream);
hipError_t launch_repack_q6k(const void* w, void* wr, int64_t m, int64_t k, hipStream_t stream);
hipError_t launch_rmsnorm_q8_1(const float* x, const float* res, const float* g, float eps,
                               float* y, void* xq, int64_t rows, int64_t n, hipStream_t stream);
hipError_t launch_swiglu_q8_1(const float* gate, const float* up, float* y, void* xq,
                              int64_t rows, int64_t n, hipStream_t stream);

}  // namespace kq
