/*
 * kq.h -- C ABI of libkq, the k-quant matmul for AMD Instinct MI355X (gfx950).
 *
 * The library multiplies llama.cpp-style k-quant weights (Q4_K, and Q6_K for
 * the output head) by activations quantised to q8_1:
 *
 *   - kq_quantize_q8_1: activations f32 -> q8_1 blocks, once per matmul input
 *     (leone-cuda "CUDA kernel design": a separate kernel quantises the
 *     activation vector to q8_1 once per GEMV input; minfer "The CUDA
 *     backend" 2.3: activations quantised once per matmul call by a small
 *     prepass before the GEMM).
 *   - kq_gemv_q4k / kq_gemv_q6k: the decode matrix-vector product at batch
 *     1..8 (minfer decodes 2..8 tokens at once on this path), weight-streaming bound (minfer "The CUDA backend" 2.2 and 2.3,
 *     MMVQ; leone-cuda "CUDA kernel design": Q4_K and Q6_K GEMV, residual
 *     epilogue; cajeta "One model, start to last token" 4.1 and 4.2).
 *   - kq_mmq_q4k / kq_mmq_q6k: the prefill matrix-matrix product over many
 *     tokens on the int8 matrix cores (minfer "The CUDA backend" 2.3, MMQ,
 *     and 3.2.6; cajeta "One model, start to last token" 3: Q4_K and Q6_K
 *     tiles).
 *   - kq_mmq_q4k_ws / kq_mmq_q6k_ws: the prefill products split along k
 *     where their tiles do not fill the device, with a caller-provided
 *     workspace.
 *   - kq_rmsnorm_q8_1 / kq_swiglu_q8_1: producers that write the q8_1 blocks
 *     of their output themselves, so the GEMV that follows needs no separate
 *     quantisation launch (leone-cuda "CUDA kernel design": RMSNorm and
 *     SwiGLU write their q8_1 blocks; minfer "The CUDA backend" 2.2).
 *
 * Formats (little-endian; the pages give the sizes and field lists, the bit
 * positions are the public GGUF k-quant layout):
 *
 *   Q4_K superblock, 256 values, 144 bytes:
 *     [0,2) f16 d   [2,4) f16 dmin   [4,16) 8 six-bit scales + 8 six-bit mins
 *     [16,144) 128 bytes of 4-bit codes.
 *     w = (d*sc_j)*q - (dmin*m_j) for the value's 32-value sub-block j.
 *   Q6_K superblock, 256 values, 210 bytes:
 *     [0,128) ql low 4 bits   [128,192) qh high 2 bits   [192,208) 16 int8
 *     scales (one per 16 values)   [208,210) f16 d.   w = (d*sc)*(q - 32).
 *   q8_1 block, 32 values, 36 bytes:
 *     [0,2) f16 d8   [2,4) f16 s (sum of the 32 source values)
 *     [4,36) 32 int8 codes.  xh = d8 * code.
 *
 * Matrices are row-major: weight row r is k/256 consecutive superblocks;
 * activations, residuals and outputs are token-major ([token][...]).
 *
 * Common contract of every call:
 *   - all data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps a pointer after the call returns;
 *   - the work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream); no call synchronises;
 *   - argument errors return KQ_ERR_ARG before anything is launched, and
 *     kq_last_error() names the call and the offending values;
 *   - KQ_ERR_UNSUPPORTED: the current HIP device is not a gfx950 GPU;
 *   - KQ_ERR_HIP: the launch failed; kq_last_error() holds the HIP error;
 *   - there is no fallback path: a call either launches its gfx950 kernel(s)
 *     or returns an error (kq_q6k_split_bytes only computes a size);
 *   - results are deterministic: the same inputs give the same output bits
 *     on every run (no atomics, fixed reduction order);
 *   - sizes of zero rows / tokens (m == 0, n == 0, rows == 0, batch rows of an
 *     empty matrix) are valid and launch nothing;
 *   - every f16 scale (d, dmin, d8) may be zero, subnormal or normal and is
 *     decoded exactly; an output that reads a non-finite scale (an f16 inf
 *     or NaN -- kq_quantize_q8_1 writes d8 = +inf for a block whose largest
 *     magnitude exceeds about 65504*127 = 8.3e6) has an unspecified value
 *     (finite, inf or NaN), and only the outputs of that weight row or that
 *     token are affected;
 *   - calls are thread-safe; the error text is per host thread.
 */
#ifndef KQ_H_
#define KQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KQ_OK = 0,
    KQ_ERR_ARG = -1,
    KQ_ERR_UNSUPPORTED = -2,
    KQ_ERR_HIP = -3
} kq_status;

/* Largest k accepted by the matmul and quantise calls. */
#define KQ_MAX_K 65536
/* Largest m / n / rows accepted (outputs are indexed with 32-bit rows). */
#define KQ_MAX_ROWS 0x7fffffff
/* Largest batch (activation columns) of one GEMV call. */
#define KQ_MAX_BATCH 8
/* Largest number of weight tensors of one segmented GEMV call. */
#define KQ_MAX_SEGMENTS 8

/*
 * Quantise f32 activations to q8_1.
 *   x     f32 [rows][k], row-major, 16-byte aligned.
 *   xq    out: [rows][k/32] q8_1 blocks of 36 bytes, 4-byte aligned.
 *   rows  >= 0;  k > 0, k % 32 == 0, k <= KQ_MAX_K.
 * Per 32-value block: amax = max|x|; d = amax/127 (f32, IEEE division);
 * id = 1/d (0 if d == 0); code = roundf(x*id) (half away from zero);
 * s = f32 pairwise-tree sum of the 32 source values (a[i] += a[i+h] for
 * h = 16, 8, 4, 2, 1); d and s stored as f16 rounded to nearest-even.
 * The result is bit-exact.  In a block whose 1/d overflows (amax below
 * 127*2^-128, where f16(d) is 0 anyway) nonzero values get +-127 and zeros
 * get 0 (x*id is NaN there).  NaN/Inf inputs are outside the contract.
 * xq must not overlap x.
 */
int kq_quantize_q8_1(const float* x, void* xq, int64_t rows, int64_t k, void* stream);

/*
 * Q4_K x q8_1 matrix-vector product for 1..8 activation vectors, with an
 * optional residual added when each output is written.
 *   w         [m][k/256] Q4_K superblocks (144 bytes), 16-byte aligned.
 *   xq        [batch][k/32] q8_1 blocks (from kq_quantize_q8_1), 16-byte aligned.
 *   y         out: f32 [batch][m], 4-byte aligned.
 *   residual  NULL, or f32 [batch][m], 4-byte aligned; y == residual is
 *             allowed (in place); any other overlap is an error.
 *   m >= 0;  k > 0, k % 256 == 0, k <= KQ_MAX_K;  1 <= batch <= KQ_MAX_BATCH.
 * y[t][r] = residual[t][r] + sum over the k/32 blocks j of
 *           d8[t][j] * (d*sc_j * A - dmin*m_j * Bq), with A the integer dot of
 * the block's 4-bit codes with the q8 codes and Bq the sum of the q8 codes
 * (the minimum term is formed from the codes, not from the stored sum s).
 * y must not overlap w or xq.
 */
int kq_gemv_q4k(const void* w, const void* xq, float* y, const float* residual,
                int64_t m, int64_t k, int32_t batch, void* stream);

/*
 * Several Q4_K GEMVs over one shared q8_1 activation in one launch -- e.g.
 * separately stored q, k and v, or gate and up (leone-cuda "CUDA kernel
 * design": QKV shares one quantisation, gate and up share one through the
 * paired GEMV; cajeta "One model, start to last token" 4: the q|k|v and
 * gate|up column segments run as one launch).
 *   nseg       1 <= nseg <= KQ_MAX_SEGMENTS.
 *   w, m, y    HOST arrays of nseg entries: device weights w[s]
 *              ([m[s]][k/256] Q4_K, 16-byte aligned), row counts m[s] >= 0,
 *              device outputs y[s] (f32 [batch][m[s]], 4-byte aligned); a
 *              segment with m[s] == 0 is skipped and its pointers may be NULL.
 *   residual   NULL, or a HOST array of nseg entries, each NULL or a device
 *              f32 [batch][m[s]] (4-byte aligned) added on the row write;
 *              y[s] == residual[s] is allowed.
 *   xq, k, batch  shared by every segment, as in kq_gemv_q4k.
 * Each y[s] equals what kq_gemv_q4k(w[s], xq, y[s], residual[s], m[s], k,
 * batch) writes, bit for bit.  The host arrays are read during the call
 * only.  No output may overlap any weight, another output or another
 * segment's residual.  When the activation does not fit the kernel's LDS
 * budget the segments run as consecutive launches on the same stream.
 */
int kq_gemv_q4k_seg(int32_t nseg, const void* const* w, const int64_t* m, float* const* y,
                    const float* const* residual, const void* xq, int64_t k, int32_t batch,
                    void* stream);

/*
 * Q6_K x q8_1 matrix-vector product for 1..8 activation vectors, with an
 * optional residual.  Same arguments and rules as kq_gemv_q4k except:
 *   w   [m][k/256] Q6_K superblocks (210 bytes), 16-byte aligned; the row
 *       stride 210*k/256 need not be a multiple of 16.
 * y[t][r] = residual[t][r] + sum over blocks j of
 *           d8[t][j] * sum over the block's two 16-value groups g of
 *           d*sc_g * (sum of (q-32)*code over the group).
 */
int kq_gemv_q6k(const void* w, const void* xq, float* y, const float* residual,
                int64_t m, int64_t k, int32_t batch, void* stream);

/*
 * Q4_K x q8_1 matrix-matrix product for n tokens on the int8 matrix cores.
 *   w    [m][k/256] Q4_K superblocks, 16-byte aligned.
 *   xq   [n][k/32] q8_1 blocks, 16-byte aligned.
 *   y    out: f32 [n][m], 4-byte aligned; must not overlap w or xq.
 *   m >= 0, n >= 0, k > 0, k % 256 == 0, k <= KQ_MAX_K, n <= 65535*128;
 *   w and xq are each smaller than 4 GiB (m*k/256*144 and n*k/32*36 bytes).
 * Same value per output as kq_gemv_q4k without a residual.
 */
int kq_mmq_q4k(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
               void* stream);

/*
 * Q6_K x q8_1 matrix-matrix product for n tokens on the int8 matrix cores:
 * the prefill product of the Q6_K tensors of a mixed Q4_K/Q6_K model (cajeta
 * "One model, start to last token" 3: the value projection and the down
 * projection of half the layers are Q6_K and run on their own tensor-core
 * tile; minfer "The CUDA backend" 2.3: integer tile products, scales applied
 * after the integer loop).
 *   w    [m][k/256] Q6_K superblocks (210 bytes), 16-byte aligned; the row
 *        stride need not be a multiple of 16.
 *   xq   [n][k/32] q8_1 blocks, 16-byte aligned.
 *   y    out: f32 [n][m], 4-byte aligned; must not overlap w or xq.
 *   m >= 0, n >= 0, k > 0, k % 256 == 0, k <= KQ_MAX_K, n <= 65535*128;
 *   w and xq are each smaller than 4 GiB (m*k/256*210 and n*k/32*36 bytes).
 * Every int8 scale value (-128..127) is accepted.  Same value per output as
 * kq_gemv_q6k without a residual, up to f32 rounding order.
 */
int kq_mmq_q6k(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
               void* stream);

/*
 * kq_mmq_q4k with a caller-provided workspace, for products whose tiles
 * leave the device's last round of workgroups partly idle (cajeta "One
 * model, start to last token" 3.1: a split along the reduction dimension
 * adds workgroups, and a fixup pass combines the pieces).
 *   kq_mmq_q4k_workspace_bytes(m, n, k): bytes of workspace the split form
 *     needs on the current device -- 0 when the product is not split, -1
 *     for invalid sizes or device.  The product runs in rounds of one
 *     192-row x 128-token tile per compute unit; the row blocks whose tiles
 *     make up the last, partly filled round (the whole product when it is
 *     less than one round) have their k/256 superblocks cut into P <= 8
 *     ranges, P chosen by an estimate of the rounds saved against the extra
 *     partial planes.  The workspace holds ranges 1..P-1 of those rows
 *     (r >= r0) as f32 [P-1][n][m - r0], and a second launch adds them to y
 *     (which holds range 0) in the order z = 1, 2, ...
 *   kq_mmq_q4k_ws: the same product; workspace rules, results and errors
 *     as for kq_mmq_q6k_ws below, except that a workspace smaller than the
 *     best split needs takes the best split that fits in ws_bytes (ws NULL
 *     or ws_bytes 0: the unsplit kq_mmq_q4k, bit for bit).
 */
int64_t kq_mmq_q4k_workspace_bytes(int64_t m, int64_t n, int64_t k);
int kq_mmq_q4k_ws(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                  void* ws, int64_t ws_bytes, void* stream);

/*
 * kq_mmq_q6k with a caller-provided workspace, for products too small to
 * fill the device (cajeta "One model, start to last token" 3.1: a split
 * along the reduction dimension adds workgroups when the output tiles alone
 * leave compute units idle, and a fixup pass combines the pieces).
 *   kq_mmq_q6k_workspace_bytes(m, n, k): bytes of workspace the split form
 *     of this product needs on the current device -- 0 when the product is
 *     not split, -1 for invalid sizes or device (kq_last_error says which).
 *     The split is taken when the product's 128-token tiles number fewer
 *     than two per compute unit: the k/256 superblocks are cut into P <= 4
 *     ranges, range z of every output tile runs as its own workgroup, and
 *     the workspace holds ranges 1..P-1 as f32 [P-1][n][m]; a second launch
 *     then adds them to y (which holds range 0) in the order z = 1, 2, ...
 *   kq_mmq_q6k_ws: the same product.  ws is a device buffer of ws_bytes
 *     bytes, 16-byte aligned, not overlapping w, xq or y, owned by the
 *     caller and used only by work enqueued by this call (do not share it
 *     between calls that may run at the same time).  When ws_bytes is below
 *     what the split needs (ws may then be NULL) the call runs exactly as
 *     kq_mmq_q6k.  Results are deterministic for a given device, size and
 *     workspace size; the split sums in another order than kq_mmq_q6k, so
 *     the two agree within the oracle's bound, not bit for bit.
 *   Other arguments and errors as kq_mmq_q6k; ws_bytes < 0, or ws_bytes > 0
 *   with ws NULL, is KQ_ERR_ARG.
 */
int64_t kq_mmq_q6k_workspace_bytes(int64_t m, int64_t n, int64_t k);
int kq_mmq_q6k_ws(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                  void* ws, int64_t ws_bytes, void* stream);

/*
 * kq_mmq_q6k_ws without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the split's ranges go to a
 * static device array of KQ_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends.  The call
 * allocates nothing.
 *   Same arguments, plan and bits as kq_mmq_q6k_ws given a workspace of
 *   kq_mmq_q6k_workspace_bytes(m, n, k) bytes.  A product whose split needs
 *   more than KQ_NOALLOC_SCRATCH_BYTES is rejected with KQ_ERR_ARG (the text
 *   names the size; use kq_mmq_q6k_ws or kq_mmq_q6k for it).
 *   Every call on a GPU uses that GPU's one array: calls that may run at the
 *   same time on one GPU (other streams, other host threads) race and give
 *   wrong results; serialise them.  Each call writes every scratch byte it
 *   reads before reading it, so nothing needs clearing between calls.
 */
#define KQ_NOALLOC_SCRATCH_BYTES (32LL << 20)
int kq_mmq_q6k_noalloc(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                       void* stream);

/*
 * The split Q6_K layout, made once at load by kq_repack_q6k (cajeta "One
 * model, start to last token" 2, residency: a Q6_K weight is split into a
 * scale prefix and 208-byte bodies so the kernels read it with aligned
 * 16-byte loads).  For superblock g = row * (k/256) + s of an m x k matrix
 * (G = m * k/256 superblocks):
 *   bytes [2g, 2g+2)                f16 d of superblock g
 *   bytes [2G, P)                   zero, P = 2G rounded up to a multiple of 16
 *   bytes [P + 208g, P + 208g+208)  the superblock's bytes 0..207 unchanged
 *                                   (ql, qh, the 16 int8 scales)
 * Every body starts 16-byte aligned (the raw 210-byte superblocks start at
 * 2 mod 4 every other time).  The values are unchanged: the split kernels
 * give bitwise the same outputs as kq_gemv_q6k / kq_mmq_q6k on the raw bytes.
 *
 * kq_q6k_split_bytes: size of the split layout, P + 208*G; -1 when m or k is
 * invalid (m < 0 or > KQ_MAX_ROWS, k not a positive multiple of 256 or
 * > KQ_MAX_K).  Host only, no device access.
 */
int64_t kq_q6k_split_bytes(int64_t m, int64_t k);

/*
 * Raw Q6_K w [m][k/256] (16-byte aligned) -> the split layout in wr
 * (kq_q6k_split_bytes(m, k) bytes, 16-byte aligned, caller-allocated, must
 * not overlap w).  One launch on the stream; asynchronous like every call.
 */
int kq_repack_q6k(const void* w, void* wr, int64_t m, int64_t k, void* stream);

/*
 * kq_gemv_q6k on a weight in the split layout (wr, kq_q6k_split_bytes(m, k)
 * bytes, 16-byte aligned).  Same arguments, rules and results otherwise.
 */
int kq_gemv_q6k_split(const void* wr, const void* xq, float* y, const float* residual,
                      int64_t m, int64_t k, int32_t batch, void* stream);

/*
 * kq_mmq_q6k on a weight in the split layout.  Same arguments, rules and
 * results otherwise (the 4 GiB limit applies to kq_q6k_split_bytes(m, k)).
 */
int kq_mmq_q6k_split(const void* wr, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                     void* stream);

/*
 * RMSNorm of each row (optionally of x + res), times the gain g, written as
 * q8_1 blocks and optionally as f32 (leone-cuda "CUDA kernel design": RMSNorm
 * with a fixed reduction order and sqrtf, writing its q8_1 blocks; the
 * residual form normalises left + right).
 *   x    f32 [rows][n], 16-byte aligned.
 *   res  NULL or f32 [rows][n], 16-byte aligned: h = x + res (one f32 add).
 *   g    f32 [n] gain, 16-byte aligned.
 *   eps  added to the mean square (eps > 0 keeps an all-zero row finite).
 *   y    NULL (only q8_1 is written) or out: f32 [rows][n], 16-byte aligned.
 *   xq   out: [rows][n/32] q8_1 blocks, 4-byte aligned.
 *   rows >= 0, n > 0, n % 256 == 0, n <= KQ_MAX_K, rows*n/256 < 2^31.
 * Per row: ss = sum of h*h in this order: lane l = 0..255 accumulates
 * fmaf(h_i, h_i, acc) over i = l, l+256, ...; then a pairwise tree over the
 * 256 lane sums (a[l] += a[l+h], h = 128 ... 1); r = 1 / sqrtf(ss/n + eps);
 * y = (h*r)*g; xq = the q8_1 blocks of y exactly as kq_quantize_q8_1 makes
 * them.  Every step is one IEEE f32 operation, so the outputs are fixed bit
 * for bit.  y and xq must not overlap x, res, g or each other (every
 * workgroup of a row reads the whole row).
 */
int kq_rmsnorm_q8_1(const float* x, const float* res, const float* g, float eps, float* y,
                    void* xq, int64_t rows, int64_t n, void* stream);

/*
 * SwiGLU y = silu(gate) * up, written as q8_1 blocks and optionally as f32
 * (leone-cuda "CUDA kernel design": SwiGLU writes its dense output and its
 * q8_1 blocks in one elementwise kernel).
 *   gate, up  f32 [rows][n], 16-byte aligned.
 *   y    NULL or out: f32 [rows][n], 16-byte aligned.
 *   xq   out: [rows][n/32] q8_1 blocks, 4-byte aligned.
 *   rows >= 0, n > 0, n % 256 == 0, n <= KQ_MAX_K, rows*n/256 < 2^31.
 * silu(t) = t / (1 + e(-t)) with e(a): +inf for a > 100, +0 for a < -110,
 * else k = rint(a * log2 e), r = fma(-k, 0.693359375, a),
 * r = fma(-k, C2, r) with C2 = ln 2 - 0.693359375 rounded to f32 (Cody and
 * Waite's reduction), p = the degree-7 Taylor polynomial of exp at 0 in
 * Horner form with fused multiply-adds (coefficients 1/j! rounded to f32),
 * e = ldexp(p, k).  Every step is one IEEE f32 operation, so the outputs are
 * fixed bit for bit.  y and xq must not overlap the inputs or each other.
 */
int kq_swiglu_q8_1(const float* gate, const float* up, float* y, void* xq, int64_t rows,
                   int64_t n, void* stream);

/*
 * Measurement helper, not part of the k-quant path: the decode GEMVs stream
 * their weights once (minfer "The CUDA backend" 2.2), and the benchmark
 * reports their rate beside what a plain read of the same bytes reaches on
 * the same device.  kq_read_probe reads nbytes at p once with 16-byte loads.
 * The bytes are cut into chunks of 256*loads 16-byte words; a grid of G
 * 256-thread workgroups takes them round robin (workgroup b reads chunks
 * b, b + G, ...), thread t loading the words 256 u + t of a chunk, u <
 * loads, all issued before any is used.  G = grid, at most the chunk count;
 * grid = 0 gives one workgroup per chunk.  Per wavefront w of workgroup b:
 *   out[4 b + w] = xor, over the workgroup's chunks c, u < loads, l < 64,
 *                  of the 32-bit words of 16-byte word
 *                  256*loads*c + 256 u + 64 w + l (words past the end read
 *                  as zero).
 *   p      device, 16-byte aligned, nbytes > 0 a multiple of 16, < 2^40.
 *   grid   0 <= grid < 2^31;  loads: 4, 8, 16 or 32.
 *   out    device uint32 [kq_read_probe_words(nbytes, grid, loads)], 4-byte
 *          aligned, not overlapping p.
 * kq_read_probe_words: that count, 4 * G; -1 for invalid arguments.  Errors
 * as the other calls (KQ_ERR_ARG, nothing launched).
 */
int64_t kq_read_probe_words(int64_t nbytes, int64_t grid, int32_t loads);
int kq_read_probe(const void* p, int64_t nbytes, uint32_t* out, int64_t grid, int32_t loads,
                  void* stream);

/* Text of the last error on this host thread ("" if none). */
const char* kq_last_error(void);

/* Version of this ABI (incremented on any incompatible change). */
int kq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H_ */
