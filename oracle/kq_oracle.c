/*
 * kq_oracle.c -- plain, slow, scalar CPU oracle for the k-quant matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * What it computes (all passages refer to the pages by title and section):
 *
 *  - q8_1 activation quantisation (leone-cuda "CUDA kernel design": one
 *    separate quantisation per GEMV input; each q8_1 block stores 32 signed
 *    codes, an f16 scale and an f16 source sum).  The pages fix the fields
 *    but not the arithmetic, which is taken here as: amax = max|x|;
 *    d = amax / 127 (f32, IEEE division); id = 1/d (0 when d == 0);
 *    q = roundf(x * id) clamped to [-127, 127] (round half away from zero),
 *    and q = 0 where x * id is NaN (x = 0 in a block whose d is so small,
 *    below 2^-128, that 1/d overflows; such a block's f16 d is 0);
 *    s = the f32 sum of the 32 source values taken as a pairwise tree
 *    (a[i] += a[i+h] for h = 16, 8, 4, 2, 1); f16(d) and f16(s) rounded to
 *    nearest-even.  Every f32 operation is a single IEEE operation.
 *
 *  - Q4_K and Q6_K dequantisation in the GGUF arithmetic order in f32
 *    (leone-cuda "CUDA kernel design": the kernel forms every product in f32
 *    with the GGUF arithmetic order).  Q4_K: w = (d*sc)*q - (dmin*m).
 *    Q6_K: w = (d*sc)*(q - 32).  Bit positions follow the public GGUF
 *    k-quant layout (the pages give only block sizes and field lists).
 *
 *  - The matmul as its plain definition: y[t][r] = sum_i w[r][i] * xh[t][i]
 *    where xh = f32(d8) * q8 is the dequantised q8_1 activation, accumulated
 *    in f64 in natural i order (minfer "The CUDA backend" section 2.3: an
 *    integer dot per block with the float scales folded in afterwards reaches
 *    this value up to rounding).  An optional f32 residual is added to the
 *    finished dot (leone-cuda "CUDA kernel design": residual added when the
 *    row is written).  For each output it also returns the tolerance
 *    denominator sum_j |T_j| + |residual|, with T_j the f64 sum of the 32
 *    products of q8_1 block j.
 *
 *  - A second, integer-factored form of the same number (used only to check
 *    the identity between the two forms): T_j = d8 * (D_j*A_j - Mn_j*Bq_j)
 *    with A_j = sum q*q8 and Bq_j = sum q8 over block j; the minimum term is
 *    formed from the q8 codes, not from the stored source sum (leone-cuda
 *    "CUDA kernel design": Q4_K forms each minimum correction from the same
 *    lane-local codes).
 *
 *  - The fused producers that emit q8_1 directly (leone-cuda "CUDA kernel
 *    design": RMSNorm and SwiGLU write their q8_1 blocks so that no
 *    standalone quantisation precedes the next GEMV; RMSNorm uses sqrtf, not
 *    an approximate reciprocal square root, and a fixed reduction order; the
 *    residual variant normalises left + right).  The pages fix neither the
 *    reduction order nor the exponential, so both are defined here and the
 *    GPU must reproduce them bit for bit:
 *      RMSNorm row of n values (n % 256 == 0): h = x (+ res), one f32 add;
 *        ss: lane l = 0..255 accumulates fmaf(h_i, h_i, acc) over
 *        i = l, l+256, l+512, ... in that order, then a pairwise tree over
 *        the 256 lane sums (a[l] += a[l+h] for h = 128, 64, ..., 1);
 *        r = 1 / sqrtf(ss / n + eps); y = (h * r) * g; q8_1 of y.
 *      SwiGLU: y = (t / (1 + e(-t))) * u for gate t and up u; q8_1 of y.
 *      e(a): +inf for a > 100, +0 for a < -110 (NaN passes through);
 *        k = rintf(a * log2(e)); r = fmaf(-k, C1, a), r = fmaf(-k, C2, r)
 *        with C1 = 0.693359375
 *        (9 bits) and C2 = ln 2 - C1 rounded to f32 (Cody and Waite's
 *        argument reduction); p = the degree-7 Taylor polynomial of exp at 0
 *        (coefficients 1/j! rounded to f32) by Horner's rule with fmaf;
 *        e = ldexpf(p, k).
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KQO_WT_Q4K 0
#define KQO_WT_Q6K 1

/* ---------------------------------------------------------------- f16 ---- */

/* Exact decode of an IEEE binary16 bit pattern (subnormals kept). */
static float h2f(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int mant = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)mant, -24);
    else if (e == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + mant), e - 25);
    return (float)(sign ? -v : v);
}

/* binary32 -> binary16, round to nearest, ties to even. */
static uint16_t f2h(float f) {
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double v = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    if (v >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (v < ldexp(1.0, -14)) {
        double q = nearbyint(v * ldexp(1.0, 24)); /* 0 .. 1024 */
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    frexp(v, &e);              /* v in [2^(e-1), 2^e) */
    int E = e - 1;
    double q = nearbyint(ldexp(v, 10 - E)); /* 1024 .. 2048 */
    return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) + ((int)q - 1024)));
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

float kqo_f16_to_f32(uint16_t h) { return h2f(h); }
uint16_t kqo_f32_to_f16(float f) { return f2h(f); }

/* -------------------------------------------------------------- q8_1 ---- */

static void quantize_block(const float* x, uint8_t* out) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    for (int i = 0; i < 32; ++i) {
        float v = roundf(x[i] * id);
        if (v != v) v = 0.0f; /* 0 * inf when 1/d overflows (d < 2^-128) */
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        out[4 + i] = (uint8_t)(int8_t)v;
    }
    float a[32];
    memcpy(a, x, sizeof a);
    for (int h = 16; h >= 1; h >>= 1)
        for (int i = 0; i < h; ++i) a[i] = a[i] + a[i + h];
    uint16_t dh = f2h(d), sh = f2h(a[0]);
    out[0] = (uint8_t)(dh & 255);
    out[1] = (uint8_t)(dh >> 8);
    out[2] = (uint8_t)(sh & 255);
    out[3] = (uint8_t)(sh >> 8);
}

/* x: f32 [rows][k]; out: [rows][k/32] blocks of 36 bytes.  k % 32 == 0. */
void kqo_quantize_q8_1(const float* x, uint8_t* out, int64_t rows, int64_t k) {
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            quantize_block(x + r * k + b * 32, out + (r * nb + b) * 36);
}

/* xq: [rows][k/32] q8_1 blocks -> f32 [rows][k], xh = f32(d8) * q8 (exact). */
void kqo_dequant_q8_1(const uint8_t* xq, float* out, int64_t rows, int64_t k) {
    int64_t nb = k / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = xq + (r * nb + b) * 36;
            float d8 = h2f(rd16(blk));
            for (int i = 0; i < 32; ++i)
                out[r * k + b * 32 + i] = d8 * (float)(int8_t)blk[4 + i];
        }
}

/* -------------------------------------------------------------- Q4_K ---- */

static void q4k_scales(const uint8_t* s, int sc[8], int mn[8]) {
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        mn[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
        mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

static void dequant_q4k_superblock(const uint8_t* b, float* y) {
    float d = h2f(rd16(b)), dmin = h2f(rd16(b + 2));
    int sc[8], mn[8];
    q4k_scales(b + 4, sc, mn);
    const uint8_t* qs = b + 16;
    for (int c = 0; c < 4; ++c) {
        float D0 = d * (float)sc[2 * c], M0 = dmin * (float)mn[2 * c];
        float D1 = d * (float)sc[2 * c + 1], M1 = dmin * (float)mn[2 * c + 1];
        for (int l = 0; l < 32; ++l) {
            int q = qs[32 * c + l];
            y[64 * c + l] = D0 * (float)(q & 15) - M0;
            y[64 * c + 32 + l] = D1 * (float)(q >> 4) - M1;
        }
    }
}

/* -------------------------------------------------------------- Q6_K ---- */

static int q6k_code(const uint8_t* b, int v) {
    int h = v / 128, g = (v % 128) / 32, l = v % 32;
    const uint8_t* ql = b;
    const uint8_t* qh = b + 128;
    int lowbyte = ql[64 * h + (g & 1) * 32 + l];
    int low = (g < 2) ? (lowbyte & 15) : (lowbyte >> 4);
    int high = (qh[32 * h + l] >> (2 * g)) & 3;
    return low | (high << 4);
}

static void dequant_q6k_superblock(const uint8_t* b, float* y) {
    float d = h2f(rd16(b + 208));
    const int8_t* sc = (const int8_t*)(b + 192);
    for (int v = 0; v < 256; ++v)
        y[v] = (d * (float)sc[v / 16]) * (float)(q6k_code(b, v) - 32);
}

static int64_t row_bytes(int wtype, int64_t k) {
    return (k / 256) * (wtype == KQO_WT_Q4K ? 144 : 210);
}

static void dequant_row(int wtype, const uint8_t* row, float* out, int64_t k) {
    int64_t s = k / 256;
    for (int64_t i = 0; i < s; ++i) {
        if (wtype == KQO_WT_Q4K)
            dequant_q4k_superblock(row + i * 144, out + i * 256);
        else
            dequant_q6k_superblock(row + i * 210, out + i * 256);
    }
}

/* w: [m][k/256] superblocks -> f32 [m][k]. */
int kqo_dequant(int wtype, const uint8_t* w, float* out, int64_t m, int64_t k) {
    if (k % 256 || (wtype != KQO_WT_Q4K && wtype != KQO_WT_Q6K)) return -1;
    int64_t rb = row_bytes(wtype, k);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r) dequant_row(wtype, w + r * rb, out + r * k, k);
    return 0;
}

/* ------------------------------------------------------------ matmul ---- */

/* One output: plain f64 dot in natural order, plus sum_j |T_j|. */
static void dot_one(const float* wr, const float* xr, int64_t k, const float* res,
                    double* y, double* den) {
    double acc = 0.0, dsum = 0.0;
    for (int64_t j = 0; j < k / 32; ++j) {
        double T = 0.0;
        for (int i = 0; i < 32; ++i) {
            double p = (double)wr[32 * j + i] * (double)xr[32 * j + i];
            acc += p;
            T += p;
        }
        dsum += fabs(T);
    }
    if (res) {
        acc += (double)*res;
        dsum += fabs((double)*res);
    }
    *y = acc;
    *den = dsum;
}

/*
 * Full matmul.  w: [m][k/256] superblocks of type wtype; xq: [n][k/32] q8_1;
 * residual: NULL or f32 [n][m]; y, den: f64 [n][m] (token-major).
 */
int kqo_matmul(int wtype, const uint8_t* w, const uint8_t* xq, const float* residual,
               int64_t m, int64_t n, int64_t k, double* y, double* den) {
    if (k % 256 || m < 0 || n < 0 || (wtype != KQO_WT_Q4K && wtype != KQO_WT_Q6K)) return -1;
    float* xh = (float*)malloc(sizeof(float) * (size_t)(n * k + 1));
    if (!xh) return -2;
    kqo_dequant_q8_1(xq, xh, n, k);
    int64_t rb = row_bytes(wtype, k);
    int fail = 0;
#pragma omp parallel
    {
        float* wr = (float*)malloc(sizeof(float) * (size_t)k);
        if (!wr) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < m; ++r) {
                dequant_row(wtype, w + r * rb, wr, k);
                for (int64_t t = 0; t < n; ++t)
                    dot_one(wr, xh + t * k, k, residual ? residual + t * m + r : NULL,
                            y + t * m + r, den + t * m + r);
            }
            free(wr);
        }
    }
    free(xh);
    return fail ? -2 : 0;
}

/*
 * Sampled outputs: the same definition evaluated for npairs (token, row)
 * pairs only.  y, den: f64 [npairs].
 */
int kqo_matmul_pairs(int wtype, const uint8_t* w, const uint8_t* xq, const float* residual,
                     int64_t m, int64_t n, int64_t k, const int64_t* tok, const int64_t* row,
                     int64_t npairs, double* y, double* den) {
    if (k % 256 || (wtype != KQO_WT_Q4K && wtype != KQO_WT_Q6K)) return -1;
    int64_t rb = row_bytes(wtype, k);
    int fail = 0;
#pragma omp parallel
    {
        float* wr = (float*)malloc(sizeof(float) * (size_t)k);
        float* xr = (float*)malloc(sizeof(float) * (size_t)k);
        if (!wr || !xr) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t p = 0; p < npairs; ++p) {
                int64_t t = tok[p], r = row[p];
                if (t < 0 || t >= n || r < 0 || r >= m) {
                    y[p] = NAN;
                    den[p] = NAN;
                    continue;
                }
                dequant_row(wtype, w + r * rb, wr, k);
                kqo_dequant_q8_1(xq + t * (k / 32) * 36, xr, 1, k);
                dot_one(wr, xr, k, residual ? residual + t * m + r : NULL, y + p, den + p);
            }
        }
        free(wr);
        free(xr);
    }
    return fail ? -2 : 0;
}

/*
 * Integer-factored second form (identity check only).  Same arguments and
 * output layout as kqo_matmul; no den.
 */
int kqo_matmul_factored(int wtype, const uint8_t* w, const uint8_t* xq, const float* residual,
                        int64_t m, int64_t n, int64_t k, double* y) {
    if (k % 256 || (wtype != KQO_WT_Q4K && wtype != KQO_WT_Q6K)) return -1;
    int64_t rb = row_bytes(wtype, k), nsb = k / 256, nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r) {
        const uint8_t* wrow = w + r * rb;
        for (int64_t t = 0; t < n; ++t) {
            const uint8_t* xrow = xq + t * nb * 36;
            double acc = 0.0;
            for (int64_t sb = 0; sb < nsb; ++sb) {
                for (int jj = 0; jj < 8; ++jj) {
                    const uint8_t* xb = xrow + (sb * 8 + jj) * 36;
                    double d8 = (double)h2f(rd16(xb));
                    const int8_t* q8 = (const int8_t*)(xb + 4);
                    double T;
                    if (wtype == KQO_WT_Q4K) {
                        const uint8_t* b = wrow + sb * 144;
                        int sc[8], mn[8];
                        q4k_scales(b + 4, sc, mn);
                        float D = h2f(rd16(b)) * (float)sc[jj];
                        float Mn = h2f(rd16(b + 2)) * (float)mn[jj];
                        int c = jj / 2, hi = jj & 1;
                        long A = 0, Bq = 0;
                        for (int l = 0; l < 32; ++l) {
                            int byte = b[16 + 32 * c + l];
                            int q = hi ? (byte >> 4) : (byte & 15);
                            A += (long)q * q8[l];
                            Bq += q8[l];
                        }
                        T = d8 * ((double)D * (double)A - (double)Mn * (double)Bq);
                    } else {
                        const uint8_t* b = wrow + sb * 210;
                        const int8_t* sc = (const int8_t*)(b + 192);
                        float d = h2f(rd16(b + 208));
                        long Alo = 0, Ahi = 0;
                        for (int l = 0; l < 32; ++l) {
                            long p = (long)(q6k_code(b, 32 * jj + l) - 32) * q8[l];
                            if (l < 16) Alo += p; else Ahi += p;
                        }
                        double D0 = (double)(d * (float)sc[2 * jj]);
                        double D1 = (double)(d * (float)sc[2 * jj + 1]);
                        T = d8 * (D0 * (double)Alo + D1 * (double)Ahi);
                    }
                    acc += T;
                }
            }
            if (residual) acc += (double)residual[t * m + r];
            y[t * m + r] = acc;
        }
    }
    return 0;
}

/* ----------------------------------------------------------- threads ---- */

void kqo_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int kqo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Array forms of the f16 conversions (for pinning against other routines). */
void kqo_f32_to_f16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f2h(in[i]);
}

void kqo_f16_to_f32_array(const uint16_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = h2f(in[i]);
}

/* --------------------------------------------------------- producers ---- */

/* e(a): Cody-Waite reduction by ln 2 and the degree-7 Taylor polynomial. */
static float exp_f32(float a) {
    if (a > 100.0f) return INFINITY;
    if (a < -110.0f) return 0.0f;
    float k = rintf(a * 1.44269504088896341f);
    float r = fmaf(-k, 0.693359375f, a);
    r = fmaf(-k, -2.12194440054690583e-4f, r);
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)k);
}

static float silu_f32(float t) { return t / (1.0f + exp_f32(-t)); }

void kqo_exp_array(const float* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = exp_f32(in[i]);
}

void kqo_silu_array(const float* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = silu_f32(in[i]);
}

/* Sum of squares of one row in the stated order (n % 256 == 0). */
static float rms_sumsq(const float* h, int64_t n) {
    float a[256];
    for (int l = 0; l < 256; ++l) {
        float acc = 0.0f;
        for (int64_t i = l; i < n; i += 256) acc = fmaf(h[i], h[i], acc);
        a[l] = acc;
    }
    for (int hh = 128; hh >= 1; hh >>= 1)
        for (int l = 0; l < hh; ++l) a[l] = a[l] + a[l + hh];
    return a[0];
}

float kqo_rms_sumsq(const float* h, int64_t n) { return rms_sumsq(h, n); }

/* x, res (may be NULL), g: f32; y: f32 [rows][n]; xq (may be NULL): q8_1 of y. */
void kqo_rmsnorm_q8_1(const float* x, const float* res, const float* g, float eps, float* y,
                      uint8_t* xq, int64_t rows, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        float* h = (float*)malloc((size_t)n * sizeof(float));
        for (int64_t i = 0; i < n; ++i)
            h[i] = res ? x[row * n + i] + res[row * n + i] : x[row * n + i];
        float ss = rms_sumsq(h, n);
        float r = 1.0f / sqrtf(ss / (float)n + eps);
        float* yr = y + row * n;
        for (int64_t i = 0; i < n; ++i) yr[i] = (h[i] * r) * g[i];
        if (xq)
            for (int64_t b = 0; b < n / 32; ++b)
                quantize_block(yr + b * 32, xq + (row * (n / 32) + b) * 36);
        free(h);
    }
}

/* gate, up: f32 [rows][n]; y: f32; xq (may be NULL): q8_1 of y. */
void kqo_swiglu_q8_1(const float* gate, const float* up, float* y, uint8_t* xq, int64_t rows,
                     int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        float* yr = y + row * n;
        for (int64_t i = 0; i < n; ++i) yr[i] = silu_f32(gate[row * n + i]) * up[row * n + i];
        if (xq)
            for (int64_t b = 0; b < n / 32; ++b)
                quantize_block(yr + b * 32, xq + (row * (n / 32) + b) * 36);
    }
}
