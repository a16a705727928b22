// kq_api.cpp -- the C ABI of libkq (declared in include/kq.h).
//
// Every entry point validates its arguments before touching the HIP runtime,
// checks that the current device is a gfx950 GPU, launches its gfx950 kernel
// on the caller's stream (one launch; a segmented GEMV whose activation does
// not fit on chip launches once per segment) and reports the launch status.
// Invariant violations return an error that names the offending values;
// nothing falls back to another path (minfer "The CUDA backend" 3.4: a
// violated invariant is an error with the values, never a silent detour).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/kq.h"
#include "kq_device.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return KQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) intersect
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Per device: 0 unknown, 1 gfx950, -1 other.  Also the LDS limit per block.
std::atomic<int> g_arch[64];
std::atomic<int> g_lds[64];
std::atomic<int> g_cus[64];

int check_device(const char* fn, int* lds_limit, int* cus = nullptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0)
        return fail(KQ_ERR_UNSUPPORTED, "%s: no HIP device (%s)", fn, hipGetErrorString(e));
    if (dev >= 64) return fail(KQ_ERR_UNSUPPORTED, "%s: device index %d out of range", fn, dev);
    int state = g_arch[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(KQ_ERR_UNSUPPORTED, "%s: hipGetDeviceProperties(%d) failed: %s", fn, dev,
                        hipGetErrorString(e));
        state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_lds[dev].store((int)prop.sharedMemPerBlock, std::memory_order_relaxed);
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch[dev].store(state, std::memory_order_release);
        if (state < 0)
            return fail(KQ_ERR_UNSUPPORTED, "%s: device %d is %s, not gfx950", fn, dev,
                        prop.gcnArchName);
    }
    if (state < 0) return fail(KQ_ERR_UNSUPPORTED, "%s: device %d is not gfx950", fn, dev);
    if (lds_limit) *lds_limit = g_lds[dev].load(std::memory_order_relaxed);
    if (cus) *cus = g_cus[dev].load(std::memory_order_relaxed);
    return KQ_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(KQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int check_k(const char* fn, int64_t k, int64_t mult) {
    if (k <= 0 || k % mult != 0 || k > KQ_MAX_K)
        return fail(KQ_ERR_ARG, "%s: k=%lld must be a positive multiple of %lld and <= %d", fn,
                    (long long)k, (long long)mult, KQ_MAX_K);
    return KQ_OK;
}

// Bytes of the split Q6_K layout of an m x k matrix: the f16 d prefix padded
// to 16 bytes, then one 208-byte body per superblock.
int64_t split_bytes(int64_t m, int64_t k) {
    const int64_t g = m * (k / 256);
    return (2 * g + 15) / 16 * 16 + 208 * g;
}

// wtotal >= 0: the weight buffer's size when it is not m*(k/256)*wbytes.
int gemv_common(const char* fn, int wbytes, const void* w, const void* xq, float* y,
                const float* residual, int64_t m, int64_t k, int32_t batch,
                int64_t wtotal = -1) {
    if (!w || !xq || !y)
        return fail(KQ_ERR_ARG, "%s: null pointer (w=%p xq=%p y=%p)", fn, w, xq, (void*)y);
    if (int rc = check_k(fn, k, 256)) return rc;
    if (m < 0 || m > KQ_MAX_ROWS)
        return fail(KQ_ERR_ARG, "%s: m=%lld out of range [0, %d]", fn, (long long)m, KQ_MAX_ROWS);
    if (batch < 1 || batch > KQ_MAX_BATCH)
        return fail(KQ_ERR_ARG, "%s: batch=%d must be in [1, %d]", fn, (int)batch, KQ_MAX_BATCH);
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(y, 4) || (residual && !aligned(residual, 4)))
        return fail(KQ_ERR_ARG,
                    "%s: misaligned pointer (w=%p xq=%p need 16, y=%p residual=%p need 4)", fn, w,
                    xq, (void*)y, (const void*)residual);
    const int64_t wn = wtotal >= 0 ? wtotal : m * (k / 256) * wbytes;
    const int64_t xn = (int64_t)batch * (k / 32) * 36;
    const int64_t yn = (int64_t)batch * m * 4;
    if (overlap(y, yn, w, wn) || overlap(y, yn, xq, xn))
        return fail(KQ_ERR_ARG, "%s: output y=%p overlaps an input (w=%p, xq=%p)", fn, (void*)y, w, xq);
    if (residual && residual != y && overlap(y, yn, residual, yn))
        return fail(KQ_ERR_ARG, "%s: y=%p partially overlaps residual=%p", fn, (void*)y,
                    (const void*)residual);
    return KQ_OK;
}

}  // namespace

extern "C" {

int kq_quantize_q8_1(const float* x, void* xq, int64_t rows, int64_t k, void* stream) {
    const char* fn = "kq_quantize_q8_1";
    if (!x || !xq) return fail(KQ_ERR_ARG, "%s: null pointer (x=%p xq=%p)", fn, (const void*)x, xq);
    if (int rc = check_k(fn, k, 32)) return rc;
    if (rows < 0 || rows > KQ_MAX_ROWS)
        return fail(KQ_ERR_ARG, "%s: rows=%lld out of range [0, %d]", fn, (long long)rows, KQ_MAX_ROWS);
    if (rows * k / 1024 >= 0x7fffffffLL)
        return fail(KQ_ERR_ARG, "%s: rows*k=%lld too large for one launch", fn, (long long)(rows * k));
    if (!aligned(x, 16) || !aligned(xq, 4))
        return fail(KQ_ERR_ARG, "%s: misaligned pointer (x=%p needs 16, xq=%p needs 4)", fn,
                    (const void*)x, xq);
    if (overlap(x, rows * k * 4, xq, rows * (k / 32) * 36))
        return fail(KQ_ERR_ARG, "%s: xq=%p overlaps x=%p", fn, xq, (const void*)x);
    if (rows == 0) return ok();
    if (int rc = check_device(fn, nullptr)) return rc;
    return launched(fn, kq::launch_quantize_q8_1(x, xq, rows, k, (hipStream_t)stream));
}

int kq_gemv_q4k(const void* w, const void* xq, float* y, const float* residual, int64_t m,
                int64_t k, int32_t batch, void* stream) {
    const char* fn = "kq_gemv_q4k";
    if (int rc = gemv_common(fn, 144, w, xq, y, residual, m, k, batch)) return rc;
    if (m == 0) return ok();
    int lds = 0, cus = 0;
    if (int rc = check_device(fn, &lds, &cus)) return rc;
    return launched(fn, kq::launch_gemv_q4k(w, xq, y, residual, m, k, batch, lds, cus,
                                            (hipStream_t)stream));
}

int kq_gemv_q4k_seg(int32_t nseg, const void* const* w, const int64_t* m, float* const* y,
                    const float* const* residual, const void* xq, int64_t k, int32_t batch,
                    void* stream) {
    const char* fn = "kq_gemv_q4k_seg";
    if (nseg < 1 || nseg > KQ_MAX_SEGMENTS)
        return fail(KQ_ERR_ARG, "%s: nseg=%d must be in [1, %d]", fn, (int)nseg, KQ_MAX_SEGMENTS);
    if (!w || !m || !y)
        return fail(KQ_ERR_ARG, "%s: null array (w=%p m=%p y=%p)", fn, (const void*)w,
                    (const void*)m, (const void*)y);
    if (!xq) return fail(KQ_ERR_ARG, "%s: null pointer (xq=%p)", fn, xq);
    if (int rc = check_k(fn, k, 256)) return rc;
    if (batch < 1 || batch > KQ_MAX_BATCH)
        return fail(KQ_ERR_ARG, "%s: batch=%d must be in [1, %d]", fn, (int)batch, KQ_MAX_BATCH);
    if (!aligned(xq, 16)) return fail(KQ_ERR_ARG, "%s: misaligned pointer (xq=%p needs 16)", fn, xq);
    int64_t total = 0;
    for (int s = 0; s < nseg; ++s) {
        if (m[s] == 0) continue;   // skipped segment: its pointers are not used
        const float* r = residual ? residual[s] : nullptr;
        if (int rc = gemv_common(fn, 144, w[s], xq, y[s], r, m[s], k, batch)) return rc;
        total += m[s];
    }
    if (total > KQ_MAX_ROWS)
        return fail(KQ_ERR_ARG, "%s: %lld rows in all segments, more than %d", fn,
                    (long long)total, KQ_MAX_ROWS);
    for (int s = 0; s < nseg; ++s) {
        if (m[s] == 0) continue;
        const int64_t yn = (int64_t)batch * m[s] * 4;
        for (int t = 0; t < nseg; ++t) {
            if (m[t] == 0) continue;
            const int64_t wt = m[t] * (k / 256) * 144, yt = (int64_t)batch * m[t] * 4;
            const float* rt = residual ? residual[t] : nullptr;
            if (overlap(y[s], yn, w[t], wt) || (t != s && overlap(y[s], yn, y[t], yt)) ||
                (t != s && rt && overlap(y[s], yn, rt, yt)))
                return fail(KQ_ERR_ARG, "%s: output y[%d]=%p overlaps a buffer of segment %d", fn,
                            s, (void*)y[s], t);
        }
    }
    if (total == 0) return ok();
    int lds = 0, cus = 0;
    if (int rc = check_device(fn, &lds, &cus)) return rc;
    return launched(fn, kq::launch_gemv_q4k_seg(nseg, w, m, y, residual, xq, k, batch, lds, cus,
                                                (hipStream_t)stream));
}

int kq_gemv_q6k(const void* w, const void* xq, float* y, const float* residual, int64_t m,
                int64_t k, int32_t batch, void* stream) {
    const char* fn = "kq_gemv_q6k";
    if (int rc = gemv_common(fn, 210, w, xq, y, residual, m, k, batch)) return rc;
    if (m == 0) return ok();
    int lds = 0, cus = 0;
    if (int rc = check_device(fn, &lds, &cus)) return rc;
    return launched(fn, kq::launch_gemv_q6k(w, xq, y, residual, m, k, batch, lds, cus,
                                            (hipStream_t)stream));
}

static int mmq_common(const char* fn, int sb_bytes, const void* w, const void* xq, float* y,
                      int64_t m, int64_t n, int64_t k, bool split = false) {
    if (!w || !xq || !y)
        return fail(KQ_ERR_ARG, "%s: null pointer (w=%p xq=%p y=%p)", fn, w, xq, (void*)y);
    if (int rc = check_k(fn, k, 256)) return rc;
    if (m < 0 || m > KQ_MAX_ROWS || n < 0 || n > 65535LL * 128)
        return fail(KQ_ERR_ARG, "%s: m=%lld or n=%lld out of range (m <= %d, n <= %lld)", fn,
                    (long long)m, (long long)n, KQ_MAX_ROWS, 65535LL * 128);
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(y, 4))
        return fail(KQ_ERR_ARG, "%s: misaligned pointer (w=%p xq=%p need 16, y=%p needs 4)", fn, w,
                    xq, (void*)y);
    const int64_t wbytes = split ? split_bytes(m, k) : m * (k / 256) * sb_bytes;
    const int64_t xbytes = n * (k / 32) * 36;
    if (wbytes >= (1LL << 32) || xbytes >= (1LL << 32))
        return fail(KQ_ERR_ARG, "%s: w (%lld bytes) or xq (%lld bytes) is 4 GiB or larger", fn,
                    (long long)wbytes, (long long)xbytes);
    const int64_t yn = n * m * 4;
    if (overlap(y, yn, w, wbytes) || overlap(y, yn, xq, xbytes))
        return fail(KQ_ERR_ARG, "%s: output y=%p overlaps an input (w=%p, xq=%p)", fn, (void*)y, w, xq);
    return KQ_OK;
}

int kq_mmq_q4k(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
               void* stream) {
    const char* fn = "kq_mmq_q4k";
    if (int rc = mmq_common(fn, 144, w, xq, y, m, n, k)) return rc;
    if (m == 0 || n == 0) return ok();
    int cus = 0;
    if (int rc = check_device(fn, nullptr, &cus)) return rc;
    return launched(fn, kq::launch_mmq_q4k(w, xq, y, m, n, k, cus, (hipStream_t)stream));
}

int kq_mmq_q6k(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
               void* stream) {
    const char* fn = "kq_mmq_q6k";
    if (int rc = mmq_common(fn, 210, w, xq, y, m, n, k)) return rc;
    if (m == 0 || n == 0) return ok();
    int cus = 0;
    if (int rc = check_device(fn, nullptr, &cus)) return rc;
    return launched(fn, kq::launch_mmq_q6k(w, xq, y, m, n, k, cus, (hipStream_t)stream));
}

int64_t kq_mmq_q4k_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const char* fn = "kq_mmq_q4k_workspace_bytes";
    if (k <= 0 || k % 256 != 0 || k > KQ_MAX_K || m < 0 || m > KQ_MAX_ROWS || n < 0 ||
        n > 65535LL * 128) {
        fail(KQ_ERR_ARG, "%s: m=%lld n=%lld k=%lld out of range", fn, (long long)m, (long long)n,
             (long long)k);
        return -1;
    }
    if (m == 0 || n == 0) return 0;
    int cus = 0;
    if (check_device(fn, nullptr, &cus)) return -1;
    return kq::plan_mmq_q4k(m, n, k, cus, INT64_MAX).ws_bytes;
}

int kq_mmq_q4k_ws(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                  void* ws, int64_t ws_bytes, void* stream) {
    const char* fn = "kq_mmq_q4k_ws";
    if (int rc = mmq_common(fn, 144, w, xq, y, m, n, k)) return rc;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws))
        return fail(KQ_ERR_ARG, "%s: ws=%p with ws_bytes=%lld", fn, ws, (long long)ws_bytes);
    if (m == 0 || n == 0) return ok();
    int cus = 0;
    if (int rc = check_device(fn, nullptr, &cus)) return rc;
    const kq::MmqPlan plan = kq::plan_mmq_q4k(m, n, k, cus, ws ? ws_bytes : 0);
    if (plan.parts > 1) {
        if (!aligned(ws, 16))
            return fail(KQ_ERR_ARG, "%s: misaligned workspace ws=%p (needs 16)", fn, ws);
        if (overlap(ws, plan.ws_bytes, w, m * (k / 256) * 144) ||
            overlap(ws, plan.ws_bytes, xq, n * (k / 32) * 36) || overlap(ws, plan.ws_bytes, y, m * n * 4))
            return fail(KQ_ERR_ARG, "%s: workspace ws=%p overlaps w, xq or y", fn, ws);
    }
    return launched(fn, kq::launch_mmq_q4k_plan(w, xq, y, m, n, k, plan, ws, (hipStream_t)stream));
}

int64_t kq_mmq_q6k_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const char* fn = "kq_mmq_q6k_workspace_bytes";
    if (k <= 0 || k % 256 != 0 || k > KQ_MAX_K || m < 0 || m > KQ_MAX_ROWS || n < 0 ||
        n > 65535LL * 128) {
        fail(KQ_ERR_ARG, "%s: m=%lld n=%lld k=%lld out of range", fn, (long long)m, (long long)n,
             (long long)k);
        return -1;
    }
    if (m == 0 || n == 0) return 0;
    int cus = 0;
    if (check_device(fn, nullptr, &cus)) return -1;
    return kq::plan_mmq_q6k(m, n, k, cus, INT64_MAX).ws_bytes;
}

int kq_mmq_q6k_ws(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                  void* ws, int64_t ws_bytes, void* stream) {
    const char* fn = "kq_mmq_q6k_ws";
    if (int rc = mmq_common(fn, 210, w, xq, y, m, n, k)) return rc;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws))
        return fail(KQ_ERR_ARG, "%s: ws=%p with ws_bytes=%lld", fn, ws, (long long)ws_bytes);
    if (m == 0 || n == 0) return ok();
    int cus = 0;
    if (int rc = check_device(fn, nullptr, &cus)) return rc;
    const kq::MmqPlan plan = kq::plan_mmq_q6k(m, n, k, cus, ws ? ws_bytes : 0);
    if (plan.parts > 1) {
        if (!aligned(ws, 16))
            return fail(KQ_ERR_ARG, "%s: misaligned workspace ws=%p (needs 16)", fn, ws);
        if (overlap(ws, plan.ws_bytes, w, m * (k / 256) * 210) ||
            overlap(ws, plan.ws_bytes, xq, n * (k / 32) * 36) || overlap(ws, plan.ws_bytes, y, m * n * 4))
            return fail(KQ_ERR_ARG, "%s: workspace ws=%p overlaps w, xq or y", fn, ws);
    }
    return launched(fn, kq::launch_mmq_q6k_plan(w, xq, y, m, n, k, plan, ws, (hipStream_t)stream));
}

static_assert(KQ_NOALLOC_SCRATCH_BYTES == kq::kNoallocScratchBytes, "scratch size mismatch");

int kq_mmq_q6k_noalloc(const void* w, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                       void* stream) {
    const char* fn = "kq_mmq_q6k_noalloc";
    if (int rc = mmq_common(fn, 210, w, xq, y, m, n, k)) return rc;
    if (m == 0 || n == 0) return ok();
    int cus = 0;
    if (int rc = check_device(fn, nullptr, &cus)) return rc;
    const kq::MmqPlan plan = kq::plan_mmq_q6k(m, n, k, cus, INT64_MAX);
    if (plan.ws_bytes > KQ_NOALLOC_SCRATCH_BYTES)
        return fail(KQ_ERR_ARG,
                    "%s: m=%lld n=%lld k=%lld needs %lld bytes of scratch, more than the %lld of the "
                    "static scratch (use kq_mmq_q6k_ws or kq_mmq_q6k)",
                    fn, (long long)m, (long long)n, (long long)k, (long long)plan.ws_bytes,
                    (long long)KQ_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (plan.ws_bytes > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return fail(KQ_ERR_HIP, "%s: hipGetDevice failed", fn);
        const hipError_t e = kq::noalloc_scratch(dev, &ws);
        if (e != hipSuccess)
            return fail(KQ_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        if (overlap(ws, plan.ws_bytes, y, m * n * 4))
            return fail(KQ_ERR_ARG, "%s: y=%p overlaps the static scratch", fn, (void*)y);
    }
    return launched(fn, kq::launch_mmq_q6k_plan(w, xq, y, m, n, k, plan, ws, (hipStream_t)stream));
}

int kq_mmq_q6k_split(const void* wr, const void* xq, float* y, int64_t m, int64_t n, int64_t k,
                     void* stream) {
    const char* fn = "kq_mmq_q6k_split";
    if (int rc = mmq_common(fn, 210, wr, xq, y, m, n, k, true)) return rc;
    if (m == 0 || n == 0) return ok();
    int cus = 0;
    if (int rc = check_device(fn, nullptr, &cus)) return rc;
    return launched(fn, kq::launch_mmq_q6k_split(wr, xq, y, m, n, k, cus, (hipStream_t)stream));
}

static bool probe_shape_ok(int64_t nbytes, int64_t grid, int32_t loads) {
    return nbytes > 0 && nbytes % 16 == 0 && nbytes < (1LL << 40) && grid >= 0 &&
           grid <= 0x7fffffffLL && (loads == 4 || loads == 8 || loads == 16 || loads == 32) &&
           kq::read_probe_words(nbytes, grid, loads) / 4 <= 0x7fffffffLL;
}

int64_t kq_read_probe_words(int64_t nbytes, int64_t grid, int32_t loads) {
    if (!probe_shape_ok(nbytes, grid, loads)) return -1;
    return kq::read_probe_words(nbytes, grid, loads);
}

int kq_read_probe(const void* p, int64_t nbytes, uint32_t* out, int64_t grid, int32_t loads,
                  void* stream) {
    const char* fn = "kq_read_probe";
    if (!p || !out) return fail(KQ_ERR_ARG, "%s: null pointer (p=%p out=%p)", fn, p, (void*)out);
    if (nbytes <= 0 || nbytes % 16 != 0 || nbytes >= (1LL << 40))
        return fail(KQ_ERR_ARG, "%s: nbytes=%lld must be a positive multiple of 16 below 2^40", fn,
                    (long long)nbytes);
    if (!probe_shape_ok(nbytes, grid, loads))
        return fail(KQ_ERR_ARG, "%s: grid=%lld loads=%d (grid in [0, 2^31), loads 4, 8, 16 or 32)",
                    fn, (long long)grid, (int)loads);
    if (!aligned(p, 16) || !aligned(out, 4))
        return fail(KQ_ERR_ARG, "%s: misaligned pointer (p=%p needs 16, out=%p needs 4)", fn, p,
                    (void*)out);
    const int64_t words = kq::read_probe_words(nbytes, grid, loads);
    if (overlap(out, words * 4, p, nbytes))
        return fail(KQ_ERR_ARG, "%s: out=%p overlaps p=%p", fn, (void*)out, p);
    if (int rc = check_device(fn, nullptr)) return rc;
    return launched(fn, kq::launch_read_probe(p, nbytes, out, grid, loads, (hipStream_t)stream));
}

int64_t kq_q6k_split_bytes(int64_t m, int64_t k) {
    if (m < 0 || m > KQ_MAX_ROWS || k <= 0 || k % 256 != 0 || k > KQ_MAX_K) return -1;
    return split_bytes(m, k);
}

int kq_repack_q6k(const void* w, void* wr, int64_t m, int64_t k, void* stream) {
    const char* fn = "kq_repack_q6k";
    if (!w || !wr) return fail(KQ_ERR_ARG, "%s: null pointer (w=%p wr=%p)", fn, w, wr);
    if (int rc = check_k(fn, k, 256)) return rc;
    if (m < 0 || m > KQ_MAX_ROWS)
        return fail(KQ_ERR_ARG, "%s: m=%lld out of range [0, %d]", fn, (long long)m, KQ_MAX_ROWS);
    if (!aligned(w, 16) || !aligned(wr, 16))
        return fail(KQ_ERR_ARG, "%s: misaligned pointer (w=%p wr=%p need 16)", fn, w, wr);
    if (overlap(wr, split_bytes(m, k), w, m * (k / 256) * 210))
        return fail(KQ_ERR_ARG, "%s: wr=%p overlaps w=%p", fn, wr, w);
    if (m == 0) return ok();
    if (int rc = check_device(fn, nullptr)) return rc;
    return launched(fn, kq::launch_repack_q6k(w, wr, m, k, (hipStream_t)stream));
}

int kq_gemv_q6k_split(const void* wr, const void* xq, float* y, const float* residual, int64_t m,
                      int64_t k, int32_t batch, void* stream) {
    const char* fn = "kq_gemv_q6k_split";
    if (int rc = gemv_common(fn, 210, wr, xq, y, residual, m, k, batch,
                             (m >= 0 && m <= KQ_MAX_ROWS && k > 0 && k <= KQ_MAX_K)
                                 ? split_bytes(m, k) : 0))
        return rc;
    if (m == 0) return ok();
    int lds = 0, cus = 0;
    if (int rc = check_device(fn, &lds, &cus)) return rc;
    return launched(fn, kq::launch_gemv_q6k_split(wr, xq, y, residual, m, k, batch, lds, cus,
                                                  (hipStream_t)stream));
}

static int producer_sizes(const char* fn, int64_t rows, int64_t n) {
    if (n <= 0 || n % 256 != 0 || n > KQ_MAX_K)
        return fail(KQ_ERR_ARG, "%s: n=%lld must be a positive multiple of 256 and <= %d", fn,
                    (long long)n, KQ_MAX_K);
    if (rows < 0 || rows > KQ_MAX_ROWS)
        return fail(KQ_ERR_ARG, "%s: rows=%lld out of range [0, %d]", fn, (long long)rows,
                    KQ_MAX_ROWS);
    if (rows * (n / 256) >= 0x7fffffffLL)
        return fail(KQ_ERR_ARG, "%s: rows*n=%lld too large for one launch", fn,
                    (long long)(rows * n));
    return KQ_OK;
}

int kq_rmsnorm_q8_1(const float* x, const float* res, const float* g, float eps, float* y,
                    void* xq, int64_t rows, int64_t n, void* stream) {
    const char* fn = "kq_rmsnorm_q8_1";
    if (!x || !g || !xq)
        return fail(KQ_ERR_ARG, "%s: null pointer (x=%p g=%p xq=%p)", fn, (const void*)x,
                    (const void*)g, xq);
    if (int rc = producer_sizes(fn, rows, n)) return rc;
    if (!aligned(x, 16) || !aligned(g, 16) || (res && !aligned(res, 16)) || (y && !aligned(y, 16)) ||
        !aligned(xq, 4))
        return fail(KQ_ERR_ARG,
                    "%s: misaligned pointer (x=%p res=%p g=%p y=%p need 16, xq=%p needs 4)", fn,
                    (const void*)x, (const void*)res, (const void*)g, (void*)y, xq);
    const int64_t fb = rows * n * 4, qb = rows * (n / 32) * 36;
    const bool bad = overlap(xq, qb, x, fb) || overlap(xq, qb, g, n * 4) ||
                     (res && overlap(xq, qb, res, fb)) ||
                     (y && (overlap(y, fb, x, fb) || overlap(y, fb, g, n * 4) ||
                            (res && overlap(y, fb, res, fb)) || overlap(y, fb, xq, qb)));
    if (bad)
        return fail(KQ_ERR_ARG, "%s: an output (y=%p, xq=%p) overlaps an input or the other output",
                    fn, (void*)y, xq);
    if (rows == 0) return ok();
    if (int rc = check_device(fn, nullptr)) return rc;
    return launched(fn, kq::launch_rmsnorm_q8_1(x, res, g, eps, y, xq, rows, n, (hipStream_t)stream));
}

int kq_swiglu_q8_1(const float* gate, const float* up, float* y, void* xq, int64_t rows,
                   int64_t n, void* stream) {
    const char* fn = "kq_swiglu_q8_1";
    if (!gate || !up || !xq)
        return fail(KQ_ERR_ARG, "%s: null pointer (gate=%p up=%p xq=%p)", fn, (const void*)gate,
                    (const void*)up, xq);
    if (int rc = producer_sizes(fn, rows, n)) return rc;
    if (!aligned(gate, 16) || !aligned(up, 16) || (y && !aligned(y, 16)) || !aligned(xq, 4))
        return fail(KQ_ERR_ARG, "%s: misaligned pointer (gate=%p up=%p y=%p need 16, xq=%p needs 4)",
                    fn, (const void*)gate, (const void*)up, (void*)y, xq);
    const int64_t fb = rows * n * 4, qb = rows * (n / 32) * 36;
    const bool bad = overlap(xq, qb, gate, fb) || overlap(xq, qb, up, fb) ||
                     (y && (overlap(y, fb, gate, fb) || overlap(y, fb, up, fb) ||
                            overlap(y, fb, xq, qb)));
    if (bad)
        return fail(KQ_ERR_ARG, "%s: an output (y=%p, xq=%p) overlaps an input or the other output",
                    fn, (void*)y, xq);
    if (rows == 0) return ok();
    if (int rc = check_device(fn, nullptr)) return rc;
    return launched(fn, kq::launch_swiglu_q8_1(gate, up, y, xq, rows, n, (hipStream_t)stream));
}

const char* kq_last_error(void) { return g_err; }

int kq_abi_version(void) { return 2; }

}  // extern "C"
