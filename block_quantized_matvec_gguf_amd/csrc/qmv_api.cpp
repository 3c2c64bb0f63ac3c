// C ABI of the block-quantized matvec library (declared in include/qmv.h):
// argument validation (rullama 0.5.0, src/backend/matmul.rs, the checks at the
// top of each matmul_* function: block-multiple k, even k for the 16-bit
// formats, the expected weight byte count), kernel selection and launch on the
// caller's stream. Of the launches it calls, two take scratch: the
// matrix-core prefill (qmv_mfma.hip) and the streaming transposed product
// (qmv_gemv_t.hip). It comes from a per-device cache of buffers kept from
// call to call (ScratchCache below), which allocates only when no kept buffer
// is large enough; qmv_run_noalloc gives the first a fixed per-device buffer
// instead. Everything else allocates nothing.
#include "qmv.h"
#include "qmv_internal.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

static_assert(QMV_NOALLOC_SCRATCH_BYTES == qmv::STATIC_SCRATCH_BYTES,
              "the header states the size of the fixed scratch");

namespace {

// Scratch of the matrix-core and streaming transposed launches on one device:
// a few buffers kept from call to call, so that a call neither allocates nor
// frees device memory once the cache holds a buffer large enough (the
// stream-ordered allocator makes the host wait for the device at every
// allocate/free pair).
//
// While every call has come from one stream, the stream's own order keeps a
// buffer's uses apart and nothing else is tracked. The first call from a
// second stream (or from the per-thread default stream, whose handle names a
// different stream in each thread) waits on the host once for the device to
// go idle, and from then on each buffer carries the stream of its last use
// and an event bound to that use's last kernel. A call then takes, in this
// order, a free buffer large enough last used on its own stream, one whose
// last use has completed, or any free one large enough, with its stream made
// to wait on the device for that buffer's event.
//
// Failing all of these, the call allocates a buffer of its size into an empty
// slot, or in place of the smallest free buffer after waiting on the host for
// that buffer's last use. With every slot lent out to concurrent calls, or
// with the stream under graph capture, it falls back to stream-ordered
// allocation. Stream handles identify streams: a stream must not be destroyed
// while library work on it is pending.
class ScratchCache final : public qmv::ScratchLender {
  public:
    // The destructor frees nothing: it may run at process exit, after the HIP
    // runtime is gone. qmv_destroy calls clear() first.
    explicit ScratchCache(int device) : device_(device) {}

    hipError_t acquire(size_t bytes, hipStream_t s, void **buf, hipEvent_t *done) override {
        *done = nullptr;
        if (bytes == 0) bytes = 1;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(s, &cs);
        if (e != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone) return hipMallocAsync(buf, bytes, s);
        std::lock_guard<std::mutex> lk(mu_);
        if (!shared_) {
            if (!sole_seen_) {
                sole_ = s;
                sole_seen_ = true;
            }
            if (s != sole_ || s == hipStreamPerThread) {
                // every use so far, all on sole_, has completed after this
                e = hipDeviceSynchronize();
                if (e != hipSuccess) return e;
                shared_ = true;
            }
        }
        const bool own_order = s != hipStreamPerThread;
        int pick = -1;
        for (int i = 0; i < SLOTS && pick < 0; i++)
            if (fits(i, bytes) && (!shared_ || (own_order && slot_[i].last == s))) pick = i;
        for (int i = 0; i < SLOTS && pick < 0; i++)
            if (fits(i, bytes) && hipEventQuery(slot_[i].done) == hipSuccess) pick = i;
        (void)hipGetLastError(); // hipEventQuery reports hipErrorNotReady as an error
        for (int i = 0; i < SLOTS && pick < 0; i++)
            if (fits(i, bytes)) {
                e = hipStreamWaitEvent(s, slot_[i].done, 0);
                if (e != hipSuccess) return e;
                pick = i;
            }
        if (pick < 0) {
            // an empty slot, else the smallest free buffer, is (re)allocated
            for (int i = 0; i < SLOTS && pick < 0; i++)
                if (!slot_[i].ptr) pick = i;
            for (int i = 0; i < SLOTS; i++)
                if (slot_[i].ptr && !slot_[i].lent &&
                    (pick < 0 || (slot_[pick].ptr && slot_[i].bytes < slot_[pick].bytes)))
                    pick = i;
            if (pick < 0) return hipMallocAsync(buf, bytes, s); // every slot is lent out
            Slot &z = slot_[pick];
            if (z.ptr) {
                // the buffer's last use: its event, or sole_'s order before sharing
                e = shared_ ? hipEventSynchronize(z.done) : hipStreamSynchronize(sole_);
                if (e != hipSuccess) return e;
                e = hipFree(z.ptr);
                z.ptr = nullptr;
                z.bytes = 0;
                z.last = nullptr;
                if (e != hipSuccess) return e;
            }
            if (!z.done) {
                e = hipEventCreateWithFlags(&z.done, hipEventDisableTiming);
                if (e != hipSuccess) {
                    z.done = nullptr;
                    return e;
                }
            }
            e = hipMalloc(&z.ptr, bytes);
            if (e != hipSuccess) {
                z.ptr = nullptr;
                return e;
            }
            z.bytes = bytes;
        }
        slot_[pick].lent = true;
        *buf = slot_[pick].ptr;
        if (shared_) *done = slot_[pick].done;
        return hipSuccess;
    }

    hipError_t release(void *buf, hipStream_t s, bool bound) override {
        {
            std::lock_guard<std::mutex> lk(mu_);
            for (Slot &z : slot_)
                if (z.lent && z.ptr == buf) {
                    z.lent = false;
                    z.last = s;
                    // sharing may have begun while this buffer was lent out
                    return shared_ && !bound ? hipEventRecord(z.done, s) : hipSuccess;
                }
        }
        return hipFreeAsync(buf, s); // came from a fallback allocation
    }

    // Waits for the device to finish, then frees buffers and events.
    void clear() {
        std::lock_guard<std::mutex> lk(mu_);
        int cur = -1;
        const bool have_cur = hipGetDevice(&cur) == hipSuccess;
        if (hipSetDevice(device_) == hipSuccess) (void)hipDeviceSynchronize();
        for (Slot &z : slot_) {
            if (z.done) (void)hipEventDestroy(z.done);
            if (z.ptr) (void)hipFree(z.ptr);
            z = Slot();
        }
        shared_ = false;
        sole_seen_ = false;
        sole_ = nullptr;
        if (have_cur) (void)hipSetDevice(cur);
        (void)hipGetLastError();
    }

  private:
    static constexpr int SLOTS = 4;
    struct Slot {
        void *ptr = nullptr;
        size_t bytes = 0;
        hipEvent_t done = nullptr; // bound to or recorded after the last use (once shared)
        hipStream_t last = nullptr;
        bool lent = false;
    };
    bool fits(int i, size_t bytes) const {
        return slot_[i].ptr && !slot_[i].lent && slot_[i].bytes >= bytes;
    }
    int device_;
    std::mutex mu_;
    bool shared_ = false;    // a second stream has used the cache
    bool sole_seen_ = false; // sole_ holds the one stream seen so far
    hipStream_t sole_ = nullptr;
    Slot slot_[SLOTS];
};

struct DevInfo {
    bool gfx950;
    int num_cu;
    void *scratch; // this device's copy of the fixed scratch (qmv_run_noalloc)
    std::shared_ptr<ScratchCache> cache;
};

std::mutex g_mu;
std::atomic<int> g_refs{0};
std::vector<DevInfo> g_dev;
thread_local std::string t_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_err = buf;
    return code;
}

int64_t block_elems(int fmt) {
    switch (fmt) {
    case QMV_FMT_F16:
    case QMV_FMT_BF16: return 2; // the pages require even k for 16-bit weights
    case QMV_FMT_Q4_0:
    case QMV_FMT_Q8_0:
    case QMV_FMT_Q5_0: return 32;
    case QMV_FMT_Q4_K:
    case QMV_FMT_Q6_K: return 256;
    default: return -1;
    }
}

int64_t row_bytes_of(int fmt, int64_t k) {
    switch (fmt) {
    case QMV_FMT_F16:
    case QMV_FMT_BF16: return 2 * k;
    case QMV_FMT_Q4_0: return (k / 32) * 18;
    case QMV_FMT_Q4_K: return (k / 256) * 144;
    case QMV_FMT_Q6_K: return (k / 256) * 210;
    case QMV_FMT_Q8_0: return (k / 32) * 34;
    case QMV_FMT_Q5_0: return (k / 32) * 22;
    default: return -1;
    }
}

const char *fmt_name(int fmt) {
    switch (fmt) {
    case QMV_FMT_F16: return "f16";
    case QMV_FMT_BF16: return "bf16";
    case QMV_FMT_Q4_0: return "q4_0";
    case QMV_FMT_Q4_K: return "q4_k";
    case QMV_FMT_Q6_K: return "q6_k";
    case QMV_FMT_Q8_0: return "q8_0";
    case QMV_FMT_Q5_0: return "q5_0";
    default: return "?";
    }
}

// Tokens from which AUTO takes the matrix-core family. The GEMV family reads
// W once per two tokens, so its time grows with m, where the matrix-core
// call costs about the same for 1 to 32 tokens (one 32-token tile per
// workgroup) and again for 33 to 64; these are the smallest counts at which
// the matrix cores win or come within ~10% on every shape measured (k x n =
// 2560 x 10240, 2048 x 1536, 4096 x 4096, 4096 x 14336, 2560 x 262144), e.g.
// Q4_K k=4096 x 14336 with 3 tokens: 29.5 us on the GEMV family, 21 us on the
// matrix cores; with 8 tokens 69.5 and 21 us.
int mfma_min_tokens(int fmt) {
    switch (fmt) {
    case qmv::FMT_Q4_K: return 3;
    case qmv::FMT_Q8_0:
    case qmv::FMT_F16:
    case qmv::FMT_BF16: return 5;
    case qmv::FMT_Q4_0:
    case qmv::FMT_Q5_0: return 6;
    default: return 8; // Q6_K: its weights take three matrix-core terms and a costlier decode
    }
}

// Which kernel family a request resolves to; -1 when the explicit choice
// cannot serve the shape.
int resolve_algo(int fmt, int64_t k, int64_t m, int algo) {
    const bool mfma_ok = qmv::plan_mfma(fmt, k, 1, m, 256, nullptr);
    qmv::GemvPlan gp;
    const bool gemv_ok = qmv::plan_gemv(fmt, k, 1, 2, 256, &gp);
    switch (algo) {
    case QMV_ALGO_AUTO:
        if (m >= mfma_min_tokens(fmt) && mfma_ok) return QMV_ALGO_MFMA;
        return gemv_ok ? QMV_ALGO_GEMV : QMV_ALGO_SIMPLE;
    case QMV_ALGO_GEMV: return gemv_ok ? QMV_ALGO_GEMV : -1;
    case QMV_ALGO_MFMA: return mfma_ok ? QMV_ALGO_MFMA : -1;
    case QMV_ALGO_SIMPLE: return QMV_ALGO_SIMPLE;
    default: return -1;
    }
}

// Kernel family of a transposed request; -1 when the explicit choice cannot
// serve the shape.
int resolve_algo_t(int fmt, int64_t k, int algo) {
    qmv::GemvTPlan tp;
    const bool stream_ok = qmv::plan_gemv_t(fmt, k, 1 << 20, 256, &tp);
    switch (algo) {
    case QMV_ALGO_AUTO: return stream_ok ? QMV_ALGO_GEMV : QMV_ALGO_SIMPLE;
    case QMV_ALGO_GEMV: return stream_ok ? QMV_ALGO_GEMV : -1;
    case QMV_ALGO_SIMPLE: return QMV_ALGO_SIMPLE;
    default: return -1;
    }
}

} // namespace

extern "C" {

int qmv_create(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    t_err.clear();
    if (g_refs.load() > 0) {
        g_refs++;
        return QMV_OK;
    }
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(QMV_ERR_NO_DEVICE, "qmv_create: no HIP device (%s)",
                    e != hipSuccess ? hipGetErrorString(e) : "count is 0");
    }
    std::vector<DevInfo> devs((size_t)count);
    bool any = false;
    for (int d = 0; d < count; d++) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, d);
        if (e != hipSuccess)
            return fail(QMV_ERR_HIP, "qmv_create: hipGetDeviceProperties(%d): %s", d,
                        hipGetErrorString(e));
        devs[d].gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        devs[d].num_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
        any = any || devs[d].gfx950;
    }
    if (!any) return fail(QMV_ERR_UNSUPPORTED_ARCH, "qmv_create: no gfx950 device visible");
    for (int d = 0; d < count; d++) {
        devs[d].scratch = nullptr;
        if (!devs[d].gfx950) continue;
        e = qmv::static_scratch_init(d, &devs[d].scratch);
        if (e != hipSuccess)
            return fail(QMV_ERR_HIP, "qmv_create: scratch address on device %d: %s", d,
                        hipGetErrorString(e));
        devs[d].cache = std::make_shared<ScratchCache>(d);
    }
    g_dev = devs;
    g_refs = 1;
    return QMV_OK;
}

void qmv_destroy(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_refs.load() <= 0) return;
    if (--g_refs == 0) {
        // each cache waits for the last use of its buffers before freeing them
        for (DevInfo &d : g_dev)
            if (d.cache) d.cache->clear();
        g_dev.clear();
    }
}

int64_t qmv_weight_bytes(int format, int64_t k, int64_t n) {
    const int64_t qk = block_elems(format);
    if (qk <= 0 || k < 0 || n < 0 || k % qk != 0) return -1;
    return row_bytes_of(format, k) * n;
}

const char *qmv_last_error(void) { return t_err.c_str(); }

const char *qmv_status_string(int status) {
    switch (status) {
    case QMV_OK: return "QMV_OK";
    case QMV_ERR_INVALID_ARGUMENT: return "QMV_ERR_INVALID_ARGUMENT";
    case QMV_ERR_MISALIGNED: return "QMV_ERR_MISALIGNED";
    case QMV_ERR_NOT_INITIALIZED: return "QMV_ERR_NOT_INITIALIZED";
    case QMV_ERR_NO_DEVICE: return "QMV_ERR_NO_DEVICE";
    case QMV_ERR_UNSUPPORTED_ARCH: return "QMV_ERR_UNSUPPORTED_ARCH";
    case QMV_ERR_HIP: return "QMV_ERR_HIP";
    case QMV_ERR_UNSUPPORTED: return "QMV_ERR_UNSUPPORTED";
    default: return "QMV_ERR_UNKNOWN";
    }
}

const char *qmv_kernel_name(int format, int64_t k, int64_t m_tokens, int algo) {
    thread_local std::string name;
    if (block_elems(format) <= 0 || k <= 0 || k % block_elems(format) != 0 || m_tokens < 0)
        return "";
    const int a = resolve_algo(format, k, m_tokens, algo);
    if (a == QMV_ALGO_GEMV) {
        qmv::GemvPlan p;
        qmv::plan_gemv(format, k, 1, 2, 256, &p);
        name = qmv::gemv_kernel_name(p);
    } else if (a == QMV_ALGO_MFMA) {
        qmv::MfmaPlan p;
        qmv::plan_mfma(format, k, 1, m_tokens, 256, &p);
        name = qmv::mfma_kernel_name(p);
    } else if (a == QMV_ALGO_SIMPLE) {
        name = "qmv_simple";
    } else {
        name = "";
    }
    return name.c_str();
}

int qmv_gemv_geometry(int format, int64_t k, int64_t rows, int64_t m_tokens, int num_cu,
                      int64_t *out) {
    if (!out || block_elems(format) <= 0 || k <= 0 || k % block_elems(format) != 0 ||
        rows < 1 || m_tokens < 1 || num_cu < 1)
        return QMV_ERR_INVALID_ARGUMENT;
    qmv::GemvPlan p;
    if (!qmv::plan_gemv(format, k, rows, m_tokens >= 2 ? 2 : 1, num_cu, &p))
        return QMV_ERR_UNSUPPORTED;
    const int64_t g[8] = {p.T, p.P, p.L, p.UPL, p.RB, p.MT, p.per_cu, p.staged};
    for (int i = 0; i < 8; i++) out[i] = g[i];
    return QMV_OK;
}

} // extern "C"

namespace {

// qmv_run_ex and qmv_run_noalloc: the same validation and kernels; with
// fixed_scratch the matrix-core staging goes to the device's fixed scratch
// instead of stream-ordered memory.
int run_impl(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
             int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate, void *stream,
             int algo, bool fixed_scratch) {
    t_err.clear();
    // ---- host-side validation: nothing is enqueued on failure
    const int64_t qk = block_elems(format);
    if (qk <= 0) return fail(QMV_ERR_INVALID_ARGUMENT, "unknown format %d", format);
    if (k < 0 || n < 0 || m_tokens < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "negative shape k=%lld n=%lld m=%lld",
                    (long long)k, (long long)n, (long long)m_tokens);
    if (k % qk != 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "k %lld must be a multiple of %lld for %s",
                    (long long)k, (long long)qk, fmt_name(format));
    if (j_start < 0 || j_end < j_start || j_end > n)
        return fail(QMV_ERR_INVALID_ARGUMENT, "row range [%lld, %lld) outside [0, %lld)",
                    (long long)j_start, (long long)j_end, (long long)n);
    if (accumulate != 0 && accumulate != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1, got %d", accumulate);
    if (algo < QMV_ALGO_AUTO || algo > QMV_ALGO_SIMPLE)
        return fail(QMV_ERR_INVALID_ARGUMENT, "unknown algo %d", algo);
    const bool work = m_tokens > 0 && j_end > j_start;
    if (work) {
        if (!y) return fail(QMV_ERR_INVALID_ARGUMENT, "y is NULL");
        if (k > 0 && (!W || !x)) return fail(QMV_ERR_INVALID_ARGUMENT, "W or x is NULL");
        if (((uintptr_t)W & 15) != 0)
            return fail(QMV_ERR_MISALIGNED, "W must be 16-byte aligned");
        if (((uintptr_t)x & 3) != 0 || ((uintptr_t)y & 3) != 0)
            return fail(QMV_ERR_MISALIGNED, "x and y must be 4-byte aligned");
    }
    if (g_refs.load() <= 0)
        return fail(QMV_ERR_NOT_INITIALIZED, "qmv_run before qmv_create");
    if (!work) return QMV_OK;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QMV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || (size_t)dev >= g_dev.size() || !g_dev[(size_t)dev].gfx950)
        return fail(QMV_ERR_UNSUPPORTED_ARCH, "device %d is not gfx950", dev);
    const int num_cu = g_dev[(size_t)dev].num_cu;
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *Wb = (const uint8_t *)W;
    const int64_t rb = row_bytes_of(format, k);

    if (k == 0) {
        if (accumulate) return QMV_OK;
        e = qmv::launch_fill_zero(y, n, m_tokens, j_start, j_end, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "fill launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }

    int a = resolve_algo(format, k, m_tokens, algo);
    if (a < 0)
        return fail(QMV_ERR_UNSUPPORTED, "algo %d cannot serve %s with k=%lld m=%lld", algo,
                    fmt_name(format), (long long)k, (long long)m_tokens);
    if (a == QMV_ALGO_MFMA && ((uintptr_t)x & 15) != 0) {
        // the matrix-core kernel reads x in 16-byte pieces
        if (algo == QMV_ALGO_MFMA)
            return fail(QMV_ERR_MISALIGNED, "the MFMA kernel needs x 16-byte aligned");
        a = resolve_algo(format, k, 1, QMV_ALGO_AUTO);
    }
    const int64_t rows = j_end - j_start;
    if (a == QMV_ALGO_MFMA && fixed_scratch && algo == QMV_ALGO_AUTO) {
        // AUTO under the fixed scratch: a staging buffer that does not fit
        // sends the request to the GEMV family instead of failing
        qmv::MfmaPlan p;
        if (qmv::plan_mfma(format, k, rows, m_tokens, num_cu, &p) &&
            qmv::mfma_scratch_bytes(p, k) > qmv::STATIC_SCRATCH_BYTES)
            a = resolve_algo(format, k, 1, QMV_ALGO_AUTO);
    }
    if (a == QMV_ALGO_SIMPLE) {
        e = qmv::launch_simple(format, Wb, x, y, k, n, m_tokens, rb, j_start, j_end,
                               accumulate, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "simple launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    if (a == QMV_ALGO_MFMA) {
        qmv::MfmaPlan p;
        if (!qmv::plan_mfma(format, k, rows, m_tokens, num_cu, &p))
            return fail(QMV_ERR_UNSUPPORTED, "mfma plan failed");
        if (fixed_scratch) {
            const size_t need = qmv::mfma_scratch_bytes(p, k);
            if (need > qmv::STATIC_SCRATCH_BYTES)
                return fail(QMV_ERR_UNSUPPORTED,
                            "qmv_run_noalloc: the matrix-core path needs %zu bytes of scratch "
                            "for m=%lld k=%lld, above the fixed %zu",
                            need, (long long)m_tokens, (long long)k, qmv::STATIC_SCRATCH_BYTES);
            void *ws = g_dev[(size_t)dev].scratch;
            if (!ws) return fail(QMV_ERR_NOT_INITIALIZED, "no fixed scratch on device %d", dev);
            e = qmv::launch_mfma_ws(p, Wb, x, y, k, n, m_tokens, rb, j_start, j_end, accumulate,
                                    ws, s);
        } else {
            e = qmv::launch_mfma(p, Wb, x, y, k, n, m_tokens, rb, j_start, j_end, accumulate,
                                 *g_dev[(size_t)dev].cache, s);
        }
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "mfma launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    // streaming GEMV: tokens in groups of up to two per launch
    for (int64_t t0 = 0; t0 < m_tokens;) {
        qmv::GemvPlan p;
        const int mt_max = (m_tokens - t0) >= 2 ? 2 : 1;
        if (!qmv::plan_gemv(format, k, rows, mt_max, num_cu, &p))
            return fail(QMV_ERR_UNSUPPORTED, "gemv plan failed");
        e = qmv::launch_gemv(p, Wb, x + t0 * k, y + t0 * n, k, n, rb, j_start, j_end,
                             accumulate, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "gemv launch: %s", hipGetErrorString(e));
        t0 += p.MT;
    }
    return QMV_OK;
}

} // namespace

extern "C" {

int qmv_run_ex(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
               int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate, void *stream,
               int algo) {
    return run_impl(format, W, x, y, k, n, m_tokens, j_start, j_end, accumulate, stream, algo,
                    false);
}

int qmv_run_noalloc(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
                    int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate,
                    void *stream, int algo) {
    return run_impl(format, W, x, y, k, n, m_tokens, j_start, j_end, accumulate, stream, algo,
                    true);
}

int qmv_run(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
            int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate, void *stream) {
    return qmv_run_ex(format, W, x, y, k, n, m_tokens, j_start, j_end, accumulate, stream,
                      QMV_ALGO_AUTO);
}

} // extern "C"

extern "C" {

const char *qmv_t_kernel_name(int format, int64_t k, int algo) {
    thread_local std::string name;
    if (block_elems(format) <= 0 || k <= 0 || k % block_elems(format) != 0) return "";
    const int a = resolve_algo_t(format, k, algo);
    if (a == QMV_ALGO_GEMV) {
        qmv::GemvTPlan p;
        qmv::plan_gemv_t(format, k, 1 << 20, 256, &p);
        name = qmv::gemv_t_kernel_name(p);
    } else if (a == QMV_ALGO_SIMPLE) {
        name = "qmv_simple_t";
    } else {
        name = "";
    }
    return name.c_str();
}

int qmv_run_t_ex(int format, const void *W, const float *dy, float *dx, int64_t k, int64_t n,
                 int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate,
                 void *stream, int algo) {
    t_err.clear();
    const int64_t qk = block_elems(format);
    if (qk <= 0) return fail(QMV_ERR_INVALID_ARGUMENT, "unknown format %d", format);
    if (k < 0 || n < 0 || m_tokens < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "negative shape k=%lld n=%lld m=%lld",
                    (long long)k, (long long)n, (long long)m_tokens);
    if (k % qk != 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "k %lld must be a multiple of %lld for %s",
                    (long long)k, (long long)qk, fmt_name(format));
    if (j_start < 0 || j_end < j_start || j_end > n)
        return fail(QMV_ERR_INVALID_ARGUMENT, "row range [%lld, %lld) outside [0, %lld)",
                    (long long)j_start, (long long)j_end, (long long)n);
    if (accumulate != 0 && accumulate != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1, got %d", accumulate);
    if (algo != QMV_ALGO_AUTO && algo != QMV_ALGO_GEMV && algo != QMV_ALGO_SIMPLE)
        return fail(QMV_ERR_INVALID_ARGUMENT, "algo %d has no transposed form", algo);
    // every dx entry is written (or, with accumulate, added to) unless the
    // sum is empty and accumulating, or there is no output at all
    const bool sum = j_end > j_start;
    const bool work = m_tokens > 0 && k > 0 && (sum || !accumulate);
    if (work) {
        if (!dx) return fail(QMV_ERR_INVALID_ARGUMENT, "dx is NULL");
        if (sum && (!W || !dy)) return fail(QMV_ERR_INVALID_ARGUMENT, "W or dy is NULL");
        if (((uintptr_t)W & 15) != 0)
            return fail(QMV_ERR_MISALIGNED, "W must be 16-byte aligned");
        if (((uintptr_t)dy & 3) != 0 || ((uintptr_t)dx & 3) != 0)
            return fail(QMV_ERR_MISALIGNED, "dy and dx must be 4-byte aligned");
    }
    if (g_refs.load() <= 0)
        return fail(QMV_ERR_NOT_INITIALIZED, "qmv_run_t before qmv_create");
    if (!work) return QMV_OK;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QMV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || (size_t)dev >= g_dev.size() || !g_dev[(size_t)dev].gfx950)
        return fail(QMV_ERR_UNSUPPORTED_ARCH, "device %d is not gfx950", dev);
    const int num_cu = g_dev[(size_t)dev].num_cu;
    hipStream_t s = (hipStream_t)stream;
    if (!sum) {
        e = qmv::launch_fill_zero_all(dx, m_tokens * k, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "fill launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    const int a = resolve_algo_t(format, k, algo);
    if (a < 0)
        return fail(QMV_ERR_UNSUPPORTED, "algo %d cannot serve the transposed %s with k=%lld",
                    algo, fmt_name(format), (long long)k);
    const uint8_t *Wb = (const uint8_t *)W;
    const int64_t rb = row_bytes_of(format, k);
    if (a == QMV_ALGO_SIMPLE) {
        e = qmv::launch_simple_t(format, Wb, dy, dx, k, n, m_tokens, rb, j_start, j_end,
                                 accumulate, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "simple launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    qmv::GemvTPlan p;
    if (!qmv::plan_gemv_t(format, k, j_end - j_start, num_cu, &p))
        return fail(QMV_ERR_UNSUPPORTED, "transposed plan failed");
    e = qmv::launch_gemv_t(p, Wb, dy, dx, k, n, m_tokens, rb, j_start, j_end, accumulate,
                           *g_dev[(size_t)dev].cache, s);
    if (e != hipSuccess) return fail(QMV_ERR_HIP, "transposed launch: %s", hipGetErrorString(e));
    return QMV_OK;
}

int qmv_run_t(int format, const void *W, const float *dy, float *dx, int64_t k, int64_t n,
              int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate, void *stream) {
    return qmv_run_t_ex(format, W, dy, dx, k, n, m_tokens, j_start, j_end, accumulate, stream,
                        QMV_ALGO_AUTO);
}

} // extern "C"

extern "C" {

const char *qmv_moe_kernel_name(int format, int64_t k, int algo) {
    thread_local std::string name;
    if (block_elems(format) <= 0 || k <= 0 || k % block_elems(format) != 0) return "";
    qmv::GemvPlan p;
    const bool stream_ok = qmv::plan_gemv(format, k, 1, 1, 256, &p);
    const int a = algo == QMV_ALGO_AUTO ? (stream_ok ? QMV_ALGO_GEMV : QMV_ALGO_SIMPLE) : algo;
    if (a == QMV_ALGO_GEMV && stream_ok)
        name = qmv::gemv_moe_kernel_name(p);
    else if (a == QMV_ALGO_SIMPLE)
        name = "qmv_simple_moe";
    else
        name = "";
    return name.c_str();
}

int qmv_run_moe_ex(int format, const void *W, const uint32_t *ids, const float *x, float *y,
                   int64_t k, int64_t n, int64_t n_experts, int64_t n_pos, int64_t top_k,
                   int accumulate, void *stream, int algo) {
    t_err.clear();
    const int64_t qk = block_elems(format);
    if (qk <= 0) return fail(QMV_ERR_INVALID_ARGUMENT, "unknown format %d", format);
    if (k < 0 || n < 0 || n_experts < 0 || n_pos < 0 || top_k < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT,
                    "negative shape k=%lld n=%lld experts=%lld positions=%lld top_k=%lld",
                    (long long)k, (long long)n, (long long)n_experts, (long long)n_pos,
                    (long long)top_k);
    if (k % qk != 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "k %lld must be a multiple of %lld for %s",
                    (long long)k, (long long)qk, fmt_name(format));
    if (accumulate != 0 && accumulate != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1, got %d", accumulate);
    if (algo != QMV_ALGO_AUTO && algo != QMV_ALGO_GEMV && algo != QMV_ALGO_SIMPLE)
        return fail(QMV_ERR_INVALID_ARGUMENT, "algo %d has no expert-indexed form", algo);
    const int64_t pairs = n_pos * top_k;
    const bool work = pairs > 0 && n > 0;
    if (work) {
        if (pairs > 65535)
            return fail(QMV_ERR_UNSUPPORTED, "n_pos * top_k = %lld exceeds 65535",
                        (long long)pairs);
        if (!y || !ids) return fail(QMV_ERR_INVALID_ARGUMENT, "y or ids is NULL");
        if (k > 0 && (!x || (n_experts > 0 && !W)))
            return fail(QMV_ERR_INVALID_ARGUMENT, "W or x is NULL");
        if (((uintptr_t)W & 15) != 0)
            return fail(QMV_ERR_MISALIGNED, "W must be 16-byte aligned");
        if (((uintptr_t)x & 3) != 0 || ((uintptr_t)y & 3) != 0 || ((uintptr_t)ids & 3) != 0)
            return fail(QMV_ERR_MISALIGNED, "x, y and ids must be 4-byte aligned");
    }
    if (g_refs.load() <= 0)
        return fail(QMV_ERR_NOT_INITIALIZED, "qmv_run_moe before qmv_create");
    if (!work) return QMV_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QMV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || (size_t)dev >= g_dev.size() || !g_dev[(size_t)dev].gfx950)
        return fail(QMV_ERR_UNSUPPORTED_ARCH, "device %d is not gfx950", dev);
    const int num_cu = g_dev[(size_t)dev].num_cu;
    hipStream_t s = (hipStream_t)stream;
    if (k == 0) {
        if (accumulate) return QMV_OK;
        e = qmv::launch_fill_zero_all(y, pairs * n, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "fill launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    const uint8_t *Wb = (const uint8_t *)W;
    const int64_t rb = row_bytes_of(format, k);
    qmv::GemvPlan p;
    // planned over the launch's rows, all pairs together: planned per expert,
    // the rule that gives small products fewer row slots per workgroup cut a
    // 1536-row expert to 2-wave workgroups (Q4_K k=2048 x 1536, 8 experts:
    // 10.8 -> 9.1 us; k=2560: 12.0 -> 8.8 us; outputs bit-identical); 32-lane
    // rows (k=2048) that fill 4 waves exactly run 8 waves per workgroup, as
    // wider rows do in every launch (Q4_K k=2048 x 1536, 8 experts: 9.3 -> 8.4 us)
    const bool stream_ok = qmv::plan_gemv(format, k, n * pairs, 1, num_cu, &p, 32);
    if (algo == QMV_ALGO_GEMV && !stream_ok)
        return fail(QMV_ERR_UNSUPPORTED, "algo %d cannot serve %s with k=%lld", algo,
                    fmt_name(format), (long long)k);
    if (algo == QMV_ALGO_SIMPLE || !stream_ok) {
        e = qmv::launch_simple_moe(format, Wb, ids, x, y, k, n, rb, n_experts, n_pos,
                                   (int)top_k, accumulate, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "simple launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    e = qmv::launch_gemv_moe(p, Wb, ids, x, y, k, n, rb, n_experts, n_pos, (int)top_k,
                             accumulate, s);
    if (e != hipSuccess) return fail(QMV_ERR_HIP, "expert launch: %s", hipGetErrorString(e));
    return QMV_OK;
}

int qmv_run_moe(int format, const void *W, const uint32_t *ids, const float *x, float *y,
                int64_t k, int64_t n, int64_t n_experts, int64_t n_pos, int64_t top_k,
                int accumulate, void *stream) {
    return qmv_run_moe_ex(format, W, ids, x, y, k, n, n_experts, n_pos, top_k, accumulate,
                          stream, QMV_ALGO_AUTO);
}

} // extern "C"

extern "C" {

const char *qmv_affine_kernel_name(int bits, int64_t k) {
    if ((bits != 4 && bits != 8) || k <= 0 || k % 64 != 0) return "";
    qmv::GemvPlan p;
    if (!qmv::plan_gemv(bits == 4 ? qmv::FMT_AFFINE4 : qmv::FMT_AFFINE8, k, 1, 1, 256, &p))
        return "";
    return bits == 4 ? "qmv_affine_gemv<4>" : "qmv_affine_gemv<8>";
}

int qmv_run_affine(int bits, const void *codes, const void *scales, const void *biases,
                   const float *x, float *y, int64_t k, int64_t n, int64_t m_tokens,
                   int64_t j_start, int64_t j_end, int accumulate, void *stream) {
    t_err.clear();
    if (bits != 4 && bits != 8)
        return fail(QMV_ERR_INVALID_ARGUMENT, "bits must be 4 or 8, got %d", bits);
    if (k < 0 || n < 0 || m_tokens < 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "negative shape k=%lld n=%lld m=%lld",
                    (long long)k, (long long)n, (long long)m_tokens);
    if (k % 64 != 0)
        return fail(QMV_ERR_INVALID_ARGUMENT, "k %lld must be a multiple of the group size 64",
                    (long long)k);
    if (j_start < 0 || j_end < j_start || j_end > n)
        return fail(QMV_ERR_INVALID_ARGUMENT, "row range [%lld, %lld) outside [0, %lld)",
                    (long long)j_start, (long long)j_end, (long long)n);
    if (accumulate != 0 && accumulate != 1)
        return fail(QMV_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1, got %d", accumulate);
    const bool work = m_tokens > 0 && j_end > j_start;
    if (work) {
        if (!y) return fail(QMV_ERR_INVALID_ARGUMENT, "y is NULL");
        if (k > 0 && (!codes || !scales || !biases || !x))
            return fail(QMV_ERR_INVALID_ARGUMENT, "codes, scales, biases or x is NULL");
        if (((uintptr_t)codes & 15) != 0)
            return fail(QMV_ERR_MISALIGNED, "codes must be 16-byte aligned");
        if (((uintptr_t)scales & 1) != 0 || ((uintptr_t)biases & 1) != 0)
            return fail(QMV_ERR_MISALIGNED, "scales and biases must be 2-byte aligned");
        if (((uintptr_t)x & 3) != 0 || ((uintptr_t)y & 3) != 0)
            return fail(QMV_ERR_MISALIGNED, "x and y must be 4-byte aligned");
    }
    if (g_refs.load() <= 0)
        return fail(QMV_ERR_NOT_INITIALIZED, "qmv_run_affine before qmv_create");
    if (!work) return QMV_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QMV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || (size_t)dev >= g_dev.size() || !g_dev[(size_t)dev].gfx950)
        return fail(QMV_ERR_UNSUPPORTED_ARCH, "device %d is not gfx950", dev);
    const int num_cu = g_dev[(size_t)dev].num_cu;
    hipStream_t s = (hipStream_t)stream;
    if (k == 0) {
        if (accumulate) return QMV_OK;
        e = qmv::launch_fill_zero(y, n, m_tokens, j_start, j_end, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "fill launch: %s", hipGetErrorString(e));
        return QMV_OK;
    }
    const int fmt = bits == 4 ? qmv::FMT_AFFINE4 : qmv::FMT_AFFINE8;
    const int64_t rows = j_end - j_start;
    for (int64_t t0 = 0; t0 < m_tokens;) {
        qmv::GemvPlan p;
        const int mt_max = (m_tokens - t0) >= 2 ? 2 : 1;
        if (!qmv::plan_gemv(fmt, k, rows, mt_max, num_cu, &p))
            return fail(QMV_ERR_UNSUPPORTED, "affine plan failed for k=%lld", (long long)k);
        e = qmv::launch_affine(p, (const uint8_t *)codes, (const uint16_t *)scales,
                               (const uint16_t *)biases, x + t0 * k, y + t0 * n, k, n, j_start,
                               j_end, accumulate, s);
        if (e != hipSuccess) return fail(QMV_ERR_HIP, "affine launch: %s", hipGetErrorString(e));
        t0 += p.MT;
    }
    return QMV_OK;
}

} // extern "C"
