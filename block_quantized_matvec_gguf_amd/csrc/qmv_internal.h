// Internal declarations shared by the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmv {

enum Fmt {
    FMT_F16 = 1,
    FMT_BF16 = 2,
    FMT_Q4_0 = 3,
    FMT_Q4_K = 4,
    FMT_Q6_K = 5,
    FMT_Q8_0 = 6,
    FMT_Q5_0 = 7,
    // internal: affine group-64 rows (codes, scales and biases in separate arrays)
    FMT_AFFINE4 = 104,
    FMT_AFFINE8 = 108
};

// Geometry of one streaming-GEMV launch (see qmv_gemv.hip for the mapping).
struct GemvPlan {
    int fmt;
    int U;        // 64-weight units per row (k / 64)
    int UPL;      // units per lane (1 or 2)
    int L;        // lanes per row slot (ceil(U / UPL))
    int G;        // lanes per shuffle-reduction group: power of two <= 16 dividing L
    int NG;       // reduction groups per row slot (L / G)
    int P;        // row slots per workgroup
    int T;        // threads per workgroup (P * L, or 256 with idle lanes past P * L)
    int RB;       // rows per slot per batch
    int MT;       // tokens per launch (1 or 2)
    int grid;     // workgroups wanted (one per batch); the launch caps it at residency
    int num_cu;   // compute units of the device
    int x_in_lds; // stage x through LDS before loading it into registers
    int staged;   // weights go through LDS (block formats)
    int buf_bytes; // bytes of one LDS weight buffer (staged kernel)
    int npt;      // 16-byte weight pieces per thread per batch (staged kernel)
    int per_cu;   // workgroups per compute unit the launch is capped at
    size_t lds_bytes;
};

// Geometry of one N-token MFMA launch.
struct MfmaPlan {
    int fmt;
    int tiles_m, tiles_n;
    int grid;
    size_t lds_bytes;
};

// Geometry of one transposed-product launch (see qmv_gemv_t.hip).
struct GemvTPlan {
    int fmt;
    int U, UPL, L; // as in GemvPlan
    int P;         // row slots per workgroup (a power of two)
    int T;         // threads per workgroup (P * L)
    int npt;       // 16-byte weight pieces per thread per batch
    int buf_bytes; // bytes of one LDS weight buffer
    int grid;      // workgroups wanted; the launch caps it at residency
    int num_cu;
    size_t lds_bytes;
};

// Fill the geometry for a GEMV launch of up to mt_max tokens over `rows` rows.
// Returns false when the shape is outside what the streaming kernel covers.
// Row slots of at least pair_lanes lanes that fill 4 waves exactly are taken
// 8 waves at a time where there are enough batches.
bool plan_gemv(int fmt, int64_t k, int64_t rows, int mt_max, int num_cu, GemvPlan *p,
               int pair_lanes = 64);

hipError_t launch_gemv(const GemvPlan &p, const uint8_t *W, const float *x, float *y,
                       int64_t k, int64_t n, int64_t row_bytes, int64_t j_start,
                       int64_t j_end, int accumulate, hipStream_t stream);
const char *gemv_kernel_name(const GemvPlan &p);

hipError_t launch_simple(int fmt, const uint8_t *W, const float *x, float *y, int64_t k,
                         int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                         int64_t j_end, int accumulate, hipStream_t stream);

hipError_t launch_fill_zero(float *y, int64_t n, int64_t m, int64_t j_start, int64_t j_end,
                            hipStream_t stream);

// Affine group-64 rows (bits 4 or 8): codes k*bits/8 bytes per row, bf16
// scales and biases k/64 per row; y (=|+=) x @ W for rows [j_start, j_end).
hipError_t launch_affine(const GemvPlan &p, const uint8_t *codes, const uint16_t *scales,
                         const uint16_t *biases, const float *x, float *y, int64_t k, int64_t n,
                         int64_t j_start, int64_t j_end, int accumulate, hipStream_t stream);

// Expert-indexed product: pair r = p*top_k + slot of n_pos*top_k computes
// y[r] (=|+=) x[p] @ W_{ids[r]} over all n rows of that expert.
hipError_t launch_gemv_moe(const GemvPlan &p, const uint8_t *W, const uint32_t *ids,
                           const float *x, float *y, int64_t k, int64_t n, int64_t row_bytes,
                           int64_t n_experts, int64_t n_pos, int top_k, int accumulate,
                           hipStream_t stream);
const char *gemv_moe_kernel_name(const GemvPlan &p);
hipError_t launch_simple_moe(int fmt, const uint8_t *W, const uint32_t *ids, const float *x,
                             float *y, int64_t k, int64_t n, int64_t row_bytes, int64_t n_experts,
                             int64_t n_pos, int top_k, int accumulate, hipStream_t stream);

// Device scratch lent to one call by the API layer. acquire() hands out a
// buffer of at least `bytes` on the current device that work enqueued on `s`
// may use at once (the lender has already ordered `s` after the buffer's
// previous user), and in *done an event (or null) that the borrower binds as
// the stop event of the last launch touching the buffer, which marks the
// buffer's last use without an event-record packet of its own. release()
// takes the buffer back once that work is enqueued, told whether the event was
// bound (if not, the lender records it on `s` itself).
struct ScratchLender {
    virtual hipError_t acquire(size_t bytes, hipStream_t s, void **buf, hipEvent_t *done) = 0;
    virtual hipError_t release(void *buf, hipStream_t s, bool bound) = 0;

  protected:
    ~ScratchLender() = default;
};

// A kernel launch on `stream`; with a non-null `stop`, that event is bound to
// the launch's completion (hipExtLaunchKernel) instead of recorded apart.
template <class K, class... A>
void launch_stop(K kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                 hipEvent_t stop, A... args) {
    if (stop)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, nullptr, stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

// Transposed product dx (=|+=) W^T dy over rows [j_start, j_end), per token.
bool plan_gemv_t(int fmt, int64_t k, int64_t rows, int num_cu, GemvTPlan *p);
// lender: supplies the per-workgroup partials
hipError_t launch_gemv_t(const GemvTPlan &p, const uint8_t *W, const float *dy, float *dx,
                         int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                         int64_t j_end, int accumulate, ScratchLender &lender,
                         hipStream_t stream);
const char *gemv_t_kernel_name(const GemvTPlan &p);
hipError_t launch_simple_t(int fmt, const uint8_t *W, const float *dy, float *dx, int64_t k,
                           int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                           int64_t j_end, int accumulate, hipStream_t stream);
hipError_t launch_fill_zero_all(float *v, int64_t count, hipStream_t stream);

bool plan_mfma(int fmt, int64_t k, int64_t rows, int64_t m, int num_cu, MfmaPlan *p);
// lender: supplies the staging buffer
hipError_t launch_mfma(const MfmaPlan &p, const uint8_t *W, const float *x, float *y,
                       int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                       int64_t j_end, int accumulate, ScratchLender &lender,
                       hipStream_t stream);
const char *mfma_kernel_name(const MfmaPlan &p);
// Bytes of the staging buffer a matrix-core launch uses, and the launch with
// that buffer supplied by the caller (device memory, 16-byte aligned).
size_t mfma_scratch_bytes(const MfmaPlan &p, int64_t k);
// `stop` (or null): an event bound to the matrix-core kernel, the last
// reader of the buffer.
hipError_t launch_mfma_ws(const MfmaPlan &p, const uint8_t *W, const float *x, float *y,
                          int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                          int64_t j_end, int accumulate, void *scratch, hipStream_t stream,
                          hipEvent_t stop = nullptr);

// Bytes of the fixed per-device scratch of qmv_run_noalloc, and its set-up:
// *ptr becomes the device address of `device`'s copy, looked up with that
// device current (the caller's current device is restored afterwards).
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t static_scratch_init(int device, void **ptr);


} // namespace qmv
