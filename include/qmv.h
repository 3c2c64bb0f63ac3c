/*
 * qmv.h -- C ABI of the block-quantized matrix-vector library for AMD
 * Instinct MI355X (gfx950).
 *
 * Operation (rullama 0.5.0, src/backend/matmul.rs, module doc and the CPU
 * helper `cpu_matmul_f32` of its tests): W holds n rows of k weights, stored
 * row after row in GGUF block form; for every token t and output j,
 *
 *     y[t*n + j] = sum_{i<k} x[t*k + i] * w_j[i]
 *
 * where w_j[i] is weight i of row j decoded from its block. Batched x/y are
 * token-major, as in the batched matmul tests of the same page
 * (`x_batch[b*k..]`, `y[b*n..]`).
 *
 * Row range and accumulate (rullama 0.5.0, src/backend/dispatch/mod.rs,
 * struct MatmulBackInputParams): a call touches only outputs j_start <= j <
 * j_end, so callers can tile a vocabulary-sized product into several
 * launches; accumulate = 0 writes the result, accumulate = 1 adds it to what y
 * holds. Outputs outside the range are never read or written. (The pages
 * apply the range to the summed axis of the transposed product; here it
 * selects rows of W, i.e. outputs of the forward product.)
 *
 * All pointers are device pointers (memory from hipMalloc or a torch CUDA
 * tensor) unless stated. The caller owns every buffer; the library keeps no
 * pointer after a call returns. The GEMV and per-row families allocate no
 * memory; the matrix-core family (qmv_run_ex) and the streaming transposed
 * family (qmv_run_t_ex) take scratch from a per-device cache of at most four
 * buffers that the library keeps from call to call and frees in the last
 * qmv_destroy (each buffer as large as the largest request it served);
 * qmv_run_noalloc runs the forward families with no allocation at all.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats. Block sizes: rullama 0.5.0, src/backend/matmul.rs, fns
 * matmul_f16, matmul_bf16 (2 bytes per weight), matmul_q4_0 (18 bytes per 32),
 * matmul_q4_k (144 bytes per 256), matmul_q6_k (210 bytes per 256); Q8_0 (34
 * bytes per 32: f16 d, 32 signed codes) and Q5_0 (22 bytes per 32: f16 d, a
 * 32-bit word of fifth bits, 16 code bytes) as laid out in the expert-matmul
 * tests of src/backend/dispatch/mod.rs. */
enum qmv_format {
    QMV_FMT_F16 = 1,
    QMV_FMT_BF16 = 2,
    QMV_FMT_Q4_0 = 3,
    QMV_FMT_Q4_K = 4,
    QMV_FMT_Q6_K = 5,
    QMV_FMT_Q8_0 = 6,
    QMV_FMT_Q5_0 = 7
};

/* Kernel families selectable with qmv_run_ex. */
enum qmv_algo {
    QMV_ALGO_AUTO = 0,   /* GEMV for small m_tokens, MFMA tiles for prefill-sized m */
    QMV_ALGO_GEMV = 1,   /* streaming matvec; m_tokens handled in small groups    */
    QMV_ALGO_MFMA = 2,   /* N-token tiles on the f16 matrix cores, exact codes     */
    QMV_ALGO_SIMPLE = 3  /* one wave per row, any valid shape (slow, for checks)   */
};

/* Status codes. 0 is success; every error is negative. */
#define QMV_OK 0
#define QMV_ERR_INVALID_ARGUMENT (-1) /* bad format, shape, range or null pointer  */
#define QMV_ERR_MISALIGNED (-2)       /* W not 16-byte or x/y not 4-byte aligned    */
#define QMV_ERR_NOT_INITIALIZED (-3)  /* qmv_run before qmv_create                  */
#define QMV_ERR_NO_DEVICE (-4)        /* no HIP device visible                      */
#define QMV_ERR_UNSUPPORTED_ARCH (-5) /* current device is not gfx950               */
#define QMV_ERR_HIP (-6)              /* a HIP runtime call or launch failed        */
#define QMV_ERR_UNSUPPORTED (-7)      /* valid request this kernel family cannot do */

/* Initialise the process-wide context: counts the HIP devices and records,
 * per device, whether it is gfx950 and its compute-unit count. Reference
 * counted: every successful qmv_create needs one qmv_destroy. Returns QMV_OK,
 * QMV_ERR_NO_DEVICE when no device is visible (nothing is then initialised),
 * or QMV_ERR_UNSUPPORTED_ARCH when no visible device is gfx950. Must not race
 * with qmv_run or qmv_destroy. */
int qmv_create(void);

/* Enqueue y (=|+=) x @ W for rows [j_start, j_end) on `stream` (a hipStream_t;
 * NULL is the default stream) of the current device, with the kernel family
 * chosen automatically. Never synchronises, with two exceptions in the
 * families that take scratch (qmv_run_ex): a call that finds every free
 * cached buffer too small replaces the smallest one, and waits on the host
 * for that buffer's last use before freeing it; and the first such call on a
 * device from a second stream waits for the device to go idle. The caller
 * keeps W, x and y alive until the stream work completes.
 *
 *   format      one of enum qmv_format.
 *   W           n rows of qmv_weight_bytes(format, k, 1) bytes, 16-byte aligned.
 *   x           m_tokens x k f32, token-major, 4-byte aligned.
 *   y           m_tokens x n f32, token-major, 4-byte aligned; indexed by the
 *               absolute row j, not j - j_start.
 *   k           weights per row: a multiple of 32 (Q4_0, Q8_0, Q5_0), 256
 *               (Q4_K, Q6_K) or 2 (F16, BF16) (rullama 0.5.0,
 *               src/backend/matmul.rs, the shape checks of each matmul_*
 *               function).
 *   n           rows of W.
 *   m_tokens    number of tokens (x rows / y rows), >= 0.
 *   j_start, j_end  0 <= j_start <= j_end <= n.
 *   accumulate  0: y = result; 1: y += result (each output read once, added,
 *               written once).
 *
 * Returns QMV_OK after a successful enqueue (or when there is nothing to do:
 * m_tokens == 0 or j_start == j_end). With k == 0 the sum is empty: y is set
 * to 0, or left as is when accumulate = 1. Argument errors are detected on the
 * host before anything is enqueued; nothing is written to y then. The result
 * of one row does not depend on j_start/j_end, so any tiling of [0, n) gives
 * bit-identical outputs. Reentrant across streams and threads. */
int qmv_run(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
            int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate,
            void *stream);

/* qmv_run with an explicit kernel family (enum qmv_algo). QMV_ALGO_MFMA
 * supports every format with k a multiple of 256 (otherwise
 * QMV_ERR_UNSUPPORTED) and needs x 16-byte aligned (otherwise
 * QMV_ERR_MISALIGNED). It is the one forward family that uses scratch memory:
 * x is first rewritten into matrix-core operand order in a buffer of about
 * m_tokens*k*4.2 bytes (m_tokens rounded up to 64) from the library's
 * per-device cache. A call allocates device memory (hipMalloc, QMV_ERR_HIP if
 * that fails) only when no free cached buffer is large enough. While all
 * scratch-taking calls on a device come from one stream, its order alone
 * separates the uses of a buffer; the first such call from another stream
 * (or from hipStreamPerThread) waits once on the host for the device to go
 * idle, and from then on a call reuses a buffer last used on its own stream
 * as is and orders `stream` after the last use of one from another stream
 * with an event wait on the device. A stream handle identifies a stream:
 * destroy a stream only after the library's work on it has completed. Under
 * graph capture of `stream` the call takes the buffer with hipMallocAsync /
 * hipFreeAsync on `stream` instead.
 * QMV_ALGO_AUTO takes it when it applies, x is 16-byte aligned and m_tokens is
 * at least 3 (Q4_K), 5 (Q8_0, F16, BF16), 6 (Q4_0, Q5_0) or 8 (Q6_K), else the
 * GEMV family (which reads W once per two tokens). All families meet the same accuracy
 * contract; they may differ in the last bits. */
int qmv_run_ex(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
               int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate,
               void *stream, int algo);

/* qmv_run_ex that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, validation, kernels and results (bit for
 * bit) as qmv_run_ex. The one family that needs scratch, QMV_ALGO_MFMA, uses a
 * fixed buffer of QMV_NOALLOC_SCRATCH_BYTES in each device's memory, set up by
 * qmv_create and held until the process ends; a call whose staging would need
 * more (about m_tokens*k*4.2 bytes, m_tokens rounded up to 64) fails with
 * QMV_ERR_UNSUPPORTED before anything is enqueued when QMV_ALGO_MFMA was asked
 * for; QMV_ALGO_AUTO then runs the GEMV family instead. Every call on a device
 * shares that device's buffer and leaves its contents behind (each call
 * rewrites all it reads): matrix-core calls that overlap in time on one
 * device, e.g. on two streams, race and give wrong results. */
#define QMV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int qmv_run_noalloc(int format, const void *W, const float *x, float *y, int64_t k, int64_t n,
                    int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate,
                    void *stream, int algo);

/* Enqueue the transposed (backward-input) product over a row range on
 * `stream`, kernel family chosen automatically:
 *
 *     dx[t*k + i] (=|+=) sum_{j_start <= j < j_end} dy[t*n + j] * w_j[i]
 *
 * for every token t < m_tokens and every i < k (rullama 0.5.0,
 * src/backend/dispatch/mod.rs, struct MatmulBackInputParams: the range bounds
 * the summed row axis so that a vocabulary-sized product can be cut into
 * several calls, the first with accumulate = 0, the others with accumulate =
 * 1; the CPU reference of the backward-input parity tests maps dy of length n
 * to dx of length k).
 *
 *   format, W, k, n  as for qmv_run.
 *   dy          m_tokens x n f32, token-major, 4-byte aligned; indexed by the
 *               absolute row j.
 *   dx          m_tokens x k f32, token-major, 4-byte aligned; every entry is
 *               written (accumulate = 0) or added to (accumulate = 1).
 *   j_start, j_end  0 <= j_start <= j_end <= n; an empty range is an empty
 *               sum (dx = 0, or unchanged when accumulating).
 *
 * Returns QMV_OK after a successful enqueue, else the same codes as qmv_run.
 * The streaming family takes scratch of at most 4 MiB * k / 1024 (one
 * partial dx per workgroup) from the same per-device cache as QMV_ALGO_MFMA
 * of qmv_run_ex (QMV_ERR_HIP if an allocation fails) and is deterministic
 * run to run; a
 * split of the range into tiles changes the rounding, not the accuracy
 * contract (|error| <= 1e-4 * sum_j |dy_j * w_j[i]|). */
int qmv_run_t(int format, const void *W, const float *dy, float *dx, int64_t k, int64_t n,
              int64_t m_tokens, int64_t j_start, int64_t j_end, int accumulate,
              void *stream);

/* qmv_run_t with an explicit kernel family: QMV_ALGO_GEMV (streaming; k a
 * multiple of 64 up to 65536, else QMV_ERR_UNSUPPORTED) or QMV_ALGO_SIMPLE
 * (one thread per output, any valid shape, f64 sums; slow, for checks).
 * QMV_ALGO_MFMA is QMV_ERR_INVALID_ARGUMENT here. */
int qmv_run_t_ex(int format, const void *W, const float *dy, float *dx, int64_t k,
                 int64_t n, int64_t m_tokens, int64_t j_start, int64_t j_end,
                 int accumulate, void *stream, int algo);

/* Enqueue the expert-indexed product of a mixture-of-experts layer on
 * `stream`, kernel family chosen automatically:
 *
 *     y[r*n + j] (=|+=) sum_{i<k} x[p*k + i] * w_{e,j}[i],
 *     r = p*top_k + slot,  e = ids[r],
 *
 * for every position p < n_pos, slot < top_k and row j < n, where W stacks
 * n_experts weight matrices of n rows each ([E][n][row bytes], expert e at
 * byte e * qmv_weight_bytes(format, k, n)) (rullama 0.5.0,
 * src/backend/dispatch/mod.rs, the expert-matmul tests: stacked experts,
 * ids[pos*top_k + slot] selecting each slot's expert, x[pos] the position's
 * input).
 *
 *   ids         n_pos * top_k uint32 device values, 4-byte aligned. They are
 *               read on the device only: a value >= n_experts is not an error
 *               the host can see; it turns that slot's n outputs into NaN.
 *   x           n_pos x k f32; y: (n_pos * top_k) x n f32 (4-byte aligned).
 *   W           16-byte aligned; n_pos * top_k <= 65535.
 *   accumulate  0: y = result; 1: y += result.
 *
 * Returns QMV_OK after a successful enqueue (nothing to do when n_pos, top_k
 * or n is 0; with k == 0, y is zeroed unless accumulating and ids are not
 * read), else the codes of qmv_run. Allocates nothing. Each output row's
 * arithmetic matches qmv_run on the same expert's matrix. */
int qmv_run_moe(int format, const void *W, const uint32_t *ids, const float *x, float *y,
                int64_t k, int64_t n, int64_t n_experts, int64_t n_pos, int64_t top_k,
                int accumulate, void *stream);

/* qmv_run_moe with an explicit kernel family: QMV_ALGO_GEMV (streaming; the
 * shapes qmv_run_ex serves with it) or QMV_ALGO_SIMPLE (one wave per output,
 * any valid shape). QMV_ALGO_MFMA is QMV_ERR_INVALID_ARGUMENT here. */
int qmv_run_moe_ex(int format, const void *W, const uint32_t *ids, const float *x, float *y,
                   int64_t k, int64_t n, int64_t n_experts, int64_t n_pos, int64_t top_k,
                   int accumulate, void *stream, int algo);

/* Enqueue y (=|+=) x @ W for rows [j_start, j_end) on `stream`, W held as
 * affine group-quantized rows (moeflux, tests/graph_diff_oracle.rs, the
 * 4-bit embedding fixture and its MatvecNTokens 4-bit / 8-bit variants):
 *
 *     w_j[i] = code_j[i] * scale_j[i / 64] + bias_j[i / 64]
 *
 *   bits        4 or 8.
 *   codes       n rows of k*bits/32 little-endian u32 words, 16-byte aligned;
 *               code i of a row is bits-wide field i mod (32/bits) of word
 *               i / (32/bits), lowest bits first.
 *   scales, biases  n rows of k/64 bfloat16 values each (2-byte aligned).
 *   x, y, k, n, m_tokens, j_start, j_end, accumulate, stream  as for qmv_run;
 *               k a multiple of 64 and at most 65536 (QMV_ERR_UNSUPPORTED
 *               above).
 *
 * Returns the codes of qmv_run. Allocates nothing; deterministic; a row's
 * result does not depend on the row range. */
int qmv_run_affine(int bits, const void *codes, const void *scales, const void *biases,
                   const float *x, float *y, int64_t k, int64_t n, int64_t m_tokens,
                   int64_t j_start, int64_t j_end, int accumulate, void *stream);

/* Name of the kernel qmv_run_affine launches, or "" for an invalid request. */
const char *qmv_affine_kernel_name(int bits, int64_t k);

/* Release one reference to the context; the last one frees it, with the
 * cached scratch buffers once their last use has completed (the host waits
 * for that). Safe to call when not initialised. Must not race with qmv_run
 * or qmv_create. */
void qmv_destroy(void);

/* Bytes of W for n rows of k weights, or -1 if the format is unknown or k is
 * not a whole number of blocks (rullama 0.5.0, src/backend/matmul.rs, the
 * expected byte counts checked by each matmul_* function: k*n*2,
 * (k/32)*18*n, (k/256)*144*n, (k/256)*210*n; and (k/32)*34*n, (k/32)*22*n for
 * Q8_0 and Q5_0). Host-only; needs no context. */
int64_t qmv_weight_bytes(int format, int64_t k, int64_t n);

/* Message for the last failing call on this thread (empty if none). The
 * pointer stays valid until the next library call on the same thread. */
const char *qmv_last_error(void);

/* Short name of a status code. */
const char *qmv_status_string(int status);

/* Name of the kernel that qmv_run_ex would launch for these arguments, or ""
 * when the request is invalid. Host-only; needs no context or device. Used
 * to find the launch in profiler output. */
const char *qmv_kernel_name(int format, int64_t k, int64_t m_tokens, int algo);

/* The same for qmv_run_t_ex and qmv_run_moe_ex. */
const char *qmv_t_kernel_name(int format, int64_t k, int algo);
const char *qmv_moe_kernel_name(int format, int64_t k, int algo);

/* Launch geometry the streaming GEMV family (QMV_ALGO_GEMV) plans for `rows`
 * rows of k weights and m_tokens tokens on a device with num_cu compute units.
 * Host-only; needs no context or device. out (host memory, 8 entries)
 * receives: threads per workgroup, row slots per workgroup, lanes per slot,
 * 64-weight units per lane, rows per slot per batch, tokens per launch (1 or
 * 2), the workgroups-per-compute-unit cap of the launch, and 1 when the
 * weights are staged through LDS (block formats) else 0. Threads past
 * slots*lanes are idle padding. Returns QMV_OK, QMV_ERR_INVALID_ARGUMENT for a
 * bad format, shape, count or null out, or QMV_ERR_UNSUPPORTED when the
 * streaming kernels do not cover the shape (the per-row kernel then runs). An
 * expert-indexed launch (qmv_run_moe_ex) is planned with rows = n times the
 * number of (position, slot) pairs, except that 4-wave workgroups of 32-lane
 * rows (k = 2048) become 8-wave ones there on the terms that rows of 64 lanes
 * and more meet here (at least two 8-wave batches per compute unit). */
int qmv_gemv_geometry(int format, int64_t k, int64_t rows, int64_t m_tokens, int num_cu,
                      int64_t *out);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
