// One-wave-per-row GEMV that decodes every weight on its own from its bytes.
// It accepts every shape the formats allow (k a multiple of the block size),
// including those the streaming kernel does not cover (k % 64 != 0), and
// serves as an independent device-side cross-check of the streaming kernel.
//
// Block layouts follow the GGUF formats named by rullama 0.5.0,
// src/backend/matmul.rs (fns matmul_q4_0, matmul_q4_k, matmul_q6_k,
// matmul_f16, matmul_bf16): Q4_0 = f16 d + 16 code bytes per 32 weights,
// Q4_K = f16 d, f16 dmin, 12 bytes of 6-bit scales/mins, 128 code bytes per
// 256, Q6_K = 128 bytes low bits, 64 bytes high bits, 16 int8 scales, f16 d.
// Q8_0 = f16 d + 32 signed code bytes per 32 weights, Q5_0 = f16 d, a 32-bit
// word of fifth bits and 16 code bytes per 32 (the field order of the expert
// matmul tests in src/backend/dispatch/mod.rs; element order as ggml's).
#include "qmv_internal.h"

namespace qmv {

__device__ __forceinline__ uint32_t rd16(const uint8_t *p) { return p[0] | (p[1] << 8); }

__device__ __forceinline__ float half_bits(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ float simple_weight(int fmt, const uint8_t *row, int64_t i) {
    switch (fmt) {
    case FMT_F16: return half_bits(rd16(row + 2 * i));
    case FMT_BF16: return __builtin_bit_cast(float, rd16(row + 2 * i) << 16);
    case FMT_Q4_0: {
        const uint8_t *b = row + (i >> 5) * 18;
        const int e = (int)(i & 31);
        const int q = e < 16 ? (b[2 + e] & 15) : (b[2 + e - 16] >> 4);
        return half_bits(rd16(b)) * (float)(q - 8);
    }
    case FMT_Q4_K: {
        const uint8_t *b = row + (i >> 8) * 144;
        const int e = (int)(i & 255);
        const int chunk = e >> 6, upper = (e >> 5) & 1, l = e & 31;
        const int s = 2 * chunk + upper;
        const uint8_t *sc = b + 4;
        int scale, mn;
        if (s < 4) {
            scale = sc[s] & 63;
            mn = sc[s + 4] & 63;
        } else {
            scale = (sc[s + 4] & 15) | ((sc[s - 4] >> 6) << 4);
            mn = (sc[s + 4] >> 4) | ((sc[s] >> 6) << 4);
        }
        const int q = (b[16 + 32 * chunk + l] >> (4 * upper)) & 15;
        return half_bits(rd16(b)) * (float)scale * (float)q -
               half_bits(rd16(b + 2)) * (float)mn;
    }
    case FMT_Q6_K: {
        const uint8_t *b = row + (i >> 8) * 210;
        const int e = (int)(i & 255);
        const int h = e >> 7, g = (e >> 5) & 3, l = e & 31;
        const int lo = (b[64 * h + 32 * (g & 1) + l] >> (4 * (g >> 1))) & 15;
        const int hi = (b[128 + 32 * h + l] >> (2 * g)) & 3;
        const int sc = (int8_t)b[192 + 8 * h + 2 * g + (l >> 4)];
        return half_bits(rd16(b + 208)) * (float)sc * (float)((lo | (hi << 4)) - 32);
    }
    case FMT_Q8_0: {
        const uint8_t *b = row + (i >> 5) * 34;
        return half_bits(rd16(b)) * (float)(int8_t)b[2 + (i & 31)];
    }
    case FMT_Q5_0: {
        const uint8_t *b = row + (i >> 5) * 22;
        const int e = (int)(i & 31);
        const uint32_t qh = rd16(b + 2) | (rd16(b + 4) << 16);
        const int lo = e < 16 ? (b[6 + e] & 15) : (b[6 + e - 16] >> 4);
        const int q = lo | (int)(((qh >> e) & 1u) << 4);
        return half_bits(rd16(b)) * (float)(q - 16);
    }
    default: return 0.f;
    }
}

__global__ __launch_bounds__(256) void qmv_simple(const uint8_t *__restrict__ W,
                                                   const float *__restrict__ x,
                                                   float *__restrict__ y, int64_t k, int64_t n,
                                                   int64_t m, int64_t row_bytes, int64_t j0,
                                                   int64_t j1, int accumulate, int fmt) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t j = j0 + wave; j < j1; j += nwaves) {
        const uint8_t *row = W + j * row_bytes;
        for (int64_t t = 0; t < m; t++) {
            float acc = 0.f;
            for (int64_t i = lane; i < k; i += 64)
                acc = fmaf(simple_weight(fmt, row, i), x[t * k + i], acc);
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
            if (lane == 0) {
                float *dst = y + t * n + j;
                *dst = accumulate ? *dst + acc : acc;
            }
        }
    }
}

hipError_t launch_simple(int fmt, const uint8_t *W, const float *x, float *y, int64_t k,
                         int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                         int64_t j_end, int accumulate, hipStream_t stream) {
    const int64_t rows = j_end - j_start;
    int64_t blocks = (rows + 3) / 4; // 4 waves per block, one row each
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(qmv_simple, dim3((unsigned)blocks), dim3(256), 0, stream, W, x, y, k, n,
                       m, row_bytes, j_start, j_end, accumulate, fmt);
    return hipGetLastError();
}

// Expert-indexed product, one wave per (row, pair): pair r applies expert
// ids[r] to x[r / top_k]; an expert number out of range gives NaN outputs.
__global__ __launch_bounds__(256) void qmv_simple_moe(const uint8_t *__restrict__ W,
                                                       const uint32_t *__restrict__ ids,
                                                       const float *__restrict__ x,
                                                       float *__restrict__ y, int64_t k,
                                                       int64_t n, int64_t row_bytes,
                                                       int64_t n_experts, int top_k,
                                                       int accumulate, int fmt) {
    const int lane = threadIdx.x & 63;
    const int64_t pair = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (j >= n) return;
    const uint32_t e = ids[pair];
    float *dst = y + pair * n + j;
    if ((int64_t)e >= n_experts) {
        if (lane == 0) *dst = __builtin_nanf("");
        return;
    }
    const uint8_t *row = W + ((int64_t)e * n + j) * row_bytes;
    const float *xp = x + (pair / top_k) * k;
    float acc = 0.f;
    for (int64_t i = lane; i < k; i += 64) acc = fmaf(simple_weight(fmt, row, i), xp[i], acc);
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) *dst = accumulate ? *dst + acc : acc;
}

hipError_t launch_simple_moe(int fmt, const uint8_t *W, const uint32_t *ids, const float *x,
                             float *y, int64_t k, int64_t n, int64_t row_bytes, int64_t n_experts,
                             int64_t n_pos, int top_k, int accumulate, hipStream_t stream) {
    const int64_t bx = (n + 3) / 4;
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(qmv_simple_moe, dim3((unsigned)bx, (unsigned)(n_pos * top_k)), dim3(256),
                       0, stream, W, ids, x, y, k, n, row_bytes, n_experts, top_k, accumulate,
                       fmt);
    return hipGetLastError();
}

// Transposed product, one thread per output (t, i): the rows of the range
// in order, every weight decoded on its own, the sum kept in f64.
__global__ __launch_bounds__(256) void qmv_simple_t(const uint8_t *__restrict__ W,
                                                     const float *__restrict__ dy,
                                                     float *__restrict__ dx, int64_t k, int64_t n,
                                                     int64_t m, int64_t row_bytes, int64_t j0,
                                                     int64_t j1, int accumulate, int fmt) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= m * k) return;
    const int64_t t = q / k, i = q - t * k;
    double acc = 0.0;
    for (int64_t j = j0; j < j1; j++)
        acc += (double)dy[t * n + j] * (double)simple_weight(fmt, W + j * row_bytes, i);
    dx[q] = accumulate ? dx[q] + (float)acc : (float)acc;
}

hipError_t launch_simple_t(int fmt, const uint8_t *W, const float *dy, float *dx, int64_t k,
                           int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                           int64_t j_end, int accumulate, hipStream_t stream) {
    const int64_t blocks = (m * k + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(qmv_simple_t, dim3((unsigned)blocks), dim3(256), 0, stream, W, dy, dx, k,
                       n, m, row_bytes, j_start, j_end, accumulate, fmt);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void qmv_fill_zero_all(float *__restrict__ v, int64_t count) {
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < count;
         q += (int64_t)gridDim.x * blockDim.x)
        v[q] = 0.f;
}

hipError_t launch_fill_zero_all(float *v, int64_t count, hipStream_t stream) {
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(qmv_fill_zero_all, dim3((unsigned)blocks), dim3(256), 0, stream, v, count);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void qmv_fill_zero(float *__restrict__ y, int64_t n,
                                                      int64_t m, int64_t j0, int64_t j1) {
    const int64_t rows = j1 - j0;
    const int64_t total = rows * m;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = q / rows, j = j0 + q % rows;
        y[t * n + j] = 0.f;
    }
}

hipError_t launch_fill_zero(float *y, int64_t n, int64_t m, int64_t j_start, int64_t j_end,
                            hipStream_t stream) {
    int64_t total = (j_end - j_start) * m;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(qmv_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, y, n, m,
                       j_start, j_end);
    return hipGetLastError();
}

} // namespace qmv
