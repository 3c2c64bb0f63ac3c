// N-token (prefill) kernel for gfx950 matrix cores:
//   Y[t][j] (=|+=) sum_i X[t][i] * w_j[i]   for many tokens t at once.
//
// Operation: rullama 0.5.0, src/backend/matmul.rs (y = x @ W over weight rows
// stored in GGUF form; the batched variant runs the same product for several
// rows of x). Block layout of Q4_K: 144-byte super-blocks of 256 weights, d and
// dmin (f16), eight 6-bit scales and mins packed in 12 bytes, 128 code bytes
// (the ggml reading of the format the page calls ggml-exact).
//
// Exactness. The 4-bit codes q are small integers, exact in bf16. x is split
// as hi = bf16(x), lo = bf16(x - hi); hi + lo keeps 16 significant bits
// (relative error below 2^-16). The MFMA multiplies codes by hi and by lo and
// accumulates the products of one 32-weight sub-block in f32 into a fresh
// tile, which an f32 FMA then scales by d*scale. The min term,
// dmin * sum_g min_g * sum(x over sub-block g), takes one more MFMA per
// super-block: the per-sub-block sums of x (f32, fixed order) split hi/lo,
// against the 6-bit mins (exact).
//
// Mapping. A workgroup owns a tile of 64 tokens x 64 rows and has 8 waves;
// the K dimension is split over the waves (wave w takes super-blocks w, w+8,
// ...), and every wave holds the whole tile as four 32x32 accumulators
// (v_mfma_f32_32x32x16_bf16: lane l feeds A[l%32][8(l/32)+i] and
// B[8(l/32)+i][l%32] and receives D[8(r/4)+4(l/32)+r%4][l%32] in register r).
// Tokens are the MFMA rows, weight rows the columns, so a lane's outputs all
// belong to one weight row and its block scales are per-lane scalars. x and
// the weight bytes go straight from memory into registers; the eight partial
// tiles are summed in LDS in a fixed order. Results depend only on k, never
// on the row range or the token tiling.
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MW = 8;         // waves per workgroup (split of K)
constexpr int TM = 64;        // tokens per workgroup
constexpr int TN = 64;        // weight rows per workgroup
constexpr int NT = 64 * MW;   // threads per workgroup
constexpr size_t RED_BYTES = (size_t)MW * TM * TN * sizeof(float);

__device__ __forceinline__ u32x4 ldw(const uint8_t *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ f32x4 ldx(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}
// Hide a value from the optimiser so that byte extractions stay single
// v_cvt_f32_ubyteN instructions instead of being folded into bit-field ops.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// x = hi + lo, both bf16, for 8 consecutive values. Pairs are rounded with
// one v_cvt_pk_bf16_f32; hi comes back to f32 exactly by placing its bits in
// the upper half of a word, so x - hi is exact and only lo rounds.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pk_bf16(a, b);
    const float ha = __builtin_bit_cast(float, hi << 16);
    const float hb = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = pk_bf16(a - ha, b - hb);
}
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split2(a[0], a[1], h0, l0);
    split2(a[2], a[3], h1, l1);
    split2(b[0], b[1], h2, l2);
    split2(b[2], b[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

// Eight codes (one per byte of u0, u1, each 0..63) as exact bf16 values.
__device__ __forceinline__ bf16x8 bytes8(uint32_t u0, uint32_t u1) {
    u0 = opaque(u0);
    u1 = opaque(u1);
    bf16x8 b;
    b[0] = (__bf16)(float)(u0 & 0xffu);
    b[1] = (__bf16)(float)((u0 >> 8) & 0xffu);
    b[2] = (__bf16)(float)((u0 >> 16) & 0xffu);
    b[3] = (__bf16)(float)(u0 >> 24);
    b[4] = (__bf16)(float)(u1 & 0xffu);
    b[5] = (__bf16)(float)((u1 >> 8) & 0xffu);
    b[6] = (__bf16)(float)((u1 >> 16) & 0xffu);
    b[7] = (__bf16)(float)(u1 >> 24);
    return b;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Byte i (0..11) of the packed scale/min field of a Q4_K header.
__device__ __forceinline__ uint32_t scb(const u32x4 &h, int i) {
    return (h[1 + (i >> 2)] >> (8 * (i & 3))) & 0xffu;
}

__global__ __launch_bounds__(NT) void qmv_mfma_q4_k(const uint8_t *__restrict__ W,
                                                    const float *__restrict__ x,
                                                    float *__restrict__ y, int64_t k, int64_t n,
                                                    int64_t m, int64_t row_bytes,
                                                    int64_t j_start, int64_t j_end,
                                                    int accumulate) {
    extern __shared__ float red[]; // [MW][TM][TN] partial tiles
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nl = lane & 31, jh = lane >> 5;
    const int64_t r0 = j_start + (int64_t)blockIdx.x * TN;
    const int64_t t0 = (int64_t)blockIdx.y * TM;
    const int nsb = (int)(k >> 8);

    // Rows and tokens beyond the tile's end are clamped for loading; their
    // results are never stored.
    const uint8_t *wr[2];
    const float *xr[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        int64_t r = r0 + nl + 32 * i;
        r = r < j_end ? r : j_end - 1;
        wr[i] = W + r * row_bytes;
        int64_t t = t0 + nl + 32 * i;
        t = t < m ? t : m - 1;
        xr[i] = x + t * k + 16 * jh;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[a][b][r] = 0.f;

    for (int s = wave; s < nsb; s += MW) {
        // This lane's bytes of the super-block of its two rows: the header
        // and, of each 32-byte code chunk c, the 16 bytes 16*jh..16*jh+15.
        u32x4 hd[2], qs[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const uint8_t *p = wr[rb] + (int64_t)144 * s;
            hd[rb] = ldw(p);
#pragma unroll
            for (int c = 0; c < 4; c++) qs[rb][c] = ldw(p + 16 + 32 * c + 16 * jh);
        }
        float dsc[2][8], dmin[2];
        bf16x8 mins[2];
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const float d = h2f(hd[rb][0]);
            dmin[rb] = h2f(hd[rb][0] >> 16);
#pragma unroll
            for (int g = 0; g < 8; g++) {
                uint32_t sc, mn;
                if (g < 4) {
                    sc = scb(hd[rb], g) & 63u;
                    mn = scb(hd[rb], g + 4) & 63u;
                } else {
                    sc = (scb(hd[rb], g + 4) & 15u) | ((scb(hd[rb], g - 4) >> 6) << 4);
                    mn = (scb(hd[rb], g + 4) >> 4) | ((scb(hd[rb], g) >> 6) << 4);
                }
                dsc[rb][g] = d * (float)sc;
                mins[rb][g] = (__bf16)(float)mn;
            }
        }

        const float *xs[2] = {xr[0] + 256 * s, xr[1] + 256 * s};
        float xsum[2][8]; // this lane's 16 of the 32 x values of sub-block g, summed
#pragma unroll
        for (int g = 0; g < 8; g++) {
            const int c = g >> 1, h = g & 1;
            // A operands of both K-steps: elements 32g + 16jh + 8tp + (0..7)
            bf16x8 ah[2][2], al[2][2];
#pragma unroll
            for (int tb = 0; tb < 2; tb++) {
                float sum = 0.f;
#pragma unroll
                for (int tp = 0; tp < 2; tp++) {
                    const f32x4 a0 = ldx(xs[tb] + 32 * g + 8 * tp);
                    const f32x4 a1 = ldx(xs[tb] + 32 * g + 8 * tp + 4);
                    split8(a0, a1, ah[tb][tp], al[tb][tp]);
                    sum += ((a0[0] + a0[1]) + (a0[2] + a0[3])) + ((a1[0] + a1[1]) + (a1[2] + a1[3]));
                }
                xsum[tb][g] = sum;
            }
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                // codes of elements 16jh + 8tp + (0..7): bytes 8tp..8tp+7 of the
                // lane's 16-byte piece, low nibbles for g even, high for g odd
                bf16x8 bq[2];
#pragma unroll
                for (int tp = 0; tp < 2; tp++) {
                    uint32_t u0 = qs[rb][c][2 * tp], u1 = qs[rb][c][2 * tp + 1];
                    if (h) {
                        u0 >>= 4;
                        u1 >>= 4;
                    }
                    bq[tp] = bytes8(u0 & 0x0f0f0f0fu, u1 & 0x0f0f0f0fu);
                }
#pragma unroll
                for (int tb = 0; tb < 2; tb++) {
                    f32x16 t = mfma(ah[tb][0], bq[0], f32x16{});
                    t = mfma(al[tb][0], bq[0], t);
                    t = mfma(ah[tb][1], bq[1], t);
                    t = mfma(al[tb][1], bq[1], t);
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[tb][rb][r] = fmaf(dsc[rb][g], t[r], acc[tb][rb][r]);
                }
            }
        }
        // Min term: A = [sum_hi(g=0..7) | sum_lo(g=0..7)] per token, B = [min_g | min_g].
#pragma unroll
        for (int tb = 0; tb < 2; tb++) {
            bf16x8 am;
#pragma unroll
            for (int g = 0; g < 8; g++) {
                const float p = xsum[tb][g];
                const float q = __builtin_bit_cast(
                    float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, p)));
                const float sg = p + q; // same value in both lanes of the pair
                const __bf16 sh = (__bf16)sg;
                am[g] = jh ? (__bf16)(sg - (float)sh) : sh;
            }
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const f32x16 t = mfma(am, mins[rb], f32x16{});
#pragma unroll
                for (int r = 0; r < 16; r++) acc[tb][rb][r] = fmaf(-dmin[rb], t[r], acc[tb][rb][r]);
            }
        }
    }

    // Sum the partial tiles of the waves in wave order, then store.
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int mm = 32 * tb + 8 * (r >> 2) + 4 * jh + (r & 3);
                red[(wave * TM + mm) * TN + 32 * rb + nl] = acc[tb][rb][r];
            }
    __syncthreads();
    for (int i = tid; i < TM * TN; i += NT) {
        float v = red[i];
#pragma unroll
        for (int w = 1; w < MW; w++) v += red[w * TM * TN + i];
        const int64_t t = t0 + i / TN, j = r0 + i % TN;
        if (t < m && j < j_end) {
            float *dst = y + t * n + j;
            *dst = accumulate ? *dst + v : v;
        }
    }
}

} // namespace

bool plan_mfma(int fmt, int64_t k, int64_t rows, int64_t m, int num_cu, MfmaPlan *p) {
    if (fmt != FMT_Q4_K || k <= 0 || (k % 256) != 0 || m < 1) return false;
    // row offsets of a 64-row tile and x offsets of a 64-token tile stay in 64 bits;
    // per-lane element offsets within a row (< k) must fit in 32 bits
    if (k > ((int64_t)1 << 30)) return false;
    if (p) {
        p->fmt = fmt;
        p->tiles_n = (int)((rows + TN - 1) / TN);
        p->tiles_m = (int)((m + TM - 1) / TM);
        p->grid = p->tiles_n * p->tiles_m;
        p->lds_bytes = RED_BYTES;
        (void)num_cu;
    }
    return true;
}

hipError_t launch_mfma(const MfmaPlan &p, const uint8_t *W, const float *x, float *y, int64_t k,
                       int64_t n, int64_t m, int64_t row_bytes, int64_t j_start, int64_t j_end,
                       int accumulate, hipStream_t stream) {
    if (p.fmt != FMT_Q4_K) return hipErrorInvalidValue;
    if (p.tiles_m > 65535) return hipErrorInvalidConfiguration;
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)qmv_mfma_q4_k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)RED_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(qmv_mfma_q4_k, dim3(p.tiles_n, p.tiles_m), dim3(NT), RED_BYTES, stream, W,
                       x, y, k, n, m, row_bytes, j_start, j_end, accumulate);
    return hipGetLastError();
}

const char *mfma_kernel_name(const MfmaPlan &p) {
    return p.fmt == FMT_Q4_K ? "qmv_mfma<q4_k>" : "";
}

} // namespace qmv
