// Streaming block-quantized GEMV for gfx950: y[t][j] (=|+=) sum_i x[t][i] * w_j[i].
//
// Operation: rullama 0.5.0, src/backend/matmul.rs (module doc: weight bytes as
// stored in GGUF, y = x @ W; the test helper cpu_matmul_f32 fixes W as n rows
// of k weights). Row range and accumulate: src/backend/dispatch/mod.rs, struct
// MatmulBackInputParams (applied here to output rows).
//
// Mapping. A row of k weights is cut into U = k/64 "units" of 64 weights. A
// workgroup holds P row slots of L lanes; lane l of a slot owns units
// l, l+L (UPL of them) for the whole launch, so the 64 x values of each owned
// unit (and the per-group sums of x the block formulas need) are loaded into
// registers once, from LDS, at kernel start. The workgroup then streams
// batches of P*RB rows: slot s takes rows base+s, base+s+P, ..., every lane
// issues the loads of its unit in all RB rows first (non-temporal, coalesced
// across the lanes of a slot), then decodes and multiplies. Per-lane partial
// sums of a row are reduced with DPP inside aligned groups of G lanes, and the
// L/G group sums go through LDS (double-buffered, one barrier per batch).
// Every row's reduction order depends only on k, never on j_start/j_end, so
// any tiling of the rows gives bit-identical outputs.
//
// Decode. 4-bit and 6-bit codes are masked into bytes and converted with
// v_cvt_f32_ubyte0..3 (one conversion per weight); the block scales are applied
// once per group in factored form, scale*sum(q*x) - min*sum(x), with the
// sums of x precomputed per lane. F16 weights go through v_fma_mix_f32; BF16
// is a shift/mask into f32.
#include "qmv_internal.h"

#include <stdio.h>

namespace qmv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 4-byte aligned multi-dword loads (dword alignment is all global loads need).
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ u32x4 ld16a4(const uint8_t *p) {
    u32x4a v = __builtin_nontemporal_load((const u32x4a *)p);
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x2 ld8a4(const uint8_t *p) {
    u32x2a v = __builtin_nontemporal_load((const u32x2a *)p);
    return u32x2{v.x, v.y};
}
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) {
    return __builtin_nontemporal_load((const uint32_t *)p);
}
__device__ __forceinline__ uint32_t ld2(const uint8_t *p) {
    return __builtin_nontemporal_load((const uint16_t *)p);
}
__device__ __forceinline__ const uint8_t *align4_down(const uint8_t *p) {
    return p - ((uintptr_t)p & 3);
}
// Keeps the compiler from folding a byte mask into per-element bit-field
// extracts, so that the byte conversions select v_cvt_f32_ubyte0..3.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}
__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xffu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }
__device__ __forceinline__ float f16lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
// acc + sum_b byte_b(q) * x[b]
__device__ __forceinline__ float dot4(uint32_t q, const float *x, float acc) {
    acc = fmaf(ub0(q), x[0], acc);
    acc = fmaf(ub1(q), x[1], acc);
    acc = fmaf(ub2(q), x[2], acc);
    acc = fmaf(ub3(q), x[3], acc);
    return acc;
}

// ------------------------------------------------------------ Q4_0 units
// A unit is two consecutive 18-byte blocks (36 bytes, dword aligned when the
// row is, i.e. when k % 64 == 0). Block layout: f16 d, 16 code bytes; element
// e < 16 is the low nibble of byte e, e >= 16 the high nibble of byte e-16;
// value d*(q-8).
struct UQ4_0 {
    struct Raw { u32x4 a, b; uint32_t c; };
    struct X { float lo[2][16], hi[2][16]; float nsum[2]; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *p = row + 36 * u;
        r.a = ld16a4(p);
        r.b = ld16a4(p + 16);
        r.c = ld4(p + 32);
    }
    static __device__ __forceinline__ void load_x(X &x, const float *xs, int u, int) {
        const float *p = xs + 64 * u;
        for (int b = 0; b < 2; b++) {
            float s = 0.f;
            for (int i = 0; i < 16; i++) {
                x.lo[b][i] = p[32 * b + i];
                x.hi[b][i] = p[32 * b + 16 + i];
            }
            for (int i = 0; i < 32; i++) s += p[32 * b + i];
            x.nsum[b] = -8.0f * s;
        }
    }
    static __device__ __forceinline__ float block(const uint32_t q[4], uint32_t dbits,
                                                  const X &x, int b) {
        float acc_lo = x.nsum[b], acc_hi = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t lo = opaque(q[j] & 0x0f0f0f0fu), hi = opaque(q[j] & 0xf0f0f0f0u);
            acc_lo = dot4(lo, &x.lo[b][4 * j], acc_lo);
            acc_hi = dot4(hi, &x.hi[b][4 * j], acc_hi); // 16x the high nibble
        }
        return f16lo(dbits) * fmaf(acc_hi, 0.0625f, acc_lo);
    }
    static __device__ __forceinline__ float dot(const Raw &r, const X &x, int) {
        uint32_t e[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.c};
        uint32_t q0[4], q1[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            q0[j] = __builtin_amdgcn_alignbyte(e[j + 1], e[j], 2); // bytes 2..17
            q1[j] = e[5 + j];                                      // bytes 20..35
        }
        return block(q0, e[0], x, 0) + block(q1, e[4] >> 16, x, 1);
    }
};

// ------------------------------------------------------------ Q4_K units
// A unit is one 64-weight chunk c of a 144-byte super-block: its 32 code
// bytes (low nibbles = sub-block 2c, high nibbles = sub-block 2c+1) plus the
// 16-byte head (f16 d, f16 dmin, 12 bytes of packed 6-bit scales/mins).
struct UQ4_K {
    struct Raw { u32x4 hd, q0, q1; };
    struct X { float lo[32], hi[32]; float slo, shi; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *sb = row + 144 * (u >> 2);
        int c = u & 3;
        r.hd = ld16(sb);
        r.q0 = ld16(sb + 16 + 32 * c);
        r.q1 = ld16(sb + 32 + 32 * c);
    }
    static __device__ __forceinline__ void load_x(X &x, const float *xs, int u, int) {
        const float *p = xs + 256 * (u >> 2) + 64 * (u & 3);
        float a = 0.f, b = 0.f;
        for (int i = 0; i < 32; i++) {
            x.lo[i] = p[i];
            x.hi[i] = p[32 + i];
        }
        for (int i = 0; i < 32; i++) a += x.lo[i];
        for (int i = 0; i < 32; i++) b += x.hi[i];
        x.slo = a;
        x.shi = b;
    }
    // 6-bit scale and min of sub-block s from the packed dwords d1..d3
    // (head bytes 4..15). s < 4: low 6 bits of byte s (scale) and byte s+4
    // (min). s >= 4: low 4 bits from the nibbles of byte s+4, top 2 bits
    // from the top bits of byte s-4 (scale) and byte s (min).
    static __device__ __forceinline__ void scale_min(uint32_t d1, uint32_t d2, uint32_t d3,
                                                     int s, uint32_t &sc, uint32_t &mn) {
        const bool low = s < 4;
        const int t = 8 * (s & 3);
        uint32_t a = low ? d1 : d3, b = low ? d2 : d3;
        int sa = t, sb = low ? t : t + 4, hs = low ? t + 4 : t + 6;
        sc = ((a >> sa) & 15u) | (((d1 >> hs) & 3u) << 4);
        mn = ((b >> sb) & 15u) | (((d2 >> hs) & 3u) << 4);
    }
    static __device__ __forceinline__ float dot(const Raw &r, const X &x, int u) {
        uint32_t q[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        float acc_lo = 0.f, acc_hi = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t lo = opaque(q[i] & 0x0f0f0f0fu), hi = opaque(q[i] & 0xf0f0f0f0u);
            acc_lo = dot4(lo, &x.lo[4 * i], acc_lo);
            acc_hi = dot4(hi, &x.hi[4 * i], acc_hi); // 16x the high nibble
        }
        const int s0 = 2 * (u & 3);
        uint32_t sc0, mn0, sc1, mn1;
        scale_min(r.hd.y, r.hd.z, r.hd.w, s0, sc0, mn0);
        scale_min(r.hd.y, r.hd.z, r.hd.w, s0 + 1, sc1, mn1);
        const float d = f16lo(r.hd.x), dmin = f16hi(r.hd.x);
        const float f0 = d * (float)sc0;
        const float f1 = (d * 0.0625f) * (float)sc1;
        const float mt = dmin * fmaf((float)mn1, x.shi, (float)mn0 * x.slo);
        return fmaf(f1, acc_hi, fmaf(f0, acc_lo, -mt));
    }
};

// ------------------------------------------------------------ Q6_K units
// A unit is (super-block, half h, lane block lq): the 64 weights
// 128h + 32g + 16lq + i (g < 4, i < 16). Their low 4 bits are bytes
// ql[64h + 16lq + i] (g = 0 low nibble, g = 2 high nibble) and
// ql[64h + 32 + 16lq + i] (g = 1, 3), their top 2 bits are bits 2g..2g+1 of
// qh[32h + 16lq + i], and their scales are the int8 scales[8h + 2g + lq].
// Super-blocks are 210 bytes, so a field may start 2 bytes off a dword
// boundary: each 16-byte field is loaded as the covering dwords and shifted
// into place with v_alignbyte_b32 (every load stays inside its super-block).
struct UQ6_K {
    struct Raw { u32x4 a, b, h; uint32_t a4, b4, h4; u32x2 s01; uint32_t s2, d, sh; };
    struct X { float v[4][16]; float nsum[4]; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *o = row + 210 * (u >> 2);
        const int h = (u >> 1) & 1, lq = u & 1;
        const uint8_t *pa = o + 64 * h + 16 * lq;
        const uint8_t *pb = pa + 32;
        const uint8_t *ph = o + 128 + 32 * h + 16 * lq;
        const uint8_t *ps = o + 192 + 8 * h;
        r.sh = (uint32_t)((uintptr_t)o & 3); // 0 or 2
        r.a = ld16a4(align4_down(pa));
        r.a4 = ld4(align4_down(pa + 14));
        r.b = ld16a4(align4_down(pb));
        r.b4 = ld4(align4_down(pb + 14));
        r.h = ld16a4(align4_down(ph));
        r.h4 = ld4(align4_down(ph + 14));
        r.s01 = ld8a4(align4_down(ps));
        r.s2 = ld4(align4_down(ps + 6));
        r.d = ld2(o + 208);
    }
    static __device__ __forceinline__ void load_x(X &x, const float *xs, int u, int) {
        const float *p = xs + 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1);
        for (int g = 0; g < 4; g++) {
            float s = 0.f;
            for (int i = 0; i < 16; i++) {
                x.v[g][i] = p[32 * g + i];
                s += x.v[g][i];
            }
            x.nsum[g] = -32.0f * s;
        }
    }
    static __device__ __forceinline__ float dot(const Raw &r, const X &x, int u) {
        const uint32_t sh = r.sh;
        uint32_t A[4], B[4], H[4];
        const uint32_t av[5] = {r.a.x, r.a.y, r.a.z, r.a.w, r.a4};
        const uint32_t bv[5] = {r.b.x, r.b.y, r.b.z, r.b.w, r.b4};
        const uint32_t hv[5] = {r.h.x, r.h.y, r.h.z, r.h.w, r.h4};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            A[j] = __builtin_amdgcn_alignbyte(av[j + 1], av[j], sh);
            B[j] = __builtin_amdgcn_alignbyte(bv[j + 1], bv[j], sh);
            H[j] = __builtin_amdgcn_alignbyte(hv[j + 1], hv[j], sh);
        }
        const uint32_t S0 = __builtin_amdgcn_alignbyte(r.s01.y, r.s01.x, sh);
        const uint32_t S1 = __builtin_amdgcn_alignbyte(r.s2, r.s01.y, sh);
        float acc[4] = {x.nsum[0], x.nsum[1], x.nsum[2], x.nsum[3]};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t q0 = opaque((A[j] & 0x0f0f0f0fu) | ((H[j] << 4) & 0x30303030u));
            const uint32_t q1 = opaque((B[j] & 0x0f0f0f0fu) | ((H[j] << 2) & 0x30303030u));
            const uint32_t q2 = opaque(((A[j] >> 4) & 0x0f0f0f0fu) | (H[j] & 0x30303030u));
            const uint32_t q3 = opaque(((B[j] >> 4) & 0x0f0f0f0fu) | ((H[j] >> 2) & 0x30303030u));
            acc[0] = dot4(q0, &x.v[0][4 * j], acc[0]);
            acc[1] = dot4(q1, &x.v[1][4 * j], acc[1]);
            acc[2] = dot4(q2, &x.v[2][4 * j], acc[2]);
            acc[3] = dot4(q3, &x.v[3][4 * j], acc[3]);
        }
        const int lq8 = 8 * (u & 1);
        const float d = f16lo(r.d);
        const float s0 = (float)__builtin_amdgcn_sbfe((int)S0, lq8, 8);
        const float s1 = (float)__builtin_amdgcn_sbfe((int)S0, lq8 + 16, 8);
        const float s2 = (float)__builtin_amdgcn_sbfe((int)S1, lq8, 8);
        const float s3 = (float)__builtin_amdgcn_sbfe((int)S1, lq8 + 16, 8);
        float r0 = (d * s0) * acc[0];
        r0 = fmaf(d * s1, acc[1], r0);
        r0 = fmaf(d * s2, acc[2], r0);
        return fmaf(d * s3, acc[3], r0);
    }
};

// ------------------------------------------------------- F16 / BF16 units
// A unit is the eight 8-weight chunks u, u+U, ..., u+7U of the row (16 bytes
// each), so that for a fixed chunk index the lanes of a slot read one
// contiguous span.
template <bool BF>
struct UHalf {
    struct Raw { u32x4 c[8]; };
    struct X { float v[8][8]; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int U) {
#pragma unroll
        for (int c = 0; c < 8; c++) r.c[c] = ld16(row + 16 * (u + U * c));
    }
    static __device__ __forceinline__ void load_x(X &x, const float *xs, int u, int U) {
        for (int c = 0; c < 8; c++)
            for (int e = 0; e < 8; e++) x.v[c][e] = xs[8 * (u + U * c) + e];
    }
    static __device__ __forceinline__ float dot(const Raw &r, const X &x, int) {
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int c = 0; c < 8; c++) {
            const uint32_t w[4] = {r.c[c].x, r.c[c].y, r.c[c].z, r.c[c].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                float lo, hi;
                if (BF) {
                    lo = __builtin_bit_cast(float, w[j] << 16);
                    hi = __builtin_bit_cast(float, w[j] & 0xffff0000u);
                } else {
                    lo = f16lo(w[j]);
                    hi = f16hi(w[j]);
                }
                acc0 = fmaf(lo, x.v[c][2 * j], acc0);
                acc1 = fmaf(hi, x.v[c][2 * j + 1], acc1);
            }
        }
        return acc0 + acc1;
    }
};

// ------------------------------------------------------------- reduction
// Sum over aligned groups of G lanes (G a power of two <= 16); every lane of
// a group ends with the group sum. Order of additions is fixed.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float group_sum(float v, int G) {
    if (G >= 2) v += dpp_mov<0xb1>(v);  // quad_perm [1,0,3,2]
    if (G >= 4) v += dpp_mov<0x4e>(v);  // quad_perm [2,3,0,1]
    if (G >= 8) v += dpp_mov<0x141>(v); // row_half_mirror
    if (G >= 16) v += dpp_mov<0x140>(v); // row_mirror
    return v;
}

// ---------------------------------------------------------------- kernel
template <class F, int MT, int UPL, int RB>
__global__ __launch_bounds__(512) void qmv_gemv(const uint8_t *__restrict__ W,
                                                 const float *__restrict__ x,
                                                 float *__restrict__ y, int64_t k, int64_t n,
                                                 int64_t row_bytes, int64_t j_start,
                                                 int64_t j_end, int accumulate, int U, int L,
                                                 int P, int G, int x_in_lds) {
    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    const int slot = tid / L;
    const int lane = tid - slot * L;
    const int NG = L / G;
    const int64_t rows_per_batch = (int64_t)P * RB;

    // ---- x: stage into LDS (coalesced), then each lane takes its units
    const float *xsrc = x;
    if (x_in_lds) {
        const int total = (int)(k * MT);
        for (int i = tid; i < total; i += blockDim.x) smem[i] = x[i];
        __syncthreads();
        xsrc = smem;
    }
    typename F::X xu[MT][UPL];
    int uid[UPL];
    bool uvalid[UPL];
#pragma unroll
    for (int i = 0; i < UPL; i++) {
        uid[i] = lane + i * L;
        uvalid[i] = uid[i] < U;
#pragma unroll
        for (int t = 0; t < MT; t++)
            if (uvalid[i]) F::load_x(xu[t][i], xsrc + t * k, uid[i], U);
    }
    float *red = smem + (x_in_lds ? k * MT : 0);
    const int red_half = P * RB * MT * NG;
    int buf = 0;

    for (int64_t base = j_start + (int64_t)blockIdx.x * rows_per_batch; base < j_end;
         base += (int64_t)gridDim.x * rows_per_batch) {
        typename F::Raw raw[RB][UPL];
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const int64_t j = base + slot + (int64_t)r * P;
            if (j < j_end) {
                const uint8_t *row = W + j * row_bytes;
#pragma unroll
                for (int i = 0; i < UPL; i++)
                    if (uvalid[i]) F::load(raw[r][i], row, uid[i], U);
            }
        }
        float part[RB][MT];
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const int64_t j = base + slot + (int64_t)r * P;
#pragma unroll
            for (int t = 0; t < MT; t++) {
                float v = 0.f;
                if (j < j_end) {
#pragma unroll
                    for (int i = 0; i < UPL; i++)
                        if (uvalid[i]) v += F::dot(raw[r][i], xu[t][i], uid[i]);
                }
                part[r][t] = group_sum(v, G);
            }
        }
        if (NG == 1) {
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < RB; r++) {
                    const int64_t j = base + slot + (int64_t)r * P;
                    if (j < j_end) {
#pragma unroll
                        for (int t = 0; t < MT; t++) {
                            float *dst = y + t * n + j;
                            *dst = accumulate ? *dst + part[r][t] : part[r][t];
                        }
                    }
                }
            }
        } else {
            float *rb = red + buf * red_half;
            if ((lane & (G - 1)) == 0) {
                const int g = lane / G;
#pragma unroll
                for (int r = 0; r < RB; r++)
#pragma unroll
                    for (int t = 0; t < MT; t++)
                        rb[((slot * RB + r) * MT + t) * NG + g] = part[r][t];
            }
            __syncthreads();
            for (int q = tid; q < P * RB * MT; q += blockDim.x) {
                const int t = q % MT;
                const int rr = q / MT; // slot * RB + r
                const int s = rr / RB, r = rr % RB;
                const int64_t j = base + s + (int64_t)r * P;
                if (j < j_end) {
                    const float *src = rb + q * NG;
                    float v = src[0];
                    for (int g = 1; g < NG; g++) v += src[g];
                    float *dst = y + t * n + j;
                    *dst = accumulate ? *dst + v : v;
                }
            }
            buf ^= 1;
        }
    }
}

// -------------------------------------------------------------- planning
static int gcd_i(int a, int b) {
    while (b) {
        int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

static int default_rb(int fmt) {
    switch (fmt) {
    case FMT_Q4_0: return 4;
    case FMT_Q4_K: return 4;
    case FMT_Q6_K: return 2;
    default: return 2; // F16 / BF16: 32 dwords of raw data per unit-row
    }
}

bool plan_gemv(int fmt, int64_t k, int64_t rows, int mt_max, int num_cu, GemvPlan *p) {
    if (k <= 0 || k % 64 != 0) return false;
    const int64_t U64 = k / 64;
    if (U64 > 1024) return false;
    GemvPlan g = {};
    g.fmt = fmt;
    g.U = (int)U64;
    g.UPL = g.U <= 512 ? 1 : 2;
    g.L = (g.U + g.UPL - 1) / g.UPL;
    g.G = g.L & -g.L;
    if (g.G > 16) g.G = 16;
    g.NG = g.L / g.G;
    g.P = 64 / gcd_i(g.L, 64);
    while (g.P * g.L * 2 <= 256) g.P *= 2;
    if (g.P * g.L > 512) g.P = 512 / g.L > 0 ? 512 / g.L : 1;
    g.T = g.P * g.L;
    g.MT = (g.UPL == 1 && mt_max >= 2) ? 2 : 1;
    g.RB = default_rb(fmt);
    int64_t batches = (rows + (int64_t)g.P * g.RB - 1) / ((int64_t)g.P * g.RB);
    if (batches < 2 * num_cu) {
        g.RB = 1;
        batches = (rows + g.P - 1) / g.P;
    }
    const int wg_per_cu = g.T <= 256 ? 8 : (g.T <= 512 ? 4 : 2);
    int64_t cap = (int64_t)num_cu * wg_per_cu;
    g.grid = (int)(batches < cap ? batches : cap);
    if (g.grid < 1) g.grid = 1;
    // LDS: the reduction buffers, plus x when everything fits in 64 KB
    // (otherwise each lane loads its x units straight from global memory).
    const size_t red = g.NG > 1 ? (size_t)2 * g.P * g.RB * g.MT * g.NG * sizeof(float) : 0;
    const size_t xb = (size_t)k * g.MT * sizeof(float);
    g.x_in_lds = (xb + red <= 64 * 1024) ? 1 : 0;
    g.lds_bytes = (g.x_in_lds ? xb : 0) + red;
    *p = g;
    return true;
}

template <class F, int MT, int UPL, int RB>
static hipError_t launch_t(const GemvPlan &p, const uint8_t *W, const float *x, float *y,
                           int64_t k, int64_t n, int64_t row_bytes, int64_t j0, int64_t j1,
                           int acc, hipStream_t s) {
    hipLaunchKernelGGL((qmv_gemv<F, MT, UPL, RB>), dim3(p.grid), dim3(p.T), p.lds_bytes, s, W,
                       x, y, k, n, row_bytes, j0, j1, acc, p.U, p.L, p.P, p.G, p.x_in_lds);
    return hipGetLastError();
}

template <class F>
static hipError_t launch_f(const GemvPlan &p, const uint8_t *W, const float *x, float *y,
                           int64_t k, int64_t n, int64_t rb, int64_t j0, int64_t j1, int acc,
                           hipStream_t s) {
    const int R = default_rb(p.fmt);
    if (p.UPL == 2) {
        if (p.RB == 1) return launch_t<F, 1, 2, 1>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        if (R == 4) return launch_t<F, 1, 2, 4>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        return launch_t<F, 1, 2, 2>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    }
    if (p.MT == 2) {
        if (p.RB == 1) return launch_t<F, 2, 1, 1>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        if (R == 4) return launch_t<F, 2, 1, 4>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        return launch_t<F, 2, 1, 2>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    }
    if (p.RB == 1) return launch_t<F, 1, 1, 1>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    if (R == 4) return launch_t<F, 1, 1, 4>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    return launch_t<F, 1, 1, 2>(p, W, x, y, k, n, rb, j0, j1, acc, s);
}

hipError_t launch_gemv(const GemvPlan &p, const uint8_t *W, const float *x, float *y,
                       int64_t k, int64_t n, int64_t row_bytes, int64_t j_start,
                       int64_t j_end, int accumulate, hipStream_t stream) {
    switch (p.fmt) {
    case FMT_Q4_0:
        return launch_f<UQ4_0>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate, stream);
    case FMT_Q4_K:
        return launch_f<UQ4_K>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate, stream);
    case FMT_Q6_K:
        return launch_f<UQ6_K>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate, stream);
    case FMT_BF16:
        return launch_f<UHalf<true>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                     stream);
    case FMT_F16:
        return launch_f<UHalf<false>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                      stream);
    default: return hipErrorInvalidValue;
    }
}

const char *gemv_kernel_name(const GemvPlan &p) {
    static const char *names[] = {"", "qmv_gemv<f16>", "qmv_gemv<bf16>", "qmv_gemv<q4_0>",
                                  "qmv_gemv<q4_k>", "qmv_gemv<q6_k>"};
    return (p.fmt >= 1 && p.fmt <= 5) ? names[p.fmt] : "";
}

} // namespace qmv
