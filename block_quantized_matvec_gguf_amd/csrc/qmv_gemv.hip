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
// Decode. Codes are masked into bytes and converted with one instruction per
// weight: Q4_0 and Q6_K codes as signed bytes holding a multiple of q-8 or
// q-32 (SDWA sign-extended v_cvt_f32_i32), Q4_K codes as unsigned bytes
// (v_cvt_f32_ubyte0..3). Block scales are applied once per group; the Q4_K min
// term is applied in factored form, dmin*m*sum(x), with the sums of x
// precomputed per lane. F16 weights go through v_fma_mix_f32; BF16 is a
// shift/mask into f32.
#include "qmv_internal.h"

#include <map>
#include <mutex>
#include <utility>

namespace qmv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
// Signed bytes: each selects v_cvt_f32_i32 with an SDWA sign-extended byte.
__device__ __forceinline__ float sb0(uint32_t v) { return (float)(int)(int8_t)(v & 0xffu); }
__device__ __forceinline__ float sb1(uint32_t v) { return (float)(int)(int8_t)((v >> 8) & 0xffu); }
__device__ __forceinline__ float sb2(uint32_t v) { return (float)(int)(int8_t)((v >> 16) & 0xffu); }
__device__ __forceinline__ float sb3(uint32_t v) { return (float)((int)v >> 24); }
// acc + sum_b signed_byte_b(q) * x[b]
__device__ __forceinline__ float sdot4(uint32_t q, const float *x, float acc) {
    acc = fmaf(sb0(q), x[0], acc);
    acc = fmaf(sb1(q), x[1], acc);
    acc = fmaf(sb2(q), x[2], acc);
    acc = fmaf(sb3(q), x[3], acc);
    return acc;
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
// value d*(q-8). The signed code q-8 is the 4-bit two's-complement reading of
// q^8: each nibble is XORed with 8 and moved to the top of its byte, where a
// sign-extending byte conversion yields 16*(q-8) exactly. Summing signed
// codes keeps the rounding error proportional to sum|w*x| (an all-8 block
// gives exactly 0).
struct UQ4_0 {
    struct Raw { u32x4 a, b; uint32_t c; };
    struct X { float lo[2][16], hi[2][16]; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *p = row + 36 * u;
        r.a = ld16a4(p);
        r.b = ld16a4(p + 16);
        r.c = ld4(p + 32);
    }
    // x of unit u as 16 float4 pieces: piece i is x4[16u + i]
    static __device__ __forceinline__ int x4_index(int u, int i, int) { return 16 * u + i; }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = q >> 4;
        i = q & 15;
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        const int b = i >> 3, j = i & 7;
        float *d = j < 4 ? &x.lo[b][4 * j] : &x.hi[b][4 * (j - 4)];
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    static __device__ __forceinline__ void finish_x(X &) {}
    static __device__ __forceinline__ float block(const uint32_t q[4], uint32_t dbits,
                                                  const X &x, int b) {
        float acc_lo = 0.f, acc_hi = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            // bytes of 16*(q-8): low nibbles moved up, then both XOR 8 in the top nibble
            const uint32_t lo = opaque(((q[j] << 4) ^ 0x80808080u) & 0xf0f0f0f0u);
            const uint32_t hi = opaque((q[j] ^ 0x80808080u) & 0xf0f0f0f0u);
            acc_lo = sdot4(lo, &x.lo[b][4 * j], acc_lo);
            acc_hi = sdot4(hi, &x.hi[b][4 * j], acc_hi);
        }
        return (f16lo(dbits) * 0.0625f) * (acc_lo + acc_hi);
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
    // x of unit u (weights 64u .. 64u+63) as 16 float4 pieces
    static __device__ __forceinline__ int x4_index(int u, int i, int) { return 16 * u + i; }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = q >> 4;
        i = q & 15;
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        float *d = i < 8 ? &x.lo[4 * i] : &x.hi[4 * (i - 8)];
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    static __device__ __forceinline__ void finish_x(X &x) {
        float a = 0.f, b = 0.f;
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
// The signed code q-32 is the 6-bit two's-complement reading of q^32: the
// high 2-bit fields are XORed with 0b10, the 6-bit code is assembled in the
// top of its byte, and a sign-extending byte conversion yields 4*(q-32).
struct UQ6_K {
    struct Raw { u32x4 a, b, h; uint32_t a4, b4, h4; u32x2 s01; uint32_t s2, d, sh; };
    struct X { float v[4][16]; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *o = row + 210 * (u >> 2);
        const int h = (u >> 1) & 1, lq = u & 1;
        const int fa = 64 * h + 16 * lq, fh = 128 + 32 * h + 16 * lq, fs = 192 + 8 * h;
        // sh = 0 or 2. al = o - sh is dword aligned; every field's covering
        // dwords start at al + offset, and the dword after each 16-byte field
        // (needed only when sh = 2) sits at o + sh + offset + 12, which for
        // sh = 0 re-reads the field's last dword. Nothing reaches past the
        // super-block's last byte.
        const uint32_t sh = (uint32_t)(uintptr_t)o & 3u;
        const uint8_t *al = o - sh;
        const uint8_t *tl = o + sh;
        r.sh = sh;
        r.a = ld16a4(al + fa);
        r.a4 = ld4(tl + fa + 12);
        r.b = ld16a4(al + fa + 32);
        r.b4 = ld4(tl + fa + 44);
        r.h = ld16a4(al + fh);
        r.h4 = ld4(tl + fh + 12);
        r.s01 = ld8a4(al + fs);
        r.s2 = ld4(tl + fs + 4);
        r.d = ld2(o + 208);
    }
    // x of unit u: piece i = 4g + i4 holds weights 128h + 32g + 16lq + 4i4 .. +3
    static __device__ __forceinline__ int x4_index(int u, int i, int) {
        return 64 * (u >> 2) + 32 * ((u >> 1) & 1) + 8 * (i >> 2) + 4 * (u & 1) + (i & 3);
    }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = 4 * (q >> 6) + 2 * ((q >> 5) & 1) + ((q >> 2) & 1);
        i = 4 * ((q >> 3) & 3) + (q & 3);
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        float *d = &x.v[i >> 2][4 * (i & 3)];
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    static __device__ __forceinline__ void finish_x(X &) {}
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
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t h = H[j] ^ 0xaaaaaaaau; // top bit of every 2-bit field flipped
            // bytes of 4*(q-32) for quarters g = 0..3
            const uint32_t q0 = opaque(((A[j] << 2) & 0x3c3c3c3cu) | ((h << 6) & 0xc0c0c0c0u));
            const uint32_t q1 = opaque(((B[j] << 2) & 0x3c3c3c3cu) | ((h << 4) & 0xc0c0c0c0u));
            const uint32_t q2 = opaque(((A[j] >> 2) & 0x3c3c3c3cu) | ((h << 2) & 0xc0c0c0c0u));
            const uint32_t q3 = opaque(((B[j] >> 2) & 0x3c3c3c3cu) | (h & 0xc0c0c0c0u));
            acc[0] = sdot4(q0, &x.v[0][4 * j], acc[0]);
            acc[1] = sdot4(q1, &x.v[1][4 * j], acc[1]);
            acc[2] = sdot4(q2, &x.v[2][4 * j], acc[2]);
            acc[3] = sdot4(q3, &x.v[3][4 * j], acc[3]);
        }
        const int lq8 = 8 * (u & 1);
        const float d = f16lo(r.d) * 0.25f;
        // the scale bytes are signed: extract with sign extension, convert as int
        const float s0 = (float)(int)__builtin_amdgcn_sbfe((int)S0, lq8, 8);
        const float s1 = (float)(int)__builtin_amdgcn_sbfe((int)S0, lq8 + 16, 8);
        const float s2 = (float)(int)__builtin_amdgcn_sbfe((int)S1, lq8, 8);
        const float s3 = (float)(int)__builtin_amdgcn_sbfe((int)S1, lq8 + 16, 8);
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
    // x of unit u: piece i = 2c + hf holds weights 8(u + cU) + 4hf .. +3
    static __device__ __forceinline__ int x4_index(int u, int i, int U) {
        return 2 * (u + U * (i >> 1)) + (i & 1);
    }
    static __device__ __forceinline__ void x4_slot(int q, int U, int &u, int &i) {
        const int chunk = q >> 1;
        const int c = chunk / U;
        u = chunk - c * U;
        i = 2 * c + (q & 1);
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        float *d = &x.v[i >> 1][4 * (i & 1)];
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    static __device__ __forceinline__ void finish_x(X &) {}
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
// Workgroup barrier that orders LDS only: global loads in flight (the next
// batch of weights) are not drained, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class F, int MT, int UPL, int RB>
__global__ __launch_bounds__(512) void qmv_gemv(const uint8_t *__restrict__ W,
                                                 const float *__restrict__ x,
                                                 float *__restrict__ y, int64_t k, int64_t n,
                                                 int64_t row_bytes, int64_t j_start,
                                                 int64_t j_end, int accumulate, int U, int L,
                                                 int P, int G, int x_in_lds) {
    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    const int T = blockDim.x;
    const int slot = tid / L;
    const int lane = tid - slot * L;
    const int NG = L / G;
    const int64_t rows_per_batch = (int64_t)P * RB;
    const int64_t stride = (int64_t)gridDim.x * rows_per_batch;
    const uint8_t *Wslot = W + (int64_t)slot * row_bytes;

    int uid[UPL];  // units owned by this lane
    int ulod[UPL]; // unit actually loaded: padding lanes re-read a valid unit
    bool uvalid[UPL];
#pragma unroll
    for (int i = 0; i < UPL; i++) {
        uid[i] = lane + i * L;
        uvalid[i] = uid[i] < U;
        ulod[i] = uvalid[i] ? uid[i] : U - 1;
    }

    // 1. x, first part: coalesced float4 loads into registers (4 per thread;
    // indexes clamped so the loads are unconditional).
    const int n4 = (int)(k >> 2);    // float4 pieces per token
    const int nt4 = n4 * MT;         // for all tokens
    const f32x4 *x4 = (const f32x4 *)x;
    f32x4 xa[4];
    if (x_in_lds) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int q = tid + s * T;
            xa[s] = x4[q < nt4 ? q : nt4 - 1];
        }
    }

    // 2. weight loads of the first batch (every workgroup has one: the grid
    // never exceeds the batch count). Rows are base + r*P + slot: the r*P
    // part is uniform across the workgroup (scalar address arithmetic), the
    // slot part a per-lane constant. Loads are branch-free: a row past j_end
    // re-reads row j_end-1 and its result is dropped, which lets the compiler
    // count outstanding loads exactly.
    typename F::Raw raw[RB][UPL];
    int64_t base = j_start + (int64_t)blockIdx.x * rows_per_batch;
    const uint8_t *last_row = W + (j_end - 1) * row_bytes;
    auto issue = [&](int64_t b) {
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const int64_t jr = b + (int64_t)r * P;
            const uint8_t *row = jr + slot < j_end ? Wslot + jr * row_bytes : last_row;
#pragma unroll
            for (int i = 0; i < UPL; i++) F::load(raw[r][i], row, ulod[i], U);
        }
    };
    issue(base);

    // 3. x into LDS, transposed so that piece i of unit u sits at [i*U + u]:
    // the per-lane reads below are then consecutive across lanes (no bank
    // conflicts). The first 4T pieces come from registers, the rest (long
    // rows only) are copied here.
    typename F::X xu[MT][UPL];
    f32x4 *xl = (f32x4 *)smem;
    if (x_in_lds) {
        auto put = [&](int q, f32x4 v) {
            const int t = q / n4, r = q - t * n4;
            int u, i;
            F::x4_slot(r, U, u, i);
            xl[t * n4 + i * U + u] = v;
        };
#pragma unroll
        for (int s = 0; s < 4; s++)
            if (tid + s * T < nt4) put(tid + s * T, xa[s]);
        for (int q = tid + 4 * T; q < nt4; q += T) put(q, x4[q]);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < UPL; i++)
#pragma unroll
            for (int t = 0; t < MT; t++) {
#pragma unroll
                for (int p = 0; p < 16; p++)
                    F::put_x(xu[t][i], p, xl[t * n4 + p * U + ulod[i]]);
                F::finish_x(xu[t][i]);
            }
    } else {
        // x straight from global memory, one float at a time (any 4-byte alignment)
#pragma unroll
        for (int i = 0; i < UPL; i++)
#pragma unroll
            for (int t = 0; t < MT; t++) {
#pragma unroll
                for (int p = 0; p < 16; p++) {
                    const float *src = x + t * k + 4 * F::x4_index(ulod[i], p, U);
                    F::put_x(xu[t][i], p, f32x4{src[0], src[1], src[2], src[3]});
                }
                F::finish_x(xu[t][i]);
            }
    }
    float *red = smem + (x_in_lds ? k * MT : 0);
    const int red_half = P * RB * MT * NG;
    int buf = 0;

    // 4. stream: decode batch i, issue the loads of batch i+1, then reduce
    // and store batch i while those loads are in flight.
    for (; base < j_end; base += stride) {
        float part[RB][MT];
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const bool live = base + (int64_t)r * P + slot < j_end;
#pragma unroll
            for (int t = 0; t < MT; t++) {
                float v = 0.f;
                if (live) {
#pragma unroll
                    for (int i = 0; i < UPL; i++)
                        if (uvalid[i]) v += F::dot(raw[r][i], xu[t][i], uid[i]);
                }
                part[r][t] = v;
            }
        }
        if (base + stride < j_end) issue(base + stride);
#pragma unroll
        for (int r = 0; r < RB; r++)
#pragma unroll
            for (int t = 0; t < MT; t++) part[r][t] = group_sum(part[r][t], G);
        if (NG == 1) {
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < RB; r++) {
                    const int64_t j = base + (int64_t)r * P + slot;
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
            lds_barrier();
            for (int q = tid; q < P * RB * MT; q += blockDim.x) {
                const int t = q % MT;
                const int rr = q / MT; // slot * RB + r
                const int s = rr / RB, r = rr % RB;
                const int64_t j = base + (int64_t)r * P + s;
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
    // Upper bound here; the launch clamps it to what stays resident
    // (compute units x workgroups per compute unit).
    g.grid = (int)(batches < (int64_t)1 << 30 ? batches : (int64_t)1 << 30);
    if (g.grid < 1) g.grid = 1;
    g.num_cu = num_cu;
    // LDS: the reduction buffers, plus x when everything fits in 64 KB
    // (otherwise each lane loads its x units straight from global memory).
    const size_t red = g.NG > 1 ? (size_t)2 * g.P * g.RB * g.MT * g.NG * sizeof(float) : 0;
    const size_t xb = (size_t)k * g.MT * sizeof(float);
    g.x_in_lds = (xb + red <= 64 * 1024) ? 1 : 0;
    g.lds_bytes = (g.x_in_lds ? xb : 0) + red;
    *p = g;
    return true;
}

// Resident workgroups per compute unit for one kernel instance at a given
// block size and LDS size (cached: the query only reads kernel metadata).
template <class F, int MT, int UPL, int RB>
static int resident_per_cu(int T, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<int, size_t>, int> cache;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find({T, lds});
    if (it != cache.end()) return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, qmv_gemv<F, MT, UPL, RB>, T, lds) !=
            hipSuccess ||
        nb < 1) {
        (void)hipGetLastError();
        nb = 1;
    }
    cache[{T, lds}] = nb;
    return nb;
}

template <class F, int MT, int UPL, int RB>
static hipError_t launch_t(const GemvPlan &p0, const uint8_t *W, const float *x, float *y,
                           int64_t k, int64_t n, int64_t row_bytes, int64_t j0, int64_t j1,
                           int acc, hipStream_t s) {
    GemvPlan p = p0;
    if (p.x_in_lds && ((uintptr_t)x & 15) != 0) { // the LDS copy moves 16-byte pieces
        p.x_in_lds = 0;
        p.lds_bytes -= (size_t)k * p.MT * sizeof(float);
    }
    const int64_t cap = (int64_t)p.num_cu * resident_per_cu<F, MT, UPL, RB>(p.T, p.lds_bytes);
    const int grid = (int)(p.grid < cap ? p.grid : cap);
    hipLaunchKernelGGL((qmv_gemv<F, MT, UPL, RB>), dim3(grid), dim3(p.T), p.lds_bytes, s, W, x,
                       y, k, n, row_bytes, j0, j1, acc, p.U, p.L, p.P, p.G, p.x_in_lds);
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
