// Weight units shared by the streaming kernels (forward and transposed
// products): per format, the registers that hold one 64-weight unit of a row,
// how to read them from a row staged in LDS (or from global memory), where
// the unit's weights sit along k, and the unit's contribution to
//   dot    the forward product: sum_e w_e * x_e over the unit
//   axpy   the transposed product: acc_e += dy * w_e for the unit's 64 e
// Layouts of the blocks: rullama 0.5.0, src/backend/matmul.rs (block sizes of
// Q4_0, Q4_K, Q6_K, F16, BF16) and src/backend/dispatch/mod.rs (the fields of
// Q8_0 and Q5_0 blocks in the expert-matmul tests); the order inside the
// blocks is ggml's.
#pragma once

#include "qmv_internal.h"

#include <map>
#include <mutex>
#include <utility>

namespace qmv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// LDS reads of 16-byte fields (Q4_K super-blocks and 16-bit rows, which sit
// on 16-byte boundaries of the staged rows): a single ds_read_b128.
typedef uint32_t u32x4h __attribute__((ext_vector_type(4), aligned(2)));

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ u32x4 lds16(const uint8_t *p) {
    const u32x4h v = *(const u32x4h *)p;
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint32_t lds2(const uint8_t *p) { return *(const uint16_t *)p; }
// Keeps the compiler from folding a byte mask into per-element bit-field
// extracts, so that the byte conversions select v_cvt_f32_{ubyte,i32 sdwa}.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}
// (m & a) | (~m & b) as one v_bfi_b32. Written out, the compiler uses the
// known-zero bits of b to re-mask it in separate instructions; the asm
// (a plain VALU operation, no memory access) keeps it to one.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xffu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }
__device__ __forceinline__ float sb0(uint32_t v) { return (float)(int)(int8_t)(v & 0xffu); }
__device__ __forceinline__ float sb1(uint32_t v) { return (float)(int)(int8_t)((v >> 8) & 0xffu); }
__device__ __forceinline__ float sb2(uint32_t v) { return (float)(int)(int8_t)((v >> 16) & 0xffu); }
__device__ __forceinline__ float sb3(uint32_t v) { return (float)((int)v >> 24); }
__device__ __forceinline__ float f16lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
// a[b] += s * byte_b(q), unsigned / signed bytes
__device__ __forceinline__ void uaxpy4(uint32_t q, float s, float *a) {
    a[0] = fmaf(ub0(q), s, a[0]);
    a[1] = fmaf(ub1(q), s, a[1]);
    a[2] = fmaf(ub2(q), s, a[2]);
    a[3] = fmaf(ub3(q), s, a[3]);
}
__device__ __forceinline__ void saxpy4(uint32_t q, float s, float *a) {
    a[0] = fmaf(sb0(q), s, a[0]);
    a[1] = fmaf(sb1(q), s, a[1]);
    a[2] = fmaf(sb2(q), s, a[2]);
    a[3] = fmaf(sb3(q), s, a[3]);
}
__device__ __forceinline__ f32x4 get4(const float *d) { return f32x4{d[0], d[1], d[2], d[3]}; }
__device__ __forceinline__ void put4(float *d, f32x4 v) {
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
}

// ------------------------------------- forward products on integer dots
// The forward product of the block formats multiplies integer codes by x.
// Instead of converting every code to f32 and issuing one FMA per weight,
// x of a unit (64 values, fixed for the whole launch) is written once as
// 24-bit integers with a power-of-two scale,
//     x_e ~= s * X_e,   X_e = x2_e * 65536 + x1_e * 256 + x0_e,
// each digit a signed byte, and the codes (signed bytes) meet the three
// digit planes in v_dot4_i32_i8: four exact multiply-adds per instruction.
// Integer partial sums of a scale group are exact; the group scale is
// applied with a 24-bit integer multiply, and the three plane sums are
// combined in f32 once per unit, then scaled by 2^E with one ldexp (so the
// scale itself never needs to be a normal f32). E is chosen per unit so
// that max|x| / 2^E lies in [2^21, 2^22): every x_e is represented with an
// absolute error of at most 2^(E-1) <= 2^-22 max|x| over its unit (values
// far below the unit's largest carry correspondingly fewer bits). A unit with
// a non-finite x gets a NaN multiplier, so its rows come out NaN.
struct XI {
    float f[64];       // the unit's x while loading: piece i is f[4i..4i+3]
    uint32_t p[3][16]; // digit planes: byte b of p[d][i] is digit d of x_{4i+b}
    float c;           // the unit's format constant (NaN for a non-finite x)
    int e;             // E
    int ofs[2][3];     // per block (or half) and plane: a format-specific integer offset
    float sum[2];      // Q4_K: f32 sums of pieces 0..7 and 8..15
};

// Digits of four values at exponent E: X = rint(v * 2^-E) (|X| <= 2^22) as
// balanced base-256 digits X = x2*65536 + x1*256 + x0, byte b of d[j] being
// digit j of value b.
__device__ __forceinline__ void x_digits4(f32x4 v, int E, uint32_t (&d)[3]) {
    const float f[4] = {v.x, v.y, v.z, v.w};
    d[0] = d[1] = d[2] = 0u;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const int X = (int)rintf(ldexpf(f[b], -E));
        const int x0 = (int)((uint32_t)X << 24) >> 24;
        const int r = (X - x0) >> 8;
        const int x1 = (int)((uint32_t)r << 24) >> 24;
        const int x2 = (r - x1) >> 8; // |x2| <= 65
        d[0] |= ((uint32_t)x0 & 0xffu) << (8 * b);
        d[1] |= ((uint32_t)x1 & 0xffu) << (8 * b);
        d[2] |= ((uint32_t)x2 & 0xffu) << (8 * b);
    }
}

// The unit's exponent E = e2 - 22 for max|x| in [2^(e2-1), 2^e2) (0 when all
// are zero) and format constant 1 (NaN when any value is not finite).
__device__ __forceinline__ void x_scale(float mx, bool finite, int &E, float &c) {
    int e2 = 0;
    if (mx > 0.f) (void)frexpf(mx, &e2);
    E = e2 - 22;
    c = finite ? 1.f : __builtin_nanf("");
}

// The unit's planes, exponent, constant and the f32 sums of values 0..31 and
// 32..63 (in order), from its 64 values in x.f.
__device__ __forceinline__ void x_planes(XI &x) {
    float mx = 0.f;
    bool finite = true;
#pragma unroll
    for (int e = 0; e < 64; e++) {
        const float a = fabsf(x.f[e]);
        finite = finite && (a <= 3.4028235e38f); // false for NaN and infinities
        mx = fmaxf(mx, a);
    }
    x_scale(mx, finite, x.e, x.c);
    // sums of values 0..31 and 32..63: each piece's four in order, then the
    // eight piece sums pairwise (the order of the shared pass below)
    float ps[16];
#pragma unroll
    for (int i = 0; i < 16; i++) ps[i] = ((x.f[4 * i] + x.f[4 * i + 1]) + x.f[4 * i + 2]) + x.f[4 * i + 3];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const float *q = ps + 8 * h;
        x.sum[h] = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
    }
#pragma unroll
    for (int i = 0; i < 16; i++) {
        uint32_t d[3];
        x_digits4(f32x4{x.f[4 * i], x.f[4 * i + 1], x.f[4 * i + 2], x.f[4 * i + 3]}, x.e, d);
        x.p[0][i] = d[0];
        x.p[1][i] = d[1];
        x.p[2][i] = d[2];
    }
}

// The same, computed once per workgroup and shared through LDS: each aligned
// group of 16 threads (the complete ones; the plans give at least 33 threads)
// takes one unit at a time, one 4-value piece per lane, exchanging maxima and
// sums by shuffles within the group; its first lane writes the unit's record.
struct XRec {
    int e;
    float c, sum0, sum1;
};
// plane dword i of digit d of unit u, token t: pl[(((t*3 + d)*4 + i/4)*U + u)*4 + i%4]
// (a lane's four consecutive dwords are one 16-byte read; lanes of
// consecutive units read consecutive 16 bytes)
// Lane exchange inside rows of 16 lanes (DPP; CTRL: quad_perm, row_ror, row_mirror...).
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, dpp_mov<CTRL>(__builtin_bit_cast(int, v)));
}
// Unit q = t*U + u from its piece i (= this lane's index in the group) v. The
// group is one 16-lane row of the wave; maxima, flags and sums move by DPP
// (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror, row_ror 8).
__device__ __forceinline__ void x_unit_planes(f32x4 v, int q, int i, int U, XRec *rec,
                                              uint32_t *pl) {
    float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    int bad = !(fabsf(v.x) <= 3.4028235e38f && fabsf(v.y) <= 3.4028235e38f &&
                fabsf(v.z) <= 3.4028235e38f && fabsf(v.w) <= 3.4028235e38f);
    float ps = ((v.x + v.y) + v.z) + v.w;
    // pairs, then quads, then halves (lanes 0-7: pieces 0..7, 8-15: 8..15),
    // then (maximum and flag only) the whole row
    mx = fmaxf(mx, dpp_mov<0xb1>(mx));
    bad |= dpp_mov<0xb1>(bad);
    ps += dpp_mov<0xb1>(ps);
    mx = fmaxf(mx, dpp_mov<0x4e>(mx));
    bad |= dpp_mov<0x4e>(bad);
    ps += dpp_mov<0x4e>(ps);
    mx = fmaxf(mx, dpp_mov<0x141>(mx));
    bad |= dpp_mov<0x141>(bad);
    ps += dpp_mov<0x141>(ps);
    mx = fmaxf(mx, dpp_mov<0x140>(mx));
    bad |= dpp_mov<0x140>(bad);
    const float s1 = dpp_mov<0x128>(ps); // lane 0: the sum of pieces 8..15
    XRec r;
    x_scale(mx, !bad, r.e, r.c);
    uint32_t d[3];
    x_digits4(v, r.e, d);
    const int t = q / U, u = q - t * U;
#pragma unroll
    for (int j = 0; j < 3; j++) pl[(((t * 3 + j) * 4 + (i >> 2)) * U + u) * 4 + (i & 3)] = d[j];
    if (i == 0) {
        r.sum0 = ps;
        r.sum1 = s1;
        rec[q] = r;
    }
}
// Bytes of a workgroup's records and planes (a multiple of 16).
__host__ __device__ constexpr long long xplanes_bytes(int MT, int U) {
    return (long long)MT * U * (sizeof(XRec) + 192);
}
__device__ __forceinline__ void x_from_planes(XI &x, const XRec *rec, const uint32_t *pl, int t,
                                              int u, int U) {
    const XRec r = rec[t * U + u];
    x.e = r.e;
    x.c = r.c;
    x.sum[0] = r.sum0;
    x.sum[1] = r.sum1;
#pragma unroll
    for (int j = 0; j < 3; j++)
#pragma unroll
        for (int i4 = 0; i4 < 4; i4++) {
            const u32x4 w = *(const u32x4 *)(pl + (((t * 3 + j) * 4 + i4) * U + u) * 4);
            x.p[j][4 * i4] = w.x;
            x.p[j][4 * i4 + 1] = w.y;
            x.p[j][4 * i4 + 2] = w.z;
            x.p[j][4 * i4 + 3] = w.w;
        }
}

// Sum of the signed digit bytes of plane dwords [i0, i1).
__device__ __forceinline__ int plane_sum(const XI &x, int d, int i0, int i1) {
    int s = 0;
    for (int i = i0; i < i1; i++) s = __builtin_amdgcn_sdot4((int)x.p[d][i], 0x01010101, s, false);
    return s;
}

__device__ __forceinline__ int sdot4i(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}
// The first dot of a chain: v_dot4_i32_i8 with a zero addend (written out,
// the compiler zeroes a register and uses the accumulating form, one more
// instruction). Plain VALU operations, no memory access.
__device__ __forceinline__ int sdot4z(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// a * b + c with a, b within 24 bits (a 24-bit multiply and an add)
__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }
// s * (A2 * 65536 + A1 * 256 + A0) for the three plane sums
__device__ __forceinline__ float planes_f32(int a0, int a1, int a2) {
    return fmaf((float)a2, 65536.f, fmaf((float)a1, 256.f, (float)a0));
}

// Each unit type below provides
//   Raw                 registers holding one unit of one row
//   load_lds / load     read them from the staged row in LDS / from global memory
//   X, x4_index, x4_slot, put_x, finish_x
//                       the unit's 64 x values as 16 float4 pieces: piece i of
//                       unit u is float4 number x4_index(u, i) of x; x4_slot
//                       is the inverse
//   dot                 the unit's contribution to the row's dot product
//   get_x               piece i back out of an X (X doubles as the
//                       accumulator of the transposed product)
//   axpy, finish_t      acc += dy * (the unit's weights), in X layout; then
//                       whatever was kept factored (the Q4_K min term) applied

// ------------------------------------------------------------ Q4_0 units
// A unit is two consecutive 18-byte blocks. Block layout: f16 d, 16 code
// bytes; element e < 16 is the low nibble of byte e, e >= 16 the high nibble
// of byte e-16; value d*(q-8). The signed code q-8 is the 4-bit two's
// complement reading of q^8: each nibble is XORed with 8 and moved to the top
// of its byte, where a sign-extending byte conversion yields 16*(q-8)
// exactly. Summing signed codes keeps the rounding error proportional to
// sum|w*x| (an all-8 block gives exactly 0).
// x of a unit of two 32-weight blocks whose element e < 16 sits in the low
// nibble of code byte e and e >= 16 in the high nibble of byte e-16 (Q4_0,
// Q5_0): piece i = 8b + j of block b is lo[b][4j..] (j < 4) or hi[b][4(j-4)..].
struct NibbleBlocksX {
    struct X { float lo[2][16], hi[2][16]; };
    static __device__ __forceinline__ int x4_index(int u, int i, int) { return 16 * u + i; }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = q >> 4;
        i = q & 15;
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        const int b = i >> 3, j = i & 7;
        put4(j < 4 ? &x.lo[b][4 * j] : &x.hi[b][4 * (j - 4)], v);
    }
    static __device__ __forceinline__ f32x4 get_x(const X &x, int i) {
        const int b = i >> 3, j = i & 7;
        return get4(j < 4 ? &x.lo[b][4 * j] : &x.hi[b][4 * (j - 4)]);
    }
    static __device__ __forceinline__ void finish_x(X &) {}
    static __device__ __forceinline__ void finish_t(X &) {}
};

struct UQ4_0 : NibbleBlocksX {
    struct Raw { u32x4 q0, q1; uint32_t d0, d1; };
    // The unit starts dword aligned (rows are 36*U bytes and every batch
    // starts at a dword multiple in LDS): nine aligned dwords hold both blocks.
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int) {
        const uint32_t *w = (const uint32_t *)(row + 36 * u);
        uint32_t e[9];
#pragma unroll
        for (int i = 0; i < 9; i++) e[i] = w[i];
        r.d0 = e[0] & 0xffffu;
        r.q0 = u32x4{__builtin_amdgcn_alignbyte(e[1], e[0], 2),
                     __builtin_amdgcn_alignbyte(e[2], e[1], 2),
                     __builtin_amdgcn_alignbyte(e[3], e[2], 2),
                     __builtin_amdgcn_alignbyte(e[4], e[3], 2)};
        r.d1 = e[4] >> 16;
        r.q1 = u32x4{e[5], e[6], e[7], e[8]};
    }
    // Forward product on integer planes (pieces 8b..8b+3 are the low nibbles
    // of block b, 8b+4..8b+7 the high nibbles). Low nibbles enter as q (0..15)
    // with -8 * sum(x) of the low half as the chain's start, high nibbles as
    // the signed byte 16*(q-8); 16 * low + high is then 16 * sum (q-8) x.
    static __device__ __forceinline__ void finish_xi(XI &x) {
        x.c *= 0.0625f;
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int d = 0; d < 3; d++) x.ofs[b][d] = -8 * plane_sum(x, d, 8 * b, 8 * b + 4);
    }
    static __device__ __forceinline__ float block_i(u32x4 qv, uint32_t dbits, const XI &x,
                                                    int b) {
        const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
        int t[3];
#pragma unroll
        for (int d = 0; d < 3; d++) {
            int lo = x.ofs[b][d];
            int hi = sdot4z((q[0] & 0xf0f0f0f0u) ^ 0x80808080u, x.p[d][8 * b + 4]);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                lo = sdot4i(q[j] & 0x0f0f0f0fu, x.p[d][8 * b + j], lo);
                if (j > 0)
                    hi = sdot4i((q[j] & 0xf0f0f0f0u) ^ 0x80808080u, x.p[d][8 * b + 4 + j], hi);
            }
            t[d] = (lo << 4) + hi;
        }
        return f16lo(dbits) * planes_f32(t[0], t[1], t[2]);
    }
    static __device__ __forceinline__ float dot_i(const Raw &r, const XI &x, int) {
        return ldexpf(x.c * (block_i(r.q0, r.d0, x, 0) + block_i(r.q1, r.d1, x, 1)), x.e);
    }
    static __device__ __forceinline__ void axpy_block(u32x4 qv, uint32_t dbits, float dy, X &a,
                                                      int b) {
        const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
        const float s = (f16lo(dbits) * 0.0625f) * dy;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            saxpy4(opaque(((q[j] << 4) ^ 0x80808080u) & 0xf0f0f0f0u), s, &a.lo[b][4 * j]);
            saxpy4(opaque((q[j] ^ 0x80808080u) & 0xf0f0f0f0u), s, &a.hi[b][4 * j]);
        }
    }
    static __device__ __forceinline__ void axpy(const Raw &r, float dy, X &a, int) {
        axpy_block(r.q0, r.d0, dy, a, 0);
        axpy_block(r.q1, r.d1, dy, a, 1);
    }
};

// ------------------------------------------------------------ Q8_0 units
// A unit is two consecutive 34-byte blocks: f16 d, then 32 signed code bytes
// in element order; value d*q. Rows are 68*U bytes, so the unit starts dword
// aligned and 17 aligned dwords hold both blocks (the first block's codes sit
// 2 bytes off a dword boundary, the second block's on one). The code bytes
// convert directly with the sign-extending byte conversion.
struct UQ8_0 {
    struct Raw { uint32_t q0[8], q1[8]; uint32_t d0, d1; };
    struct X { float v[2][32]; };
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int) {
        const uint32_t *w = (const uint32_t *)(row + 68 * u);
        uint32_t e[17];
#pragma unroll
        for (int i = 0; i < 17; i++) e[i] = w[i];
        r.d0 = e[0] & 0xffffu;
#pragma unroll
        for (int j = 0; j < 8; j++) r.q0[j] = __builtin_amdgcn_alignbyte(e[j + 1], e[j], 2);
        r.d1 = e[8] >> 16;
#pragma unroll
        for (int j = 0; j < 8; j++) r.q1[j] = e[9 + j];
    }
    static __device__ __forceinline__ int x4_index(int u, int i, int) { return 16 * u + i; }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = q >> 4;
        i = q & 15;
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        put4(&x.v[i >> 3][4 * (i & 7)], v);
    }
    static __device__ __forceinline__ f32x4 get_x(const X &x, int i) {
        return get4(&x.v[i >> 3][4 * (i & 7)]);
    }
    static __device__ __forceinline__ void finish_x(X &) {}
    static __device__ __forceinline__ void finish_t(X &) {}
    static __device__ __forceinline__ void axpy(const Raw &r, float dy, X &a, int) {
        const float s0 = f16lo(r.d0) * dy, s1 = f16lo(r.d1) * dy;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            saxpy4(r.q0[j], s0, &a.v[0][4 * j]);
            saxpy4(r.q1[j], s1, &a.v[1][4 * j]);
        }
    }
    // Forward product on integer planes: the code bytes are the signed
    // multipliers as they are (pieces 8b..8b+7 = block b).
    static __device__ __forceinline__ void finish_xi(XI &) {}
    static __device__ __forceinline__ float block_i(const uint32_t (&q)[8], uint32_t dbits,
                                                    const XI &x, int b) {
        int t[3];
#pragma unroll
        for (int d = 0; d < 3; d++) {
            int a = sdot4z(q[0], x.p[d][8 * b]);
#pragma unroll
            for (int j = 1; j < 8; j++) a = sdot4i(q[j], x.p[d][8 * b + j], a);
            t[d] = a;
        }
        return f16lo(dbits) * planes_f32(t[0], t[1], t[2]);
    }
    static __device__ __forceinline__ float dot_i(const Raw &r, const XI &x, int) {
        return ldexpf(x.c * (block_i(r.q0, r.d0, x, 0) + block_i(r.q1, r.d1, x, 1)), x.e);
    }
};

// ------------------------------------------------------------ Q5_0 units
// A unit is two consecutive 22-byte blocks: f16 d, a little-endian 32-bit
// word qh, 16 code bytes. Element e takes its low 4 bits from the low nibble
// of code byte e (e < 16) or the high nibble of byte e-16, and bit e of qh as
// its fifth bit; value d*(q-16). Rows are 44*U bytes: the unit starts dword
// aligned and 11 dwords hold both blocks. The signed code q-16 is the 5-bit
// two's-complement reading of q^16: each nibble goes to bits 3..6 of its byte
// and the inverted fifth bit to bit 7 (four bits of ~qh are spread to the top
// of four bytes by one 24-bit multiply: bit i of a 4-bit field times 0x204081
// lands on bit 8i), so a sign-extending byte conversion yields 8*(q-16).
struct UQ5_0 : NibbleBlocksX {
    struct Raw { u32x4 q0, q1; uint32_t h0, h1, d0, d1; };
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int) {
        const uint32_t *w = (const uint32_t *)(row + 44 * u);
        uint32_t e[11];
#pragma unroll
        for (int i = 0; i < 11; i++) e[i] = w[i];
        r.d0 = e[0] & 0xffffu;
        r.h0 = __builtin_amdgcn_alignbyte(e[1], e[0], 2);
        r.q0 = u32x4{__builtin_amdgcn_alignbyte(e[2], e[1], 2),
                     __builtin_amdgcn_alignbyte(e[3], e[2], 2),
                     __builtin_amdgcn_alignbyte(e[4], e[3], 2),
                     __builtin_amdgcn_alignbyte(e[5], e[4], 2)};
        r.d1 = e[5] >> 16;
        r.h1 = e[6];
        r.q1 = u32x4{e[7], e[8], e[9], e[10]};
    }
    // bits at..at+3 of nh moved to bits 7, 15, 23, 31 (the multiply is kept
    // apart from the shift, else the two fold into a quarter-rate 32-bit one)
    static __device__ __forceinline__ uint32_t spread4(uint32_t nh, int at) {
        const uint32_t m = opaque(__umul24(__builtin_amdgcn_ubfe(nh, at, 4), 0x204081u));
        return (m & 0x01010101u) << 7;
    }
    // Forward product on integer planes: the signed bytes 8*(q-16) of both
    // halves of block b meet pieces 8b..8b+7.
    static __device__ __forceinline__ void finish_xi(XI &x) { x.c *= 0.125f; }
    static __device__ __forceinline__ float block_i(u32x4 qv, uint32_t qh, uint32_t dbits,
                                                    const XI &x, int b) {
        const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
        const uint32_t nh = ~qh;
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            c[j] = ((q[j] << 3) & 0x78787878u) | spread4(nh, 4 * j);
            c[4 + j] = ((q[j] >> 1) & 0x78787878u) | spread4(nh, 16 + 4 * j);
        }
        int t[3];
#pragma unroll
        for (int d = 0; d < 3; d++) {
            int a = sdot4z(c[0], x.p[d][8 * b]);
#pragma unroll
            for (int j = 1; j < 8; j++) a = sdot4i(c[j], x.p[d][8 * b + j], a);
            t[d] = a;
        }
        return f16lo(dbits) * planes_f32(t[0], t[1], t[2]);
    }
    static __device__ __forceinline__ float dot_i(const Raw &r, const XI &x, int) {
        return ldexpf(x.c * (block_i(r.q0, r.h0, r.d0, x, 0) + block_i(r.q1, r.h1, r.d1, x, 1)),
                      x.e);
    }
    static __device__ __forceinline__ void axpy_block(u32x4 qv, uint32_t qh, uint32_t dbits,
                                                      float dy, X &a, int b) {
        const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
        const uint32_t nh = ~qh;
        const float s = (f16lo(dbits) * 0.125f) * dy;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            saxpy4(opaque(((q[j] << 3) & 0x78787878u) | spread4(nh, 4 * j)), s, &a.lo[b][4 * j]);
            saxpy4(opaque(((q[j] >> 1) & 0x78787878u) | spread4(nh, 16 + 4 * j)), s,
                   &a.hi[b][4 * j]);
        }
    }
    static __device__ __forceinline__ void axpy(const Raw &r, float dy, X &a, int) {
        axpy_block(r.q0, r.h0, r.d0, dy, a, 0);
        axpy_block(r.q1, r.h1, r.d1, dy, a, 1);
    }
};

// ------------------------------------------------------------ Q4_K units
// A unit is one 64-weight chunk c of a 144-byte super-block: its 32 code
// bytes (low nibbles = sub-block 2c, high nibbles = sub-block 2c+1) plus the
// 16-byte head (f16 d, f16 dmin, 12 bytes of packed 6-bit scales/mins).
struct UQ4_K {
    struct Raw { u32x4 hd, q0, q1; };
    struct X { float lo[32], hi[32]; float slo, shi; };
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *sb = row + 144 * (u >> 2);
        const int c = u & 3;
        r.hd = lds16(sb);
        r.q0 = lds16(sb + 16 + 32 * c);
        r.q1 = lds16(sb + 32 + 32 * c);
    }
    static __device__ __forceinline__ int x4_index(int u, int i, int) { return 16 * u + i; }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = q >> 4;
        i = q & 15;
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        put4(i < 8 ? &x.lo[4 * i] : &x.hi[4 * (i - 8)], v);
    }
    static __device__ __forceinline__ f32x4 get_x(const X &x, int i) {
        return get4(i < 8 ? &x.lo[4 * i] : &x.hi[4 * (i - 8)]);
    }
    // transposed product: slo/shi hold sum_rows dy * dmin * m of the two
    // sub-blocks, subtracted from every element at the end
    static __device__ __forceinline__ void finish_t(X &a) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
            a.lo[i] -= a.slo;
            a.hi[i] -= a.shi;
        }
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
        const uint32_t a = low ? d1 : d3, b = low ? d2 : d3;
        const int sa = t, sb = low ? t : t + 4, hs = low ? t + 4 : t + 6;
        sc = ((a >> sa) & 15u) | (((d1 >> hs) & 3u) << 4);
        mn = ((b >> sb) & 15u) | (((d2 >> hs) & 3u) << 4);
    }
    // Forward product on integer planes. Pieces 0..7 are the low nibbles
    // (sub-block 2c), 8..15 the high nibbles (2c+1). Low nibbles enter as q
    // (0..15); high nibbles as the signed byte 16*(q-8), the chain starting at
    // 128 * sum(x) over the high pieces, which gives 16 * sum q x. The min
    // term dmin * m * sum(x) uses the f32 sums of the two halves.
    static __device__ __forceinline__ void finish_xi(XI &x) {
        x.c *= 0.0625f;
#pragma unroll
        for (int d = 0; d < 3; d++) x.ofs[0][d] = 128 * plane_sum(x, d, 8, 16);
    }
    static __device__ __forceinline__ float dot_i(const Raw &r, const XI &x, int u) {
        const uint32_t q[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        const int s0 = 2 * (u & 3);
        uint32_t sc0, mn0, sc1, mn1;
        scale_min(r.hd.y, r.hd.z, r.hd.w, s0, sc0, mn0);
        scale_min(r.hd.y, r.hd.z, r.hd.w, s0 + 1, sc1, mn1);
        int t[3];
#pragma unroll
        for (int d = 0; d < 3; d++) {
            int lo = sdot4z(q[0] & 0x0f0f0f0fu, x.p[d][0]), hi = x.ofs[0][d];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if (i > 0) lo = sdot4i(q[i] & 0x0f0f0f0fu, x.p[d][i], lo);
                hi = sdot4i((q[i] & 0xf0f0f0f0u) ^ 0x80808080u, x.p[d][8 + i], hi);
            }
            t[d] = mad24((int)sc0 << 4, lo, __mul24((int)sc1, hi)); // 16 * sum sc q x
        }
        const float d = f16lo(r.hd.x), dmin = f16hi(r.hd.x);
        const float mt = dmin * fmaf((float)mn1, x.sum[1], (float)mn0 * x.sum[0]);
        return ldexpf((d * x.c) * planes_f32(t[0], t[1], t[2]), x.e) - mt;
    }
    static __device__ __forceinline__ void axpy(const Raw &r, float dy, X &a, int u) {
        const int s0 = 2 * (u & 3);
        uint32_t sc0, mn0, sc1, mn1;
        scale_min(r.hd.y, r.hd.z, r.hd.w, s0, sc0, mn0);
        scale_min(r.hd.y, r.hd.z, r.hd.w, s0 + 1, sc1, mn1);
        const float d = f16lo(r.hd.x) * dy, dmin = f16hi(r.hd.x) * dy;
        const float f0 = d * (float)sc0;
        const float f1 = (d * 0.0625f) * (float)sc1;
        const uint32_t q[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uaxpy4(opaque(q[i] & 0x0f0f0f0fu), f0, &a.lo[4 * i]);
            uaxpy4(opaque(q[i] & 0xf0f0f0f0u), f1, &a.hi[4 * i]); // 16x the high nibble
        }
        a.slo = fmaf(dmin, (float)mn0, a.slo);
        a.shi = fmaf(dmin, (float)mn1, a.shi);
    }
};

// ------------------------------------------------------------ Q6_K units
// A unit is (super-block, half h, lane block lq): the 64 weights
// 128h + 32g + 16lq + i (g < 4, i < 16). Their low 4 bits are bytes
// ql[64h + 16lq + i] (g = 0 low nibble, g = 2 high nibble) and
// ql[64h + 32 + 16lq + i] (g = 1, 3), their top 2 bits are bits 2g..2g+1 of
// qh[32h + 16lq + i], and their scales are the int8 scales[8h + 2g + lq].
// The signed code q-32 is the 6-bit two's-complement reading of q^32: the
// high 2-bit fields are XORed with 0b10, the 6-bit code is assembled in the
// top of its byte, and a sign-extending byte conversion yields 4*(q-32).
//
// Super-blocks are 210 bytes, so a unit's fields sit either on a dword
// boundary (sh = 0) or 2 bytes past one (sh = 2), the same for all of its
// fields. They are read as dwords at aligned LDS addresses and realigned by
// funnel shifts that also place the nibbles: with the ql dwords read from
// 4 - sh bytes before the field, alignbit(a[j+1], a[j], 30 - 8 sh) is the
// field's dword j shifted left by 2 (low nibbles in bits 2..5 of each byte)
// and alignbit of two such neighbours by 4 is dword j shifted right by 2
// (high nibbles in bits 2..5). The dword before a field lies in LDS (the
// previous block, or padding in front of the weight buffers); its bits only
// reach masked-off positions.
struct UQ6_K {
    struct Raw {
        uint32_t a[6], b[6]; // ql dwords from 4 - sh bytes before the field
        uint32_t h[5];       // qh dwords from sh bytes before the field
        int s[4];            // the unit's four scales
        uint32_t d, sh;
    };
    struct X { float v[4][16]; };
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int) {
        const uint8_t *o = row + 210 * (u >> 2);
        const int h = (u >> 1) & 1, lq = u & 1;
        const uint32_t sh = (uint32_t)(uintptr_t)o & 2u;
        r.sh = sh;
        const uint32_t *dl = (const uint32_t *)(o + sh - 4);
        const uint32_t *dh = (const uint32_t *)(o - sh);
        const int fa = 16 * h + 4 * lq, fh = 32 + 8 * h + 4 * lq;
#pragma unroll
        for (int i = 0; i < 6; i++) {
            r.a[i] = dl[fa + i];
            r.b[i] = dl[fa + 8 + i];
        }
#pragma unroll
        for (int i = 0; i < 5; i++) r.h[i] = dh[fh + i];
#pragma unroll
        for (int i = 0; i < 4; i++) r.s[i] = *(const int8_t *)(o + 192 + 8 * h + 2 * i + lq);
        r.d = lds2(o + 208);
    }
    // piece i = 4g + i4 holds weights 128h + 32g + 16lq + 4i4 .. +3
    static __device__ __forceinline__ int x4_index(int u, int i, int) {
        return 64 * (u >> 2) + 32 * ((u >> 1) & 1) + 8 * (i >> 2) + 4 * (u & 1) + (i & 3);
    }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = 4 * (q >> 6) + 2 * ((q >> 5) & 1) + ((q >> 2) & 1);
        i = 4 * ((q >> 3) & 3) + (q & 3);
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) {
        put4(&x.v[i >> 2][4 * (i & 3)], v);
    }
    static __device__ __forceinline__ f32x4 get_x(const X &x, int i) {
        return get4(&x.v[i >> 2][4 * (i & 3)]);
    }
    static __device__ __forceinline__ void finish_x(X &) {}
    static __device__ __forceinline__ void finish_t(X &) {}
    // q[g][j]: bytes of 4*(q-32) for quarter g, weights 16lq + 4j .. +3.
    // Each byte is assembled as (nibble << 2) | ((high 2 bits ^ 2) << 6): the
    // nibble from a funnel-shifted ql dword (bits 2..5 of every byte), the
    // two high bits from the qh dword with the top bit of every 2-bit field
    // flipped, fields 0/2 and 1/3 masked apart so that each of the four
    // shifted copies below has zeros in bits 0..1 of every byte; one bit-field
    // insert (bits 2..5 from the nibble side) then yields the code byte.
    static __device__ __forceinline__ void codes(const Raw &r, uint32_t (&q)[4][4]) {
        const uint32_t fl = 30u - 8u * r.sh;
        constexpr uint32_t NIB = 0x3c3c3c3cu;
        uint32_t a2[5], b2[5]; // ql dword j << 2 (bits 0..1 of each byte: don't care)
#pragma unroll
        for (int j = 0; j < 5; j++) {
            a2[j] = __builtin_amdgcn_alignbit(r.a[j + 1], r.a[j], fl);
            b2[j] = __builtin_amdgcn_alignbit(r.b[j + 1], r.b[j], fl);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t h = __builtin_amdgcn_alignbyte(r.h[j + 1], r.h[j], r.sh);
            const uint32_t hA = (h ^ 0xaaaaaaaau) & 0x33333333u; // fields 0 and 2
            const uint32_t hB = (h ^ 0xaaaaaaaau) & 0xccccccccu; // fields 1 and 3
            const uint32_t ar = __builtin_amdgcn_alignbit(a2[j + 1], a2[j], 4); // dword j >> 2
            const uint32_t br = __builtin_amdgcn_alignbit(b2[j + 1], b2[j], 4);
            q[0][j] = bfi(NIB, a2[j], hA << 6);
            q[1][j] = bfi(NIB, b2[j], hB << 4);
            q[2][j] = bfi(NIB, ar, hA << 2);
            q[3][j] = bfi(NIB, br, hB);
        }
    }
    static __device__ __forceinline__ void axpy(const Raw &r, float dy, X &a, int) {
        uint32_t q[4][4];
        codes(r, q);
        const float d = (f16lo(r.d) * 0.25f) * dy;
        float s[4];
#pragma unroll
        for (int g = 0; g < 4; g++) s[g] = d * (float)r.s[g];
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int g = 0; g < 4; g++) saxpy4(q[g][j], s[g], &a.v[g][4 * j]);
    }
    // Forward product on integer planes: the signed bytes 4*(q-32) of quarter
    // g meet pieces 4g..4g+3; each quarter's three plane sums take its int8
    // scale by a 24-bit multiply-add.
    static __device__ __forceinline__ void finish_xi(XI &x) { x.c *= 0.25f; }
    static __device__ __forceinline__ float dot_i(const Raw &r, const XI &x, int) {
        uint32_t q[4][4];
        codes(r, q);
        int a[3] = {0, 0, 0};
#pragma unroll
        for (int g = 0; g < 4; g++)
#pragma unroll
            for (int d = 0; d < 3; d++) {
                int t = sdot4z(q[g][0], x.p[d][4 * g]);
#pragma unroll
                for (int j = 1; j < 4; j++) t = sdot4i(q[g][j], x.p[d][4 * g + j], t);
                a[d] = g == 0 ? __mul24(r.s[g], t) : mad24(r.s[g], t, a[d]);
            }
        return ldexpf((f16lo(r.d) * x.c) * planes_f32(a[0], a[1], a[2]), x.e);
    }
};

// ------------------------------------------------------- F16 / BF16 units
// A unit is the eight 8-weight chunks u, u+U, ..., u+7U of the row (16 bytes
// each), so that for a fixed chunk index the lanes of a slot read one
// contiguous span straight from global memory.
template <bool BF>
struct UHalf {
    struct Raw { u32x4 c[8]; };
    struct X { float v[8][8]; };
    struct Aux {}; // nothing beyond the row's bytes
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int U,
                                                const Aux &, int64_t) {
#pragma unroll
        for (int c = 0; c < 8; c++) r.c[c] = ld16(row + 16 * (u + U * c));
    }
    // from a row staged in LDS (rows are 128*U bytes, so 16-byte aligned
    // relative to the batch start)
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int U) {
#pragma unroll
        for (int c = 0; c < 8; c++) r.c[c] = lds16(row + 16 * (u + U * c));
    }
    // piece i = 2c + hf holds weights 8(u + cU) + 4hf .. +3
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
        put4(&x.v[i >> 1][4 * (i & 1)], v);
    }
    static __device__ __forceinline__ f32x4 get_x(const X &x, int i) {
        return get4(&x.v[i >> 1][4 * (i & 1)]);
    }
    static __device__ __forceinline__ void finish_x(X &) {}
    static __device__ __forceinline__ void finish_t(X &) {}
    static __device__ __forceinline__ void axpy(const Raw &r, float dy, X &a, int) {
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
                a.v[c][2 * j] = fmaf(lo, dy, a.v[c][2 * j]);
                a.v[c][2 * j + 1] = fmaf(hi, dy, a.v[c][2 * j + 1]);
            }
        }
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

// Forward-product view of a block unit U: its raw registers and LDS reads,
// x as integer planes (XI), and U::dot_i for the unit's contribution.
template <class U>
struct IntX {
    using Raw = typename U::Raw;
    using X = XI;
    static __device__ __forceinline__ void load_lds(Raw &r, const uint8_t *row, int u, int U_) {
        U::load_lds(r, row, u, U_);
    }
    static __device__ __forceinline__ int x4_index(int u, int i, int U_) {
        return U::x4_index(u, i, U_);
    }
    static __device__ __forceinline__ void x4_slot(int q, int U_, int &u, int &i) {
        U::x4_slot(q, U_, u, i);
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) { put4(&x.f[4 * i], v); }
    static __device__ __forceinline__ void finish_x(X &x) {
        x_planes(x);
        U::finish_xi(x);
    }
    // after x_from_planes
    static __device__ __forceinline__ void finish_shared(X &x) { U::finish_xi(x); }
    static __device__ __forceinline__ float dot(const Raw &r, const X &x, int u) {
        return U::dot_i(r, x, u);
    }
};

// ------------------------------------------------------ shared device code
// Workgroup barrier that orders LDS only: global loads in flight (the next
// batch of weights) are not drained, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------- affine group-64 units
// Rows of affine group-quantized weights (moeflux, tests/graph_diff_oracle.rs:
// codes packed into u32 words, one bf16 scale and one bf16 bias per group of
// 64 weights, value code * scale + bias), held in three arrays: the code
// words (k*BITS/8 bytes per row), the scales and the biases (k/64 per row).
// Code i of a word sits at bits BITS*i .. BITS*i+BITS-1. A unit is one group:
// its 32 (4-bit) or 64 (8-bit) code bytes, loaded as 16-byte pieces, and its
// scale and bias. Each weight is decoded exactly as the oracle does (fma of
// the code with the scale and the bias: the product is exact, one rounding),
// then multiplied into the sum.
template <int BITS>
struct UAffine {
    struct Aux {
        const uint16_t *scales, *biases;
        int64_t groups; // per row
    };
    struct Raw { u32x4 c[BITS / 2]; uint32_t s, b; };
    struct X { float v[64]; };
    static __device__ __forceinline__ void load(Raw &r, const uint8_t *row, int u, int,
                                                const Aux &a, int64_t j) {
#pragma unroll
        for (int c = 0; c < BITS / 2; c++) r.c[c] = ld16(row + 8 * BITS * u + 16 * c);
        r.s = a.scales[j * a.groups + u];
        r.b = a.biases[j * a.groups + u];
    }
    static __device__ __forceinline__ int x4_index(int u, int i, int) { return 16 * u + i; }
    static __device__ __forceinline__ void x4_slot(int q, int, int &u, int &i) {
        u = q >> 4;
        i = q & 15;
    }
    static __device__ __forceinline__ void put_x(X &x, int i, f32x4 v) { put4(&x.v[4 * i], v); }
    static __device__ __forceinline__ f32x4 get_x(const X &x, int i) { return get4(&x.v[4 * i]); }
    static __device__ __forceinline__ void finish_x(X &) {}
    static __device__ __forceinline__ float dot(const Raw &r, const X &x, int) {
        const float s = __builtin_bit_cast(float, r.s << 16);
        const float b = __builtin_bit_cast(float, r.b << 16);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int w = 0; w < 2 * BITS; w++) {
            const uint32_t word = r.c[w >> 2][w & 3];
            if (BITS == 4) {
                // bytes of lo: codes 0, 2, 4, 6 of the word; of hi: 1, 3, 5, 7
                const uint32_t lo = opaque(word & 0x0f0f0f0fu);
                const uint32_t hi = opaque((word >> 4) & 0x0f0f0f0fu);
                const float *xv = &x.v[8 * w];
                a0 = fmaf(fmaf(ub0(lo), s, b), xv[0], a0);
                a1 = fmaf(fmaf(ub0(hi), s, b), xv[1], a1);
                a0 = fmaf(fmaf(ub1(lo), s, b), xv[2], a0);
                a1 = fmaf(fmaf(ub1(hi), s, b), xv[3], a1);
                a0 = fmaf(fmaf(ub2(lo), s, b), xv[4], a0);
                a1 = fmaf(fmaf(ub2(hi), s, b), xv[5], a1);
                a0 = fmaf(fmaf(ub3(lo), s, b), xv[6], a0);
                a1 = fmaf(fmaf(ub3(hi), s, b), xv[7], a1);
            } else {
                const float *xv = &x.v[4 * w];
                a0 = fmaf(fmaf(ub0(word), s, b), xv[0], a0);
                a1 = fmaf(fmaf(ub1(word), s, b), xv[1], a1);
                a0 = fmaf(fmaf(ub2(word), s, b), xv[2], a0);
                a1 = fmaf(fmaf(ub3(word), s, b), xv[3], a1);
            }
        }
        return a0 + a1;
    }
};

// Lane geometry common to both kernels.
template <int UPL>
struct Lanes {
    int tid, T, slot, lane, NG;
    int uid[UPL];  // units owned by this lane
    int ulod[UPL]; // unit actually read: padding lanes re-read a valid unit
    bool uvalid[UPL];
    __device__ __forceinline__ Lanes(int U, int L, int G) : Lanes(U, L, G, blockDim.x) {}
    // T given: the workgroup size as launched (saves reading it at run time)
    __device__ __forceinline__ Lanes(int U, int L, int G, int T_) {
        tid = threadIdx.x;
        T = T_;
        slot = tid / L;
        lane = tid - slot * L;
        NG = L / G;
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            uid[i] = lane + i * L;
            uvalid[i] = uid[i] < U;
            ulod[i] = uvalid[i] ? uid[i] : U - 1;
        }
    }
};

// Workgroups per compute unit that the streaming GEMV kernels (staged,
// direct, affine, transposed) are launched with. A workgroup's waves are dealt
// to the four SIMDs of a compute unit in turn, starting at the first SIMD, so
// workgroups of 4w+1 waves (e.g. 320 threads) pile two waves of every
// workgroup onto one SIMD: a third such workgroup rarely finds room (measured
// mean residency about 7 waves per compute unit) and two per compute unit
// stream best. Launches whose workgroups were padded to 256 threads (4 waves,
// spread evenly) take four per compute unit, 4 waves per SIMD: on the Q6_K
// vocabulary product 128 us with two, 118 us with three, 114 us with four.
// The expert-indexed launches keep every resident workgroup.
constexpr int STREAM_PER_CU = 2;
constexpr int STREAM_PER_CU_4W = 4;

// The dispatcher deals the workgroups of a launch to the 8 XCDs in turn
// (workgroup b to XCD b % 8), and each XCD has its own L2. The streaming
// kernels give consecutive batch numbers to workgroups of one XCD: XCD x's
// workgroups x, x + 8, x + 16, ... become batches x*q + min(x, r), +1, +2, ...
// (q = G / 8, r = G % 8, a bijection of [0, G)), so the y values of
// neighbouring batches, which share cache lines, are written through one L2
// instead of partial lines from several.
__device__ __forceinline__ int xcd_block(int b, int G) {
    const int q = G >> 3, r = G & 7, x = b & 7;
    return x * q + (x < r ? x : r) + (b >> 3);
}

// Buffer descriptor over [p, p + bytes) (raw buffer loads check the range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t batch_rsrc(const uint8_t *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, bytes, 0x00020000);
}

// Resident workgroups per compute unit for one kernel at a given block size
// and LDS size (cached: the query only reads kernel metadata).
template <typename K>
inline int resident_per_cu(K kernel, int T, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<int, size_t>, int> cache;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find({T, lds});
    if (it != cache.end()) return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, T, lds) != hipSuccess ||
        nb < 1) {
        (void)hipGetLastError();
        nb = 1;
    }
    cache[{T, lds}] = nb;
    return nb;
}

} // namespace qmv
