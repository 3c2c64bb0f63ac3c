// N-token (prefill) path for gfx950 matrix cores:
//   Y[t][j] (=|+=) sum_i X[t][i] * w_j[i]   for many tokens t at once.
//
// Operation: rullama 0.5.0, src/backend/matmul.rs (y = x @ W over weight rows
// stored in GGUF form; the batched variant runs the same product for several
// rows of x). Block layout of Q4_K: 144-byte super-blocks of 256 weights, d and
// dmin (f16), eight 6-bit scales and mins packed in 12 bytes, 128 code bytes
// (the ggml reading of the format the page calls ggml-exact); weight
// w = d*sc*q - dmin*m.
//
// Two kernels on the caller's stream:
//  1. qmv_mfma_prep_x, one wave per (token, pair of super-blocks): finds the
//     power of two p with max|x_t|/p in [2^14, 2^15) and writes x_t/p as two
//     f16 terms hi = f16(x/p), lo = f16(x/p - hi) (22 significant bits
//     together) in the order the main kernel's A operands take them, so that
//     each of its wave loads reads one contiguous kilobyte; also the f32 sum
//     of each 32-weight sub-block (fixed order) divided by 32p, split hi/lo,
//     and p.
//  2. qmv_mfma_q4_k: v_mfma_f32_32x32x16_f16 with B = sc*q, an exact f16
//     integer (<= 945) made by inserting the nibble into the mantissa of 1024
//     and one packed f16 FMA, against hi and lo. The 16 K-steps of a
//     super-block accumulate in a fresh f32 tile; then acc += d*tile. The min
//     term dmin * sum_g m_g * sum(x over g) takes one more MFMA per
//     super-block (A = the hi/lo sums, B = the 6-bit mins, exact); the token's
//     p scales the result once, at the store (by its exponent, so that p need
//     not be a normal f32).
//
// Mapping of the main kernel. A workgroup owns 64 tokens x 64 rows and has 4
// waves, one per SIMD; wave w takes super-blocks w, w+4, ... and all 64 x 64
// outputs, as four 32x32 accumulators (token tile tt x row tile rt). Lane l feeds
// A[l%32][8(l/32)+i] and B[8(l/32)+i][l%32] and receives
// D[8(r/4)+4(l/32)+r%4][l%32] in register r: tokens are the MFMA rows, weight
// rows the columns, so a lane's block scales are those of one weight row. Each
// decoded B operand feeds four MFMAs (two token tiles, hi and lo) and each A
// operand two (both row tiles). Each wave copies its super-blocks' bytes of the
// 64 rows into its own LDS slots (buffer_load ... lds, two slots, one
// super-block ahead) and reads its lanes' fields from there; its A operands
// come from the staged x in global memory (L2), six K-steps ahead in
// registers. At the end the four waves' partial tiles are summed in LDS in
// wave order. Results depend
// only on k, never on the row range or the token tiling.
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64;          // tokens per tile
constexpr int TN = 64;          // weight rows per tile
constexpr int KW = 4;           // waves per workgroup (split of the super-blocks)
constexpr int NT = 64 * KW;     // threads per workgroup
constexpr int SBB = 144;        // bytes of a Q4_K super-block
constexpr int SLOT = TN * SBB;  // one super-block of the tile's rows in LDS
constexpr int PF = 6;           // K-steps of A operands loaded ahead
constexpr int RING = 8;         // A operand slots (16 K-steps per super-block: a multiple)
static_assert((size_t)(KW / 2) * TM * TN * sizeof(float) <= (size_t)KW * SLOT,
              "the partial tiles of half the waves fit in one slot array");

// Staged x, per 64-token group T and super-block s (nsb = k/256):
//   XS: [T][s][j 16][tt 2][h 2][lane 64] x 16 bytes (8 f16, h = 0 hi, 1 lo);
//       lane l holds token 32tt + l%32, elements 32(j/2) + 16(l/32) + 8(j%2) +
//       perm8(i) of the super-block in slot i
//   SM: [T][s][tt 2][lane 64] x 16 bytes: sub-block sums / 32p (lanes 0-31 hi,
//       32-63 lo; slot g = sub-block g)
//   PE: [T][token 64] ints: the exponent of p
constexpr size_t xs_bytes(int64_t tiles, int64_t nsb) { return (size_t)tiles * nsb * 64 * 1024; }
constexpr size_t sm_bytes(int64_t tiles, int64_t nsb) { return (size_t)tiles * nsb * 2 * 1024; }
constexpr size_t pe_bytes(int64_t tiles) { return (size_t)tiles * 64 * 4; }

// Slot i of an 8-wide operand piece holds element perm8(i): the order in which
// the code decoder below produces its f16 pairs (bytes 0 and 2 of a word, then
// bytes 1 and 3).
__device__ __forceinline__ int perm8(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}
// bf16 of f (round to nearest even; NaN stays NaN) and back
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t h) { return __builtin_bit_cast(float, h << 16); }
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// ------------------------------------------------------------ x staging

// One wave per (token of the padded token range, pair of super-blocks c);
// tokens at or past m stage zeros. Lane q takes 8-element group G = 64c + q;
// group G of super-block s = G/32 covers elements 8(G%32) .. +7, which is
// K-step j = 2g + j2 of lane half kh for g = (G%32)/4, kh = (G/2)%2, j2 = G%2. Every wave first finds the token's largest magnitude over all of k
// (the row is read again from cache by each wave of the token).
template <bool BF>
__global__ __launch_bounds__(64) void qmv_mfma_prep_x(const float *__restrict__ x, int64_t k,
                                                      int64_t m, uint8_t *__restrict__ xs,
                                                      uint8_t *__restrict__ sm,
                                                      int *__restrict__ pe) {
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.y;
    const int64_t T = t >> 6;
    const int tt = (int)((t >> 5) & 1), ln = (int)(t & 31);
    const int64_t nsb = k >> 8;
    const int64_t ng = k >> 3; // 8-element groups
    const bool live = t < m;
    const f32x4 *xt = (const f32x4 *)(x + (live ? t : 0) * k);

    // this lane's group, loaded before the max pass so that both are in flight
    const int64_t G = (int64_t)blockIdx.x * 64 + lane;
    const bool has = G < ng; // a lone last super-block leaves lanes 32-63 idle
    float v[8];
    if (live && has) {
        const f32x4 a = xt[2 * G], b = xt[2 * G + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = 0.f;
    }

    // the token's largest magnitude
    float mx = 0.f;
    if (live) {
        // sixteen independent loads in flight per lane (k/4 is a multiple of 64)
        int64_t q = lane;
        for (; q + 960 < 2 * ng; q += 1024) {
            f32x4 c[16];
#pragma unroll
            for (int u = 0; u < 16; u++) c[u] = xt[q + 64 * u];
#pragma unroll
            for (int u = 0; u < 16; u++)
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(c[u].x), fabsf(c[u].y)),
                                     fmaxf(fabsf(c[u].z), fabsf(c[u].w))));
        }
        for (; q < 2 * ng; q += 64) {
            const f32x4 c = xt[q];
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
        }
    }
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    int e = 0;
    if (mx > 0.f) {
        (void)frexpf(mx, &e); // mx = f * 2^e, f in [0.5, 1)
        e -= 15;              // mx / 2^e in [2^14, 2^15)
    }
    if (blockIdx.x == 0 && lane == 0) pe[t] = e;

    if (!has) return; // whole sub-blocks of lanes leave together
    const int64_t s = G >> 5;
    const int gi = (int)(G & 31);
    const int g = gi >> 2, kh = (gi >> 1) & 1, j2 = gi & 1;
    float w[8], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        w[i] = ldexpf(v[perm8(i)], -e);
        sum += ldexpf(v[i], -e);
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if constexpr (BF) {
            const uint32_t h0 = bf16_bits(w[2 * i]), h1 = bf16_bits(w[2 * i + 1]);
            hi[i] = h0 | (h1 << 16);
            lo[i] = bf16_bits(w[2 * i] - bf2f(h0)) | (bf16_bits(w[2 * i + 1] - bf2f(h1)) << 16);
        } else {
            const _Float16 h0 = (_Float16)w[2 * i], h1 = (_Float16)w[2 * i + 1];
            hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
            lo[i] = pk_f16(w[2 * i] - (float)h0, w[2 * i + 1] - (float)h1);
        }
    }
    const int j = 2 * g + j2;
    uint8_t *dst = xs + ((size_t)((T * nsb + s) * 16 + j) * 4 + tt * 2) * 1024 +
                   (size_t)(ln + 32 * kh) * 16;
    *(u32x4 *)dst = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4 *)(dst + 1024) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    if constexpr (BF) return; // the sums serve the Q4_K min term only
    // sub-block sum over its four groups (consecutive lanes), fixed order
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    if ((gi & 3) == 0) {
        // a sum of 32 values below 2^15 can reach 2^20: divided by 32
        const float sv = sum * 0.03125f;
        const _Float16 h = (_Float16)sv;
        _Float16 *sd = (_Float16 *)(sm + ((size_t)(T * nsb + s) * 2 + tt) * 1024);
        sd[ln * 8 + g] = h;
        sd[(ln + 32) * 8 + g] = (_Float16)(sv - (float)h);
    }
}

// The four waves' partial tiles (waves 0-1 in red0, 2-3 in red1, register
// order) summed in wave order, scaled by each token's p and stored. Thread
// tid takes outputs o = tid + 256 i; the 16 exponents (every padded token has
// one) and, when accumulating, the old values are all loaded before any store.
__device__ __forceinline__ void tile_store(const float *red0, const float *red1,
                                           const int *__restrict__ pe, float *__restrict__ y,
                                           int64_t T, int64_t n, int64_t m, int64_t r0, int rows,
                                           int accumulate, int tid) {
    constexpr int PER = TM * TN / NT;
    int ex[PER];
    float old[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int o = tid + NT * i;
        const int ln = o & 63, r = (o >> 6) & 15, rt = (o >> 10) & 1, tt = o >> 11;
        const int tok = 32 * tt + 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
        const int row = 32 * rt + (ln & 31);
        const int64_t t = T * TM + tok;
        ex[i] = pe[t];
        old[i] = (accumulate && t < m && row < rows) ? y[t * n + r0 + row] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int o = tid + NT * i;
        float v = red0[o];
#pragma unroll
        for (int w = 1; w < KW; w++)
            v += (w < KW / 2 ? red0 : red1)[(w % (KW / 2)) * TM * TN + o];
        const int ln = o & 63, r = (o >> 6) & 15, rt = (o >> 10) & 1, tt = o >> 11;
        const int tok = 32 * tt + 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
        const int row = 32 * rt + (ln & 31);
        const int64_t t = T * TM + tok;
        if (t < m && row < rows) y[t * n + r0 + row] = old[i] + ldexpf(v, ex[i]);
    }
}

// ------------------------------------------------------------ main kernel

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Hide a value from the optimiser (keeps bit-field inserts as v_bfi_b32).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Code decode. A 4-bit code q sits in a byte of the packed chunk, low nibble
// (sub-block 2c) or high nibble (sub-block 2c+1). Inserted into the mantissa
// of the f16 1024 (bits 0-3: 1024 + q; bits 4-7: 1024 + 16q) it is turned into
// the exact f16 integer sc*q by one packed FMA: (1024 + q)*sc - 1024*sc, or
// (1024 + 16q)*(sc/16) - 64*sc. Bytes 0 and 2 of a word give one f16 pair,
// bytes 1 and 3 (after a one-byte rotation) the other.
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t mask, f16x2 sc, f16x2 off) {
    const uint32_t mag = (w & mask) | (0x64006400u & ~mask); // one v_bfi_b32
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_fma(__builtin_bit_cast(f16x2, mag), sc, off));
}
__device__ __forceinline__ f16x8 codes_b(uint32_t w0, uint32_t w1, uint32_t mask, f16x2 sc,
                                         f16x2 off) {
    const uint32_t r0 = __builtin_amdgcn_alignbyte(w0, w0, 1);
    const uint32_t r1 = __builtin_amdgcn_alignbyte(w1, w1, 1);
    const u32x4 r = {code_pair(w0, mask, sc, off), code_pair(r0, mask, sc, off),
                     code_pair(w1, mask, sc, off), code_pair(r1, mask, sc, off)};
    return __builtin_bit_cast(f16x8, r);
}

// Byte i (0..11) of the packed scale/min field of a Q4_K header.
__device__ __forceinline__ uint32_t scb(const u32x4 &h, int i) {
    return (h[1 + (i >> 2)] >> (8 * (i & 3))) & 0xffu;
}
__device__ __forceinline__ void scale_min(const u32x4 &h, int g, uint32_t &sc, uint32_t &mn) {
    if (g < 4) {
        sc = scb(h, g) & 63u;
        mn = scb(h, g + 4) & 63u;
    } else {
        sc = (scb(h, g + 4) & 15u) | ((scb(h, g - 4) >> 6) << 4);
        mn = (scb(h, g + 4) >> 4) | ((scb(h, g) >> 6) << 4);
    }
}

// TT: 32-token tiles per workgroup (2; 1 when the call has at most 32 tokens,
// which skips the operand loads and MFMAs of the empty second half)
template <int TT>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void qmv_mfma_q4_k(const uint8_t *__restrict__ W,
                                                       const uint8_t *__restrict__ xs,
                                                       const uint8_t *__restrict__ sm,
                                                       const int *__restrict__ pe,
                                                       float *__restrict__ y, int64_t k, int64_t n,
                                                       int64_t m, int64_t row_bytes,
                                                       int64_t j_start, int64_t j_end,
                                                       int accumulate) {
    // Two statically separate LDS arrays for the two weight slots, so that the
    // compiler can tell that the copy in flight into one slot never touches
    // the slot being read (otherwise it waits for the copy before every read).
    __shared__ __attribute__((aligned(16))) uint8_t slot0[KW][SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[KW][SLOT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 31, kh = lane >> 5;
    const int64_t r0 = j_start + (int64_t)blockIdx.x * TN;
    const int64_t T = blockIdx.y;
    const int nsb = (int)(k >> 8);
    const int rows = (int)(j_end - r0 < TN ? j_end - r0 : TN); // live rows of the tile
    const uint32_t mlo = opaque(0x000f000fu), mhi = opaque(0x00f000f0u);

    // Staging copy: piece p = 64*i + lane of a super-block is bytes
    // 16*(p%9).. of row p/9; it lands at 16*p, so rows sit 144 bytes apart.
    // Rows beyond the tile's end repeat its last live row (never stored).
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(W + r0 * row_bytes), (short)0,
                                          (int)(rows * row_bytes), 0x00020000);
    int poff[9];
#pragma unroll
    for (int i = 0; i < 9; i++) {
        const int p = 64 * i + lane, r = p / 9;
        poff[i] = (r < rows ? r : rows - 1) * (int)row_bytes + 16 * (p - 9 * r);
    }
    // A descriptor with no records: every load through it is out of range,
    // reads nothing and returns zeros. Copies and operand loads past the last
    // super-block go through it, so that every path issues the same memory
    // instructions and the compiler's wait counts stay exact (a load issued
    // on one branch only makes it wait for every load in flight).
    const __amdgpu_buffer_rsrc_t rnull =
        __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, 0, 0x00020000);
    auto copy_sb = [&](int s, uint8_t *dst) {
        const bool ok = s >= 0;
#pragma unroll
        for (int i = 0; i < 9; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ok ? rs : rnull, (__attribute__((address_space(3))) void *)(dst + 1024 * i), 16,
                poff[i], ok ? SBB * s : 0, 0, 2 /* nontemporal */);
    };

    f32x16 acc[TT][2];
#pragma unroll
    for (int a = 0; a < TT; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[a][b][r] = 0.f;

    // This wave's super-blocks: wave, wave + KW, ...; the next one's bytes
    // are copied into the other slot while one is decoded. A operands of
    // K-step j of super-block s sit at xw + 65536 s + 4096 j + 1024 (2 tt + h);
    // they are loaded PF K-steps ahead (into the next super-block at the end
    // of one), the loads pinned there against the scheduler, which would
    // otherwise sink them next to their MFMAs.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xs + (size_t)T * nsb * 65536), (short)0, nsb * 65536, 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(sm + (size_t)T * nsb * 2048), (short)0, nsb * 2048, 0x00020000);
    f16x8 ring[RING][TT][2];
    auto load_a = [&](int s, int j, int bi) {
        const bool ok = s >= 0;
#pragma unroll
        for (int a = 0; a < 2 * TT; a++)
            ring[bi][a >> 1][a & 1] = __builtin_bit_cast(
                f16x8, __builtin_amdgcn_raw_buffer_load_b128(ok ? xr : rnull, lane * 16,
                                                             ok ? s * 65536 + 4096 * j + 1024 * a : 0, 0));
    };
    {
        const int s0 = wave < nsb ? wave : -1;
        copy_sb(s0, slot0[wave]);
#pragma unroll
        for (int j = 0; j < PF; j++) load_a(s0, j, j);
    }
    auto super_block = [&](int s, const uint8_t *cur_slot, uint8_t *nxt) {
        // this super-block's bytes have landed once at most the 2*TT*PF operand
        // loads issued after its copy are outstanding (loads complete in order)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * TT * PF) : "memory");
        const int sn = s + KW < nsb ? s + KW : -1;
        copy_sb(sn, nxt);
        // the sub-block sums of x for the min term, needed at the end
        f16x8 am[TT];
#pragma unroll
        for (int tt = 0; tt < TT; tt++)
            am[tt] = __builtin_bit_cast(
                f16x8, __builtin_amdgcn_raw_buffer_load_b128(sr, lane * 16, s * 2048 + 1024 * tt, 0));
        const uint8_t *wsb = cur_slot;
        const uint8_t *wrow[2] = {wsb + nl * SBB, wsb + (nl + 32) * SBB};
        u32x4 hd[2];
        float dd[2], dm[2];
#pragma unroll
        for (int rt = 0; rt < 2; rt++) {
            hd[rt] = *(const u32x4 *)wrow[rt];
            dd[rt] = h2f(hd[rt][0]);
            dm[rt] = h2f(hd[rt][0] >> 16);
        }
        f32x16 tile[TT][2];
#pragma unroll
        for (int g = 0; g < 8; g++) {
            const int c = g >> 1, hn = g & 1;
            u32x4 q[2];
            f16x2 sc2[2], off2[2];
#pragma unroll
            for (int rt = 0; rt < 2; rt++) {
                q[rt] = *(const u32x4 *)(wrow[rt] + 16 + 32 * c + 16 * kh);
                uint32_t sc, mn;
                scale_min(hd[rt], g, sc, mn);
                const float scf = (float)sc;
                const _Float16 sch = (_Float16)(hn ? scf * 0.0625f : scf);
                const _Float16 off = (_Float16)(hn ? -64.f * scf : -1024.f * scf);
                sc2[rt] = f16x2{sch, sch};
                off2[rt] = f16x2{off, off};
            }
#pragma unroll
            for (int j2 = 0; j2 < 2; j2++) {
                const int j = 2 * g + j2;
                const int cur = j % RING;
                // operands PF K-steps ahead, into the next super-block at the end
                if (j + PF < 16)
                    load_a(s, j + PF, (j + PF) % RING);
                else
                    load_a(sn, j + PF - 16, (j + PF) % RING);
                __builtin_amdgcn_sched_barrier(0x0386); // VALU, SALU and LDS may cross
                f16x8 b[2];
#pragma unroll
                for (int rt = 0; rt < 2; rt++)
                    b[rt] = codes_b(q[rt][2 * j2], q[rt][2 * j2 + 1], hn ? mhi : mlo, sc2[rt],
                                    off2[rt]);
                // hi for all four tiles, then lo: no accumulator is reused back to back
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int tt = 0; tt < TT; tt++)
#pragma unroll
                        for (int rt = 0; rt < 2; rt++)
                            tile[tt][rt] = mfma(ring[cur][tt][h], b[rt],
                                                (j == 0 && h == 0) ? f32x16{} : tile[tt][rt]);
            }
        }
        // acc += d * tile - 32 * dmin * (sum_g m_g * sum_g(x) / 32)
        f16x8 mins[2];
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int g = 0; g < 8; g++) {
                uint32_t sc, mn;
                scale_min(hd[rt], g, sc, mn);
                mins[rt][g] = (_Float16)(float)mn;
            }
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
#pragma unroll
            for (int rt = 0; rt < 2; rt++) {
                const f32x16 mt = mfma(am[tt], mins[rt], f32x16{});
                const float md = -32.f * dm[rt];
#pragma unroll
                for (int e = 0; e < 16; e++)
                    acc[tt][rt][e] = fmaf(md, mt[e], fmaf(dd[rt], tile[tt][rt][e], acc[tt][rt][e]));
            }
        }
        };
    // pairs of super-blocks, then an odd last one: no branch inside the loop
    // body, so that the compiler's wait counts hold across its iterations
    int s = wave;
    for (; s + KW < nsb; s += 2 * KW) {
        super_block(s, slot0[wave], slot1[wave]);
        super_block(s + KW, slot1[wave], slot0[wave]);
    }
    if (s < nsb) super_block(s, slot0[wave], slot1[wave]);

    // Sum the four waves' partial tiles in wave order, scale by p, store.
    __syncthreads(); // every wave is done with its staged bytes
    // (waves 0-1 write into the first array, 2-3 into the second)
    float *red0 = (float *)&slot0[0][0], *red1 = (float *)&slot1[0][0];
    float *mine = (wave < KW / 2 ? red0 : red1) + (size_t)(wave % (KW / 2)) * TM * TN;
#pragma unroll
    for (int tt = 0; tt < TT; tt++)
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                mine[((tt * 2 + rt) * 16 + r) * 64 + lane] = acc[tt][rt][r];
    // (with TT = 1 the second half's slots hold nothing: no token there is stored)
    __syncthreads();
    tile_store(red0, red1, pe, y, T, n, m, r0, rows, accumulate, tid);
}

// ------------------------------------------------------------ other formats
// Every other format has per-weight values v = s*q' that are exact in f32 (a
// scale times a small integer) or are f16/bf16 themselves. The B operand is
// then v split into two f16 terms, B_hi = f16(v) and B_lo = f16(v - B_hi)
// (together exact while v stays within the normal f16 range), and each K-step
// adds A_hi*B_hi + A_lo*B_hi + A_hi*B_lo (the A_lo*B_lo term is below 2^-22
// of the product); f16 weights need no B_lo, and bf16 weights run the bf16
// matrix cores against x split into two bf16 terms (16 significant bits).
// There is no per-block step: the scales sit in B, so one accumulator per
// tile runs over all of k. A chunk is the run of K that one LDS slot holds:
// 256 weights (one super-block, or eight 32-weight blocks), 128 for f16/bf16.
//
// Decoders: dec(row, m, j, kh, bh, bl) fills the B operand of K-step j of the
// chunk for lane half kh, i.e. weights e0 + perm8(i) in slot i with
// e0 = 32(j/2) + 16kh + 8(j%2), from the row's chunk bytes at row + m (row:
// the 16-byte aligned start of the row's copy in LDS; m is 0 except for Q6_K,
// whose 210-byte super-blocks start anywhere in a 16-byte piece). Reads may
// run up to 12 bytes past the chunk (the slots keep 16 bytes of slack).

// The four dwords that hold bytes [o, o+16) of an LDS row, o any offset:
// aligned dword reads and one funnel shift each.
__device__ __forceinline__ void lds_bytes16(const uint8_t *row, int o, uint32_t (&w)[4]) {
    const uint32_t *a = (const uint32_t *)(row + (o & ~3));
    const uint32_t sh = (uint32_t)o & 3u;
    uint32_t d[5];
#pragma unroll
    for (int i = 0; i < 5; i++) d[i] = a[i];
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
}
__device__ __forceinline__ void lds_bytes8(const uint8_t *row, int o, uint32_t (&w)[2]) {
    const uint32_t *a = (const uint32_t *)(row + (o & ~3));
    const uint32_t sh = (uint32_t)o & 3u;
    const uint32_t d0 = a[0], d1 = a[1], d2 = a[2];
    w[0] = __builtin_amdgcn_alignbyte(d1, d0, sh);
    w[1] = __builtin_amdgcn_alignbyte(d2, d1, sh);
}
__device__ __forceinline__ uint32_t lds_u16(const uint8_t *row, int o) {
    const uint32_t *a = (const uint32_t *)(row + (o & ~3));
    return __builtin_amdgcn_alignbyte(a[1], a[0], (uint32_t)o & 3u) & 0xffffu;
}

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// B_hi, B_lo of v = s*q for a pair of exact f16 integers q and the scale pair
// s (hi and lo f16 terms of an f32 scale; sl = 0 when s is one f16).
__device__ __forceinline__ void hl_pair(f16x2 q, f16x2 sh, f16x2 sl, uint32_t &bh, uint32_t &bl) {
    const f16x2 h = q * sh;                                     // rounded to f16
    const f16x2 r = __builtin_elementwise_fma(q, sh, -h);      // its exact remainder
    bh = as_u(h);
    bl = as_u(__builtin_elementwise_fma(q, sl, r));
}

// Code bytes: bytes 0 and 2 of a word, then (after a one-byte rotation) 1 and
// 3, give the f16 pairs of slots (0,1), (2,3); the second word slots (4..7).
// Signed 8-bit codes: (b ^ 0x80) inserted into the mantissa of 1024 is
// 1152 + q; minus 1152 is q, exact.
__device__ __forceinline__ f16x2 q8_pair(uint32_t w) {
    const uint32_t v = (w & 0x00ff00ffu) ^ 0x64806480u;
    return as_h2(v) + f16x2{(_Float16)-1152.f, (_Float16)-1152.f};
}

struct DQ8_0 { // 8 blocks of 34 bytes: f16 d, 32 signed codes
    static constexpr int CK = 256, CB = 272, NP = 17;
    static constexpr bool LO = true, BF = false, SHIFTED = false;
    static __device__ __forceinline__ void dec(const uint8_t *row, int m, int j, int kh,
                                              uint32_t (&bh)[4], uint32_t (&bl)[4]) {
        const int b = j >> 1, o = 34 * b + 2 + 16 * kh + 8 * (j & 1);
        uint32_t w[2];
        lds_bytes8(row, o, w);
        const uint32_t d = lds_u16(row, 34 * b);
        const f16x2 s = as_h2(d | (d << 16)), z = {};
#pragma unroll
        for (int h = 0; h < 2; h++) {
            hl_pair(q8_pair(w[h]), s, z, bh[2 * h], bl[2 * h]);
            hl_pair(q8_pair(__builtin_amdgcn_alignbyte(w[h], w[h], 1)), s, z, bh[2 * h + 1],
                    bl[2 * h + 1]);
        }
    }
};

// 4-bit codes in bytes: lane half 0 takes the low nibbles (1024 + q inserted
// into the mantissa), lane half 1 the high nibbles (1024 + 16q, scaled by
// 1/16); `off` is then subtracted. hb (5-bit codes) are fifth bits already
// at bit 4 of each half (low nibble) or bit 8 (high nibble).
__device__ __forceinline__ f16x2 q4_pair(uint32_t w, int kh, uint32_t hb, _Float16 off) {
    if (kh == 0) {
        const uint32_t v = (w & 0x000f000fu) | 0x64006400u | hb;
        return as_h2(v) - f16x2{(_Float16)1024.f + off, (_Float16)1024.f + off};
    }
    const uint32_t v = (w & 0x00f000f0u) | 0x64006400u | hb;
    return __builtin_elementwise_fma(as_h2(v), f16x2{(_Float16)0.0625f, (_Float16)0.0625f},
                                     f16x2{-(_Float16)64.f - off, -(_Float16)64.f - off});
}

struct DQ4_0 { // 8 blocks of 18 bytes: f16 d, 16 bytes of nibbles (e, e+16)
    static constexpr int CK = 256, CB = 144, NP = 9;
    static constexpr bool LO = true, BF = false, SHIFTED = false;
    static __device__ __forceinline__ void dec(const uint8_t *row, int m, int j, int kh,
                                              uint32_t (&bh)[4], uint32_t (&bl)[4]) {
        const int b = j >> 1, o = 18 * b + 2 + 8 * (j & 1);
        uint32_t w[2];
        lds_bytes8(row, o, w);
        const uint32_t d = lds_u16(row, 18 * b);
        const f16x2 s = as_h2(d | (d << 16)), z = {};
#pragma unroll
        for (int h = 0; h < 2; h++) {
            hl_pair(q4_pair(w[h], kh, 0u, (_Float16)8.f), s, z, bh[2 * h], bl[2 * h]);
            hl_pair(q4_pair(__builtin_amdgcn_alignbyte(w[h], w[h], 1), kh, 0u, (_Float16)8.f), s,
                    z, bh[2 * h + 1], bl[2 * h + 1]);
        }
    }
};

struct DQ5_0 { // 8 blocks of 22 bytes: f16 d, 32 fifth bits, 16 bytes of nibbles
    static constexpr int CK = 256, CB = 176, NP = 11;
    static constexpr bool LO = true, BF = false, SHIFTED = false;
    static __device__ __forceinline__ void dec(const uint8_t *row, int m, int j, int kh,
                                              uint32_t (&bh)[4], uint32_t (&bl)[4]) {
        const int b = j >> 1, o = 22 * b + 6 + 8 * (j & 1);
        uint32_t w[2];
        lds_bytes8(row, o, w);
        const uint32_t d = lds_u16(row, 22 * b);
        const uint32_t qh = lds_u16(row, 22 * b + 2) | (lds_u16(row, 22 * b + 4) << 16);
        // fifth bits of weights e0 + t (t = 0..7): bit t of hb8
        const uint32_t hb8 = (qh >> (16 * kh + 8 * (j & 1))) & 0xffu;
        // bit t at 4 + t (low half) and bit t+2 at 20 + t (high half)
        const uint32_t sp = (hb8 << 4) | (hb8 << 18);
        const int hs = kh ? 4 : 0; // high nibbles put the fifth bit at bit 8
        const f16x2 s = as_h2(d | (d << 16)), z = {};
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int r = 0; r < 2; r++) {
                const int t = 4 * h + r; // weights t and t + 2 of the pair
                const uint32_t hb = ((sp >> t) & 0x00100010u) << hs;
                const uint32_t ww = r ? __builtin_amdgcn_alignbyte(w[h], w[h], 1) : w[h];
                hl_pair(q4_pair(ww, kh, hb, (_Float16)16.f), s, z, bh[2 * h + r], bl[2 * h + r]);
            }
    }
};

struct DQ6_K { // one 210-byte super-block: ql[128], qh[64], 16 int8 scales, f16 d
    static constexpr int CK = 256, CB = 210, NP = 15; // 15 pieces cover it at any alignment
    static constexpr bool LO = true, BF = false, SHIFTED = true;
    static __device__ __forceinline__ void dec(const uint8_t *row, int m, int j, int kh,
                                              uint32_t (&bh)[4], uint32_t (&bl)[4]) {
        const int e0 = 32 * (j >> 1) + 16 * kh + 8 * (j & 1);
        const int h = e0 >> 7, g = (e0 >> 5) & 3, l0 = e0 & 31;
        uint32_t lo[2], hi[2];
        lds_bytes8(row, m + 64 * h + 32 * (g & 1) + l0, lo);
        lds_bytes8(row, m + 128 + 32 * h + l0, hi);
        const uint32_t sd = lds_u16(row, m + 208);
        const uint32_t scw = lds_u16(row, m + 192 + (e0 >> 4) - ((e0 >> 4) & 1));
        const int sc = (int)(int8_t)(uint8_t)(scw >> (8 * ((e0 >> 4) & 1)));
        // s = d * sc exactly in f32, as two f16 terms
        const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)sd) * (float)sc;
        const _Float16 s1 = (_Float16)sf, s2 = (_Float16)(sf - (float)s1);
        const f16x2 sh = {s1, s1}, sl = {s2, s2};
        const int ns = 4 * (g >> 1), hsft = 2 * g;
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
            for (int r = 0; r < 2; r++) {
                const uint32_t a = r ? __builtin_amdgcn_alignbyte(lo[p], lo[p], 1) : lo[p];
                const uint32_t c = r ? __builtin_amdgcn_alignbyte(hi[p], hi[p], 1) : hi[p];
                // 1024 + q (q = low 4 bits | high 2 bits << 4), then q - 32
                const uint32_t v = ((a >> ns) & 0x000f000fu) | (((c >> hsft) & 0x00030003u) << 4) |
                                   0x64006400u;
                const f16x2 q = as_h2(v) - f16x2{(_Float16)1056.f, (_Float16)1056.f};
                hl_pair(q, sh, sl, bh[2 * p + r], bl[2 * p + r]);
            }
    }
};

template <bool B16>
struct DHalf { // f16 (B16 false) or bf16 weights, 128 per chunk
    static constexpr int CK = 128, CB = 256, NP = 16;
    static constexpr bool LO = false, BF = B16, SHIFTED = false;
    static __device__ __forceinline__ void dec(const uint8_t *row, int, int j, int kh,
                                              uint32_t (&bh)[4], uint32_t (&)[4]) {
        const int e0 = 32 * (j >> 1) + 16 * kh + 8 * (j & 1);
        const u32x4 w = *(const u32x4 *)(row + 2 * e0);
        // slots hold weights (0,2), (1,3), (4,6), (5,7)
        bh[0] = __builtin_amdgcn_perm(w.y, w.x, 0x05040100u);
        bh[1] = __builtin_amdgcn_perm(w.y, w.x, 0x07060302u);
        bh[2] = __builtin_amdgcn_perm(w.w, w.z, 0x05040100u);
        bh[3] = __builtin_amdgcn_perm(w.w, w.z, 0x07060302u);
    }
};

__device__ __forceinline__ f32x16 mfma_bf(u32x4 a, u32x4 b, f32x16 c) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(s16x8, a),
                                                    __builtin_bit_cast(s16x8, b), c, 0, 0, 0);
}

// Main kernels for the formats above (one per format, all this body). Same tiling and staging as the Q4_K
// kernel: a workgroup owns 64 tokens x 64 rows, wave w takes chunks w, w+4,
// ..., copies its chunk's 64 rows into one of its two LDS slots (NP 16-byte
// pieces per row, one chunk ahead) and loads its A operands six K-steps ahead
// from the staged x; the four waves' tiles are summed in LDS at the end.
// TT: 32-token tiles per workgroup (as for Q4_K)
template <class D, int TT>
__device__ __forceinline__ void hl_body(const uint8_t *__restrict__ W, const uint8_t *__restrict__ xs,
                                        const int *__restrict__ pe, float *__restrict__ y,
                                        int64_t k, int64_t n, int64_t m, int64_t row_bytes,
                                        int64_t j_start, int64_t j_end, int accumulate) {
    constexpr int RS = 16 * D::NP;         // bytes of a row in a slot
    constexpr int HSLOT = TN * RS + 16;    // one chunk of the tile's rows (+ slack)
    __shared__ __attribute__((aligned(16))) uint8_t slot0[KW][HSLOT];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[KW][HSLOT];
    static_assert((size_t)(KW / 2) * TM * TN * sizeof(float) <= (size_t)KW * HSLOT,
                  "the partial tiles of half the waves fit in one slot array");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 31, kh = lane >> 5;
    const int64_t r0 = j_start + (int64_t)blockIdx.x * TN;
    const int64_t T = blockIdx.y;
    constexpr int NJ = D::CK / 16; // K-steps per chunk (a multiple of RING)
    static_assert(NJ % RING == 0 && NJ > PF, "operand ring indices fixed per chunk");
    const int nch = (int)(k / D::CK);
    const int rows = (int)(j_end - r0 < TN ? j_end - r0 : TN);

    // The tile's bytes from the 16-byte granule holding row r0's start to the
    // end of the granule holding its last byte (W is 16-byte aligned, so that
    // granule lies in the same page; the range check works on whole dwords);
    // rows past the tile's end are out of the descriptor's range and stage
    // zeros.
    const int64_t a0 = r0 * row_bytes, base = a0 & ~(int64_t)15;
    const int lead = (int)(a0 - base);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + base), (short)0, (lead + (int)(rows * row_bytes) + 15) & ~15, 0x00020000);
    const __amdgpu_buffer_rsrc_t rnull =
        __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, 0, 0x00020000);
    // piece p = 64*i + lane of a chunk is piece p % NP of row p / NP; the row's
    // chunk starts at rowoff + D::CB * c bytes past the descriptor base
    int prow[D::NP], rowoff[D::NP];
#pragma unroll
    for (int i = 0; i < D::NP; i++) {
        const int p = 64 * i + lane, r = p / D::NP;
        prow[i] = p - D::NP * r;
        rowoff[i] = lead + r * (int)row_bytes;
    }
    auto copy_chunk = [&](int c, uint8_t *dst) {
        const bool ok = c >= 0;
#pragma unroll
        for (int i = 0; i < D::NP; i++) {
            const int o = rowoff[i] + (ok ? D::CB * c : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ok ? rs : rnull, (__attribute__((address_space(3))) void *)(dst + 1024 * i), 16,
                (o & ~15) + 16 * prow[i], 0, 0, 2 /* nontemporal */);
        }
    };
    // in-piece offset of this lane's two rows' chunk c
    const int rb0 = lead + nl * (int)row_bytes, rb1 = rb0 + 32 * (int)row_bytes;

    f32x16 acc[TT][2];
#pragma unroll
    for (int a = 0; a < TT; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) acc[a][b] = f32x16{};

    // staged x: 4 KB per K-step (both token tiles, hi and lo), K-steps in
    // order; with TT = 1 only the first 2 KB of each are read
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xs + (size_t)T * (k >> 4) * 4096), (short)0, (int)((k >> 4) * 4096), 0x00020000);
    u32x4 ring[RING][TT][2];
    auto load_a = [&](int c, int j, int bi) {
        const bool ok = c >= 0;
#pragma unroll
        for (int a = 0; a < 2 * TT; a++)
            ring[bi][a >> 1][a & 1] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           ok ? xr : rnull, lane * 16, ok ? (c * NJ + j) * 4096 + 1024 * a : 0, 0));
    };
    {
        const int c0 = wave < nch ? wave : -1;
        copy_chunk(c0, slot0[wave]);
#pragma unroll
        for (int j = 0; j < PF; j++) load_a(c0, j, j);
    }
    auto chunk = [&](int c, const uint8_t *cur_slot, uint8_t *nxt) {
        // this chunk's bytes have landed once at most the 2*TT*PF operand
        // loads issued after its copy are outstanding (loads complete in order)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * TT * PF) : "memory");
        const int cn = c + KW < nch ? c + KW : -1;
        copy_chunk(cn, nxt);
        const uint8_t *rowp[2] = {cur_slot + nl * RS, cur_slot + (nl + 32) * RS};
        const int mm[2] = {D::SHIFTED ? (rb0 + D::CB * c) & 15 : 0,
                           D::SHIFTED ? (rb1 + D::CB * c) & 15 : 0};
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int cur = j % RING;
            if (j + PF < NJ)
                load_a(c, j + PF, (j + PF) % RING);
            else
                load_a(cn, j + PF - NJ, (j + PF) % RING);
            __builtin_amdgcn_sched_barrier(0x0386); // VALU, SALU and LDS may cross
            uint32_t bh[2][4], bl[2][4];
#pragma unroll
            for (int rt = 0; rt < 2; rt++) D::dec(rowp[rt], mm[rt], j, kh, bh[rt], bl[rt]);
            // A_hi*B_hi for the four tiles, then A_lo*B_hi, then A_hi*B_lo: no
            // accumulator is reused back to back
#pragma unroll
            for (int term = 0; term < (D::LO ? 3 : 2); term++)
#pragma unroll
                for (int tt = 0; tt < TT; tt++)
#pragma unroll
                    for (int rt = 0; rt < 2; rt++) {
                        const u32x4 av = ring[cur][tt][term == 1 ? 1 : 0];
                        const uint32_t *bv = term == 2 ? bl[rt] : bh[rt];
                        const u32x4 b4 = {bv[0], bv[1], bv[2], bv[3]};
                        if constexpr (D::BF)
                            acc[tt][rt] = mfma_bf(av, b4, acc[tt][rt]);
                        else
                            acc[tt][rt] = mfma(__builtin_bit_cast(f16x8, av),
                                               __builtin_bit_cast(f16x8, b4), acc[tt][rt]);
                    }
        }
    };
    int c = wave;
    for (; c + KW < nch; c += 2 * KW) {
        chunk(c, slot0[wave], slot1[wave]);
        chunk(c + KW, slot1[wave], slot0[wave]);
    }
    if (c < nch) chunk(c, slot0[wave], slot1[wave]);

    // Sum the four waves' tiles in wave order, scale by p, store.
    __syncthreads();
    float *red0 = (float *)&slot0[0][0], *red1 = (float *)&slot1[0][0];
    float *mine = (wave < KW / 2 ? red0 : red1) + (size_t)(wave % (KW / 2)) * TM * TN;
#pragma unroll
    for (int tt = 0; tt < TT; tt++)
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                mine[((tt * 2 + rt) * 16 + r) * 64 + lane] = acc[tt][rt][r];
    // (with TT = 1 the second half's slots hold nothing: no token there is stored)
    __syncthreads();
    tile_store(red0, red1, pe, y, T, n, m, r0, rows, accumulate, tid);
}

#define QMV_MFMA_HL_KERNEL(NAME, D)                                                              \
    template <int TT>                                                                            \
    __global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void NAME(    \
        const uint8_t *__restrict__ W, const uint8_t *__restrict__ xs,                           \
        const int *__restrict__ pe, float *__restrict__ y, int64_t k, int64_t n, int64_t m,      \
        int64_t row_bytes, int64_t j_start, int64_t j_end, int accumulate) {                     \
        hl_body<D, TT>(W, xs, pe, y, k, n, m, row_bytes, j_start, j_end, accumulate);            \
    }
QMV_MFMA_HL_KERNEL(qmv_mfma_q4_0, DQ4_0)
QMV_MFMA_HL_KERNEL(qmv_mfma_q5_0, DQ5_0)
QMV_MFMA_HL_KERNEL(qmv_mfma_q8_0, DQ8_0)
QMV_MFMA_HL_KERNEL(qmv_mfma_q6_k, DQ6_K)
QMV_MFMA_HL_KERNEL(qmv_mfma_f16, DHalf<false>)
QMV_MFMA_HL_KERNEL(qmv_mfma_bf16, DHalf<true>)
#undef QMV_MFMA_HL_KERNEL

template <class K>
void launch_hl(K kernel, const MfmaPlan &p, const uint8_t *W, const uint8_t *xs, const int *pe,
               float *y, int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
               int64_t j_end, int accumulate, hipStream_t stream, hipEvent_t stop) {
    launch_stop(kernel, dim3(p.tiles_n, p.tiles_m), dim3(NT), 0, stream, stop, W, xs, pe, y, k, n,
                m, row_bytes, j_start, j_end, accumulate);
}

} // namespace

// 16-byte pieces per row of a chunk in LDS, per format (0: no matrix-core path)
static int mfma_pieces(int fmt) {
    switch (fmt) {
    case FMT_Q4_0: return DQ4_0::NP;
    case FMT_Q5_0: return DQ5_0::NP;
    case FMT_Q8_0: return DQ8_0::NP;
    case FMT_Q6_K: return DQ6_K::NP;
    case FMT_F16:
    case FMT_BF16: return DHalf<false>::NP;
    default: return 0;
    }
}

bool plan_mfma(int fmt, int64_t k, int64_t rows, int64_t m, int num_cu, MfmaPlan *p) {
    if ((fmt != FMT_Q4_K && mfma_pieces(fmt) == 0) || k <= 0 || (k % 256) != 0 || m < 1)
        return false;
    int64_t rb;
    switch (fmt) {
    case FMT_Q4_K: rb = (k / 256) * 144; break;
    case FMT_Q6_K: rb = (k / 256) * 210; break;
    case FMT_Q4_0: rb = (k / 32) * 18; break;
    case FMT_Q5_0: rb = (k / 32) * 22; break;
    case FMT_Q8_0: rb = (k / 32) * 34; break;
    default: rb = 2 * k; break;
    }
    // the weight copy addresses a 64-row tile (plus 16 bytes) with 32-bit offsets
    if (rb * TN + 16 >= ((int64_t)1 << 31)) return false;
    // and a token tile's staged x (64 KB per 256 weights) too
    if ((k / 256) * 65536 >= ((int64_t)1 << 31)) return false;
    if (p) {
        p->fmt = fmt;
        p->tiles_n = (int)((rows + TN - 1) / TN);
        p->tiles_m = (int)((m + TM - 1) / TM);
        p->grid = p->tiles_n * p->tiles_m;
        p->lds_bytes = fmt == FMT_Q4_K ? (size_t)2 * KW * SLOT
                                       : (size_t)2 * KW * (TN * 16 * mfma_pieces(fmt) + 16);
        (void)num_cu;
    }
    return true;
}

size_t mfma_scratch_bytes(const MfmaPlan &p, int64_t k) {
    const int64_t nsb = k / 256;
    return xs_bytes(p.tiles_m, nsb) + sm_bytes(p.tiles_m, nsb) + pe_bytes(p.tiles_m);
}

hipError_t launch_mfma_ws(const MfmaPlan &p, const uint8_t *W, const float *x, float *y,
                          int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                          int64_t j_end, int accumulate, void *scratch, hipStream_t stream,
                          hipEvent_t stop) {
    const int64_t nsb = k / 256;
    if (p.tiles_m > 65535 || (int64_t)p.tiles_m * TM > 0x7fffffff) return hipErrorInvalidConfiguration;
    uint8_t *xs = (uint8_t *)scratch, *sm = xs + xs_bytes(p.tiles_m, nsb);
    int *pe = (int *)(sm + sm_bytes(p.tiles_m, nsb));
    const dim3 pg((unsigned)((nsb + 1) / 2), (unsigned)(p.tiles_m * TM));
    if (p.fmt == FMT_BF16)
        hipLaunchKernelGGL(qmv_mfma_prep_x<true>, pg, dim3(64), 0, stream, x, k, m, xs, sm, pe);
    else
        hipLaunchKernelGGL(qmv_mfma_prep_x<false>, pg, dim3(64), 0, stream, x, k, m, xs, sm, pe);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one 32-token tile per workgroup when the call has at most 32 tokens
    const bool one = m <= TM / 2;
    switch (p.fmt) {
    case FMT_Q4_K:
        if (one)
            launch_stop(qmv_mfma_q4_k<1>, dim3(p.tiles_n, p.tiles_m), dim3(NT), 0, stream, stop, W,
                        xs, sm, pe, y, k, n, m, row_bytes, j_start, j_end, accumulate);
        else
            launch_stop(qmv_mfma_q4_k<2>, dim3(p.tiles_n, p.tiles_m), dim3(NT), 0, stream, stop, W,
                        xs, sm, pe, y, k, n, m, row_bytes, j_start, j_end, accumulate);
        break;
#define QMV_HL(K)                                                                                \
    (one ? launch_hl(K<1>, p, W, xs, pe, y, k, n, m, row_bytes, j_start, j_end, accumulate,       \
                     stream, stop)                                                                \
         : launch_hl(K<2>, p, W, xs, pe, y, k, n, m, row_bytes, j_start, j_end, accumulate,       \
                     stream, stop))
    case FMT_Q4_0: QMV_HL(qmv_mfma_q4_0); break;
    case FMT_Q5_0: QMV_HL(qmv_mfma_q5_0); break;
    case FMT_Q8_0: QMV_HL(qmv_mfma_q8_0); break;
    case FMT_Q6_K: QMV_HL(qmv_mfma_q6_k); break;
    case FMT_F16: QMV_HL(qmv_mfma_f16); break;
    case FMT_BF16: QMV_HL(qmv_mfma_bf16); break;
#undef QMV_HL
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mfma(const MfmaPlan &p, const uint8_t *W, const float *x, float *y, int64_t k,
                       int64_t n, int64_t m, int64_t row_bytes, int64_t j_start, int64_t j_end,
                       int accumulate, ScratchLender &lender, hipStream_t stream) {
    void *buf = nullptr;
    hipEvent_t done = nullptr;
    hipError_t e = lender.acquire(mfma_scratch_bytes(p, k), stream, &buf, &done);
    if (e != hipSuccess) return e;
    e = launch_mfma_ws(p, W, x, y, k, n, m, row_bytes, j_start, j_end, accumulate, buf, stream,
                       done);
    const hipError_t f = lender.release(buf, stream, e == hipSuccess && done);
    return e != hipSuccess ? e : f;
}

// Fixed scratch for callers that cannot allocate (qmv_run_noalloc): one copy
// in every device's memory, held until the process ends. Host code never
// passes `scratch` itself (its host-side name is no device address): set-up
// looks up each device's copy with hipGetSymbolAddress and the launches take
// that address.
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch_init(int device, void **ptr) {
    *ptr = nullptr;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    e = hipSetDevice(device);
    if (e == hipSuccess) e = hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) *ptr = nullptr;
    const hipError_t r = hipSetDevice(cur);
    return e != hipSuccess ? e : r;
}

const char *mfma_kernel_name(const MfmaPlan &p) {
    switch (p.fmt) {
    case FMT_Q4_K: return "qmv_mfma<q4_k>";
    case FMT_Q4_0: return "qmv_mfma<q4_0>";
    case FMT_Q5_0: return "qmv_mfma<q5_0>";
    case FMT_Q8_0: return "qmv_mfma<q8_0>";
    case FMT_Q6_K: return "qmv_mfma<q6_k>";
    case FMT_F16: return "qmv_mfma<f16>";
    case FMT_BF16: return "qmv_mfma<bf16>";
    default: return "";
    }
}

} // namespace qmv
