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
        const _Float16 h0 = (_Float16)w[2 * i], h1 = (_Float16)w[2 * i + 1];
        hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lo[i] = pk_f16(w[2 * i] - (float)h0, w[2 * i + 1] - (float)h1);
    }
    const int j = 2 * g + j2;
    uint8_t *dst = xs + ((size_t)((T * nsb + s) * 16 + j) * 4 + tt * 2) * 1024 +
                   (size_t)(ln + 32 * kh) * 16;
    *(u32x4 *)dst = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4 *)(dst + 1024) = u32x4{lo[0], lo[1], lo[2], lo[3]};
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

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
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
    f16x8 ring[RING][2][2];
    auto load_a = [&](int s, int j, int bi) {
        const bool ok = s >= 0;
#pragma unroll
        for (int a = 0; a < 4; a++)
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
        // this super-block's bytes have landed once at most the 4*PF operand
        // loads issued after its copy are outstanding (loads complete in order)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PF) : "memory");
        const int sn = s + KW < nsb ? s + KW : -1;
        copy_sb(sn, nxt);
        // the sub-block sums of x for the min term, needed at the end
        f16x8 am[2];
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
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
        f32x16 tile[2][2];
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
                    for (int tt = 0; tt < 2; tt++)
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
        for (int tt = 0; tt < 2; tt++) {
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
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                mine[((tt * 2 + rt) * 16 + r) * 64 + lane] = acc[tt][rt][r];
    __syncthreads();
    // Thread tid takes outputs o = tid + 256 i; the 16 exponents (every padded
    // token has one) and, when accumulating, the old values are all loaded
    // before any store.
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

} // namespace

bool plan_mfma(int fmt, int64_t k, int64_t rows, int64_t m, int num_cu, MfmaPlan *p) {
    if (fmt != FMT_Q4_K || k <= 0 || (k % 256) != 0 || m < 1) return false;
    // the staging copy addresses a 64-row tile with 32-bit offsets
    if ((k / 256) * SBB * TN >= ((int64_t)1 << 31)) return false;
    // and a token tile's staged x (64 KB per super-block) with 32-bit offsets
    if ((k / 256) * 65536 >= ((int64_t)1 << 31)) return false;
    if (p) {
        p->fmt = fmt;
        p->tiles_n = (int)((rows + TN - 1) / TN);
        p->tiles_m = (int)((m + TM - 1) / TM);
        p->grid = p->tiles_n * p->tiles_m;
        p->lds_bytes = (size_t)2 * KW * SLOT;
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
                          int64_t j_end, int accumulate, void *scratch, hipStream_t stream) {
    if (p.fmt != FMT_Q4_K) return hipErrorInvalidValue;
    const int64_t nsb = k / 256;
    if (p.tiles_m > 65535 || (int64_t)p.tiles_m * TM > 0x7fffffff) return hipErrorInvalidConfiguration;
    uint8_t *xs = (uint8_t *)scratch, *sm = xs + xs_bytes(p.tiles_m, nsb);
    int *pe = (int *)(sm + sm_bytes(p.tiles_m, nsb));
    hipLaunchKernelGGL(qmv_mfma_prep_x, dim3((unsigned)((nsb + 1) / 2), (unsigned)(p.tiles_m * TM)),
                       dim3(64), 0, stream, x, k, m, xs, sm, pe);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(qmv_mfma_q4_k, dim3(p.tiles_n, p.tiles_m), dim3(NT), 0, stream, W,
                       xs, sm, pe, y, k, n, m, row_bytes, j_start, j_end, accumulate);
    return hipGetLastError();
}

hipError_t launch_mfma(const MfmaPlan &p, const uint8_t *W, const float *x, float *y, int64_t k,
                       int64_t n, int64_t m, int64_t row_bytes, int64_t j_start, int64_t j_end,
                       int accumulate, hipStream_t stream) {
    void *buf = nullptr;
    hipError_t e = hipMallocAsync(&buf, mfma_scratch_bytes(p, k), stream);
    if (e != hipSuccess) return e;
    e = launch_mfma_ws(p, W, x, y, k, n, m, row_bytes, j_start, j_end, accumulate, buf, stream);
    const hipError_t f = hipFreeAsync(buf, stream);
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
    return p.fmt == FMT_Q4_K ? "qmv_mfma<q4_k>" : "";
}

} // namespace qmv
