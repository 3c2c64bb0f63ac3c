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
//  1. qmv_mfma_prep_x: for every (token, super-block) choose a power of two
//     p = 2^e with max|x|/p in [2^14, 2^15), and write x/p as two f16 terms
//     hi = f16(x/p), lo = f16(x/p - hi) (22 significant bits together; the
//     scaling keeps hi and lo normal for all but negligible values), laid out
//     in the MFMA operand order so that every wave load of the main kernel
//     reads one contiguous KB. It also writes, per token and 32-weight
//     sub-block, the f32 sum of x (fixed order) divided by 32p, split hi/lo, and
//     the table of p. Staging memory comes from the stream's device pool
//     (hipMallocAsync/hipFreeAsync), m*k*4 bytes plus k*m/8 + k*m/64.
//  2. qmv_mfma_q4_k: each super-block's product runs on
//     v_mfma_f32_32x32x16_f16 with B = sc*q, an exact f16 integer (<= 945),
//     against hi and lo; the 16 K-steps of a super-block accumulate in f32 in
//     a fresh tile, then one f32 FMA per output adds d*p*tile. The min term
//     dmin * sum_g m_g * sum(x over g) takes one more MFMA per super-block
//     (A = the hi/lo sums, B = the 6-bit mins, exact), scaled by dmin*p.
//
// Mapping of the main kernel. A workgroup owns 64 tokens x 64 rows and has 8
// waves: wave w takes token half th = w&1 and K quarter kq = w>>1 (super-blocks
// kq, kq+4, ...) and holds its 32 tokens x 64 rows as two 32x32 accumulators
// (lane l feeds A[l%32][8(l/32)+i] and B[8(l/32)+i][l%32] and receives
// D[8(r/4)+4(l/32)+r%4][l%32] in register r). Tokens are the MFMA rows and
// weight rows the columns, so a lane's block scales are scalars. Each quarter
// stages the weight bytes of its super-blocks in LDS (buffer_load ... lds, one
// contiguous run per row), the next super-block's while one is decoded (two
// slots per quarter, each copy split between the quarter's two waves); the
// four quarters' partial tiles are summed in LDS in quarter order. Results
// depend only on k, never on the row range or the token tiling.
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64;      // tokens per tile
constexpr int TN = 64;      // weight rows per tile
constexpr int KQ = 4;       // split of K over the waves of the main kernel
constexpr int NT = 64 * 2 * KQ; // threads per workgroup: 2 token halves x KQ
constexpr int SBB = 144;    // bytes of a Q4_K super-block
constexpr int PF = 3;       // sub-blocks of x operands loaded ahead
constexpr int QUARTER_W = TN * SBB * 2; // a quarter's two staging slots (one super-block each)
constexpr size_t RED_BYTES = (size_t)KQ * TM * TN * sizeof(float); // partial tiles
constexpr size_t LDS_BYTES =
    (size_t)KQ * QUARTER_W > RED_BYTES ? (size_t)KQ * QUARTER_W : RED_BYTES;

// Staging layout, per 64-token tile T and super-block s (NSB = k/256):
//   XS: [T][s][g 8][tp 2][tb 2][hl 2][lane 64] x 16 bytes (8 f16)
//   SM: [T][s][tb 2][lane 64] x 16 bytes (8 f16 sums/(32p): lanes 0-31 hi, 32-63 lo)
//   PS: [T][s][token 64] floats (the power of two p)
// Lane (nl, jh) of (g, tp, tb) holds token 32tb+nl, elements
// 32g + 16jh + 8tp + PERM[i] of the super-block: the order in which the code
// decoder below produces its f16 pairs.
constexpr size_t xs_bytes(int64_t tiles, int64_t nsb) { return (size_t)tiles * nsb * 64 * 1024; }
constexpr size_t sm_bytes(int64_t tiles, int64_t nsb) { return (size_t)tiles * nsb * 2 * 64 * 16; }
constexpr size_t ps_bytes(int64_t tiles, int64_t nsb) { return (size_t)tiles * nsb * 64 * 4; }

__device__ __forceinline__ int perm8(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }

// Staged x is read by every row tile: ordinary cached loads.
__device__ __forceinline__ u32x4 ldc(const uint8_t *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// ------------------------------------------------------------ x staging

// One wave per (4-token group of a 64-token tile, super-block): grid
// (k/256, tiles, 16), 64 threads.
__global__ __launch_bounds__(64) void qmv_mfma_prep_x(const float *__restrict__ x, int64_t k,
                                                      int64_t m, uint8_t *__restrict__ xs,
                                                      uint8_t *__restrict__ sm,
                                                      float *__restrict__ ps) {
    __shared__ int e_tok[4];
    __shared__ float s_tok[4][8];
    __shared__ f32x4 xv[4][64]; // the group's x slice, read once from memory
    const int lane = threadIdx.x;
    const int s = blockIdx.x, T = blockIdx.y, qg = blockIdx.z; // tokens 4qg..4qg+3 of T
    const int64_t nsb = k >> 8;
    const int64_t ts = (int64_t)T * nsb + s; // (tile, super-block) index

    // Phase 1: per token, the exponent and the eight sub-block sums; lane l
    // takes elements 4l..4l+3 of each of the 4 tokens.
    float v[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t t = (int64_t)T * TM + 4 * qg + i;
#pragma unroll
        for (int j = 0; j < 4; j++)
            v[i][j] = t < m ? x[t * k + 256 * (int64_t)s + 4 * lane + j] : 0.f;
        xv[i][lane] = f32x4{v[i][0], v[i][1], v[i][2], v[i][3]};
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float mx = fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])),
                         fmaxf(fabsf(v[i][2]), fabsf(v[i][3])));
        float sum = (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
        // sub-block g = lane / 8: sum over 8 lanes in a fixed pattern
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) sum += __shfl_xor(sum, o, 64);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if (lane == 0) {
            int e = 0;
            if (mx > 0.f) {
                (void)frexpf(mx, &e); // mx = f * 2^e, f in [0.5, 1)
                e -= 15;              // mx / 2^e in [2^14, 2^15)
                e = e < -100 ? -100 : (e > 100 ? 100 : e);
            }
            e_tok[i] = e;
        }
        if ((lane & 7) == 0) s_tok[i][lane >> 3] = sum;
    }
    __syncthreads();

    // Phase 2: the operand pieces of the group's tokens: piece (g, tp, jh,
    // token) gives the hi and lo 16-byte pieces of that slot. Token tt of the
    // tile sits in MFMA row nl = tt % 32 of token half tb = tt / 32.
    uint8_t *xt = xs + ts * 64 * 1024;
#pragma unroll
    for (int it = 0; it < 2; it++) {
        const int pc = lane + 64 * it;
        const int lq = pc & 3, jh = (pc >> 2) & 1, tp = (pc >> 3) & 1, g = pc >> 4;
        const int tt = 4 * qg + lq, tb = tt >> 5, ln = (tt & 31) + 32 * jh;
        float w[8];
        {
            const float *p = (const float *)&xv[lq][0] + 32 * g + 16 * jh + 8 * tp;
#pragma unroll
            for (int j = 0; j < 8; j++) w[j] = ldexpf(p[perm8(j)], -e_tok[lq]);
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const _Float16 h0 = (_Float16)w[2 * j], h1 = (_Float16)w[2 * j + 1];
            hi[j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
            lo[j] = pk_f16(w[2 * j] - (float)h0, w[2 * j + 1] - (float)h1);
        }
        const size_t base = ((((size_t)g * 2 + tp) * 2 + tb) * 2) * 1024 + (size_t)ln * 16;
        *(u32x4 *)(xt + base) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *(u32x4 *)(xt + base + 1024) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
    // Sums for the min term and the table of p.
    if (lane < 8) {
        const int lq = lane & 3, jh = lane >> 2;
        const int tt = 4 * qg + lq, tb = tt >> 5, ln = (tt & 31) + 32 * jh;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            float a2[2];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                // a sum of 32 values below 2^15 can reach 2^20: scale by 2^-5 more
                const float sv = ldexpf(s_tok[lq][2 * j + q], -e_tok[lq] - 5);
                const float h = (float)(_Float16)sv;
                a2[q] = jh ? sv - h : h;
            }
            o[j] = pk_f16(a2[0], a2[1]);
        }
        *(u32x4 *)(sm + (ts * 2 + tb) * 64 * 16 + (size_t)ln * 16) = u32x4{o[0], o[1], o[2], o[3]};
    } else if (lane < 12) {
        const int tq = lane - 8;
        ps[ts * TM + 4 * qg + tq] = ldexpf(1.f, e_tok[tq]);
    }
}

// ------------------------------------------------------------ main kernel

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Byte i (0..11) of the packed scale/min field of a Q4_K header.
__device__ __forceinline__ uint32_t scb(const u32x4 &h, int i) {
    return (h[1 + (i >> 2)] >> (8 * (i & 3))) & 0xffu;
}

// s_waitcnt operand: vmcnt 0, expcnt and lgkmcnt left free (gfx9 encoding).
constexpr int WAIT_VM0 = 0x0f70;

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
struct CodeMasks {
    uint32_t lo, hi; // 0x000f000f, 0x00f000f0 (opaque)
};
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t mask, f16x2 sc, f16x2 off) {
    const uint32_t mag = (w & mask) | (0x64006400u & ~mask); // one v_bfi_b32
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_fma(__builtin_bit_cast(f16x2, mag), sc, off));
}
// B operand of K-step tp of sub-block 2c+h from the lane's 16 code bytes of
// chunk c: slots in perm8 order.
__device__ __forceinline__ f16x8 codes_b(const u32x4 &q, int tp, uint32_t mask, f16x2 sc,
                                         f16x2 off) {
    const uint32_t w0 = q[2 * tp], w1 = q[2 * tp + 1];
    const uint32_t r0 = __builtin_amdgcn_alignbyte(w0, w0, 1);
    const uint32_t r1 = __builtin_amdgcn_alignbyte(w1, w1, 1);
    const u32x4 r = {code_pair(w0, mask, sc, off), code_pair(r0, mask, sc, off),
                     code_pair(w1, mask, sc, off), code_pair(r1, mask, sc, off)};
    return __builtin_bit_cast(f16x8, r);
}

// Main kernel: 8 waves per workgroup; wave w takes token half th = w&1 of
// the 64-token tile and K quarter kq = w>>1 (super-blocks kq, kq+4, ...).
// The two waves of a quarter share its staged weight bytes.
__global__ __launch_bounds__(NT) void qmv_mfma_q4_k(const uint8_t *__restrict__ W,
                                                    const uint8_t *__restrict__ xs,
                                                    const uint8_t *__restrict__ sm,
                                                    const float *__restrict__ ps,
                                                    float *__restrict__ y, int64_t k, int64_t n,
                                                    int64_t m, int64_t row_bytes,
                                                    int64_t j_start, int64_t j_end,
                                                    int accumulate) {
    // LDS: during the K loop, per quarter the staged super-blocks of its
    // round; afterwards the [KQ][TM][TN] partial tiles.
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float *red = (float *)lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int th = wave & 1, kq = wave >> 1;
    const int nl = lane & 31, jh = lane >> 5;
    const int64_t r0 = j_start + (int64_t)blockIdx.x * TN;
    const int T = blockIdx.y;
    const int64_t t0 = (int64_t)T * TM;
    const int nsb = (int)(k >> 8);
    const int rows = (int)(j_end - r0 < TN ? j_end - r0 : TN); // live rows of the tile
    uint8_t *wl = lds + kq * QUARTER_W;
    const CodeMasks cm = {opaque(0x000f000fu), opaque(0x00f000f0u)};

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

    f32x16 acc[2];
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[b][r] = 0.f;

    // super-blocks of this quarter (nw); every wave runs nmax iterations. The
    // quarter's next super-block is copied into its other slot while one is
    // decoded; the two waves of the quarter split each copy.
    const int nw = kq < nsb ? (nsb - kq + KQ - 1) / KQ : 0;
    const int nmax = (nsb + KQ - 1) / KQ;
    auto copy_sb = [&](int i, int slot) {
        const int sboff = SBB * (kq + KQ * i);
        for (int c = th; c < 9; c += 2) {
            uint8_t *dst = wl + slot * (TN * SBB) + 1024 * c;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)dst, 16, poff[c] + sboff, 0, 0,
                2 /* nontemporal */);
        }
    };
    if (nw > 0) copy_sb(0, 0);
    f16x8 ring[4][4]; // x operands of four sub-blocks: [sub-block & 3][2*tp + hl]
    for (int i = 0; i < nmax; i++) {
        __builtin_amdgcn_s_waitcnt(WAIT_VM0); // this wave's part of super-block i has landed
        __syncthreads(); // and the partner's; the other slot's super-block is read
        if (i + 1 < nw) copy_sb(i + 1, (i + 1) & 1);
        if (i == 0 && nw > 0) {
            // first PF sub-blocks of the wave's first super-block
            const uint8_t *xf0 = xs + ((int64_t)T * nsb + kq) * 64 * 1024 + lane * 16;
#pragma unroll
            for (int g = 0; g < PF; g++)
#pragma unroll
                for (int f = 0; f < 4; f++)
                    ring[g][f] = __builtin_bit_cast(
                        f16x8, ldc(xf0 + ((8 * g + 4 * (f >> 1) + 2 * th + (f & 1)) << 10)));
        }
        if (i < nw) {
            const int s = kq + KQ * i;
            const int64_t ts = (int64_t)T * nsb + s;
            const uint8_t *xf = xs + ts * 64 * 1024 + lane * 16 + (2 * th << 10);
            const uint8_t *xfn =
                i + 1 < nw ? xf + (int64_t)KQ * 64 * 1024 : xf; // next super-block
            const uint8_t *wsb = wl + (i & 1) * (TN * SBB);
            const uint8_t *wrow[2] = {wsb + nl * SBB, wsb + (nl + 32) * SBB};

            // block scales of the lane's two rows
            float dd[2], dm[2];
            uint32_t scg[2][8];
            f16x8 mins[2];
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const u32x4 hd = *(const u32x4 *)wrow[rb];
                dd[rb] = h2f(hd[0]);
                dm[rb] = h2f(hd[0] >> 16);
#pragma unroll
                for (int g = 0; g < 8; g++) {
                    uint32_t sc, mn;
                    if (g < 4) {
                        sc = scb(hd, g) & 63u;
                        mn = scb(hd, g + 4) & 63u;
                    } else {
                        sc = (scb(hd, g + 4) & 15u) | ((scb(hd, g - 4) >> 6) << 4);
                        mn = (scb(hd, g + 4) >> 4) | ((scb(hd, g) >> 6) << 4);
                    }
                    scg[rb][g] = sc;
                    mins[rb][g] = (_Float16)(float)mn;
                }
            }

            f32x16 tile[2];
#pragma unroll
            for (int b = 0; b < 2; b++)
#pragma unroll
                for (int e = 0; e < 16; e++) tile[b][e] = 0.f;
            // A operands: fragment (g, tp, tb, hl) at KB 8g + 4tp + 2tb + hl. A
            // ring of four sub-blocks keeps the loads PF sub-blocks ahead,
            // running into the wave's next super-block.
#pragma unroll
            for (int g = 0; g < 8; g++) {
                const int c = g >> 1, h = g & 1, cb = g & 3;
                {
                    const int gn = g + PF, nb = gn & 3;
                    const uint8_t *src = gn < 8 ? xf + ((8 * gn) << 10) : xfn + ((8 * (gn - 8)) << 10);
#pragma unroll
                    for (int f = 0; f < 4; f++)
                        ring[nb][f] = __builtin_bit_cast(
                            f16x8, ldc(src + ((4 * (f >> 1) + (f & 1)) << 10)));
                }
#pragma unroll
                for (int rb = 0; rb < 2; rb++) {
                    const u32x4 q = *(const u32x4 *)(wrow[rb] + 16 + 32 * c + 16 * jh);
                    const float scf = (float)scg[rb][g];
                    const _Float16 sch = (_Float16)(h ? scf * 0.0625f : scf);
                    const _Float16 off = (_Float16)(h ? -64.f * scf : -1024.f * scf);
                    const f16x2 sc2 = {sch, sch}, off2 = {off, off};
                    const uint32_t mask = h ? cm.hi : cm.lo;
#pragma unroll
                    for (int tp = 0; tp < 2; tp++) {
                        const f16x8 b = codes_b(q, tp, mask, sc2, off2);
                        tile[rb] = mfma(ring[cb][2 * tp], b, tile[rb]);
                        tile[rb] = mfma(ring[cb][2 * tp + 1], b, tile[rb]);
                    }
                }
                // keep the loads ahead of this sub-block's work
                __builtin_amdgcn_sched_barrier(0);
            }
            // y += d*p*tile - 32*dmin*p*(sum_g m_g * sum_g(x)/32), p per token (D row)
            const f16x8 am = __builtin_bit_cast(
                f16x8, ldc(sm + (ts * 2 + th) * 64 * 16 + (size_t)lane * 16));
            f32x4 pv[4];
#pragma unroll
            for (int qd = 0; qd < 4; qd++)
                pv[qd] = *(const f32x4 *)(ps + ts * TM + 32 * th + 8 * qd + 4 * jh);
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const f32x16 mt = mfma(am, mins[rb], f32x16{});
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const float p = pv[e >> 2][e & 3];
                    acc[rb][e] = fmaf(dd[rb] * p, tile[rb][e], acc[rb][e]);
                    acc[rb][e] = fmaf(-32.f * dm[rb] * p, mt[e], acc[rb][e]);
                }
            }
        }
    }

    // Sum the partial tiles of the quarters in order, then store.
    __syncthreads(); // every wave is done with the staged weights
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int mm = 32 * th + 8 * (r >> 2) + 4 * jh + (r & 3);
            red[(kq * TM + mm) * TN + 32 * rb + nl] = acc[rb][r];
        }
    __syncthreads();
    for (int i = tid; i < TM * TN; i += NT) {
        float v = red[i];
#pragma unroll
        for (int q = 1; q < KQ; q++) v += red[q * TM * TN + i];
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
    // the staging copy addresses a 64-row tile with 32-bit offsets
    if ((k / 256) * SBB * TN >= ((int64_t)1 << 31)) return false;
    if (p) {
        p->fmt = fmt;
        p->tiles_n = (int)((rows + TN - 1) / TN);
        p->tiles_m = (int)((m + TM - 1) / TM);
        p->grid = p->tiles_n * p->tiles_m;
        p->lds_bytes = LDS_BYTES;
        (void)num_cu;
    }
    return true;
}

hipError_t launch_mfma(const MfmaPlan &p, const uint8_t *W, const float *x, float *y, int64_t k,
                       int64_t n, int64_t m, int64_t row_bytes, int64_t j_start, int64_t j_end,
                       int accumulate, hipStream_t stream) {
    if (p.fmt != FMT_Q4_K) return hipErrorInvalidValue;
    const int64_t nsb = k / 256;
    if (p.tiles_m > 65535 || nsb > 0x7fffffff) return hipErrorInvalidConfiguration;
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)qmv_mfma_q4_k,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const size_t bx = xs_bytes(p.tiles_m, nsb), bs = sm_bytes(p.tiles_m, nsb),
                 bp = ps_bytes(p.tiles_m, nsb);
    void *buf = nullptr;
    hipError_t e = hipMallocAsync(&buf, bx + bs + bp, stream);
    if (e != hipSuccess) return e;
    uint8_t *xs = (uint8_t *)buf, *sm = xs + bx;
    float *ps = (float *)(sm + bs);
    hipLaunchKernelGGL(qmv_mfma_prep_x, dim3((unsigned)nsb, p.tiles_m, TM / 4), dim3(64), 0, stream,
                       x, k, m, xs, sm, ps);
    e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(qmv_mfma_q4_k, dim3(p.tiles_n, p.tiles_m), dim3(NT), LDS_BYTES,
                           stream, W, xs, sm, ps, y, k, n, m, row_bytes, j_start, j_end,
                           accumulate);
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(buf, stream);
    return e != hipSuccess ? e : f;
}

const char *mfma_kernel_name(const MfmaPlan &p) {
    return p.fmt == FMT_Q4_K ? "qmv_mfma<q4_k>" : "";
}

} // namespace qmv
