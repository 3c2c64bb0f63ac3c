// Streaming block-quantized GEMV for gfx950: y[t][j] (=|+=) sum_i x[t][i] * w_j[i].
//
// Operation: rullama 0.5.0, src/backend/matmul.rs (module doc: weight bytes as
// stored in GGUF, y = x @ W; the test helper cpu_matmul_f32 fixes W as n rows
// of k weights). Row range and accumulate: src/backend/dispatch/mod.rs, struct
// MatmulBackInputParams (applied here to output rows).
//
// Mapping. A row of k weights is cut into U = k/64 "units" of 64 weights. A
// workgroup holds P row slots of L lanes; lane l of a slot owns units l,
// l+L, ... (UPL of them) for the whole launch, and keeps the x of each owned
// unit in registers: for F16/BF16 the 64 values, loaded once at kernel start
// from a transposed copy of x in LDS (conflict-free); for the block formats
// the unit's exponent and three signed 8-bit digit planes, computed once per
// workgroup straight from x in global memory and shared through LDS. The
// workgroup then processes batches of P*RB consecutive rows (slot s takes rows
// base+s, base+s+P, ...). Per-lane partial sums of a row are reduced with DPP
// inside aligned groups of G lanes; the L/G group sums of each row go through
// LDS. Every row's arithmetic and reduction order depend only on k, never on
// the row range, so any tiling of the rows gives bit-identical outputs.
//
// Weight streaming. Wave loads must cover whole, contiguous cache lines: a
// load instruction whose 64 lanes touch scattered 16-byte pieces costs the L1
// one tag lookup per line piece and multiplies the L1->L2 requests.
//  * F16/BF16 rows are plain arrays: each lane loads eight 16-byte chunks at a
//    stride of U chunks, so every load instruction reads one contiguous span
//    ("direct" kernel).
//  * Block formats (Q4_0, Q4_K, Q6_K, Q8_0, Q5_0) interleave fields of odd
//    sizes. There each batch's rows, one contiguous byte range, are copied
//    straight from memory into a double-buffered LDS area (buffer_load ...
//    lds, one contiguous kilobyte per wave instruction; batches 0 and 1 at
//    the start, then one batch ahead), from which lanes read their unit's
//    fields ("staged" kernel). One LDS-only barrier per batch covers the
//    buffer swap and the cross-group reduction.
//
// Decode. Block formats multiply integer codes (signed bytes holding a
// multiple of q-8, q-16 or q-32 for Q4_0, Q5_0, Q6_K; Q8_0 codes as they are;
// Q4_K nibbles) with the digit planes by v_dot4_i32_i8, apply group scales to
// the three plane sums by 24-bit integer multiply-adds and combine the planes
// in f32 once per unit; the Q4_K min term is applied in factored form,
// dmin*m*sum(x). F16 weights go through v_fma_mix_f32; BF16 is a shift/mask
// into f32.
#include "qmv_internal.h"
#include "qmv_units.h"

#include <map>
#include <mutex>
#include <utility>

namespace qmv {

// Sum over aligned groups of G lanes (G a power of two <= 16); every lane of
// a group ends with the group sum. Order of additions is fixed.
__device__ __forceinline__ float group_sum(float v, int G) {
    if (G >= 2) v += dpp_mov<0xb1>(v);  // quad_perm [1,0,3,2]
    if (G >= 4) v += dpp_mov<0x4e>(v);  // quad_perm [2,3,0,1]
    if (G >= 8) v += dpp_mov<0x141>(v); // row_half_mirror
    if (G >= 16) v += dpp_mov<0x140>(v); // row_mirror
    return v;
}

// x, first part: coalesced float4 loads into registers (4 per thread; the
// index is clamped so the loads are unconditional and their count is known).
__device__ __forceinline__ void x_prefetch(const float *x, int nt4, int tid, int T,
                                           f32x4 xa[4]) {
    const f32x4 *x4 = (const f32x4 *)x;
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const int q = tid + s * T;
        xa[s] = x4[q < nt4 ? q : nt4 - 1];
    }
}

// x into LDS, transposed so that piece i of unit u of token t sits at
// [t*n4 + i*U + u]: the per-lane reads are then consecutive across lanes. With
// UNITS the pieces of a unit sit together instead, at [t*n4 + 16u + i] (read
// one piece per lane by the shared integer-plane pass).
template <class F, bool UNITS = false>
__device__ __forceinline__ void x_to_lds(const float *x, f32x4 *xl, int n4, int nt4, int U,
                                         int tid, int T, const f32x4 xa[4]) {
    auto put = [&](int q, f32x4 v) {
        const int t = q / n4, r = q - t * n4;
        int u, i;
        F::x4_slot(r, U, u, i);
        xl[t * n4 + (UNITS ? 16 * u + i : i * U + u)] = v;
    };
#pragma unroll
    for (int s = 0; s < 4; s++)
        if (tid + s * T < nt4) put(tid + s * T, xa[s]);
    const f32x4 *x4 = (const f32x4 *)x;
    for (int q = tid + 4 * T; q < nt4; q += T) put(q, x4[q]);
}

template <class F, int MT, int UPL>
__device__ __forceinline__ void x_units_from_lds(typename F::X (&xu)[MT][UPL], const f32x4 *xl,
                                                 int n4, int U, const int (&ulod)[UPL]) {
#pragma unroll
    for (int i = 0; i < UPL; i++)
#pragma unroll
        for (int t = 0; t < MT; t++) {
#pragma unroll
            for (int p = 0; p < 16; p++) F::put_x(xu[t][i], p, xl[t * n4 + p * U + ulod[i]]);
            F::finish_x(xu[t][i]);
        }
}

// Integer-plane units: every lane's unit from the workgroup's shared records
// and planes in LDS.
template <class F, int MT, int UPL>
__device__ __forceinline__ void x_units_from_planes(typename F::X (&xu)[MT][UPL], const XRec *rec,
                                                    const uint32_t *pl, int U,
                                                    const int (&ulod)[UPL]) {
#pragma unroll
    for (int i = 0; i < UPL; i++)
#pragma unroll
        for (int t = 0; t < MT; t++) {
            x_from_planes(xu[t][i], rec, pl, t, ulod[i], U);
            F::finish_shared(xu[t][i]);
        }
}

// x straight from global memory, one float at a time (any 4-byte alignment).
template <class F, int MT, int UPL>
__device__ __forceinline__ void x_units_from_global(typename F::X (&xu)[MT][UPL],
                                                    const float *x, int64_t k, int U,
                                                    const int (&ulod)[UPL]) {
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

// Outputs of a batch are numbered q = (slot*RB + r)*MT + t (row base + r*P +
// slot, token t). With accumulate, the old values of y are read one batch
// ahead, together with that batch's weights, and parked in LDS (ybuf): a
// global read issued later than the weight prefetch would make the in-order
// load counter drain that prefetch.
template <int MT, int RB>
struct YPrefetch {
    float v[2];
    __device__ __forceinline__ void fetch(const float *y, int64_t n, int64_t b, int64_t j_end,
                                          int P, int tid, int T) {
        const int nq = P * RB * MT;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            int q = tid + s * T;
            q = q < nq ? q : nq - 1;
            const int t = q % MT, rr = q / MT;
            const int64_t j = b + (int64_t)(rr % RB) * P + rr / RB;
            v[s] = y[t * n + (j < j_end ? j : j_end - 1)];
        }
    }
    __device__ __forceinline__ void stash(float *ybuf, int P, int tid, int T) const {
        const int nq = P * RB * MT;
#pragma unroll
        for (int s = 0; s < 2; s++)
            if (tid + s * T < nq) ybuf[tid + s * T] = v[s];
    }
};

// Store one output (ybuf holds the old values when accumulating).
__device__ __forceinline__ void store_y(float *dst, float v, int accumulate, const float *ybuf,
                                        int q) {
    *dst = accumulate ? ybuf[q] + v : v;
}

// Sum the NG group partials of every (row, token) of a batch and store them.
template <int MT, int RB>
__device__ __forceinline__ void finish_batch(const float *rb, const float *ybuf, int NG, int P,
                                             int tid, int T, int64_t base, int64_t j_end,
                                             float *y, int64_t n, int accumulate) {
    for (int q = tid; q < P * RB * MT; q += T) {
        const int t = q % MT;
        const int rr = q / MT; // slot * RB + r
        const int s = rr / RB, r = rr % RB;
        const int64_t j = base + (int64_t)r * P + s;
        if (j < j_end) {
            // the group sums in order g = 0, 1, ...; the reads of each run of
            // eight are issued together rather than one LDS round trip each
            const float *src = rb + q * NG;
            float v = src[0];
            for (int g0 = 1; g0 < NG; g0 += 8) {
                float c[8];
#pragma unroll
                for (int i = 0; i < 8; i++) c[i] = g0 + i < NG ? src[g0 + i] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if (g0 + i < NG) v += c[i];
            }
            store_y(y + t * n + j, v, accumulate, ybuf, q);
        }
    }
}

// DPP-reduce the batch partials, then either store (one group per row) or
// leave the group sums in LDS for finish_batch.
template <int MT, int RB, int UPL>
__device__ __forceinline__ void reduce_batch(float (&part)[RB][MT], const Lanes<UPL> &ln, int G,
                                             int P, float *rb, const float *ybuf, int64_t base,
                                             int64_t j_end, float *y, int64_t n,
                                             int accumulate) {
#pragma unroll
    for (int r = 0; r < RB; r++)
#pragma unroll
        for (int t = 0; t < MT; t++) part[r][t] = group_sum(part[r][t], G);
    if (ln.slot >= P) return; // lanes past the last row slot (workgroup padding)
    if (ln.NG == 1) {
        if (ln.lane == 0) {
#pragma unroll
            for (int r = 0; r < RB; r++) {
                const int64_t j = base + (int64_t)r * P + ln.slot;
                if (j < j_end) {
#pragma unroll
                    for (int t = 0; t < MT; t++)
                        store_y(y + t * n + j, part[r][t], accumulate, ybuf,
                                (ln.slot * RB + r) * MT + t);
                }
            }
        }
    } else if ((ln.lane & (G - 1)) == 0) {
        const int g = ln.lane / G;
#pragma unroll
        for (int r = 0; r < RB; r++)
#pragma unroll
            for (int t = 0; t < MT; t++)
                rb[((ln.slot * RB + r) * MT + t) * ln.NG + g] = part[r][t];
    }
}

// ------------------------------------------------------- direct kernel
// F16/BF16: every lane loads its units straight from global memory; the next
// batch's loads are issued before the current batch is reduced. XL: x goes
// through LDS (else each lane reads its x units from global memory).
template <class F, int MT, int UPL, int RB, bool XL>
__device__ __forceinline__ void direct_body(const uint8_t *__restrict__ W,
                                            const float *__restrict__ x, float *__restrict__ y,
                                            int64_t k, int64_t n, int64_t row_bytes,
                                            int64_t j_start, int64_t j_end, int accumulate,
                                            int U, int L, int P, int G,
                                            const typename F::Aux &aux) {
    extern __shared__ float smem[];
    const Lanes<UPL> ln(U, L, G);
    const int64_t rows_per_batch = (int64_t)P * RB;
    const int64_t stride = (int64_t)gridDim.x * rows_per_batch;
    const uint8_t *Wslot = W + (int64_t)ln.slot * row_bytes;
    const int n4 = (int)(k >> 2), nt4 = n4 * MT;
    const int nq = P * RB * MT;
    float *red = smem + (XL ? k * MT : 0); // 2 x nq*NG group sums, then 2 x nq old y
    float *ybuf = red + 2 * nq * ln.NG;

    typename F::X xu[MT][UPL];
    if (!XL) x_units_from_global<F, MT, UPL>(xu, x, k, U, ln.ulod);
    f32x4 xa[4];
    if (XL) x_prefetch(x, nt4, ln.tid, ln.T, xa);

    // Rows are base + r*P + slot: the r*P part is uniform across the
    // workgroup (scalar address arithmetic), the slot part a per-lane
    // constant. Loads are branch-free: a row past j_end re-reads row j_end-1
    // and its result is dropped, which lets the compiler count outstanding
    // loads exactly.
    typename F::Raw raw[RB][UPL];
    YPrefetch<MT, RB> yp;
    int64_t base = j_start + (int64_t)xcd_block(blockIdx.x, gridDim.x) * rows_per_batch;
    const uint8_t *last_row = W + (j_end - 1) * row_bytes;
    auto issue = [&](int64_t b) {
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const int64_t jr = b + (int64_t)r * P;
            const bool in = ln.slot < P && jr + ln.slot < j_end;
            const uint8_t *row = in ? Wslot + jr * row_bytes : last_row;
            const int64_t j = in ? jr + ln.slot : j_end - 1; // the row index (per-row fields)
#pragma unroll
            for (int i = 0; i < UPL; i++) F::load(raw[r][i], row, ln.ulod[i], U, aux, j);
        }
        if (accumulate) yp.fetch(y, n, b, j_end, P, ln.tid, ln.T);
    };
    issue(base); // every workgroup has a first batch: the grid never exceeds the batch count

    if (XL) {
        f32x4 *xl = (f32x4 *)smem;
        x_to_lds<F>(x, xl, n4, nt4, U, ln.tid, ln.T, xa);
        lds_barrier();
        x_units_from_lds<F, MT, UPL>(xu, xl, n4, U, ln.ulod);
    }
    int buf = 0;

    for (; base < j_end; base += stride) {
        float part[RB][MT];
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const bool live = ln.slot < P && base + (int64_t)r * P + ln.slot < j_end;
#pragma unroll
            for (int t = 0; t < MT; t++) {
                float v = 0.f;
                if (live) {
#pragma unroll
                    for (int i = 0; i < UPL; i++)
                        if (ln.uvalid[i]) v += F::dot(raw[r][i], xu[t][i], ln.uid[i]);
                }
                part[r][t] = v;
            }
        }
        float *yb = ybuf + buf * nq;
        if (accumulate) yp.stash(yb, P, ln.tid, ln.T);
        if (base + stride < j_end) issue(base + stride);
        float *rb = red + buf * nq * ln.NG;
        if (ln.NG == 1 && accumulate) lds_barrier();
        reduce_batch<MT, RB, UPL>(part, ln, G, P, rb, yb, base, j_end, y, n, accumulate);
        if (ln.NG > 1) {
            lds_barrier();
            finish_batch<MT, RB>(rb, yb, ln.NG, P, ln.tid, ln.T, base, j_end, y, n,
                                 accumulate);
        }
        buf ^= 1;
    }
}

// ------------------------------------------------------- staged kernel
// LDS of the staged kernel: [x part][buffer 0][buffer 1][2 x nq*(NG+1) floats
// of group sums and old y][sink]; the x part and the buffers are multiples of
// 16 bytes, the sink starts at the next multiple of 16.
constexpr int STAGED_SINK_BYTES = 1024;
__host__ __device__ constexpr int staged_sink_offset(int x_part, int buf_bytes, int nq_ng1) {
    return (x_part + 2 * buf_bytes + 2 * nq_ng1 * 4 + 15) & ~15;
}
// Block formats. The byte range of a batch, [base*row_bytes,
// end*row_bytes), is copied in 16-byte pieces aligned down to 16 bytes of
// the 16-byte aligned base pointer (so
// up to 15 bytes before it and, at the very end of W, up to 15 bytes after it
// inside the same 16-byte granule, are read and ignored; W is 16-byte
// aligned, so such a granule never crosses a page). The copy goes straight
// from memory into LDS (buffer_load_dwordx4 ... lds): each wave instruction
// moves one contiguous kilobyte, no registers hold the data, and the
// compiler does not make the decode's LDS reads of the other buffer wait for
// it. The batch start is the scalar base of a buffer descriptor sized to the
// batch; lanes whose piece lies past the batch issue no copy (the
// descriptor's range check is a second guard), so a buffer holds exactly the
// largest batch. Batches 0 and 1 are copied at the start, both buffers at
// once; afterwards the copy of batch i+1 runs while batch i is decoded and is
// waited for at the end-of-batch barrier. XL: the units' records and integer
// planes are shared through LDS (else each lane converts its own from global
// memory).

// Single-token, one-row-per-slot instances fit in 128 registers without
// spilling, i.e. 4 waves per SIMD; the others are left to the compiler.
template <int MT, int UPL, int RB, int NPT>
struct StagedOccupancy {
    static constexpr int waves = (MT == 1 && UPL == 1 && RB == 1 && NPT <= 4) ? 4 : 1;
};

// W is 16-byte aligned; the matrix's row 0 starts w_off bytes after it (a
// stacked expert's slice need not start on a 16-byte boundary).
template <class F, int MT, int UPL, int RB, int NPT, bool XL>
__device__ __forceinline__ void staged_body(const uint8_t *__restrict__ W, int64_t w_off,
                                            const float *__restrict__ x, float *__restrict__ y,
                                            int64_t k, int64_t n, int64_t row_bytes,
                                            int64_t j_start, int64_t j_end, int accumulate,
                                            int U, int L, int P, int G, int buf_bytes, int T) {
    extern __shared__ float smem[];
    const Lanes<UPL> ln(U, L, G, T);
    const int64_t rows_per_batch = (int64_t)P * RB;
    const int64_t stride = (int64_t)gridDim.x * rows_per_batch;
    const int n4 = (int)(k >> 2);
    const int nq = P * RB * MT;
    const int rbytes = (int)row_bytes; // a row of one batch fits in LDS, so in 32 bits
    const int wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6); // in a scalar register
    // LDS: [x records and planes][weight buffer 0][weight buffer 1][2 x group
    // sums][2 x old y][1 KB sink] (without x in LDS, 16 bytes of padding in
    // front instead: unit reads may touch the dword before a row)
    XRec *rec = (XRec *)smem;
    uint32_t *pl = (uint32_t *)(rec + MT * U);
    uint8_t *wb = (uint8_t *)smem + (XL ? xplanes_bytes(MT, U) : 16);
    float *red = (float *)(wb + 2 * buf_bytes);
    float *ybuf = red + 2 * nq * ln.NG;
    uint8_t *sink = (uint8_t *)smem + staged_sink_offset(XL ? (int)xplanes_bytes(MT, U) : 16,
                                                         buf_bytes, nq * (ln.NG + 1));

    // Start copying batch b into weight buffer bi; b at or past j_end copies
    // nothing. The per-lane offset carries the whole piece number and the
    // descriptor covers exactly the batch's pieces, so lanes past them read
    // nothing (range check) and write at most 63 pieces past the batch's last
    // one, into the buffer's slack. A wave whose pieces all lie past the
    // batch skips its instruction (scalar branch), or with `all` still issues
    // it with its LDS writes pointed at the sink: then every wave issues all
    // NPT copy instructions whatever b is, and the compiler's load counts
    // stay exact.
    auto copy = [&](int64_t b, int bi, bool all) {
        const bool any = b < j_end;
        const int64_t r1 = b + rows_per_batch < j_end ? b + rows_per_batch : j_end;
        const int64_t s0 = w_off + b * row_bytes, s1 = w_off + r1 * row_bytes;
        const int64_t a0 = any ? s0 & ~(int64_t)15 : 0;
        const int np = any ? (int)((((s1 + 15) & ~(int64_t)15) - a0) >> 4) : 0;
        const __amdgpu_buffer_rsrc_t rs = batch_rsrc(W + a0, 16 * np);
        uint8_t *dst = wb + bi * buf_bytes;
#pragma unroll
        for (int s = 0; s < NPT; s++) {
            // lane l of this wave copies piece s*T + 64*wave + l
            const int first = s * ln.T + 64 * wave; // wave-uniform
            if (!all && first >= np) break;
            uint8_t *slot = first < np ? dst + 16 * first : sink;
            const int voff = 16 * (s * ln.T + ln.tid);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)slot, 16, voff, 0, 0,
                2 /* nontemporal */);
        }
    };

    typename F::X xu[MT][UPL];
    if (!XL) x_units_from_global<F, MT, UPL>(xu, x, k, U, ln.ulod);
    int64_t base = j_start + (int64_t)xcd_block(blockIdx.x, gridDim.x) * rows_per_batch;
    const int64_t b1 = base + stride;
    // Start-up: the first pieces of x and the old y of the first two batches
    // (accumulating) are requested, then both weight buffers are filled
    // (batches 0 and 1), and the x units are turned into their shared
    // records and planes while those copies are in flight. Every workgroup
    // has a first batch: the grid never exceeds the batch count.
    constexpr int XR = 4; // x pieces per thread loaded ahead of the copies
    const int g16 = ln.tid >> 4, ng = ln.T >> 4, pi = ln.tid & 15, nu = MT * U;
    f32x4 xr[XR];
    const f32x4 *x4 = (const f32x4 *)x;
    auto x_piece = [&](int q) { // piece pi of unit q = t*U + u
        const int t = q / U, u = q - t * U;
        return x4[t * n4 + F::x4_index(u, pi, U)];
    };
    if (XL) {
#pragma unroll
        for (int r = 0; r < XR; r++) {
            const int q = g16 + r * ng;
            xr[r] = x_piece(q < nu ? q : nu - 1);
        }
    }
    YPrefetch<MT, RB> yp, yp1;
    if (accumulate) {
        yp.fetch(y, n, base, j_end, P, ln.tid, ln.T);
        yp1.fetch(y, n, b1, j_end, P, ln.tid, ln.T);
    }
    copy(base, 0, true);
    copy(b1, 1, true);
    if (XL) {
        if (g16 < ng) {
#pragma unroll
            for (int r = 0; r < XR; r++)
                if (g16 + r * ng < nu) x_unit_planes(xr[r], g16 + r * ng, pi, U, rec, pl);
            for (int q = g16 + XR * ng; q < nu; q += ng) x_unit_planes(x_piece(q), q, pi, U, rec, pl);
        }
    }
    if (accumulate) {
        yp.stash(ybuf, P, ln.tid, ln.T);
        yp1.stash(ybuf + nq, P, ln.tid, ln.T);
    }
    // Wait for this wave's copy of batch 0 (the NPT copy instructions of
    // batch 1, issued after it, may still be in flight) and its LDS writes,
    // then for the other waves: batch 0 and the planes are then in LDS. (No
    // compiler fence here: it would also wait for batch 1.)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NPT) : "memory");
    if (XL) x_units_from_planes<F, MT, UPL>(xu, rec, pl, U, ln.ulod);

    int cur = 0;
    int64_t prev = -1; // batch whose group sums wait in LDS
    for (bool first = true; base < j_end; base += stride, first = false) {
        const int64_t nb = base + stride;
        // batch 1 is already on its way; later, the next batch
        const bool fetch_next = !first && nb < j_end;
        if (accumulate) yp.fetch(y, n, nb, j_end, P, ln.tid, ln.T);
        if (fetch_next) copy(nb, cur ^ 1, false);
        if (ln.NG > 1 && prev >= 0)
            finish_batch<MT, RB>(red + (cur ^ 1) * nq * ln.NG, ybuf + (cur ^ 1) * nq, ln.NG,
                                 P, ln.tid, ln.T, prev, j_end, y, n, accumulate);
        const int off = (int)((w_off + base * row_bytes) & 15);
        const uint8_t *bl = wb + cur * buf_bytes + off;
        float part[RB][MT];
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const int rr = r * P + ln.slot;
            const bool live = ln.slot < P && base + rr < j_end;
            const uint8_t *row = bl + (live ? rr : 0) * rbytes;
#pragma unroll
            for (int t = 0; t < MT; t++) part[r][t] = 0.f;
#pragma unroll
            for (int i = 0; i < UPL; i++) {
                typename F::Raw raw;
                F::load_lds(raw, row, ln.ulod[i], U);
#pragma unroll
                for (int t = 0; t < MT; t++)
                    if (live && ln.uvalid[i]) part[r][t] += F::dot(raw, xu[t][i], ln.uid[i]);
            }
        }
        reduce_batch<MT, RB, UPL>(part, ln, G, P, red + cur * nq * ln.NG, ybuf + cur * nq, base,
                                  j_end, y, n, accumulate);
        if (accumulate && fetch_next) yp.stash(ybuf + (cur ^ 1) * nq, P, ln.tid, ln.T);
        lds_barrier(); // also waits for the copy of the next batch
        prev = base;
        cur ^= 1;
    }
    if (ln.NG > 1 && prev >= 0)
        finish_batch<MT, RB>(red + (cur ^ 1) * nq * ln.NG, ybuf + (cur ^ 1) * nq, ln.NG, P,
                             ln.tid, ln.T, prev, j_end, y, n, accumulate);
}

// --------------------------------------------------------------- kernels
template <class F, int MT, int UPL, int RB, bool XL>
__global__ __launch_bounds__(512) void qmv_gemv_direct(const uint8_t *__restrict__ W,
                                                        const float *__restrict__ x,
                                                        float *__restrict__ y, int64_t k,
                                                        int64_t n, int64_t row_bytes,
                                                        int64_t j_start, int64_t j_end,
                                                        int accumulate, int U, int L, int P,
                                                        int G, int, int) {
    direct_body<F, MT, UPL, RB, XL>(W, x, y, k, n, row_bytes, j_start, j_end, accumulate, U, L,
                                    P, G, typename F::Aux{});
}

template <class F, int MT, int UPL, int RB, int NPT, bool XL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(
    StagedOccupancy<MT, UPL, RB, NPT>::waves))) void qmv_gemv_staged(const uint8_t *__restrict__ W,
                                                                  const float *__restrict__ x,
                                                                  float *__restrict__ y,
                                                                  int64_t k, int64_t n,
                                                                  int64_t row_bytes,
                                                                  int64_t j_start, int64_t j_end,
                                                                  int accumulate, int U, int L,
                                                                  int P, int G, int buf_bytes,
                                                                  int T) {
    staged_body<F, MT, UPL, RB, NPT, XL>(W, 0, x, y, k, n, row_bytes, j_start, j_end,
                                         accumulate, U, L, P, G, buf_bytes, T);
}

// Expert-indexed product (rullama 0.5.0, src/backend/dispatch/mod.rs, the
// batched expert-matmul test): output row `pair` = blockIdx.y is
// x[pair / top_k] @ W_e over all n rows of expert e = ids[pair], where W
// stacks the experts' matrices ([E][n][row bytes]). The blockIdx.x workgroups
// of a pair stream its expert's rows exactly as the plain kernels do. An
// expert number outside [0, n_experts) turns the pair's outputs into NaN.
__device__ __forceinline__ bool moe_pair(const uint32_t *ids, int64_t n_experts, int64_t n,
                                         float *y, uint32_t &e) {
    e = __builtin_amdgcn_readfirstlane(ids[blockIdx.y]);
    if ((int64_t)e < n_experts) return true;
    if (blockIdx.x == 0)
        for (int64_t j = threadIdx.x; j < n; j += blockDim.x)
            y[(int64_t)blockIdx.y * n + j] = __builtin_nanf("");
    return false;
}

template <class F, int UPL, int RB, bool XL>
__global__ __launch_bounds__(512) void qmv_gemv_moe_direct(const uint8_t *__restrict__ W,
                                                            const uint32_t *__restrict__ ids,
                                                            const float *__restrict__ x,
                                                            float *__restrict__ y, int64_t k,
                                                            int64_t n, int64_t row_bytes,
                                                            int64_t n_experts, int top_k,
                                                            int accumulate, int U, int L, int P,
                                                            int G, int, int) {
    uint32_t e;
    if (!moe_pair(ids, n_experts, n, y, e)) return;
    direct_body<F, 1, UPL, RB, XL>(W + (int64_t)e * n * row_bytes,
                                   x + (int64_t)(blockIdx.y / top_k) * k,
                                   y + (int64_t)blockIdx.y * n, k, n, row_bytes, 0, n,
                                   accumulate, U, L, P, G, typename F::Aux{});
}

template <class F, int UPL, int RB, int NPT, bool XL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(
    StagedOccupancy<1, UPL, RB, NPT>::waves))) void qmv_gemv_moe_staged(
    const uint8_t *__restrict__ W, const uint32_t *__restrict__ ids, const float *__restrict__ x,
    float *__restrict__ y, int64_t k, int64_t n, int64_t row_bytes, int64_t n_experts, int top_k,
    int accumulate, int U, int L, int P, int G, int buf_bytes, int T) {
    uint32_t e;
    if (!moe_pair(ids, n_experts, n, y, e)) return;
    staged_body<F, 1, UPL, RB, NPT, XL>(W, (int64_t)e * n * row_bytes,
                                        x + (int64_t)(blockIdx.y / top_k) * k,
                                        y + (int64_t)blockIdx.y * n, k, n, row_bytes, 0, n,
                                        accumulate, U, L, P, G, buf_bytes, T);
}

// Affine group-64 rows: the direct body over the code words, with the scales
// and biases of each (row, group) read alongside.
template <int BITS, int MT, int UPL, int RB, bool XL>
__global__ __launch_bounds__(512) void qmv_affine_gemv(const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ biases,
                                                        const float *__restrict__ x,
                                                        float *__restrict__ y, int64_t k,
                                                        int64_t n, int64_t j_start, int64_t j_end,
                                                        int accumulate, int U, int L, int P,
                                                        int G) {
    const typename UAffine<BITS>::Aux aux = {scales, biases, k / 64};
    direct_body<UAffine<BITS>, MT, UPL, RB, XL>(codes, x, y, k, n, k * BITS / 8, j_start, j_end,
                                                accumulate, U, L, P, G, aux);
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

static bool staged_format(int fmt) {
    return fmt == FMT_Q4_0 || fmt == FMT_Q4_K || fmt == FMT_Q6_K || fmt == FMT_Q8_0 ||
           fmt == FMT_Q5_0;
}

static constexpr size_t LDS_BUDGET = 80 * 1024; // weight buffers + reductions

static bool plan_gemv_upl(int fmt, int64_t k, int64_t rows, int mt_max, int num_cu, GemvPlan *p,
                          int pair_lanes, int upl) {
    if (k <= 0 || k % 64 != 0) return false;
    const int64_t U64 = k / 64;
    if (U64 > 1024) return false;
    GemvPlan g = {};
    g.fmt = fmt;
    g.U = (int)U64;
    g.UPL = upl ? upl : g.U <= 512 ? 1 : 2;
    g.L = (g.U + g.UPL - 1) / g.UPL;
    g.G = g.L & -g.L;
    if (g.G > 16) g.G = 16;
    g.NG = g.L / g.G;
    g.P = 64 / gcd_i(g.L, 64);
    while (g.P * g.L * 2 <= 256) g.P *= 2;
    if (g.P * g.L > 512) g.P = 512 / g.L > 0 ? 512 / g.L : 1;
    // small problems: fewer row slots per workgroup, so that more
    // workgroups share the rows
    while (g.P > 1 && g.P * g.L > 64 && (rows + g.P - 1) / g.P < num_cu) g.P /= 2;
    g.T = g.P * g.L;
    g.per_cu = STREAM_PER_CU;
    // Row slots that fill 4 waves exactly (64, 128 or 256 lanes per row: k =
    // 4096, 8192, 16384): 8 waves of them where that leaves at least two
    // batches per compute unit, which halves the batches, barriers and
    // reductions per row and doubles the waves resident per compute unit.
    // Measured (one token), 4 -> 8 waves: k=4096, 128256 rows: Q6_K 81.7 ->
    // 67.1 us, Q4_K 70.6 -> 52.7, Q4_0 68.1 -> 51.5, Q5_0 80.9 -> 64.0, BF16
    // 154 -> 152, Q8_0 unchanged (91.9); 14336 rows: Q4_K 12.9 -> 11.1, Q4_0
    // 11.8 -> 10.8, BF16 21.5 -> 21.1; k=8192, 8192 rows: Q4_K 15.8 -> 12.5;
    // 28672 rows: BF16 71.9 -> 68.5; 3072 rows: Q4_K 10.3 -> 9.6. Four 4-wave
    // workgroups per compute unit instead: Q6_K 73 us, Q4_K k=8192 16.7.
    // Narrower rows lose (k=2048 x 12288, Q4_K: 7.1 -> 7.9 us; k=1024 x 16384:
    // 5.4 -> 6.4), except in the expert-indexed launch (k=2048, 8 x 1536
    // rows: 9.3 -> 8.4 us), which passes pair_lanes = 32. The affine rows gain
    // with 4-bit codes (k=4096 x 128256: 79.5 -> 65.0 us; x 14336: 13.1 ->
    // 12.1) and lose with 8-bit ones (x 14336: 22.5 -> 23.6; k=8192 x 28672:
    // 72.1 -> 75.4), which keep 4 waves.
    if (g.T == 256 && g.L >= pair_lanes && fmt != FMT_AFFINE8 &&
        (rows + 2 * g.P - 1) / (2 * g.P) >= 2 * (int64_t)num_cu) {
        g.P *= 2;
        g.T = 512;
    }
    // The waves of a workgroup are dealt to the compute unit's four SIMDs in
    // turn, so a workgroup of 4w+1 waves puts two waves of every workgroup on
    // one SIMD, which then carries twice the decode work of the others, and
    // every batch's barrier waits for it. Where the row slots do not fill
    // whole groups of four waves (e.g. 40 lanes per row: 8 slots = 5 waves)
    // the workgroup is padded with idle lanes past the last slot, if that
    // idles at most 1/8 of them: workgroups of 5-7 waves (block formats: 3
    // and 5-7) to 512 threads (8 waves, two per SIMD, two workgroups per
    // compute unit) where that keeps every compute unit busy (at least two
    // batches per compute unit, or one round of workgroups where the unpadded
    // slots needed two); the direct kernel's launches with at least 4 batches
    // for each of 4 workgroups per compute unit to 256 threads instead (four
    // per compute unit). 3 waves to 8, measured: k=3072 (48 lanes) x 8192
    // rows, Q4_K 8.8 -> 8.1 us, Q6_K 9.3 -> 8.9; x 128256 (from 4 waves, four
    // per compute unit) Q4_K 43.5 -> 40.0, Q6_K 55.0 -> 52.4; k=6144 (96
    // lanes) x 16384, Q4_K 23.9 -> 16.0; BF16 k=3072 x 8192 10.0 -> 11.1,
    // hence the block formats only. There up to a quarter of the lanes may
    // idle: k=12288 (192 lanes, one slot of 3 waves -> two slots in 8 waves)
    // x 4096 rows Q4_K 21.5 -> 14.8 us, Q6_K 22.1 -> 15.6, Q8_0 22.8 -> 14.9,
    // Q4_0 21.1 -> 14.5; x 16384 Q4_K 49.9 -> 32.1, Q6_K 53.2 -> 43.4; x 1024
    // Q4_K 13.0 -> 10.1 (4 waves, 64 idle lanes, instead: 5-16% faster); and
    // 5-7-wave ones with more than an eighth idle: k=13824 (216 lanes, 2 slots)
    // x 5120 Q4_K 20.6 -> 19.3-20.0, Q4_0 19.8 -> 18.9, Q6_K 22.2 -> 21.7, Q8_0
    // 24.6 -> 25.2; x 1024 Q4_K 12.2 -> 11.3; k=9216 x 4096 12.0 -> 11.2;
    // k=13312 x 4096 16.5 -> 15.0. Measured,
    // k=2560 (40 lanes): the vocabulary products (262144 rows) Q6_K 120 us
    // unpadded, 113 with 256, 89.7-90.0 against 92.3-92.5 us with 512 rather
    // than 256 (Q4_K 70.1 against 73.3-74.6; BF16 with 512: 8 tiles 3%
    // slower); the 10240-row products 1-9% slower with 256 and 4-25% faster
    // with 512; 2560 and 6144 rows 13-25% faster with 512, 4096 rows 3-4%
    // slower without the busy-units condition.
    if (g.T % 256 != 0 && g.T > 64 && g.L <= 256) {
        const int P4 = 256 / g.L, P8 = 512 / g.L;
        const bool many = P4 >= 1 && (256 - P4 * g.L) * 8 <= 256 &&
                          (rows + P4 - 1) / P4 >= 16 * (int64_t)num_cu;
        // block formats: up to a quarter of the lanes idle
        const bool blk = staged_format(fmt);
        bool pad8 = (g.T > 256 || (g.T > 128 && blk)) && P8 >= 1 &&
                    (512 - P8 * g.L) * (blk ? 4 : 8) <= 512;
        if (pad8) {
            const int64_t b8 = (rows + P8 - 1) / P8, bp = (rows + g.P - 1) / g.P;
            pad8 = b8 >= 2 * (int64_t)num_cu || (b8 <= num_cu && bp > num_cu);
        }
        if (pad8 && (staged_format(fmt) || !many)) {
            g.P = P8;
            g.T = 512;
        } else if (many) {
            g.P = P4;
            g.T = 256;
            g.per_cu = STREAM_PER_CU_4W;
        }
    }
    g.MT = (g.UPL == 1 && mt_max >= 2) ? 2 : 1;
    int64_t rb;
    switch (fmt) {
    case FMT_F16:
    case FMT_BF16: rb = 2 * k; break;
    case FMT_Q4_0: rb = (k / 32) * 18; break;
    case FMT_Q8_0: rb = (k / 32) * 34; break;
    case FMT_Q5_0: rb = (k / 32) * 22; break;
    case FMT_Q4_K:
        if (k % 256) return false;
        rb = (k / 256) * 144;
        break;
    case FMT_Q6_K:
        if (k % 256) return false;
        rb = (k / 256) * 210;
        break;
    case FMT_AFFINE4: rb = k / 2; break;
    case FMT_AFFINE8: rb = k; break;
    default: return false;
    }
    g.staged = staged_format(fmt) ? 1 : 0;
    // Rows per slot per batch: the largest of 2 and 1 that fits the register
    // budget (staged: at most 8 pieces per thread) and the LDS budget,
    // keeping at least two batches per compute unit where the rows allow.
    g.RB = 0;
    // first within the budget that leaves room for two workgroups per compute
    // unit; long rows fall back to one workgroup per compute unit
    for (int attempt = 0; attempt < 2 && g.RB == 0; attempt++)
    for (int cand = 2; cand >= 1 && g.RB == 0; cand /= 2) {
        const int64_t budget = attempt == 0 ? (int64_t)LDS_BUDGET : (int64_t)144 * 1024;
        if (!g.staged && cand > 1 && (g.MT > 1 || g.UPL > 1)) continue; // registers
        // staged: one row per slot per batch (two measured slower: the larger
        // buffers leave fewer workgroups per compute unit)
        if (g.staged && cand > 1) continue;
        int npt = 0;
        if (g.staged) {
            const int64_t pieces = ((int64_t)g.P * cand * rb + 30 + 15) / 16;
            const int64_t need = (pieces + g.T - 1) / g.T;
            npt = need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
            if (npt == 0) continue;
        }
        // the batch's pieces plus 63 (the slack the last copying wave may
        // write into), rounded to 64 bytes
        const int64_t buf =
            g.staged ? ((((g.P * cand * rb + 30 + 15) / 16 + 63) * 16 + 63) & ~(int64_t)63) : 0;
        const int64_t red = (int64_t)2 * g.P * cand * g.MT * (g.NG + 1) * 4;
        if (2 * buf + red > budget) continue;
        if ((int64_t)g.P * cand * g.MT > 2 * (int64_t)g.T) continue; // y prefetch: 2 per thread
        const int64_t batches = (rows + (int64_t)g.P * cand - 1) / ((int64_t)g.P * cand);
        if (cand > 1 && batches < 2 * (int64_t)num_cu) continue;
        g.RB = cand;
        g.npt = npt;
        g.buf_bytes = (int)buf;
    }
    if (g.RB == 0) return false;
    const int64_t batches = (rows + (int64_t)g.P * g.RB - 1) / ((int64_t)g.P * g.RB);
    // upper bound; the launch clamps it to what stays resident
    g.grid = (int)(batches < ((int64_t)1 << 30) ? batches : ((int64_t)1 << 30));
    if (g.grid < 1) g.grid = 1;
    g.num_cu = num_cu;
    // x in LDS: the staged kernels keep each unit's record and integer planes
    // there, the direct ones x itself
    const size_t xb = g.staged ? (size_t)xplanes_bytes(g.MT, g.U) : (size_t)k * g.MT * sizeof(float);
    const size_t red = (size_t)2 * g.P * g.RB * g.MT * (g.NG + 1) * sizeof(float);
    const size_t wbuf = (size_t)2 * g.buf_bytes;
    // x goes through LDS when everything fits in 96 KB; otherwise each lane
    // reads its x units straight from global memory
    g.x_in_lds = (xb + wbuf + red <= 96 * 1024) ? 1 : 0;
    g.lds_bytes = g.staged ? staged_sink_offset(g.x_in_lds ? (int)xb : 16, g.buf_bytes,
                                                (int)(red / (2 * sizeof(float)))) +
                                 STAGED_SINK_BYTES
                           : (g.x_in_lds ? xb : 0) + wbuf + red;
    if (g.lds_bytes > 160 * 1024) return false;
    *p = g;
    return true;
}

// Rows of 192+ units (k >= 12288) and many of them, one token, block formats:
// two units per lane, which gives the 8-wave workgroup about 512/(U/2) row
// slots, where that leaves at least 8 batches per workgroup at two per
// compute unit and two workgroups' staging buffers fit a compute unit's LDS
// (else one unit per lane). Measured (Q4_K, one token, same process): k=28672 x 8192 42.5 ->
// 39.3 us, k=16384 x 53248 112.5 -> 92.9; with fewer batches it loses
// (k=14336 x 4096 15.2 -> 22.0, k=12288 x 4096 21.2 -> 22.1, k=16384 x 4096
// 15.5 -> 22.8).
bool plan_gemv(int fmt, int64_t k, int64_t rows, int mt_max, int num_cu, GemvPlan *p,
               int pair_lanes) {
    const int64_t U = k / 64;
    GemvPlan two;
    if (k > 0 && k % 64 == 0 && U >= 192 && U <= 512 && mt_max == 1 && staged_format(fmt) &&
        rows >= 16 * (int64_t)num_cu * (512 / ((U + 1) / 2)) &&
        plan_gemv_upl(fmt, k, rows, mt_max, num_cu, &two, pair_lanes, 2) &&
        two.lds_bytes <= LDS_BUDGET) {
        *p = two;
        return true;
    }
    return plan_gemv_upl(fmt, k, rows, mt_max, num_cu, p, pair_lanes, 0);
}

template <typename K>
static hipError_t launch_k(K kernel, const GemvPlan &p, const uint8_t *W, const float *x,
                           float *y, int64_t k, int64_t n, int64_t row_bytes, int64_t j0,
                           int64_t j1, int acc, hipStream_t s) {
    if (p.lds_bytes > 64 * 1024 &&
        hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds_bytes) != hipSuccess)
        return hipGetLastError();
    int res = resident_per_cu(kernel, p.T, p.lds_bytes);
    if (res > p.per_cu) res = p.per_cu;
    const int64_t cap = (int64_t)p.num_cu * res;
    const int grid = (int)(p.grid < cap ? p.grid : cap);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(p.T), p.lds_bytes, s, W, x, y, k, n, row_bytes,
                       j0, j1, acc, p.U, p.L, p.P, p.G, p.buf_bytes, p.T);
    return hipGetLastError();
}

template <class F, int MT, int UPL, int RB, bool XL>
static hipError_t launch_staged_npt(const GemvPlan &p, const uint8_t *W, const float *x,
                                    float *y, int64_t k, int64_t n, int64_t rb, int64_t j0,
                                    int64_t j1, int acc, hipStream_t s) {
    switch (p.npt) {
    case 2:
        return launch_k(qmv_gemv_staged<F, MT, UPL, RB, 2, XL>, p, W, x, y, k, n, rb, j0, j1,
                        acc, s);
    case 4:
        return launch_k(qmv_gemv_staged<F, MT, UPL, RB, 4, XL>, p, W, x, y, k, n, rb, j0, j1,
                        acc, s);
    default:
        return launch_k(qmv_gemv_staged<F, MT, UPL, RB, 8, XL>, p, W, x, y, k, n, rb, j0, j1,
                        acc, s);
    }
}

// (the staged plan always has one row per slot per batch)
template <class F, int MT, int UPL, bool XL>
static hipError_t launch_staged_rb(const GemvPlan &p, const uint8_t *W, const float *x,
                                   float *y, int64_t k, int64_t n, int64_t rb, int64_t j0,
                                   int64_t j1, int acc, hipStream_t s) {
    if (p.RB != 1) return hipErrorInvalidValue;
    return launch_staged_npt<F, MT, UPL, 1, XL>(p, W, x, y, k, n, rb, j0, j1, acc, s);
}

template <class F, int MT, int UPL, bool XL>
static hipError_t launch_direct_rb(const GemvPlan &p, const uint8_t *W, const float *x,
                                   float *y, int64_t k, int64_t n, int64_t rb, int64_t j0,
                                   int64_t j1, int acc, hipStream_t s) {
    if (p.RB == 2)
        return launch_k(qmv_gemv_direct<F, MT, UPL, 2, XL>, p, W, x, y, k, n, rb, j0, j1, acc,
                        s);
    return launch_k(qmv_gemv_direct<F, MT, UPL, 1, XL>, p, W, x, y, k, n, rb, j0, j1, acc, s);
}

// x goes through LDS when the plan allows it and x is 16-byte aligned (x is
// read in 16-byte pieces).
static bool use_x_lds(GemvPlan &p, const float *x, int64_t k) {
    if (p.x_in_lds && ((uintptr_t)x & 15) == 0) return true;
    if (p.x_in_lds)
        p.lds_bytes -= p.staged ? (size_t)xplanes_bytes(p.MT, p.U) - 16
                                : (size_t)k * p.MT * sizeof(float);
    // (the staged layout's parts after x are multiples of 16 bytes, so the
    // sink offset moves by exactly the difference)
    p.x_in_lds = 0;
    return false;
}

template <class F>
static hipError_t launch_staged(const GemvPlan &p0, const uint8_t *W, const float *x, float *y,
                                int64_t k, int64_t n, int64_t rb, int64_t j0, int64_t j1, int acc,
                                hipStream_t s) {
    GemvPlan p = p0;
    if (use_x_lds(p, x, k)) {
        if (p.UPL == 2) return launch_staged_rb<F, 1, 2, true>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        if (p.MT == 2) return launch_staged_rb<F, 2, 1, true>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        return launch_staged_rb<F, 1, 1, true>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    }
    if (p.UPL == 2) return launch_staged_rb<F, 1, 2, false>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    if (p.MT == 2) return launch_staged_rb<F, 2, 1, false>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    return launch_staged_rb<F, 1, 1, false>(p, W, x, y, k, n, rb, j0, j1, acc, s);
}

template <class F>
static hipError_t launch_direct(const GemvPlan &p0, const uint8_t *W, const float *x, float *y,
                                int64_t k, int64_t n, int64_t rb, int64_t j0, int64_t j1, int acc,
                                hipStream_t s) {
    GemvPlan p = p0;
    if (use_x_lds(p, x, k)) {
        if (p.UPL == 2) return launch_direct_rb<F, 1, 2, true>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        if (p.MT == 2) return launch_direct_rb<F, 2, 1, true>(p, W, x, y, k, n, rb, j0, j1, acc, s);
        return launch_direct_rb<F, 1, 1, true>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    }
    if (p.UPL == 2) return launch_direct_rb<F, 1, 2, false>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    if (p.MT == 2) return launch_direct_rb<F, 2, 1, false>(p, W, x, y, k, n, rb, j0, j1, acc, s);
    return launch_direct_rb<F, 1, 1, false>(p, W, x, y, k, n, rb, j0, j1, acc, s);
}

// ------------------------------------------------ affine launches
struct AffineArgs {
    const uint16_t *scales, *biases;
};

template <int BITS, int MT, int UPL, int RB, bool XL>
static hipError_t launch_affine_k(const GemvPlan &p, const uint8_t *q, const AffineArgs &a,
                                  const float *x, float *y, int64_t k, int64_t n, int64_t j0,
                                  int64_t j1, int acc, hipStream_t s) {
    auto kernel = qmv_affine_gemv<BITS, MT, UPL, RB, XL>;
    if (p.lds_bytes > 64 * 1024 &&
        hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds_bytes) != hipSuccess)
        return hipGetLastError();
    int res = resident_per_cu(kernel, p.T, p.lds_bytes);
    if (res > p.per_cu) res = p.per_cu;
    const int64_t cap = (int64_t)p.num_cu * res;
    const int grid = (int)(p.grid < cap ? p.grid : cap);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(p.T), p.lds_bytes, s, q, a.scales, a.biases, x, y,
                       k, n, j0, j1, acc, p.U, p.L, p.P, p.G);
    return hipGetLastError();
}

template <int BITS, bool XL>
static hipError_t launch_affine_x(const GemvPlan &p, const uint8_t *q, const AffineArgs &a,
                                  const float *x, float *y, int64_t k, int64_t n, int64_t j0,
                                  int64_t j1, int acc, hipStream_t s) {
    if (p.UPL == 2) return launch_affine_k<BITS, 1, 2, 1, XL>(p, q, a, x, y, k, n, j0, j1, acc, s);
    if (p.MT == 2) return launch_affine_k<BITS, 2, 1, 1, XL>(p, q, a, x, y, k, n, j0, j1, acc, s);
    if (p.RB == 2) return launch_affine_k<BITS, 1, 1, 2, XL>(p, q, a, x, y, k, n, j0, j1, acc, s);
    return launch_affine_k<BITS, 1, 1, 1, XL>(p, q, a, x, y, k, n, j0, j1, acc, s);
}

hipError_t launch_affine(const GemvPlan &p0, const uint8_t *codes, const uint16_t *scales,
                         const uint16_t *biases, const float *x, float *y, int64_t k, int64_t n,
                         int64_t j_start, int64_t j_end, int accumulate, hipStream_t s) {
    GemvPlan p = p0;
    const AffineArgs a = {scales, biases};
    const bool xl = use_x_lds(p, x, k);
    if (p.fmt == FMT_AFFINE4)
        return xl ? launch_affine_x<4, true>(p, codes, a, x, y, k, n, j_start, j_end, accumulate, s)
                  : launch_affine_x<4, false>(p, codes, a, x, y, k, n, j_start, j_end, accumulate,
                                              s);
    if (p.fmt == FMT_AFFINE8)
        return xl ? launch_affine_x<8, true>(p, codes, a, x, y, k, n, j_start, j_end, accumulate, s)
                  : launch_affine_x<8, false>(p, codes, a, x, y, k, n, j_start, j_end, accumulate,
                                              s);
    return hipErrorInvalidValue;
}

// ------------------------------------------------ expert-indexed launches
struct MoeArgs {
    const uint32_t *ids;
    int64_t n_experts;
    int top_k, pairs;
};

// blockIdx.y = pair; the residency cap is shared by the pairs
template <typename K>
static hipError_t launch_moe_k(K kernel, const GemvPlan &p, const uint8_t *W, const MoeArgs &a,
                               const float *x, float *y, int64_t k, int64_t n, int64_t rb,
                               int acc, hipStream_t s) {
    if (p.lds_bytes > 64 * 1024 &&
        hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds_bytes) != hipSuccess)
        return hipGetLastError();
    // (every resident workgroup: the pairs' short row ranges are latency-bound)
    const int64_t cap = (int64_t)p.num_cu * resident_per_cu(kernel, p.T, p.lds_bytes);
    int64_t per = cap / a.pairs;
    if (per > p.grid) per = p.grid;
    if (per < 1) per = 1;
    hipLaunchKernelGGL(kernel, dim3((unsigned)per, (unsigned)a.pairs), dim3(p.T), p.lds_bytes, s,
                       W, a.ids, x, y, k, n, rb, a.n_experts, a.top_k, acc, p.U, p.L, p.P, p.G,
                       p.buf_bytes, p.T);
    return hipGetLastError();
}

template <class F, int UPL, bool XL>
static hipError_t launch_moe_staged_x(const GemvPlan &p, const uint8_t *W, const MoeArgs &a,
                                      const float *x, float *y, int64_t k, int64_t n, int64_t rb,
                                      int acc, hipStream_t s) {
    switch (p.npt) { // the staged plan always has one row per slot per batch
    case 2:
        return launch_moe_k(qmv_gemv_moe_staged<F, UPL, 1, 2, XL>, p, W, a, x, y, k, n, rb, acc, s);
    case 4:
        return launch_moe_k(qmv_gemv_moe_staged<F, UPL, 1, 4, XL>, p, W, a, x, y, k, n, rb, acc, s);
    default:
        return launch_moe_k(qmv_gemv_moe_staged<F, UPL, 1, 8, XL>, p, W, a, x, y, k, n, rb, acc, s);
    }
}

template <class F, int UPL, bool XL>
static hipError_t launch_moe_direct_x(const GemvPlan &p, const uint8_t *W, const MoeArgs &a,
                                      const float *x, float *y, int64_t k, int64_t n, int64_t rb,
                                      int acc, hipStream_t s) {
    if (p.RB == 2)
        return launch_moe_k(qmv_gemv_moe_direct<F, UPL, 2, XL>, p, W, a, x, y, k, n, rb, acc, s);
    return launch_moe_k(qmv_gemv_moe_direct<F, UPL, 1, XL>, p, W, a, x, y, k, n, rb, acc, s);
}

template <class F, bool STAGED>
static hipError_t launch_moe_f(const GemvPlan &p0, const uint8_t *W, const MoeArgs &a,
                               const float *x, float *y, int64_t k, int64_t n, int64_t rb,
                               int acc, hipStream_t s) {
    GemvPlan p = p0;
    const bool xl = use_x_lds(p, x, k);
    if constexpr (STAGED) {
        if (p.UPL == 2)
            return xl ? launch_moe_staged_x<F, 2, true>(p, W, a, x, y, k, n, rb, acc, s)
                      : launch_moe_staged_x<F, 2, false>(p, W, a, x, y, k, n, rb, acc, s);
        return xl ? launch_moe_staged_x<F, 1, true>(p, W, a, x, y, k, n, rb, acc, s)
                  : launch_moe_staged_x<F, 1, false>(p, W, a, x, y, k, n, rb, acc, s);
    } else {
        if (p.UPL == 2)
            return xl ? launch_moe_direct_x<F, 2, true>(p, W, a, x, y, k, n, rb, acc, s)
                      : launch_moe_direct_x<F, 2, false>(p, W, a, x, y, k, n, rb, acc, s);
        return xl ? launch_moe_direct_x<F, 1, true>(p, W, a, x, y, k, n, rb, acc, s)
                  : launch_moe_direct_x<F, 1, false>(p, W, a, x, y, k, n, rb, acc, s);
    }
}

hipError_t launch_gemv_moe(const GemvPlan &p, const uint8_t *W, const uint32_t *ids,
                           const float *x, float *y, int64_t k, int64_t n, int64_t row_bytes,
                           int64_t n_experts, int64_t n_pos, int top_k, int accumulate,
                           hipStream_t s) {
    const MoeArgs a = {ids, n_experts, top_k, (int)(n_pos * top_k)};
    const int64_t rb = row_bytes;
    switch (p.fmt) {
    case FMT_Q4_0: return launch_moe_f<IntX<UQ4_0>, true>(p, W, a, x, y, k, n, rb, accumulate, s);
    case FMT_Q4_K: return launch_moe_f<IntX<UQ4_K>, true>(p, W, a, x, y, k, n, rb, accumulate, s);
    case FMT_Q6_K: return launch_moe_f<IntX<UQ6_K>, true>(p, W, a, x, y, k, n, rb, accumulate, s);
    case FMT_Q8_0: return launch_moe_f<IntX<UQ8_0>, true>(p, W, a, x, y, k, n, rb, accumulate, s);
    case FMT_Q5_0: return launch_moe_f<IntX<UQ5_0>, true>(p, W, a, x, y, k, n, rb, accumulate, s);
    case FMT_BF16:
        return launch_moe_f<UHalf<true>, false>(p, W, a, x, y, k, n, rb, accumulate, s);
    case FMT_F16:
        return launch_moe_f<UHalf<false>, false>(p, W, a, x, y, k, n, rb, accumulate, s);
    default: return hipErrorInvalidValue;
    }
}

const char *gemv_moe_kernel_name(const GemvPlan &p) {
    static const char *names[] = {"",
                                  "qmv_gemv_moe_direct<f16>",
                                  "qmv_gemv_moe_direct<bf16>",
                                  "qmv_gemv_moe_staged<q4_0>",
                                  "qmv_gemv_moe_staged<q4_k>",
                                  "qmv_gemv_moe_staged<q6_k>",
                                  "qmv_gemv_moe_staged<q8_0>",
                                  "qmv_gemv_moe_staged<q5_0>"};
    return (p.fmt >= 1 && p.fmt <= 7) ? names[p.fmt] : "";
}

hipError_t launch_gemv(const GemvPlan &p, const uint8_t *W, const float *x, float *y,
                       int64_t k, int64_t n, int64_t row_bytes, int64_t j_start,
                       int64_t j_end, int accumulate, hipStream_t stream) {
    switch (p.fmt) {
    case FMT_Q4_0:
        return launch_staged<IntX<UQ4_0>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                    stream);
    case FMT_Q4_K:
        return launch_staged<IntX<UQ4_K>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                    stream);
    case FMT_Q6_K:
        return launch_staged<IntX<UQ6_K>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                    stream);
    case FMT_Q8_0:
        return launch_staged<IntX<UQ8_0>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                    stream);
    case FMT_Q5_0:
        return launch_staged<IntX<UQ5_0>>(p, W, x, y, k, n, row_bytes, j_start, j_end, accumulate,
                                    stream);
    case FMT_BF16:
        return launch_direct<UHalf<true>>(p, W, x, y, k, n, row_bytes, j_start, j_end,
                                          accumulate, stream);
    case FMT_F16:
        return launch_direct<UHalf<false>>(p, W, x, y, k, n, row_bytes, j_start, j_end,
                                           accumulate, stream);
    default: return hipErrorInvalidValue;
    }
}

const char *gemv_kernel_name(const GemvPlan &p) {
    static const char *names[] = {"",
                                  "qmv_gemv_direct<f16>",
                                  "qmv_gemv_direct<bf16>",
                                  "qmv_gemv_staged<q4_0>",
                                  "qmv_gemv_staged<q4_k>",
                                  "qmv_gemv_staged<q6_k>",
                                  "qmv_gemv_staged<q8_0>",
                                  "qmv_gemv_staged<q5_0>"};
    return (p.fmt >= 1 && p.fmt <= 7) ? names[p.fmt] : "";
}

} // namespace qmv
