// Transposed (backward-input) product for gfx950, one token at a time:
//   dx[i] (=|+=) sum_{j_start <= j < j_end} dy[j] * w_j[i]     for all i < k.
//
// Operation: rullama 0.5.0, src/backend/dispatch/mod.rs, struct
// MatmulBackInputParams (the row range bounds the summed axis, so a
// vocabulary-sized product can be cut into several submissions: the first
// writes dx, the others add to it) and the backward-input parity tests of the
// same page (dy of length n in, dx of length k out).
//
// Two kernels on the caller's stream:
//  1. qmv_gemv_t_staged: a persistent grid streams the rows of the range in
//     batches of P consecutive rows, exactly as the forward staged kernel does
//     (the batch is copied one batch ahead from memory into double-buffered
//     LDS, 16-byte pieces, one contiguous kilobyte per wave instruction). Row
//     slot s of a workgroup takes row base + s of each batch; lane l of the
//     slot owns the 64-weight units l, l + L, ... of k and keeps, per unit, 64
//     f32 accumulators acc_e += dy_j * w_j[e] in registers for the whole
//     launch. At the end the P slots' vectors are added in a fixed tree in LDS
//     and the workgroup writes its partial dx (k floats) to scratch.
//  2. qmv_gemv_t_reduce: adds the partials of all workgroups in a fixed order
//     (64 interleaved running sums, then a fixed tree) and writes or adds dx.
// Scratch (grid * k floats) is lent by the library's per-device scratch cache
// (reused across calls; see qmv_api.cpp). Rows are assigned to workgroups by the
// row range and the grid size only, so a launch is deterministic run to run.
#include "qmv_internal.h"
#include "qmv_units.h"

namespace qmv {
namespace {

constexpr int T_MAX_GRID = 1024; // partials the reduction kernel takes

template <class F, int UPL, int NPT>
__global__ __launch_bounds__(512) void qmv_gemv_t_staged(const uint8_t *__restrict__ W,
                                                          const float *__restrict__ dy,
                                                          float *__restrict__ part, int64_t k,
                                                          int64_t row_bytes, int64_t j_start,
                                                          int64_t j_end, int U, int L, int P,
                                                          int buf_bytes) {
    extern __shared__ float smem[];
    const Lanes<UPL> ln(U, L, L);
    const int64_t stride = (int64_t)gridDim.x * P;
    const int rbytes = (int)row_bytes;
    const int wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6); // in a scalar register
    // [16 bytes of padding][weight buffer 0][weight buffer 1]: unit reads may
    // touch the dword before a row
    uint8_t *wb = (uint8_t *)smem + 16;

    // Start copying the rows [b, b + P) (clipped to j_end) into buffer bi.
    auto copy = [&](int64_t b, int bi) {
        const int64_t r1 = b + P < j_end ? b + P : j_end;
        const int64_t s0 = b * row_bytes, s1 = r1 * row_bytes;
        const int64_t a0 = s0 & ~(int64_t)15;
        const int np = (int)((((s1 + 15) & ~(int64_t)15) - a0) >> 4);
        const __amdgpu_buffer_rsrc_t rs = batch_rsrc(W + a0, 16 * np);
        const int last = 16 * (np - 1);
        uint8_t *dst = wb + bi * buf_bytes;
        const int voff = 16 * ln.tid;
#pragma unroll
        for (int s = 0; s < NPT; s++) {
            const int soff = 16 * s * ln.T;
            uint8_t *slot = dst + 16 * (s * ln.T + 64 * wave);
            if (voff <= last - soff)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)slot, 16, voff, soff, 0,
                    2 /* nontemporal */);
        }
    };
    auto dy_of = [&](int64_t b) {
        const int64_t j = b + ln.slot;
        return j < j_end ? dy[j] : 0.f;
    };

    typename F::X acc[UPL];
#pragma unroll
    for (int i = 0; i < UPL; i++) {
#pragma unroll
        for (int p = 0; p < 16; p++) F::put_x(acc[i], p, f32x4{0.f, 0.f, 0.f, 0.f});
        F::finish_x(acc[i]); // zero sums where the unit keeps any
    }

    int64_t base = j_start + (int64_t)blockIdx.x * P;
    copy(base, 0); // every workgroup has a first batch: the grid never exceeds the batch count
    float dyc = dy_of(base);
    lds_barrier();
    int cur = 0;
    for (; base < j_end; base += stride) {
        const int64_t nb = base + stride;
        float dyn = 0.f;
        if (nb < j_end) {
            copy(nb, cur ^ 1);
            dyn = dy_of(nb);
        }
        if (base + ln.slot < j_end) {
            const uint8_t *row =
                wb + cur * buf_bytes + (int)((base * row_bytes) & 15) + ln.slot * rbytes;
#pragma unroll
            for (int i = 0; i < UPL; i++) {
                if (ln.uvalid[i]) {
                    typename F::Raw raw;
                    F::load_lds(raw, row, ln.ulod[i], U);
                    F::axpy(raw, dyc, acc[i], ln.uid[i]);
                }
            }
        }
        lds_barrier(); // also waits for the copy of the next batch
        cur ^= 1;
        dyc = dyn;
    }
#pragma unroll
    for (int i = 0; i < UPL; i++) F::finish_t(acc[i]);

    // Slots h..2h-1 hand their vectors to slots 0..h-1 (h = P/2, P/4, ..., 1).
    float *red = smem; // the weight buffers are free: the last barrier drained the copies
    for (int h = P >> 1; h >= 1; h >>= 1) {
        if (ln.slot >= h && ln.slot < 2 * h) {
            float *o = red + (int64_t)(ln.slot - h) * k;
#pragma unroll
            for (int i = 0; i < UPL; i++)
                if (ln.uvalid[i])
#pragma unroll
                    for (int p = 0; p < 16; p++)
                        *(f32x4 *)(o + 4 * F::x4_index(ln.uid[i], p, U)) = F::get_x(acc[i], p);
        }
        lds_barrier();
        if (ln.slot < h) {
            const float *o = red + (int64_t)ln.slot * k;
#pragma unroll
            for (int i = 0; i < UPL; i++)
                if (ln.uvalid[i])
#pragma unroll
                    for (int p = 0; p < 16; p++)
                        F::put_x(acc[i], p,
                                 F::get_x(acc[i], p) +
                                     *(const f32x4 *)(o + 4 * F::x4_index(ln.uid[i], p, U)));
        }
        lds_barrier();
    }
    if (ln.slot == 0) {
        float *o = part + (int64_t)blockIdx.x * k;
#pragma unroll
        for (int i = 0; i < UPL; i++)
            if (ln.uvalid[i])
#pragma unroll
                for (int p = 0; p < 16; p++)
                    *(f32x4 *)(o + 4 * F::x4_index(ln.uid[i], p, U)) = F::get_x(acc[i], p);
    }
}

// dx (=|+=) sum over the G workgroup partials. Workgroup: 16 consecutive
// outputs (4 float4 pieces) x 64 running sums; running sum g adds partials
// g, g+64, g+128, ... in that order, then the 64 sums meet in a fixed tree.
__global__ __launch_bounds__(256) void qmv_gemv_t_reduce(const float *__restrict__ part,
                                                         float *__restrict__ dx, int64_t k, int G,
                                                         int accumulate) {
    __shared__ f32x4 red[64][4];
    const int p = threadIdx.x & 3, g = threadIdx.x >> 2;
    const int64_t e = (int64_t)blockIdx.x * 16 + 4 * p;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    int q = g;
    for (; q + 64 * 7 < G; q += 64 * 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = *(const f32x4 *)(part + (int64_t)(q + 64 * u) * k + e);
#pragma unroll
        for (int u = 0; u < 8; u++) s += v[u];
    }
    for (; q < G; q += 64) s += *(const f32x4 *)(part + (int64_t)q * k + e);
    red[g][p] = s;
    __syncthreads();
    for (int h = 32; h >= 1; h >>= 1) {
        if (g < h) red[g][p] += red[g + h][p];
        __syncthreads();
    }
    if (g == 0) { // dx is only 4-byte aligned
        const f32x4 r = red[0][p];
        float *d = dx + e;
        d[0] = accumulate ? d[0] + r.x : r.x;
        d[1] = accumulate ? d[1] + r.y : r.y;
        d[2] = accumulate ? d[2] + r.z : r.z;
        d[3] = accumulate ? d[3] + r.w : r.w;
    }
}

} // namespace

bool plan_gemv_t(int fmt, int64_t k, int64_t rows, int num_cu, GemvTPlan *out) {
    if (k <= 0 || k % 64 != 0 || rows <= 0) return false;
    const int64_t U64 = k / 64;
    if (U64 > 1024) return false;
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
    default: return false;
    }
    GemvTPlan g = {};
    g.fmt = fmt;
    g.U = (int)U64;
    g.UPL = g.U <= 512 ? 1 : 2;
    g.L = (g.U + g.UPL - 1) / g.UPL;
    // P row slots (a power of two), P*L <= 512 threads, aiming at 4+ waves;
    // 8 for the block formats' rows of 64+ lanes (k >= 4096), which halves
    // the batches and barriers per row. Measured (one token, 4 -> 8 waves):
    // k=4096 x 14336 Q4_K 23.5 -> 21.9 us, Q6_K 22.1 -> 20.8, Q8_0 27.2 ->
    // 25.8, Q4_0 23.1 -> 22.0; k=8192 x 8192 Q4_K 29.4 -> 25.4; k=4096 x
    // 128256 Q6_K 76.9-80.6 -> 76.7-77.1. F16/BF16 mixed (F16 k=8192 x 28672
    // 80.9 -> 78.3, BF16 k=4096 x 14336 27.5 -> 28.4): 4 waves.
    const bool wide8 = g.L >= 64 && fmt != FMT_F16 && fmt != FMT_BF16;
    g.P = 1;
    while (g.P * 2 * g.L <= 512 && g.P * g.L < (wide8 ? 512 : 256)) g.P *= 2;
    // small problems: fewer slots, so that more workgroups share the rows
    while (g.P > 1 && (rows + g.P - 1) / g.P < 2 * (int64_t)num_cu) g.P /= 2;
    // A batch of P rows spans P*rb bytes; when rows are not a whole number
    // of 16-byte pieces its start and end may each add a partial piece.
    const int64_t slack = rb % 16 ? 30 : 0;
    // at most 8 pieces of 16 bytes per thread per batch: fewer slots for
    // long rows
    for (;;) {
        g.T = g.P * g.L;
        const int64_t pieces = ((int64_t)g.P * rb + slack + 15) / 16;
        const int64_t need = (pieces + g.T - 1) / g.T;
        g.npt = need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
        if (g.npt != 0) break;
        if (g.P == 1) return false;
        g.P /= 2;
    }
    g.buf_bytes = (int)((((g.P * rb + slack + 15) / 16) * 16 + 63) & ~(int64_t)63);
    const size_t wbuf = (size_t)2 * g.buf_bytes;
    const size_t red = (size_t)(g.P / 2) * k * sizeof(float);
    // (+16 in front of the weight buffers and +16 after them: the unaligned
    // field reads may touch one dword before or past a row)
    g.lds_bytes = (wbuf + 16 > red ? wbuf + 16 : red) + 16;
    if (g.lds_bytes > 160 * 1024) return false;
    // enough batches per workgroup (8) to pipeline the copies, at least one
    // workgroup per compute unit, at most T_MAX_GRID partials
    const int64_t batches = (rows + g.P - 1) / g.P;
    int64_t want = batches / 8 > num_cu ? batches / 8 : num_cu;
    if (want > batches) want = batches;
    g.grid = (int)(want < T_MAX_GRID ? want : T_MAX_GRID);
    g.num_cu = num_cu;
    *out = g;
    return true;
}

namespace {

template <class F, int UPL, int NPT>
hipError_t launch_t_k(const GemvTPlan &p, const uint8_t *W, const float *dy, float *dx,
                      int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                      int64_t j_end, int accumulate, ScratchLender &lender,
                      hipStream_t s) {
    auto kernel = qmv_gemv_t_staged<F, UPL, NPT>;
    if (p.lds_bytes > 64 * 1024 &&
        hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds_bytes) != hipSuccess)
        return hipGetLastError();
    int res = resident_per_cu(kernel, p.T, p.lds_bytes);
    if (res > STREAM_PER_CU) res = STREAM_PER_CU;
    const int64_t cap = (int64_t)p.num_cu * res;
    const int grid = (int)(p.grid < cap ? p.grid : cap);
    void *buf = nullptr;
    hipEvent_t done = nullptr;
    hipError_t e = lender.acquire((size_t)grid * k * sizeof(float), s, &buf, &done);
    if (e != hipSuccess) return e;
    float *part = (float *)buf;
    for (int64_t t = 0; t < m && e == hipSuccess; t++) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(p.T), p.lds_bytes, s, W, dy + t * n, part, k,
                           row_bytes, j_start, j_end, p.U, p.L, p.P, p.buf_bytes);
        e = hipGetLastError();
        if (e != hipSuccess) break;
        // the last reduce is the buffer's last reader
        launch_stop(qmv_gemv_t_reduce, dim3((unsigned)(k / 16)), dim3(256), 0, s,
                    t + 1 == m ? done : nullptr, part, dx + t * k, k, grid, accumulate);
        e = hipGetLastError();
    }
    const hipError_t f = lender.release(buf, s, e == hipSuccess && done && m > 0);
    return e != hipSuccess ? e : f;
}

template <class F>
hipError_t launch_t_f(const GemvTPlan &p, const uint8_t *W, const float *dy, float *dx,
                      int64_t k, int64_t n, int64_t m, int64_t rb, int64_t j0, int64_t j1,
                      int acc, ScratchLender &lender, hipStream_t s) {
    if (p.UPL == 2) {
        if (p.npt == 2) return launch_t_k<F, 2, 2>(p, W, dy, dx, k, n, m, rb, j0, j1, acc, lender, s);
        if (p.npt == 4) return launch_t_k<F, 2, 4>(p, W, dy, dx, k, n, m, rb, j0, j1, acc, lender, s);
        return launch_t_k<F, 2, 8>(p, W, dy, dx, k, n, m, rb, j0, j1, acc, lender, s);
    }
    if (p.npt == 2) return launch_t_k<F, 1, 2>(p, W, dy, dx, k, n, m, rb, j0, j1, acc, lender, s);
    if (p.npt == 4) return launch_t_k<F, 1, 4>(p, W, dy, dx, k, n, m, rb, j0, j1, acc, lender, s);
    return launch_t_k<F, 1, 8>(p, W, dy, dx, k, n, m, rb, j0, j1, acc, lender, s);
}

} // namespace

hipError_t launch_gemv_t(const GemvTPlan &p, const uint8_t *W, const float *dy, float *dx,
                         int64_t k, int64_t n, int64_t m, int64_t row_bytes, int64_t j_start,
                         int64_t j_end, int accumulate, ScratchLender &lender, hipStream_t s) {
    switch (p.fmt) {
    case FMT_Q4_0:
        return launch_t_f<UQ4_0>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end, accumulate, lender, s);
    case FMT_Q4_K:
        return launch_t_f<UQ4_K>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end, accumulate, lender, s);
    case FMT_Q6_K:
        return launch_t_f<UQ6_K>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end, accumulate, lender, s);
    case FMT_Q8_0:
        return launch_t_f<UQ8_0>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end, accumulate, lender, s);
    case FMT_Q5_0:
        return launch_t_f<UQ5_0>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end, accumulate, lender, s);
    case FMT_BF16:
        return launch_t_f<UHalf<true>>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end,
                                       accumulate, lender, s);
    case FMT_F16:
        return launch_t_f<UHalf<false>>(p, W, dy, dx, k, n, m, row_bytes, j_start, j_end,
                                        accumulate, lender, s);
    default: return hipErrorInvalidValue;
    }
}

const char *gemv_t_kernel_name(const GemvTPlan &p) {
    static const char *names[] = {"",
                                  "qmv_gemv_t_staged<f16>",
                                  "qmv_gemv_t_staged<bf16>",
                                  "qmv_gemv_t_staged<q4_0>",
                                  "qmv_gemv_t_staged<q4_k>",
                                  "qmv_gemv_t_staged<q6_k>",
                                  "qmv_gemv_t_staged<q8_0>",
                                  "qmv_gemv_t_staged<q5_0>"};
    return (p.fmt >= 1 && p.fmt <= 7) ? names[p.fmt] : "";
}

} // namespace qmv
