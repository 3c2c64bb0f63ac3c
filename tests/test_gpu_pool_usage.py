"""Which entry points take device memory per call.

The header states that the single-token and few-token GEMV family, the
per-row family, the expert-indexed product and the affine product allocate
nothing, and that the matrix-core family and the streaming transposed
product take their scratch from the library's own per-device cache, which
allocates with hipMalloc only when no cached buffer is large enough. Each
call below runs with the device's stream-ordered pool's high-water mark reset
before it and read after it (the pool a hipMallocAsync on the stream would
draw from; the probe's positive control is such an allocation of the test's
own), and the cache's reuse is seen in the device's free memory.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

pytestmark = pytest.mark.gpu

POOL_ATTR_USED_MEM_HIGH = 8  # hipMemPoolAttrUsedMemHigh


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def _pool():
    hip = ctypes.CDLL("libamdhip64.so")
    device = ctypes.c_int(0)
    assert hip.hipGetDevice(ctypes.byref(device)) == 0
    pool = ctypes.c_void_p()
    assert hip.hipDeviceGetMemPool(ctypes.byref(pool), device) == 0
    return hip, pool


def _high_after(fn):
    hip, pool = _pool()
    zero = ctypes.c_uint64(0)
    torch.cuda.synchronize()
    assert hip.hipMemPoolSetAttribute(pool, POOL_ATTR_USED_MEM_HIGH, ctypes.byref(zero)) == 0
    rc = fn()
    assert rc == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    high = ctypes.c_uint64(0)
    assert hip.hipMemPoolGetAttribute(pool, POOL_ATTR_USED_MEM_HIGH, ctypes.byref(high)) == 0
    return high.value


def _stream():
    return torch.cuda.current_stream().cuda_stream


# (format, k, n, m tokens, algo)
FORWARD = [
    (synth.Q6_K, 2560, 1024, 1, qb.QMV_ALGO_GEMV),
    (synth.Q4_K, 2048, 512, 2, qb.QMV_ALGO_GEMV),
    (synth.BF16, 1024, 512, 1, qb.QMV_ALGO_GEMV),
    (synth.Q4_0, 96, 40, 3, qb.QMV_ALGO_SIMPLE),
    (synth.Q8_0, 1024, 300, 1, qb.QMV_ALGO_AUTO),
]


@pytest.mark.parametrize("fmt,k,n,m,algo", FORWARD)
def test_forward_families_take_no_pool_memory(fmt, k, n, m, algo):
    print("case pool forward fmt=%d k=%d n=%d m=%d algo=%d" % (fmt, k, n, m, algo), flush=True)
    rng = np.random.default_rng(31 + fmt)
    W = torch.from_numpy(synth.gen_weights(fmt, rng, n, k)).cuda()
    x = torch.from_numpy(synth.gen_x(rng, m, k)).cuda()
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    high = _high_after(lambda: qb.qmv_run_ex(fmt, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n,
                                             m, 0, n, 0, _stream(), algo))
    assert high == 0


def test_expert_indexed_takes_no_pool_memory():
    k, n, E, n_pos, top_k = 512, 96, 6, 2, 2
    print("case pool expert-indexed q4_k k=%d n=%d E=%d" % (k, n, E), flush=True)
    rng = np.random.default_rng(41)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n * E, k)).cuda()
    ids = torch.tensor([0, 5, 3, 3], dtype=torch.int32, device="cuda")
    x = torch.from_numpy(synth.gen_x(rng, n_pos, k)).cuda()
    y = torch.zeros((n_pos * top_k, n), dtype=torch.float32, device="cuda")
    high = _high_after(lambda: qb.qmv_run_moe(synth.Q4_K, W.data_ptr(), ids.data_ptr(), x.data_ptr(),
                                              y.data_ptr(), k, n, E, n_pos, top_k, 0, _stream()))
    assert high == 0


def test_affine_takes_no_pool_memory():
    k, n, bits = 512, 200, 4
    print("case pool affine bits=%d k=%d n=%d" % (bits, k, n), flush=True)
    rng = np.random.default_rng(43)
    words, scales, biases = synth.gen_affine(rng, bits, n, k)
    codes = torch.from_numpy(words).cuda()
    sc = torch.from_numpy(scales).cuda()
    bi = torch.from_numpy(biases).cuda()
    x = torch.from_numpy(synth.gen_x(rng, 1, k)).cuda()
    y = torch.zeros((1, n), dtype=torch.float32, device="cuda")
    high = _high_after(lambda: qb.qmv_run_affine(bits, codes.data_ptr(), sc.data_ptr(), bi.data_ptr(),
                                                 x.data_ptr(), y.data_ptr(), k, n, 1, 0, n, 0,
                                                 _stream()))
    assert high == 0


def _own_async_allocation(nbytes):
    hip = ctypes.CDLL("libamdhip64.so")
    buf = ctypes.c_void_p()
    s = ctypes.c_void_p(_stream())
    assert hip.hipMallocAsync(ctypes.byref(buf), ctypes.c_size_t(nbytes), s) == 0
    assert hip.hipFreeAsync(buf, s) == 0
    return qb.QMV_OK


def test_probe_sees_stream_ordered_allocation():
    print("case pool probe control", flush=True)
    assert _high_after(lambda: _own_async_allocation(1 << 20)) >= 1 << 20


def test_matrix_core_and_transposed_leave_the_pool_alone():
    # their scratch comes from the library's cache, not the stream's pool
    rng = np.random.default_rng(47)
    k, n, m = 1024, 128, 32
    print("case pool scratch families q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    x = torch.from_numpy(synth.gen_x(rng, m, k)).cuda()
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    assert _high_after(lambda: qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(),
                                             k, n, m, 0, n, 0, _stream(), qb.QMV_ALGO_MFMA)) == 0
    dy = torch.from_numpy(synth.gen_x(rng, 1, n)).cuda()
    dx = torch.zeros((1, k), dtype=torch.float32, device="cuda")
    assert _high_after(lambda: qb.qmv_run_t_ex(synth.Q4_K, W.data_ptr(), dy.data_ptr(),
                                               dx.data_ptr(), k, n, 1, 0, n, 0, _stream(),
                                               qb.QMV_ALGO_GEMV)) == 0


def _empty_cache():
    # Release the binding's context reference (the only one) and take it again:
    # the last release frees the cached scratch buffers.
    torch.cuda.synchronize()
    qb.qmv_destroy()
    assert qb.qmv_create() == qb.QMV_OK, qb.qmv_last_error()


def _free_after(fn):
    torch.cuda.synchronize()
    rc = fn()
    assert rc == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_scratch_cache_grows_once_then_reuses():
    # a matrix-core request larger than any before it allocates once; the same
    # request again, and a smaller one, allocate nothing
    rng = np.random.default_rng(53)
    k, n, m_small, m_big = 8192, 64, 16, 1024
    print("case scratch cache q4_k k=%d n=%d m=%d then %d" % (k, n, m_small, m_big), flush=True)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    x = torch.from_numpy(synth.gen_x(rng, m_big, k)).cuda()
    y = torch.zeros((m_big, n), dtype=torch.float32, device="cuda")

    def call(m):
        return lambda: qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n,
                                     m, 0, n, 0, _stream(), qb.QMV_ALGO_MFMA)

    want = torch.empty_like(y)
    _empty_cache()
    free0 = _free_after(call(m_small))  # kernels loaded, a small buffer cached
    free1 = _free_after(call(m_big))
    # about m_big * k * 4.2 bytes of staging were allocated
    assert free0 - free1 >= m_big * k * 4
    want.copy_(y)
    for mm in (m_big, m_small, m_big):
        assert _free_after(call(mm)) == free1
    assert torch.equal(y.view(torch.int32), want.view(torch.int32))


def test_scratch_cache_across_streams():
    # alternating calls on two streams share the cached buffers; each result
    # equals the same call made alone
    rng = np.random.default_rng(59)
    k, n, m = 4096, 384, 256
    print("case scratch cache two streams q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    xs = [torch.from_numpy(synth.gen_x(rng, m, k)).cuda() for _ in range(4)]
    alone = []
    for x in xs:
        y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
        assert qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0, n,
                             0, _stream(), qb.QMV_ALGO_MFMA) == qb.QMV_OK
        alone.append(y)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.zeros((m, n), dtype=torch.float32, device="cuda") for _ in range(16)]
    torch.cuda.synchronize()
    for i, y in enumerate(outs):
        x = xs[i % 4]
        st = streams[i % 2]
        assert qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0, n,
                             0, st.cuda_stream, qb.QMV_ALGO_MFMA) == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    for i, y in enumerate(outs):
        assert torch.equal(y.view(torch.int32), alone[i % 4].view(torch.int32)), i


def test_scratch_cache_from_two_host_threads():
    # two host threads, each with its own stream, call the matrix-core and
    # transposed products at once; every result equals the same call made alone
    import threading

    rng = np.random.default_rng(61)
    k, n, m = 2048, 320, 96
    print("case scratch cache two threads q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    xs = [torch.from_numpy(synth.gen_x(rng, m, k)).cuda() for _ in range(2)]
    dys = [torch.from_numpy(synth.gen_x(rng, 1, n)).cuda() for _ in range(2)]

    def fwd(x, y, s):
        return qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0, n,
                             0, s, qb.QMV_ALGO_MFMA)

    def bwd(dy, dx, s):
        return qb.qmv_run_t_ex(synth.Q4_K, W.data_ptr(), dy.data_ptr(), dx.data_ptr(), k, n, 1, 0,
                               n, 0, s, qb.QMV_ALGO_GEMV)

    alone_y, alone_dx = [], []
    for i in range(2):
        y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
        dx = torch.zeros((1, k), dtype=torch.float32, device="cuda")
        assert fwd(xs[i], y, _stream()) == qb.QMV_OK
        assert bwd(dys[i], dx, _stream()) == qb.QMV_OK
        alone_y.append(y)
        alone_dx.append(dx)
    torch.cuda.synchronize()
    calls = 12
    outs = [[(torch.zeros((m, n), dtype=torch.float32, device="cuda"),
              torch.zeros((1, k), dtype=torch.float32, device="cuda")) for _ in range(calls)]
            for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = streams[i].cuda_stream
            for y, dx in outs[i]:
                rc = fwd(xs[i], y, s)
                assert rc == qb.QMV_OK, qb.qmv_last_error()
                rc = bwd(dys[i], dx, s)
                assert rc == qb.QMV_OK, qb.qmv_last_error()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for y, dx in outs[i]:
            assert torch.equal(y.view(torch.int32), alone_y[i].view(torch.int32))
            assert torch.equal(dx.view(torch.int32), alone_dx[i].view(torch.int32))


def test_scratch_cache_on_per_thread_stream():
    # hipStreamPerThread names a different stream in each thread: the cache
    # orders such calls by events rather than by the handle
    HIP_STREAM_PER_THREAD = 2
    rng = np.random.default_rng(67)
    k, n, m = 1024, 200, 64
    print("case scratch cache per-thread stream q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    x = torch.from_numpy(synth.gen_x(rng, m, k)).cuda()
    want = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    assert qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), want.data_ptr(), k, n, m, 0, n,
                         0, _stream(), qb.QMV_ALGO_MFMA) == qb.QMV_OK
    torch.cuda.synchronize()
    outs = [torch.zeros((m, n), dtype=torch.float32, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    for y in outs:
        rc = qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0, n, 0,
                           HIP_STREAM_PER_THREAD, qb.QMV_ALGO_MFMA)
        assert rc == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y.view(torch.int32), want.view(torch.int32))
