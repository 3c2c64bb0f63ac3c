"""qmv_run_noalloc, the entry point that allocates nothing, against qmv_run_ex
through the C ABI.

Both run the same kernels, so every output must be equal bit for bit (the
float32 words compared as integers), on two calls in a row with the second
smaller than the first (the fixed scratch keeps the first call's contents).
The matrix-core family must allocate no device memory (none from hipMalloc,
none from the stream's memory pool), and a request whose staging exceeds the
fixed scratch is refused on the host with y untouched.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

pytestmark = pytest.mark.gpu

SENTINEL = -7777.25
POOL_ATTR_USED_MEM_HIGH = 8  # hipMemPoolAttrUsedMemHigh


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def _case(fmt, k, n, m, seed):
    rng = np.random.default_rng(seed)
    W = torch.from_numpy(synth.gen_weights(fmt, rng, n, k)).cuda()
    x = torch.from_numpy(synth.gen_x(rng, m, k)).cuda()
    base = torch.from_numpy(rng.uniform(-1, 1, size=(m, n)).astype(np.float32)).cuda()
    return W, x, base


def _call(entry, fmt, W, x, base, k, n, m, algo, j0, j1, acc):
    y = base.clone()
    torch.cuda.synchronize()
    rc = entry(fmt, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, j0, j1, acc,
               torch.cuda.current_stream().cuda_stream, algo)
    assert rc == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    return y


# (format, algo, first call, second smaller call); a call is (k, n, m, j0, j1, accumulate)
PAIRS = [
    (synth.Q4_K, qb.QMV_ALGO_MFMA, (4096, 1000, 64, 0, 1000, 0), (1024, 300, 20, 17, 250, 1)),
    (synth.Q4_K, qb.QMV_ALGO_AUTO, (2304, 200, 130, 0, 200, 1), (512, 64, 16, 3, 61, 0)),
    (synth.Q6_K, qb.QMV_ALGO_GEMV, (2560, 512, 3, 0, 512, 0), (256, 64, 1, 5, 60, 1)),
    (synth.Q8_0, qb.QMV_ALGO_AUTO, (1024, 96, 2, 0, 96, 0), (64, 33, 1, 0, 33, 0)),
]


@pytest.mark.parametrize("fmt,algo,first,second", PAIRS)
def test_noalloc_equals_run_ex(fmt, algo, first, second):
    for i, (k, n, m, j0, j1, acc) in enumerate((first, second)):
        print("case fmt=%s algo=%d call=%d k=%d n=%d m=%d range=[%d,%d) acc=%d"
              % (synth.FORMAT_NAMES[fmt], algo, i, k, n, m, j0, j1, acc), flush=True)
        W, x, base = _case(fmt, k, n, m, seed=k + n + m + i)
        want = _call(qb.qmv_run_ex, fmt, W, x, base, k, n, m, algo, j0, j1, acc)
        got = _call(qb.qmv_run_noalloc, fmt, W, x, base, k, n, m, algo, j0, j1, acc)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))
        # outside the row range nothing moved
        assert torch.equal(got[:, :j0].view(torch.int32), base[:, :j0].view(torch.int32))
        assert torch.equal(got[:, j1:].view(torch.int32), base[:, j1:].view(torch.int32))


def _pool():
    hip = ctypes.CDLL("libamdhip64.so")
    device = ctypes.c_int(0)
    assert hip.hipGetDevice(ctypes.byref(device)) == 0
    pool = ctypes.c_void_p()
    assert hip.hipDeviceGetMemPool(ctypes.byref(pool), device) == 0
    return hip, pool


def _used_high_after(hip, pool, fn):
    zero = ctypes.c_uint64(0)
    torch.cuda.synchronize()
    assert hip.hipMemPoolSetAttribute(pool, POOL_ATTR_USED_MEM_HIGH, ctypes.byref(zero)) == 0
    fn()
    torch.cuda.synchronize()
    high = ctypes.c_uint64(0)
    assert hip.hipMemPoolGetAttribute(pool, POOL_ATTR_USED_MEM_HIGH, ctypes.byref(high)) == 0
    return high.value


def test_noalloc_takes_no_device_memory():
    k, n, m = 2048, 256, 48
    print("case allocation probe q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W, x, base = _case(synth.Q4_K, k, n, m, seed=5)
    hip, pool = _pool()
    y = base.clone()
    stream = torch.cuda.current_stream().cuda_stream

    def run(entry, mm):
        rc = entry(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, mm, 0, n, 0,
                   stream, qb.QMV_ALGO_MFMA)
        assert rc == qb.QMV_OK, qb.qmv_last_error()

    def free_after(fn):
        torch.cuda.synchronize()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.mem_get_info()[0]

    # the probe's positive control: run_ex on an empty scratch cache (the
    # context released and taken again) grows it (hipMalloc); the fixed scratch
    # serves the same request with no allocation at all, from hipMalloc or from
    # the stream's pool
    big = 16384  # about 141 MB of staging
    xb = torch.zeros((big, k), dtype=torch.float32, device="cuda")
    yb = torch.zeros((big, n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    qb.qmv_destroy()
    assert qb.qmv_create() == qb.QMV_OK, qb.qmv_last_error()
    free0 = free_after(lambda: None)
    free1 = free_after(lambda: qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), xb.data_ptr(),
                                             yb.data_ptr(), k, n, big, 0, n, 0, stream,
                                             qb.QMV_ALGO_MFMA))
    assert free0 - free1 >= big * k * 4
    run(qb.qmv_run_noalloc, m)  # kernels loaded
    assert free_after(lambda: run(qb.qmv_run_noalloc, m)) == free_after(lambda: None)
    assert _used_high_after(hip, pool, lambda: run(qb.qmv_run_noalloc, m)) == 0


def test_noalloc_refuses_oversize_staging():
    # 1024 tokens (16 tiles of 64) x 64 super-blocks need about 67 MB of staging;
    # the buffers are real and whole, though nothing may be enqueued
    k, n, m = 16384, 64, 1024
    print("case oversize q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    rng = np.random.default_rng(11)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    x = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    y = torch.full((m, n), SENTINEL, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    rc = qb.qmv_run_noalloc(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0,
                            n, 0, torch.cuda.current_stream().cuda_stream, qb.QMV_ALGO_MFMA)
    assert rc == qb.QMV_ERR_UNSUPPORTED
    assert "scratch" in qb.qmv_last_error()
    torch.cuda.synchronize()
    assert bool((y == SENTINEL).all())


def test_noalloc_auto_falls_back_when_staging_does_not_fit():
    # 8 tokens of k=65536 would need about 17.6 MB of matrix-core staging, more
    # than the fixed scratch: AUTO then runs the GEMV family, bit for bit
    # what qmv_run_ex gives with QMV_ALGO_GEMV
    k, n, m = 65536, 40, 8
    print("case auto fallback q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W, x, base = _case(synth.Q4_K, k, n, m, seed=13)
    want = _call(qb.qmv_run_ex, synth.Q4_K, W, x, base, k, n, m, qb.QMV_ALGO_GEMV, 0, n, 0)
    got = _call(qb.qmv_run_noalloc, synth.Q4_K, W, x, base, k, n, m, qb.QMV_ALGO_AUTO, 0, n, 0)
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
