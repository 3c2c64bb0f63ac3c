"""The process-wide context on the GPU: releasing its last reference frees the
scratch cache (after the device finishes), calls then fail as uninitialised,
and a new context serves the same calls with the same results.

The binding holds one reference for the whole test session; the test drops it
and takes it back, so later tests see the context as before.
"""
import numpy as np
import pytest
import torch

from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def test_last_destroy_frees_the_cache_and_create_restores():
    rng = np.random.default_rng(71)
    k, n, m = 4096, 128, 4096  # about 70 MB of matrix-core staging
    print("case context teardown q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    W = torch.from_numpy(synth.gen_weights(synth.Q4_K, rng, n, k)).cuda()
    x = torch.from_numpy(synth.gen_x(rng, m, k)).cuda()
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    dy = torch.from_numpy(synth.gen_x(rng, 1, n)).cuda()
    dx = torch.zeros((1, k), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def calls():
        rc = qb.qmv_run_ex(synth.Q4_K, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0, n, 0,
                           s, qb.QMV_ALGO_MFMA)
        if rc != qb.QMV_OK:
            return rc
        return qb.qmv_run_t_ex(synth.Q4_K, W.data_ptr(), dy.data_ptr(), dx.data_ptr(), k, n, 1, 0,
                               n, 0, s, qb.QMV_ALGO_GEMV)

    assert calls() == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    want_y, want_dx = y.clone(), dx.clone()
    torch.cuda.synchronize()
    before = torch.cuda.mem_get_info()[0]
    # one more reference, then both released: the last release frees the cache
    assert qb.qmv_create() == qb.QMV_OK
    qb.qmv_destroy()
    assert torch.cuda.mem_get_info()[0] == before  # not the last reference
    qb.qmv_destroy()
    try:
        freed = torch.cuda.mem_get_info()[0] - before
        assert freed >= m * k * 4, freed  # at least the staging buffer of the first call
        assert calls() == qb.QMV_ERR_NOT_INITIALIZED
    finally:
        assert qb.qmv_create() == qb.QMV_OK  # the binding's reference again
    y.zero_()
    dx.zero_()
    torch.cuda.synchronize()
    assert calls() == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), want_y.view(torch.int32))
    assert torch.equal(dx.view(torch.int32), want_dx.view(torch.int32))
