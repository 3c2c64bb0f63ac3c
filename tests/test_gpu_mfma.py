"""N-token (prefill) matrix-core kernel against the CPU oracle, through the C ABI.

Same acceptance as the GEMV tests: per output |y_gpu - y_ref| <= 1e-4 *
sum_i |x_i * w_ji| (+ half an f32 ulp of the expected value when
accumulating onto a base), cosine >= 0.9999; outputs outside the row range
keep their bits; row tiling and token tiling change no bit.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

from test_gpu_parity import SENTINEL, check_case, dev, gen, run_gpu

pytestmark = pytest.mark.gpu

Q4_K = synth.Q4_K


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


# k: one super-block (fewer than the waves that split K), a ragged split,
# the measured k; m: below, at and above one 32-token MFMA tile and a 64-token
# workgroup tile; n: ragged against the 64-row tile.
MFMA_SHAPES = [(256, 64, 64), (2304, 100, 16), (4096, 200, 33), (1024, 37, 1),
               (512, 130, 65), (768, 64, 130), (4096, 1000, 64)]


@pytest.mark.parametrize("k,n,m", MFMA_SHAPES)
def test_mfma_shapes(k, n, m):
    check_case(Q4_K, k, n, m, algo="mfma", seed=3 * k + n + m)


def test_mfma_row_range_and_accumulate():
    k, n, m = 1536, 500, 40
    check_case(Q4_K, k, n, m, algo="mfma", j0=13, j1=433, seed=11)
    check_case(Q4_K, k, n, m, algo="mfma", j0=64, j1=65, accumulate=True, seed=12)
    check_case(Q4_K, k, n, m, algo="mfma", j0=0, j1=n, accumulate=True, seed=13)


def test_mfma_auto_selects_for_prefill_sizes():
    assert qb.qmv_kernel_name(Q4_K, 4096, 64) == "qmv_mfma<q4_k>"
    check_case(Q4_K, 2048, 300, 24, algo="auto", seed=21)


def test_mfma_row_tiling_bit_exact():
    """8 row tiles: (a) all writing equals untiled; (b) tile 0 writes and the
    rest add onto zeros, equal to untiled."""
    k, n, m = 2048, 1100, 48
    W, x = gen(Q4_K, k, n, m, 31)
    Wd, xd = dev(W), dev(x)
    y_un = run_gpu(Q4_K, W, x, k, n, np.zeros((m, n), np.float32), algo="mfma", Wd=Wd, xd=xd)
    edges = [t * n // 8 for t in range(9)]
    for acc_of, init in ((lambda t: False, SENTINEL), (lambda t: t > 0, 0.0)):
        yd = dev(np.full((m, n), init, np.float32))
        for t in range(8):
            qb.matvec(Q4_K, Wd, xd, k, n, y=yd, j_start=edges[t], j_end=edges[t + 1],
                      accumulate=acc_of(t), algo="mfma")
        torch.cuda.synchronize()
        assert np.array_equal(yd.cpu().numpy().view(np.uint32), y_un.view(np.uint32))
    rows = np.arange(0, n, 7)
    yref, sref = oracle.gemv_rows(Q4_K, W, x, k, n, rows)
    assert oracle.check_parity(y_un[:, rows], yref, sref)["ok"]


def test_mfma_token_tiling_bit_exact():
    """A token's outputs do not depend on which token tile it falls in."""
    k, n, m = 1024, 200, 130
    W, x = gen(Q4_K, k, n, m, 41)
    Wd = dev(W)
    y_all = run_gpu(Q4_K, W, x, k, n, np.zeros((m, n), np.float32), algo="mfma", Wd=Wd)
    y_tail = run_gpu(Q4_K, W, x[37:], k, n, np.zeros((m - 37, n), np.float32), algo="mfma",
                     Wd=Wd)
    assert np.array_equal(y_all[37:].view(np.uint32), y_tail.view(np.uint32))
    y_one = run_gpu(Q4_K, W, x[100:101], k, n, np.zeros((1, n), np.float32), algo="mfma",
                    Wd=Wd)
    assert np.array_equal(y_all[100:101].view(np.uint32), y_one.view(np.uint32))


def test_mfma_zero_and_exact_blocks():
    """d = dmin = 0 gives exact zeros; d = 1, dmin = 0, every scale 1 and
    dyadic x make every product and partial sum exact, so the result equals
    the oracle bit for bit."""
    k, n, m = 512, 70, 20
    W, x = gen(Q4_K, k, n, m, 51)
    Wz = W.copy()
    Wz.reshape(-1, 144)[:, 0:4] = 0
    y = run_gpu(Q4_K, Wz, x, k, n, np.full((m, n), SENTINEL, np.float32), algo="mfma")
    assert not np.any(y)
    We = W.copy().reshape(-1, 144)
    We[:, 0:4] = np.array([0x00, 0x3C, 0x00, 0x00], np.uint8)  # d = 1, dmin = 0
    We[:, 4:8] = 1    # scales 0..3 = 1, high bits of scales 4..7 = 0
    We[:, 8:12] = 0   # mins 0..3 = 0
    We[:, 12:16] = 1  # scales 4..7 = 1, mins 4..7 = 0
    We = We.reshape(-1)
    xe = (np.random.default_rng(52).integers(-8, 9, size=(m, k)) / 8.0).astype(np.float32)
    y = run_gpu(Q4_K, We, xe, k, n, np.zeros((m, n), np.float32), algo="mfma")
    yref, _ = oracle.gemv(Q4_K, We, xe, k, n)
    assert np.array_equal(y.astype(np.float64), yref)


def test_mfma_large_dynamic_range_x():
    """x spread over many binades (the hi/lo split must keep each value's own
    relative precision)."""
    k, n, m = 2048, 128, 32
    rng = np.random.default_rng(61)
    W = synth.gen_q4_k(rng, n, k)
    x = (rng.uniform(-1, 1, size=(m, k)) * 2.0 ** rng.integers(-30, 30, size=(m, k)))
    check_case(Q4_K, k, n, m, algo="mfma", W=W, x=x.astype(np.float32))


def test_mfma_misaligned_x():
    """x that is 4- but not 16-byte aligned: AUTO falls back to the GEMV
    family, an explicit MFMA request is refused."""
    k, n, m = 512, 64, 32
    W, x = gen(Q4_K, k, n, m, 71)
    Wd = dev(W)
    xbuf = dev(np.concatenate([np.zeros(1, np.float32), x.reshape(-1)]))
    yd = dev(np.zeros((m, n), np.float32))
    s = torch.cuda.current_stream().cuda_stream
    rc = qb.qmv_run_ex(Q4_K, Wd.data_ptr(), xbuf.data_ptr() + 4, yd.data_ptr(), k, n, m, 0, n,
                       0, s, qb.QMV_ALGO_MFMA)
    assert rc == qb.QMV_ERR_MISALIGNED
    rc = qb.qmv_run(Q4_K, Wd.data_ptr(), xbuf.data_ptr() + 4, yd.data_ptr(), k, n, m, 0, n, 0, s)
    assert rc == qb.QMV_OK
    torch.cuda.synchronize()
    yref, sref = oracle.gemv(Q4_K, W, x, k, n)
    assert oracle.check_parity(yd.cpu().numpy(), yref, sref)["ok"]


def test_mfma_agrees_with_gemv():
    k, n, m = 3072, 256, 20
    W, x = gen(Q4_K, k, n, m, 81)
    Wd, xd = dev(W), dev(x)
    base = np.zeros((m, n), np.float32)
    y_m = run_gpu(Q4_K, W, x, k, n, base, algo="mfma", Wd=Wd, xd=xd)
    y_g = run_gpu(Q4_K, W, x, k, n, base, algo="gemv", Wd=Wd, xd=xd)
    yref, sref = oracle.gemv(Q4_K, W, x, k, n)
    assert oracle.check_parity(y_m, yref, sref)["ok"]
    assert oracle.check_parity(y_g, yref, sref)["ok"]


def test_prefill_workload_mfma():
    """The measured prefill shape, Q4_K m=64, k=4096, n=14336: all 64 tokens
    of sampled rows (both ends, tile edges, random) against the oracle."""
    f, W, x, spec = synth.workload("q4_k_prefill")
    n = spec["n"]
    rng = np.random.default_rng(91)
    rows = np.unique(np.concatenate([np.arange(70), np.arange(n - 70, n),
                                     np.arange(64, n, 64 * 37), rng.integers(0, n, 512)]))
    check_case(f, spec["k"], n, spec["m"], algo="mfma", W=W, x=x, rows=rows)
