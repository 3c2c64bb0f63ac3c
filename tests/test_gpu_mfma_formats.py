"""Matrix-core (N-token) path of the formats other than Q4_K, through the C
ABI, against the CPU oracle: weights v = s*q' as exact f16 hi/lo B terms
(Q4_0, Q5_0, Q8_0, Q6_K), raw f16 weights, and bf16 weights on the bf16
matrix cores against x split into two bf16 terms.

Same acceptance as every parity test: per output |y_gpu - y_ref| <= 1e-4 *
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
from test_gpu_ranges import full_range_weights

pytestmark = pytest.mark.gpu

FORMATS = [synth.Q4_0, synth.Q5_0, synth.Q8_0, synth.Q6_K, synth.F16, synth.BF16]


def names(f):
    return synth.FORMAT_NAMES[f]


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


# k: one 256-weight chunk, a ragged count of chunks (Q6_K rows then start
# off 16-byte boundaries: 2304 * 210/256 = 1890 bytes), the FFN k; m: a single
# token, below / at / above one 64-token tile; n: ragged against 64 rows.
SHAPES = [(256, 64, 16), (2304, 100, 33), (2560, 130, 64), (768, 37, 1), (512, 200, 130)]


@pytest.mark.parametrize("fmt", FORMATS, ids=names)
@pytest.mark.parametrize("k,n,m", SHAPES)
def test_mfma_format_shapes(fmt, k, n, m):
    check_case(fmt, k, n, m, algo="mfma", seed=7 * k + n + m + fmt)


@pytest.mark.parametrize("fmt", FORMATS, ids=names)
def test_mfma_format_auto_and_range(fmt):
    assert qb.qmv_kernel_name(fmt, 2560, 64) == "qmv_mfma<%s>" % names(fmt)
    check_case(fmt, 1536, 300, 40, algo="auto", j0=13, j1=277, seed=300 + fmt)
    check_case(fmt, 1536, 300, 40, algo="mfma", j0=64, j1=130, accumulate=True, seed=310 + fmt)


@pytest.mark.parametrize("fmt", FORMATS, ids=names)
def test_mfma_format_row_tiling_bit_exact(fmt):
    """Eight row tiles writing, then tile 0 writing and the rest adding onto
    zeros: both equal the untiled result bit for bit."""
    k, n, m = 1024, 700, 24
    W, x = gen(fmt, k, n, m, 400 + fmt)
    Wd, xd = dev(W), dev(x)
    y_un = run_gpu(fmt, W, x, k, n, np.zeros((m, n), np.float32), algo="mfma", Wd=Wd, xd=xd)
    edges = [t * n // 8 for t in range(9)]
    for acc_of, init in ((lambda t: False, SENTINEL), (lambda t: t > 0, 0.0)):
        yd = dev(np.full((m, n), init, np.float32))
        for t in range(8):
            qb.matvec(fmt, Wd, xd, k, n, y=yd, j_start=edges[t], j_end=edges[t + 1],
                      accumulate=acc_of(t), algo="mfma")
        torch.cuda.synchronize()
        assert np.array_equal(yd.cpu().numpy().view(np.uint32), y_un.view(np.uint32))
    yref, sref = oracle.gemv(fmt, W, x, k, n)
    assert oracle.check_parity(y_un, yref, sref)["ok"]


@pytest.mark.parametrize("fmt", [synth.Q6_K, synth.BF16], ids=names)
def test_mfma_format_token_tiling_bit_exact(fmt):
    k, n, m = 1024, 150, 130
    W, x = gen(fmt, k, n, m, 500 + fmt)
    Wd = dev(W)
    y_all = run_gpu(fmt, W, x, k, n, np.zeros((m, n), np.float32), algo="mfma", Wd=Wd)
    y_tail = run_gpu(fmt, W, x[37:], k, n, np.zeros((m - 37, n), np.float32), algo="mfma",
                     Wd=Wd)
    assert np.array_equal(y_all[37:].view(np.uint32), y_tail.view(np.uint32))


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q5_0, synth.Q8_0, synth.Q6_K], ids=names)
def test_mfma_format_full_range_scales(fmt):
    """Block scales of both signs and (Q6_K) every int8 scale value."""
    k, n, m = 2560, 300, 48
    rng = np.random.default_rng(600 + fmt)
    W = full_range_weights(fmt, rng, n, k)
    x = synth.gen_x(rng, m, k)
    check_case(fmt, k, n, m, algo="mfma", W=W, x=x)


@pytest.mark.parametrize("fmt", FORMATS, ids=names)
def test_mfma_format_large_dynamic_range_x(fmt):
    k, n, m = 1024, 96, 20
    rng = np.random.default_rng(700 + fmt)
    W = synth.gen_weights(fmt, rng, n, k)
    x = (rng.uniform(-1, 1, size=(m, k)) * 2.0 ** rng.integers(-30, 30, size=(m, k)))
    check_case(fmt, k, n, m, algo="mfma", W=W, x=x.astype(np.float32))


@pytest.mark.parametrize("fmt", FORMATS, ids=names)
def test_mfma_format_agrees_with_gemv(fmt):
    k, n, m = 2560, 256, 20
    W, x = gen(fmt, k, n, m, 800 + fmt)
    Wd, xd = dev(W), dev(x)
    base = np.zeros((m, n), np.float32)
    y_m = run_gpu(fmt, W, x, k, n, base, algo="mfma", Wd=Wd, xd=xd)
    y_g = run_gpu(fmt, W, x, k, n, base, algo="gemv", Wd=Wd, xd=xd)
    yref, sref = oracle.gemv(fmt, W, x, k, n)
    assert oracle.check_parity(y_m, yref, sref)["ok"]
    assert oracle.check_parity(y_g, yref, sref)["ok"]


@pytest.mark.parametrize("fmt", [synth.Q4_K] + FORMATS, ids=names)
def test_mfma_one_token_tile_equals_two(fmt):
    """Calls of at most 32 tokens run one 32-token tile per workgroup; each
    token's sums are the same operations as in a two-tile call, so the 20
    tokens of a 20-token call equal, bit for bit, the first 20 of a 40-token
    call on the same x (within tolerance of the oracle through the other
    tests)."""
    k, n = 2560, 200
    print("case one tile fmt=%s k=%d n=%d" % (names(fmt), k, n), flush=True)
    W, x = gen(fmt, k, n, 40, 900 + fmt)
    Wd = dev(W)
    y40 = run_gpu(fmt, W, x, k, n, np.zeros((40, n), np.float32), algo="mfma", Wd=Wd)
    y20 = run_gpu(fmt, W, x[:20].copy(), k, n, np.zeros((20, n), np.float32), algo="mfma", Wd=Wd)
    assert np.array_equal(y20.view(np.uint32), y40[:20].view(np.uint32))
