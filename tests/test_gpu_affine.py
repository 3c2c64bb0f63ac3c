"""Affine group-64 GEMV (4-bit and 8-bit codes in u32 words, bf16 scale and
bias per group of 64; moeflux, tests/graph_diff_oracle.rs) on the GPU against
the CPU oracle, through the C ABI.

Acceptance as for qmv_run: per output |y_gpu - y_ref| <= 1e-4 *
sum_i |x_i * w_ji| (plus half an ulp when accumulating), cosine >= 0.9999;
outputs outside the row range keep their bits; tiling changes no bit.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

from test_gpu_parity import SENTINEL, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def gen_a(bits, k, n, m, seed):
    rng = np.random.default_rng(seed)
    words, sc, bi = synth.gen_affine(rng, bits, n, k)
    return words, sc, bi, synth.gen_x(rng, m, k)


def run_a(bits, words, sc, bi, x, k, n, base, j0=0, j1=None, accumulate=False):
    yd = dev(base)
    qb.matvec_affine(bits, dev(words.view(np.int32)), dev(sc.view(np.int16)),
                     dev(bi.view(np.int16)), dev(x), k, n, y=yd, j_start=j0, j_end=j1,
                     accumulate=accumulate)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def check_a(bits, k, n, m, j0=0, j1=None, accumulate=False, seed=1, arrays=None):
    print("case affine bits=%d k=%d n=%d m=%d range=[%d,%s) acc=%d"
          % (bits, k, n, m, j0, j1, accumulate), flush=True)
    words, sc, bi, x = gen_a(bits, k, n, m, seed) if arrays is None else arrays
    j1 = n if j1 is None else j1
    rng = np.random.default_rng(seed + 5)
    base = (rng.uniform(-1, 1, size=(m, n)).astype(np.float32) if accumulate
            else np.full((m, n), SENTINEL, np.float32))
    y = run_a(bits, words, sc, bi, x, k, n, base, j0, j1, accumulate)
    out = np.ones(n, bool)
    out[j0:j1] = False
    assert np.array_equal(y[:, out].view(np.uint32), base[:, out].view(np.uint32))
    ref, s = oracle.affine_gemv(bits, words, sc, bi, x, k, n, j0, j1)
    res = oracle.check_parity(y[:, j0:j1], ref, s, base=base[:, j0:j1] if accumulate else None)
    assert res["ok"], res
    return y


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("k,n,m", [(64, 33, 1), (2560, 1000, 1), (4096, 777, 2), (1024, 300, 3),
                                   (40960, 50, 1)])
def test_affine_shapes(bits, k, n, m):
    check_a(bits, k, n, m, seed=k + n + m + bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_affine_range_accumulate_tiling(bits):
    k, n, m = 2048, 1500, 2
    arrays = gen_a(bits, k, n, m, 11 + bits)
    check_a(bits, k, n, m, j0=17, j1=1401, arrays=arrays, seed=2)
    check_a(bits, k, n, m, accumulate=True, arrays=arrays, seed=3)
    y_un = check_a(bits, k, n, m, arrays=arrays, seed=4)
    words, sc, bi, x = arrays
    edges = [0, 1, 400, 401, 999, n]
    yd = dev(np.full((m, n), SENTINEL, np.float32))
    for t in range(len(edges) - 1):
        qb.matvec_affine(bits, dev(words.view(np.int32)), dev(sc.view(np.int16)),
                         dev(bi.view(np.int16)), dev(x), k, n, y=yd, j_start=edges[t],
                         j_end=edges[t + 1])
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy().view(np.uint32), y_un.view(np.uint32))


def test_affine_golden_rows_and_exact_sums():
    """The hand-built rows of tests/golden/affine_hand_rows.txt with dyadic x:
    every product and partial sum is exact, so the GPU equals the oracle bit
    for bit (a code read from the wrong nibble or group shows)."""
    from conftest import read_golden
    g = read_golden("affine_hand_rows.txt")
    rng = np.random.default_rng(5)
    for b, w, sc, bi in zip(g["bits"], g["words"], g["scale"], g["bias"]):
        bits = int(b)
        words = np.array([int(t, 16) for t in w.split()], dtype=np.uint32)
        n, k = 40, 64
        W = np.tile(words, (n, 1))
        S = np.full((n, 1), int(sc, 16), np.uint16)
        B = np.full((n, 1), int(bi, 16), np.uint16)
        x = (rng.integers(-8, 9, size=(2, k)) / 8.0).astype(np.float32)
        y = run_a(bits, W, S, B, x, k, n, np.zeros((2, n), np.float32))
        ref, _ = oracle.affine_gemv(bits, W, S, B, x, k, n)
        assert np.array_equal(y.astype(np.float64), ref), bits


def test_affine_zero_rows_and_errors():
    k, n = 256, 64
    words, sc, bi, x = gen_a(4, k, n, 1, 9)
    sc[:] = 0
    bi[:] = 0
    y = run_a(4, words, sc, bi, x, k, n, np.full((1, n), SENTINEL, np.float32))
    assert not np.any(y)
    s = torch.cuda.current_stream().cuda_stream
    buf = dev(np.zeros(1024, np.uint8))
    assert qb.qmv_run_affine(5, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                             buf.data_ptr(), 64, 1, 1, 0, 1, 0, s) == qb.QMV_ERR_INVALID_ARGUMENT
    assert qb.qmv_run_affine(4, buf.data_ptr() + 4, buf.data_ptr(), buf.data_ptr(),
                             buf.data_ptr(), buf.data_ptr(), 64, 1, 1, 0, 1, 0,
                             s) == qb.QMV_ERR_MISALIGNED
    assert qb.qmv_run_affine(4, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                             buf.data_ptr(), 96, 1, 1, 0, 1, 0, s) == qb.QMV_ERR_INVALID_ARGUMENT


def test_affine_ffn_workload():
    """The measured affine shape: 4-bit, k=2560, n=10240, m=1, every output."""
    spec = synth.WORKLOADS["affine4_ffn_up"]
    words, sc, bi, x = synth.affine_workload("affine4_ffn_up")
    check_a(4, spec["k"], spec["n"], spec["m"], arrays=(words, sc, bi, x))


@pytest.mark.parametrize("bits", [4, 8])
def test_affine_padded_workgroups(bits):
    """k=2560 with enough rows that the launch pads its workgroups to 256
    threads (6 row slots + 16 idle lanes; the direct body's layout for 4096+
    batches): every output against the oracle,
    and every bit equal to row tiles of 2048 (unpadded launches)."""
    k, n, m = 2560, 6 * 4096 + 5, 1
    arrays = gen_a(bits, k, n, m, 31 + bits)
    y_un = check_a(bits, k, n, m, arrays=arrays, seed=6)
    words, sc, bi, x = arrays
    Wd, Sd, Bd, xd = (dev(words.view(np.int32)), dev(sc.view(np.int16)),
                      dev(bi.view(np.int16)), dev(x))
    yd = dev(np.full((m, n), SENTINEL, np.float32))
    for j0 in range(0, n, 2048):
        qb.matvec_affine(bits, Wd, Sd, Bd, xd, k, n, y=yd, j_start=j0, j_end=min(n, j0 + 2048))
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy().view(np.uint32), y_un.view(np.uint32))
