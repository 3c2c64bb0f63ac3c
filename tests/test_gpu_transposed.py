"""Transposed (backward-input) product dx = dy @ W[j_start:j_end] on the GPU
against the CPU oracle, through the C ABI.

Acceptance per output: |dx_gpu - dx_ref| <= 1e-4 * sum_j |dy_j * w_j[i]| (plus
half an f32 ulp of the expected value when accumulating onto a base), cosine
>= 0.9999. The streaming kernel is deterministic run to run; a split of the
row range into tiles (first tile writes, the others add: rullama 0.5.0,
src/backend/dispatch/mod.rs, struct MatmulBackInputParams) changes rounding
only.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

from test_gpu_parity import dev

pytestmark = pytest.mark.gpu

F16, BF16, Q4_0, Q4_K, Q6_K = synth.F16, synth.BF16, synth.Q4_0, synth.Q4_K, synth.Q6_K
Q8_0, Q5_0 = synth.Q8_0, synth.Q5_0
ALL_FORMATS = [Q4_0, Q4_K, Q6_K, BF16, F16, Q8_0, Q5_0]
SENTINEL = np.float32(-5555.5)


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def gen_t(fmt, k, n, m, seed):
    rng = np.random.default_rng(seed)
    W = synth.gen_weights(fmt, rng, n, k)
    dy = synth.gen_x(rng, m, n)
    return W, dy


def run_t(fmt, W, dy, k, n, base, algo="auto", j0=0, j1=None, accumulate=False, Wd=None,
          dyd=None):
    Wd = dev(W) if Wd is None else Wd
    dyd = dev(dy) if dyd is None else dyd
    dxd = dev(base)
    qb.matvec_t(fmt, Wd, dyd, k, n, dx=dxd, j_start=j0, j_end=j1, accumulate=accumulate,
                algo=algo)
    torch.cuda.synchronize()
    return dxd.cpu().numpy()


def check_t(fmt, k, n, m, algo="auto", j0=0, j1=None, accumulate=False, seed=1, W=None,
            dy=None, cols=None):
    print("case fmt=%s k=%d n=%d m=%d algo=%s range=[%d,%s) acc=%d"
          % (synth.FORMAT_NAMES[fmt], k, n, m, algo, j0, j1, accumulate), flush=True)
    if W is None:
        W, dy = gen_t(fmt, k, n, m, seed)
    j1 = n if j1 is None else j1
    rng = np.random.default_rng(seed + 77)
    base = (rng.uniform(-1, 1, size=(m, k)).astype(np.float32) if accumulate
            else np.full((m, k), SENTINEL, np.float32))
    dx = run_t(fmt, W, dy, k, n, base, algo, j0, j1, accumulate)
    cols = np.arange(k) if cols is None else np.asarray(cols)
    ref, s = oracle.gemv_t_cols(fmt, W, dy, k, n, cols, j0, j1)
    res = oracle.check_parity(dx[:, cols], ref, s, base=base[:, cols] if accumulate else None)
    assert res["ok"], res
    return dx, W, dy


SHAPES = [(256, 37, 1), (768, 1000, 2), (2560, 333, 1), (512, 1, 1), (1024, 4000, 1)]


@pytest.mark.parametrize("fmt", ALL_FORMATS, ids=lambda f: synth.FORMAT_NAMES[f])
@pytest.mark.parametrize("k,n,m", SHAPES)
@pytest.mark.parametrize("algo", ["gemv", "simple"])
def test_t_formats(fmt, k, n, m, algo):
    check_t(fmt, k, n, m, algo=algo, seed=k * 3 + n + m + fmt)


@pytest.mark.parametrize("fmt,k,n,m", [
    (Q4_K, 4096, 4100, 1), (Q6_K, 4096, 4103, 2), (Q8_0, 4096, 4100, 1), (Q4_0, 4096, 4100, 2),
    (Q5_0, 4096, 4101, 1), (BF16, 4096, 4100, 1), (Q4_K, 8192, 2100, 2), (Q6_K, 16384, 1030, 1)],
    ids=lambda v: str(v))
def test_t_wide_rows(fmt, k, n, m):
    """Rows of 64, 128 and 256 lanes (k = 4096, 8192, 16384) with enough rows
    that the block formats run 8 row slots of 64 lanes (4 of 128, 2 of 256)
    per workgroup; ragged last batch; every dx column against the oracle."""
    check_t(fmt, k, n, m, algo="gemv", seed=k + n + m + fmt)


@pytest.mark.parametrize("fmt", ALL_FORMATS, ids=lambda f: synth.FORMAT_NAMES[f])
def test_t_range_and_accumulate(fmt):
    k, n, m = 1280 if fmt not in (Q4_K, Q6_K) else 1536, 900, 2
    check_t(fmt, k, n, m, j0=13, j1=700, seed=5)
    check_t(fmt, k, n, m, j0=100, j1=101, accumulate=True, seed=6)
    check_t(fmt, k, n, m, j0=0, j1=n, accumulate=True, seed=7)


def test_t_empty_range():
    """An empty range is an empty sum: dx = 0, or unchanged when accumulating."""
    k, n = 512, 50
    W, dy = gen_t(Q4_K, k, n, 2, 8)
    dx = run_t(Q4_K, W, dy, k, n, np.full((2, k), SENTINEL, np.float32), j0=20, j1=20)
    assert not np.any(dx)
    base = np.full((2, k), 1.25, np.float32)
    dx = run_t(Q4_K, W, dy, k, n, base, j0=20, j1=20, accumulate=True)
    assert np.array_equal(dx, base)


def test_t_shapes_only_the_simple_kernel_covers():
    check_t(Q4_0, 96, 40, 2, seed=9)
    check_t(F16, 10, 33, 1, seed=10)
    assert qb.qmv_t_kernel_name(Q4_0, 96) == "qmv_simple_t"
    W, dy = gen_t(Q4_0, 96, 40, 1, 1)
    with pytest.raises(qb.QmvError) as e:
        run_t(Q4_0, W, dy, 96, 40, np.zeros((1, 96), np.float32), algo="gemv")
    assert e.value.status == qb.QMV_ERR_UNSUPPORTED


@pytest.mark.parametrize("fmt", [Q4_0, Q8_0, Q5_0], ids=lambda f: synth.FORMAT_NAMES[f])
def test_t_exact_32_weight_blocks(fmt):
    """d = 1 and dyadic dy: every product and partial sum is exact in f32, so
    any summation order gives the oracle's value bit for bit."""
    k, n, m = 1024, 2000, 1
    rng = np.random.default_rng(50 + fmt)
    W = synth.gen_weights(fmt, rng, n, k)
    W.reshape(-1, synth.BLOCK[fmt][1])[:, 0:2] = np.array([0x00, 0x3C], np.uint8)
    dy = (rng.integers(-8, 9, size=(m, n)) / 8.0).astype(np.float32)
    for algo in ("gemv", "simple"):
        dx = run_t(fmt, W, dy, k, n, np.zeros((m, k), np.float32), algo=algo)
        ref, _ = oracle.gemv_t(fmt, W, dy, k, n)
        assert np.array_equal(dx.astype(np.float64), ref), algo


def _lcg_bytes(count, state):
    """The byte stream of the pages' backward-input parity tests: a 32-bit
    linear congruential generator (multiplier 1664525, increment 1013904223),
    one byte (bits 16..23 of the state) per step."""
    out = np.empty(count, np.uint8)
    for i in range(count):
        state = (state * 1664525 + 1013904223) & 0xFFFFFFFF
        out[i] = (state >> 16) & 0xFF
    return out


@pytest.mark.parametrize("case", ["q4_k", "q4_0", "q6_k"])
def test_t_pages_parity_cases(case):
    """The pages' three backward-input parity cases (rullama 0.5.0,
    src/backend/dispatch/mod.rs, tests matmul_q4_k/q4_0/q6_k_backward_input
    _gpu_vs_cpu): n = 16 rows of LCG bytes with the f16 scales clamped, dy_j =
    (j - 8) / 4; the pages' bar is max_abs < 1e-3."""
    n = 16
    if case == "q4_k":
        fmt, k = Q4_K, 256
        W = _lcg_bytes(n * 144, 0xDEADBEEF).reshape(n, 144)
        W[:, 0:2] = [0x00, 0x2C]  # d = 0.0625
        W[:, 2:4] = [0x00, 0x28]  # dmin = 0.03125
    elif case == "q4_0":
        fmt, k = Q4_0, 64
        W = _lcg_bytes(n * 2 * 18, 0xBEEFF00D).reshape(n * 2, 18)
        W[:, 0:2] = [0x00, 0x2C]
    else:
        fmt, k = Q6_K, 256
        W = _lcg_bytes(n * 210, 0xCAFEBABE).reshape(n, 210)
        W[:, 208:210] = [0x00, 0x28]
    W = W.reshape(-1)
    dy = ((np.arange(n) - 8) * 0.25).astype(np.float32).reshape(1, n)
    for algo in ("gemv", "simple"):
        dx, _, _ = check_t(fmt, k, n, 1, algo=algo, W=W, dy=dy)
        ref, _ = oracle.gemv_t(fmt, W, dy, k, n)
        assert np.max(np.abs(dx - ref)) < 1e-3


def test_t_tiles_and_determinism():
    """Q6_K k=2560 over 32768 rows (one eighth of the vocabulary): untiled,
    then 8 tiles (tile 0 writes, tiles 1..7 add), both within tolerance of the
    oracle; the untiled launch repeats bit for bit."""
    fmt, k, n = Q6_K, 2560, 32768
    W, dy = gen_t(fmt, k, n, 1, 60)
    Wd, dyd = dev(W), dev(dy)
    zeros = np.zeros((1, k), np.float32)
    dx1 = run_t(fmt, W, dy, k, n, zeros, Wd=Wd, dyd=dyd)
    dx2 = run_t(fmt, W, dy, k, n, zeros, Wd=Wd, dyd=dyd)
    assert np.array_equal(dx1.view(np.uint32), dx2.view(np.uint32))
    ref, s = oracle.gemv_t(fmt, W, dy, k, n)
    assert oracle.check_parity(dx1, ref, s)["ok"]
    edges = [t * n // 8 for t in range(9)]
    dxd = dev(np.full((1, k), SENTINEL, np.float32))
    for t in range(8):
        qb.matvec_t(fmt, Wd, dyd, k, n, dx=dxd, j_start=edges[t], j_end=edges[t + 1],
                    accumulate=t > 0)
    torch.cuda.synchronize()
    res = oracle.check_parity(dxd.cpu().numpy(), ref, s)
    assert res["ok"], res


def test_t_vocab_sampled():
    """The vocabulary-sized product: Q6_K k=2560, n=262144, m=1, untiled and
    in 8 tiles, on 96 sampled columns (both ends, random) against the oracle."""
    f, W, x, spec = synth.workload("q6_k_vocab_outproj")
    k, n = spec["k"], spec["n"]
    dy = synth.gen_x(np.random.default_rng(0x51A72004), 1, n)
    Wd, dyd = dev(W), dev(dy)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(k - 16, k),
                                     np.random.default_rng(61).integers(0, k, 64)]))
    ref, s = oracle.gemv_t_cols(f, W, dy, k, n, cols)
    print("vocab transposed untiled", flush=True)
    dx = run_t(f, W, dy, k, n, np.zeros((1, k), np.float32), Wd=Wd, dyd=dyd)
    res = oracle.check_parity(dx[:, cols], ref, s)
    assert res["ok"], res
    print("vocab transposed tiled", flush=True)
    edges = [t * n // 8 for t in range(9)]
    dxd = dev(np.full((1, k), SENTINEL, np.float32))
    for t in range(8):
        qb.matvec_t(f, Wd, dyd, k, n, dx=dxd, j_start=edges[t], j_end=edges[t + 1],
                    accumulate=t > 0)
    torch.cuda.synchronize()
    res = oracle.check_parity(dxd.cpu().numpy()[:, cols], ref, s)
    assert res["ok"], res


def test_t_misaligned_dx_and_errors():
    """dx only 4-byte aligned is served; MFMA has no transposed form."""
    k, n = 512, 300
    W, dy = gen_t(Q4_K, k, n, 1, 70)
    Wd, dyd = dev(W), dev(dy)
    buf = dev(np.zeros(k + 1, np.float32))
    s = torch.cuda.current_stream().cuda_stream
    rc = qb.qmv_run_t(Q4_K, Wd.data_ptr(), dyd.data_ptr(), buf.data_ptr() + 4, k, n, 1, 0, n, 0,
                      s)
    assert rc == qb.QMV_OK
    torch.cuda.synchronize()
    ref, sref = oracle.gemv_t(Q4_K, W, dy, k, n)
    assert oracle.check_parity(buf.cpu().numpy()[1:].reshape(1, k), ref, sref)["ok"]
    rc = qb.qmv_run_t_ex(Q4_K, Wd.data_ptr(), dyd.data_ptr(), buf.data_ptr(), k, n, 1, 0, n, 0,
                         s, qb.QMV_ALGO_MFMA)
    assert rc == qb.QMV_ERR_INVALID_ARGUMENT
