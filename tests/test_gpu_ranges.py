"""Forward products on inputs that span the full range the formats and f32
allow, through the C ABI, against the CPU oracle (per output |y_gpu - y_ref|
<= 1e-4 * sum_i |x_i * w_ji|, cosine >= 0.9999):

* Q6_K int8 scales over all of -128..127 (the measured workload draws
  -32..31),
* negative block scales d (Q4_0, Q8_0, Q5_0, Q6_K) and negative d and dmin
  (Q4_K),
* x spread over many binades, x with outlier channels, x with all-zero
  stretches, and x made only of subnormal f32 values,
* stacked experts whose slices start off a 16-byte boundary.

The streaming family meets x as 24-bit integers with a power-of-two scale per
64-weight unit; these inputs exercise that representation at its edges.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

from test_gpu_parity import check_case, dev
from test_gpu_moe import check_moe

pytestmark = pytest.mark.gpu

F16, BF16, Q4_0, Q4_K, Q6_K = synth.F16, synth.BF16, synth.Q4_0, synth.Q4_K, synth.Q6_K
Q8_0, Q5_0 = synth.Q8_0, synth.Q5_0
ALL_FORMATS = [Q4_0, Q4_K, Q6_K, BF16, F16, Q8_0, Q5_0]
BLOCK_FORMATS = [Q4_0, Q4_K, Q6_K, Q8_0, Q5_0]
names = lambda f: synth.FORMAT_NAMES[f]  # noqa: E731


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def f16_bytes(v):
    return np.asarray(v, np.float64).astype("<f2").view(np.uint8).reshape(-1, 2)


def full_range_weights(fmt, rng, n, k):
    """Weights whose block scales take both signs and (Q6_K) every int8
    scale value."""
    W = synth.gen_weights(fmt, rng, n, k)
    if fmt in (F16, BF16):
        return W
    bb = synth.BLOCK[fmt][1]
    blk = W.reshape(-1, bb)
    nb = blk.shape[0]
    sign = np.where(rng.integers(0, 2, nb) == 1, -1.0, 1.0)
    if fmt == Q6_K:
        blk[:, 192:208] = rng.integers(-128, 128, size=(nb, 16)).astype(np.int8).view(np.uint8)
        blk[:, 208:210] = f16_bytes(sign * rng.uniform(0.0005, 0.01, nb))
    elif fmt == Q4_K:
        blk[:, 0:2] = f16_bytes(sign * rng.uniform(0.001, 0.02, nb))
        blk[:, 2:4] = f16_bytes(rng.uniform(-0.01, 0.01, nb))
    else:
        blk[:, 0:2] = f16_bytes(sign * rng.uniform(0.001, 0.02, nb))
    return W


@pytest.mark.parametrize("fmt", BLOCK_FORMATS, ids=names)
@pytest.mark.parametrize("k,n,m", [(2560, 700, 1), (1024, 333, 2), (6400, 97, 3)])
@pytest.mark.parametrize("algo", ["gemv", "simple"])
def test_full_range_scales(fmt, k, n, m, algo):
    rng = np.random.default_rng(1000 + fmt + k + m)
    W = full_range_weights(fmt, rng, n, k)
    x = synth.gen_x(rng, m, k)
    check_case(fmt, k, n, m, algo=algo, W=W, x=x)


def test_q6_k_extreme_scales_and_codes():
    """Q6_K blocks with every scale -128 or 127 and codes 0 or 63 (the largest
    integer products the code and scale bytes hold)."""
    k, n = 2560, 256
    rng = np.random.default_rng(1100)
    W = synth.gen_q6_k(rng, n, k)
    blk = W.reshape(-1, 210)
    nb = blk.shape[0]
    blk[:, 0:128] = np.where(rng.integers(0, 2, (nb, 128)) == 1, 0xFF, 0x00).astype(np.uint8)
    blk[:, 128:192] = np.where(rng.integers(0, 2, (nb, 64)) == 1, 0xFF, 0x00).astype(np.uint8)
    blk[:, 192:208] = np.where(rng.integers(0, 2, (nb, 16)) == 1, 0x80, 0x7F).astype(np.uint8)
    x = synth.gen_x(rng, 1, k)
    check_case(Q6_K, k, n, 1, algo="gemv", W=W, x=x)


def x_binades(rng, m, k):
    return (rng.uniform(-1, 1, size=(m, k)) * 2.0 ** rng.integers(-30, 30, size=(m, k))
            ).astype(np.float32)


def x_outliers(rng, m, k):
    x = rng.uniform(-1, 1, size=(m, k))
    ch = rng.choice(k, size=max(1, k // 100), replace=False)
    x[:, ch] *= 2000.0
    return x.astype(np.float32)


def x_zero_stretches(rng, m, k):
    x = rng.uniform(-1, 1, size=(m, k)).astype(np.float32)
    x[:, : k // 4] = 0.0
    x[:, k // 2: k // 2 + 200] = 0.0
    return x


def x_subnormal(rng, m, k):
    # every value a subnormal f32 (|x| < 2^-126), nonzero
    mant = rng.integers(1, 1 << 23, size=(m, k), dtype=np.uint32)
    sign = (rng.integers(0, 2, size=(m, k), dtype=np.uint32) << 31)
    return (mant | sign).view(np.float32)


X_KINDS = {"binades": x_binades, "outliers": x_outliers, "zero_stretches": x_zero_stretches}


@pytest.mark.parametrize("fmt", ALL_FORMATS, ids=names)
@pytest.mark.parametrize("kind", sorted(X_KINDS))
def test_x_dynamic_range(fmt, kind):
    k, n, m = 2560, 400, 2
    rng = np.random.default_rng(1200 + fmt)
    W = full_range_weights(fmt, rng, n, k)
    x = X_KINDS[kind](rng, m, k)
    check_case(fmt, k, n, m, algo="gemv", W=W, x=x)


@pytest.mark.parametrize("fmt", ALL_FORMATS, ids=names)
def test_x_subnormal(fmt):
    """Every x a subnormal f32: results far below the normal range still meet
    the bar (scaled by 2^100 on both sides, so that the reference and the
    bound are representable; the product is linear in x)."""
    k, n, m = 1024, 200, 1
    rng = np.random.default_rng(1300 + fmt)
    W = synth.gen_weights(fmt, rng, n, k)
    x = x_subnormal(rng, m, k)
    y = np.full((m, n), -1.0, np.float32)
    yd = dev(y)
    qb.matvec(fmt, dev(W), dev(x), k, n, y=yd, algo="gemv")
    torch.cuda.synchronize()
    yg = yd.cpu().numpy().astype(np.float64)
    yref, sref = oracle.gemv(fmt, W, x, k, n)
    # f32 outputs this small carry absolute rounding of up to 2^-150
    err = np.abs(yg - yref)
    assert np.all(err <= 1e-4 * sref + 2.0 ** -149), (err.max(), sref.max())


@pytest.mark.parametrize("fmt,k,n", [(Q6_K, 768, 7), (Q8_0, 64, 5), (Q4_0, 96, 3),
                                     (Q5_0, 64, 9), (Q6_K, 2560, 3)], ids=lambda v: str(v))
def test_moe_expert_slices_off_16_bytes(fmt, k, n):
    """Stacked experts whose slices (n rows of the format's row bytes) are not
    a multiple of 16 bytes, so expert e > 0 starts off a 16-byte boundary
    (Q6_K k=768 n=7: 4410 bytes per expert; Q4_K rows, 144 bytes, are
    always whole 16-byte pieces): every output against the oracle, the last
    expert included (its copy reaches the end of W)."""
    E, top_k, n_pos = 6, 3, 4
    assert (n * synth.row_bytes(fmt, k)) % 16 != 0
    rng = np.random.default_rng(1400 + fmt)
    W = synth.gen_weights(fmt, rng, n * E, k)
    x = synth.gen_x(rng, n_pos, k)
    ids = np.array([5, 0, 3, 1, 5, 2, 4, 3, 1, 5, 0, 2], np.int32)
    check_moe(fmt, W, ids, x, k, n, E, top_k)
    check_moe(fmt, W, ids, x, k, n, E, top_k, accumulate=True, seed=3)
