"""Expert-indexed product (mixture-of-experts GEMV) on the GPU against the CPU
oracle, through the C ABI: output row p*top_k + slot is x[p] @ W_e with
e = ids[p*top_k + slot] over stacked experts (rullama 0.5.0,
src/backend/dispatch/mod.rs, the expert-matmul tests).

Acceptance as for qmv_run: per output |y_gpu - y_ref| <= 1e-4 *
sum_i |x_i * w_ji| (plus half an ulp when accumulating), cosine >= 0.9999.
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


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def run_moe(fmt, W, ids, x, k, n, E, top_k, base=None, accumulate=False, algo="auto"):
    n_pos = x.shape[0]
    base = np.zeros((n_pos * top_k, n), np.float32) if base is None else base
    yd = dev(base)
    qb.matvec_moe(fmt, dev(W), dev(np.asarray(ids, np.int32)), dev(x), k, n, E, top_k, y=yd,
                  accumulate=accumulate, algo=algo)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def check_moe(fmt, W, ids, x, k, n, E, top_k, accumulate=False, algo="auto", seed=0):
    print("case fmt=%s k=%d n=%d E=%d n_pos=%d top_k=%d algo=%s acc=%d"
          % (synth.FORMAT_NAMES[fmt], k, n, E, x.shape[0], top_k, algo, accumulate), flush=True)
    base = (np.random.default_rng(seed).uniform(-1, 1, size=(x.shape[0] * top_k, n))
            .astype(np.float32) if accumulate else None)
    y = run_moe(fmt, W, ids, x, k, n, E, top_k, base, accumulate, algo)
    ref, s = oracle.moe(fmt, W, ids, x, k, n, E, top_k)
    res = oracle.check_parity(y, ref, s, base=base)
    assert res["ok"], res
    return y, ref


def test_moe_pages_q5_0_single_position():
    """The pages' Q5_0 case: stacked experts [k=64, n=4, E=5] built from the
    test's byte formulas, x_i = sin(0.37 i), slots 0 and 1 taking experts 3
    and 1; the pages' bar is |cpu - gpu| <= 1e-3 * max(|cpu|, 1)."""
    k, n, E = 64, 4, 5
    bpr = k // 32
    W = np.zeros((E, n, bpr, 22), np.uint8)
    for e in range(E):
        for j in range(n):
            for b in range(bpr):
                d = np.float16(0.25 + ((e * 3 + j + b) % 6) * 0.2)
                W[e, j, b, 0:2] = np.frombuffer(d.tobytes(), np.uint8)
                qh = ((e * 0x9E3779B9) & 0xFFFFFFFF) ^ (j << 5) ^ b
                W[e, j, b, 2:6] = np.frombuffer(np.uint32(qh).tobytes(), np.uint8)
                for l in range(16):
                    W[e, j, b, 6 + l] = (e * 41 + j * 17 + b * 7 + l * 3) % 256
    W = W.reshape(-1)
    x = np.sin(np.arange(k, dtype=np.float32) * np.float32(0.37)).astype(np.float32)[None, :]
    for algo in ("gemv", "simple"):
        y, ref = check_moe(Q5_0, W, [3, 1], x, k, n, E, 2, algo=algo)
        assert np.all(np.abs(y - ref) <= 1e-3 * np.maximum(np.abs(ref), 1.0))


def test_moe_pages_q8_0_batched():
    """The pages' batched Q8_0 case: [k=64, n=5, E=6], 3 positions, top_k=2,
    ids (4,0) (5,2) (1,3), x_i = sin(0.41 i) over all positions."""
    k, n, E, n_pos, top_k = 64, 5, 6, 3, 2
    bpr = k // 32
    W = np.zeros((E, n, bpr, 34), np.uint8)
    for e in range(E):
        for j in range(n):
            for b in range(bpr):
                d = np.float16(0.25 + ((e * 3 + j) % 5) * 0.25)
                W[e, j, b, 0:2] = np.frombuffer(d.tobytes(), np.uint8)
                for l in range(32):
                    W[e, j, b, 2 + l] = (e * 53 + j * 19 + b * 11 + l * 7) % 256
    W = W.reshape(-1)
    x = np.sin(np.arange(n_pos * k, dtype=np.float32) * np.float32(0.41)).astype(
        np.float32).reshape(n_pos, k)
    for algo in ("gemv", "simple"):
        check_moe(Q8_0, W, [4, 0, 5, 2, 1, 3], x, k, n, E, top_k, algo=algo)


@pytest.mark.parametrize("fmt", ALL_FORMATS, ids=lambda f: synth.FORMAT_NAMES[f])
@pytest.mark.parametrize("algo", ["auto", "simple"])
def test_moe_formats(fmt, algo):
    k, n, E, n_pos, top_k = 2048, 700, 8, 2, 3
    rng = np.random.default_rng(100 + fmt)
    W = synth.gen_weights(fmt, rng, n * E, k)
    ids = np.concatenate([rng.permutation(E)[:top_k] for _ in range(n_pos)])
    x = synth.gen_x(rng, n_pos, k)
    check_moe(fmt, W, ids, x, k, n, E, top_k, algo=algo)
    check_moe(fmt, W, ids, x, k, n, E, top_k, accumulate=True, algo=algo, seed=3)


@pytest.mark.parametrize("fmt", [Q4_K, Q6_K, BF16, Q5_0], ids=lambda f: synth.FORMAT_NAMES[f])
def test_moe_rows_match_plain_product(fmt):
    """Every output row equals, bit for bit, qmv_run on that expert's matrix."""
    k, n, E, n_pos, top_k = 1536, 900, 5, 3, 2
    rng = np.random.default_rng(200 + fmt)
    W = synth.gen_weights(fmt, rng, n * E, k)
    ids = [4, 0, 2, 2, 1, 3]
    x = synth.gen_x(rng, n_pos, k)
    y = run_moe(fmt, W, ids, x, k, n, E, top_k)
    slab = qb.qmv_weight_bytes(fmt, k, n)
    for r, e in enumerate(ids):
        yr = dev(np.zeros((1, n), np.float32))
        qb.matvec(fmt, dev(W[e * slab:(e + 1) * slab]), dev(x[r // top_k]), k, n, y=yr)
        torch.cuda.synchronize()
        assert np.array_equal(yr.cpu().numpy()[0].view(np.uint32), y[r].view(np.uint32)), r


def test_moe_bad_ids_and_shapes():
    """An expert number out of range gives NaN outputs for its slot only;
    k not a multiple of 64 runs on the per-row kernel."""
    k, n, E, top_k = 512, 300, 4, 2
    rng = np.random.default_rng(7)
    W = synth.gen_weights(Q4_K, rng, n * E, k)
    x = synth.gen_x(rng, 2, k)
    ids = [1, 9, 3, 0]
    y = run_moe(Q4_K, W, ids, x, k, n, E, top_k)
    ref, s = oracle.moe(Q4_K, W, ids, x, k, n, E, top_k)
    assert np.all(np.isnan(y[1]))
    good = [0, 2, 3]
    assert oracle.check_parity(y[good], ref[good], s[good])["ok"]
    W0 = synth.gen_weights(Q4_0, rng, 40 * 3, 96)
    x0 = synth.gen_x(rng, 1, 96)
    assert qb.qmv_moe_kernel_name(Q4_0, 96) == "qmv_simple_moe"
    check_moe(Q4_0, W0, [2, 0], x0, 96, 40, 3, 2)


def test_moe_decode_workload():
    """The measured expert-indexed decode shape: Q4_K, 64 experts of
    k=2048 x n=1536, top_k=8, one position (8-wave workgroups of 16 row
    slots of 32 lanes); every output against the oracle."""
    f, W, x, spec = synth.workload("q4_k_moe_decode")
    ids = synth.moe_ids(spec)
    check_moe(f, W, ids, x, spec["k"], spec["n"], spec["experts"], spec["top_k"])


@pytest.mark.parametrize("fmt", [Q6_K, BF16], ids=lambda f: synth.FORMAT_NAMES[f])
def test_moe_padded_workgroups(fmt):
    """Experts of k=2560 x 24581 rows: the launch pads its workgroups (Q6_K:
    512 threads, 12 row slots + 32 idle lanes; BF16: 256 threads, 6 slots +
    16 idle lanes). Against the oracle, and every row
    bit-equal to qmv_run on that expert's matrix."""
    k, n, E, n_pos, top_k = 2560, 6 * 4096 + 5, 2, 1, 2
    rng = np.random.default_rng(300 + fmt)
    W = synth.gen_weights(fmt, rng, n * E, k)
    ids = [1, 0]
    x = synth.gen_x(rng, n_pos, k)
    y, _ = check_moe(fmt, W, ids, x, k, n, E, top_k)
    slab = qb.qmv_weight_bytes(fmt, k, n)
    for r, e in enumerate(ids):
        yr = dev(np.zeros((1, n), np.float32))
        qb.matvec(fmt, dev(W[e * slab:(e + 1) * slab]), dev(x[r // top_k]), k, n, y=yr)
        torch.cuda.synchronize()
        assert np.array_equal(yr.cpu().numpy()[0].view(np.uint32), y[r].view(np.uint32)), r


@pytest.mark.parametrize("fmt", [Q4_K, BF16], ids=lambda f: synth.FORMAT_NAMES[f])
def test_moe_eight_wave_workgroups(fmt):
    """Experts of k=2560 x 4000 rows: a few batches per workgroup, so the
    launch pads its 5-wave workgroups to 8 waves (12 row slots + 32 idle
    lanes). Against the oracle, and every row bit-equal to qmv_run on that
    expert's matrix."""
    k, n, E, n_pos, top_k = 2560, 4000, 3, 2, 2
    # the launch is planned over all pairs' rows
    rc, g = qb.qmv_gemv_geometry(fmt, k, n * n_pos * top_k, 1, 256)
    assert rc == qb.QMV_OK and g["threads"] == 512 and g["slots"] == 12
    rng = np.random.default_rng(310 + fmt)
    W = synth.gen_weights(fmt, rng, n * E, k)
    ids = [2, 0, 1, 2]
    x = synth.gen_x(rng, n_pos, k)
    y, _ = check_moe(fmt, W, ids, x, k, n, E, top_k)
    slab = qb.qmv_weight_bytes(fmt, k, n)
    for r, e in enumerate(ids):
        yr = dev(np.zeros((1, n), np.float32))
        qb.matvec(fmt, dev(W[e * slab:(e + 1) * slab]), dev(x[r // top_k]), k, n, y=yr)
        torch.cuda.synchronize()
        assert np.array_equal(yr.cpu().numpy()[0].view(np.uint32), y[r].view(np.uint32)), r


@pytest.mark.parametrize("fmt", [Q6_K, BF16], ids=lambda f: synth.FORMAT_NAMES[f])
def test_moe_narrow_rows_eight_waves(fmt):
    """Experts of k=2048 (32 lanes per row) x 2100 rows, 4 pairs: the
    expert-indexed launch takes its whole 4-wave workgroups of 8 row slots
    as 8-wave ones of 16 (a plain product of that many rows keeps 4 waves).
    Against the oracle, and every row bit-equal to qmv_run on that expert's
    matrix."""
    k, n, E, n_pos, top_k = 2048, 2100, 4, 2, 2
    rc, g = qb.qmv_gemv_geometry(fmt, k, n * n_pos * top_k, 1, 256)
    assert rc == qb.QMV_OK and (g["threads"], g["slots"], g["lanes"]) == (256, 8, 32)
    assert (n * n_pos * top_k + 15) // 16 >= 2 * 256
    rng = np.random.default_rng(320 + fmt)
    W = synth.gen_weights(fmt, rng, n * E, k)
    ids = [3, 1, 0, 3]
    x = synth.gen_x(rng, n_pos, k)
    y, _ = check_moe(fmt, W, ids, x, k, n, E, top_k)
    slab = qb.qmv_weight_bytes(fmt, k, n)
    for r, e in enumerate(ids):
        yr = dev(np.zeros((1, n), np.float32))
        qb.matvec(fmt, dev(W[e * slab:(e + 1) * slab]), dev(x[r // top_k]), k, n, y=yr)
        torch.cuda.synchronize()
        assert np.array_equal(yr.cpu().numpy()[0].view(np.uint32), y[r].view(np.uint32)), r
