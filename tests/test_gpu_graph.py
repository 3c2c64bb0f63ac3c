"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

qmv_run_noalloc is the entry point for code under graph capture; qmv_run_ex
and qmv_run_t_ex, whose matrix-core and streaming transposed families take
scratch, switch to stream-ordered allocation (graph memory nodes) while their
stream is being captured. Each graph below is replayed several times, with
new inputs copied in eagerly and the device synchronised between replays, and
every replay must equal, bit for bit, the same call made eagerly on the same
inputs.
"""
import numpy as np
import pytest
import torch

from block_quantized_matvec_gguf_amd import binding as qb
from block_quantized_matvec_gguf_amd import synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def gpu_context():
    assert torch.cuda.is_available(), "the GPU tests need a visible GPU"
    qb.ensure_context()
    yield


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check_replays(call, inp, out, fresh_inputs):
    """call(stream) enqueues the product reading `inp` and writing `out`."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        rc = call(_stream())
        assert rc == qb.QMV_OK, qb.qmv_last_error()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        inp.copy_(fresh_inputs[r])
        torch.cuda.synchronize()
        want = out.clone()
        rc = call(_stream())  # eager on the same inputs
        assert rc == qb.QMV_OK, qb.qmv_last_error()
        torch.cuda.synchronize()
        want.copy_(out)
        out.fill_(-3.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), r


# (entry, format, k, n, m, algo)
FORWARD = [
    ("noalloc", synth.Q4_K, 2048, 320, 64, qb.QMV_ALGO_MFMA),
    ("noalloc", synth.Q6_K, 2560, 500, 1, qb.QMV_ALGO_GEMV),
    ("run_ex", synth.Q4_K, 1024, 256, 40, qb.QMV_ALGO_MFMA),
    ("run_ex", synth.Q8_0, 1024, 300, 2, qb.QMV_ALGO_AUTO),
]


@pytest.mark.parametrize("entry,fmt,k,n,m,algo", FORWARD)
def test_forward_graph_replays(entry, fmt, k, n, m, algo):
    print("case graph %s fmt=%s k=%d n=%d m=%d algo=%d"
          % (entry, synth.FORMAT_NAMES[fmt], k, n, m, algo), flush=True)
    rng = np.random.default_rng(k + n + m + fmt)
    W = torch.from_numpy(synth.gen_weights(fmt, rng, n, k)).cuda()
    x = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    fresh = [torch.from_numpy(synth.gen_x(rng, m, k)).cuda() for _ in range(REPLAYS)]
    fn = qb.qmv_run_noalloc if entry == "noalloc" else qb.qmv_run_ex

    def call(s):
        return fn(fmt, W.data_ptr(), x.data_ptr(), y.data_ptr(), k, n, m, 0, n, 0, s, algo)

    x.copy_(fresh[0])
    _check_replays(call, x, y, fresh)


def test_transposed_graph_replays():
    fmt, k, n, m = synth.Q4_K, 1024, 700, 2
    print("case graph run_t_ex q4_k k=%d n=%d m=%d" % (k, n, m), flush=True)
    rng = np.random.default_rng(77)
    W = torch.from_numpy(synth.gen_weights(fmt, rng, n, k)).cuda()
    dy = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    dx = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    fresh = [torch.from_numpy(synth.gen_x(rng, m, n)).cuda() for _ in range(REPLAYS)]

    def call(s):
        return qb.qmv_run_t_ex(fmt, W.data_ptr(), dy.data_ptr(), dx.data_ptr(), k, n, m, 0, n, 0,
                               s, qb.QMV_ALGO_GEMV)

    dy.copy_(fresh[0])
    _check_replays(call, dy, dx, fresh)
