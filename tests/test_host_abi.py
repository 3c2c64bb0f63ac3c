"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/qmv.h declares, and rejects bad arguments before touching a
device."""
import ctypes
import os
import re

import pytest

from block_quantized_matvec_gguf_amd import binding as qb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qb.LIB_PATH):
        from block_quantized_matvec_gguf_amd import build
        build.build()
    return qb.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qmv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for need in ("qmv_create", "qmv_run", "qmv_destroy", "qmv_run_ex", "qmv_weight_bytes",
                 "qmv_last_error", "qmv_run_t", "qmv_run_t_ex", "qmv_t_kernel_name",
                 "qmv_run_moe", "qmv_run_moe_ex", "qmv_moe_kernel_name", "qmv_run_affine",
                 "qmv_affine_kernel_name", "qmv_run_noalloc"):
        assert need in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(qb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_weight_bytes(lib):
    assert qb.qmv_weight_bytes(qb.QMV_FMT_F16, 2560, 10240) == 2560 * 10240 * 2
    assert qb.qmv_weight_bytes(qb.QMV_FMT_BF16, 64, 3) == 384
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q4_0, 256, 512) == 8 * 18 * 512
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q4_K, 2560, 10240) == 14745600
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q6_K, 2560, 262144) == 550502400
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q4_K, 4096, 14336) == 33030144
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q4_0, 48, 1) == -1
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q6_K, 128, 1) == -1
    assert qb.qmv_weight_bytes(qb.QMV_FMT_F16, 3, 1) == -1
    assert qb.qmv_weight_bytes(9, 256, 1) == -1
    assert qb.qmv_weight_bytes(8, 256, 1) == -1
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q4_0, 0, 7) == 0
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q8_0, 2560, 10240) == 80 * 34 * 10240
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q5_0, 2560, 10240) == 80 * 22 * 10240
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q8_0, 48, 1) == -1
    assert qb.qmv_weight_bytes(qb.QMV_FMT_Q5_0, 16, 1) == -1


def test_status_strings(lib):
    assert qb.qmv_status_string(0) == "QMV_OK"
    assert qb.qmv_status_string(qb.QMV_ERR_NOT_INITIALIZED) == "QMV_ERR_NOT_INITIALIZED"
    assert qb.qmv_status_string(-99) == "QMV_ERR_UNKNOWN"


def test_kernel_names(lib):
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q6_K, 2560, 1) == "qmv_gemv_staged<q6_k>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_0, 96, 1) == "qmv_simple"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_0, 96, 1, qb.QMV_ALGO_GEMV) == ""
    assert qb.qmv_kernel_name(qb.QMV_FMT_F16, 10, 1) == "qmv_simple"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_K, 300, 1) == ""
    # prefill-sized token counts go to the matrix-core kernel where it applies
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_K, 4096, 64) == "qmv_mfma<q4_k>"
    # AUTO moves to the matrix cores from 3 (Q4_K), 5 (Q8_0, F16, BF16), 6 (Q4_0,
    # Q5_0) or 8 (Q6_K) tokens
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_K, 4096, 2) == "qmv_gemv_staged<q4_k>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_K, 4096, 3) == "qmv_mfma<q4_k>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q8_0, 4096, 4) == "qmv_gemv_staged<q8_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q8_0, 4096, 5) == "qmv_mfma<q8_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_BF16, 4096, 4) == "qmv_gemv_direct<bf16>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_BF16, 4096, 5) == "qmv_mfma<bf16>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_0, 4096, 5) == "qmv_gemv_staged<q4_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_0, 4096, 6) == "qmv_mfma<q4_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q6_K, 4096, 7) == "qmv_gemv_staged<q6_k>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q6_K, 4096, 8) == "qmv_mfma<q6_k>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q4_K, 256, 1, qb.QMV_ALGO_MFMA) == "qmv_mfma<q4_k>"
    # every format has the matrix-core path for k a multiple of 256
    for f, name in ((qb.QMV_FMT_BF16, "bf16"), (qb.QMV_FMT_F16, "f16"), (qb.QMV_FMT_Q4_0, "q4_0"),
                    (qb.QMV_FMT_Q5_0, "q5_0"), (qb.QMV_FMT_Q8_0, "q8_0"),
                    (qb.QMV_FMT_Q6_K, "q6_k")):
        assert qb.qmv_kernel_name(f, 4096, 64, qb.QMV_ALGO_MFMA) == "qmv_mfma<%s>" % name
        assert qb.qmv_kernel_name(f, 2560, 16) == "qmv_mfma<%s>" % name
    assert qb.qmv_kernel_name(qb.QMV_FMT_BF16, 2496, 64, qb.QMV_ALGO_MFMA) == ""
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q8_0, 2560, 1) == "qmv_gemv_staged<q8_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q5_0, 2560, 1) == "qmv_gemv_staged<q5_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q5_0, 2560, 5) == "qmv_gemv_staged<q5_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q5_0, 2560, 6) == "qmv_mfma<q5_0>"
    assert qb.qmv_kernel_name(qb.QMV_FMT_Q8_0, 32, 1) == "qmv_simple"


def test_transposed_kernel_names(lib):
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_Q6_K, 2560) == "qmv_gemv_t_staged<q6_k>"
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_BF16, 2560) == "qmv_gemv_t_staged<bf16>"
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_Q5_0, 4096) == "qmv_gemv_t_staged<q5_0>"
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_Q4_0, 96) == "qmv_simple_t"
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_Q4_0, 96, qb.QMV_ALGO_GEMV) == ""
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_Q4_K, 4096, qb.QMV_ALGO_MFMA) == ""
    assert qb.qmv_t_kernel_name(qb.QMV_FMT_Q4_K, 300) == ""


def test_moe_kernel_names_and_errors(lib):
    assert qb.qmv_moe_kernel_name(qb.QMV_FMT_Q4_K, 2048) == "qmv_gemv_moe_staged<q4_k>"
    assert qb.qmv_moe_kernel_name(qb.QMV_FMT_F16, 2048) == "qmv_gemv_moe_direct<f16>"
    assert qb.qmv_moe_kernel_name(qb.QMV_FMT_Q8_0, 32) == "qmv_simple_moe"
    assert qb.qmv_moe_kernel_name(qb.QMV_FMT_Q8_0, 32, qb.QMV_ALGO_GEMV) == ""

    def run(**kw):
        a = dict(format=qb.QMV_FMT_Q4_K, W=0x1000, ids=0x4000, x=0x2000, y=0x3000, k=256, n=8,
                 E=4, n_pos=2, top_k=2, accumulate=0, stream=None, algo=0)
        a.update(kw)
        return qb.qmv_run_moe_ex(a["format"], a["W"], a["ids"], a["x"], a["y"], a["k"], a["n"],
                                 a["E"], a["n_pos"], a["top_k"], a["accumulate"], a["stream"],
                                 a["algo"])
    E = qb.QMV_ERR_INVALID_ARGUMENT
    assert run(format=0) == E
    assert run(k=100) == E
    assert run(top_k=-1) == E
    assert run(ids=0) == E
    assert run(algo=qb.QMV_ALGO_MFMA) == E
    assert run(ids=0x4002) == qb.QMV_ERR_MISALIGNED
    assert run(W=0x1008) == qb.QMV_ERR_MISALIGNED
    assert run(n_pos=70000, top_k=1) == qb.QMV_ERR_UNSUPPORTED
    assert run() == qb.QMV_ERR_NOT_INITIALIZED
    assert run(n_pos=0, ids=0, x=0, y=0) == qb.QMV_ERR_NOT_INITIALIZED


def test_affine_kernel_names_and_errors(lib):
    assert qb.qmv_affine_kernel_name(4, 2560) == "qmv_affine_gemv<4>"
    assert qb.qmv_affine_kernel_name(8, 64) == "qmv_affine_gemv<8>"
    assert qb.qmv_affine_kernel_name(4, 96) == ""
    assert qb.qmv_affine_kernel_name(3, 64) == ""

    def run(**kw):
        a = dict(bits=4, codes=0x1000, scales=0x2000, biases=0x3000, x=0x4000, y=0x5000, k=128,
                 n=8, m=1, j0=0, j1=8, acc=0)
        a.update(kw)
        return qb.qmv_run_affine(a["bits"], a["codes"], a["scales"], a["biases"], a["x"],
                                 a["y"], a["k"], a["n"], a["m"], a["j0"], a["j1"], a["acc"],
                                 None)
    E = qb.QMV_ERR_INVALID_ARGUMENT
    assert run(bits=2) == E
    assert run(k=96) == E
    assert run(j1=9) == E
    assert run(biases=0) == E
    assert run(codes=0x1004) == qb.QMV_ERR_MISALIGNED
    assert run(scales=0x2001) == qb.QMV_ERR_MISALIGNED
    assert run() == qb.QMV_ERR_NOT_INITIALIZED


def _run_t(**kw):
    a = dict(format=qb.QMV_FMT_Q6_K, W=0x1000, dy=0x2000, dx=0x3000, k=256, n=8, m_tokens=1,
             j_start=0, j_end=8, accumulate=0, stream=None, algo=0)
    a.update(kw)
    return qb.qmv_run_t_ex(a["format"], a["W"], a["dy"], a["dx"], a["k"], a["n"],
                           a["m_tokens"], a["j_start"], a["j_end"], a["accumulate"],
                           a["stream"], a["algo"])


def test_transposed_argument_errors_are_host_side(lib):
    E = qb.QMV_ERR_INVALID_ARGUMENT
    assert _run_t(format=0) == E
    assert _run_t(k=300) == E
    assert _run_t(j_start=5, j_end=4) == E
    assert _run_t(j_end=9) == E
    assert _run_t(accumulate=2) == E
    assert _run_t(algo=qb.QMV_ALGO_MFMA) == E
    assert _run_t(dx=0) == E
    assert _run_t(dy=0) == E
    assert _run_t(W=0x1001) == qb.QMV_ERR_MISALIGNED
    assert _run_t(dx=0x3002) == qb.QMV_ERR_MISALIGNED
    # an empty sum still writes dx (zeros) unless accumulating
    assert _run_t(j_start=3, j_end=3, W=0, dy=0) == qb.QMV_ERR_NOT_INITIALIZED
    assert _run_t(j_start=3, j_end=3, accumulate=1, dx=0) == qb.QMV_ERR_NOT_INITIALIZED


def _run(**kw):
    a = dict(format=qb.QMV_FMT_Q4_K, W=0x1000, x=0x2000, y=0x3000, k=256, n=8, m_tokens=1,
             j_start=0, j_end=8, accumulate=0, stream=None, algo=0)
    a.update(kw)
    return qb.qmv_run_ex(a["format"], a["W"], a["x"], a["y"], a["k"], a["n"], a["m_tokens"],
                         a["j_start"], a["j_end"], a["accumulate"], a["stream"], a["algo"])


def test_argument_errors_are_host_side(lib):
    E = qb.QMV_ERR_INVALID_ARGUMENT
    assert _run(format=0) == E
    assert _run(k=300) == E
    assert _run(format=qb.QMV_FMT_F16, k=7) == E
    assert _run(k=-256) == E
    assert _run(n=-1) == E
    assert _run(m_tokens=-1) == E
    assert _run(j_start=5, j_end=4) == E
    assert _run(j_end=9) == E
    assert _run(j_start=-1) == E
    assert _run(accumulate=2) == E
    assert _run(algo=7) == E
    assert _run(y=0) == E
    assert _run(W=0) == E
    assert _run(j_end=9) == E and "row range" in qb.qmv_last_error()
    assert _run(W=0x1001) == qb.QMV_ERR_MISALIGNED
    assert _run(x=0x2002) == qb.QMV_ERR_MISALIGNED
    assert _run(y=0x3001) == qb.QMV_ERR_MISALIGNED
    assert qb.qmv_last_error()


def test_noalloc_argument_errors_are_host_side(lib):
    def run(**kw):
        a = dict(format=qb.QMV_FMT_Q4_K, W=0x1000, x=0x2000, y=0x3000, k=256, n=8, m_tokens=64,
                 j_start=0, j_end=8, accumulate=0, stream=None, algo=qb.QMV_ALGO_MFMA)
        a.update(kw)
        return qb.qmv_run_noalloc(a["format"], a["W"], a["x"], a["y"], a["k"], a["n"],
                                  a["m_tokens"], a["j_start"], a["j_end"], a["accumulate"],
                                  a["stream"], a["algo"])
    E = qb.QMV_ERR_INVALID_ARGUMENT
    assert run(format=0) == E
    assert run(k=300) == E
    assert run(j_start=5, j_end=4) == E
    assert run(accumulate=2) == E
    assert run(algo=7) == E
    assert run(y=0) == E
    assert run(W=0x1001) == qb.QMV_ERR_MISALIGNED
    # valid arguments reach the initialisation check (no device is set up here)
    assert run() == qb.QMV_ERR_NOT_INITIALIZED


def test_run_before_create(lib):
    # this process never called qmv_create
    assert _run() == qb.QMV_ERR_NOT_INITIALIZED
    assert "qmv_create" in qb.qmv_last_error()
    qb.qmv_destroy()  # safe when not initialised


def test_create_without_a_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    rc = qb.qmv_create()
    assert rc in (qb.QMV_ERR_NO_DEVICE, qb.QMV_ERR_UNSUPPORTED_ARCH)
    assert _run() == qb.QMV_ERR_NOT_INITIALIZED


def test_gemv_geometry(lib):
    """Host-side launch planning of the streaming GEMV family (no device):
    5-wave workgroups of 40-lane rows are padded to 8 waves (two per SIMD, two
    per compute unit) where every compute unit stays busy; the direct kernel's
    large launches pad to 4 waves instead and take four per compute unit; row
    slots that fill 4 waves exactly take 8 from two batches per compute unit."""
    geo = qb.qmv_gemv_geometry
    rc, g = geo(qb.QMV_FMT_Q6_K, 2560, 262144, 1, 256)  # vocabulary projection
    assert rc == qb.QMV_OK
    assert g == dict(threads=512, slots=12, lanes=40, units_per_lane=1, rows_per_slot=1,
                     tokens=1, per_cu=2, staged=1)
    rc, g = geo(qb.QMV_FMT_Q4_K, 2560, 10240, 1, 256)  # k=2560 x 10240: a few batches each
    assert rc == qb.QMV_OK
    assert (g["threads"], g["slots"], g["lanes"], g["per_cu"]) == (512, 12, 40, 2)
    rc, g = geo(qb.QMV_FMT_BF16, 2560, 262144, 1, 256)  # direct kernel: 4-wave padding
    assert (g["threads"], g["slots"], g["per_cu"], g["staged"]) == (256, 6, 4, 0)
    rc, g = geo(qb.QMV_FMT_Q4_K, 4096, 14336, 2, 256)  # 64 lanes: 4 whole waves taken twice
    assert (g["threads"], g["slots"], g["lanes"], g["tokens"], g["per_cu"]) == (512, 8, 64, 2, 2)
    rc, g = geo(qb.QMV_FMT_BF16, 8192, 28672, 1, 256)  # direct kernel too
    assert (g["threads"], g["slots"], g["lanes"], g["per_cu"], g["staged"]) == (512, 4, 128, 2, 0)
    # 8 waves of whole-wave slots from two batches per compute unit on
    assert geo(qb.QMV_FMT_Q4_K, 4096, 8 * 512, 1, 256)[1]["threads"] == 512
    assert geo(qb.QMV_FMT_Q4_K, 4096, 8 * 511, 1, 256)[1]["threads"] == 256
    assert geo(qb.QMV_FMT_Q4_K, 16384, 2 * 512, 1, 256)[1]["slots"] == 2
    assert geo(qb.QMV_FMT_Q4_K, 16384, 2 * 511, 1, 256)[1]["slots"] == 1
    # 3-wave workgroups of 192-lane rows: two slots in 8 waves (a quarter idle)
    rc, g = geo(qb.QMV_FMT_Q4_K, 12288, 4096, 1, 256)
    assert (g["threads"], g["slots"], g["lanes"], g["units_per_lane"]) == (512, 2, 192, 1)
    assert geo(qb.QMV_FMT_BF16, 12288, 4096, 1, 256)[1]["threads"] == 192
    # two units per lane: rows of 192+ units, one token, 8+ batches per workgroup
    assert geo(qb.QMV_FMT_Q4_K, 28672, 8192, 1, 256)[1]["units_per_lane"] == 2
    assert geo(qb.QMV_FMT_Q4_K, 28672, 8191, 1, 256)[1]["units_per_lane"] == 1
    assert geo(qb.QMV_FMT_Q4_K, 28672, 8192, 2, 256)[1]["units_per_lane"] == 1
    assert geo(qb.QMV_FMT_BF16, 28672, 8192, 1, 256)[1]["units_per_lane"] == 1
    assert geo(qb.QMV_FMT_Q4_K, 14336, 4096, 1, 256)[1]["units_per_lane"] == 1
    # ... and only where two workgroups' staging buffers fit a compute unit
    assert geo(qb.QMV_FMT_Q6_K, 16384, 262144, 1, 256)[1]["units_per_lane"] == 1
    assert geo(qb.QMV_FMT_Q4_K, 16384, 262144, 1, 256)[1]["units_per_lane"] == 2
    # the direct kernel's 4-wave threshold: at least 4 batches per workgroup at
    # 4 per compute unit
    assert geo(qb.QMV_FMT_BF16, 2560, 6 * 4096, 1, 256)[1]["threads"] == 256
    assert geo(qb.QMV_FMT_BF16, 2560, 6 * 4096 - 6, 1, 256)[1]["threads"] == 512
    assert geo(qb.QMV_FMT_BF16, 2560, 6 * 4096 + 5, 1, 256)[1]["threads"] == 256
    assert geo(qb.QMV_FMT_Q6_K, 2560, 6 * 4096 + 5, 1, 256)[1]["threads"] == 512
    # 8-wave padding only where every compute unit stays busy
    assert geo(qb.QMV_FMT_Q4_K, 2560, 4096, 1, 256)[1]["threads"] == 320
    assert geo(qb.QMV_FMT_Q4_K, 2560, 2560, 1, 256)[1]["threads"] == 512
    # invariants over shapes
    for fmt in (qb.QMV_FMT_Q4_0, qb.QMV_FMT_Q4_K, qb.QMV_FMT_Q6_K, qb.QMV_FMT_BF16,
                qb.QMV_FMT_Q8_0, qb.QMV_FMT_Q5_0):
        for k in (256, 1024, 2304, 2560, 3072, 4096, 6144, 8192, 12288, 16384, 28672):
            for rows in (1, 7, 300, 10240, 262144):
                for m in (1, 2):
                    rc, g = geo(fmt, k, rows, m, 256)
                    assert rc == qb.QMV_OK, (fmt, k, rows, m)
                    busy = g["slots"] * g["lanes"]
                    assert busy <= g["threads"] <= 512
                    assert g["lanes"] * g["units_per_lane"] >= k // 64
                    if g["per_cu"] == 4:
                        assert g["threads"] == 256 and (256 - busy) * 8 <= 256
                    elif g["threads"] == 512 and busy < 512:
                        # 5-7 waves of row slots padded to 8 whole waves (block
                        # formats: also 3 waves, up to a quarter of the lanes idle)
                        idle_cap = 4 if g["staged"] else 8
                        assert g["per_cu"] == 2 and (512 - busy) * idle_cap <= 512 and busy > 256
                    else:
                        assert g["per_cu"] == 2 and g["threads"] == busy
                    # whole groups of 4 waves, or a workgroup below 256 threads, or
                    # one row slot of more than 256 lanes (k=28672 with one unit
                    # per lane: 448 threads)
                    assert (g["threads"] % 256 == 0 or g["threads"] <= 256 or
                            (g["slots"] == 1 and g["lanes"] > 256))
    # shapes the streaming kernels do not take, and bad arguments
    assert geo(qb.QMV_FMT_F16, 96, 10, 1, 256)[0] == qb.QMV_ERR_UNSUPPORTED
    assert geo(qb.QMV_FMT_Q4_K, 2560, 0, 1, 256)[0] == qb.QMV_ERR_INVALID_ARGUMENT
    assert geo(qb.QMV_FMT_Q4_K, 2500, 10, 1, 256)[0] == qb.QMV_ERR_INVALID_ARGUMENT
    assert geo(9, 2560, 10, 1, 256)[0] == qb.QMV_ERR_INVALID_ARGUMENT
    assert lib.qmv_gemv_geometry(qb.QMV_FMT_Q4_K, 2560, 10, 1, 256, None) == \
        qb.QMV_ERR_INVALID_ARGUMENT
