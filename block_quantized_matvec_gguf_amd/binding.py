"""ctypes binding of libqmv.so (include/qmv.h), with the same names as the C
ABI, plus `matvec`, a convenience that takes torch CUDA tensors and the
current torch stream. Argument marshalling only: every step of the product
runs in the HIP kernels behind the library. There is no CPU fallback; when the
library is missing or fails, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmv.so")

QMV_FMT_F16, QMV_FMT_BF16, QMV_FMT_Q4_0, QMV_FMT_Q4_K, QMV_FMT_Q6_K = 1, 2, 3, 4, 5
QMV_FMT_Q8_0, QMV_FMT_Q5_0 = 6, 7
QMV_ALGO_AUTO, QMV_ALGO_GEMV, QMV_ALGO_MFMA, QMV_ALGO_SIMPLE = 0, 1, 2, 3
ALGOS = {"auto": QMV_ALGO_AUTO, "gemv": QMV_ALGO_GEMV, "mfma": QMV_ALGO_MFMA,
         "simple": QMV_ALGO_SIMPLE}

QMV_OK = 0
QMV_ERR_INVALID_ARGUMENT = -1
QMV_ERR_MISALIGNED = -2
QMV_ERR_NOT_INITIALIZED = -3
QMV_ERR_NO_DEVICE = -4
QMV_ERR_UNSUPPORTED_ARCH = -5
QMV_ERR_HIP = -6
QMV_ERR_UNSUPPORTED = -7


class QmvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (qmv_status_string(status), message))
        self.status = status


_lib = None
_lock = threading.Lock()


def load(path: str | None = None):
    """Load libqmv.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("libqmv.so not built (%s): run "
                               "python -m block_quantized_matvec_gguf_amd.build" % p)
        lib = ctypes.CDLL(p)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.qmv_create.argtypes = []
        lib.qmv_create.restype = ci
        lib.qmv_destroy.argtypes = []
        lib.qmv_destroy.restype = None
        run_args = [ci, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp]
        lib.qmv_run.argtypes = run_args
        lib.qmv_run.restype = ci
        lib.qmv_run_ex.argtypes = run_args + [ci]
        lib.qmv_run_ex.restype = ci
        lib.qmv_run_noalloc.argtypes = run_args + [ci]
        lib.qmv_run_noalloc.restype = ci
        lib.qmv_weight_bytes.argtypes = [ci, i64, i64]
        lib.qmv_weight_bytes.restype = i64
        lib.qmv_last_error.argtypes = []
        lib.qmv_last_error.restype = ctypes.c_char_p
        lib.qmv_status_string.argtypes = [ci]
        lib.qmv_status_string.restype = ctypes.c_char_p
        lib.qmv_kernel_name.argtypes = [ci, i64, i64, ci]
        lib.qmv_kernel_name.restype = ctypes.c_char_p
        lib.qmv_gemv_geometry.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(i64)]
        lib.qmv_gemv_geometry.restype = ci
        lib.qmv_run_t.argtypes = run_args
        lib.qmv_run_t.restype = ci
        lib.qmv_run_t_ex.argtypes = run_args + [ci]
        lib.qmv_run_t_ex.restype = ci
        lib.qmv_t_kernel_name.argtypes = [ci, i64, ci]
        lib.qmv_t_kernel_name.restype = ctypes.c_char_p
        moe_args = [ci, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp]
        lib.qmv_run_moe.argtypes = moe_args
        lib.qmv_run_moe.restype = ci
        lib.qmv_run_moe_ex.argtypes = moe_args + [ci]
        lib.qmv_run_moe_ex.restype = ci
        lib.qmv_moe_kernel_name.argtypes = [ci, i64, ci]
        lib.qmv_moe_kernel_name.restype = ctypes.c_char_p
        lib.qmv_run_affine.argtypes = [ci, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp]
        lib.qmv_run_affine.restype = ci
        lib.qmv_affine_kernel_name.argtypes = [ci, i64]
        lib.qmv_affine_kernel_name.restype = ctypes.c_char_p
        _lib = lib
        return lib


# ---------------------------------------------------------- C-ABI mirrors

def qmv_create() -> int:
    return int(load().qmv_create())


def qmv_destroy() -> None:
    load().qmv_destroy()


def qmv_run(format: int, W: int, x: int, y: int, k: int, n: int, m_tokens: int,
            j_start: int, j_end: int, accumulate: int, stream: int | None) -> int:
    return int(load().qmv_run(format, W, x, y, k, n, m_tokens, j_start, j_end, accumulate,
                              stream))


def qmv_run_ex(format: int, W: int, x: int, y: int, k: int, n: int, m_tokens: int,
               j_start: int, j_end: int, accumulate: int, stream: int | None,
               algo: int) -> int:
    return int(load().qmv_run_ex(format, W, x, y, k, n, m_tokens, j_start, j_end, accumulate,
                                 stream, algo))


def qmv_run_noalloc(format: int, W: int, x: int, y: int, k: int, n: int, m_tokens: int,
                    j_start: int, j_end: int, accumulate: int, stream: int,
                    algo: int = QMV_ALGO_AUTO) -> int:
    return int(load().qmv_run_noalloc(format, W, x, y, k, n, m_tokens, j_start, j_end,
                                      accumulate, stream, algo))


def qmv_run_t(format: int, W: int, dy: int, dx: int, k: int, n: int, m_tokens: int,
              j_start: int, j_end: int, accumulate: int, stream: int | None) -> int:
    return int(load().qmv_run_t(format, W, dy, dx, k, n, m_tokens, j_start, j_end, accumulate,
                                stream))


def qmv_run_t_ex(format: int, W: int, dy: int, dx: int, k: int, n: int, m_tokens: int,
                 j_start: int, j_end: int, accumulate: int, stream: int | None,
                 algo: int) -> int:
    return int(load().qmv_run_t_ex(format, W, dy, dx, k, n, m_tokens, j_start, j_end,
                                   accumulate, stream, algo))


def qmv_t_kernel_name(format: int, k: int, algo: int = QMV_ALGO_AUTO) -> str:
    return load().qmv_t_kernel_name(format, k, algo).decode()


def qmv_run_moe(format: int, W: int, ids: int, x: int, y: int, k: int, n: int,
                n_experts: int, n_pos: int, top_k: int, accumulate: int,
                stream: int | None) -> int:
    return int(load().qmv_run_moe(format, W, ids, x, y, k, n, n_experts, n_pos, top_k,
                                  accumulate, stream))


def qmv_run_moe_ex(format: int, W: int, ids: int, x: int, y: int, k: int, n: int,
                   n_experts: int, n_pos: int, top_k: int, accumulate: int,
                   stream: int | None, algo: int) -> int:
    return int(load().qmv_run_moe_ex(format, W, ids, x, y, k, n, n_experts, n_pos, top_k,
                                     accumulate, stream, algo))


def qmv_moe_kernel_name(format: int, k: int, algo: int = QMV_ALGO_AUTO) -> str:
    return load().qmv_moe_kernel_name(format, k, algo).decode()


def qmv_run_affine(bits: int, codes: int, scales: int, biases: int, x: int, y: int, k: int,
                   n: int, m_tokens: int, j_start: int, j_end: int, accumulate: int,
                   stream: int | None) -> int:
    return int(load().qmv_run_affine(bits, codes, scales, biases, x, y, k, n, m_tokens,
                                     j_start, j_end, accumulate, stream))


def qmv_affine_kernel_name(bits: int, k: int) -> str:
    return load().qmv_affine_kernel_name(bits, k).decode()


def qmv_weight_bytes(format: int, k: int, n: int) -> int:
    return int(load().qmv_weight_bytes(format, k, n))


def qmv_last_error() -> str:
    return load().qmv_last_error().decode()


def qmv_status_string(status: int) -> str:
    return load().qmv_status_string(status).decode()


def qmv_kernel_name(format: int, k: int, m_tokens: int, algo: int = QMV_ALGO_AUTO) -> str:
    return load().qmv_kernel_name(format, k, m_tokens, algo).decode()


GEOMETRY_FIELDS = ("threads", "slots", "lanes", "units_per_lane", "rows_per_slot", "tokens",
                   "per_cu", "staged")


def qmv_gemv_geometry(format: int, k: int, rows: int, m_tokens: int, num_cu: int):
    """(status, dict of the streaming GEMV launch geometry or None)."""
    out = (ctypes.c_int64 * 8)()
    rc = load().qmv_gemv_geometry(format, k, rows, m_tokens, num_cu, out)
    return rc, (dict(zip(GEOMETRY_FIELDS, list(out))) if rc == QMV_OK else None)


# ------------------------------------------------------- torch convenience

_ctx_ready = False


def ensure_context() -> None:
    """qmv_create once per process; raises QmvError if no gfx950 device."""
    global _ctx_ready
    if _ctx_ready:
        return
    rc = qmv_create()
    if rc != QMV_OK:
        raise QmvError(rc, qmv_last_error())
    _ctx_ready = True


def _fmt(fmt) -> int:
    from .synth import fmt_id
    return fmt_id(fmt)


def _check_w(f, W, k, n):
    import torch
    if W.dtype != torch.uint8 or not W.is_cuda or not W.is_contiguous():
        raise ValueError("W must be a contiguous uint8 CUDA tensor")
    want = qmv_weight_bytes(f, k, n)
    if want < 0 or W.numel() != want:
        raise ValueError("W has %d bytes, expected %d for format %d k=%d n=%d"
                         % (W.numel(), want, f, k, n))


def matvec_t(fmt, W, dy, k: int, n: int, dx=None, j_start: int = 0, j_end: int | None = None,
             accumulate: bool = False, algo="auto", stream=None):
    """dx (=|+=) dy @ W[j_start:j_end] on the GPU (the transposed product).

    W as for matvec; dy: float32 CUDA tensor (m, n) or (n,); dx: float32 CUDA
    tensor (m, k) (allocated when None). Enqueued on `stream` (default:
    torch's current stream); returns dx.
    """
    import torch
    f = _fmt(fmt)
    a = ALGOS[algo] if isinstance(algo, str) else int(algo)
    if j_end is None:
        j_end = n
    _check_w(f, W, k, n)
    if dy.dtype != torch.float32 or not dy.is_cuda or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous float32 CUDA tensor")
    dy2 = dy.reshape(1, -1) if dy.dim() == 1 else dy
    if dy2.shape[1] != n:
        raise ValueError("dy has %d columns, expected n=%d" % (dy2.shape[1], n))
    m = dy2.shape[0]
    if dx is None:
        dx = torch.empty((m, k), dtype=torch.float32, device=dy.device)
    if dx.dtype != torch.float32 or not dx.is_cuda or not dx.is_contiguous() or \
            dx.numel() != m * k:
        raise ValueError("dx must be a contiguous float32 CUDA tensor of m*k elements")
    ensure_context()
    s = stream if stream is not None else torch.cuda.current_stream(dy.device)
    with torch.cuda.device(dy.device):
        rc = qmv_run_t_ex(f, W.data_ptr(), dy2.data_ptr(), dx.data_ptr(), k, n, m, j_start,
                          j_end, 1 if accumulate else 0, s.cuda_stream, a)
    if rc != QMV_OK:
        raise QmvError(rc, qmv_last_error())
    return dx


def matvec_moe(fmt, W, ids, x, k: int, n: int, n_experts: int, top_k: int, y=None,
               accumulate: bool = False, algo="auto", stream=None):
    """y (=|+=) the expert-indexed product on the GPU.

    W: uint8 CUDA tensor of n_experts * qmv_weight_bytes(fmt, k, n) bytes;
    ids: int32 or uint32-valued int32 CUDA tensor of n_pos * top_k expert
    numbers; x: float32 CUDA tensor (n_pos, k); y: float32 CUDA tensor
    (n_pos * top_k, n) (allocated when None). Returns y.
    """
    import torch
    f = _fmt(fmt)
    a = ALGOS[algo] if isinstance(algo, str) else int(algo)
    want = qmv_weight_bytes(f, k, n)
    if W.dtype != torch.uint8 or not W.is_cuda or not W.is_contiguous() or want < 0 or \
            W.numel() != want * n_experts:
        raise ValueError("W must be a contiguous uint8 CUDA tensor of n_experts * %d bytes"
                         % want)
    if ids.dtype != torch.int32 or not ids.is_cuda or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 CUDA tensor")
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    n_pos = x2.shape[0]
    if x2.shape[1] != k or ids.numel() != n_pos * top_k:
        raise ValueError("x must be (n_pos, k) and ids hold n_pos * top_k entries")
    if y is None:
        y = torch.empty((n_pos * top_k, n), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous() or \
            y.numel() != n_pos * top_k * n:
        raise ValueError("y must be a contiguous float32 CUDA tensor of n_pos*top_k*n elements")
    ensure_context()
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        rc = qmv_run_moe_ex(f, W.data_ptr(), ids.data_ptr(), x2.data_ptr(), y.data_ptr(), k, n,
                            n_experts, n_pos, top_k, 1 if accumulate else 0, s.cuda_stream, a)
    if rc != QMV_OK:
        raise QmvError(rc, qmv_last_error())
    return y


def matvec_affine(bits: int, codes, scales, biases, x, k: int, n: int, y=None,
                  j_start: int = 0, j_end: int | None = None, accumulate: bool = False,
                  stream=None):
    """y (=|+=) x @ W on the GPU for affine group-64 rows: codes, scales and
    biases are contiguous CUDA tensors of n*k*bits/8, n*k/32 and n*k/32 bytes
    (any dtype holding those bits); x float32 (m, k); y float32 (m, n)."""
    import torch
    if j_end is None:
        j_end = n
    for name, t, nb in (("codes", codes, n * k * bits // 8), ("scales", scales, n * k // 32),
                        ("biases", biases, n * k // 32)):
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() != nb:
            raise ValueError("%s must be a contiguous CUDA tensor of %d bytes" % (name, nb))
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    if x2.shape[1] != k:
        raise ValueError("x has %d columns, expected k=%d" % (x2.shape[1], k))
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous() or y.numel() != m * n:
        raise ValueError("y must be a contiguous float32 CUDA tensor of m*n elements")
    ensure_context()
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        rc = qmv_run_affine(bits, codes.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                            x2.data_ptr(), y.data_ptr(), k, n, m, j_start, j_end,
                            1 if accumulate else 0, s.cuda_stream)
    if rc != QMV_OK:
        raise QmvError(rc, qmv_last_error())
    return y


def matvec(fmt, W, x, k: int, n: int, y=None, j_start: int = 0, j_end: int | None = None,
           accumulate: bool = False, algo="auto", stream=None):
    """y (=|+=) x @ W on the GPU for rows [j_start, j_end).

    W: uint8 CUDA tensor of qmv_weight_bytes(fmt, k, n) bytes; x: float32 CUDA
    tensor (m, k) or (k,); y: float32 CUDA tensor (m, n) (allocated when
    None). Enqueued on `stream` (default: torch's current stream); returns y.
    """
    import torch
    f = _fmt(fmt)
    a = ALGOS[algo] if isinstance(algo, str) else int(algo)
    if j_end is None:
        j_end = n
    _check_w(f, W, k, n)
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    if x2.shape[1] != k:
        raise ValueError("x has %d columns, expected k=%d" % (x2.shape[1], k))
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous() or y.numel() != m * n:
        raise ValueError("y must be a contiguous float32 CUDA tensor of m*n elements")
    ensure_context()
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        rc = qmv_run_ex(f, W.data_ptr(), x2.data_ptr(), y.data_ptr(), k, n, m, j_start, j_end,
                        1 if accumulate else 0, s.cuda_stream, a)
    if rc != QMV_OK:
        raise QmvError(rc, qmv_last_error())
    return y
