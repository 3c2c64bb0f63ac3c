"""CPU oracle for the block-quantized matrix-vector product y = x @ W.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The GPU library never
loads it, and it imports nothing from the GPU package.

The arithmetic lives in ``qmv_oracle.c`` (plain C, f32 per-element decode, f64
serial accumulation; see the header of that file for the passages it follows).
This module only builds and loads that file and splits a row range across
host threads; every row is still summed serially in the C code, so results do
not depend on the thread count.

Parity against real GGUF files is unpinned: the block layouts inside Q4_K,
Q6_K and Q5_0 and the element order of Q4_0 are a reading of the ggml format,
pinned by hand-built blocks only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16, Q4_0, Q4_K, Q6_K, Q8_0, Q5_0 = 1, 2, 3, 4, 5, 6, 7
FORMAT_NAMES = {F16: "f16", BF16: "bf16", Q4_0: "q4_0", Q4_K: "q4_k", Q6_K: "q6_k",
                Q8_0: "q8_0", Q5_0: "q5_0"}

_lib = None


def build(force: bool = True) -> str:
    """Compile qmv_oracle.c with gcc into liboracle.so (no fused multiply-add
    contraction, so the f32 decode rounds exactly as written)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load an oracle shared library built from qmv_oracle.c (or from a copy
    of it) and declare its C signatures."""
    lib = ctypes.CDLL(path)
    c_i64, c_int, c_vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    for name in ("oracle_block_elems", "oracle_block_bytes"):
        getattr(lib, name).argtypes = [c_int]
        getattr(lib, name).restype = c_i64
    lib.oracle_row_bytes.argtypes = [c_int, c_i64]
    lib.oracle_row_bytes.restype = c_i64
    lib.oracle_elem.argtypes = [c_int, c_vp, c_i64]
    lib.oracle_elem.restype = ctypes.c_float
    lib.oracle_dequant_row.argtypes = [c_int, c_vp, c_i64, c_vp]
    lib.oracle_dequant_row.restype = c_int
    lib.oracle_gemv_rows.argtypes = [c_int, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64,
                                     c_vp, c_vp]
    lib.oracle_gemv_rows.restype = c_int
    lib.oracle_gemv_range.argtypes = [c_int, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                      c_vp, c_vp]
    lib.oracle_gemv_range.restype = c_int
    if hasattr(lib, "oracle_affine_gemv_rows"):
        lib.oracle_affine_elem.argtypes = [c_int, c_vp, c_vp, c_vp, c_i64]
        lib.oracle_affine_elem.restype = ctypes.c_float
        lib.oracle_affine_gemv_rows.argtypes = [c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                c_i64, c_vp, c_i64, c_vp, c_vp]
        lib.oracle_affine_gemv_rows.restype = c_int
    if hasattr(lib, "oracle_gemv_t_cols"):
        lib.oracle_gemv_t_cols.argtypes = [c_int, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                           c_vp, c_i64, c_vp, c_vp]
        lib.oracle_gemv_t_cols.restype = c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def use_library(lib):
    """Swap the library behind this module's functions (tests use it to run
    the pins against a mutated oracle); returns the previous one."""
    global _lib
    prev = _lib
    _lib = lib
    return prev


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def row_bytes(fmt: int, k: int) -> int:
    return int(_load().oracle_row_bytes(fmt, k))


def f16_to_f32(h: int) -> float:
    return float(_load().oracle_f16_to_f32(h))


def bf16_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(b))


def dequant_row(fmt: int, row: np.ndarray, k: int) -> np.ndarray:
    """Decode one row's bytes to k f32 weights."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    rb = row_bytes(fmt, k)
    if rb < 0 or row.size < rb:
        raise ValueError("bad format/k or short row")
    w = np.empty(k, dtype=np.float32)
    if _load().oracle_dequant_row(fmt, _ptr(row), k, _ptr(w)) != 0:
        raise ValueError("oracle_dequant_row failed")
    return w


def dequant(fmt: int, W: np.ndarray, k: int, n: int) -> np.ndarray:
    """Decode the whole matrix to an (n, k) f32 array."""
    rb = row_bytes(fmt, k)
    W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
    if rb < 0 or W.size < rb * n:
        raise ValueError("bad format/k or short W")
    out = np.empty((n, k), dtype=np.float32)
    for j in range(n):
        out[j] = dequant_row(fmt, W[j * rb:(j + 1) * rb], k)
    return out


def _threads(threads):
    if threads is not None:
        return max(1, int(threads))
    return max(1, min(os.cpu_count() or 1, 16))


def gemv_rows(fmt: int, W: np.ndarray, x: np.ndarray, k: int, n: int, rows,
              threads: int | None = None):
    """y, s for the listed rows: arrays of shape (m, len(rows)) in f64.

    x is (m, k) or (k,) float32. s[t, r] = sum_i |x[t,i] * w_rows[r][i]|.
    """
    lib = _load()
    W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float32)
    x2 = x.reshape(1, -1) if x.ndim == 1 else x
    m = x2.shape[0]
    if x2.shape[1] != k:
        raise ValueError("x has %d columns, expected k=%d" % (x2.shape[1], k))
    rb = row_bytes(fmt, k)
    if rb < 0 or W.size < rb * n:
        raise ValueError("bad format/k or short W")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    nr = rows.size
    y = np.empty((m, nr), dtype=np.float64)
    s = np.empty((m, nr), dtype=np.float64)
    nt = min(_threads(threads), max(1, nr))
    bounds = [nr * i // nt for i in range(nt + 1)]

    def work(i):
        a, b = bounds[i], bounds[i + 1]
        if b <= a:
            return 0
        sub = rows[a:b]
        ys = np.empty((m, b - a), dtype=np.float64)
        ss = np.empty((m, b - a), dtype=np.float64)
        rc = lib.oracle_gemv_rows(fmt, _ptr(W), _ptr(x2), k, n, m, _ptr(sub), b - a,
                                  _ptr(ys), _ptr(ss))
        if rc == 0:
            y[:, a:b] = ys
            s[:, a:b] = ss
        return rc

    if nt == 1:
        rcs = [work(0)]
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            rcs = list(ex.map(work, range(nt)))
    if any(rc != 0 for rc in rcs):
        raise ValueError("oracle_gemv_rows failed: %r" % (rcs,))
    return y, s


def gemv(fmt: int, W: np.ndarray, x: np.ndarray, k: int, n: int, j_start: int = 0,
         j_end: int | None = None, threads: int | None = None):
    """y, s for rows j_start <= j < j_end, each (m, j_end - j_start) f64."""
    if j_end is None:
        j_end = n
    return gemv_rows(fmt, W, x, k, n, np.arange(j_start, j_end, dtype=np.int64),
                     threads=threads)


def gemv_t_cols(fmt: int, W: np.ndarray, dy: np.ndarray, k: int, n: int, cols,
                j_start: int = 0, j_end: int | None = None, threads: int | None = None):
    """dx, s of the transposed product for the listed columns: arrays of shape
    (m, len(cols)) in f64, dx[t, c] = sum_{j_start <= j < j_end} dy[t, j] *
    w_j[cols[c]].

    dy is (m, n) or (n,) float32.
    """
    lib = _load()
    if j_end is None:
        j_end = n
    W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    dy2 = dy.reshape(1, -1) if dy.ndim == 1 else dy
    m = dy2.shape[0]
    if dy2.shape[1] != n:
        raise ValueError("dy has %d columns, expected n=%d" % (dy2.shape[1], n))
    rb = row_bytes(fmt, k)
    if rb < 0 or W.size < rb * n:
        raise ValueError("bad format/k or short W")
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64).reshape(-1))
    nc = cols.size
    dx = np.empty((m, nc), dtype=np.float64)
    s = np.empty((m, nc), dtype=np.float64)
    nt = min(_threads(threads), max(1, nc))
    bounds = [nc * i // nt for i in range(nt + 1)]

    def work(i):
        a, b = bounds[i], bounds[i + 1]
        if b <= a:
            return 0
        sub = np.ascontiguousarray(cols[a:b])
        ds = np.empty((m, b - a), dtype=np.float64)
        ss = np.empty((m, b - a), dtype=np.float64)
        rc = lib.oracle_gemv_t_cols(fmt, _ptr(W), _ptr(dy2), k, n, m, j_start, j_end, _ptr(sub),
                                    b - a, _ptr(ds), _ptr(ss))
        if rc == 0:
            dx[:, a:b] = ds
            s[:, a:b] = ss
        return rc

    if nt == 1:
        rcs = [work(0)]
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            rcs = list(ex.map(work, range(nt)))
    if any(rc != 0 for rc in rcs):
        raise ValueError("oracle_gemv_t_cols failed: %r" % (rcs,))
    return dx, s


def gemv_t(fmt: int, W: np.ndarray, dy: np.ndarray, k: int, n: int, j_start: int = 0,
           j_end: int | None = None, threads: int | None = None):
    """dx, s of the transposed product for all k columns, each (m, k) f64."""
    return gemv_t_cols(fmt, W, dy, k, n, np.arange(k, dtype=np.int64), j_start, j_end,
                       threads=threads)


def moe(fmt: int, W: np.ndarray, ids, x: np.ndarray, k: int, n: int, n_experts: int,
        top_k: int, threads: int | None = None):
    """y, s of the expert-indexed product, each (n_pos * top_k, n) f64.

    W stacks n_experts weight matrices of n rows ([E][n][row bytes]); ids holds
    n_pos * top_k expert numbers; x is (n_pos, k). Output row p*top_k + slot is
    x[p] @ W_e with e = ids[p*top_k + slot] (rullama 0.5.0,
    src/backend/dispatch/mod.rs, the batched expert-matmul test: each
    (position, slot) applies its own expert to x[pos]). An expert number
    outside [0, n_experts) gives a row of NaN.
    """
    rb = row_bytes(fmt, k)
    W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    x2 = np.ascontiguousarray(x, dtype=np.float32)
    x2 = x2.reshape(1, -1) if x2.ndim == 1 else x2
    if rb < 0 or W.size < rb * n * n_experts:
        raise ValueError("bad format/k or short W")
    if ids.size != x2.shape[0] * top_k:
        raise ValueError("ids must hold n_pos * top_k entries")
    slab = rb * n
    y = np.empty((ids.size, n), dtype=np.float64)
    s = np.empty((ids.size, n), dtype=np.float64)
    for r, e in enumerate(ids):
        if e < 0 or e >= n_experts:
            y[r] = np.nan
            s[r] = np.nan
            continue
        yr, sr = gemv(fmt, W[e * slab:(e + 1) * slab], x2[r // top_k], k, n, threads=threads)
        y[r] = yr[0]
        s[r] = sr[0]
    return y, s


def _affine_arrays(bits, words, scales, biases, k, n):
    words = np.ascontiguousarray(words, dtype=np.uint32).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
    biases = np.ascontiguousarray(biases, dtype=np.uint16).reshape(-1)
    if bits not in (4, 8) or k % 64 or words.size < n * k * bits // 32 or \
            scales.size < n * (k // 64) or biases.size < n * (k // 64):
        raise ValueError("bad affine shapes")
    return words, scales, biases


def affine_dequant(bits, words, scales, biases, k, n):
    """Decode affine group-quantized rows to an (n, k) f32 array."""
    lib = _load()
    words, scales, biases = _affine_arrays(bits, words, scales, biases, k, n)
    out = np.empty((n, k), dtype=np.float32)
    wpr, gpr = k * bits // 32, k // 64
    for j in range(n):
        wj, sj, bj = words[j * wpr:], scales[j * gpr:], biases[j * gpr:]
        for i in range(k):
            out[j, i] = lib.oracle_affine_elem(bits, _ptr(wj), _ptr(sj), _ptr(bj), i)
    return out


def affine_gemv(bits, words, scales, biases, x, k, n, j_start=0, j_end=None,
                threads: int | None = None):
    """y, s of the forward product over affine group-quantized weights for rows
    j_start <= j < j_end, each (m, j_end - j_start) f64."""
    lib = _load()
    if j_end is None:
        j_end = n
    words, scales, biases = _affine_arrays(bits, words, scales, biases, k, n)
    x2 = np.ascontiguousarray(x, dtype=np.float32)
    x2 = x2.reshape(1, -1) if x2.ndim == 1 else x2
    m = x2.shape[0]
    rows = np.arange(j_start, j_end, dtype=np.int64)
    nr = rows.size
    y = np.empty((m, nr), dtype=np.float64)
    s = np.empty((m, nr), dtype=np.float64)
    nt = min(_threads(threads), max(1, nr))
    bounds = [nr * i // nt for i in range(nt + 1)]

    def work(i):
        a, b = bounds[i], bounds[i + 1]
        if b <= a:
            return 0
        sub = np.ascontiguousarray(rows[a:b])
        ys = np.empty((m, b - a), dtype=np.float64)
        ss = np.empty((m, b - a), dtype=np.float64)
        rc = lib.oracle_affine_gemv_rows(bits, _ptr(words), _ptr(scales), _ptr(biases),
                                         _ptr(x2), k, n, m, _ptr(sub), b - a, _ptr(ys),
                                         _ptr(ss))
        if rc == 0:
            y[:, a:b] = ys
            s[:, a:b] = ss
        return rc

    if nt == 1:
        rcs = [work(0)]
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            rcs = list(ex.map(work, range(nt)))
    if any(rc != 0 for rc in rcs):
        raise ValueError("oracle_affine_gemv_rows failed: %r" % (rcs,))
    return y, s


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """Cosine similarity accumulated in f64; a zero norm gives 0 (a failure
    against any positive floor), as in the moeflux graph_diff_oracle tests."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    na = float(np.dot(a, a))
    nb = float(np.dot(b, b))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (np.sqrt(na) * np.sqrt(nb)))


COSINE_FLOOR = 0.9999
REL_TOL = 1e-4


def check_parity(y_gpu, y_ref, s_ref, base=None):
    """Acceptance test of one GPU result against the oracle.

    Per output: |y_gpu - y_ref| <= 1e-4 * s (plus half an f32 ulp of the
    expected value when the result was accumulated onto a base vector);
    over all outputs: cosine >= 0.9999 in f64. Outputs whose bound is 0 must be
    exactly y_ref (resp. base). Returns a dict of statistics with key "ok".
    """
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    expect = y_ref if base is None else np.asarray(base, dtype=np.float64) + y_ref
    tol = REL_TOL * s_ref
    if base is not None:
        tol = tol + np.abs(expect) * 2.0 ** -24
    err = np.abs(y_gpu - expect)
    finite = bool(np.all(np.isfinite(y_gpu)))
    within = bool(np.all(err <= tol))
    ratio = float(np.max(np.where(tol > 0, err / np.where(tol > 0, tol, 1.0),
                                  np.where(err > 0, np.inf, 0.0)))) if err.size else 0.0
    cos = cosine(y_gpu, expect) if err.size else 1.0
    all_zero = err.size > 0 and not np.any(expect) and not np.any(y_gpu)
    cos_ok = cos >= COSINE_FLOOR or all_zero or err.size == 0
    return {"ok": finite and within and cos_ok, "max_err": float(err.max()) if err.size else 0.0,
            "max_ratio": ratio, "cosine": cos, "finite": finite, "n": int(err.size)}
