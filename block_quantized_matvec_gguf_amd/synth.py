"""Seeded synthetic inputs for the block-quantized matvec.

This module only draws random numbers and lays them out as stored blocks; it
holds none of the product's arithmetic (no decoding, no dot products). Both the
GPU path's tests/benchmark and the CPU oracle consume what it produces.

Value distributions follow the five workloads the method is measured on (the
Q8_0 and Q5_0 draws mirror Q4_0's, as no measured workload uses them):

* Q4_0: per 32-weight block an f16 scale d ~ U[0.001, 0.02] and 16 uniform
  random code bytes (so every 4-bit code is uniform on 0..15).
* Q4_K: per 256-weight super-block f16 d ~ U[0.001, 0.02], f16 dmin ~
  U[0, 0.01], 12 uniform random bytes of packed scales/mins (every packed
  6-bit scale and min is then uniform on 0..63) and 128 uniform code bytes.
* Q6_K: 128 uniform ql bytes, 64 uniform qh bytes, 16 signed 8-bit scales
  uniform on -32..31 and f16 d ~ U[0.0005, 0.01].
* Q8_0: per 32-weight block f16 d ~ U[0.001, 0.02] and 32 uniform random code
  bytes (every signed 8-bit code uniform on -128..127).
* Q5_0: per 32-weight block f16 d ~ U[0.001, 0.02], a uniform random 32-bit
  word of fifth bits and 16 uniform code bytes (every 5-bit code uniform on
  0..31).
* F16 / BF16: weights ~ N(0, 0.02), the f64 draw rounded once, to nearest
  even, to the storage type.
* Affine 4-bit / 8-bit group-64 rows: uniform u32 code words and, per group,
  a bf16 scale 0.05 u + 0.01 and a bf16 bias 0.2 u' - 0.1 with u, u' ~
  U[-1, 1) (the draws of the pages' 4-bit fixture: scales in [-0.04, 0.06),
  biases in [-0.3, 0.1); rounded to nearest even where the fixture
  truncates).
* x: f32 ~ U[-1, 1].

All generators take a numpy Generator (PCG64); the named workloads use fixed
seeds. The inputs only need to be seeded and reproducible, so numpy's
generator serves; the tests that rebuild the pages' own fixtures use the
pages' byte formulas and generator instead.
"""
from __future__ import annotations

import numpy as np

F16, BF16, Q4_0, Q4_K, Q6_K, Q8_0, Q5_0 = 1, 2, 3, 4, 5, 6, 7
FORMAT_IDS = {"f16": F16, "bf16": BF16, "q4_0": Q4_0, "q4_k": Q4_K, "q6_k": Q6_K,
              "q8_0": Q8_0, "q5_0": Q5_0}
FORMAT_NAMES = {v: k for k, v in FORMAT_IDS.items()}

# weights per block, bytes per block (GGUF block sizes)
BLOCK = {F16: (1, 2), BF16: (1, 2), Q4_0: (32, 18), Q4_K: (256, 144), Q6_K: (256, 210),
         Q8_0: (32, 34), Q5_0: (32, 22)}


def fmt_id(fmt) -> int:
    if isinstance(fmt, str):
        return FORMAT_IDS[fmt.lower()]
    return int(fmt)


def row_bytes(fmt, k: int) -> int:
    qk, bb = BLOCK[fmt_id(fmt)]
    if k % qk:
        raise ValueError("k=%d is not a multiple of the block size %d" % (k, qk))
    return (k // qk) * bb


def weight_bytes(fmt, k: int, n: int) -> int:
    return row_bytes(fmt, k) * n


def _f16_bytes(values: np.ndarray) -> np.ndarray:
    """Little-endian f16 (round to nearest even) as a (..., 2) uint8 array."""
    h = np.asarray(values, dtype=np.float64).astype("<f2")
    return h.view(np.uint8).reshape(h.shape + (2,))


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """Round values to bfloat16 (nearest, ties to even) and return the 16-bit
    patterns. f64 input is rounded once, from f64 (it must be finite and zero
    or at least 2^-126 in magnitude, where bf16 keeps 8 significant bits);
    any other input is taken as f32 (finite)."""
    v = np.asarray(values)
    if v.dtype == np.float64:
        u = np.ascontiguousarray(v).view(np.uint64)
        # keep the top 8 significant bits of the f64 (bit 45 up), ties to even
        half = np.uint64((1 << 44) - 1)
        r = (u + half + ((u >> np.uint64(45)) & np.uint64(1))) & ~np.uint64((1 << 45) - 1)
        f = r.view(np.float64).astype(np.float32)  # exact: 8 significant bits
        return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    f = np.ascontiguousarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def gen_x(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    return rng.uniform(-1.0, 1.0, size=(m, k)).astype(np.float32)


def gen_f16(rng, n, k, std=0.02) -> np.ndarray:
    w = rng.normal(0.0, std, size=(n, k))  # f64, rounded once to f16
    return np.ascontiguousarray(w.astype("<f2")).view(np.uint8).reshape(-1)


def gen_bf16(rng, n, k, std=0.02) -> np.ndarray:
    w = rng.normal(0.0, std, size=(n, k))
    w[np.abs(w) < 2.0 ** -126] = 0.0  # (never drawn in practice)
    return bf16_bits(w).astype("<u2").view(np.uint8).reshape(-1)


def gen_q4_0(rng, n, k, d_range=(0.001, 0.02)) -> np.ndarray:
    nb = n * (k // 32)
    if k % 32:
        raise ValueError("Q4_0 needs k % 32 == 0")
    blk = np.empty((nb, 18), dtype=np.uint8)
    blk[:, 0:2] = _f16_bytes(rng.uniform(d_range[0], d_range[1], size=nb))
    blk[:, 2:18] = rng.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    return blk.reshape(-1)


def gen_q4_k(rng, n, k, d_range=(0.001, 0.02), dmin_range=(0.0, 0.01)) -> np.ndarray:
    if k % 256:
        raise ValueError("Q4_K needs k % 256 == 0")
    nb = n * (k // 256)
    blk = np.empty((nb, 144), dtype=np.uint8)
    blk[:, 0:2] = _f16_bytes(rng.uniform(d_range[0], d_range[1], size=nb))
    blk[:, 2:4] = _f16_bytes(rng.uniform(dmin_range[0], dmin_range[1], size=nb))
    blk[:, 4:144] = rng.integers(0, 256, size=(nb, 140), dtype=np.uint8)
    return blk.reshape(-1)


def gen_q6_k(rng, n, k, d_range=(0.0005, 0.01)) -> np.ndarray:
    if k % 256:
        raise ValueError("Q6_K needs k % 256 == 0")
    nb = n * (k // 256)
    blk = np.empty((nb, 210), dtype=np.uint8)
    blk[:, 0:192] = rng.integers(0, 256, size=(nb, 192), dtype=np.uint8)
    blk[:, 192:208] = rng.integers(-32, 32, size=(nb, 16), dtype=np.int8).view(np.uint8)
    blk[:, 208:210] = _f16_bytes(rng.uniform(d_range[0], d_range[1], size=nb))
    return blk.reshape(-1)


def gen_q8_0(rng, n, k, d_range=(0.001, 0.02)) -> np.ndarray:
    if k % 32:
        raise ValueError("Q8_0 needs k % 32 == 0")
    nb = n * (k // 32)
    blk = np.empty((nb, 34), dtype=np.uint8)
    blk[:, 0:2] = _f16_bytes(rng.uniform(d_range[0], d_range[1], size=nb))
    blk[:, 2:34] = rng.integers(0, 256, size=(nb, 32), dtype=np.uint8)
    return blk.reshape(-1)


def gen_q5_0(rng, n, k, d_range=(0.001, 0.02)) -> np.ndarray:
    if k % 32:
        raise ValueError("Q5_0 needs k % 32 == 0")
    nb = n * (k // 32)
    blk = np.empty((nb, 22), dtype=np.uint8)
    blk[:, 0:2] = _f16_bytes(rng.uniform(d_range[0], d_range[1], size=nb))
    blk[:, 2:22] = rng.integers(0, 256, size=(nb, 20), dtype=np.uint8)
    return blk.reshape(-1)


def gen_affine(rng, bits, n, k):
    """Affine group-quantized rows: uniform random u32 code words (k*bits/32
    per row) and, per group of 64, a bf16 scale 0.05 u + 0.01 and a bf16
    bias 0.2 u' - 0.1 with u, u' ~ U[-1, 1) (the pages' 4-bit fixture draws
    its scales and biases this way). Returns (words, scales, biases) as
    uint32 (n, k*bits/32), uint16 (n, k/64), uint16 (n, k/64)."""
    if bits not in (4, 8) or k % 64:
        raise ValueError("affine rows need bits 4 or 8 and k % 64 == 0")
    words = rng.integers(0, 2 ** 32, size=(n, k * bits // 32), dtype=np.uint64).astype(np.uint32)
    g = k // 64
    sc = 0.05 * rng.uniform(-1.0, 1.0, size=(n, g)) + 0.01
    bi = 0.2 * rng.uniform(-1.0, 1.0, size=(n, g)) - 0.1
    sc[np.abs(sc) < 2.0 ** -126] = 0.0  # (never drawn in practice)
    bi[np.abs(bi) < 2.0 ** -126] = 0.0
    return words, bf16_bits(sc), bf16_bits(bi)


def gen_weights(fmt, rng, n, k) -> np.ndarray:
    f = fmt_id(fmt)
    return {F16: gen_f16, BF16: gen_bf16, Q4_0: gen_q4_0, Q4_K: gen_q4_k,
            Q6_K: gen_q6_k, Q8_0: gen_q8_0, Q5_0: gen_q5_0}[f](rng, n, k)


# The measured workloads. Seeds: W stream 0x51A70000 + id, x stream 0x51A71000 + id.
WORKLOADS = {
    "q4_0_small": dict(id=1, fmt="q4_0", k=256, n=512, m=1),
    "bf16_ffn_up": dict(id=2, fmt="bf16", k=2560, n=10240, m=1),
    "f16_ffn_up": dict(id=2, fmt="f16", k=2560, n=10240, m=1),
    "q4_k_ffn_up": dict(id=3, fmt="q4_k", k=2560, n=10240, m=1),
    "q8_0_ffn_up": dict(id=6, fmt="q8_0", k=2560, n=10240, m=1),
    "q5_0_ffn_up": dict(id=7, fmt="q5_0", k=2560, n=10240, m=1),
    "q6_k_vocab_outproj": dict(id=4, fmt="q6_k", k=2560, n=262144, m=1, tiles=8),
    "q4_k_prefill": dict(id=5, fmt="q4_k", k=4096, n=14336, m=64),
    # expert-indexed decode: 64 stacked experts of n rows, 8 chosen per position
    "q4_k_moe_decode": dict(id=8, fmt="q4_k", k=2048, n=1536, m=1, experts=64, top_k=8),
    # affine group-64 rows (codes, scales and biases in three arrays)
    "affine4_ffn_up": dict(id=9, fmt="affine", bits=4, k=2560, n=10240, m=1),
    "affine8_ffn_up": dict(id=10, fmt="affine", bits=8, k=2560, n=10240, m=1),
    # the vocabulary-sized shape in other formats (streaming rate at a size
    # where launch latency does not matter)
    "q4_k_vocab": dict(id=11, fmt="q4_k", k=2560, n=262144, m=1, tiles=8),
    "q8_0_vocab": dict(id=12, fmt="q8_0", k=2560, n=262144, m=1, tiles=8),
    "bf16_vocab": dict(id=13, fmt="bf16", k=2560, n=262144, m=1, tiles=8),
    # the prefill shape in the other formats (matrix-core path)
    "q6_k_prefill": dict(id=14, fmt="q6_k", k=4096, n=14336, m=64),
    "q4_0_prefill": dict(id=15, fmt="q4_0", k=4096, n=14336, m=64),
    "q8_0_prefill": dict(id=16, fmt="q8_0", k=4096, n=14336, m=64),
    "bf16_prefill": dict(id=17, fmt="bf16", k=4096, n=14336, m=64),
    "f16_prefill": dict(id=18, fmt="f16", k=4096, n=14336, m=64),
}


def workload(name: str, n: int | None = None):
    """(fmt_id, W bytes, x (m,k) f32, spec) for a named workload. n may cap
    the row count (the first n rows of the full matrix are then generated by
    the same draws only when n is the full size; a capped n is its own draw)."""
    spec = dict(WORKLOADS[name])
    if n is not None:
        spec["n"] = n
    f = fmt_id(spec["fmt"])
    rw = np.random.default_rng(0x51A70000 + spec["id"] + (0 if n is None else 7919 * n))
    rx = np.random.default_rng(0x51A71000 + spec["id"])
    W = gen_weights(f, rw, spec["n"] * spec.get("experts", 1), spec["k"])
    x = gen_x(rx, spec["m"], spec["k"])
    return f, W, x, spec


def affine_workload(name: str):
    """(words, scales, biases, x) of a named affine workload."""
    spec = WORKLOADS[name]
    rw = np.random.default_rng(0x51A70000 + spec["id"])
    rx = np.random.default_rng(0x51A71000 + spec["id"])
    words, sc, bi = gen_affine(rw, spec["bits"], spec["n"], spec["k"])
    return words, sc, bi, gen_x(rx, spec["m"], spec["k"])


def moe_ids(spec) -> np.ndarray:
    """Seeded expert numbers of an expert-indexed workload: top_k distinct
    experts per position, int32 (n_pos * top_k,)."""
    r = np.random.default_rng(0x51A73000 + spec["id"])
    return np.concatenate([r.permutation(spec["experts"])[:spec["top_k"]]
                           for _ in range(spec["m"])]).astype(np.int32)
