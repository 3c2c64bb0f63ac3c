"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix: library conversions of every f16/bf16
bit pattern, hand-built blocks from ``tests/golden/`` (values derived by hand),
invariants (blocks that must decode to zero, scales that must silence exactly
their own elements), packer/unpacker round trips (the packers here are written
from the layout description, independently of the oracle's decoders), one-hot
brute force, exact small-integer products, and a factored per-block evaluation
of the same sums written with numpy.

The functions are plain so that ``test_oracle_mutants.py`` can run all of them
against deliberately broken copies of the oracle and show that each plausible
mistake is caught.
"""
from __future__ import annotations

import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from block_quantized_matvec_gguf_amd import synth  # noqa: E402

from conftest import read_golden  # noqa: E402

F16, BF16, Q4_0, Q4_K, Q6_K = oracle.F16, oracle.BF16, oracle.Q4_0, oracle.Q4_K, oracle.Q6_K
Q8_0, Q5_0 = oracle.Q8_0, oracle.Q5_0


# ------------------------------------------------------------ test packers
# Written from the layout description (value -> bytes), the inverse direction
# of the oracle's decoders.

def f16_le(v: float) -> list:
    return list(np.array([v], dtype="<f2").view(np.uint8))


def pack_q4_0(codes, d: float) -> np.ndarray:
    """codes: 32 ints 0..15 in element order."""
    codes = list(codes)
    out = f16_le(d)
    for b in range(16):
        out.append(codes[b] | (codes[16 + b] << 4))
    return np.array(out, dtype=np.uint8)


def pack_q4_k_scales(scales, mins) -> list:
    out = [0] * 12
    for j in range(4):
        out[j] = scales[j] | ((scales[j + 4] >> 4) << 6)
        out[j + 4] = mins[j] | ((mins[j + 4] >> 4) << 6)
        out[j + 8] = (scales[j + 4] & 15) | ((mins[j + 4] & 15) << 4)
    return out


def pack_q4_k(codes, scales, mins, d: float, dmin: float) -> np.ndarray:
    """codes: 256 ints 0..15 in element order."""
    out = f16_le(d) + f16_le(dmin) + pack_q4_k_scales(scales, mins)
    qs = [0] * 128
    for chunk in range(4):
        for l in range(32):
            qs[32 * chunk + l] = codes[64 * chunk + l] | (codes[64 * chunk + 32 + l] << 4)
    return np.array(out + qs, dtype=np.uint8)


def q6_k_position(e: int):
    """(half, quarter, lane) of element e of a Q6_K super-block."""
    return e // 128, (e % 128) // 32, e % 32


def q6_k_scale_slot(e: int) -> int:
    h, g, l = q6_k_position(e)
    return 8 * h + 2 * g + l // 16


def pack_q6_k(codes, scales, d: float) -> np.ndarray:
    """codes: 256 ints 0..63 in element order; scales: 16 ints -128..127."""
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        h, g, l = q6_k_position(e)
        lo, hi = codes[e] & 15, codes[e] >> 4
        p = 64 * h + 32 * (g % 2) + l
        ql[p] |= lo << (4 * (g // 2))
        qh[32 * h + l] |= hi << (2 * g)
    sc = [s & 0xFF for s in scales]
    return np.array(ql + qh + sc + f16_le(d), dtype=np.uint8)


def pack_q8_0(codes, d: float) -> np.ndarray:
    """codes: 32 ints -128..127 in element order."""
    return np.array(f16_le(d) + [c & 0xFF for c in codes], dtype=np.uint8)


def pack_q5_0(codes, d: float) -> np.ndarray:
    """codes: 32 ints 0..31 in element order."""
    codes = list(codes)
    qh = 0
    for e in range(32):
        qh |= (codes[e] >> 4) << e
    qs = [(codes[b] & 15) | ((codes[16 + b] & 15) << 4) for b in range(16)]
    return np.array(f16_le(d) + [(qh >> (8 * i)) & 0xFF for i in range(4)] + qs,
                    dtype=np.uint8)


def hexbytes(s: str) -> np.ndarray:
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)


# --------------------------------------------------------------- the pins

def pin_f16_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "f16 NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 decode differs from numpy float16"


def pin_bf16_every_pattern():
    import torch
    bits = np.arange(65536, dtype=np.int64)
    ref = torch.tensor(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f32(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 decode differs from torch bfloat16"


def pin_q4_0_golden():
    g = read_golden("q4_0_hand_block.txt")
    for b, v in zip(g["bytes"], g["values"]):
        blk = hexbytes(b)
        want = np.array([float(t) for t in v.split()], dtype=np.float64)
        got = oracle.dequant_row(Q4_0, blk, 32).astype(np.float64)
        assert np.array_equal(got, want), (got, want)
    # the packer reproduces the hand-built bytes
    codes = [l for l in range(16)] + [15 - l for l in range(16)]
    assert np.array_equal(pack_q4_0(codes, 1.0), hexbytes(g["bytes"][0]))


def pin_q4_0_zero_blocks():
    rng = np.random.default_rng(11)
    # every code 8 -> all zero whatever d is
    for d in (0.0123, -3.5, 65504.0):
        blk = pack_q4_0([8] * 32, d)
        assert not np.any(oracle.dequant_row(Q4_0, blk, 32))
    # d = 0 -> all zero whatever the codes are
    blk = pack_q4_0(list(rng.integers(0, 16, 32)), 0.0)
    assert not np.any(oracle.dequant_row(Q4_0, blk, 32))


def pin_q4_0_roundtrip():
    rng = np.random.default_rng(12)
    for _ in range(50):
        codes = [int(c) for c in rng.integers(0, 16, 32)]
        d = float(np.float16(rng.uniform(-0.1, 0.1)))
        got = oracle.dequant_row(Q4_0, pack_q4_0(codes, d), 32)
        want = np.float32(d) * (np.array(codes, dtype=np.float32) - np.float32(8))
        assert np.array_equal(got, want)


def pin_q4_k_golden_scales():
    g = read_golden("q4_k_hand_scales.txt")
    scales = [int(t) for t in g["scales"][0].split()]
    mins = [int(t) for t in g["mins"][0].split()]
    packed = hexbytes(g["bytes"][0])
    assert list(packed) == pack_q4_k_scales(scales, mins), "test packer vs hand bytes"
    # d=1, dmin=0, every code 1: element of sub-block s decodes to scale_s.
    blk = np.concatenate([np.array(f16_le(1.0) + f16_le(0.0), np.uint8), packed,
                          np.full(128, 0x11, np.uint8)])
    w = oracle.dequant_row(Q4_K, blk, 256)
    for e in range(256):
        s = 2 * (e // 64) + (e % 64) // 32
        assert w[e] == scales[s], (e, w[e], scales[s])
    # d=0, dmin=1: element of sub-block s decodes to -min_s.
    blk[0:4] = f16_le(0.0) + f16_le(1.0)
    w = oracle.dequant_row(Q4_K, blk, 256)
    for e in range(256):
        s = 2 * (e // 64) + (e % 64) // 32
        assert w[e] == -mins[s], (e, w[e], mins[s])


def pin_q4_k_scale_roundtrip():
    """Every (scale, min) pair in every slot survives pack -> oracle decode.
    Codes are all 1, d = 1, dmin = 1/64, so element value = scale - min/64,
    which identifies the pair uniquely."""
    rng = np.random.default_rng(13)
    pairs = [(a, b) for a in range(64) for b in range(64)]
    blocks = []
    expect = []
    for slot in range(8):
        for a, b in pairs[slot::8] + pairs[(slot + 3) % 8::8]:
            sc = [int(v) for v in rng.integers(0, 64, 8)]
            mn = [int(v) for v in rng.integers(0, 64, 8)]
            sc[slot], mn[slot] = a, b
            blocks.append(pack_q4_k([1] * 256, sc, mn, 1.0, 1.0 / 64))
            expect.append((sc, mn))
    W = np.concatenate(blocks)
    w = oracle.dequant(Q4_K, W, 256, len(blocks))
    for r, (sc, mn) in enumerate(expect):
        for s in range(8):
            e0 = 64 * (s // 2) + 32 * (s % 2)
            want = np.float32(sc[s]) - np.float32(mn[s]) / np.float32(64)
            assert np.all(w[r, e0:e0 + 32] == want), (r, s)


def pin_q4_k_element_ownership():
    """Only sub-block s has a non-zero scale: exactly its 32 elements are
    non-zero and they carry their own codes."""
    rng = np.random.default_rng(14)
    codes = [int(c) for c in rng.integers(1, 16, 256)]
    for s in range(8):
        sc = [0] * 8
        sc[s] = 1
        w = oracle.dequant_row(Q4_K, pack_q4_k(codes, sc, [0] * 8, 1.0, 0.0), 256)
        owned = [e for e in range(256) if 2 * (e // 64) + (e % 64) // 32 == s]
        assert set(np.nonzero(w)[0].tolist()) == set(owned), s
        for e in owned:
            assert w[e] == codes[e]


def pin_q4_k_zero_blocks():
    rng = np.random.default_rng(15)
    codes = [int(c) for c in rng.integers(0, 16, 256)]
    sc = [int(c) for c in rng.integers(0, 64, 8)]
    mn = [int(c) for c in rng.integers(0, 64, 8)]
    assert not np.any(oracle.dequant_row(Q4_K, pack_q4_k(codes, sc, mn, 0.0, 0.0), 256))
    assert not np.any(oracle.dequant_row(Q4_K, pack_q4_k(codes, [0] * 8, [0] * 8, 0.7, 0.3), 256))
    assert not np.any(oracle.dequant_row(Q4_K, pack_q4_k([0] * 256, sc, [0] * 8, 0.7, 0.3), 256))


def pin_q6_k_golden():
    g = read_golden("q6_k_hand_block.txt")
    ql = [(p % 16) * 0x11 for p in range(128)]
    qh = [0x88 if p % 32 < 16 else 0xDD for p in range(64)]
    sc = list(hexbytes(g["scales"][0]))
    d = list(hexbytes(g["d"][0]))
    blk = np.array(ql + qh + sc + d, dtype=np.uint8)
    w = oracle.dequant_row(Q6_K, blk, 256)
    for item in g["spot"][0].split():
        e, v = item.split(":")
        assert w[int(e)] == float(v), (e, w[int(e)], v)
    for e in range(256):
        assert w[e] == (q6_k_scale_slot(e) - 8) * (e % 64 - 32), e
    # the test packer reproduces the hand-built bytes
    assert np.array_equal(pack_q6_k([e % 64 for e in range(256)], [s - 8 for s in range(16)],
                                    1.0), blk)


def pin_q6_k_zero_blocks():
    rng = np.random.default_rng(16)
    sc = [int(v) for v in rng.integers(-32, 32, 16)]
    assert not np.any(oracle.dequant_row(Q6_K, pack_q6_k([32] * 256, sc, 0.01), 256))
    codes = [int(v) for v in rng.integers(0, 64, 256)]
    assert not np.any(oracle.dequant_row(Q6_K, pack_q6_k(codes, sc, 0.0), 256))


def pin_q6_k_scale_ownership():
    """Zeroing scale slot s zeroes exactly its 16 elements."""
    rng = np.random.default_rng(17)
    codes = [int(v) for v in rng.integers(0, 64, 256)]
    codes = [c if c != 32 else 33 for c in codes]  # no code that is zero anyway
    for s in range(16):
        sc = [int(v) for v in rng.integers(1, 32, 16)]
        sc[s] = 0
        w = oracle.dequant_row(Q6_K, pack_q6_k(codes, sc, 0.25), 256)
        zeros = set(np.nonzero(w == 0)[0].tolist())
        assert zeros == {e for e in range(256) if q6_k_scale_slot(e) == s}, s


def pin_q6_k_roundtrip():
    rng = np.random.default_rng(18)
    for _ in range(40):
        codes = [int(v) for v in rng.integers(0, 64, 256)]
        sc = [int(v) for v in rng.integers(-128, 128, 16)]
        d = float(np.float16(rng.uniform(-0.02, 0.02)))
        w = oracle.dequant_row(Q6_K, pack_q6_k(codes, sc, d), 256)
        for e in range(256):
            want = (np.float32(d) * np.float32(sc[q6_k_scale_slot(e)])) * np.float32(codes[e] - 32)
            assert w[e] == want, e


def _golden_blocks(name, fmt):
    g = read_golden(name)
    assert len(g["bytes"]) == len(g["values"]) > 0
    for b, v in zip(g["bytes"], g["values"]):
        blk = hexbytes(b)
        want = np.array([float(t) for t in v.split()], dtype=np.float64)
        got = oracle.dequant_row(fmt, blk, 32).astype(np.float64)
        assert np.array_equal(got, want), (name, got, want)
    return g


def pin_q8_0_golden():
    g = _golden_blocks("q8_0_hand_block.txt", Q8_0)
    assert np.array_equal(pack_q8_0([l - 16 for l in range(32)], 1.0), hexbytes(g["bytes"][0]))


def pin_q8_0_zero_blocks_and_roundtrip():
    rng = np.random.default_rng(22)
    assert not np.any(oracle.dequant_row(Q8_0, pack_q8_0([0] * 32, 3.25), 32))
    codes = [int(c) for c in rng.integers(-128, 128, 32)]
    assert not np.any(oracle.dequant_row(Q8_0, pack_q8_0(codes, 0.0), 32))
    for _ in range(50):
        codes = [int(c) for c in rng.integers(-128, 128, 32)]
        d = float(np.float16(rng.uniform(-0.1, 0.1)))
        got = oracle.dequant_row(Q8_0, pack_q8_0(codes, d), 32)
        assert np.array_equal(got, np.float32(d) * np.array(codes, dtype=np.float32))


def pin_q5_0_golden():
    g = _golden_blocks("q5_0_hand_block.txt", Q5_0)
    codes = [16 + l for l in range(16)] + [15 - l for l in range(16)]
    assert np.array_equal(pack_q5_0(codes, 1.0), hexbytes(g["bytes"][0]))


def pin_q5_0_fifth_bit_ownership():
    """Low codes all 0 and only bit e of qh set: element e decodes to 0, every
    other element to -16*d."""
    for e in range(32):
        codes = [0] * 32
        codes[e] = 16
        w = oracle.dequant_row(Q5_0, pack_q5_0(codes, 0.5), 32)
        want = np.full(32, -8.0, dtype=np.float32)
        want[e] = 0.0
        assert np.array_equal(w, want), e


def pin_q5_0_zero_blocks_and_roundtrip():
    rng = np.random.default_rng(23)
    assert not np.any(oracle.dequant_row(Q5_0, pack_q5_0([16] * 32, 1.5), 32))
    codes = [int(c) for c in rng.integers(0, 32, 32)]
    assert not np.any(oracle.dequant_row(Q5_0, pack_q5_0(codes, 0.0), 32))
    for _ in range(50):
        codes = [int(c) for c in rng.integers(0, 32, 32)]
        d = float(np.float16(rng.uniform(-0.1, 0.1)))
        got = oracle.dequant_row(Q5_0, pack_q5_0(codes, d), 32)
        want = np.float32(d) * (np.array(codes, dtype=np.float32) - np.float32(16))
        assert np.array_equal(got, want)


def _random_matrix(fmt, n, k, seed):
    rng = np.random.default_rng(seed)
    return synth.gen_weights(fmt, rng, n, k)


def pin_onehot_bruteforce():
    """x = e_i picks column i: y_j must equal the decoded weight w_j[i]."""
    for fmt, k in ((Q4_0, 32), (Q4_0, 64), (Q4_K, 256), (Q6_K, 256), (F16, 24), (BF16, 24),
                   (Q8_0, 64), (Q5_0, 64)):
        n = 6
        W = _random_matrix(fmt, n, k, 100 + fmt)
        dense = oracle.dequant(fmt, W, k, n)
        X = np.eye(k, dtype=np.float32)
        y, s = oracle.gemv(fmt, W, X, k, n)
        assert np.array_equal(y, dense.T.astype(np.float64)), fmt
        assert np.array_equal(s, np.abs(dense.T.astype(np.float64))), fmt


def pin_dense_route_matches_gemv():
    """Decode everything, then a library f64 matmul: same sums as the oracle's
    gemv to f64 rounding."""
    for fmt, k, n in ((Q4_0, 128, 16), (Q4_K, 512, 9), (Q6_K, 512, 7), (F16, 40, 5),
                      (BF16, 64, 11), (Q8_0, 96, 8), (Q5_0, 160, 6)):
        W = _random_matrix(fmt, n, k, 200 + fmt)
        x = synth.gen_x(np.random.default_rng(300 + fmt), 3, k)
        dense = oracle.dequant(fmt, W, k, n).astype(np.float64)
        want = x.astype(np.float64) @ dense.T
        y, s = oracle.gemv(fmt, W, x, k, n)
        assert np.all(np.abs(y - want) <= 1e-12 * s + 1e-300), fmt


def _factored_q4_0(W, x, k, n):
    blk = W.reshape(n, k // 32, 18)
    d = blk[:, :, 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    qs = blk[:, :, 2:18].astype(np.int64)
    codes = np.concatenate([qs & 15, qs >> 4], axis=2) - 8  # (n, nb, 32)
    xb = x.astype(np.float64).reshape(-1, k // 32, 32)
    return np.einsum("jb,tbe,jbe->tj", d, xb, codes.astype(np.float64))


def _factored_q4_k(W, x, k, n):
    nb = k // 256
    blk = W.reshape(n, nb, 144)
    d = blk[:, :, 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    dmin = blk[:, :, 2:4].copy().view("<f2")[..., 0].astype(np.float64)
    sc = blk[:, :, 4:16].astype(np.int64)
    lo6 = sc & 63
    scale = np.concatenate([lo6[..., 0:4], (sc[..., 8:12] & 15) | ((sc[..., 0:4] >> 6) << 4)], -1)
    mins = np.concatenate([lo6[..., 4:8], (sc[..., 8:12] >> 4) | ((sc[..., 4:8] >> 6) << 4)], -1)
    qs = blk[:, :, 16:144].astype(np.int64).reshape(n, nb, 4, 32)
    codes = np.stack([qs & 15, qs >> 4], axis=3).reshape(n, nb, 8, 32)  # sub-block major
    xb = x.astype(np.float64).reshape(-1, nb, 8, 32)
    qx = np.einsum("tbse,jbse->tjbs", xb, codes.astype(np.float64))
    sx = xb.sum(-1)  # (t, nb, 8)
    return (np.einsum("jb,jbs,tjbs->tj", d, scale.astype(np.float64), qx)
            - np.einsum("jb,jbs,tbs->tj", dmin, mins.astype(np.float64), sx))


def _factored_q6_k(W, x, k, n):
    nb = k // 256
    blk = W.reshape(n, nb, 210)
    ql = blk[:, :, 0:128].astype(np.int64).reshape(n, nb, 2, 2, 32)   # h, g%2, l
    qh = blk[:, :, 128:192].astype(np.int64).reshape(n, nb, 2, 32)    # h, l
    sc = blk[:, :, 192:208].view(np.int8).astype(np.float64).reshape(n, nb, 2, 4, 2)  # h, g, l//16
    d = blk[:, :, 208:210].copy().view("<f2")[..., 0].astype(np.float64)
    lo = np.stack([ql[:, :, :, 0] & 15, ql[:, :, :, 1] & 15, ql[:, :, :, 0] >> 4,
                   ql[:, :, :, 1] >> 4], axis=3)                      # n, nb, h, g, l
    hi = np.stack([(qh >> (2 * g)) & 3 for g in range(4)], axis=3)
    codes = (lo | (hi << 4)) - 32
    xb = x.astype(np.float64).reshape(-1, nb, 2, 4, 2, 16)            # t, b, h, g, l//16, l%16
    cq = codes.reshape(n, nb, 2, 4, 2, 16).astype(np.float64)
    part = np.einsum("tbhgce,jbhgce->tjbhgc", xb, cq)
    return np.einsum("jb,jbhgc,tjbhgc->tj", d, sc, part)


def _factored_q8_0(W, x, k, n):
    blk = W.reshape(n, k // 32, 34)
    d = blk[:, :, 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    codes = blk[:, :, 2:34].view(np.int8).astype(np.float64)  # (n, nb, 32)
    xb = x.astype(np.float64).reshape(-1, k // 32, 32)
    return np.einsum("jb,tbe,jbe->tj", d, xb, codes)


def _factored_q5_0(W, x, k, n):
    blk = W.reshape(n, k // 32, 22)
    d = blk[:, :, 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    qh = blk[:, :, 2:6].copy().view("<u4")[..., 0].astype(np.int64)  # (n, nb)
    qs = blk[:, :, 6:22].astype(np.int64)
    low = np.concatenate([qs & 15, qs >> 4], axis=2)                   # (n, nb, 32)
    fifth = (qh[..., None] >> np.arange(32)) & 1
    codes = (low | (fifth << 4)) - 16
    xb = x.astype(np.float64).reshape(-1, k // 32, 32)
    return np.einsum("jb,tbe,jbe->tj", d, xb, codes.astype(np.float64))


def pin_factored_route_matches_gemv():
    """Per-block factored sums (scale * sum(q*x) - min * sum(x)) in f64 agree
    with the oracle's decode-then-sum to within the f32 rounding of the decoded
    weights."""
    for fmt, k, n, fn in ((Q4_0, 256, 13, _factored_q4_0), (Q4_K, 768, 7, _factored_q4_k),
                          (Q6_K, 512, 9, _factored_q6_k), (Q8_0, 128, 11, _factored_q8_0),
                          (Q5_0, 192, 10, _factored_q5_0)):
        W = _random_matrix(fmt, n, k, 400 + fmt)
        x = synth.gen_x(np.random.default_rng(500 + fmt), 2, k)
        want = fn(W, x, k, n)
        y, s = oracle.gemv(fmt, W, x, k, n)
        assert np.all(np.abs(y - want) <= 2.0 ** -22 * s + 1e-300), fmt


def pin_exact_small_integers():
    """Small-integer f16/bf16 weights and dyadic x: every partial sum is exact,
    so the result equals the rational sum exactly."""
    rng = np.random.default_rng(19)
    k, n = 48, 5
    wi = rng.integers(-9, 10, size=(n, k))
    xi = rng.integers(-8, 9, size=(2, k))
    x = (xi / 8.0).astype(np.float32)
    for fmt in (F16, BF16):
        if fmt == F16:
            W = wi.astype("<f2").view(np.uint8).reshape(-1)
        else:
            W = synth.bf16_bits(wi.astype(np.float32)).astype("<u2").view(np.uint8).reshape(-1)
        y, _ = oracle.gemv(fmt, W, x, k, n)
        for t in range(2):
            for j in range(n):
                want = sum(Fraction(int(wi[j, i])) * Fraction(int(xi[t, i]), 8) for i in range(k))
                assert Fraction(y[t, j]) == want, (fmt, t, j)


def pin_identity_f16():
    """The pages' identity check (matmul.rs, test f16_matmul_3x4_eye): W = I
    (n = k = 4), x = (i+1)/4, y = x."""
    k = n = 4
    W = np.eye(n, k).astype("<f2").view(np.uint8).reshape(-1)
    x = ((np.arange(k) + 1) * 0.25).astype(np.float32)
    y, _ = oracle.gemv(F16, W, x, k, n)
    assert np.array_equal(y[0], x.astype(np.float64))


def pin_linearity():
    rng = np.random.default_rng(20)
    for fmt, k, n in ((Q4_K, 256, 6), (Q6_K, 256, 6), (Q4_0, 64, 6), (Q8_0, 64, 6),
                      (Q5_0, 64, 6)):
        W = _random_matrix(fmt, n, k, 600 + fmt)
        # dyadic x so that 2*x1 + x2 is exact in f32
        x1 = (rng.integers(-64, 65, size=(1, k)) / 64.0).astype(np.float32)
        x2 = (rng.integers(-64, 65, size=(1, k)) / 64.0).astype(np.float32)
        y1, s1 = oracle.gemv(fmt, W, x1, k, n)
        y2, s2 = oracle.gemv(fmt, W, x2, k, n)
        y3, _ = oracle.gemv(fmt, W, 2 * x1 + x2, k, n)
        assert np.all(np.abs(y3 - (2 * y1 + y2)) <= 1e-12 * (2 * s1 + s2) + 1e-300)


def pin_ranges_and_threads():
    """Row ranges, row lists, tiling and thread count give identical bits."""
    fmt, k, n = Q6_K, 512, 37
    W = _random_matrix(fmt, n, k, 700)
    x = synth.gen_x(np.random.default_rng(701), 2, k)
    y_all, s_all = oracle.gemv(fmt, W, x, k, n, threads=1)
    y_mt, _ = oracle.gemv(fmt, W, x, k, n, threads=8)
    assert np.array_equal(y_all, y_mt)
    tiles = [oracle.gemv(fmt, W, x, k, n, a, b)[0] for a, b in ((0, 5), (5, 6), (6, 30), (30, 37))]
    assert np.array_equal(np.concatenate(tiles, axis=1), y_all)
    rows = [36, 0, 17, 17]
    y_r, s_r = oracle.gemv_rows(fmt, W, x, k, n, rows)
    assert np.array_equal(y_r, y_all[:, rows]) and np.array_equal(s_r, s_all[:, rows])


def pin_pages_q4_0_case():
    """The pages' Q4_0 parity case shape (matmul.rs, test
    q4_0_matmul_gpu_vs_cpu_oracle: k=128, n=16, d in [-0.1, 0.1), random code
    bytes, x in [-0.5, 0.5)) against the factored evaluation, with that test's
    own bar max_abs < 1e-4."""
    rng = np.random.default_rng(21)
    k, n = 128, 16
    W = synth.gen_q4_0(rng, n, k, d_range=(-0.1, 0.1))
    x = (rng.uniform(-0.5, 0.5, size=(1, k))).astype(np.float32)
    y, _ = oracle.gemv(Q4_0, W, x, k, n)
    assert np.max(np.abs(y - _factored_q4_0(W, x, k, n))) < 1e-4


# ------------------------------------------------ transposed product pins

def pin_t_adjoint_of_forward():
    """u . (W v) = (W^T u) . v: the transposed oracle is the adjoint of the
    (separately pinned) forward oracle, to f64 rounding."""
    rng = np.random.default_rng(24)
    for fmt, k, n in ((Q4_K, 512, 13), (Q6_K, 256, 9), (Q4_0, 96, 11), (Q8_0, 64, 7),
                      (Q5_0, 128, 10), (F16, 48, 6), (BF16, 40, 5)):
        W = _random_matrix(fmt, n, k, 800 + fmt)
        v = rng.uniform(-1, 1, size=(1, k)).astype(np.float32)
        u = rng.uniform(-1, 1, size=(2, n)).astype(np.float32)
        yf, sf = oracle.gemv(fmt, W, v, k, n)                    # (1, n)
        dx, sx = oracle.gemv_t(fmt, W, u, k, n)                  # (2, k)
        for t in range(2):
            lhs = float(np.dot(u[t].astype(np.float64), yf[0]))
            rhs = float(np.dot(dx[t], v[0].astype(np.float64)))
            bound = float(np.dot(np.abs(u[t]).astype(np.float64), sf[0]))
            assert abs(lhs - rhs) <= 1e-12 * bound + 1e-300, (fmt, t, lhs, rhs)


def pin_t_onehot_rows():
    """dy = e_j gives dx = w_j (the decoded row) exactly, and zeros when j
    lies outside the summed range."""
    for fmt, k, n in ((Q4_K, 256, 6), (Q6_K, 256, 5), (Q4_0, 64, 7), (Q8_0, 32, 4),
                      (Q5_0, 64, 5), (BF16, 16, 3)):
        W = _random_matrix(fmt, n, k, 900 + fmt)
        dense = oracle.dequant(fmt, W, k, n).astype(np.float64)
        dy = np.eye(n, dtype=np.float32)
        dx, s = oracle.gemv_t(fmt, W, dy, k, n)
        assert np.array_equal(dx, dense), fmt
        assert np.array_equal(s, np.abs(dense)), fmt
        dx, _ = oracle.gemv_t(fmt, W, dy, k, n, 1, n - 1)
        assert not np.any(dx[0]) and not np.any(dx[n - 1]), fmt
        assert np.array_equal(dx[1:n - 1], dense[1:n - 1]), fmt


def pin_t_dense_route_and_ranges():
    """A library f64 product of the decoded matrix agrees with the oracle; a
    split of the row range adds up; an empty range is zero."""
    rng = np.random.default_rng(25)
    for fmt, k, n in ((Q4_K, 512, 21), (Q6_K, 256, 33), (Q5_0, 96, 17)):
        W = _random_matrix(fmt, n, k, 1000 + fmt)
        dy = rng.uniform(-1, 1, size=(3, n)).astype(np.float32)
        dense = oracle.dequant(fmt, W, k, n).astype(np.float64)
        dx, s = oracle.gemv_t(fmt, W, dy, k, n)
        want = dy.astype(np.float64) @ dense
        assert np.all(np.abs(dx - want) <= 1e-12 * s + 1e-300), fmt
        a, _ = oracle.gemv_t(fmt, W, dy, k, n, 0, 7)
        b, _ = oracle.gemv_t(fmt, W, dy, k, n, 7, n)
        assert np.all(np.abs(a + b - dx) <= 1e-12 * s + 1e-300), fmt
        want_a = dy[:, 0:7].astype(np.float64) @ dense[0:7]
        assert np.all(np.abs(a - want_a) <= 1e-12 * s + 1e-300), fmt
        e, es = oracle.gemv_t(fmt, W, dy, k, n, 5, 5)
        assert not np.any(e) and not np.any(es)
        cols = [k - 1, 0, 3, 3]
        c, cs = oracle.gemv_t_cols(fmt, W, dy, k, n, cols)
        assert np.array_equal(c, dx[:, cols]) and np.array_equal(cs, s[:, cols])


# ------------------------------------------------ expert-indexed pins

def pin_moe_dense_route():
    """Each output row is x[pos] times the decoded matrix of the expert its
    (position, slot) names: a library f64 product of the decoded slices."""
    rng = np.random.default_rng(26)
    for fmt, k, n, E in ((Q5_0, 64, 4, 5), (Q8_0, 64, 5, 6), (Q4_K, 256, 7, 3)):
        W = _random_matrix(fmt, n * E, k, 1100 + fmt)
        n_pos, top_k = 3, 2
        ids = rng.permutation(E)[:top_k].tolist() + rng.permutation(E)[:top_k].tolist() + \
            rng.permutation(E)[:top_k].tolist()
        x = rng.uniform(-1, 1, size=(n_pos, k)).astype(np.float32)
        y, s = oracle.moe(fmt, W, ids, x, k, n, E, top_k)
        dense = oracle.dequant(fmt, W, k, n * E).astype(np.float64).reshape(E, n, k)
        for r, e in enumerate(ids):
            want = dense[e] @ x[r // top_k].astype(np.float64)
            assert np.all(np.abs(y[r] - want) <= 1e-12 * s[r] + 1e-300), (fmt, r)


def pin_moe_expert_relabeling():
    """Permuting the stacked experts and renumbering ids to match leaves every
    output bit unchanged; an out-of-range id gives a NaN row."""
    rng = np.random.default_rng(27)
    fmt, k, n, E, top_k = Q4_0, 96, 6, 4, 2
    W = _random_matrix(fmt, n * E, k, 1200)
    x = rng.uniform(-1, 1, size=(2, k)).astype(np.float32)
    ids = [3, 1, 0, 3]
    y, _ = oracle.moe(fmt, W, ids, x, k, n, E, top_k)
    perm = [2, 0, 3, 1]                  # new slab i holds old expert perm[i]
    slab = oracle.row_bytes(fmt, k) * n
    W2 = np.concatenate([W[p * slab:(p + 1) * slab] for p in perm])
    ids2 = [perm.index(e) for e in ids]
    y2, _ = oracle.moe(fmt, W2, ids2, x, k, n, E, top_k)
    assert np.array_equal(y, y2)
    y3, _ = oracle.moe(fmt, W, [3, 7, 0, 1], x, k, n, E, top_k)
    assert np.all(np.isnan(y3[1])) and np.array_equal(y3[0], y[0])


# ------------------------------------------------ affine group-64 pins

def pack_affine(bits, codes):
    """codes: k ints in element order -> u32 words, least significant first."""
    per = 32 // bits
    words = []
    for w in range(len(codes) // per):
        v = 0
        for p in range(per):
            v |= int(codes[w * per + p]) << (bits * p)
        words.append(v)
    return np.array(words, dtype=np.uint32)


def pin_affine_golden():
    g = read_golden("affine_hand_rows.txt")
    assert len(g["words"]) == len(g["values"]) == 3
    for b, w, sc, bi, v in zip(g["bits"], g["words"], g["scale"], g["bias"], g["values"]):
        words = np.array([int(t, 16) for t in w.split()], dtype=np.uint32)
        got = oracle.affine_dequant(int(b), words, np.array([int(sc, 16)], np.uint16),
                                    np.array([int(bi, 16)], np.uint16), 64, 1)[0]
        want = np.array([float(t) for t in v.split()], dtype=np.float32)
        assert np.array_equal(got, want), (b, got, want)
    codes4 = [e % 16 if e < 32 else 15 - e % 16 for e in range(64)]
    assert pack_affine(4, codes4).tolist() == [int(t, 16) for t in g["words"][0].split()]
    assert pack_affine(8, [4 * e for e in range(64)]).tolist() == \
        [int(t, 16) for t in g["words"][2].split()]


def pin_affine_roundtrip_and_groups():
    """Random codes, scales and biases through the packer: every element is
    code * scale + bias of its own group; a scale of zero leaves the bias."""
    rng = np.random.default_rng(28)
    for bits in (4, 8):
        k, n = 256, 3
        codes = rng.integers(0, 2 ** bits, size=(n, k))
        sc = synth.bf16_bits(rng.uniform(-0.1, 0.1, size=(n, k // 64)).astype(np.float32))
        bi = synth.bf16_bits(rng.uniform(-0.5, 0.5, size=(n, k // 64)).astype(np.float32))
        words = np.stack([pack_affine(bits, codes[j]) for j in range(n)])
        w = oracle.affine_dequant(bits, words, sc, bi, k, n)
        scf = (sc.astype(np.uint32) << 16).view(np.float32)
        bif = (bi.astype(np.uint32) << 16).view(np.float32)
        for j in range(n):
            for i in range(k):
                want = np.float32(codes[j, i]) * scf[j, i // 64] + bif[j, i // 64]
                assert w[j, i] == want, (bits, j, i)
        sc0 = sc.copy()
        sc0[:, 1] = 0
        w0 = oracle.affine_dequant(bits, words, sc0, bi, k, n)
        assert np.array_equal(w0[:, 64:128], np.repeat(bif[:, 1:2], 64, axis=1))
        assert np.array_equal(w0[:, :64], w[:, :64]) and np.array_equal(w0[:, 128:], w[:, 128:])


def pin_affine_dense_route_and_onehot():
    rng = np.random.default_rng(29)
    for bits in (4, 8):
        k, n = 192, 7
        words, sc, bi = synth.gen_affine(rng, bits, n, k)
        dense = oracle.affine_dequant(bits, words, sc, bi, k, n).astype(np.float64)
        x = synth.gen_x(rng, 2, k)
        y, s = oracle.affine_gemv(bits, words, sc, bi, x, k, n)
        assert np.all(np.abs(y - x.astype(np.float64) @ dense.T) <= 1e-12 * s + 1e-300)
        y1, s1 = oracle.affine_gemv(bits, words, sc, bi, np.eye(k, dtype=np.float32), k, n)
        assert np.array_equal(y1, dense.T) and np.array_equal(s1, np.abs(dense.T))
        yr, _ = oracle.affine_gemv(bits, words, sc, bi, x, k, n, 2, 5)
        assert np.array_equal(yr, y[:, 2:5])


ALL_PINS = [v for name, v in sorted(globals().items()) if name.startswith("pin_")]
