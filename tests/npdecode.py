"""Second, independent decoders and block packers written with numpy.

Used only by the tests to cross-check the C oracle: they are vectorised over
whole arrays of blocks (field extraction by array slicing and bit masks) rather
than walked block by block, so a slip in either implementation shows up as a
disagreement.  The packers are the inverse direction: they write chosen
(d, dmin, scale, min, quant) fields into block bytes.
"""

from __future__ import annotations

import numpy as np


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- Q4_K
def q4k_fields(blocks: np.ndarray):
    """blocks uint8 [nb,144] -> d, dmin [nb]; sc, m [nb,8]; q [nb,256] (weight order)."""
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 144)
    d = f16_bits_to_f64(b[:, 0:2].copy().view("<u2")[:, 0])
    dmin = f16_bits_to_f64(b[:, 2:4].copy().view("<u2")[:, 0])
    S = b[:, 4:16].astype(np.int64)
    sc = np.zeros((b.shape[0], 8), dtype=np.int64)
    m = np.zeros((b.shape[0], 8), dtype=np.int64)
    sc[:, 0:4] = S[:, 0:4] % 64
    m[:, 0:4] = S[:, 4:8] % 64
    sc[:, 4:8] = (S[:, 8:12] % 16) + 16 * (S[:, 0:4] // 64)
    m[:, 4:8] = (S[:, 8:12] // 16) + 16 * (S[:, 4:8] // 64)
    Q = b[:, 16:144].reshape(-1, 4, 32).astype(np.int64)
    q = np.concatenate([Q % 16, Q // 16], axis=2).reshape(-1, 256)  # [c][lo32|hi32]
    return d, dmin, sc, m, q


def q4k_decode(blocks: np.ndarray) -> np.ndarray:
    d, dmin, sc, m, q = q4k_fields(blocks)
    sub = np.repeat(np.arange(8), 32)  # sub-block of each weight position
    return d[:, None] * sc[:, sub] * q - dmin[:, None] * m[:, sub]


def q4k_pack(d16: np.ndarray, dmin16: np.ndarray, sc: np.ndarray, m: np.ndarray,
             q: np.ndarray) -> np.ndarray:
    """Inverse of q4k_fields.  d16/dmin16 are float16 arrays [nb]; sc, m in
    0..63 [nb,8]; q in 0..15 [nb,256] in weight order."""
    nb = len(d16)
    out = np.zeros((nb, 144), dtype=np.uint8)
    out[:, 0:2] = np.asarray(d16, dtype=np.float16).view(np.uint16).astype("<u2")[:, None].view(
        np.uint8).reshape(nb, 2)
    out[:, 2:4] = np.asarray(dmin16, dtype=np.float16).view(np.uint16).astype("<u2")[:, None].view(
        np.uint8).reshape(nb, 2)
    sc = np.asarray(sc, dtype=np.int64)
    m = np.asarray(m, dtype=np.int64)
    S = np.zeros((nb, 12), dtype=np.int64)
    for j in range(4):
        S[:, j] = (sc[:, j] & 63) | ((sc[:, j + 4] >> 4) << 6)
        S[:, j + 4] = (m[:, j] & 63) | ((m[:, j + 4] >> 4) << 6)
        S[:, j + 8] = (sc[:, j + 4] & 15) | ((m[:, j + 4] & 15) << 4)
    out[:, 4:16] = S.astype(np.uint8)
    q = np.asarray(q, dtype=np.int64).reshape(nb, 4, 2, 32)
    out[:, 16:144] = (q[:, :, 0, :] | (q[:, :, 1, :] << 4)).reshape(nb, 128).astype(np.uint8)
    return out


# ---------------------------------------------------------------- Q8_0
def q8_0_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 34)
    d = f16_bits_to_f64(b[:, 0:2].copy().view("<u2")[:, 0])
    q = b[:, 2:34].view(np.int8).astype(np.float64)
    return d[:, None] * q


# ---------------------------------------------------------------- TQ1_G128
def tq1_digits(codes: np.ndarray, n: int) -> np.ndarray:
    """Base-3 digits, least significant first: [..., n]."""
    c = np.asarray(codes, dtype=np.int64)
    out = []
    for _ in range(n):
        out.append(c % 3)
        c = c // 3
    return np.stack(out, axis=-1)


def tq1_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 28)
    s = f16_bits_to_f64(b[:, 26:28].copy().view("<u2")[:, 0])
    full = tq1_digits(b[:, 0:25], 5).reshape(-1, 125)
    tail = tq1_digits(b[:, 25], 3)
    t = np.concatenate([full, tail], axis=1) - 1
    return t * s[:, None]


def tq1_pack(trits: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """trits in {-1,0,1} [nb,128]; scale16 float16 [nb]."""
    t = np.asarray(trits, dtype=np.int64) + 1
    nb = t.shape[0]
    out = np.zeros((nb, 28), dtype=np.uint8)
    full = t[:, :125].reshape(nb, 25, 5)
    out[:, 0:25] = (full * (3 ** np.arange(5))).sum(axis=2).astype(np.uint8)
    out[:, 25] = (t[:, 125:128] * (3 ** np.arange(3))).sum(axis=1).astype(np.uint8)
    out[:, 26:28] = np.asarray(scale16, dtype=np.float16).view(np.uint16).astype("<u2")[:, None].view(
        np.uint8).reshape(nb, 2)
    return out


# ---------------------------------------------------------------- helpers
QK = {"q4_k": 256, "q8_0": 32, "tq1_g128": 128}
BB = {"q4_k": 144, "q8_0": 34, "tq1_g128": 28}
_DEC = {"q4_k": q4k_decode, "q8_0": q8_0_decode, "tq1_g128": tq1_decode}


def decode_matrix(kind: str, w: np.ndarray, rows: int, k: int) -> np.ndarray:
    blocks = np.asarray(w, dtype=np.uint8).reshape(rows * (k // QK[kind]), BB[kind])
    return _DEC[kind](blocks).reshape(rows, k)


def act_f64(x: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dt == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dt == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dt)
