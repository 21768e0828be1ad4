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


# ---------------------------------------------------------------- GGUF legacy 32-weight blocks
def _f16_bytes(v16: np.ndarray) -> np.ndarray:
    v = np.asarray(v16, dtype=np.float16).view(np.uint16).astype("<u2")
    return v[:, None].view(np.uint8).reshape(len(v), 2)


def _nibbles(qs: np.ndarray) -> np.ndarray:
    """qs uint8 [nb,16] -> [nb,32]: low nibbles are weights 0..15, high 16..31."""
    q = qs.astype(np.int64)
    return np.concatenate([q & 15, q >> 4], axis=1)


def _q5_high(qh: np.ndarray) -> np.ndarray:
    """qh uint8 [nb,4] -> the fifth bit of each of the 32 weights [nb,32]."""
    word = qh.copy().view("<u4")[:, 0].astype(np.int64)
    return (word[:, None] >> np.arange(32)) & 1


def q4_0_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 18)
    d = f16_bits_to_f64(b[:, 0:2].copy().view("<u2")[:, 0])
    return d[:, None] * (_nibbles(b[:, 2:18]) - 8)


def q5_0_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 22)
    d = f16_bits_to_f64(b[:, 0:2].copy().view("<u2")[:, 0])
    q = _nibbles(b[:, 6:22]) + 16 * _q5_high(b[:, 2:6])
    return d[:, None] * (q - 16)


def q5_1_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 24)
    d = f16_bits_to_f64(b[:, 0:2].copy().view("<u2")[:, 0])
    m = f16_bits_to_f64(b[:, 2:4].copy().view("<u2")[:, 0])
    q = _nibbles(b[:, 8:24]) + 16 * _q5_high(b[:, 4:8])
    return d[:, None] * q + m[:, None]


def legacy_pack(kind: str, q: np.ndarray, d16: np.ndarray, m16=None) -> np.ndarray:
    """Blocks of Q4_0 / Q5_0 / Q5_1 from quants q [nb,32] (0..15 or 0..31)."""
    q = np.asarray(q, dtype=np.int64)
    nb = q.shape[0]
    lo = q & 15
    qs = (lo[:, :16] | (lo[:, 16:] << 4)).astype(np.uint8)
    if kind == "q4_0":
        return np.concatenate([_f16_bytes(d16), qs], axis=1)
    word = ((q >> 4) << np.arange(32)).sum(axis=1).astype("<u4")
    qh = word[:, None].view(np.uint8).reshape(nb, 4)
    if kind == "q5_0":
        return np.concatenate([_f16_bytes(d16), qh, qs], axis=1)
    return np.concatenate([_f16_bytes(d16), _f16_bytes(m16), qh, qs], axis=1)


# ---------------------------------------------------------------- Q6_K
def _q6k_maps():
    """Per weight position e of a super-block: the ql byte, its nibble shift,
    the qh byte, its 2-bit shift and the scale index (GGUF Q6_K layout:
    halves of 128 weights, each four runs of 32)."""
    e = np.arange(256)
    h, r = e // 128, e % 128
    u, l = r // 32, r % 32
    return (64 * h + l + 32 * (u % 2), 4 * (u // 2), 32 * h + l, 2 * u, 8 * h + l // 16 + 2 * u)


def q6k_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 210)
    ql, qh = b[:, 0:128].astype(np.int64), b[:, 128:192].astype(np.int64)
    sc = b[:, 192:208].view(np.int8).astype(np.int64)
    d = f16_bits_to_f64(b[:, 208:210].copy().view("<u2")[:, 0])
    qli, qls, qhi, qhs, sci = _q6k_maps()
    q = ((ql[:, qli] >> qls) & 15) | (((qh[:, qhi] >> qhs) & 3) << 4)
    return d[:, None] * sc[:, sci] * (q - 32)


def q6k_pack(q: np.ndarray, sc: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """Q6_K blocks from quants q [nb,256] in 0..63, int8 scales [nb,16], fp16 d [nb]."""
    q = np.asarray(q, dtype=np.int64)
    nb = q.shape[0]
    qli, qls, qhi, qhs, _ = _q6k_maps()
    ql = np.zeros((nb, 128), dtype=np.int64)
    qh = np.zeros((nb, 64), dtype=np.int64)
    for e in range(256):
        ql[:, qli[e]] |= (q[:, e] & 15) << qls[e]
        qh[:, qhi[e]] |= (q[:, e] >> 4) << qhs[e]
    return np.concatenate([ql.astype(np.uint8), qh.astype(np.uint8),
                           np.asarray(sc, dtype=np.int8).view(np.uint8), _f16_bytes(d16)], axis=1)


# ---------------------------------------------------------------- GGUF Q2_K / Q3_K / Q5_K
def _run_maps():
    """Per weight position e of a 256-weight super-block laid out as two
    halves of four 32-weight runs: the quant byte (32h + l), the 2-bit shift
    within it (2u), the 16-weight scale index (8h + 2u + l // 16) and the
    plane of the third bit (4h + u) for Q3_K."""
    e = np.arange(256)
    h, u, l = e // 128, (e % 128) // 32, e % 32
    return 32 * h + l, 2 * u, 8 * h + 2 * u + l // 16, 4 * h + u


def q2k_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 84)
    scb, qs = b[:, 0:16].astype(np.int64), b[:, 16:80].astype(np.int64)
    d = f16_bits_to_f64(b[:, 80:82].copy().view("<u2")[:, 0])
    dmin = f16_bits_to_f64(b[:, 82:84].copy().view("<u2")[:, 0])
    qb, qsh, si, _ = _run_maps()
    q = (qs[:, qb] >> qsh) & 3
    sc = scb[:, si]
    return d[:, None] * (sc & 15) * q - dmin[:, None] * (sc >> 4)


def q2k_pack(q, sc, mn, d16, dmin16) -> np.ndarray:
    """Q2_K blocks from quants q [nb,256] in 0..3, scales and mins [nb,16] in
    0..15, fp16 d and dmin [nb]."""
    q = np.asarray(q, dtype=np.int64)
    nb = q.shape[0]
    qb, qsh, _, _ = _run_maps()
    qs = np.zeros((nb, 64), dtype=np.int64)
    for e in range(256):
        qs[:, qb[e]] |= q[:, e] << qsh[e]
    scb = (np.asarray(sc, np.int64) & 15) | ((np.asarray(mn, np.int64) & 15) << 4)
    return np.concatenate([scb.astype(np.uint8), qs.astype(np.uint8), _f16_bytes(d16),
                           _f16_bytes(dmin16)], axis=1)


def q3k_scales(S: np.ndarray) -> np.ndarray:
    """12 packed bytes [nb,12] -> the 16 signed scales [nb,16] (stored + 32):
    nibble planes from bytes 0..7 (low nibbles first, then high nibbles),
    2-bit planes from bytes 8..11 (bit pair p of byte 8 + r is scale 4p + r)."""
    S = np.asarray(S, dtype=np.int64)
    low = np.concatenate([S[:, 0:8] & 15, S[:, 0:8] >> 4], axis=1)
    top = np.stack([(S[:, 8:12] >> (2 * p)) & 3 for p in range(4)], axis=1).reshape(-1, 16)
    return (low | (top << 4)) - 32


def q3k_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 110)
    hm, qs = b[:, 0:32].astype(np.int64), b[:, 32:96].astype(np.int64)
    sc = q3k_scales(b[:, 96:108])
    d = f16_bits_to_f64(b[:, 108:110].copy().view("<u2")[:, 0])
    qb, qsh, si, plane = _run_maps()
    l = np.arange(256) % 32
    third = (hm[:, l] >> plane) & 1
    q = ((qs[:, qb] >> qsh) & 3) + 4 * third - 4
    return d[:, None] * sc[:, si] * q


def q3k_pack(q, sc, d16) -> np.ndarray:
    """Q3_K blocks from quants q [nb,256] in -4..3, scales [nb,16] in -32..31
    and fp16 d [nb]."""
    q = np.asarray(q, dtype=np.int64) + 4
    nb = q.shape[0]
    qb, qsh, _, plane = _run_maps()
    hm = np.zeros((nb, 32), dtype=np.int64)
    qs = np.zeros((nb, 64), dtype=np.int64)
    for e in range(256):
        qs[:, qb[e]] |= (q[:, e] & 3) << qsh[e]
        hm[:, e % 32] |= (q[:, e] >> 2) << plane[e]
    u = np.asarray(sc, dtype=np.int64) + 32
    S = np.zeros((nb, 12), dtype=np.int64)
    S[:, 0:8] = (u[:, 0:8] & 15) | ((u[:, 8:16] & 15) << 4)
    for r in range(4):
        S[:, 8 + r] = sum(((u[:, 4 * p + r] >> 4) & 3) << (2 * p) for p in range(4))
    return np.concatenate([hm.astype(np.uint8), qs.astype(np.uint8), S.astype(np.uint8),
                           _f16_bytes(d16)], axis=1)


def q5k_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.asarray(blocks, dtype=np.uint8).reshape(-1, 176)
    # the Q4_K fields from a Q4_K-shaped view (head + scales + nibbles)
    view = np.concatenate([b[:, 0:16], b[:, 48:176]], axis=1)
    d, dmin, sc, m, q4 = q4k_fields(view)
    qh = b[:, 16:48].astype(np.int64)
    e = np.arange(256)
    fifth = (qh[:, e % 32] >> (e // 32)) & 1
    sub = e // 32
    return d[:, None] * sc[:, sub] * (q4 + 16 * fifth) - dmin[:, None] * m[:, sub]


def q5k_pack(d16, dmin16, sc, m, q) -> np.ndarray:
    """Q5_K blocks from the Q4_K fields with quants q [nb,256] in 0..31."""
    q = np.asarray(q, dtype=np.int64)
    head = q4k_pack(d16, dmin16, sc, m, q & 15)
    nb = q.shape[0]
    qh = np.zeros((nb, 32), dtype=np.int64)
    for j in range(8):
        qh |= (q[:, 32 * j:32 * j + 32] >> 4) << j
    return np.concatenate([head[:, 0:16], qh.astype(np.uint8), head[:, 16:144]], axis=1)


# ---------------------------------------------------------------- helpers
QK = {"q4_k": 256, "q8_0": 32, "tq1_g128": 128, "q4_0": 32, "q5_0": 32, "q5_1": 32, "q6_k": 256,
      "q2_k": 256, "q3_k": 256, "q5_k": 256}
BB = {"q4_k": 144, "q8_0": 34, "tq1_g128": 28, "q4_0": 18, "q5_0": 22, "q5_1": 24, "q6_k": 210,
      "q2_k": 84, "q3_k": 110, "q5_k": 176}
_DEC = {"q4_k": q4k_decode, "q8_0": q8_0_decode, "tq1_g128": tq1_decode, "q4_0": q4_0_decode,
        "q5_0": q5_0_decode, "q5_1": q5_1_decode, "q6_k": q6k_decode, "q2_k": q2k_decode,
        "q3_k": q3k_decode, "q5_k": q5k_decode}


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
