"""Seeded generators for block-quantized weights, activations and MoE routing.

Every function takes a ``numpy.random.Generator`` (PCG64) and draws its tensors
in a fixed order, so one seed gives one byte-identical workload on any machine.

Block byte layouts written here (the positions only; decoding lives elsewhere):

* Q4_K, 144 bytes per 256 weights: [0,2) d as fp16 LE, [2,4) dmin as fp16 LE,
  [4,16) twelve bytes of packed 6-bit sub-block scales and mins, [16,144) 128
  bytes of 4-bit quants.  The scale/min and quant bytes are uniform random
  bytes; d and dmin are uniform in [1e-3, 2e-2], rounded to fp16.
* Q8_0, 34 bytes per 32 weights: [0,2) d as fp16 LE, [2,34) int8 quants uniform
  in [-127, 127].
* TQ1_G128, 28 bytes per 128 weights: [0,25) code bytes, [25] tail code byte,
  [26,28) scale as fp16 LE.  A code byte uniform over 0..242 is exactly five
  independent trits uniform over {-1,0,+1} (243 = 3^5 equally likely values),
  and a tail byte uniform over 0..26 is exactly three, so drawing the byte is
  the same distribution as drawing the trits.

Activations are ``standard_normal`` in float32, rounded to the storage dtype
with the library casts (numpy for fp16, torch for bf16).  fp16 and bf16 tensors
are returned as their raw ``uint16`` bit patterns.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "QK", "BLOCK_BYTES", "TYPE_NAMES", "rng_for", "q4k_blocks", "q8_0_blocks",
    "tq1_blocks", "legacy_blocks", "q6k_blocks", "kquant_blocks", "weight_blocks", "activations",
    "moe_routing",
    "row_bytes",
]

TYPE_NAMES = ("q4_k", "q8_0", "tq1_g128", "q4_0", "q5_0", "q5_1", "q6_k", "q2_k", "q3_k", "q5_k")
QK = {"q4_k": 256, "q8_0": 32, "tq1_g128": 128, "q4_0": 32, "q5_0": 32, "q5_1": 32, "q6_k": 256,
      "q2_k": 256, "q3_k": 256, "q5_k": 256}
BLOCK_BYTES = {"q4_k": 144, "q8_0": 34, "tq1_g128": 28, "q4_0": 18, "q5_0": 22, "q5_1": 24,
               "q6_k": 210, "q2_k": 84, "q3_k": 110, "q5_k": 176}

SCALE_LO = 1e-3
SCALE_HI = 2e-2


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def row_bytes(kind: str, k: int) -> int:
    if k % QK[kind]:
        raise ValueError(f"k={k} is not a multiple of {QK[kind]} for {kind}")
    return (k // QK[kind]) * BLOCK_BYTES[kind]


def _fp16_scales(rng: np.random.Generator, n: int) -> np.ndarray:
    """n fp16 values uniform in [1e-3, 2e-2], as little-endian byte pairs."""
    v = rng.uniform(SCALE_LO, SCALE_HI, size=n).astype(np.float16)
    return v.view(np.uint16).astype("<u2").view(np.uint8).reshape(n, 2)


def q4k_blocks(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: random Q4_K super-blocks."""
    nb = rows * (k // 256)
    blk = rng.integers(0, 256, size=(nb, 144), dtype=np.uint8)
    blk[:, 0:2] = _fp16_scales(rng, nb)
    blk[:, 2:4] = _fp16_scales(rng, nb)
    return blk.reshape(rows, row_bytes("q4_k", k))


def q8_0_blocks(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: random Q8_0 blocks."""
    nb = rows * (k // 32)
    blk = np.empty((nb, 34), dtype=np.uint8)
    blk[:, 0:2] = _fp16_scales(rng, nb)
    blk[:, 2:34] = rng.integers(-127, 128, size=(nb, 32), dtype=np.int8).view(np.uint8)
    return blk.reshape(rows, row_bytes("q8_0", k))


def tq1_blocks(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: random TQ1_G128 blocks (all bytes legal)."""
    nb = rows * (k // 128)
    blk = np.empty((nb, 28), dtype=np.uint8)
    blk[:, 0:25] = rng.integers(0, 243, size=(nb, 25), dtype=np.uint8)
    blk[:, 25] = rng.integers(0, 27, size=nb, dtype=np.uint8)
    blk[:, 26:28] = _fp16_scales(rng, nb)
    return blk.reshape(rows, row_bytes("tq1_g128", k))


def legacy_blocks(kind: str, rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: random Q4_0 / Q5_0 / Q5_1 blocks: random quant
    bytes, fp16 d in [1e-3, 2e-2] and (Q5_1) an fp16 offset m in [-0.3, 0.3]."""
    bb = BLOCK_BYTES[kind]
    nb = rows * (k // 32)
    blk = rng.integers(0, 256, size=(nb, bb), dtype=np.uint8)
    blk[:, 0:2] = _fp16_scales(rng, nb)
    if kind == "q5_1":
        m = rng.uniform(-0.3, 0.3, size=nb).astype(np.float16)
        blk[:, 2:4] = m.view(np.uint16).astype("<u2").view(np.uint8).reshape(nb, 2)
    return blk.reshape(rows, row_bytes(kind, k))


def q6k_blocks(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: random Q6_K super-blocks: random quant bytes,
    int8 scales in [-64, 64], fp16 d in [1e-3, 2e-2]."""
    nb = rows * (k // 256)
    blk = rng.integers(0, 256, size=(nb, 210), dtype=np.uint8)
    blk[:, 192:208] = rng.integers(-64, 65, size=(nb, 16), dtype=np.int8).view(np.uint8)
    blk[:, 208:210] = _fp16_scales(rng, nb)
    return blk.reshape(rows, row_bytes("q6_k", k))


def kquant_blocks(kind: str, rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: random Q2_K / Q3_K / Q5_K super-blocks: random
    quant and scale bytes, fp16 d (and dmin) in [1e-3, 2e-2]."""
    bb = BLOCK_BYTES[kind]
    nb = rows * (k // 256)
    blk = rng.integers(0, 256, size=(nb, bb), dtype=np.uint8)
    if kind == "q2_k":
        blk[:, 80:82] = _fp16_scales(rng, nb)
        blk[:, 82:84] = _fp16_scales(rng, nb)
    elif kind == "q3_k":
        blk[:, 108:110] = _fp16_scales(rng, nb)
    else:
        blk[:, 0:2] = _fp16_scales(rng, nb)
        blk[:, 2:4] = _fp16_scales(rng, nb)
    return blk.reshape(rows, row_bytes(kind, k))


_GEN = {"q4_k": q4k_blocks, "q8_0": q8_0_blocks, "tq1_g128": tq1_blocks, "q6_k": q6k_blocks,
        "q4_0": lambda rng, r, k: legacy_blocks("q4_0", rng, r, k),
        "q5_0": lambda rng, r, k: legacy_blocks("q5_0", rng, r, k),
        "q5_1": lambda rng, r, k: legacy_blocks("q5_1", rng, r, k),
        "q2_k": lambda rng, r, k: kquant_blocks("q2_k", rng, r, k),
        "q3_k": lambda rng, r, k: kquant_blocks("q3_k", rng, r, k),
        "q5_k": lambda rng, r, k: kquant_blocks("q5_k", rng, r, k)}


def weight_blocks(kind: str, rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    return _GEN[kind](rng, rows, k)


def activations(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) activations rounded to ``dtype``.

    Returns float32 for "f32", and the uint16 bit pattern for "f16"/"bf16".
    """
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown activation dtype {dtype!r}")


def moe_routing(rng: np.random.Generator, n_tokens: int, n_experts: int, top_k: int):
    """Expert ids drawn uniformly without replacement, and softmax router weights.

    Returns (ids uint32 [T, top_k], scores float32 [T, top_k]).  The weights are
    the softmax over top_k N(0,1) logits, taken in float32, so each token's
    weights sum to one (top-k routing with renormalisation).
    """
    ids = np.empty((n_tokens, top_k), dtype=np.uint32)
    for t in range(n_tokens):
        ids[t] = rng.choice(n_experts, size=top_k, replace=False)
    logits = rng.standard_normal(size=(n_tokens, top_k), dtype=np.float32)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    scores = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, scores
