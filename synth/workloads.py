"""The five benchmark workloads as concrete seeded inputs.

Each builder draws its tensors from ``numpy.random.Generator(PCG64(seed))`` in
the order listed, with the shapes, value distributions and dtypes below.
Weight matrices are [N, K] (N output rows, K the reduction dimension).

  C1 seed 101  Q4_K 2048x2048; x fp32 [1, 2048]; y fp32.  Also dequantized.
  C2 seed 102  Q4_K 14336x4096 then 4096x14336; x fp16 [8, K] per shape (batch
               1 and 4 use the leading rows); y fp16.
  C3 seed 103  Q4_K 4096x4096, Q4_K 14336x4096, Q8_0 4096x4096,
               Q8_0 14336x4096; x bf16 [2048, 4096] (M = 512 uses the
               leading rows); y bf16.
  C4 seed 104  128 experts; Q4_K gate [128][2048 x 7168], up [128][2048 x
               7168], down [128][7168 x 2048]; x fp16 [256, 7168] (decode uses
               token 0); ids [256, 8] without replacement; softmax router
               weights over 8 N(0,1) logits.  h and the output are fp32:
               with these weights |h| reaches ~5e5 and the output ~1e8,
               past the fp16 range.
  C5 seed 105  TQ1 17408x5120 then 5120x17408; x fp16 [512, K] per shape
               (batch 1 uses row 0); y fp16.
"""

from __future__ import annotations

from . import gen

SEEDS = {"C1": 101, "C2": 102, "C3": 103, "C4": 104, "C5": 105}


def c1():
    rng = gen.rng_for(SEEDS["C1"])
    w = gen.q4k_blocks(rng, 2048, 2048)
    x = gen.activations(rng, (1, 2048), "f32")
    return {"kind": "q4_k", "n": 2048, "k": 2048, "w": w, "x": x, "x_dt": "f32", "y_dt": "f32"}


def c2():
    rng = gen.rng_for(SEEDS["C2"])
    out = []
    for n, k in ((14336, 4096), (4096, 14336)):
        w = gen.q4k_blocks(rng, n, k)
        out.append({"kind": "q4_k", "n": n, "k": k, "w": w})
    for case in out:
        case["x"] = gen.activations(rng, (8, case["k"]), "f16")
        case["x_dt"], case["y_dt"] = "f16", "f16"
    return out


def c3(which=None):
    """List of weight cases (kind, n, k, w) and the shared x [2048, 4096] bf16."""
    rng = gen.rng_for(SEEDS["C3"])
    cases = []
    for kind, n in (("q4_k", 4096), ("q4_k", 14336), ("q8_0", 4096), ("q8_0", 14336)):
        w = gen.weight_blocks(kind, rng, n, 4096)
        cases.append({"kind": kind, "n": n, "k": 4096, "w": w})
    x = gen.activations(rng, (2048, 4096), "bf16")
    if which is not None:
        cases = [c for c in cases if (c["kind"], c["n"]) == which]
    return cases, x


def c4():
    rng = gen.rng_for(SEEDS["C4"])
    E, H, F, T, top_k = 128, 7168, 2048, 256, 8
    gate = gen.q4k_blocks(rng, E * F, H)
    up = gen.q4k_blocks(rng, E * F, H)
    down = gen.q4k_blocks(rng, E * H, F)
    x = gen.activations(rng, (T, H), "f16")
    ids, scores = gen.moe_routing(rng, T, E, top_k)
    return {"kind": "q4_k", "n_experts": E, "hidden": H, "ffn": F, "T": T, "top_k": top_k,
            "gate": gate, "up": up, "down": down, "x": x, "ids": ids, "scores": scores,
            "gate_stride": F * gen.row_bytes("q4_k", H), "down_stride": H * gen.row_bytes("q4_k", F)}


def c5():
    rng = gen.rng_for(SEEDS["C5"])
    out = []
    for n, k in ((17408, 5120), (5120, 17408)):
        w = gen.tq1_blocks(rng, n, k)
        out.append({"kind": "tq1_g128", "n": n, "k": k, "w": w})
    for case in out:
        case["x"] = gen.activations(rng, (512, case["k"]), "f16")
        case["x_dt"], case["y_dt"] = "f16", "f16"
    return out
