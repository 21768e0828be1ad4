"""GPU parity of the expert-routed entry points (kq_moe_route, kq_qmm_id,
kq_moe_glu) against the CPU oracle, through the C ABI.

The routing schedule is integer work and is compared exactly.  Products use
the dense rule |gpu - ref| <= tau * S.  The GLU output h = silu(g) * u is
checked against the bound that the gate and up tolerances imply:
|h - h_ref| <= E * (1 + u_h) + u_h * |h_ref| + eta_h,
E = tau * (max|silu'| * |u| * S_g + |silu(g)| * S_u)
with max|silu'| < 1.1 (for the tanh-approximated GELU: gelu and 1.13),
u_h the unit roundoff of h's storage type and eta_h
half its subnormal spacing (the stored value is the computed one, within E
of h_ref, rounded once).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads
from tests.gpu_util import ETA, TAU, UNIT, check_tol, device, empty, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    from block_quantized_weight_q4_amd import _build, kq as mod

    _build.build_if_missing()
    mod.lib()
    return mod


def _say(*a):
    print("[case]", *a, flush=True)


def _ws(kq, E, T, top_k, n_out=0):
    nbytes = kq.kq_moe_workspace_bytes(E, T, top_k, n_out)
    return torch.empty(nbytes, dtype=torch.uint8, device=device())


def _ids(rng, T, E, top_k):
    return np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.uint32)


@pytest.mark.parametrize("E,T,top_k", [(1, 1, 1), (8, 1, 8), (128, 1, 8), (128, 256, 8),
                                       (16, 300, 4), (5, 2000, 2), (4096, 64, 16), (32, 31, 4),
                                       (32, 32, 4)])
@pytest.mark.parametrize("defect", ["none", "range", "repeat"])
def test_route_schedule_exact(kq, E, T, top_k, defect):
    """The schedule bit for bit against the oracle's, with out-of-range ids
    (three of them) or one id repeated within a token: below 32 tokens the
    matrix-vector rule (schedule of the valid rows), from 32 on the
    matrix-matrix rule (no tiles)."""
    rng = synth.rng_for(E * 1000 + T)
    ids = _ids(rng, T, E, top_k)
    if defect == "range" and T * top_k > 8:
        ids.ravel()[rng.integers(0, T * top_k, 3)] = [E, E + 1, 0xFFFFFFFF]
    elif defect == "repeat" and top_k > 1:
        t = int(rng.integers(0, T))
        ids[t, top_k - 1] = ids[t, 0]
    elif defect != "none":
        pytest.skip("no such defect at this shape")
    _say("route", E, T, top_k, defect)
    ws = _ws(kq, E, T, top_k)
    kq.kq_moe_route(to_dev(ids), T, top_k, E, ws)
    torch.cuda.synchronize()
    got = kq.moe_schedule(ws, E, T, top_k)
    ref = oracle.route(ids, E, kq.MOE_TILE_ROWS)
    assert got["n_invalid"] == ref["n_invalid"]
    for key in ("counts", "offsets", "perm", "tiles"):
        assert np.array_equal(got[key], ref[key]), key


def _moe_case(kind, E, n, k, T, top_k, seed):
    rng = synth.rng_for(seed)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k)).astype(np.float32)
    return rng, w, stride, ids, scores


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("mixed", [False, True])
@pytest.mark.parametrize("E,T,top_k", [(8, 1, 8), (8, 5, 3), (4, 70, 4)])
def test_qmm_id_small(kq, kind, layout, mixed, E, T, top_k):
    n, k = 96, {"q4_k": 512, "q8_0": 160, "tq1_g128": 384}[kind]
    rng, w, stride, ids, scores = _moe_case(kind, E, n, k, T, top_k, 40 + T)
    x_rows = T if layout == 0 else T * top_k
    x = synth.activations(rng, (x_rows, k), "f16")
    _say("qmm_id", kind, layout, mixed, E, T, top_k)
    y = empty((T if mixed else T * top_k, n), "f32")
    ws = _ws(kq, E, T, top_k, n if mixed else 0)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x, "f16"), layout, to_dev(ids), T,
                 top_k, to_dev(scores) if mixed else None, y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, "f16", layout == 1, ids, T, top_k,
                           scores if mixed else None)
    check_tol(to_f64(y), ref, s, TAU["f16"], f"qmm_id {kind}")


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("mixed", [False, True])
@pytest.mark.parametrize("E,T,top_k", [(8, 1, 8), (8, 5, 3), (4, 70, 4)])
def test_qmm_id_f32_activations(kq, kind, layout, mixed, E, T, top_k):
    # fp32 activations whose rows span 1e-3 .. 1e5 in magnitude (past the
    # fp16 range), held to the fp32 tolerance
    n, k = 80, {"q4_k": 768, "q8_0": 160, "tq1_g128": 384}[kind]
    rng, w, stride, ids, scores = _moe_case(kind, E, n, k, T, top_k, 90 + T)
    x_rows = T if layout == 0 else T * top_k
    x = synth.activations(rng, (x_rows, k), "f32")
    x *= (10.0 ** rng.uniform(-3, 5, size=(x_rows, 1))).astype(np.float32)
    _say("qmm_id f32", kind, layout, mixed, E, T, top_k)
    y = empty((T if mixed else T * top_k, n), "f32")
    ws = _ws(kq, E, T, top_k, n if mixed else 0)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x), layout, to_dev(ids), T,
                 top_k, to_dev(scores) if mixed else None, y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, "f32", layout == 1, ids, T, top_k,
                           scores if mixed else None)
    check_tol(to_f64(y), ref, s, TAU["f32"], f"qmm_id f32 {kind}")


@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("nsb", [1, 5])
def test_qmm_id_tiles_over_16_rows_long_k(kq, x_dt, layout, nsb):
    """Q4_K routed product with tiles of more than 16 rows over one and five
    super-blocks of K: the activation rows go through LDS in one-chunk-ahead
    copies (fp16: chunks of two super-blocks, the last possibly of one; fp32:
    one super-block at a time), every output against the oracle."""
    E, T, top_k, n, k = 4, 70, 4, 96, 256 * nsb
    rng, w, stride, ids, scores = _moe_case("q4_k", E, n, k, T, top_k, 60 + layout + 2 * nsb)
    x_rows = T if layout == 0 else T * top_k
    x = synth.activations(rng, (x_rows, k), x_dt)
    _say("qmm_id long k", x_dt, layout, nsb)
    y = empty((T, n), "f32")
    ws = _ws(kq, E, T, top_k, n)
    kq.kq_qmm_id("q4_k", to_dev(w), E, n, k, stride, to_dev(x, x_dt), layout, to_dev(ids), T,
                 top_k, to_dev(scores), y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id("q4_k", w, E, n, k, stride, x, x_dt, layout == 1, ids, T, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"qmm_id long k {x_dt}")


@pytest.mark.parametrize("T,defect", [(1, False), (20, True), (40, False), (40, True)])
def test_reused_schedule_matches_rebuilt(kq, T, defect):
    # gate/up then down on one workspace: the down call that keeps the
    # schedule built by the GLU gives the same bits as one that rebuilds it
    E, F, H, top_k = 8, 256, 256, 4
    rng = synth.rng_for(300 + T)
    gate = synth.weight_blocks("q4_k", rng, E * F, H)
    up = synth.weight_blocks("q4_k", rng, E * F, H)
    down = synth.weight_blocks("q4_k", rng, E * H, F)
    ids = _ids(rng, T, E, top_k)
    if defect:
        # an out-of-range id: token 0's output is NaN below 32 tokens, the
        # whole output from 32 tokens on
        ids.ravel()[0] = E + 3
    scores = rng.uniform(0.05, 1.0, size=(T, top_k)).astype(np.float32)
    x = synth.activations(rng, (T, H), "f16")
    gs, ds = F * synth.row_bytes("q4_k", H), H * synth.row_bytes("q4_k", F)
    dev = {k: to_dev(v) for k, v in (("gate", gate), ("up", up), ("down", down), ("ids", ids),
                                     ("scores", scores))}
    ws = _ws(kq, E, T, top_k, H)
    h = empty((T, top_k, F), "f32")
    outs = []
    for flags in (0, kq.REUSE_SCHEDULE):
        _say("reuse", T, flags)
        kq.kq_moe_glu("q4_k", dev["gate"], dev["up"], E, F, H, gs, to_dev(x, "f16"), dev["ids"],
                      T, top_k, h, ws)
        out = empty((T, H), "f32")
        kq.kq_qmm_id("q4_k", dev["down"], E, H, F, ds, h, kq.LAYOUT_SLOTTED | flags,
                     dev["ids"], T, top_k, dev["scores"], out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    if defect and T < 32:
        assert np.isnan(outs[0][0]).all() and not np.isnan(outs[0][1:]).any()
    elif defect:
        assert np.isnan(outs[0]).all()
    else:
        assert not np.isnan(outs[0]).any()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("defect", ["repeat", "range"])
@pytest.mark.parametrize("T", [31, 32, 70])
def test_routing_rule_matrix_matrix(kq, defect, T):
    """mlx-native "quantized_matmul_id_ggml.rs" id contract: from 32 tokens on
    a repeated or out-of-range id makes the entire output NaN (unmixed, mixed
    and GLU forms, and a down projection that reuses the poisoned schedule);
    below 32 tokens only an out-of-range id's rows are NaN and a repeated id
    is computed as written, compared with the oracle."""
    E, n, k, top_k = 8, 64, 512, 4
    rng, w, stride, ids, scores = _moe_case("q4_k", E, n, k, T, top_k, 500 + T)
    ids = ids.copy()
    if defect == "repeat":
        ids[T // 2, 3] = ids[T // 2, 1]
    else:
        ids[T // 2, 2] = E + 7
    x = synth.activations(rng, (T, k), "f16")
    wd, idd, xd, scd = to_dev(w), to_dev(ids), to_dev(x, "f16"), to_dev(scores)
    _say("routing rule", defect, T)
    for mixed in (False, True):
        y = empty((T if mixed else T * top_k, n), "f32")
        ws = _ws(kq, E, T, top_k, n if mixed else 0)
        kq.kq_qmm_id("q4_k", wd, E, n, k, stride, xd, 0, idd, T, top_k, scd if mixed else None,
                     y, ws)
        torch.cuda.synchronize()
        got = to_f64(y)
        ref, s = oracle.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, ids, T, top_k,
                               scores if mixed else None)
        bad = np.isnan(ref).all(axis=1)
        assert np.array_equal(np.isnan(got).all(axis=1), bad)
        assert not np.isnan(got[~bad]).any()
        if T >= 32:
            assert bad.all()
        else:
            assert bad.sum() == (0 if defect == "repeat" else 1)
            check_tol(got[~bad], ref[~bad], s[~bad], TAU["f16"], f"rule {defect} T={T}")
    # GLU h [T, top_k, 256], then a down projection (64 rows of 256 columns
    # per expert) that keeps the GLU's schedule
    F, H = 256, 64
    gate = synth.weight_blocks("q4_k", rng, E * F, k)
    down = synth.weight_blocks("q4_k", rng, E * H, F)
    gs, ds = F * synth.row_bytes("q4_k", k), H * synth.row_bytes("q4_k", F)
    ws = _ws(kq, E, T, top_k, H)
    h = empty((T, top_k, F), "f32")
    gd = to_dev(gate)
    kq.kq_moe_glu("q4_k", gd, gd, E, F, k, gs, xd, idd, T, top_k, h, ws)
    out = empty((T, H), "f32")
    kq.kq_qmm_id("q4_k", to_dev(down), E, H, F, ds, h, kq.LAYOUT_SLOTTED | kq.REUSE_SCHEDULE,
                 idd, T, top_k, scd, out, ws)
    torch.cuda.synchronize()
    hg, og = to_f64(h), to_f64(out)
    if T >= 32:
        assert np.isnan(hg).all() and np.isnan(og).all()
    else:
        rows_bad = np.isnan(hg).all(axis=2)
        assert rows_bad.sum() == (0 if defect == "repeat" else 1)
        assert not np.isnan(hg[~rows_bad]).any()


@pytest.mark.parametrize("x_dt", ["f16", "f32"])
def test_qmm_id_invalid_ids_poison(kq, x_dt):
    E, n, k, T, top_k = 6, 64, 256, 4, 2
    rng, w, stride, ids, scores = _moe_case("q4_k", E, n, k, T, top_k, 77)
    ids = ids.copy()
    ids[1, 1] = E       # out of range
    ids[3, 0] = 1 << 30
    x = synth.activations(rng, (T, k), x_dt)
    for mixed in (False, True):
        y = empty((T if mixed else T * top_k, n), "f16")
        ws = _ws(kq, E, T, top_k, n if mixed else 0)
        kq.kq_qmm_id("q4_k", to_dev(w), E, n, k, stride, to_dev(x, x_dt), 0, to_dev(ids), T,
                     top_k, to_dev(scores) if mixed else None, y, ws)
        torch.cuda.synchronize()
        got = to_f64(y)
        ref, s = oracle.qmm_id("q4_k", w, E, n, k, stride, x, x_dt, False, ids, T, top_k,
                               scores if mixed else None)
        bad = np.isnan(ref).all(axis=1)
        assert bad.sum() == 2
        assert np.isnan(got[bad]).all()
        check_tol(got[~bad], ref[~bad], s[~bad], TAU[x_dt], "valid rows",
                  out_dt="f16" if x_dt == "f32" else None)


@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("layout", [0, 1])
def test_single_token_invalid_id_poisons(kq, x_dt, layout):
    """One token with an invalid id among its slots: the mixed output is
    NaN, the GLU slot row of that id is NaN and the other slots are valid."""
    E, n, k, top_k = 6, 64, 512, 3
    rng, w, stride, ids, scores = _moe_case("q4_k", E, n, k, 1, top_k, 78)
    ids = ids.copy()
    ids[0, 1] = E + 1
    x_rows = 1 if layout == 0 else top_k
    x = synth.activations(rng, (x_rows, k), x_dt)
    _say("single token poison", x_dt, layout)
    y = empty((1, n), "f32")
    ws = _ws(kq, E, 1, top_k, n)
    kq.kq_qmm_id("q4_k", to_dev(w), E, n, k, stride, to_dev(x, x_dt), layout, to_dev(ids), 1,
                 top_k, to_dev(scores), y, ws)
    torch.cuda.synchronize()
    assert np.isnan(to_f64(y)).all()
    if layout == 0:
        h = empty((1, top_k, n), "f32")
        kq.kq_moe_glu("q4_k", to_dev(w), to_dev(w), E, n, k, stride, to_dev(x, x_dt), to_dev(ids),
                      1, top_k, h, ws)
        torch.cuda.synchronize()
        got = to_f64(h)[0]
        assert np.isnan(got[1]).all() and not np.isnan(got[[0, 2]]).any()


def _check_glu(h, ref, tau, h_dt, what, act=0, limit=0.0):
    """act 0: silu (|silu'| < 1.1); act 1: gelu, tanh approximation
    (|gelu'| < 1.13); act 2: silu(min(g, limit)) * clip(u, -limit, limit),
    whose derivatives are bounded by those of silu(g) * u (min and clip are
    1-Lipschitz)."""
    g, u, sg, su = ref["g"], ref["u"], ref["sg"], ref["su"]
    assert not np.isnan(h).any(), what
    if h_dt == "f16":
        # values past the fp16 range must be stored as infinities of the right sign
        over = np.abs(ref["h"]) >= 65520.0
        assert np.array_equal(h[over], np.sign(ref["h"][over]) * np.inf), what
        h, g, u, sg, su = h[~over], g[~over], u[~over], sg[~over], su[~over]
        ref = {"h": ref["h"][~over]}
    with np.errstate(over="ignore"):
        if act == 1:
            a_g, dmax = 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3))), 1.13
        elif act == 2:
            gc = np.minimum(g, limit)
            a_g, dmax = gc / (1.0 + np.exp(-gc)), 1.1
        else:
            a_g, dmax = g / (1.0 + np.exp(-g)), 1.1
    # the computed h may be off by the product tolerance, and storing it
    # rounds once more: relative UNIT of the stored value, |h_ref| + that error
    comp = tau * (dmax * np.abs(u) * sg + np.abs(a_g) * su)
    bound = comp * (1.0 + UNIT[h_dt]) + UNIT[h_dt] * np.abs(ref["h"]) + ETA[h_dt]
    err = np.abs(h - ref["h"])
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} outside; worst {np.max(err - bound):.3e}"


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("h_dt", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("T", [1, 9])
def test_moe_glu_small(kq, kind, h_dt, x_dt, T):
    E, n, k, top_k = 6, 80, {"q4_k": 512, "q8_0": 96, "tq1_g128": 256}[kind], 3
    rng = synth.rng_for(90)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T, k), x_dt)
    _say("moe_glu", kind, h_dt, x_dt)
    h = empty((T, top_k, n), h_dt)
    ws = _ws(kq, E, T, top_k)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, x_dt), to_dev(ids),
                  T, top_k, h, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, x_dt, ids, T, top_k)
    _check_glu(to_f64(h), ref, TAU[x_dt], h_dt, f"moe_glu {kind} {h_dt} x={x_dt}")


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("T", [1, 9, 40])
def test_moe_glu_gelu(kq, kind, x_dt, T):
    """act = GELU (tanh approximation) through every GLU kernel: one token
    (read ids directly for Q4_K with fp16 x), tiles of <= 16 rows, and a
    routing with tiles of more than 16 rows (T = 40, top-3 of 6)."""
    E, n, k, top_k = 6, 80, {"q4_k": 512, "q8_0": 96, "tq1_g128": 256}[kind], 3
    rng = synth.rng_for(95)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T, k), x_dt)
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, x_dt, ids, T, top_k, act=1)
    for h_dt in ("f32", "f16"):
        _say("moe_glu gelu", kind, x_dt, T, h_dt)
        h = empty((T, top_k, n), h_dt)
        ws = _ws(kq, E, T, top_k)
        kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, x_dt), to_dev(ids),
                      T, top_k, h, ws, act=kq.ACT_GELU_TANH)
        torch.cuda.synchronize()
        _check_glu(to_f64(h), ref, TAU[x_dt], h_dt, f"moe_glu gelu {kind} {h_dt} x={x_dt} T={T}", act=1)


@pytest.fixture(scope="module")
def c4_dev(kq):
    c = workloads.c4()
    d = {key: c[key] for key in c}
    d["gate_d"], d["up_d"], d["down_d"] = to_dev(c["gate"]), to_dev(c["up"]), to_dev(c["down"])
    return d


def _moe_layer_gpu(kq, c, T):
    """The layer as the benchmark times it: gate/up with the GLU, then the
    mixed down projection over the slotted h that keeps the GLU's schedule."""
    E, H, F, top_k = c["n_experts"], c["hidden"], c["ffn"], c["top_k"]
    x = to_dev(c["x"][:T], "f16")
    ids = to_dev(c["ids"][:T])
    scores = to_dev(c["scores"][:T])
    # h and the layer output are fp32: with these unnormalised random weights
    # h reaches ~5e5 and the output ~1e8, past the fp16 range
    h = empty((T, top_k, F), "f32")
    ws = _ws(kq, E, T, top_k, H)
    kq.kq_moe_glu("q4_k", c["gate_d"], c["up_d"], E, F, H, c["gate_stride"], x, ids, T, top_k, h,
                  ws)
    out = empty((T, H), "f32")
    kq.kq_qmm_id("q4_k", c["down_d"], E, H, F, c["down_stride"], h,
                 kq.LAYOUT_SLOTTED | kq.REUSE_SCHEDULE, ids, T, top_k, scores, out, ws)
    torch.cuda.synchronize()
    return to_f64(h), to_f64(out)


def test_moe_c4_decode_full(kq, c4_dev):
    """C4 decode (1 token, top-8 of 128): every output of the layer."""
    c = c4_dev
    _say("moe C4 decode")
    h, out = _moe_layer_gpu(kq, c, 1)
    ref, s = oracle.moe_layer("q4_k", c["gate"], c["up"], c["down"], c["n_experts"], c["hidden"],
                              c["ffn"], c["gate_stride"], c["down_stride"], c["x"][:1], "f16",
                              c["ids"][:1], 1, c["top_k"], c["scores"][:1])
    check_tol(out, ref, s, TAU["f16"], "moe C4 decode")
    g = oracle.moe_glu("q4_k", c["gate"], c["up"], c["n_experts"], c["ffn"], c["hidden"],
                       c["gate_stride"], c["x"][:1], "f16", c["ids"][:1], 1, c["top_k"])
    _check_glu(h, g, TAU["f16"], "f32", "moe C4 decode h")


def _c4_prefill_tokens(ids, E, tile_rows=32):
    """Tokens whose routed rows open the first tile or sit in the partial last
    tile of several experts' segments (the schedule sorts each expert's rows by
    token), plus the first and last token."""
    flat = ids.ravel()
    picked = {0, ids.shape[0] - 1}
    for e in (0, 1, 37, 64, 100, E - 1):
        rows = np.nonzero(flat == e)[0]  # ascending: the expert's segment order
        if rows.size:
            picked.add(int(rows[0] // ids.shape[1]))       # first row of the first tile
            last_tile = (rows.size - 1) // tile_rows * tile_rows
            picked.add(int(rows[last_tile] // ids.shape[1]))  # first row of the last tile
            picked.add(int(rows[-1] // ids.shape[1]))       # last row of the segment
    return sorted(picked)


def test_moe_c4_prefill_sampled_tokens(kq, c4_dev):
    """C4 prefill (256 tokens) in the launch sequence the benchmark times:
    whole output rows and h rows of at least 16 tokens, chosen to hit the
    first and the partial last schedule tile of several experts."""
    c = c4_dev
    _say("moe C4 prefill")
    h, out = _moe_layer_gpu(kq, c, c["T"])
    toks = _c4_prefill_tokens(c["ids"], c["n_experts"], kq.MOE_TILE_ROWS)
    extra = [t for t in range(c["T"]) if t not in toks]
    toks = sorted(toks + extra[:max(0, 16 - len(toks))])
    assert len(toks) >= 16
    sel = np.array(toks)
    ref, s = oracle.moe_layer("q4_k", c["gate"], c["up"], c["down"], c["n_experts"], c["hidden"],
                              c["ffn"], c["gate_stride"], c["down_stride"], c["x"][sel], "f16",
                              c["ids"][sel], len(sel), c["top_k"], c["scores"][sel])
    check_tol(out[sel], ref, s, TAU["f16"], f"moe C4 prefill tokens {toks}")
    g = oracle.moe_glu("q4_k", c["gate"], c["up"], c["n_experts"], c["ffn"], c["hidden"],
                       c["gate_stride"], c["x"][sel], "f16", c["ids"][sel], len(sel), c["top_k"])
    _check_glu(h[sel], g, TAU["f16"], "f32", "moe C4 prefill h")


# ---------------------------------------------------------------- silu_limit, shared expert
def _shexp_inputs(kind, E, n, k, T, top_k, seed, x_dt="f16"):
    rng = synth.rng_for(seed)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    sg = synth.weight_blocks(kind, rng, n, k)
    su = synth.weight_blocks(kind, rng, n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T, k), x_dt)
    return rng, gate, up, sg, su, stride, ids, x


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("T", [1, 9, 40])
@pytest.mark.parametrize("shexp,act,limit", [(False, 2, 5.0), (True, 2, 5.0), (True, 0, 0.0)])
def test_moe_glu_ex(kq, kind, x_dt, T, shexp, act, limit):
    """kq_moe_glu_ex: silu_limit (mlx-kquant moe_glu_gather_kq act='silu_limit')
    and the shared expert as the last slot (moe_glu_gather_shexp_kq), against
    the oracle; one token takes the direct single-token kernels for Q4_K with
    fp16 activations."""
    E, top_k = 6, 3
    n, k = 80, {"q4_k": 512, "q8_0": 96, "tq1_g128": 256}[kind]
    rng, gate, up, sg, su, stride, ids, x = _shexp_inputs(kind, E, n, k, T, top_k, 600 + T, x_dt)
    S = top_k + (1 if shexp else 0)
    _say("moe_glu_ex", kind, x_dt, T, shexp, act)
    ws = _ws(kq, E + (1 if shexp else 0), T, S)
    h = empty((T, S, n), "f32")
    kq.kq_moe_glu_ex(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, x_dt), to_dev(ids),
                     T, top_k, h, ws, act, limit, to_dev(sg) if shexp else None,
                     to_dev(su) if shexp else None)
    torch.cuda.synchronize()
    ref = oracle.moe_glu_ex(kind, gate, up, E, n, k, stride, x, x_dt, ids, T, top_k, act, limit,
                            sg if shexp else None, su if shexp else None)
    _check_glu(to_f64(h), ref, TAU[x_dt], "f32", f"glu_ex {kind} {x_dt} T={T}", act=act, limit=limit)


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("T", [1, 5, 40])
def test_qmm_id_mix_shexp(kq, kind, x_dt, T):
    """kq_qmm_id_mix_shexp (mlx-kquant gather_qmv_mix_kq): the routed slots and
    the shared expert's last slot mixed by score, against the oracle."""
    E, top_k, n = 6, 3, 72
    k = {"q4_k": 512, "q8_0": 160, "tq1_g128": 256}[kind]
    rng = synth.rng_for(700 + T)
    w = synth.weight_blocks(kind, rng, E * n, k)
    wsh = synth.weight_blocks(kind, rng, n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T * (top_k + 1), k), x_dt)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k + 1)).astype(np.float32)
    _say("mix shexp", kind, x_dt, T)
    y = empty((T, n), "f32")
    ws = _ws(kq, E + 1, T, top_k + 1, n)
    kq.kq_qmm_id_mix_shexp(kind, to_dev(w), E, n, k, stride, to_dev(wsh), to_dev(x, x_dt),
                           to_dev(ids), T, top_k, to_dev(scores), y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id_mix_shexp(kind, w, E, n, k, stride, wsh, x, x_dt, ids, T, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"mix shexp {kind} {x_dt} T={T}")


@pytest.mark.parametrize("T", [1, 20, 40])
def test_shexp_layer_reuses_schedule(kq, T):
    """A layer with a shared expert as the benchmark would run it: the GLU
    builds the schedule (one more expert and slot), the down projection keeps
    it; the down output equals a rebuilt-schedule call bit for bit and the
    oracle on the GPU's h.  From 32 tokens on a repeated routed id makes both
    outputs NaN; the shared slot itself never poisons."""
    E, F, H, top_k = 8, 256, 256, 2
    rng, gate, up, sg, su, stride, ids, x = _shexp_inputs("q4_k", E, F, H, T, top_k, 800 + T)
    down = synth.weight_blocks("q4_k", rng, E * H, F)
    dsh = synth.weight_blocks("q4_k", rng, H, F)
    ds = H * synth.row_bytes("q4_k", F)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k + 1)).astype(np.float32)
    dev = {k_: to_dev(v) for k_, v in (("gate", gate), ("up", up), ("sg", sg), ("su", su),
                                       ("down", down), ("dsh", dsh), ("ids", ids), ("sc", scores))}
    ws = _ws(kq, E + 1, T, top_k + 1, H)
    outs = []
    for flags in (0, kq.REUSE_SCHEDULE):
        h = empty((T, top_k + 1, F), "f32")
        kq.kq_moe_glu_ex("q4_k", dev["gate"], dev["up"], E, F, H, stride, to_dev(x, "f16"),
                         dev["ids"], T, top_k, h, ws, kq.ACT_SILU, 0.0, dev["sg"], dev["su"])
        out = empty((T, H), "f32")
        kq.kq_qmm_id_mix_shexp("q4_k", dev["down"], E, H, F, ds, dev["dsh"], h, dev["ids"], T,
                               top_k, dev["sc"], out, ws, flags)
        torch.cuda.synchronize()
        outs.append((to_f64(h), out.cpu().numpy()))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    hg = outs[0][0].astype(np.float32)
    ref, s = oracle.qmm_id_mix_shexp("q4_k", down, E, H, F, ds, dsh, hg.reshape(-1, F), "f32",
                                     ids, T, top_k, scores)
    check_tol(outs[0][1].astype(np.float64), ref, s, TAU["f32"], f"shexp layer T={T}")
    if T >= 32:
        bad = ids.copy()
        bad[5, 1] = bad[5, 0]
        h = empty((T, top_k + 1, F), "f32")
        kq.kq_moe_glu_ex("q4_k", dev["gate"], dev["up"], E, F, H, stride, to_dev(x, "f16"),
                         to_dev(bad), T, top_k, h, ws, kq.ACT_SILU, 0.0, dev["sg"], dev["su"])
        out = empty((T, H), "f32")
        kq.kq_qmm_id_mix_shexp("q4_k", dev["down"], E, H, F, ds, dev["dsh"], h, to_dev(bad), T,
                               top_k, dev["sc"], out, ws, kq.REUSE_SCHEDULE)
        torch.cuda.synchronize()
        assert np.isnan(to_f64(h)).all() and np.isnan(to_f64(out)).all()
