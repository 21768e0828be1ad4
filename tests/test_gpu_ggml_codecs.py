"""GPU parity of the further GGUF blocks (Q4_0, Q5_0, Q5_1, Q6_K, Q2_K, Q3_K,
Q5_K) against the CPU oracle, through the C ABI, over every entry point that
takes them.

mlx-native "quantized_matmul_id_ggml.rs" dispatches these types
(GgmlType::Q4_0 ... Q5_K) to its mv_id / mm_id kernels.  Here they
decode chunk by chunk on the vector units for every product shape, so the
weights enter the products as exact fp32 values: dequantization is compared
bit for bit, products with |gpu - ref| <= tau * sum|w*x| as for the other
codecs, and a one-hot activation returns the decoded column exactly.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import TAU, bits, check_tol, device, empty, to_dev, to_f64

pytestmark = pytest.mark.gpu

KINDS = ["q4_0", "q5_0", "q5_1", "q6_k", "q2_k", "q3_k", "q5_k"]
QK = {"q4_0": 32, "q5_0": 32, "q5_1": 32, "q6_k": 256, "q2_k": 256, "q3_k": 256, "q5_k": 256}


def _k(kind, blocks32):
    """A row length of about blocks32 32-weight blocks (whole super-blocks of
    the 256-weight codecs)."""
    return 32 * blocks32 if QK[kind] == 32 else 256 * max(1, blocks32 // 8)


@pytest.fixture(scope="module")
def kq():
    from block_quantized_weight_q4_amd import _build, kq as mod

    _build.build_if_missing()
    mod.lib()
    return mod


def _say(*a):
    print("[case]", *a, flush=True)


def _ids(rng, T, E, top_k):
    return np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.uint32)


def _moe_ws(kq, E, T, top_k, n_out=0):
    return torch.empty(kq.kq_moe_workspace_bytes(E, T, top_k, n_out), dtype=torch.uint8,
                       device=device())


# ---------------------------------------------------------------- dequantize
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,nblk", [(1, 1), (7, 3), (129, 5), (300, 48)])
def test_dequant_bit_exact(kq, kind, dt, rows, nblk):
    k = QK[kind] * nblk
    _say("dequant", kind, dt, rows, k)
    w = synth.weight_blocks(kind, synth.rng_for(5000 + rows), rows, k)
    out = empty((rows, k), dt)
    kq.kq_dequantize(kind, to_dev(w), rows, k, out)
    torch.cuda.synchronize()
    ref = oracle.dequant_as(kind, w, rows, k, dt)
    assert np.array_equal(bits(out), ref.view(np.uint32) if dt == "f32" else ref)


# ---------------------------------------------------------------- products
def _run(kq, fn, kind, w, n, k, x, x_dt, m, y_dt):
    wd, xd = to_dev(w), to_dev(x, x_dt)
    y = empty((m, n), y_dt)
    if fn == "kq_qmm_ws":
        nb = kq.kq_qmm_workspace_bytes(kind, n, k, m, xd.dtype)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=xd.device)
        kq.kq_qmm_ws(kind, wd, n, k, xd, m, y, ws)
    else:
        getattr(kq, fn)(kind, wd, n, k, xd, m, y)
    torch.cuda.synchronize()
    return to_f64(y)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("n,nblk", [(67, 6), (130, 150)])
def test_qmv(kq, kind, x_dt, m, n, nblk):
    # 150 blocks of 32 (or 18 super-blocks of 256, 144 chunks): each lane
    # of a wave takes two or three chunks, the last pass ragged
    k = _k(kind, nblk)
    rng = synth.rng_for(5100 + m + n)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (m, k), x_dt)
    for y_dt in ("f32", "f16", "bf16"):
        _say("qmv", kind, x_dt, m, n, k, y_dt)
        got = _run(kq, "kq_qmv", kind, w, n, k, x, x_dt, m, y_dt)
        ref, s = oracle.qmm(kind, w, n, k, x, x_dt, m)
        check_tol(got, ref, s, TAU[x_dt], f"qmv {kind} {x_dt} m={m} y={y_dt}",
                  out_dt=y_dt if y_dt != "f32" else None)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n,k", [(16, 2048), (45, 4096), (300, 6144), (33, 14336), (1, 2048)])
def test_qmv_one_row_lds_kernel(kq, kind, n, k):
    """One fp16 activation row with rows a whole number of the LDS kernel's
    chunks (1024 or 2048 weights): several chunks, ragged row tiles, every
    output dtype; and a second call gives the same bits."""
    rng = synth.rng_for(5170 + n)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (1, k), "f16")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", 1)
    for y_dt in ("f32", "f16", "bf16"):
        _say("qmv one row", kind, n, k, y_dt)
        got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", 1, y_dt)
        check_tol(got, ref, s, TAU["f16"], f"qmv one row {kind} {n}x{k} y={y_dt}",
                  out_dt=y_dt if y_dt != "f32" else None)
        assert np.array_equal(got, _run(kq, "kq_qmm_ws", kind, w, n, k, x, "f16", 1, y_dt))


@pytest.mark.parametrize("kind,k", [("q4_0", 61440), ("q6_k", 51200), ("q8_0", 45056), ("q2_k", 69632)])
def test_qmv_one_row_longest_rows(kq, kind, k):
    """Rows near the longest the one-row LDS kernel stages (the activation
    row and two chunk buffers fill most of the 160 KB of LDS)."""
    n = 5
    rng = synth.rng_for(5190)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (1, k), "f16")
    _say("qmv longest rows", kind, k)
    got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", 1, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", 1)
    check_tol(got, ref, s, TAU["f16"], f"qmv longest {kind} k={k}")
    assert np.array_equal(got, _run(kq, "kq_qmm_noalloc", kind, w, n, k, x, "f16", 1, "f32"))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_qmv_one_row_full_size_sampled(kq, kind, n, k):
    """The C2 GEMV shapes as the benchmark times them (batch 1, fp16 x and
    y), checked on 256 sampled outputs the oracle computes one by one."""
    rng = synth.rng_for(5180)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (1, k), "f16")
    _say("qmv full sampled", kind, n, k)
    got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", 1, "f16")
    pn = np.unique(np.concatenate([rng.integers(0, n, 250), [0, 15, 16, n - 1]]))
    pm = np.zeros_like(pn)
    ref, s = oracle.qmm_points(kind, w, n, k, x, "f16", 1, pm, pn)
    check_tol(got[0, pn], ref, s, TAU["f16"], f"qmv full {kind} {n}x{k}", out_dt="f16")


@pytest.mark.parametrize("kind", KINDS + ["q8_0"])
@pytest.mark.parametrize("m", [2, 5, 8, 9, 16])
@pytest.mark.parametrize("n,k", [(45, 2048), (300, 6144), (40, 9216)])
def test_qmv_batched_matrix_cores(kq, kind, m, n, k):
    """2..16 fp16 activation rows with rows a whole number of the batched
    kernel's chunks (9216: a long row that the long-row chunk of Q5_K and
    Q2_K does not divide, and that Q6_K and Q3_K leave to the vector units):
    the weight stream on the matrix
    cores, 9..16 rows in one pass or two, ragged row tiles; every output
    dtype, and the no-allocation entry gives the same bits."""
    rng = synth.rng_for(5200 + 31 * m + n)
    w = synth.weight_blocks(kind, rng, n, k)
    if kind == "q8_0":
        w.reshape(-1, 34)[::5, 2 + 9] = 0x80  # q = -128, never written by the encoder
    x = synth.activations(rng, (m, k), "f16")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", m)
    for y_dt in ("f32", "f16", "bf16"):
        _say("qmv batched", kind, m, n, k, y_dt)
        got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", m, y_dt)
        check_tol(got, ref, s, TAU["f16"], f"qmv batched {kind} m={m} {n}x{k} y={y_dt}",
                  out_dt=y_dt if y_dt != "f32" else None)
    assert np.array_equal(got, _run(kq, "kq_qmm_noalloc", kind, w, n, k, x, "f16", m, "bf16"))


FOLDED = ("q4_0", "q5_0", "q5_1", "q8_0")  # one fp16 scale per 32 weights


@pytest.mark.parametrize("kind", KINDS + ["q8_0"])
@pytest.mark.parametrize("m", [5, 16])
def test_qmv_batched_one_hot_columns(kq, kind, m):
    """x = e_c through the batched matrix-core GEMV returns column c: the
    weight rounded once to fp16 for the 32-weight blocks (their scale is
    folded into the fp16 weights), the exact weight for the K-quants (their
    scales are applied to fp32 results)."""
    n, k = 40, 2048 if kind in ("q6_k", "q3_k") else 1024
    w = synth.weight_blocks(kind, synth.rng_for(5310), n, k)
    W64 = oracle.dequant(kind, w, n, k)
    ref = (W64.astype(np.float16) if kind in FOLDED else W64).astype(np.float32)
    for c0 in range(0, k, m):
        mm = min(m, k - c0)
        if mm < 2:
            continue
        x = np.zeros((mm, k), np.float16)
        x[np.arange(mm), c0 + np.arange(mm)] = 1.0
        _say("qmv batched one-hot", kind, m, c0)
        got = _run(kq, "kq_qmv", kind, w, n, k, x.view(np.uint16), "f16", mm, "f32")
        assert np.array_equal(got, ref[:, c0:c0 + mm].T), (kind, m, c0)


@pytest.mark.parametrize("kind", KINDS + ["q8_0"])
@pytest.mark.parametrize("m", [3, 16])
def test_qmv_batched_large_scales_take_exact_path(kq, kind, m):
    """Blocks with d = 30000 scattered over the matrix: a wave whose chunk
    buffer holds one (its weights could pass the fp16 range when folded)
    takes the exact form, the others the folded one; the result matches the
    oracle."""
    n, k = 96, 4096
    rng = synth.rng_for(5320 + m)
    w = synth.weight_blocks(kind, rng, n, k)
    bb = synth.BLOCK_BYTES[kind]
    blocks = w.reshape(n, -1, bb)
    big = np.array([30000.0], np.float16).view(np.uint8)
    off = {"q6_k": 208, "q2_k": 80, "q3_k": 108}.get(kind, 0)
    blocks[::3, ::7, off:off + 2] = big
    x = synth.activations(rng, (m, k), "f16")
    _say("qmv batched exact path", kind, m)
    got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", m, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", m)
    check_tol(got, ref, s, TAU["f16"], f"qmv batched exact path {kind} m={m}")


@pytest.mark.parametrize("kind", KINDS + ["q8_0"])
@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("m", [8, 16])
def test_qmv_batched_full_size_sampled(kq, kind, n, k, m):
    """The C2 GEMV shapes at batch 8 and 16 as the benchmark times them (fp16
    x and y), checked on sampled outputs the oracle computes one by one."""
    rng = synth.rng_for(5210 + m)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (m, k), "f16")
    _say("qmv batched full sampled", kind, n, k)
    got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", m, "f16")
    pn = np.concatenate([rng.integers(0, n, 120), [0, 15, 16, n - 1]])
    pm = np.concatenate([rng.integers(0, m, 120), [0, m - 1, 3, 7]])
    ref, s = oracle.qmm_points(kind, w, n, k, x, "f16", m, pm, pn)
    check_tol(got[pm, pn], ref, s, TAU["f16"], f"qmv batched full {kind} {n}x{k}", out_dt="f16")


@pytest.mark.parametrize("kind", KINDS + ["q8_0"])
@pytest.mark.parametrize("m", [3, 8])
@pytest.mark.parametrize("scale", [2.0**-20, 6.0e4])
def test_qmv_batched_activation_range(kq, kind, m, scale):
    """fp16 activations from subnormals to near the fp16 maximum through the
    matrix-core products (exact fp16 products, fp32 sums): within the bound."""
    n, k = 80, 4096
    rng = synth.rng_for(5220 + m)
    w = synth.weight_blocks(kind, rng, n, k)
    xf = rng.uniform(-1.0, 1.0, size=(m, k)).astype(np.float32) * np.float32(scale)
    x = xf.astype(np.float16).view(np.uint16)
    _say("qmv batched range", kind, m, scale)
    got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", m, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", m)
    check_tol(got, ref, s, TAU["f16"], f"qmv batched {kind} m={m} x scale {scale}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("scale", [2.0**-20, 1.0, 6.0e4])
def test_qmv_activation_range(kq, kind, m, scale):
    """fp16 activations from subnormals to near the fp16 maximum through the
    fp16 pair products (v_dot2_f32_f16): still within the bound."""
    n, k = 96, _k(kind, 128)
    rng = synth.rng_for(5150 + m)
    w = synth.weight_blocks(kind, rng, n, k)
    xf = rng.uniform(-1.0, 1.0, size=(m, k)).astype(np.float32) * np.float32(scale)
    x = xf.astype(np.float16).view(np.uint16)
    _say("qmv range", kind, m, scale)
    got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", m, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", m)
    check_tol(got, ref, s, TAU["f16"], f"qmv {kind} m={m} x scale {scale}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m", [17, 40, 130])
@pytest.mark.parametrize("fn", ["kq_qmm", "kq_qmm_ws", "kq_qmm_noalloc"])
def test_qmm(kq, kind, x_dt, m, fn):
    """m > 16 through the three prefill entry points: the matrix-core GEMM for
    fp16 and bf16 activations, the vector kernel for fp32."""
    n, k = 75, _k(kind, 72)
    rng = synth.rng_for(5200 + m)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (m, k), x_dt)
    _say("qmm", kind, x_dt, m, fn)
    got = _run(kq, fn, kind, w, n, k, x, x_dt, m, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, x_dt, m)
    check_tol(got, ref, s, TAU[x_dt], f"{fn} {kind} {x_dt} m={m}")


@pytest.mark.parametrize("kind", KINDS)
def test_one_hot_columns_exact(kq, kind):
    """x = e_c returns column c of the decoded weights, for every c: exactly in
    the vector-unit decode forms (m <= 16, fp32 and fp16 activations; 17
    blocks of 32 are no whole number of the batched matrix-core kernel's
    chunks, whose one-hot test is test_qmv_batched_one_hot_columns) and the
    fp32 prefill form, and as the weight rounded once to fp16 in the
    matrix-core prefill (m = k, fp16 activations)."""
    n, k = 40, _k(kind, 17)
    w = synth.weight_blocks(kind, synth.rng_for(5300), n, k)
    W64 = oracle.dequant(kind, w, n, k)
    W = W64.astype(np.float32)
    W16 = W64.astype(np.float16).astype(np.float32)  # one rounding of the exact weight
    for fn, m, x_dt in (("kq_qmv", 16, "f32"), ("kq_qmv", 16, "f16"), ("kq_qmm", k, "f32"),
                        ("kq_qmm", k, "f16")):
        ref = W16 if (fn == "kq_qmm" and x_dt == "f16") else W
        for c0 in range(0, k, m):
            mm = min(m, k - c0)
            x = np.zeros((mm, k), np.float32)
            x[np.arange(mm), c0 + np.arange(mm)] = 1.0
            _say("one-hot", kind, fn, x_dt, c0)
            xa = x if x_dt == "f32" else x.astype(np.float16).view(np.uint16)
            got = _run(kq, fn, kind, w, n, k, xa, x_dt, mm, "f32")
            assert np.array_equal(got, ref[:, c0:c0 + mm].T), (fn, x_dt, c0)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dt", ["f16", "bf16"])
@pytest.mark.parametrize("m,n,nb32", [(300, 200, 33), (512, 384, 64), (65, 1000, 136)])
@pytest.mark.parametrize("fn", ["kq_qmm", "kq_qmm_ws"])
def test_qmm_gemm(kq, kind, x_dt, m, n, nb32, fn):
    """The matrix-core prefill GEMM: several tiles with ragged edges; rows of
    an odd count of 32-weight blocks for the 32-weight codecs (a half step at
    the row end); K split over workgroups with a workspace (few tiles)."""
    k = 32 * nb32 if QK[kind] == 32 else 256 * max(1, nb32 // 8)
    rng = synth.rng_for(5250 + m)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (m, k), x_dt)
    _say("qmm gemm", kind, x_dt, m, n, k, fn)
    got = _run(kq, fn, kind, w, n, k, x, x_dt, m, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, x_dt, m)
    check_tol(got, ref, s, TAU[x_dt], f"gemm {fn} {kind} {x_dt} m={m} n={n} k={k}")


@pytest.mark.parametrize("kind", KINDS)
def test_qmm_gemm_large_weights_take_exact_path(kq, kind):
    """Blocks whose weights reach past the fp16 range (d = 30000 on a third of
    the rows) send their tiles to the exact fp32 path; the result still
    matches the oracle (fp16 activations)."""
    n, m = 96, 40
    k = 32 * 24 if QK[kind] == 32 else 512
    rng = synth.rng_for(5270)
    w = synth.weight_blocks(kind, rng, n, k)
    bb = synth.BLOCK_BYTES[kind]
    blocks = w.reshape(n, -1, bb)
    big = np.array([30000.0], np.float16).view(np.uint8)
    off = {"q4_0": 0, "q5_0": 0, "q5_1": 0, "q6_k": 208, "q2_k": 80, "q3_k": 108, "q5_k": 0}[kind]
    blocks[::3, :, off:off + 2] = big
    x = synth.activations(rng, (m, k), "f16")
    _say("qmm gemm exact path", kind)
    got = _run(kq, "kq_qmm", kind, w, n, k, x, "f16", m, "f32")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", m)
    check_tol(got, ref, s, TAU["f16"], f"gemm exact path {kind}")


# ---------------------------------------------------------------- expert-routed forms
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("mixed", [False, True])
@pytest.mark.parametrize("E,T,top_k", [(8, 1, 8), (8, 5, 3), (4, 70, 4)])
def test_qmm_id(kq, kind, x_dt, layout, mixed, E, T, top_k):
    n, k = 96, _k(kind, 16)
    rng = synth.rng_for(5400 + T)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k)).astype(np.float32)
    x_rows = T if layout == 0 else T * top_k
    x = synth.activations(rng, (x_rows, k), x_dt)
    _say("qmm_id", kind, x_dt, layout, mixed, E, T, top_k)
    y = empty((T if mixed else T * top_k, n), "f32")
    ws = _moe_ws(kq, E, T, top_k, n if mixed else 0)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x, x_dt), layout, to_dev(ids), T,
                 top_k, to_dev(scores) if mixed else None, y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, x_dt, layout == 1, ids, T, top_k,
                           scores if mixed else None)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"qmm_id {kind} {x_dt}")


def _glu_bound_ok(h, ref, tau, act, limit):
    """The GLU bound of the other codecs' tests (fp32 outputs): the gate and
    up products within tau of the oracle's, through max|act'| <= 1.13 and
    |act(g)|, plus one rounding of the stored value."""
    g, u, sg, su = ref["g"], ref["u"], ref["sg"], ref["su"]
    with np.errstate(over="ignore"):
        if act == 1:
            a_g = 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))
        else:
            gc = np.minimum(g, limit) if act == 2 else g
            a_g = gc / (1.0 + np.exp(-gc))
    comp = tau * (1.13 * np.abs(u) * sg + np.abs(a_g) * su)
    bound = comp * (1.0 + 2.0**-24) + 2.0**-24 * np.abs(ref["h"]) + 2.0**-150
    return not np.isnan(h).any() and bool((np.abs(h - ref["h"]) <= bound).all())


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("T", [1, 9, 40])
@pytest.mark.parametrize("act", [0, 1])
def test_moe_glu(kq, kind, x_dt, T, act):
    E, n, top_k = 6, 80, 3
    k = _k(kind, 16)
    rng = synth.rng_for(5500 + T)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T, k), x_dt)
    _say("moe_glu", kind, x_dt, T, act)
    h = empty((T, top_k, n), "f32")
    ws = _moe_ws(kq, E, T, top_k)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, x_dt), to_dev(ids),
                  T, top_k, h, ws, act)
    torch.cuda.synchronize()
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, x_dt, ids, T, top_k, act)
    assert _glu_bound_ok(to_f64(h), ref, TAU[x_dt], act, 0.0), f"moe_glu {kind} {x_dt} T={T}"


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("T", [1, 40])
def test_moe_glu_ex_shexp_silu_limit(kq, kind, T):
    """silu_limit and a shared expert in the last slot (kq_moe_glu_ex)."""
    E, n, top_k, limit = 6, 80, 3, 5.0
    k = _k(kind, 16)
    rng = synth.rng_for(5600 + T)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    sg = synth.weight_blocks(kind, rng, n, k)
    su = synth.weight_blocks(kind, rng, n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T, k), "f16")
    _say("moe_glu_ex", kind, T)
    h = empty((T, top_k + 1, n), "f32")
    ws = _moe_ws(kq, E + 1, T, top_k + 1)
    kq.kq_moe_glu_ex(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, "f16"),
                     to_dev(ids), T, top_k, h, ws, 2, limit, to_dev(sg), to_dev(su))
    torch.cuda.synchronize()
    ref = oracle.moe_glu_ex(kind, gate, up, E, n, k, stride, x, "f16", ids, T, top_k, 2, limit,
                            sg, su)
    assert _glu_bound_ok(to_f64(h), ref, TAU["f16"], 2, limit), f"glu_ex {kind} T={T}"


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("T", [1, 5, 40])
def test_qmm_id_mix_shexp(kq, kind, x_dt, T):
    E, top_k, n = 6, 3, 72
    k = _k(kind, 16)
    rng = synth.rng_for(5700 + T)
    w = synth.weight_blocks(kind, rng, E * n, k)
    wsh = synth.weight_blocks(kind, rng, n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T * (top_k + 1), k), x_dt)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k + 1)).astype(np.float32)
    _say("mix shexp", kind, x_dt, T)
    y = empty((T, n), "f32")
    ws = _moe_ws(kq, E + 1, T, top_k + 1, n)
    kq.kq_qmm_id_mix_shexp(kind, to_dev(w), E, n, k, stride, to_dev(wsh), to_dev(x, x_dt),
                           to_dev(ids), T, top_k, to_dev(scores), y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id_mix_shexp(kind, w, E, n, k, stride, wsh, x, x_dt, ids, T, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"mix shexp {kind} {x_dt} T={T}")


# ---------------------------------------------------------------- one token, routed, LDS stream
# One token with k a whole number of the single-token kernels' chunks (2048
# weights serve every codec): the gate/up form with the activation fused and
# the down projection with the weighted sum over slots, expert ids read
# directly, each slot's expert rows streamed through LDS.
ROUTED = KINDS + ["q8_0"]


@pytest.mark.parametrize("kind", ROUTED)
@pytest.mark.parametrize("act", [0, 1])
def test_moe_glu_one_token_lds(kq, kind, act):
    E, n, top_k, k = 6, 72, 3, 2048
    rng = synth.rng_for(5800 + act)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    x = synth.activations(rng, (1, k), "f16")
    _say("moe_glu one token", kind, act)
    h = empty((1, top_k, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, "f16"), to_dev(ids), 1, top_k,
                  h, ws, act)
    torch.cuda.synchronize()
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, "f16", ids, 1, top_k, act)
    assert _glu_bound_ok(to_f64(h), ref, TAU["f16"], act, 0.0), f"moe_glu one token {kind} act={act}"


@pytest.mark.parametrize("kind", ROUTED)
def test_moe_glu_ex_one_token_lds_shexp_silu_limit(kq, kind):
    E, n, top_k, k, limit = 6, 72, 3, 2048, 5.0
    rng = synth.rng_for(5810)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    sg = synth.weight_blocks(kind, rng, n, k)
    su = synth.weight_blocks(kind, rng, n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    x = synth.activations(rng, (1, k), "f16")
    _say("moe_glu_ex one token", kind)
    h = empty((1, top_k + 1, n), "f32")
    ws = _moe_ws(kq, E + 1, 1, top_k + 1)
    kq.kq_moe_glu_ex(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, "f16"), to_dev(ids), 1, top_k,
                     h, ws, 2, limit, to_dev(sg), to_dev(su))
    torch.cuda.synchronize()
    ref = oracle.moe_glu_ex(kind, gate, up, E, n, k, stride, x, "f16", ids, 1, top_k, 2, limit, sg, su)
    assert _glu_bound_ok(to_f64(h), ref, TAU["f16"], 2, limit), f"glu_ex one token {kind}"


@pytest.mark.parametrize("kind", ["q4_0", "q6_k", "q8_0"])
def test_moe_glu_one_token_lds_invalid_id(kq, kind):
    """A slot whose id is out of range gets NaN rows; the other slots are
    computed."""
    E, n, top_k, k = 6, 40, 3, 2048
    rng = synth.rng_for(5820)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = np.array([[2, E + 3, 0]], np.uint32)
    x = synth.activations(rng, (1, k), "f16")
    _say("moe_glu one token invalid", kind)
    h = empty((1, top_k, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, "f16"), to_dev(ids), 1, top_k,
                  h, ws, 0)
    torch.cuda.synchronize()
    got = to_f64(h)
    assert np.isnan(got[0, 1]).all()
    ok_ids = np.array([[2, 0, 0]], np.uint32)
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, "f16", ok_ids, 1, top_k, 0)
    for slot in (0, 2):
        sub = {key: ref[key][:, slot:slot + 1] for key in ("g", "u", "sg", "su", "h")}
        assert _glu_bound_ok(got[:, slot:slot + 1], sub, TAU["f16"], 0, 0.0), f"{kind} slot {slot}"


@pytest.mark.parametrize("kind", ROUTED)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("n", [72, 2100])
def test_qmm_id_mixed_one_token_lds(kq, kind, x_dt, layout, n):
    """fp32 rows are split into fp16 hi + lo in the workspace's slot buffer
    when top_k * n * 4 bytes hold them (n = 2100), else by each workgroup
    (n = 72)."""
    E, top_k, k = 6, 3, 2048
    rng = synth.rng_for(5830 + layout + n)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(1, top_k)).astype(np.float32)
    x = synth.activations(rng, (1 if layout == 0 else top_k, k), x_dt)
    _say("qmm_id mixed one token", kind, x_dt, layout)
    y = empty((1, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k, n)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x, x_dt), layout, to_dev(ids), 1, top_k,
                 to_dev(scores), y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, x_dt, layout == 1, ids, 1, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"qmm_id mixed one token {kind} {x_dt} layout {layout}")


@pytest.mark.parametrize("kind", ROUTED)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
def test_qmm_id_mix_shexp_one_token_lds(kq, kind, x_dt):
    E, top_k, n, k = 6, 3, 72, 2048
    rng = synth.rng_for(5840)
    w = synth.weight_blocks(kind, rng, E * n, k)
    wsh = synth.weight_blocks(kind, rng, n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    x = synth.activations(rng, (top_k + 1, k), x_dt)
    scores = rng.uniform(0.05, 1.0, size=(1, top_k + 1)).astype(np.float32)
    _say("mix shexp one token", kind, x_dt)
    y = empty((1, n), "f32")
    ws = _moe_ws(kq, E + 1, 1, top_k + 1, n)
    kq.kq_qmm_id_mix_shexp(kind, to_dev(w), E, n, k, stride, to_dev(wsh), to_dev(x, x_dt), to_dev(ids), 1,
                           top_k, to_dev(scores), y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id_mix_shexp(kind, w, E, n, k, stride, wsh, x, x_dt, ids, 1, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"mix shexp one token {kind} {x_dt}")


@pytest.mark.parametrize("kind", ["q4_0", "q5_1", "q6_k", "q2_k", "q8_0"])
@pytest.mark.parametrize("n", [48, 2100])
def test_qmm_id_mixed_one_token_lds_fp32_range(kq, kind, n):
    """fp32 slot rows at very different magnitudes (1e-30, 1e-3, 1e5, and a
    row of zeros): each row is split into fp16 hi + lo at its own power of
    two (in the workgroups, and beforehand into the workspace), within
    tau = 1e-5."""
    E, top_k, k = 6, 4, 2048
    rng = synth.rng_for(5850)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(1, top_k)).astype(np.float32)
    x = rng.standard_normal((top_k, k)).astype(np.float32)
    x *= np.array([[1e-30], [1e-3], [1e5], [0.0]], np.float32)
    _say("qmm_id one token fp32 range", kind)
    y = empty((1, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k, n)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x), 1, to_dev(ids), 1, top_k, to_dev(scores), y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, "f32", True, ids, 1, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU["f32"], f"qmm_id one token fp32 range {kind}")


@pytest.mark.parametrize("kind", ["q4_0", "q6_k", "q8_0"])
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("n", [40, 2100])
def test_qmm_id_mixed_one_token_lds_invalid_id(kq, kind, x_dt, n):
    """An out-of-range id makes the token's whole output NaN."""
    E, top_k, k = 6, 3, 2048
    rng = synth.rng_for(5860)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = np.array([[1, 4, E]], np.uint32)
    scores = np.full((1, top_k), 0.5, np.float32)
    x = synth.activations(rng, (top_k, k), x_dt)
    _say("qmm_id one token invalid", kind, x_dt)
    y = empty((1, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k, n)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x, x_dt), 1, to_dev(ids), 1, top_k, to_dev(scores),
                 y, ws)
    torch.cuda.synchronize()
    assert np.isnan(to_f64(y)).all()


@pytest.mark.parametrize("kind", ["q4_0", "q8_0", "q6_k", "q5_k"])
def test_moe_one_token_c4_shapes(kq, kind):
    """One token through a whole layer at the C4 matrix shapes (8 experts,
    top-8, gate/up 2048x7168, down 7168x2048, fp32 h): every output against
    the oracle."""
    E, top_k, H, F = 8, 8, 7168, 2048
    rng = synth.rng_for(5870)
    gate = synth.weight_blocks(kind, rng, E * F, H)
    up = synth.weight_blocks(kind, rng, E * F, H)
    down = synth.weight_blocks(kind, rng, E * H, F)
    gs, ds = F * synth.row_bytes(kind, H), H * synth.row_bytes(kind, F)
    ids = _ids(rng, 1, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(1, top_k)).astype(np.float32)
    x = synth.activations(rng, (1, H), "f16")
    _say("moe one token C4 shapes", kind)
    h = empty((1, top_k, F), "f32")
    ws = _moe_ws(kq, E, 1, top_k, H)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, F, H, gs, to_dev(x, "f16"), to_dev(ids), 1, top_k, h, ws)
    out = empty((1, H), "f32")
    kq.kq_qmm_id(kind, to_dev(down), E, H, F, ds, h, 1, to_dev(ids), 1, top_k, to_dev(scores), out, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_glu(kind, gate, up, E, F, H, gs, x, "f16", ids, 1, top_k, 0)
    hg = to_f64(h)
    assert _glu_bound_ok(hg, ref, TAU["f16"], 0, 0.0), f"C4 glu {kind}"
    # the down projection against the oracle on the h the GPU produced
    hx = hg.astype(np.float32).reshape(top_k, F)
    yref, s = oracle.qmm_id(kind, down, E, H, F, ds, hx, "f32", True, ids, 1, top_k, scores)
    check_tol(to_f64(out), yref, s, TAU["f32"], f"C4 down {kind}")


# ---------------------------------------------------------------- Q6_K / Q3_K by 4-byte copies
# Rows that are no whole number of the 16-byte-copy unit (8 super-blocks)
# stream by 4-byte copies in chunks of 1024 weights (k a multiple of 1024) or
# 512: the one-row GEMV and the single-token MoE forms.
@pytest.mark.parametrize("kind", ["q6_k", "q3_k"])
@pytest.mark.parametrize("n,k", [(16, 512), (45, 1536), (300, 5120), (33, 7168), (70, 4608)])
def test_qmv_one_row_dword_stream(kq, kind, n, k):
    rng = synth.rng_for(5900 + n)
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (1, k), "f16")
    ref, s = oracle.qmm(kind, w, n, k, x, "f16", 1)
    for y_dt in ("f32", "f16", "bf16"):
        _say("qmv one row dword", kind, n, k, y_dt)
        got = _run(kq, "kq_qmv", kind, w, n, k, x, "f16", 1, y_dt)
        check_tol(got, ref, s, TAU["f16"], f"qmv one row dword {kind} {n}x{k} y={y_dt}",
                  out_dt=y_dt if y_dt != "f32" else None)
    assert np.array_equal(got, _run(kq, "kq_qmm_noalloc", kind, w, n, k, x, "f16", 1, "bf16"))


@pytest.mark.parametrize("kind", ["q6_k", "q3_k"])
@pytest.mark.parametrize("k", [7168, 2560])
def test_moe_glu_one_token_dword_stream(kq, kind, k):
    E, n, top_k = 6, 72, 3
    rng = synth.rng_for(5910 + k)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    x = synth.activations(rng, (1, k), "f16")
    _say("moe_glu one token dword", kind, k)
    h = empty((1, top_k, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, "f16"), to_dev(ids), 1, top_k,
                  h, ws, 0)
    torch.cuda.synchronize()
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, "f16", ids, 1, top_k, 0)
    assert _glu_bound_ok(to_f64(h), ref, TAU["f16"], 0, 0.0), f"moe_glu one token dword {kind} k={k}"


@pytest.mark.parametrize("kind", ["q6_k", "q3_k"])
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("k", [3072, 1536])
def test_qmm_id_mixed_one_token_dword_stream(kq, kind, x_dt, k):
    """n = 3100 >= k: fp32 rows are split beforehand into the workspace."""
    E, top_k, n = 6, 3, 3100
    rng = synth.rng_for(5920 + k)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, 1, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(1, top_k)).astype(np.float32)
    x = synth.activations(rng, (top_k, k), x_dt)
    _say("qmm_id mixed one token dword", kind, x_dt, k)
    y = empty((1, n), "f32")
    ws = _moe_ws(kq, E, 1, top_k, n)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x, x_dt), 1, to_dev(ids), 1, top_k, to_dev(scores),
                 y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, x_dt, True, ids, 1, top_k, scores)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"qmm_id mixed one token dword {kind} {x_dt} k={k}")


# ---------------------------------------------------------------- routed tiles on the matrix cores
# Routings over a schedule (more than one token), k a whole number of 512
# weights: the tile kernel (up to 32 gathered rows per tile, ragged tiles).
@pytest.mark.parametrize("kind", ROUTED)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("act", [0, 1])
def test_moe_glu_routed_tiles(kq, kind, x_dt, act):
    E, n, top_k, T, k = 8, 200, 4, 24, 1536
    rng = synth.rng_for(5950 + act)
    gate = synth.weight_blocks(kind, rng, E * n, k)
    up = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    x = synth.activations(rng, (T, k), x_dt)
    _say("moe_glu routed tiles", kind, x_dt, act)
    h = empty((T, top_k, n), "f32")
    ws = _moe_ws(kq, E, T, top_k)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, n, k, stride, to_dev(x, x_dt), to_dev(ids), T, top_k, h, ws,
                  act)
    torch.cuda.synchronize()
    ref = oracle.moe_glu(kind, gate, up, E, n, k, stride, x, x_dt, ids, T, top_k, act)
    assert _glu_bound_ok(to_f64(h), ref, TAU[x_dt], act, 0.0), f"moe_glu routed {kind} {x_dt} act={act}"


@pytest.mark.parametrize("kind", ROUTED)
@pytest.mark.parametrize("x_dt", ["f16", "f32"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("mixed", [False, True])
def test_qmm_id_routed_tiles(kq, kind, x_dt, layout, mixed):
    """Four experts and 70 tokens of top-4: about 70 rows per expert, tiles
    of 32, 32 and a ragged one."""
    E, top_k, T, n, k = 4, 4, 70, 136, 1024
    rng = synth.rng_for(5960 + layout)
    w = synth.weight_blocks(kind, rng, E * n, k)
    stride = n * synth.row_bytes(kind, k)
    ids = _ids(rng, T, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k)).astype(np.float32)
    x = synth.activations(rng, (T if layout == 0 else T * top_k, k), x_dt)
    _say("qmm_id routed tiles", kind, x_dt, layout, mixed)
    y = empty((T if mixed else T * top_k, n), "f32")
    ws = _moe_ws(kq, E, T, top_k, n if mixed else 0)
    kq.kq_qmm_id(kind, to_dev(w), E, n, k, stride, to_dev(x, x_dt), layout, to_dev(ids), T, top_k,
                 to_dev(scores) if mixed else None, y, ws)
    torch.cuda.synchronize()
    ref, s = oracle.qmm_id(kind, w, E, n, k, stride, x, x_dt, layout == 1, ids, T, top_k,
                           scores if mixed else None)
    check_tol(to_f64(y), ref, s, TAU[x_dt], f"qmm_id routed {kind} {x_dt} layout {layout} mixed {mixed}")


@pytest.mark.parametrize("kind", ["q4_0", "q8_0", "q6_k", "q2_k"])
def test_moe_prefill_c4_shapes_sampled_tokens(kq, kind):
    """A 256-token layer at the C4 matrix shapes (32 experts, top-8, fp16 x,
    fp32 h) with the schedule reused by the down projection, as the benchmark
    times it; tokens 0, 97 and 255 against the oracle."""
    E, top_k, H, F, T = 32, 8, 7168, 2048, 256
    rng = synth.rng_for(5970)
    gate = synth.weight_blocks(kind, rng, E * F, H)
    up = synth.weight_blocks(kind, rng, E * F, H)
    down = synth.weight_blocks(kind, rng, E * H, F)
    gs, ds = F * synth.row_bytes(kind, H), H * synth.row_bytes(kind, F)
    ids = _ids(rng, T, E, top_k)
    scores = rng.uniform(0.05, 1.0, size=(T, top_k)).astype(np.float32)
    x = synth.activations(rng, (T, H), "f16")
    _say("moe prefill C4 shapes", kind)
    h = empty((T, top_k, F), "f32")
    out = empty((T, H), "f32")
    ws = _moe_ws(kq, E, T, top_k, H)
    idd = to_dev(ids)
    kq.kq_moe_glu(kind, to_dev(gate), to_dev(up), E, F, H, gs, to_dev(x, "f16"), idd, T, top_k, h, ws)
    kq.kq_qmm_id(kind, to_dev(down), E, H, F, ds, h, kq.LAYOUT_SLOTTED | kq.REUSE_SCHEDULE, idd, T, top_k,
                 to_dev(scores), out, ws)
    torch.cuda.synchronize()
    hg, og = to_f64(h), to_f64(out)
    for t in (0, 97, 255):
        ref = oracle.moe_glu(kind, gate, up, E, F, H, gs, x[t:t + 1], "f16", ids[t:t + 1], 1, top_k, 0)
        assert _glu_bound_ok(hg[t:t + 1], ref, TAU["f16"], 0, 0.0), f"prefill glu {kind} token {t}"
        hx = hg[t].astype(np.float32)
        yref, s = oracle.qmm_id(kind, down, E, H, F, ds, hx, "f32", True, ids[t:t + 1], 1, top_k, scores[t:t + 1])
        check_tol(og[t:t + 1], yref, s, TAU["f32"], f"prefill down {kind} token {t}")
