"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, hand-worked examples from the pages (tests/golden), library
routines (numpy/torch casts, numpy matmul), brute force on tiny inputs, and
invariants.  CPU only.
"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from tests import npdecode as npd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------------------------ scalars
def test_half_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_to_double(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _f32_probe_values():
    rng = _rng(1)
    rand_bits = rng.integers(0, 2**32, size=60000, dtype=np.uint64).astype(np.uint32)
    vals = [rand_bits.view(np.float32)]
    # every binade of the fp16/bf16 ranges, with halfway and near-halfway points
    for e in range(-30, 20):
        base = np.float64(2.0) ** e
        frac = rng.integers(0, 2**23, size=200)
        vals.append((base * (1 + frac / 2**23)).astype(np.float32))
        # exact ties for fp16 (11 bits) and bf16 (8 bits) grids
        for p in (11, 8):
            k = rng.integers(0, 2 ** (p - 1), size=50)
            vals.append((base * (1 + (k + 0.5) / 2 ** (p - 1))).astype(np.float32))
    special = np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 65536.0, 1e9, -1e9,
                        2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-14, 2.0**-15, np.inf, -np.inf,
                        3.3895313892515355e38, 3.4e38], dtype=np.float32)
    vals.append(special)
    v = np.concatenate(vals).astype(np.float32)
    return v[~np.isnan(v)]


def test_f32_to_half_rne_matches_numpy(orc):
    v = _f32_probe_values()
    with np.errstate(over="ignore"):  # the probes include values past the fp16 range (-> inf)
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([orc.float_to_half_rne(x) for x in v], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    assert orc.float_to_half_rne(float("nan")) & 0x7C00 == 0x7C00


def test_f32_to_bf16_rne_matches_torch(orc):
    v = _f32_probe_values()
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.float_to_bf16_rne(x) for x in v], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ------------------------------------------------------------------ Q4_K
def _q4k_block(d=1.0, dmin=0.0, S=None, Q=None):
    b = np.zeros(144, dtype=np.uint8)
    b[0:2] = np.array([d], dtype=np.float16).view(np.uint8)
    b[2:4] = np.array([dmin], dtype=np.float16).view(np.uint8)
    b[4:16] = np.zeros(12, np.uint8) if S is None else np.asarray(S, np.uint8)
    b[16:144] = np.zeros(128, np.uint8) if Q is None else np.asarray(Q, np.uint8)
    return b


def test_q4k_identity_block(orc):
    """d = 1, dmin = 0, every scale 1 and every min 0: weights are the quants.
    Low nibbles of chunk c are weights 64c..64c+31, high nibbles 64c+32..."""
    Q = (np.arange(128) * 37 + 11) % 256
    b = _q4k_block(1.0, 0.0, [1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], Q)
    w = orc.dequant("q4_k", b, 1, 256)[0]
    expect = np.empty(256)
    for c in range(4):
        for l in range(32):
            expect[64 * c + l] = Q[32 * c + l] & 15
            expect[64 * c + 32 + l] = Q[32 * c + l] >> 4
    assert np.array_equal(w, expect)
    for j in range(8):
        assert orc.q4k_scale_min(b[4:16], j) == (1, 0)


def test_q4k_zero_nibbles_give_minus_dmin_m(orc):
    rng = _rng(2)
    m = rng.integers(0, 64, size=(1, 8))
    sc = rng.integers(0, 64, size=(1, 8))
    blk = npd.q4k_pack(np.array([0.0123], np.float16), np.array([0.00731], np.float16), sc, m,
                       np.zeros((1, 256), np.int64))
    w = orc.dequant("q4_k", blk, 1, 256)[0]
    dmin = float(np.float16(0.00731))
    for j in range(8):
        assert np.all(w[32 * j:32 * j + 32] == -dmin * m[0, j])


@pytest.mark.parametrize("field", range(16))
def test_q4k_single_field_probe(orc, field):
    """Setting one 6-bit field changes exactly one sub-block, by that field."""
    is_min, j = divmod(field, 8)
    for v in (1, 5, 16, 33, 63):
        sc = np.zeros((1, 8), np.int64)
        m = np.zeros((1, 8), np.int64)
        (m if is_min else sc)[0, j] = v
        blk = npd.q4k_pack(np.array([1.0], np.float16), np.array([1.0], np.float16), sc, m,
                           np.ones((1, 256), np.int64))
        w = orc.dequant("q4_k", blk, 1, 256)[0]
        expect = np.zeros(256)
        expect[32 * j:32 * j + 32] = -v if is_min else v
        assert np.array_equal(w, expect), (field, v)
        for jj in range(8):
            got = orc.q4k_scale_min(blk[0, 4:16], jj)
            want = (v if (jj == j and not is_min) else 0, v if (jj == j and is_min) else 0)
            assert got == want


def test_q4k_round_trip_tiny_matrix(orc):
    """Chosen fields -> packed bytes -> oracle decode == d*sc*q - dmin*m."""
    rng = _rng(3)
    rows, k = 4, 512
    nb = rows * k // 256
    d = rng.uniform(1e-3, 2e-2, nb).astype(np.float16)
    dmin = rng.uniform(1e-3, 2e-2, nb).astype(np.float16)
    sc = rng.integers(0, 64, size=(nb, 8))
    m = rng.integers(0, 64, size=(nb, 8))
    q = rng.integers(0, 16, size=(nb, 256))
    blk = npd.q4k_pack(d, dmin, sc, m, q)
    w = orc.dequant("q4_k", blk.reshape(rows, -1), rows, k).reshape(nb, 256)
    for b in range(nb):
        for i in range(256):
            j = i // 32
            want = float(d[b]) * int(sc[b, j]) * int(q[b, i]) - float(dmin[b]) * int(m[b, j])
            assert w[b, i] == want


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
def test_independent_decoders_agree(orc, kind):
    """C oracle and the vectorised numpy decoder agree bit for bit on random
    blocks (Q4_K with arbitrary fp16 d/dmin bit patterns, not just the
    generator's range)."""
    import synth

    rng = _rng(4)
    rows, k = 400, 256 * 1  # 400 Q4_K blocks; more for the smaller formats
    k = {"q4_k": 256 * 250, "q8_0": 32 * 250, "tq1_g128": 128 * 250}[kind]
    w = synth.weight_blocks(kind, rng, rows, k)
    if kind == "q4_k":
        # also cover arbitrary finite fp16 d/dmin (exponents across the range)
        blocks = w.reshape(-1, 144)
        half = rng.integers(0, 0x7BFF, size=(blocks.shape[0], 2)).astype(np.uint16)
        sign = rng.integers(0, 2, size=(blocks.shape[0], 2)).astype(np.uint16) << 15
        blocks[::2, 0:4] = (half | sign)[::2].astype("<u2").view(np.uint8)
    got = orc.dequant(kind, w, rows, k)
    ref = npd.decode_matrix(kind, w, rows, k)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ Q8_0
def test_q8_0_golden_block(orc):
    lines = [ln for ln in open(os.path.join(GOLDEN, "q8_0_block.txt")) if not ln.startswith("#")]
    blk = np.array([int(t, 16) for t in lines[0].split()[1:]], dtype=np.uint8)
    want = np.array([float(t) for t in lines[1].split()[1:]])
    assert blk.size == 34 and want.size == 32
    assert np.array_equal(orc.dequant("q8_0", blk, 1, 32)[0], want)


def test_q8_0_all_quant_values(orc):
    for d in (1.0, 0.0137):
        blk = np.zeros((8, 34), np.uint8)
        blk[:, 0:2] = np.array([d], np.float16).view(np.uint8)
        blk[:, 2:34] = np.arange(256, dtype=np.uint32).astype(np.uint8).reshape(8, 32)
        w = orc.dequant("q8_0", blk.reshape(1, -1), 1, 256)[0]
        q = np.arange(256, dtype=np.uint32).astype(np.uint8).view(np.int8).astype(np.float64)
        assert np.array_equal(w, float(np.float16(d)) * q)


# ------------------------------------------------------------------ TQ1
def _golden_rows(name):
    rows = []
    for ln in open(os.path.join(GOLDEN, name)):
        if ln.strip() and not ln.startswith("#"):
            rows.append(ln.split())
    return rows


def test_tq1_golden_codes(orc):
    for kind, code, *trits in _golden_rows("tq1_codes.txt"):
        trits = [int(t) for t in trits]
        blk = np.zeros(28, np.uint8)
        blk[0:25] = 121  # all-zero trits elsewhere
        blk[25] = 13
        blk[26:28] = np.array([1.0], np.float16).view(np.uint8)
        if kind == "full":
            blk[7] = int(code)
            w = orc.dequant("tq1_g128", blk, 1, 128)[0]
            assert list(w[35:40]) == trits
            assert np.all(np.delete(w, range(35, 40)) == 0)
        else:
            blk[25] = int(code)
            w = orc.dequant("tq1_g128", blk, 1, 128)[0]
            assert list(w[125:128]) == trits
            assert np.all(w[:125] == 0)


def test_tq1_golden_columns(orc):
    for col, slot, digit in _golden_rows("tq1_columns.txt"):
        col, slot, digit = int(col), int(slot), int(digit)
        blk = np.zeros(28, np.uint8)
        blk[0:25] = 121
        blk[25] = 13
        blk[26:28] = np.array([2.0], np.float16).view(np.uint8)
        blk[slot] += 3 ** digit  # raise exactly that digit from 1 to 2
        w = orc.dequant("tq1_g128", blk, 1, 128)[0]
        assert w[col] == 2.0 and np.count_nonzero(w) == 1


def test_tq1_brute_force_all_codes(orc):
    """Every legal full (0..242) and tail (0..26) byte: the decoded digits
    recompose to the byte."""
    for code in range(243):
        blk = np.zeros(28, np.uint8)
        blk[0:25] = code
        blk[25] = code % 27
        blk[26:28] = np.array([1.0], np.float16).view(np.uint8)
        w = orc.dequant("tq1_g128", blk, 1, 128)[0]
        digits = (w + 1).astype(int)
        for s in range(25):
            assert sum(int(digits[5 * s + i]) * 3 ** i for i in range(5)) == code
        assert sum(int(digits[125 + i]) * 3 ** i for i in range(3)) == code % 27


def test_tq1_scale_and_byte_accounting(orc):
    rng = _rng(5)
    trits = rng.integers(-1, 2, size=(64, 128))
    s = rng.uniform(1e-3, 2e-2, 64).astype(np.float16)
    blk = npd.tq1_pack(trits, s)
    assert blk.shape == (64, 28)  # 28 bytes per 128 weights
    assert blk.size * 8 / trits.size == 1.75
    w = orc.dequant("tq1_g128", blk.reshape(1, -1), 1, 64 * 128).reshape(64, 128)
    assert np.array_equal(w, trits * s.astype(np.float64)[:, None])
    # scale 1 gives the trits exactly
    blk1 = npd.tq1_pack(trits, np.ones(64, np.float16))
    w1 = orc.dequant("tq1_g128", blk1.reshape(1, -1), 1, 64 * 128).reshape(64, 128)
    assert np.array_equal(w1, trits)


def test_lut23_split_identity():
    """(p * 57) >> 9 == p // 9 for every p <= 511 (the LUT23 split of a code
    byte into its low two and high three trits)."""
    for p in range(512):
        assert (p * 57) >> 9 == p // 9


# ------------------------------------------------------------------ stored dequant
@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_dequant_store_is_rounded_exact_value(orc, kind, dt):
    import synth

    rng = _rng(6)
    rows, k = 16, {"q4_k": 512, "q8_0": 512, "tq1_g128": 512}[kind]
    w = synth.weight_blocks(kind, rng, rows, k)
    exact = npd.decode_matrix(kind, w, rows, k)
    got = orc.dequant_as(kind, w, rows, k, dt)
    f32 = exact.astype(np.float32)  # numpy's double->float cast is RNE
    if dt == "f32":
        assert np.array_equal(got, f32)
    elif dt == "f16":
        assert np.array_equal(got, f32.astype(np.float16).view(np.uint16))
    else:
        ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref)


# ------------------------------------------------------------------ products
@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
def test_qmm_one_hot_columns(orc, kind):
    """x = e_c gives y[., n] = w[n, c] exactly, for every c."""
    import synth

    rng = _rng(7)
    n, k = 5, 256
    w = synth.weight_blocks(kind, rng, n, k)
    x = np.eye(k, dtype=np.float32)
    y, s = orc.qmm(kind, w, n, k, x, "f32", k)
    W = npd.decode_matrix(kind, w, n, k)
    assert np.array_equal(y, W.T)
    assert np.array_equal(s, np.abs(W.T))


def test_qmm_integer_case(orc):
    """Identity Q4_K blocks and x = 1: y is the exact integer sum of nibbles."""
    rng = _rng(8)
    n, k = 6, 512
    Q = rng.integers(0, 256, size=(n * 2, 128))
    blocks = np.stack([_q4k_block(1.0, 0.0, [1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], q) for q in Q])
    x = np.ones((1, k), np.float32)
    y, _ = orc.qmm("q4_k", blocks.reshape(n, -1), n, k, x, "f32", 1)
    nib = (Q & 15) + (Q >> 4)
    assert np.array_equal(y[0], nib.reshape(n, -1).sum(axis=1).astype(np.float64))


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_qmm_brute_force_vs_numpy(orc, kind, dt):
    import synth

    rng = _rng(9)
    m, n, k = 3, 40, 512
    w = synth.weight_blocks(kind, rng, n, k)
    x = synth.activations(rng, (m, k), dt)
    y, s = orc.qmm(kind, w, n, k, x, dt, m)
    W = npd.decode_matrix(kind, w, n, k)
    X = npd.act_f64(x, dt)
    ref = X @ W.T
    sref = np.abs(X) @ np.abs(W.T)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * sref.max())
    assert np.allclose(s, sref, rtol=1e-13)
    # sampled points agree with the full product exactly (same sum order)
    pm = rng.integers(0, m, 20)
    pn = rng.integers(0, n, 20)
    yp, sp = orc.qmm_points(kind, w, n, k, x, dt, m, pm, pn)
    assert np.array_equal(yp, y[pm, pn]) and np.array_equal(sp, s[pm, pn])


# ------------------------------------------------------------------ expert-routed
def _moe_small(kind="q4_k", E=4, n=64, k=256, T=3, top_k=2, seed=10):
    import synth

    rng = _rng(seed)
    w = synth.weight_blocks(kind, rng, E * n, k)  # [E*n, row_bytes] == [E][n][.]
    stride = n * synth.row_bytes(kind, k)
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.uint32)
    scores = rng.uniform(0.1, 1.0, size=(T, top_k)).astype(np.float32)
    return rng, w, stride, ids, scores


def test_qmm_id_reduces_to_dense_for_one_expert(orc):
    import synth

    rng = _rng(11)
    n, k, T = 48, 512, 5
    w = synth.weight_blocks("q4_k", rng, n, k)
    x = synth.activations(rng, (T, k), "f16")
    ids = np.zeros((T, 1), np.uint32)
    y, s = orc.qmm_id("q4_k", w, 1, n, k, w.nbytes, x, "f16", False, ids, T, 1)
    yd, sd = orc.qmm("q4_k", w, n, k, x, "f16", T)
    assert np.array_equal(y, yd) and np.array_equal(s, sd)
    ys, _ = orc.qmm_id("q4_k", w, 1, n, k, w.nbytes, x, "f16", False, ids, T, 1,
                       scores=np.ones((T, 1), np.float32))
    assert np.array_equal(ys, yd)


def test_qmm_id_brute_force_and_invariants(orc):
    import synth

    E, n, k, T, top_k = 4, 64, 256, 3, 2
    rng, w, stride, ids, scores = _moe_small(E=E, n=n, k=k, T=T, top_k=top_k)
    x = synth.activations(rng, (T, top_k, k), "f16")
    y, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", True, ids, T, top_k)
    W = npd.decode_matrix("q4_k", w, E * n, k).reshape(E, n, k)
    X = npd.act_f64(x, "f16")
    for t in range(T):
        for r in range(top_k):
            ref = W[ids[t, r]] @ X[t, r]
            assert np.allclose(y[t * top_k + r], ref, rtol=0, atol=1e-12 * np.abs(ref).sum())
    mixed, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", True, ids, T, top_k, scores)
    for t in range(T):
        ref = sum(float(scores[t, r]) * (W[ids[t, r]] @ X[t, r]) for r in range(top_k))
        assert np.allclose(mixed[t], ref, rtol=0, atol=1e-12 * np.abs(ref).sum())
    # slot permutation invariance of the mixed form (up to summation order)
    p = [1, 0]
    mixed_p, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x[:, p], "f16", True, ids[:, p], T,
                            top_k, scores[:, p])
    assert np.allclose(mixed_p, mixed, rtol=1e-13, atol=1e-13)
    # one-hot router weights select one expert's rows
    oh = np.zeros_like(scores)
    oh[:, 1] = 1.0
    sel, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", True, ids, T, top_k, oh)
    assert np.array_equal(sel, y[1::top_k])


def test_qmm_id_invalid_id_poisons_its_row(orc):
    import synth

    E, n, k, T, top_k = 4, 32, 256, 3, 2
    rng, w, stride, ids, scores = _moe_small(E=E, n=n, k=k, T=T, top_k=top_k)
    ids = ids.copy()
    ids[1, 0] = E + 3
    x = synth.activations(rng, (T, k), "f16")
    y, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, ids, T, top_k)
    assert np.all(np.isnan(y[2])) and np.all(np.isfinite(np.delete(y, 2, axis=0)))
    ym, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, ids, T, top_k, scores)
    assert np.all(np.isnan(ym[1])) and np.all(np.isfinite(ym[[0, 2]]))


def test_silu_definition(orc):
    from scipy.special import expit

    for z in np.linspace(-30, 30, 241):
        assert orc.silu(z) == pytest.approx(z * expit(z), rel=1e-14, abs=1e-300)
    assert orc.silu(0.0) == 0.0


def test_gelu_tanh_pins(orc):
    """GELU's tanh approximation (mlx-kquant "bindings.cpp", moe_glu_gather_kq,
    act='gelu') against facts that do not restate its formula: the identity
    gelu(z) - gelu(-z) = z (1/2 (1 + tanh y) + 1/2 (1 - tanh y) = 1), slope 1/2
    at 0 and the limits z and 0, and the known closeness of the approximation to
    the exact GELU z * Phi(z) (a dropped cubic term is off by 0.03 at z = 2)."""
    from scipy.special import erf

    zs = np.linspace(-12.0, 12.0, 961)
    for z in zs:
        assert orc.gelu_tanh(z) - orc.gelu_tanh(-z) == pytest.approx(z, rel=1e-14, abs=1e-14)
    assert orc.gelu_tanh(0.0) == 0.0
    assert orc.gelu_tanh(1e-8) / 1e-8 == pytest.approx(0.5, abs=1e-7)
    assert orc.gelu_tanh(40.0) == 40.0 and abs(orc.gelu_tanh(-40.0)) < 1e-300
    exact = 0.5 * zs * (1.0 + erf(zs / np.sqrt(2.0)))
    diff = np.abs(np.array([orc.gelu_tanh(z) for z in zs]) - exact)
    assert diff.max() < 1e-3 and diff.max() > 1e-5  # the approximation, not the exact function


def test_moe_glu_act_selects_the_activation(orc):
    """h = act(g) * u with the g and u the oracle returns: act 0 silu, act 1
    gelu (tanh approximation); an unknown act is rejected."""
    import synth

    rng = _rng(31)
    E, n, k, T, top_k = 3, 24, 256, 2, 2
    gate = synth.weight_blocks("q4_k", rng, E * n, k)
    up = synth.weight_blocks("q4_k", rng, E * n, k)
    stride = n * synth.row_bytes("q4_k", k)
    x = synth.activations(rng, (T, k), "f16")
    ids = np.array([[0, 2], [1, 0]], np.uint32)
    for act, fn in ((0, orc.silu), (1, orc.gelu_tanh)):
        r = orc.moe_glu("q4_k", gate, up, E, n, k, stride, x, "f16", ids, T, top_k, act)
        want = np.vectorize(fn)(r["g"]) * r["u"]
        assert np.allclose(r["h"], want, rtol=1e-14, atol=0.0)
    with pytest.raises(ValueError):
        orc.moe_glu("q4_k", gate, up, E, n, k, stride, x, "f16", ids, T, top_k, 7)


def test_moe_layer_one_expert_is_dense_composition(orc):
    import synth

    rng = _rng(12)
    H, F, T = 512, 256, 3
    gate = synth.weight_blocks("q4_k", rng, F, H)
    up = synth.weight_blocks("q4_k", rng, F, H)
    down = synth.weight_blocks("q4_k", rng, H, F)
    x = synth.activations(rng, (T, H), "f16")
    ids = np.zeros((T, 1), np.uint32)
    out, s = orc.moe_layer("q4_k", gate, up, down, 1, H, F, gate.nbytes, down.nbytes, x, "f16",
                           ids, T, 1, np.ones((T, 1), np.float32))
    Wg = npd.decode_matrix("q4_k", gate, F, H)
    Wu = npd.decode_matrix("q4_k", up, F, H)
    Wd = npd.decode_matrix("q4_k", down, H, F)
    X = npd.act_f64(x, "f16")
    from scipy.special import expit

    g = X @ Wg.T
    u = X @ Wu.T
    h = g * expit(g) * u
    ref = h @ Wd.T
    assert np.allclose(out, ref, rtol=0, atol=1e-11 * np.abs(ref).max())
    sref = np.abs(h) @ np.abs(Wd.T)
    assert np.allclose(s, sref, rtol=1e-12)
    glu = orc.moe_glu("q4_k", gate, up, 1, F, H, gate.nbytes, x, "f16", ids, T, 1)
    assert np.allclose(glu["g"][:, 0], g, rtol=0, atol=1e-11 * np.abs(g).max())
    assert np.allclose(glu["h"][:, 0], h, rtol=0, atol=1e-11 * np.abs(h).max())


def test_moe_layer_brute_force_small(orc):
    import synth
    from scipy.special import expit

    rng = _rng(13)
    E, H, F, T, top_k = 4, 256, 256, 3, 2
    gate = synth.weight_blocks("q4_k", rng, E * F, H)
    up = synth.weight_blocks("q4_k", rng, E * F, H)
    down = synth.weight_blocks("q4_k", rng, E * H, F)
    gs, ds = F * synth.row_bytes("q4_k", H), H * synth.row_bytes("q4_k", F)
    x = synth.activations(rng, (T, H), "f16")
    ids, scores = synth.moe_routing(rng, T, E, top_k)
    out, _ = orc.moe_layer("q4_k", gate, up, down, E, H, F, gs, ds, x, "f16", ids, T, top_k,
                           scores)
    Wg = npd.decode_matrix("q4_k", gate, E * F, H).reshape(E, F, H)
    Wu = npd.decode_matrix("q4_k", up, E * F, H).reshape(E, F, H)
    Wd = npd.decode_matrix("q4_k", down, E * H, F).reshape(E, H, F)
    X = npd.act_f64(x, "f16")
    for t in range(T):
        ref = np.zeros(H)
        for r in range(top_k):
            e = ids[t, r]
            g = Wg[e] @ X[t]
            h = g * expit(g) * (Wu[e] @ X[t])
            ref += float(scores[t, r]) * (Wd[e] @ h)
        assert np.allclose(out[t], ref, rtol=0, atol=1e-11 * np.abs(ref).max())
    assert np.allclose(scores.sum(axis=1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ routing schedule
@pytest.mark.parametrize("tile_rows", [1, 4, 16, 64])
def test_route_schedule_invariants(orc, tile_rows):
    rng = _rng(14)
    E, T, top_k = 16, 50, 4
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.uint32)
    ids.ravel()[[5, 77]] = [E, E + 9]  # two invalid ids
    r = orc.route(ids, E, tile_rows)
    flat = ids.ravel()
    valid = flat < E
    assert r["n_invalid"] == 2
    assert np.array_equal(r["counts"], np.bincount(flat[valid], minlength=E))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]))
    perm = r["perm"]
    assert sorted(perm.tolist()) == np.nonzero(valid)[0].tolist()  # bijection onto valid rows
    assert np.array_equal(flat[perm], np.sort(flat[valid], kind="stable"))  # grouped by expert
    for e in range(E):  # stable inside each expert
        seg = perm[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
    covered = np.zeros(perm.size, int)
    for e, start, nrows in r["tiles"]:
        assert 1 <= nrows <= tile_rows
        assert r["offsets"][e] <= start and start + nrows <= r["offsets"][e + 1]
        end = start + nrows
        if end != r["offsets"][e + 1]:
            assert nrows == tile_rows  # only the last tile of an expert is partial
        covered[start:end] += 1
    assert np.all(covered == 1)
