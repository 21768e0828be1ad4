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


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128", "q4_0", "q5_0", "q5_1", "q6_k",
                                  "q2_k", "q3_k", "q5_k"])
def test_independent_decoders_agree(orc, kind):
    """C oracle and the vectorised numpy decoder agree bit for bit on random
    blocks (Q4_K with arbitrary fp16 d/dmin bit patterns, not just the
    generator's range)."""
    import synth

    rng = _rng(4)
    rows, k = 400, 256 * 1  # 400 Q4_K blocks; more for the smaller formats
    k = {"q4_k": 256 * 250, "q8_0": 32 * 250, "tq1_g128": 128 * 250, "q4_0": 32 * 250,
         "q5_0": 32 * 250, "q5_1": 32 * 250, "q6_k": 256 * 250, "q2_k": 256 * 250,
         "q3_k": 256 * 250, "q5_k": 256 * 250}[kind]
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


# ------------------------------------------------------------------ GGUF Q4_0 / Q5_0 / Q5_1 / Q6_K
# The [MID] page's codec table names these blocks; their layouts are the GGUF
# convention (a reading).  Pins: hand-built blocks whose every weight is known
# from its fields, single-bit and single-weight probes of the bit maps, and
# the independent numpy decoder above.
@pytest.mark.parametrize("kind", ["q4_0", "q5_0", "q5_1"])
def test_legacy_blocks_from_fields(orc, kind):
    """Blocks packed from chosen quants decode to d*(q - 8) (Q4_0), d*(q - 16)
    (Q5_0) and d*q + m (Q5_1), weight i from quant i."""
    rng = _rng(60)
    nb = 64
    qmax = 16 if kind == "q4_0" else 32
    q = rng.integers(0, qmax, size=(nb, 32))
    d16 = rng.uniform(-2.0, 2.0, nb).astype(np.float16)
    m16 = rng.uniform(-3.0, 3.0, nb).astype(np.float16)
    blocks = npd.legacy_pack(kind, q, d16, m16)
    got = orc.dequant(kind, blocks, nb, 32)
    d, m = d16.astype(np.float64)[:, None], m16.astype(np.float64)[:, None]
    want = {"q4_0": d * (q - 8), "q5_0": d * (q - 16), "q5_1": d * q + m}[kind]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind", ["q5_0", "q5_1"])
def test_q5_high_bit_map(orc, kind):
    """All nibbles zero and a single high bit i set: weight i alone carries the
    extra 16 (bit i of the little-endian qh word is weight i's fifth bit)."""
    for i in range(32):
        q = np.zeros((1, 32), np.int64)
        q[0, i] = 16
        blk = npd.legacy_pack(kind, q, np.array([1.0], np.float16), np.array([0.0], np.float16))
        # the bit sits in qh byte i // 8, bit i % 8
        qh = blk[0, 2:6] if kind == "q5_0" else blk[0, 4:8]
        assert qh[i // 8] == 1 << (i % 8) and qh.sum() == qh[i // 8]
        got = orc.dequant(kind, blk, 1, 32)[0]
        base = -16.0 if kind == "q5_0" else 0.0
        want = np.full(32, base)
        want[i] = base + 16.0
        assert np.array_equal(got, want)


def test_q6k_blocks_from_fields(orc):
    """Q6_K packed from chosen 6-bit quants and int8 scales decodes to
    d * scale[j] * (q - 32), scale j for weights 16j..16j+15."""
    rng = _rng(61)
    nb = 40
    q = rng.integers(0, 64, size=(nb, 256))
    sc = rng.integers(-128, 128, size=(nb, 16))
    d16 = rng.uniform(-0.5, 0.5, nb).astype(np.float16)
    blocks = npd.q6k_pack(q, sc, d16)
    got = orc.dequant("q6_k", blocks, nb, 256)
    want = d16.astype(np.float64)[:, None] * np.repeat(sc, 16, axis=1) * (q - 32)
    assert np.array_equal(got, want)


def test_q6k_single_weight_probes(orc):
    """One weight at 32 + v, every other at 32 (zero): exactly that weight is
    nonzero, for every position, so no two positions share low or high bits."""
    for e in range(256):
        q = np.full((1, 256), 32)
        q[0, e] = 32 + 1 + (e % 31)
        blk = npd.q6k_pack(q, np.ones((1, 16), np.int64), np.array([1.0], np.float16))
        got = orc.dequant("q6_k", blk, 1, 256)[0]
        nz = np.flatnonzero(got)
        assert list(nz) == [e] and got[e] == 1 + (e % 31)


def test_q6k_layout_bytes(orc):
    """The byte layout: ql[128], qh[64], 16 int8 scales, fp16 d (210 bytes).
    Raising ql byte 0's low nibble by one raises weight 0 by d*scale[0];
    its high nibble, weight 64; qh byte 0's bits 2-3 by one, weight 32 by
    16*d*scale[2]; scale byte 192+5 scales weights 80..95; the last two
    bytes are d."""
    blk = np.zeros((1, 210), np.uint8)
    blk[0, 192:208] = np.arange(1, 17, dtype=np.int8).view(np.uint8)
    blk[0, 208:210] = np.array([1.0], np.float16).view(np.uint8)
    base = orc.dequant("q6_k", blk, 1, 256)[0]  # every q = 0: -32 * scale
    assert np.array_equal(base, -32.0 * np.repeat(np.arange(1, 17), 16))
    b = blk.copy()
    b[0, 0] = 0x01
    assert np.flatnonzero(orc.dequant("q6_k", b, 1, 256)[0] - base).tolist() == [0]
    b = blk.copy()
    b[0, 0] = 0x10
    diff = orc.dequant("q6_k", b, 1, 256)[0] - base
    assert np.flatnonzero(diff).tolist() == [64] and diff[64] == 1.0 * 5
    b = blk.copy()
    b[0, 128] = 0x04
    diff = orc.dequant("q6_k", b, 1, 256)[0] - base
    assert np.flatnonzero(diff).tolist() == [32] and diff[32] == 16.0 * 3
    b = blk.copy()
    b[0, 197] = 0  # scale 5 -> 0
    assert np.array_equal(np.flatnonzero(orc.dequant("q6_k", b, 1, 256)[0] - base), np.arange(80, 96))


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


# ------------------------------------------------------------------ GGUF Q2_K / Q3_K / Q5_K
# The rest of the [MID] page's K-quant table.  Pins as for Q6_K: blocks packed
# from chosen fields, raw-byte probes of the layout read in words (which byte
# and bit each weight, scale and min comes from), and the numpy decoder.
def test_q2k_blocks_from_fields(orc):
    """Q2_K from chosen 2-bit quants, 4-bit scales and mins: weight e is
    d * sc[e // 16] * q - dmin * mn[e // 16]."""
    rng = _rng(62)
    nb = 40
    q = rng.integers(0, 4, size=(nb, 256))
    sc = rng.integers(0, 16, size=(nb, 16))
    mn = rng.integers(0, 16, size=(nb, 16))
    d16 = rng.uniform(-0.5, 0.5, nb).astype(np.float16)
    dm16 = rng.uniform(-0.5, 0.5, nb).astype(np.float16)
    got = orc.dequant("q2_k", npd.q2k_pack(q, sc, mn, d16, dm16), nb, 256)
    d, dm = d16.astype(np.float64)[:, None], dm16.astype(np.float64)[:, None]
    want = d * np.repeat(sc, 16, axis=1) * q - dm * np.repeat(mn, 16, axis=1)
    assert np.array_equal(got, want)


def test_q2k_layout_bytes(orc):
    """Raw bytes: scale byte j's low nibble scales weights 16j..16j+15 and its
    high nibble is their min; bits 2u..2u+1 of qs byte 32h + l are weight
    128h + 32u + l; d and dmin are the last four bytes."""
    blk = np.zeros((1, 84), np.uint8)
    blk[0, 80:82] = np.array([1.0], np.float16).view(np.uint8)
    blk[0, 82:84] = np.array([0.5], np.float16).view(np.uint8)
    assert np.array_equal(orc.dequant("q2_k", blk, 1, 256)[0], np.zeros(256))
    for j in range(16):
        b = blk.copy()
        b[0, j] = 0x30  # min 3, scale 0
        want = np.zeros(256)
        want[16 * j:16 * j + 16] = -1.5
        assert np.array_equal(orc.dequant("q2_k", b, 1, 256)[0], want)
    for e in range(256):
        h, u, l = e // 128, (e % 128) // 32, e % 32
        b = blk.copy()
        b[0, 0:16] = 0x05  # every scale 5, min 0
        b[0, 16 + 32 * h + l] = 2 << (2 * u)
        got = orc.dequant("q2_k", b, 1, 256)[0]
        assert np.flatnonzero(got).tolist() == [e] and got[e] == 10.0


def test_q3k_blocks_from_fields(orc):
    """Q3_K from chosen quants in -4..3 and 6-bit scales in -32..31: weight e
    is d * sc[e // 16] * q."""
    rng = _rng(63)
    nb = 40
    q = rng.integers(-4, 4, size=(nb, 256))
    sc = rng.integers(-32, 32, size=(nb, 16))
    d16 = rng.uniform(-0.5, 0.5, nb).astype(np.float16)
    got = orc.dequant("q3_k", npd.q3k_pack(q, sc, d16), nb, 256)
    want = d16.astype(np.float64)[:, None] * np.repeat(sc, 16, axis=1) * q
    assert np.array_equal(got, want)


def test_q3k_scale_bytes(orc):
    """Raw scale bytes (offset 96): the low nibble of byte i is the low four
    bits of scale i (i < 8), its high nibble those of scale i + 8; bit pair p
    of byte 8 + r is the top of scale 4p + r; stored values are offset by 32.
    Every quant is -4 (all quant bits clear) and d = 1."""
    blk = np.zeros((1, 110), np.uint8)
    blk[0, 108:110] = np.array([1.0], np.float16).view(np.uint8)
    # stored 0 everywhere: scale -32, weight 128
    assert np.array_equal(orc.dequant("q3_k", blk, 1, 256)[0], np.full(256, 128.0))
    for i in range(16):
        for stored in (1, 9, 17, 33, 47, 63):
            b = blk.copy()
            lo, top = stored & 15, stored >> 4
            if i < 8:
                b[0, 96 + i] |= lo
            else:
                b[0, 96 + i - 8] |= lo << 4
            b[0, 96 + 8 + i % 4] |= top << (2 * (i // 4))
            want = np.full(256, 128.0)
            want[16 * i:16 * i + 16] = -4.0 * (stored - 32)
            assert np.array_equal(orc.dequant("q3_k", b, 1, 256)[0], want), (i, stored)
            assert orc.q3k_scale(b[0, 96:108], i) == stored - 32


def test_q3k_quant_bit_probes(orc):
    """Raw quant bytes: bits 2u..2u+1 of qs byte 32 + 32h + l and bit 4h + u of
    hmask byte l belong to weight 128h + 32u + l alone; the hmask bit adds 4."""
    blk = np.zeros((1, 110), np.uint8)
    # every scale 1 and d = 1 from the packer; quant bits cleared
    blk[0, 96:110] = npd.q3k_pack(np.zeros((1, 256)), np.full((1, 16), 1),
                                   np.array([1.0], np.float16))[0, 96:110]
    base = orc.dequant("q3_k", blk, 1, 256)[0]
    assert np.array_equal(base, np.full(256, -4.0))
    for e in range(256):
        h, u, l = e // 128, (e % 128) // 32, e % 32
        b = blk.copy()
        b[0, 32 + 32 * h + l] = 3 << (2 * u)
        diff = orc.dequant("q3_k", b, 1, 256)[0] - base
        assert np.flatnonzero(diff).tolist() == [e] and diff[e] == 3.0
        b = blk.copy()
        b[0, l] = 1 << (4 * h + u)
        diff = orc.dequant("q3_k", b, 1, 256)[0] - base
        assert np.flatnonzero(diff).tolist() == [e] and diff[e] == 4.0


def test_q5k_blocks_from_fields(orc):
    """Q5_K from chosen Q4_K scales and mins and 5-bit quants: weight e is
    d * sc[e // 32] * q - dmin * m[e // 32]."""
    rng = _rng(64)
    nb = 40
    q = rng.integers(0, 32, size=(nb, 256))
    sc = rng.integers(0, 64, size=(nb, 8))
    m = rng.integers(0, 64, size=(nb, 8))
    d16 = rng.uniform(-0.5, 0.5, nb).astype(np.float16)
    dm16 = rng.uniform(-0.5, 0.5, nb).astype(np.float16)
    got = orc.dequant("q5_k", npd.q5k_pack(d16, dm16, sc, m, q), nb, 256)
    d, dm = d16.astype(np.float64)[:, None], dm16.astype(np.float64)[:, None]
    want = d * np.repeat(sc, 32, axis=1) * q - dm * np.repeat(m, 32, axis=1)
    assert np.array_equal(got, want)


def test_q5k_fifth_bit_and_layout(orc):
    """Raw bytes: bit j of qh byte 16 + l adds 16 to weight 32j + l alone; the
    nibbles sit at offset 48 in the Q4_K order; the scales at 4..15 are Q4_K's."""
    head = npd.q4k_pack(np.array([1.0], np.float16), np.array([0.0], np.float16),
                        np.ones((1, 8), np.int64), np.zeros((1, 8), np.int64),
                        np.zeros((1, 256), np.int64))[0]
    blk = np.zeros((1, 176), np.uint8)
    blk[0, 0:16] = head[0:16]
    assert np.array_equal(orc.dequant("q5_k", blk, 1, 256)[0], np.zeros(256))
    for e in range(256):
        j, l = e // 32, e % 32
        b = blk.copy()
        b[0, 16 + l] = 1 << j
        got = orc.dequant("q5_k", b, 1, 256)[0]
        assert np.flatnonzero(got).tolist() == [e] and got[e] == 16.0
        b = blk.copy()
        b[0, 48 + 32 * (j // 2) + l] = 7 << (4 * (j % 2))
        got = orc.dequant("q5_k", b, 1, 256)[0]
        assert np.flatnonzero(got).tolist() == [e] and got[e] == 7.0


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
@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128", "q4_0", "q5_0", "q5_1", "q6_k",
                                  "q2_k", "q3_k", "q5_k"])
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


@pytest.mark.parametrize("kind", ["q4_k", "q8_0", "tq1_g128", "q4_0", "q5_0", "q5_1", "q6_k",
                                  "q2_k", "q3_k", "q5_k"])
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


def _dup_case(T, seed):
    import synth

    E, n, k, top_k = 6, 32, 256, 3
    rng, w, stride, ids, scores = _moe_small(E=E, n=n, k=k, T=T, top_k=top_k, seed=seed)
    x = synth.activations(rng, (T, k), "f16")
    return E, n, k, top_k, w, stride, ids.copy(), scores, x


def test_routing_rule_below_32_tokens(orc):
    """mlx-native "quantized_matmul_id_ggml.rs": the matrix-vector route only
    bounds-checks.  Below 32 tokens a repeated id is computed as written (its
    slot equals the first slot with that id) and an out-of-range id poisons
    only the rows it touches."""
    T = 31
    E, n, k, top_k, w, stride, ids, scores, x = _dup_case(T, 61)
    ids[4, 2] = ids[4, 0]
    ids[9, 1] = E
    assert not orc.routing_poisons_all(ids, E)
    y, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, ids, T, top_k)
    assert np.array_equal(y[4 * top_k + 2], y[4 * top_k + 0])
    bad = 9 * top_k + 1
    assert np.all(np.isnan(y[bad])) and np.all(np.isfinite(np.delete(y, bad, axis=0)))
    ym, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, ids, T, top_k, scores)
    assert np.all(np.isnan(ym[9])) and np.all(np.isfinite(np.delete(ym, 9, axis=0)))
    want4 = sum(float(scores[4, r]) * y[4 * top_k + r] for r in range(top_k))
    assert np.allclose(ym[4], want4, rtol=1e-13, atol=0)
    r = orc.route(ids, E, 32)
    assert r["n_invalid"] == 1 and len(r["tiles"]) > 0


@pytest.mark.parametrize("defect", ["repeat", "range"])
def test_routing_rule_from_32_tokens(orc, defect):
    """mlx-native "quantized_matmul_id_ggml.rs": the matrix-matrix route (from
    32 tokens on) requires distinct ids per token, and any out-of-range or
    repeated id writes NaN to the entire output and leaves the schedule with
    no tiles (no weight is read)."""
    T = 32
    E, n, k, top_k, w, stride, ids, scores, x = _dup_case(T, 62)
    good = ids.copy()
    assert not orc.routing_poisons_all(good, E)
    y0, _ = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, good, T, top_k)
    assert np.all(np.isfinite(y0))
    if defect == "repeat":
        ids[17, 1] = ids[17, 2]
    else:
        ids[17, 1] = E + 100
    assert orc.routing_poisons_all(ids, E)
    for sc in (None, scores):
        y, s = orc.qmm_id("q4_k", w, E, n, k, stride, x, "f16", False, ids, T, top_k, sc)
        assert np.all(np.isnan(y)) and np.all(np.isnan(s))
    glu = orc.moe_glu("q4_k", w, w, E, n, k, stride, x, "f16", ids, T, top_k)
    assert all(np.all(np.isnan(glu[key])) for key in glu)
    r = orc.route(ids, E, 32)
    assert r["n_invalid"] == 1 and len(r["tiles"]) == 0
    flat = ids.ravel()
    assert np.array_equal(r["counts"], np.bincount(flat[flat < E], minlength=E))
    # the same defect in a 31-token call follows the matrix-vector rule
    assert not orc.routing_poisons_all(ids[1:], E)


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


def test_gelu_tanh_against_torch(orc):
    """The same function from an independent implementation: torch's GELU with
    approximate='tanh', evaluated in float64.  A mistyped cubic coefficient
    (0.0447 for 0.044715) moves the result by ~1e-5 and fails here."""
    import torch

    zs = np.concatenate([np.linspace(-12.0, 12.0, 2401), np.geomspace(1e-6, 12.0, 200),
                         -np.geomspace(1e-6, 12.0, 200)])
    ref = torch.nn.functional.gelu(torch.from_numpy(zs), approximate="tanh").numpy()
    got = np.array([orc.gelu_tanh(z) for z in zs])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)


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
    import torch

    # the activations from torch (float64), not from the oracle itself
    acts = ((0, lambda g: torch.nn.functional.silu(torch.from_numpy(g)).numpy()),
            (1, lambda g: torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy()))
    for act, fn in acts:
        r = orc.moe_glu("q4_k", gate, up, E, n, k, stride, x, "f16", ids, T, top_k, act)
        want = fn(r["g"]) * r["u"]
        assert np.allclose(r["h"], want, rtol=1e-12, atol=0.0)
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
@pytest.mark.parametrize("T,n_bad", [(20, 2), (50, 0)])
def test_route_schedule_invariants(orc, tile_rows, T, n_bad):
    rng = _rng(14)
    E, top_k = 16, 4
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.uint32)
    if n_bad:
        ids.ravel()[[5, 77]] = [E, E + 9]  # two out-of-range ids (matrix-vector rule)
    r = orc.route(ids, E, tile_rows)
    flat = ids.ravel()
    valid = flat < E
    assert r["n_invalid"] == n_bad
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


# ------------------------------------------------------------------ encoders
def _q4k_grid_blocks(rng, rows, k):
    """Q4_K blocks whose every sub-block holds both q = 0 and q = 15, with one
    sub-block at sc = 63 and one at m = 63 (positive normal d, dmin): the
    grid points that the min-max encoder must reproduce byte for byte."""
    from tests.test_gpu_precision import _pack_q4k_scales

    nb = rows * (k // 256)
    out = np.zeros((nb, 144), np.uint8)
    for b in range(nb):
        sc = rng.integers(1, 64, 8)
        m = rng.integers(0, 64, 8)
        sc[rng.integers(0, 8)] = 63
        m[rng.integers(0, 8)] = 63
        d = np.float16(rng.uniform(1e-3, 2e-2))
        dmin = np.float16(rng.uniform(1e-3, 2e-2))
        out[b, 0:2] = np.array([d]).view(np.uint8)
        out[b, 2:4] = np.array([dmin]).view(np.uint8)
        out[b, 4:16] = _pack_q4k_scales(sc, m)
        q = rng.integers(0, 16, 256)
        for j in range(8):
            q[32 * j] = 0
            q[32 * j + 1] = 15
        rng.shuffle(q.reshape(8, 32), axis=1)
        for c in range(4):
            lo, hi = q[64 * c:64 * c + 32], q[64 * c + 32:64 * c + 64]
            out[b, 16 + 32 * c:48 + 32 * c] = lo | (hi << 4)
    return out.reshape(rows, -1)


def test_encoders_reproduce_decoded_blocks(orc):
    """A block the encoder could have produced decodes to values that encode
    back to the same bytes: Q8_0 with d > 0 and some |q| = 127, TQ1 with s > 0
    and some nonzero trit, Q4_K grid blocks."""
    import synth

    rng = _rng(40)
    rows = 20
    q8 = synth.q8_0_blocks(rng, rows, 320).reshape(-1, 34)
    q8[:, 2] = 127  # one |q| = 127 per block
    q8 = q8.reshape(rows, -1)
    tq = synth.tq1_blocks(rng, rows, 384).reshape(-1, 28)
    tq[:, 0] = 242  # some nonzero trits
    tq = tq.reshape(rows, -1)
    q4 = _q4k_grid_blocks(rng, rows, 512)
    for kind, b, k in (("q8_0", q8, 320), ("tq1_g128", tq, 384), ("q4_k", q4, 512)):
        w = orc.dequant(kind, b, rows, k).astype(np.float32)
        assert np.array_equal(w.astype(np.float64), orc.dequant(kind, b, rows, k)), kind
        again = orc.quantize(kind, w, "f32", rows, k)
        assert np.array_equal(again, b), kind


def test_q4k_encoder_picks_nearest_levels(orc):
    """Whatever scales the encoder chose, every weight decodes to a level of
    its sub-block's grid nearest to it (levels from the independent numpy
    decoder), and the error stays within half the largest step plus the
    6-bit scale rounding."""
    rng = _rng(41)
    rows, k = 16, 1024
    w = (rng.standard_normal((rows, k)) * rng.uniform(0.01, 3.0, (rows, 1))).astype(np.float32)
    w[3] = np.abs(w[3])          # all positive rows (min 0)
    w[4] = -np.abs(w[4])         # all negative rows
    for imp in (None, rng.uniform(0.0, 2.0, k).astype(np.float32)):
        b = orc.quantize("q4_k", w, "f32", rows, k, imp)
        dec = npd.decode_matrix("q4_k", b, rows, k)
        # the 16 levels of each sub-block: decode blocks with every nibble q
        blocks = b.reshape(-1, 144)
        lv = np.empty((blocks.shape[0], 8, 16))
        for q in range(16):
            bq = blocks.copy()
            bq[:, 16:] = q | (q << 4)
            lv[:, :, q] = npd.decode_matrix("q4_k", bq, blocks.shape[0], 256)[:, ::32]
        lv = lv.reshape(rows, k // 256, 8, 1, 16)
        ww = w.astype(np.float64).reshape(rows, k // 256, 8, 32, 1)
        best = np.abs(ww - lv).min(axis=-1).reshape(rows, k)
        err = np.abs(dec - w)
        assert np.all(err <= best + 1e-6 * np.abs(w).max()), np.max(err - best)
        if imp is not None:
            continue  # a shrunk range may clip weights of low importance
        # inside its grid a weight is within half a step; the plain min-max
        # grid misses the sub-block's range by at most the 6-bit rounding of
        # its scale (d / 2 per step, 15 steps) and of its min (dmin / 2)
        hd = blocks[:, 0:4].copy().view(np.float16).astype(np.float64).reshape(rows, k // 256, 2)
        step = (lv[..., 1] - lv[..., 0]).reshape(rows, k // 256, 8, 1)
        bound = 0.5 * step + 7.5 * hd[..., 0, None, None] + 0.5 * hd[..., 1, None, None]
        assert np.all(err.reshape(rows, k // 256, 8, 32) <= bound * (1 + 1e-6) + 1e-7)


def test_q8_0_and_tq1_encoder_bounds(orc):
    rng = _rng(42)
    rows = 12
    w = (rng.standard_normal((rows, 384)) * rng.uniform(1e-3, 50.0, (rows, 1))).astype(np.float32)
    b = orc.quantize("q8_0", w, "f32", rows, 384)
    d = b.reshape(-1, 34)[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(rows, -1)
    amax = np.abs(w.reshape(rows, -1, 32)).max(axis=2)
    assert np.all(np.abs(d - amax / 127) <= 2.0**-11 * amax / 127)  # one fp16 rounding
    err = np.abs(orc.dequant("q8_0", b, rows, 384) - w).reshape(rows, -1, 32)
    assert np.all(err <= 0.5 * d[..., None] * (1 + 2.0**-10) + 1e-12)
    assert (b.reshape(-1, 34)[:, 2:] == 0x80).sum() == 0  # never -128
    t = orc.quantize("tq1_g128", w, "f32", rows, 384)
    assert orc.tq1_illegal(t, rows, 384) == 0
    s = t.reshape(-1, 28)[:, 26:28].copy().view(np.float16).astype(np.float64).reshape(rows, -1)
    err = np.abs(orc.dequant("tq1_g128", t, rows, 384) - w).reshape(rows, -1, 128)
    assert np.all(err <= 0.5 * s[..., None] * (1 + 2.0**-10) + 1e-12)


def test_encoders_zero_blocks_and_dtypes(orc):
    z = np.zeros((2, 256), np.float32)
    assert np.all(orc.quantize("q8_0", z, "f32", 2, 256) == 0)
    assert np.all(orc.quantize("q4_k", z, "f32", 2, 256) == 0)
    t = orc.quantize("tq1_g128", z, "f32", 2, 256).reshape(-1, 28)
    assert np.all(t[:, :25] == 1 + 3 + 9 + 27 + 81) and np.all(t[:, 25] == 1 + 3 + 9)
    assert np.all(t[:, 26:] == 0)
    # fp16 / bf16 inputs are the same values as their fp32 conversion
    import torch

    rng = _rng(43)
    w = rng.standard_normal((4, 512)).astype(np.float32)
    h = w.astype(np.float16)
    bf = torch.from_numpy(w).to(torch.bfloat16)
    for kind in ("q4_k", "q8_0", "tq1_g128"):
        a = orc.quantize(kind, h.view(np.uint16), "f16", 4, 512)
        assert np.array_equal(a, orc.quantize(kind, h.astype(np.float32), "f32", 4, 512))
        a = orc.quantize(kind, bf.view(torch.int16).numpy().view(np.uint16), "bf16", 4, 512)
        assert np.array_equal(a, orc.quantize(kind, bf.float().numpy(), "f32", 4, 512))


def test_q4k_importance_vector(orc):
    """Scaling the importances by a power of two changes nothing; an importance
    on one weight only never makes that weight worse than the plain min-max
    range of its sub-block would (the unshrunk range is a candidate)."""
    rng = _rng(44)
    rows, k = 6, 512
    w = rng.standard_normal((rows, k)).astype(np.float32)
    imp = rng.uniform(0.0, 3.0, k).astype(np.float32)
    a = orc.quantize("q4_k", w, "f32", rows, k, imp)
    assert np.array_equal(a, orc.quantize("q4_k", w, "f32", rows, k, imp * 4.0))
    assert not np.array_equal(a, orc.quantize("q4_k", w, "f32", rows, k, None))
    plain = npd.decode_matrix("q4_k", orc.quantize("q4_k", w, "f32", rows, k, None), rows, k)
    for col in (5, 100, 300):
        one = np.zeros(k, np.float32)
        one[col] = 1.0
        got = npd.decode_matrix("q4_k", orc.quantize("q4_k", w, "f32", rows, k, one), rows, k)
        # same d/dmin rounding effects aside, the focused weight does not get worse
        assert np.all(np.abs(got[:, col] - w[:, col]) <= np.abs(plain[:, col] - w[:, col]) + 0.05)


def test_tq1_illegal_count(orc):
    import synth

    w = synth.tq1_blocks(_rng(45), 3, 256)
    assert orc.tq1_illegal(w, 3, 256) == 0
    bad = w.copy().reshape(-1, 28)
    bad[0, 3] = 243
    bad[1, 25] = 27
    bad[5, 24] = 255
    assert orc.tq1_illegal(bad.reshape(3, -1), 3, 256) == 3


# ------------------------------------------------------------------ silu_limit, shared expert
def test_silu_limit_against_torch(orc):
    """mlx-kquant moe_glu_gather_kq act='silu_limit': silu(min(g, limit)) *
    clip(u, -limit, limit), checked against torch's silu and clamp (float64)."""
    import torch

    rng = _rng(50)
    g = rng.uniform(-40, 40, 500)
    u = rng.uniform(-40, 40, 500)
    for limit in (0.5, 7.0, 1e6):
        ref = (torch.nn.functional.silu(torch.clamp(torch.from_numpy(g), max=limit)) *
               torch.clamp(torch.from_numpy(u), -limit, limit)).numpy()
        got = np.array([orc.silu_limit(a, b, limit) for a, b in zip(g, u)])
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-300)
    # a limit past every value is plain silu(g) * u
    assert orc.silu_limit(3.0, -2.0, 1e9) == pytest.approx(orc.silu(3.0) * -2.0, rel=1e-15)


def _shexp_case(seed, E=5, n=64, k=512, T=4, top_k=2):
    import synth

    rng = _rng(seed)
    gate = synth.weight_blocks("q4_k", rng, E * n, k)
    up = synth.weight_blocks("q4_k", rng, E * n, k)
    sg = synth.weight_blocks("q4_k", rng, n, k)
    su = synth.weight_blocks("q4_k", rng, n, k)
    stride = n * synth.row_bytes("q4_k", k)
    x = synth.activations(rng, (T, k), "f16")
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.uint32)
    return rng, E, n, k, T, top_k, gate, up, sg, su, stride, x, ids


def test_moe_glu_shared_expert_slot(orc):
    """mlx-kquant moe_glu_gather_shexp_kq: the shared expert is one extra,
    last slot computed with its own matrices; the routed slots are unchanged.
    Checked with the independent numpy decoder, for silu, gelu and silu_limit."""
    import torch

    rng, E, n, k, T, top_k, gate, up, sg, su, stride, x, ids = _shexp_case(51)
    X = npd.act_f64(x, "f16")
    Gs = X @ npd.decode_matrix("q4_k", sg, n, k).T
    Us = X @ npd.decode_matrix("q4_k", su, n, k).T
    acts = {0: lambda g, u: torch.nn.functional.silu(g) * u,
            1: lambda g, u: torch.nn.functional.gelu(g, approximate="tanh") * u,
            2: lambda g, u: torch.nn.functional.silu(torch.clamp(g, max=3.0)) * torch.clamp(u, -3.0, 3.0)}
    for act, fn in acts.items():
        r = orc.moe_glu_ex("q4_k", gate, up, E, n, k, stride, x, "f16", ids, T, top_k, act, 3.0,
                           sg, su)
        assert r["h"].shape == (T, top_k + 1, n)
        want = fn(torch.from_numpy(Gs), torch.from_numpy(Us)).numpy()
        assert np.allclose(r["h"][:, top_k], want, rtol=1e-11, atol=1e-11 * np.abs(want).max())
        routed = orc.moe_glu_ex("q4_k", gate, up, E, n, k, stride, x, "f16", ids, T, top_k, act, 3.0)
        assert np.array_equal(r["h"][:, :top_k], routed["h"])


def test_mix_with_shared_expert_brute_force(orc):
    """mlx-kquant gather_qmv_mix_kq: y[t] = sum over routed slots of score *
    W[e] x[t, r] plus the last score times the shared matrix applied to the
    last slot's row, against numpy with the independent decoder."""
    import synth

    rng, E, n, k, T, top_k, gate, up, sg, su, stride, x, ids = _shexp_case(52, n=64, k=256)
    H = 96
    down = synth.weight_blocks("q4_k", rng, E * H, n * 4)
    dsh = synth.weight_blocks("q4_k", rng, H, n * 4)
    kk = n * 4
    xs = synth.activations(rng, (T, top_k + 1, kk), "f16")
    scores = rng.uniform(0.05, 1.0, (T, top_k + 1)).astype(np.float32)
    dstride = H * synth.row_bytes("q4_k", kk)
    y, s = orc.qmm_id_mix_shexp("q4_k", down, E, H, kk, dstride, dsh, xs, "f16", ids, T, top_k,
                                scores)
    Wd = npd.decode_matrix("q4_k", down, E * H, kk).reshape(E, H, kk)
    Ws = npd.decode_matrix("q4_k", dsh, H, kk)
    X = npd.act_f64(xs.reshape(-1, kk), "f16").reshape(T, top_k + 1, kk)
    for t in range(T):
        ref = sum(float(scores[t, r]) * (Wd[ids[t, r]] @ X[t, r]) for r in range(top_k))
        ref = ref + float(scores[t, top_k]) * (Ws @ X[t, top_k])
        assert np.allclose(y[t], ref, rtol=0, atol=1e-11 * np.abs(ref).max())
        sref = sum(abs(float(scores[t, r])) * (np.abs(Wd[ids[t, r]]) @ np.abs(X[t, r]))
                   for r in range(top_k)) + abs(float(scores[t, top_k])) * (np.abs(Ws) @ np.abs(X[t, top_k]))
        assert np.allclose(s[t], sref, rtol=1e-12)


def test_shared_expert_poison_rules(orc):
    """The shared slot is never invalid; routed ids poison as without it."""
    import synth

    rng, E, n, k, T, top_k, gate, up, sg, su, stride, x, ids = _shexp_case(53, T=40)
    bad = ids.copy()
    bad[7, 1] = bad[7, 0]  # a repeat, 40 tokens: matrix-matrix rule
    r = orc.moe_glu_ex("q4_k", gate, up, E, n, k, stride, x, "f16", bad, 40, top_k, 0, 0.0, sg, su)
    assert np.all(np.isnan(r["h"]))
    small = ids[:10].copy()
    small[3, 0] = E + 2    # out of range, 10 tokens: only that routed row
    r = orc.moe_glu_ex("q4_k", gate, up, E, n, k, stride, x[:10], "f16", small, 10, top_k, 0, 0.0,
                       sg, su)
    nanrows = np.isnan(r["h"]).all(axis=2)
    assert nanrows.sum() == 1 and nanrows[3, 0] and np.all(np.isfinite(r["h"][:, top_k]))
