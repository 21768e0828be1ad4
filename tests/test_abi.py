"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and its host-side logic (sizes, workspace layout, argument
validation that rejects before any launch) behaves as documented.  No call
here reaches a kernel."""

from __future__ import annotations

import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


@pytest.fixture(scope="module")
def kq():
    from block_quantized_weight_q4_amd import _build, kq as mod

    _build.build_if_missing()
    mod.lib()
    return mod


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_match_binding(kq):
    assert _declared() == sorted(kq.SYMBOLS)


def test_binding_constants_match_header():
    """Every enum constant KQ_X of the header that the binding also names (X)
    has the same value there."""
    import block_quantized_weight_q4_amd.kq as mod

    text = open(HEADER).read()
    consts = {}
    for body in re.findall(r"enum\s*\w*\s*\{([^}]*)\}", text):
        for name, val in re.findall(r"\bKQ_(\w+)\s*=\s*(0x[0-9a-fA-F]+|\d+)", body):
            consts[name] = int(val, 0)
    assert "ACT_GELU_TANH" in consts
    shared = [n for n in consts if hasattr(mod, n)]
    assert {"ACT_SILU", "ACT_GELU_TANH"} <= set(shared)
    for n in shared:
        assert getattr(mod, n) == consts[n], n


def test_library_exports_every_declared_symbol(kq):
    from block_quantized_weight_q4_amd._build import LIB

    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (kq_[a-z_0-9]+)$", out, flags=re.M))
    missing = [s for s in _declared() if s not in exported]
    assert not missing
    L = kq.lib()
    for s in _declared():
        assert getattr(L, s) is not None


def test_read_ceiling_library_is_separate(kq):
    """The benchmark's streaming-read measuring stick lives in its own
    library: libkq.so does not export it, libkq_hbmread.so does, and its
    host-side argument check rejects bad input before any launch."""
    from block_quantized_weight_q4_amd._build import LIB, READ_LIB

    main = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                          check=True).stdout
    assert "kq_hbm_read" not in main
    out = subprocess.run(["nm", "-D", "--defined-only", READ_LIB], capture_output=True, text=True,
                         check=True).stdout
    assert re.search(r"\bT kq_hbm_read$", out, flags=re.M)
    rd = C.CDLL(READ_LIB)
    rd.kq_hbm_read.restype = C.c_int
    rd.kq_hbm_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_uint32, C.c_void_p,
                               C.c_void_p]
    assert rd.kq_hbm_read(None, 16, 1, 4, 0, 16, None) == -1
    assert rd.kq_hbm_read(16, 15, 1, 4, 0, 16, None) == -1
    assert rd.kq_hbm_read(16, 16, 0, 4, 0, 16, None) == -1
    assert rd.kq_hbm_read(16, 16, 1, 3, 0, 16, None) == -1


def test_block_geometry(kq):
    assert (kq.kq_qk("q4_k"), kq.kq_block_bytes("q4_k")) == (256, 144)
    assert (kq.kq_qk("q8_0"), kq.kq_block_bytes("q8_0")) == (32, 34)
    assert (kq.kq_qk("tq1_g128"), kq.kq_block_bytes("tq1_g128")) == (128, 28)
    assert kq.kq_row_bytes("q4_k", 4096) == 16 * 144
    assert kq.kq_row_bytes("q8_0", 4096) == 128 * 34
    assert kq.kq_row_bytes("tq1_g128", 5120) == 40 * 28
    assert kq.kq_row_bytes("q4_k", 100) == -1
    assert kq.kq_row_bytes("q4_k", 0) == -1
    assert kq.lib().kq_qk(10) == 0


def test_ggml_block_geometry(kq):
    """The further GGUF blocks: QK and block bytes of the GGUF layouts, and
    their row strides."""
    for kind, qk, bb in (("q4_0", 32, 18), ("q5_0", 32, 22), ("q5_1", 32, 24), ("q6_k", 256, 210),
                         ("q2_k", 256, 84), ("q3_k", 256, 110), ("q5_k", 256, 176)):
        assert (kq.kq_qk(kind), kq.kq_block_bytes(kind)) == (qk, bb), kind
        assert kq.kq_row_bytes(kind, 4096) == 4096 // qk * bb, kind
    assert kq.kq_row_bytes("q6_k", 4096 + 32) == -1


def test_ggml_codecs_workspace_and_no_encoder(kq):
    """Their decode products take no workspace; their prefill GEMM takes the
    same workspace plan as Q4_K's (bf16 rows, split K for few tiles);
    kq_quantize rejects them before touching memory."""
    import torch

    for kind in ("q4_0", "q5_0", "q5_1", "q6_k", "q2_k", "q3_k", "q5_k"):
        for m, dt in ((1, torch.float16), (16, torch.bfloat16)):
            assert kq.kq_qmm_workspace_bytes(kind, 512, 4096, m, dt) == 0, (kind, m)
        for m, dt in ((512, torch.float16), (2048, torch.bfloat16), (64, torch.float32)):
            assert (kq.kq_qmm_workspace_bytes(kind, 512, 4096, m, dt)
                    == kq.kq_qmm_workspace_bytes("q4_k", 512, 4096, m, dt)), (kind, m)
    L = kq.lib()
    P = C.c_void_p
    base = 1 << 40
    for t in (3, 4, 5, 6, 7, 8, 9):
        assert L.kq_quantize(t, P(base), 0, 4, 256, None, P(base + (1 << 30)), None) == 2
        assert kq.kq_last_error() == "no encoder for this weight type"


def test_status_strings(kq):
    assert kq.kq_status_string(0) == "ok"
    for s in range(1, 5):
        assert kq.kq_status_string(s) not in ("ok", "unknown status")


def test_workspace_layout(kq):
    E, T, top_k, n = 128, 256, 8, 7168
    R = T * top_k
    max_tiles = min(R, (R + 31) // 32 + E)
    route_words = 2 + E + (E + 1) + R + 3 * max_tiles + R
    slot_off = (route_words * 4 + 255) // 256 * 256
    assert kq.kq_moe_workspace_bytes(E, T, top_k, 0) == slot_off
    assert kq.kq_moe_workspace_bytes(E, T, top_k, n) == slot_off + R * n * 4
    assert kq.kq_moe_workspace_bytes(0, T, top_k, 0) == 0
    assert kq.kq_moe_workspace_bytes(E, 2**31, 8, 0) == 0


def _call_qmv(L, t=0, w=16, n=8, k=256, x=16, xdt=1, m=1, y=4096, ydt=1):
    P = lambda v: C.c_void_p(v) if v else None  # noqa: E731  fake addresses, never dereferenced
    return L.kq_qmv(t, P(w), n, k, P(x), xdt, m, P(y), ydt, None)


def test_validation_rejects_before_launch(kq):
    """Every rejected call returns before any HIP call, so fake addresses are safe."""
    L = kq.lib()
    base = 1 << 40
    ok = dict(w=base, x=base + (1 << 30), y=base + (2 << 30))
    assert _call_qmv(L, **{**ok, "k": 100}) == 1          # k % QK
    assert _call_qmv(L, **{**ok, "n": 0}) == 1            # zero dim
    assert _call_qmv(L, **{**ok, "m": 0}) == 1
    assert _call_qmv(L, **{**ok, "m": 17}) == 1           # qmv takes <= 16 rows
    assert _call_qmv(L, **{**ok, "w": 0}) == 1            # null
    assert _call_qmv(L, **{**ok, "x": base + (1 << 30) + 2}) == 1  # misaligned
    assert _call_qmv(L, **{**ok, "y": base + 16}) == 1    # y overlaps w
    assert _call_qmv(L, **{**ok, "t": 10}) == 2           # unknown type
    assert _call_qmv(L, **{**ok, "xdt": 7}) == 2          # unknown dtype
    assert kq.kq_last_error() == "unknown dtype"
    big = dict(w=base, x=base + (1 << 36), y=base + (2 << 36))
    assert _call_qmv(L, **{**big, "n": 2**26 + 1}) == 1   # launch geometry bound on n
    assert kq.kq_last_error() == "n exceeds 2^26 weight rows"
    assert _call_qmv(L, **{**big, "k": 2**24 + 256}) == 1  # bound on k
    assert kq.kq_last_error() == "k exceeds 2^24 columns"


def test_expert_validation(kq):
    L = kq.lib()
    P = C.c_void_p
    base = 1 << 40
    w, x, ids, y, ws = (P(base + (i << 32)) for i in range(5))

    def call(**kw):
        a = dict(t=0, w=w, E=8, n=64, k=256, stride=64 * 144, x=x, xdt=1, layout=0, ids=ids,
                 T=4, top_k=2, scores=None, y=y, ydt=1, ws=ws, wsb=1 << 20)
        a.update(kw)
        return L.kq_qmm_id(a["t"], a["w"], a["E"], a["n"], a["k"], a["stride"], a["x"], a["xdt"],
                           a["layout"], a["ids"], a["T"], a["top_k"], a["scores"], a["y"], a["ydt"],
                           a["ws"], a["wsb"], None)

    assert call(top_k=0) == 1
    assert call(top_k=9) == 1                 # top_k > n_experts
    assert call(E=0) == 1
    assert call(stride=64 * 144 - 16) == 1    # stride below one expert
    assert call(stride=64 * 144 + 8) == 1     # stride alignment
    assert call(layout=5) == 1
    assert call(wsb=16) == 3                  # workspace too small
    assert call(T=2**31 // 2 + 1) == 1        # rows > INT32_MAX
    assert call(n=2**26 + 1, stride=(2**26 + 1) * 144) == 1  # launch geometry bound on n
    assert call(y=P(base + (1 << 32) + 64)) == 1  # output overlaps x
    assert call(T=1_100_000) == 1              # more than 65535 schedule tiles
    assert "65535" in kq.kq_last_error()
    for act in (2, 9, -1):
        assert L.kq_moe_glu(0, w, w, 8, 64, 256, 64 * 144, x, 1, ids, 4, 2, act, y, 1, ws, 1 << 20,
                            None) == 2        # unknown activation


def test_qmm_row_bound(kq):
    L = kq.lib()
    P = C.c_void_p
    base = 1 << 40
    m = 2**19 + 1
    rc = L.kq_qmm(0, P(base), 8, 256, P(base + (1 << 36)), 2, m, P(base + (2 << 36)), 2, None)
    assert rc == 1 and kq.kq_last_error() == "m exceeds 2^19 activation rows"


def test_qmm_workspace_sizes_and_validation(kq):
    """kq_qmm_workspace_bytes: none for decode shapes or fp32 activations, the
    converted activation rows (m*k fp16 + m exponents) for bf16, fp32 partial
    sums when K is split; kq_qmm_ws rejects a small or missing workspace
    before launching (fake addresses are never dereferenced)."""
    import torch

    bf, f16, f32 = torch.bfloat16, torch.float16, torch.float32
    assert kq.kq_qmm_workspace_bytes("q4_k", 4096, 4096, 16, bf) == 0
    assert kq.kq_qmm_workspace_bytes("q4_k", 4096, 4096, 512, f32) == 0
    assert kq.kq_qmm_workspace_bytes("q4_k", 4096, 100, 512, bf) == 0   # k % QK
    big = kq.kq_qmm_workspace_bytes("q4_k", 14336, 4096, 2048, bf)
    assert big >= 2048 * 4096 * 2 + 2048 * 4
    assert kq.kq_qmm_workspace_bytes("q4_k", 14336, 4096, 2048, f16) == 0  # many tiles: no split
    few = kq.kq_qmm_workspace_bytes("q4_k", 512, 4096, 200, f16)         # few tiles: split K
    assert few >= 2 * 200 * 512 * 4
    # the TQ1 decode product of one fp16 row: split K when its 16-row tiles
    # are fewer than 512 (5120 rows: 320 tiles, four pieces of 36 blocks)
    assert kq.kq_qmm_workspace_bytes("tq1_g128", 5120, 17408, 1, f16) == 4 * 5120 * 4
    assert kq.kq_qmm_workspace_bytes("tq1_g128", 17408, 5120, 1, f16) == 0   # 1088 tiles
    assert kq.kq_qmm_workspace_bytes("tq1_g128", 5120, 17408, 2, f16) == 0   # m > 1
    assert kq.kq_qmm_workspace_bytes("tq1_g128", 5120, 17408, 1, bf) == 0    # bf16 x
    assert kq.kq_qmm_workspace_bytes("tq1_g128", 300, 1536, 1, f16) == 0     # 12 blocks: too short
    for m in (1, 4, 8, 16):                                                 # Q4_K decode: no split
        assert kq.kq_qmm_workspace_bytes("q4_k", 4096, 14336, m, f16) == 0
    L = kq.lib()
    P = C.c_void_p
    base = 1 << 40
    args = (0, P(base), 14336, 4096, P(base + (1 << 36)), 2, 2048, P(base + (2 << 36)), 2)
    assert L.kq_qmm_ws(*args, P(base + (3 << 36)), big - 256, None) == 3
    assert L.kq_qmm_ws(*args, None, 0, None) == 3
    assert L.kq_qmm_ws(*args, P(base + (3 << 36) + 16), big, None) == 3  # misaligned
    assert L.kq_qmm_ws(*args, P(base + (1 << 36)), big, None) == 1       # overlaps x


def test_binding_checks_tensors_before_calling(kq):
    """The binding refuses strided, short or mixed-device tensors before any C
    call (host tensors here: nothing reaches a kernel)."""
    import torch

    w = torch.zeros(8 * 144, dtype=torch.uint8)
    x = torch.zeros((2, 512), dtype=torch.float16)
    y = torch.zeros((1, 8), dtype=torch.float16)
    with pytest.raises(kq.KQError, match="contiguous"):
        kq.kq_qmv("q4_k", w, 8, 256, x[:, ::2], 1, y)
    with pytest.raises(kq.KQError, match="bytes"):
        kq.kq_qmv("q4_k", w[:100], 8, 256, x, 1, y)
    with pytest.raises(kq.KQError, match="bytes"):
        kq.kq_qmv("q4_k", w, 8, 256, x, 1, y[:, :4])
    with pytest.raises(kq.KQError, match="device"):
        kq.kq_qmv("q4_k", w, 8, 256, x.to("meta"), 1, y)


def test_product_path_has_no_fallback():
    """The binding refuses to run without libkq.so instead of computing elsewhere."""
    import block_quantized_weight_q4_amd.kq as mod

    src = open(mod.__file__).read()
    assert "oracle" not in src
    for path in os.listdir(os.path.join(ROOT, "block_quantized_weight_q4_amd")):
        if path.endswith(".py"):
            text = open(os.path.join(ROOT, "block_quantized_weight_q4_amd", path)).read()
            assert "import oracle" not in text and "from oracle" not in text
