"""ctypes front end of the C oracle (kq_oracle.c).  Test infrastructure only.

All arrays are numpy on the host.  Weights are uint8 block bytes, activations
are float32 or the uint16 bit patterns of fp16/bf16, exactly as the seeded
generators produce them.  Results are float64 (exact decodes, fp64 sums).
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import build_oracle

__all__ = [
    "TYPES", "DTYPES", "lib", "half_to_double", "bf16_to_double", "float_to_half_rne",
    "float_to_bf16_rne", "q4k_scale_min", "dequant", "dequant_as", "qmm", "qmm_points",
    "qmm_id", "moe_glu", "moe_layer", "route", "routing_poisons_all", "quantize", "tq1_illegal", "silu_limit", "moe_glu_ex", "qmm_id_mix_shexp", "silu", "gelu_tanh", "num_threads", "q3k_scale",
]

TYPES = {"q4_k": 0, "q8_0": 1, "tq1_g128": 2, "q4_0": 3, "q5_0": 4, "q5_1": 5, "q6_k": 6,
         "q2_k": 7, "q3_k": 8, "q5_k": 9}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build_oracle()
        L = C.CDLL(path)
        P = C.c_void_p
        i64 = C.c_int64
        L.or_half_to_double.restype = C.c_double
        L.or_half_to_double.argtypes = [C.c_uint16]
        L.or_bf16_to_double.restype = C.c_double
        L.or_bf16_to_double.argtypes = [C.c_uint16]
        L.or_float_to_half_rne.restype = C.c_uint16
        L.or_float_to_half_rne.argtypes = [C.c_float]
        L.or_float_to_bf16_rne.restype = C.c_uint16
        L.or_float_to_bf16_rne.argtypes = [C.c_float]
        L.or_round_f32.restype = C.c_float
        L.or_round_f32.argtypes = [C.c_double]
        L.or_silu.restype = C.c_double
        L.or_silu.argtypes = [C.c_double]
        L.or_gelu_tanh.restype = C.c_double
        L.or_gelu_tanh.argtypes = [C.c_double]
        L.or_q4k_scale_min.restype = None
        L.or_q4k_scale_min.argtypes = [P, C.c_int, C.POINTER(C.c_int), C.POINTER(C.c_int)]
        L.or_q3k_scale.restype = C.c_int
        L.or_q3k_scale.argtypes = [P, C.c_int]
        L.or_dequant.restype = C.c_int
        L.or_dequant.argtypes = [C.c_int, P, i64, i64, P]
        L.or_dequant_store.restype = C.c_int
        L.or_dequant_store.argtypes = [C.c_int, P, i64, i64, C.c_int, P]
        L.or_qmm.restype = C.c_int
        L.or_qmm.argtypes = [C.c_int, P, i64, i64, P, C.c_int, i64, P, P]
        L.or_qmm_points.restype = C.c_int
        L.or_qmm_points.argtypes = [C.c_int, P, i64, i64, P, C.c_int, i64, i64, P, P, P, P]
        L.or_qmm_id.restype = C.c_int
        L.or_qmm_id.argtypes = [C.c_int, P, i64, i64, i64, i64, P, C.c_int, C.c_int, P, i64,
                                i64, P, P, P]
        L.or_moe_glu.restype = C.c_int
        L.or_moe_glu.argtypes = [C.c_int, P, P, i64, i64, i64, i64, P, C.c_int, P, i64, i64,
                                 C.c_int, P, P, P, P, P]
        L.or_silu_limit.restype = C.c_double
        L.or_silu_limit.argtypes = [C.c_double, C.c_double, C.c_double]
        L.or_moe_glu_ex.restype = C.c_int
        L.or_moe_glu_ex.argtypes = [C.c_int, P, P, i64, i64, i64, i64, P, P, P, C.c_int, P, i64,
                                    i64, C.c_int, C.c_double, P, P, P, P, P]
        L.or_qmm_id_mix_shexp.restype = C.c_int
        L.or_qmm_id_mix_shexp.argtypes = [C.c_int, P, i64, i64, i64, i64, P, P, C.c_int, P, i64,
                                          i64, P, P, P]
        L.or_moe_layer.restype = C.c_int
        L.or_moe_layer.argtypes = [C.c_int, P, P, P, i64, i64, i64, i64, i64, P, C.c_int, P,
                                   i64, i64, P, P, P]
        L.or_quantize.restype = C.c_int
        L.or_quantize.argtypes = [C.c_int, P, C.c_int, i64, i64, P, P]
        L.or_tq1_illegal.restype = C.c_int64
        L.or_tq1_illegal.argtypes = [P, i64, i64]
        L.or_route.restype = C.c_int64
        L.or_route.argtypes = [P, i64, i64, i64, i64, P, P, P, P, i64, P]
        L.or_routing_poisons_all.restype = C.c_int
        L.or_routing_poisons_all.argtypes = [P, i64, i64, i64]
        _lib = L
    return _lib


def num_threads() -> int:
    """Threads the OpenMP runtime will use (OMP_NUM_THREADS, else all cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def half_to_double(bits: int) -> float:
    return lib().or_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().or_bf16_to_double(int(bits))


def float_to_half_rne(f: float) -> int:
    return int(lib().or_float_to_half_rne(float(f)))


def float_to_bf16_rne(f: float) -> int:
    return int(lib().or_float_to_bf16_rne(float(f)))


def silu(z: float) -> float:
    return lib().or_silu(float(z))


def gelu_tanh(z: float) -> float:
    return lib().or_gelu_tanh(float(z))


def q4k_scale_min(scale_bytes, j: int):
    s = _c(scale_bytes, np.uint8)
    assert s.size == 12
    sc, m = C.c_int(), C.c_int()
    lib().or_q4k_scale_min(_p(s), int(j), C.byref(sc), C.byref(m))
    return sc.value, m.value


def q3k_scale(scale_bytes, i: int) -> int:
    """Signed scale i (0..15) of a Q3_K super-block's 12 packed scale bytes."""
    s = _c(scale_bytes, np.uint8)
    assert s.size == 12
    return int(lib().or_q3k_scale(_p(s), int(i)))


def dequant(kind: str, w: np.ndarray, rows: int, k: int) -> np.ndarray:
    """Exact decoded weights [rows, k] as float64."""
    w = _c(w, np.uint8)
    out = np.empty((rows, k), dtype=np.float64)
    rc = lib().or_dequant(TYPES[kind], _p(w), rows, k, _p(out))
    if rc:
        raise ValueError(f"or_dequant failed ({rc})")
    return out


def dequant_as(kind: str, w: np.ndarray, rows: int, k: int, out_dt: str) -> np.ndarray:
    """The stored result of dequantization in ``out_dt``: float32 values, or the
    uint16 bit patterns of fp16/bf16 (rounded from the fp32 value, ties to even)."""
    w = _c(w, np.uint8)
    out = np.empty((rows, k), dtype=np.float32 if out_dt == "f32" else np.uint16)
    rc = lib().or_dequant_store(TYPES[kind], _p(w), rows, k, DTYPES[out_dt], _p(out))
    if rc:
        raise ValueError(f"or_dequant_store failed ({rc})")
    return out


def qmm(kind, w, n, k, x, x_dt, m):
    """(y, s): y[m,n] = sum_k x*w in fp64 and s = sum_k |x*w|."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    y = np.empty((m, n), dtype=np.float64)
    s = np.empty((m, n), dtype=np.float64)
    rc = lib().or_qmm(TYPES[kind], _p(w), n, k, _p(x), DTYPES[x_dt], m, _p(y), _p(s))
    if rc:
        raise ValueError(f"or_qmm failed ({rc})")
    return y, s


def qmm_points(kind, w, n, k, x, x_dt, m, pm, pn):
    w = _c(w, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    pm = _c(pm, np.int64)
    pn = _c(pn, np.int64)
    y = np.empty(pm.size, dtype=np.float64)
    s = np.empty(pm.size, dtype=np.float64)
    rc = lib().or_qmm_points(TYPES[kind], _p(w), n, k, _p(x), DTYPES[x_dt], m, pm.size, _p(pm),
                             _p(pn), _p(y), _p(s))
    if rc:
        raise ValueError(f"or_qmm_points failed ({rc})")
    return y, s


def qmm_id(kind, w, n_experts, n, k, expert_stride, x, x_dt, slotted, ids, T, top_k,
           scores=None):
    w = _c(w, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    ids = _c(ids, np.uint32)
    sc = None if scores is None else _c(scores, np.float32)
    rows = T if sc is not None else T * top_k
    y = np.empty((rows, n), dtype=np.float64)
    s = np.empty((rows, n), dtype=np.float64)
    rc = lib().or_qmm_id(TYPES[kind], _p(w), n_experts, n, k, expert_stride, _p(x), DTYPES[x_dt],
                         int(bool(slotted)), _p(ids), T, top_k, _p(sc), _p(y), _p(s))
    if rc:
        raise ValueError(f"or_qmm_id failed ({rc})")
    return y, s


def moe_glu(kind, gate_w, up_w, n_experts, n, k, expert_stride, x, x_dt, ids, T, top_k, act=0):
    """dict of h, g, u, sg, su, each [T, top_k, n] float64; act 0 is silu,
    1 gelu (tanh approximation)."""
    gate_w = _c(gate_w, np.uint8)
    up_w = _c(up_w, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    ids = _c(ids, np.uint32)
    out = {key: np.empty((T, top_k, n), dtype=np.float64) for key in ("h", "g", "u", "sg", "su")}
    rc = lib().or_moe_glu(TYPES[kind], _p(gate_w), _p(up_w), n_experts, n, k, expert_stride,
                          _p(x), DTYPES[x_dt], _p(ids), T, top_k, act, _p(out["h"]), _p(out["g"]),
                          _p(out["u"]), _p(out["sg"]), _p(out["su"]))
    if rc:
        raise ValueError(f"or_moe_glu failed ({rc})")
    return out


def moe_layer(kind, gate_w, up_w, down_w, n_experts, hidden, ffn, gate_stride, down_stride, x,
              x_dt, ids, T, top_k, scores):
    """(out, s_out), each [T, hidden] float64: the whole MoE layer in fp64."""
    gate_w = _c(gate_w, np.uint8)
    up_w = _c(up_w, np.uint8)
    down_w = _c(down_w, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    ids = _c(ids, np.uint32)
    scores = _c(scores, np.float32)
    out = np.empty((T, hidden), dtype=np.float64)
    s = np.empty((T, hidden), dtype=np.float64)
    rc = lib().or_moe_layer(TYPES[kind], _p(gate_w), _p(up_w), _p(down_w), n_experts, hidden,
                            ffn, gate_stride, down_stride, _p(x), DTYPES[x_dt], _p(ids), T, top_k,
                            _p(scores), _p(out), _p(s))
    if rc:
        raise ValueError(f"or_moe_layer failed ({rc})")
    return out, s


def routing_poisons_all(ids, n_experts) -> bool:
    """ids [T, top_k]: True when the matrix-matrix rule (32 tokens or more)
    poisons the whole output (an out-of-range or a repeated id in a token)."""
    ids = np.atleast_2d(_c(ids, np.uint32))
    T, top_k = ids.shape
    return bool(lib().or_routing_poisons_all(_p(ids), T, top_k, n_experts))


def route(ids, n_experts, tile_rows):
    """dict(counts, offsets, perm, tiles[n_tiles,3], n_invalid) from ids
    [n_tokens, top_k] (a 1-D array is one slot per token)."""
    ids = _c(ids, np.uint32)
    if ids.ndim == 1:
        ids = ids.reshape(-1, 1)
    T, top_k = ids.shape
    n = ids.size
    counts = np.zeros(n_experts, dtype=np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    perm = np.full(n, -1, dtype=np.int32)
    max_tiles = n + n_experts
    tiles = np.zeros((max_tiles, 3), dtype=np.int32)
    bad = np.zeros(1, dtype=np.int64)
    nt = lib().or_route(_p(ids), T, top_k, n_experts, tile_rows, _p(counts), _p(offsets),
                        _p(perm), _p(tiles), max_tiles, _p(bad))
    if nt < 0:
        raise ValueError("or_route: tile capacity exceeded")
    valid = int(offsets[-1])
    return {"counts": counts, "offsets": offsets, "perm": perm[:valid], "tiles": tiles[:nt],
            "n_invalid": int(bad[0])}


def quantize(kind, w, w_dt, rows, k, imatrix=None):
    """uint8 [rows, row_bytes]: the encoder's bytes for float weights w
    [rows, k] (float32, or the uint16 bits of fp16/bf16)."""
    w = _c(w, np.float32 if w_dt == "f32" else np.uint16)
    imp = None if imatrix is None else _c(imatrix, np.float32)
    qk = {"q4_k": 256, "q8_0": 32, "tq1_g128": 128}[kind]
    bb = {"q4_k": 144, "q8_0": 34, "tq1_g128": 28}[kind]
    out = np.zeros((rows, (k // qk) * bb), dtype=np.uint8)
    rc = lib().or_quantize(TYPES[kind], _p(w), DTYPES[w_dt], rows, k, _p(imp), _p(out))
    if rc:
        raise ValueError(f"or_quantize failed ({rc})")
    return out


def tq1_illegal(w, rows, k) -> int:
    w = _c(w, np.uint8)
    return int(lib().or_tq1_illegal(_p(w), rows, k))


def silu_limit(g: float, u: float, limit: float) -> float:
    return lib().or_silu_limit(float(g), float(u), float(limit))


def moe_glu_ex(kind, gate_w, up_w, n_experts, n, k, expert_stride, x, x_dt, ids, T, top_k,
               act=0, limit=0.0, shexp_gate=None, shexp_up=None):
    """dict of h, g, u, sg, su, each [T, S, n] float64 with S = top_k (+1 with
    a shared expert, its slot last); act 0 silu, 1 gelu (tanh), 2 silu_limit."""
    gate_w = _c(gate_w, np.uint8)
    up_w = _c(up_w, np.uint8)
    sg_ = None if shexp_gate is None else _c(shexp_gate, np.uint8)
    su_ = None if shexp_up is None else _c(shexp_up, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    ids = _c(ids, np.uint32)
    S = top_k + (1 if sg_ is not None else 0)
    out = {key: np.empty((T, S, n), dtype=np.float64) for key in ("h", "g", "u", "sg", "su")}
    rc = lib().or_moe_glu_ex(TYPES[kind], _p(gate_w), _p(up_w), n_experts, n, k, expert_stride,
                             _p(sg_), _p(su_), _p(x), DTYPES[x_dt], _p(ids), T, top_k, act,
                             float(limit), _p(out["h"]), _p(out["g"]), _p(out["u"]),
                             _p(out["sg"]), _p(out["su"]))
    if rc:
        raise ValueError(f"or_moe_glu_ex failed ({rc})")
    return out


def qmm_id_mix_shexp(kind, w, n_experts, n, k, expert_stride, shexp_w, x, x_dt, ids, T, top_k,
                     scores):
    """(y, s), each [T, n]: the mixed down projection over T x (top_k + 1)
    slotted rows, the shared expert last."""
    w = _c(w, np.uint8)
    sw = _c(shexp_w, np.uint8)
    x = _c(x, np.float32 if x_dt == "f32" else np.uint16)
    ids = _c(ids, np.uint32)
    scores = _c(scores, np.float32)
    y = np.empty((T, n), dtype=np.float64)
    s = np.empty((T, n), dtype=np.float64)
    rc = lib().or_qmm_id_mix_shexp(TYPES[kind], _p(w), n_experts, n, k, expert_stride, _p(sw),
                                   _p(x), DTYPES[x_dt], _p(ids), T, top_k, _p(scores), _p(y), _p(s))
    if rc:
        raise ValueError(f"or_qmm_id_mix_shexp failed ({rc})")
    return y, s
