"""Thin Python binding of libkq (include/kq.h).

Argument marshalling only: every function has the name of the C entry point
it calls, takes torch tensors that already live where the C side expects
them (device memory for data, host scalars for sizes), passes their
``data_ptr()`` and the current HIP stream, and turns a non-OK status into a
``KQError``.  No arithmetic of the method happens here, and there is no
fallback: if libkq.so is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

from ._build import LIB

__all__ = [
    "KQError", "TYPES", "lib", "kq_status_string", "kq_last_error", "kq_qk", "kq_block_bytes",
    "kq_row_bytes", "kq_dequantize", "kq_quantize", "kq_validate_tq1", "kq_qmv", "kq_qmm", "kq_qmm_workspace_bytes", "kq_qmm_ws",
    "kq_qmm_noalloc_max_bytes", "kq_qmm_noalloc", "kq_moe_workspace_bytes", "kq_moe_route",
    "kq_qmm_id", "kq_moe_glu", "kq_moe_glu_ex", "kq_qmm_id_mix_shexp", "moe_schedule", "SYMBOLS",
    "LAYOUT_SHARED", "LAYOUT_SLOTTED", "REUSE_SCHEDULE", "ACT_SILU", "ACT_GELU_TANH",
    "ACT_SILU_LIMIT", "MOE_TILE_ROWS",
]

TYPES = {"q4_k": 0, "q8_0": 1, "tq1_g128": 2, "q4_0": 3, "q5_0": 4, "q5_1": 5, "q6_k": 6,
         "q2_k": 7, "q3_k": 8, "q5_k": 9}
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
LAYOUT_SHARED, LAYOUT_SLOTTED = 0, 1
REUSE_SCHEDULE = 0x100  # OR into the layout of a mixed kq_qmm_id: keep the workspace schedule
ACT_SILU = 0
ACT_GELU_TANH = 1
ACT_SILU_LIMIT = 2
MOE_TILE_ROWS = 32

# Every function include/kq.h declares.
SYMBOLS = (
    "kq_status_string", "kq_last_error", "kq_qk", "kq_block_bytes", "kq_row_bytes",
    "kq_dequantize", "kq_quantize", "kq_validate_tq1", "kq_qmv", "kq_qmm",
    "kq_qmm_workspace_bytes", "kq_qmm_ws", "kq_qmm_noalloc_max_bytes", "kq_qmm_noalloc", "kq_moe_workspace_bytes", "kq_moe_route",
    "kq_qmm_id", "kq_moe_glu", "kq_moe_glu_ex", "kq_qmm_id_mix_shexp",
)


class KQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{kq_status_string(status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libkq.so with argument types set.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError(
            f"libkq.so not found at {LIB}; build it with "
            "`python -m block_quantized_weight_q4_amd._build` (hipcc, gfx950)")
    L = C.CDLL(LIB)
    P, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    L.kq_status_string.restype = C.c_char_p
    L.kq_status_string.argtypes = [i32]
    L.kq_last_error.restype = C.c_char_p
    L.kq_last_error.argtypes = []
    L.kq_qk.restype = i32
    L.kq_qk.argtypes = [i32]
    L.kq_block_bytes.restype = i32
    L.kq_block_bytes.argtypes = [i32]
    L.kq_row_bytes.restype = i64
    L.kq_row_bytes.argtypes = [i32, i64]
    L.kq_dequantize.restype = i32
    L.kq_dequantize.argtypes = [i32, P, i64, i64, P, i32, P]
    L.kq_quantize.restype = i32
    L.kq_quantize.argtypes = [i32, P, i32, i64, i64, P, P, P]
    L.kq_validate_tq1.restype = i32
    L.kq_validate_tq1.argtypes = [P, i64, i64, P, P]
    for name in ("kq_qmv", "kq_qmm"):
        f = getattr(L, name)
        f.restype = i32
        f.argtypes = [i32, P, i64, i64, P, i32, i64, P, i32, P]
    L.kq_qmm_workspace_bytes.restype = C.c_size_t
    L.kq_qmm_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    L.kq_qmm_ws.restype = i32
    L.kq_qmm_ws.argtypes = [i32, P, i64, i64, P, i32, i64, P, i32, P, C.c_size_t, P]
    L.kq_qmm_noalloc_max_bytes.restype = C.c_size_t
    L.kq_qmm_noalloc_max_bytes.argtypes = []
    L.kq_qmm_noalloc.restype = i32
    L.kq_qmm_noalloc.argtypes = [i32, P, i64, i64, P, i32, i64, P, i32, P]
    L.kq_moe_workspace_bytes.restype = C.c_size_t
    L.kq_moe_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.kq_moe_route.restype = i32
    L.kq_moe_route.argtypes = [P, i64, i64, i64, P, C.c_size_t, P]
    L.kq_qmm_id.restype = i32
    L.kq_qmm_id.argtypes = [i32, P, i64, i64, i64, i64, P, i32, i32, P, i64, i64, P, P, i32, P,
                            C.c_size_t, P]
    L.kq_moe_glu.restype = i32
    L.kq_moe_glu.argtypes = [i32, P, P, i64, i64, i64, i64, P, i32, P, i64, i64, i32, P, i32, P,
                             C.c_size_t, P]
    L.kq_moe_glu_ex.restype = i32
    L.kq_moe_glu_ex.argtypes = [i32, P, P, i64, i64, i64, i64, P, P, P, i32, P, i64, i64, i32,
                                C.c_float, P, i32, P, C.c_size_t, P]
    L.kq_qmm_id_mix_shexp.restype = i32
    L.kq_qmm_id_mix_shexp.argtypes = [i32, P, i64, i64, i64, i64, P, P, i32, i32, P, i64, i64, P,
                                      P, i32, P, C.c_size_t, P]
    _lib = L
    return L


def kq_status_string(status: int) -> str:
    return lib().kq_status_string(int(status)).decode()


def kq_last_error() -> str:
    return lib().kq_last_error().decode()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(*tensors):
    for t in tensors:
        if t is not None and t.is_cuda:
            return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def _check(status: int):
    if status != 0:
        raise KQError(status, kq_last_error())


def _tensors(*specs):
    """Marshalling checks before a call: each (name, tensor, bytes the call
    reads or writes through it) must be contiguous, on the device of the first
    tensor, and at least that large.  A size the C side will reject (None or
    negative) is left to it."""
    dev = None
    for name, t, need in specs:
        if t is None:
            continue
        if not t.is_contiguous():
            raise KQError(1, f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise KQError(1, f"{name} is on device {t.device}; the call's other tensors are on {dev}")
        have = t.numel() * t.element_size()
        if need is not None and need > 0 and have < need:
            raise KQError(1, f"{name} holds {have} bytes; the call uses {need}")


def _rows_bytes(kind: str, rows: int, k: int):
    rb = lib().kq_row_bytes(TYPES[kind], int(k)) if kind in TYPES else -1
    return rows * rb if rb > 0 and rows > 0 else None


def _esz(t):
    return None if t is None else t.element_size()


def _dt(t) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise KQError(2, f"unsupported tensor dtype {t.dtype}") from None


def kq_qk(kind: str) -> int:
    return lib().kq_qk(TYPES[kind])


def kq_block_bytes(kind: str) -> int:
    return lib().kq_block_bytes(TYPES[kind])


def kq_row_bytes(kind: str, k: int) -> int:
    return lib().kq_row_bytes(TYPES[kind], int(k))


def kq_dequantize(kind: str, w, rows: int, k: int, out):
    _tensors(("w", w, _rows_bytes(kind, rows, k)), ("out", out, rows * k * out.element_size()))
    _check(lib().kq_dequantize(TYPES[kind], _ptr(w), rows, k, _ptr(out), _dt(out), _stream(w, out)))
    return out


def kq_quantize(kind: str, w, rows: int, k: int, out, imatrix=None):
    """Encode float weights w [rows, k] into out (uint8 block bytes)."""
    _tensors(("w", w, rows * k * w.element_size()), ("imatrix", imatrix, k * 4),
             ("out", out, _rows_bytes(kind, rows, k)))
    _check(lib().kq_quantize(TYPES[kind], _ptr(w), _dt(w), rows, k, _ptr(imatrix), _ptr(out),
                             _stream(w, out)))
    return out


def kq_validate_tq1(w, rows: int, k: int, count):
    """count: a device int64 tensor of one element that receives the number
    of illegal code bytes."""
    _tensors(("w", w, _rows_bytes("tq1_g128", rows, k)), ("count", count, 8))
    _check(lib().kq_validate_tq1(_ptr(w), rows, k, _ptr(count), _stream(w, count)))
    return count


def kq_qmv(kind: str, w, n: int, k: int, x, m: int, y):
    _tensors(("w", w, _rows_bytes(kind, n, k)), ("x", x, m * k * x.element_size()),
             ("y", y, m * n * y.element_size()))
    _check(lib().kq_qmv(TYPES[kind], _ptr(w), n, k, _ptr(x), _dt(x), m, _ptr(y), _dt(y),
                        _stream(w, x, y)))
    return y


def kq_qmm(kind: str, w, n: int, k: int, x, m: int, y):
    _tensors(("w", w, _rows_bytes(kind, n, k)), ("x", x, m * k * x.element_size()),
             ("y", y, m * n * y.element_size()))
    _check(lib().kq_qmm(TYPES[kind], _ptr(w), n, k, _ptr(x), _dt(x), m, _ptr(y), _dt(y),
                        _stream(w, x, y)))
    return y


def kq_qmm_workspace_bytes(kind: str, n: int, k: int, m: int, x_dtype) -> int:
    """Scratch bytes kq_qmm_ws needs; x_dtype is a torch dtype."""
    return int(lib().kq_qmm_workspace_bytes(TYPES[kind], n, k, m, _DT[x_dtype]))


def kq_qmm_ws(kind: str, w, n: int, k: int, x, m: int, y, workspace):
    _tensors(("w", w, _rows_bytes(kind, n, k)), ("x", x, m * k * x.element_size()),
             ("y", y, m * n * y.element_size()), ("workspace", workspace, None))
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kq_qmm_ws(TYPES[kind], _ptr(w), n, k, _ptr(x), _dt(x), m, _ptr(y), _dt(y),
                           _ptr(workspace), nbytes, _stream(w, x, y)))
    return y


def kq_qmm_noalloc_max_bytes() -> int:
    return int(lib().kq_qmm_noalloc_max_bytes())


def kq_qmm_noalloc(kind: str, w, n: int, k: int, x, m: int, y):
    _tensors(("w", w, _rows_bytes(kind, n, k)), ("x", x, m * k * x.element_size()),
             ("y", y, m * n * y.element_size()))
    _check(lib().kq_qmm_noalloc(TYPES[kind], _ptr(w), n, k, _ptr(x), _dt(x), m, _ptr(y), _dt(y),
                                _stream(w, x, y)))
    return y


def kq_moe_workspace_bytes(n_experts: int, n_tokens: int, top_k: int, n_out: int = 0) -> int:
    return int(lib().kq_moe_workspace_bytes(n_experts, n_tokens, top_k, n_out))


def kq_moe_route(ids, n_tokens: int, top_k: int, n_experts: int, workspace):
    _tensors(("ids", ids, n_tokens * top_k * 4), ("workspace", workspace, None))
    _check(lib().kq_moe_route(_ptr(ids), n_tokens, top_k, n_experts, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(ids, workspace)))
    return workspace


def kq_qmm_id(kind: str, w, n_experts: int, n: int, k: int, expert_stride: int, x, layout: int,
              ids, n_tokens: int, top_k: int, scores, y, workspace):
    rows = n_tokens * top_k
    x_rows = n_tokens if (layout & ~REUSE_SCHEDULE) == LAYOUT_SHARED else rows
    one = _rows_bytes(kind, n, k)
    _tensors(("w", w, None if one is None else (n_experts - 1) * expert_stride + one),
             ("x", x, x_rows * k * x.element_size()), ("ids", ids, rows * 4),
             ("scores", scores, rows * 4),
             ("y", y, (n_tokens if scores is not None else rows) * n * y.element_size()),
             ("workspace", workspace, None))
    _check(lib().kq_qmm_id(TYPES[kind], _ptr(w), n_experts, n, k, expert_stride, _ptr(x), _dt(x),
                           layout, _ptr(ids), n_tokens, top_k, _ptr(scores), _ptr(y), _dt(y),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(w, x, y)))
    return y


def kq_moe_glu(kind: str, gate_w, up_w, n_experts: int, n: int, k: int, expert_stride: int, x,
               ids, n_tokens: int, top_k: int, h, workspace, act: int = ACT_SILU):
    one = _rows_bytes(kind, n, k)
    wneed = None if one is None else (n_experts - 1) * expert_stride + one
    _tensors(("gate_w", gate_w, wneed), ("up_w", up_w, wneed),
             ("x", x, n_tokens * k * x.element_size()), ("ids", ids, n_tokens * top_k * 4),
             ("h", h, n_tokens * top_k * n * h.element_size()), ("workspace", workspace, None))
    _check(lib().kq_moe_glu(TYPES[kind], _ptr(gate_w), _ptr(up_w), n_experts, n, k, expert_stride,
                            _ptr(x), _dt(x), _ptr(ids), n_tokens, top_k, act, _ptr(h), _dt(h),
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(gate_w, x, h)))
    return h


def kq_moe_glu_ex(kind: str, gate_w, up_w, n_experts: int, n: int, k: int, expert_stride: int,
                  x, ids, n_tokens: int, top_k: int, h, workspace, act: int = ACT_SILU,
                  limit: float = 0.0, shexp_gate_w=None, shexp_up_w=None):
    one = _rows_bytes(kind, n, k)
    wneed = None if one is None else (n_experts - 1) * expert_stride + one
    S = top_k + (1 if shexp_gate_w is not None else 0)
    _tensors(("gate_w", gate_w, wneed), ("up_w", up_w, wneed), ("shexp_gate_w", shexp_gate_w, one),
             ("shexp_up_w", shexp_up_w, one), ("x", x, n_tokens * k * x.element_size()),
             ("ids", ids, n_tokens * top_k * 4), ("h", h, n_tokens * S * n * h.element_size()),
             ("workspace", workspace, None))
    _check(lib().kq_moe_glu_ex(TYPES[kind], _ptr(gate_w), _ptr(up_w), n_experts, n, k,
                               expert_stride, _ptr(shexp_gate_w), _ptr(shexp_up_w), _ptr(x), _dt(x),
                               _ptr(ids), n_tokens, top_k, act, float(limit), _ptr(h), _dt(h),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(gate_w, x, h)))
    return h


def kq_qmm_id_mix_shexp(kind: str, w, n_experts: int, n: int, k: int, expert_stride: int,
                        shexp_w, x, ids, n_tokens: int, top_k: int, scores, y, workspace,
                        flags: int = 0):
    one = _rows_bytes(kind, n, k)
    _tensors(("w", w, None if one is None else (n_experts - 1) * expert_stride + one),
             ("shexp_w", shexp_w, one), ("x", x, n_tokens * (top_k + 1) * k * x.element_size()),
             ("ids", ids, n_tokens * top_k * 4), ("scores", scores, n_tokens * (top_k + 1) * 4),
             ("y", y, n_tokens * n * y.element_size()), ("workspace", workspace, None))
    _check(lib().kq_qmm_id_mix_shexp(TYPES[kind], _ptr(w), n_experts, n, k, expert_stride,
                                     _ptr(shexp_w), _ptr(x), _dt(x), flags, _ptr(ids), n_tokens,
                                     top_k, _ptr(scores), _ptr(y), _dt(y), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(w, x, y)))
    return y


def moe_schedule(workspace, n_experts: int, n_tokens: int, top_k: int) -> dict:
    """Views of the schedule kq_moe_route leaves at the start of the workspace
    (layout documented in include/kq.h), copied to the host."""
    E, R = n_experts, n_tokens * top_k
    max_tiles = min(R, (R + MOE_TILE_ROWS - 1) // MOE_TILE_ROWS + E)
    words = 2 + E + (E + 1) + R + 3 * max_tiles
    w = workspace.view(torch.int32)[:words].cpu().numpy()
    n_tiles, n_invalid = int(w[0]), int(w[1])
    counts = w[2:2 + E]
    offsets = w[2 + E:3 + 2 * E]
    valid = int(offsets[E])
    perm = w[3 + 2 * E:3 + 2 * E + R][:valid]
    tiles = w[3 + 2 * E + R:].reshape(-1, 3)[:n_tiles]
    return {"counts": counts, "offsets": offsets, "perm": perm, "tiles": tiles,
            "n_invalid": n_invalid}
