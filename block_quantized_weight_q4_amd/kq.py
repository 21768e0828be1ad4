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
    "kq_row_bytes", "kq_dequantize", "kq_qmv", "kq_qmm", "kq_moe_workspace_bytes", "kq_moe_route",
    "kq_qmm_id", "kq_moe_glu", "moe_schedule", "SYMBOLS", "LAYOUT_SHARED", "LAYOUT_SLOTTED", "REUSE_SCHEDULE",
    "ACT_SILU", "ACT_GELU_TANH", "MOE_TILE_ROWS",
]

TYPES = {"q4_k": 0, "q8_0": 1, "tq1_g128": 2}
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
LAYOUT_SHARED, LAYOUT_SLOTTED = 0, 1
REUSE_SCHEDULE = 0x100  # OR into the layout of a mixed kq_qmm_id: keep the workspace schedule
ACT_SILU = 0
ACT_GELU_TANH = 1
MOE_TILE_ROWS = 32

# Every function include/kq.h declares.
SYMBOLS = (
    "kq_status_string", "kq_last_error", "kq_qk", "kq_block_bytes", "kq_row_bytes",
    "kq_dequantize", "kq_qmv", "kq_qmm", "kq_moe_workspace_bytes", "kq_moe_route", "kq_qmm_id",
    "kq_moe_glu",
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
    for name in ("kq_qmv", "kq_qmm"):
        f = getattr(L, name)
        f.restype = i32
        f.argtypes = [i32, P, i64, i64, P, i32, i64, P, i32, P]
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
    _lib = L
    return L


def kq_status_string(status: int) -> str:
    return lib().kq_status_string(int(status)).decode()


def kq_last_error() -> str:
    return lib().kq_last_error().decode()


def _check(status: int):
    if status != 0:
        raise KQError(status, kq_last_error())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(*tensors):
    for t in tensors:
        if t is not None and t.is_cuda:
            return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


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
    _check(lib().kq_dequantize(TYPES[kind], _ptr(w), rows, k, _ptr(out), _dt(out), _stream(w, out)))
    return out


def kq_qmv(kind: str, w, n: int, k: int, x, m: int, y):
    _check(lib().kq_qmv(TYPES[kind], _ptr(w), n, k, _ptr(x), _dt(x), m, _ptr(y), _dt(y),
                        _stream(w, x, y)))
    return y


def kq_qmm(kind: str, w, n: int, k: int, x, m: int, y):
    _check(lib().kq_qmm(TYPES[kind], _ptr(w), n, k, _ptr(x), _dt(x), m, _ptr(y), _dt(y),
                        _stream(w, x, y)))
    return y


def kq_moe_workspace_bytes(n_experts: int, n_tokens: int, top_k: int, n_out: int = 0) -> int:
    return int(lib().kq_moe_workspace_bytes(n_experts, n_tokens, top_k, n_out))


def kq_moe_route(ids, n_tokens: int, top_k: int, n_experts: int, workspace):
    _check(lib().kq_moe_route(_ptr(ids), n_tokens, top_k, n_experts, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(ids, workspace)))
    return workspace


def kq_qmm_id(kind: str, w, n_experts: int, n: int, k: int, expert_stride: int, x, layout: int,
              ids, n_tokens: int, top_k: int, scores, y, workspace):
    _check(lib().kq_qmm_id(TYPES[kind], _ptr(w), n_experts, n, k, expert_stride, _ptr(x), _dt(x),
                           layout, _ptr(ids), n_tokens, top_k, _ptr(scores), _ptr(y), _dt(y),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(w, x, y)))
    return y


def kq_moe_glu(kind: str, gate_w, up_w, n_experts: int, n: int, k: int, expert_stride: int, x,
               ids, n_tokens: int, top_k: int, h, workspace, act: int = ACT_SILU):
    _check(lib().kq_moe_glu(TYPES[kind], _ptr(gate_w), _ptr(up_w), n_experts, n, k, expert_stride,
                            _ptr(x), _dt(x), _ptr(ids), n_tokens, top_k, act, _ptr(h), _dt(h),
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(gate_w, x, h)))
    return h


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
