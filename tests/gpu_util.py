"""Helpers of the GPU parity tests: device copies and the tolerance checks."""

from __future__ import annotations

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TAU = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
# unit roundoff of the stored output format
UNIT = {"f32": 2.0**-24, "f16": 2.0**-11, "bf16": 2.0**-8}
# half the spacing of the format's subnormals: the absolute rounding error
# of storing a value below the normal range
ETA = {"f32": 2.0**-150, "f16": 2.0**-25, "bf16": 2.0**-134}


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dt: str | None = None) -> torch.Tensor:
    """Host array -> device tensor.  uint16 arrays are reinterpreted as dt."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(TORCH_DT[dt])
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(device())


def empty(shape, dt: str) -> torch.Tensor:
    return torch.empty(shape, dtype=TORCH_DT[dt], device=device())


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns (uint16 / uint32) of a device tensor."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def check_tol(got: np.ndarray, ref: np.ndarray, s: np.ndarray, tau: float, what: str,
              out_dt: str | None = None):
    """|got - ref| <= tau * S element by element; NaN anywhere fails.

    With ``out_dt``, one rounding of the stored output (its unit roundoff times
    |ref|) is allowed on top: used only for structured inputs whose result can
    be as large as S, where the store alone could exceed tau * S."""
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    bound = tau * s
    if out_dt is not None:
        bound = bound + UNIT[out_dt] * np.abs(ref) + ETA[out_dt]
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
            f"got {got[i]!r} ref {ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}")
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(s > 0, err / s, 0.0)
    return float(ratio.max()) if ratio.size else 0.0
