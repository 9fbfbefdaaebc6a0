"""Helpers for the GPU parity tests: move seeded storage-form inputs to the device and back, and the tolerance
checks.

Tolerances: fp32 relative Frobenius error <= 1e-5; bf16 (fp32 accumulation) relative Frobenius error <= 1e-2 and
max absolute error <= 3e-2 on unit-scale outputs.  "Unit scale" divides each element's error by its unit:
the RMS of the reference (of the whole tensor, or of the element's row for attention outputs, whose rows average a
varying number of value rows), or the element's own magnitude where that is larger -- a value stored in bf16
carries a rounding error up to 2^-9 of its own magnitude, so an element far above the RMS (heavy-tailed SwiGLU
products, peaked attention rows) cannot meet a bound that ignores its size."""
import numpy as np
import torch

import oracle as O

F32_REL_FROB = 1e-5
BF16_REL_FROB = 1e-2
BF16_MAX_ABS_UNIT = 3e-2


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage form (uint16 bf16 patterns or float32) -> device tensor of that dtype, same bits."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage form (bits for bf16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def empty(shape, dtype: str) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def max_err_unit_scale(got: np.ndarray, ref: np.ndarray, row_unit: bool = False) -> float:
    """max |got - ref| / unit, unit = max(RMS of the reference (per row if row_unit), |ref|)."""
    g = got.reshape(got.shape[0], -1) if got.ndim else got.reshape(1, 1)
    r = ref.reshape(ref.shape[0], -1) if ref.ndim else ref.reshape(1, 1)
    if row_unit:
        rms = np.sqrt(np.mean(r * r, axis=1))[:, None]
    else:
        rms = np.full((r.shape[0], 1), np.sqrt(np.mean(r * r)) if r.size else 1.0)
    unit = np.maximum(rms, np.abs(r))
    unit = np.where(unit > 0, unit, 1.0)
    return float(np.max(np.abs(g - r) / unit)) if r.size else 0.0


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", row_unit: bool = False):
    """Relative Frobenius error, then (bf16) the max error on the unit scale described in the module docstring."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rf = O.rel_frobenius(got, ref)
    if dtype == "f32":
        assert rf <= F32_REL_FROB, f"{what}: rel Frobenius {rf:.3e} > {F32_REL_FROB}"
        return rf, None
    ma = max_err_unit_scale(got, ref, row_unit)
    assert rf <= BF16_REL_FROB, f"{what}: rel Frobenius {rf:.3e} > {BF16_REL_FROB}"
    assert ma <= BF16_MAX_ABS_UNIT, f"{what}: max abs (unit scale) {ma:.3e} > {BF16_MAX_ABS_UNIT}"
    return rf, ma


def say(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
