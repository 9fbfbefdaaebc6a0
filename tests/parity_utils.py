"""Helpers for the GPU parity tests: move seeded storage-form inputs to the device and back, and the tolerance
checks.

Tolerances: fp32 relative Frobenius error <= 1e-5; bf16 (fp32 accumulation) relative Frobenius error <= 1e-2 and
max absolute error <= 3e-2 on unit-scale outputs.

"Unit scale" means the error of an element is measured against the RMS of the reference: of the whole tensor, or
of the element's row for attention outputs (each row averages a different number of value rows, so the rows'
scales differ by design).  Each element may err by
    max(3e-2 * RMS, 2^-7 * |ref|):
3e-2 of the unit scale, widened only for an element so far above the RMS (beyond 3.84 RMS) that two bf16 rounding
steps of its own size (a bf16 value carries up to 2^-8 of its magnitude from one round-to-nearest) exceed it.
max_err_unit_scale reports max |got - ref| / max(RMS, KAPPA * |ref|) with KAPPA = 2^-7 / 3e-2, which is <= 3e-2
exactly when every element meets that allowance."""
import numpy as np
import torch

import oracle as O

F32_REL_FROB = 1e-5
BF16_REL_FROB = 1e-2
BF16_MAX_ABS_UNIT = 3e-2
# an element's own-size allowance is 2^-7 |ref|; on the unit scale that is KAPPA * |ref| against BF16_MAX_ABS_UNIT
KAPPA = 2.0 ** -7 / BF16_MAX_ABS_UNIT


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


def storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """An oracle value (float64) in the storage form dev() takes: bf16 patterns after rounding to fp32 then to bf16
    (the value O.stored gives), or float32."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return O.f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def empty(shape, dtype: str) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def max_err_unit_scale(got: np.ndarray, ref: np.ndarray, row_unit: bool = False) -> float:
    """max |got - ref| / unit, unit = max(RMS of the reference (per row if row_unit), KAPPA * |ref|)."""
    g = got.reshape(got.shape[0], -1) if got.ndim else got.reshape(1, 1)
    r = ref.reshape(ref.shape[0], -1) if ref.ndim else ref.reshape(1, 1)
    if row_unit:
        rms = np.sqrt(np.mean(r * r, axis=1))[:, None]
    else:
        rms = np.full((r.shape[0], 1), np.sqrt(np.mean(r * r)) if r.size else 1.0)
    unit = np.maximum(rms, KAPPA * np.abs(r))
    unit = np.where(unit > 0, unit, 1.0)
    return float(np.max(np.abs(g - r) / unit)) if r.size else 0.0


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", row_unit: bool = False,
                elem_ref=None):
    """Relative Frobenius error against ref, then (bf16) the max error on the unit scale described in the module
    docstring, against elem_ref when given (else ref).

    elem_ref is the oracle's value of the same output along the block's bf16 data flow (store="bf16": the
    activations the block keeps between steps rounded to bf16 where it stores them), when ref is the exact chain.
    Both come from the oracle alone; the element bound then measures what the kernel adds to the rounding the data
    flow itself imposes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rf = O.rel_frobenius(got, ref)
    if dtype == "f32":
        assert rf <= F32_REL_FROB, f"{what}: rel Frobenius {rf:.3e} > {F32_REL_FROB}"
        return rf, None
    er = ref if elem_ref is None else np.asarray(elem_ref, dtype=np.float64)
    assert er.shape == ref.shape, (what, er.shape, ref.shape)
    ma = max_err_unit_scale(got, er, row_unit)
    assert rf <= BF16_REL_FROB, f"{what}: rel Frobenius {rf:.3e} > {BF16_REL_FROB}"
    assert ma <= BF16_MAX_ABS_UNIT, f"{what}: max abs (unit scale) {ma:.3e} > {BF16_MAX_ABS_UNIT}"
    return rf, ma


def say(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
