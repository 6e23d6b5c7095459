"""Parity metric shared by the GPU tests.

The bound is a maximum relative error: for each (batch, head) slice (decode: each
(sequence, head) slice and step), ||x - x_ref||_inf / ||x_ref||_inf, maximised
over slices, separately for the outputs o and the final states.  A purely
elementwise ratio is ill-posed where o crosses zero, so it is not the gate.
"""
import numpy as np

TOL_FP32 = 1e-4   # fp32 inputs
TOL_BF16 = 2e-2   # bf16 inputs with fp32 accumulation and state


def slice_rel(x, ref, slice_axes):
    """Max over slices of ||x - ref||_inf / ||ref||_inf.

    ``slice_axes`` are the axes that index slices; every other axis belongs to
    the slice.
    """
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    other = tuple(a for a in range(x.ndim) if a not in slice_axes)
    if not other:
        other = None
    err = np.max(np.abs(x - ref), axis=other)
    scale = np.max(np.abs(ref), axis=other)
    scale = np.where(scale > 0, scale, 1.0)
    return float(np.max(err / scale)) if err.size else 0.0


def to_np(t):
    return t.detach().float().cpu().numpy() if t is not None else None
