"""Error metrics for comparing a scan result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Row-normalised max relative error: for each output row (token t, head h),
max_j |o - o*| divided by max_j |o*|, the row's own scale, floored at
1e-6 times the largest |o*| of the whole array so that rows whose exact value
is (near) zero do not divide by zero.  The result is the maximum over rows.
Final states use the same rule with one (view, head) d_k x d_v matrix as the
"row".
"""
import numpy as np


def _as_np(x):
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_err(out, ref):
    out, ref = _as_np(out), _as_np(ref)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if out.size == 0:
        return 0.0
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    floor = 1e-6 * float(np.abs(ref).max())
    if floor == 0.0:
        return float(num.max())
    return float((num / np.maximum(den, floor)).max())


def state_rel_err(st, ref):
    st, ref = _as_np(st), _as_np(ref)
    if st.size == 0:
        return 0.0
    shp = st.shape[:-2] + (st.shape[-2] * st.shape[-1],)
    return row_rel_err(st.reshape(shp), ref.reshape(shp))
