"""Comparison metric for GPU-vs-oracle parity (test infrastructure only).

For an output row x (one query's vector along the last axis: q_cat or o_lat per head,
v or out per token):  max |x_gpu - x_oracle| <= tol * rms(x_oracle), tol = 1e-4 in
float32 mode and 2e-2 in bf16 / Q8_0 mode.  Outputs stored in bf16 are additionally
allowed half a bf16 ulp of the exact value, the rounding of the stored result itself.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2, "q8_0": 2e-2}


def half_ulp_bf16(r):
    """Half a bfloat16 unit in the last place at |r| (8 significant bits)."""
    r = np.abs(np.asarray(r, np.float64))
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - 7)


def row_error(g, r, mode):
    """Largest over rows of max|g - r| / rms(r_row), after the storage allowance."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    d = np.abs(g - r)
    if mode != "f32":
        d = np.maximum(d - half_ulp_bf16(r), 0.0)
    rms = np.sqrt((r ** 2).mean(axis=-1))
    return float((d.max(axis=-1) / np.maximum(rms, 1e-30)).max())
