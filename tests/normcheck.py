"""The check of a gated-RMS-normalised output y against the float64 oracle's y.

The norm is scale-free per (token, head) row, so y inherits each row's relative error
of o whatever the row's magnitude, and a plain whole-tensor relative L2 of y weights
every row alike: rows whose |o| is small (fast-decaying gates make many) carry
relative errors far above o's magnitude-weighted error.  Weighting each row of the
error and of the reference by that row's oracle RMS of o removes this: with
c = w * sigmoid(z) and r the row's oracle RMS,

    (y - y_ref) * r  ~=  c * (o - o_ref)_perp + r * (rounding of y),
    y_ref * r        ~=  c * o_ref,

so the weighted relative L2 of y is bounded by o's own relative error (whose gate is
TOL_O) plus one bf16 rounding of y (2^-9 relative), independently of any other check.
"""
import numpy as np

TOL_O = 5e-3
TOL_Y_WEIGHTED = TOL_O + 2.0 ** -9


def weighted_rel_l2(y, y_ref, o_ref, eps=1e-6):
    """||(y - y_ref) r|| / ||y_ref r|| with r = sqrt(mean(o_ref^2) + eps) per row (last axis)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    r = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + eps)
    num = np.linalg.norm(((y - y_ref) * r).ravel())
    den = np.linalg.norm((y_ref * r).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
