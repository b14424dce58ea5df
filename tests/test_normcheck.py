"""CPU checks of the weighted output-norm metric (tests/normcheck.py): it passes an
output whose only error is o's own (at the bf16 level, with floor gates making many rows
of tiny |o|) plus the bf16 rounding of y, and it fails plausible epilogue mistakes by
itself, without help from the other two checks."""
import numpy as np
import pytest
import torch

import normcheck
import oracle


def _case(seed=0, rows=4000, V=128):
    rng = np.random.default_rng(seed)
    # row magnitudes spread over four decades, as under gates at the -5 floor
    o_ref = rng.standard_normal((rows, V)) * 10.0 ** rng.uniform(-4, 0, (rows, 1))
    z = torch.randn(rows, V, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16).float().numpy()
    w = 1.0 + 0.1 * rng.standard_normal(V)
    # a kernel o: relative error 4e-3 of the whole tensor, spread like o itself
    o_k = o_ref + 4e-3 * np.linalg.norm(o_ref) / np.sqrt(o_ref.size) * rng.standard_normal(o_ref.shape)
    return o_ref, o_k, z, w


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_weighted_metric_accepts_o_error_plus_rounding():
    o_ref, o_k, z, w = _case()
    y_ref = oracle.gated_rmsnorm(o_ref, z, w, 1e-6)
    y = _bf16(oracle.gated_rmsnorm(o_k, z, w, 1e-6))
    e_w = normcheck.weighted_rel_l2(y, y_ref, o_ref)
    assert e_w <= normcheck.TOL_Y_WEIGHTED, e_w
    # the unweighted metric is dominated by the rows of tiny |o|: it cannot be the gate
    assert oracle.rel_l2(y, y_ref) > 10 * normcheck.TOL_Y_WEIGHTED


@pytest.mark.parametrize("kind", ["scale_1pct", "three_of_four_partials", "gate_sign", "eps_dropped_mean",
                                  "weight_missing"])
def test_weighted_metric_catches_epilogue_mistake(kind):
    o_ref, o_k, z, w = _case(1)
    y_ref = oracle.gated_rmsnorm(o_ref, z, w, 1e-6)
    ms = np.mean(o_k * o_k, axis=-1, keepdims=True)
    gate = 1.0 / (1.0 + np.exp(-z))
    if kind == "scale_1pct":
        y = 1.01 * oracle.gated_rmsnorm(o_k, z, w, 1e-6)
    elif kind == "three_of_four_partials":       # one consumer wave's sum of squares lost
        ms3 = np.mean(o_k[:, :96] * o_k[:, :96], axis=-1, keepdims=True) * 0.75
        y = o_k / np.sqrt(ms3 + 1e-6) * w * gate
    elif kind == "gate_sign":
        y = o_k / np.sqrt(ms + 1e-6) * w * (1.0 - gate)
    elif kind == "eps_dropped_mean":             # sum of squares over V instead of the mean
        y = o_k / np.sqrt(ms * o_k.shape[-1] + 1e-6) * w * gate
    else:
        y = o_k / np.sqrt(ms + 1e-6) * gate
    e_w = normcheck.weighted_rel_l2(_bf16(y), y_ref, o_ref)
    assert e_w > normcheck.TOL_Y_WEIGHTED, (kind, e_w)


def test_weighted_metric_hand_values():
    """Two rows: r = 1 and r = 100 (eps = 0); an error of 0.1 on the first row only gives
    0.1 / sqrt(1 * 1 + 100^2 * 1) against references of norm 1 in each row."""
    o_ref = np.array([[1.0, 1.0, 1.0, 1.0], [100.0, 100.0, 100.0, 100.0]])
    y_ref = np.array([[1.0, 0.0, 0.0, 0.0], [1.0, 0.0, 0.0, 0.0]])
    y = y_ref.copy()
    y[0, 1] = 0.1
    e = normcheck.weighted_rel_l2(y, y_ref, o_ref, eps=0.0)
    assert abs(e - 0.1 / np.sqrt(1.0 + 1e4)) < 1e-15
