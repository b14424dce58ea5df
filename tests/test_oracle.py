"""Pins of the float64 oracle against facts other than itself (CPU only).

Each pin is a function of an implementation with the oracle's signature
(q, k, v, g, beta, initial_state, cu_seqlens) -> (o, final_state).  Both oracle
implementations (numpy and C) must pass every pin, and each planted mistake in
``MUTANTS`` (a copy of the recurrence with one plausible error) must fail at
least one pin, which shows the pins can see that class of mistake.

P1  beta = 0: pure decay, closed form.
P2  g = 0, beta = 1, orthonormal keys: the textbook delta rule is an exact
    orthogonal projection; reading a written key returns its value.
P3  two steps at d = 2 worked by hand.
P4  the per-step identity k^T S_t = (1 - b|k|^2) k^T D S_{t-1} + b|k|^2 v^T.
P5  linearity in (V, S0) and the segment map S_T = M S0 + C.
P6  split invariance: continuing from the intermediate state is exact.
P7  the brute-force chunked (WY/UT) form, chunk 16 and 64, agrees to 1e-12.
P8  packing independence: varlen == separate runs; heads are independent.
"""
import numpy as np
import pytest

import oracle
from oracle.chunked import chunked

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rand_case(seed, lengths, H=2, DK=8, DV=6, zero_state=False, gate_lo=-5.0, unit_keys=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, DK))
    k = rng.standard_normal((T, H, DK))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, DV))
    g = gate_lo / (1.0 + np.exp(-rng.standard_normal((T, H, DK))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    s0 = None if zero_state else 0.1 * rng.standard_normal((len(lengths), H, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0, cu_seqlens=cu)


def call(impl, c):
    return impl(c["q"], c["k"], c["v"], c["g"], c["beta"], c["initial_state"], c["cu_seqlens"])


# ---------------------------------------------------------------- pins -----

def pin_beta_zero(impl):
    c = rand_case(1, [9, 0, 5], H=2, DK=5, DV=4)
    c["beta"] = np.zeros_like(c["beta"])
    o, sT = call(impl, c)
    cu = c["cu_seqlens"]
    for n in range(len(cu) - 1):
        for h in range(2):
            Gam = np.zeros(5)
            for t in range(cu[n], cu[n + 1]):
                Gam = Gam + c["g"][t, h]
                want = c["initial_state"][n, h].T @ (np.exp(Gam) * c["q"][t, h])
                if not np.allclose(o[t, h], want, rtol=1e-13, atol=1e-15):
                    return False
            if not np.allclose(sT[n, h], np.exp(Gam)[:, None] * c["initial_state"][n, h],
                               rtol=1e-13, atol=1e-15):
                return False
    return True


def pin_orthonormal_delta_rule(impl):
    rng = np.random.default_rng(2)
    DK, DV, T = 8, 5, 6
    K = np.linalg.qr(rng.standard_normal((DK, DK)))[0][:, :T].T   # T orthonormal rows
    V = rng.standard_normal((T, DV))
    S0 = rng.standard_normal((DK, DV))
    o, sT = impl(K[:, None, :], K[:, None, :], V[:, None, :], np.zeros((T, 1, DK)),
                 np.ones((T, 1)), S0[None, None], np.array([0, T]))
    want_S = (np.eye(DK) - K.T @ K) @ S0 + K.T @ V
    return bool(np.allclose(sT[0, 0], want_S, rtol=1e-12, atol=1e-12)
                and np.allclose(o[:, 0], V, rtol=1e-12, atol=1e-12))


def pin_hand_worked_d2(impl):
    # Token 1: S0=[[1,2],[3,4]], g=[ln .5, ln .25] -> D S0=[[.5,1],[.75,1]];
    #   k=[.6,.8]: r = k^T D S0 = [.9, 1.4]; v=[1,-1]: v-r = [.1,-2.4];
    #   beta=.5: beta k (v-r)^T = [[.03,-.72],[.04,-.96]] -> S1=[[.53,.28],[.79,.04]];
    #   q=[.2,.5]: o1 = S1^T q = [.501, .076].
    # Token 2: g=[0, ln .5] -> D S1=[[.53,.28],[.395,.02]]; k=[1,0], beta=1:
    #   r=[.53,.28], v=[2,3] -> row 0 becomes v: S2=[[2,3],[.395,.02]];
    #   q=[0,1]: o2 = [.395, .02].
    q = np.array([[[0.2, 0.5]], [[0.0, 1.0]]])
    k = np.array([[[0.6, 0.8]], [[1.0, 0.0]]])
    v = np.array([[[1.0, -1.0]], [[2.0, 3.0]]])
    g = np.log(np.array([[[0.5, 0.25]], [[1.0, 0.5]]]))
    beta = np.array([[0.5], [1.0]])
    S0 = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    o, sT = impl(q, k, v, g, beta, S0, np.array([0, 2]))
    return bool(np.allclose(o[:, 0], [[0.501, 0.076], [0.395, 0.02]], rtol=0, atol=1e-14)
                and np.allclose(sT[0, 0], [[2.0, 3.0], [0.395, 0.02]], rtol=0, atol=1e-14))


def pin_step_identity(impl):
    c = rand_case(4, [7], H=1, DK=6, DV=5, unit_keys=False)
    S = c["initial_state"][0, 0]
    for t in range(7):
        one = {key: (c[key][t:t + 1] if key in ("q", "k", "v", "g", "beta") else None) for key in c}
        one["initial_state"] = S[None, None]
        one["cu_seqlens"] = np.array([0, 1])
        _, sT = call(impl, one)
        k, b = c["k"][t, 0], c["beta"][t, 0]
        nk = float(k @ k)
        lhs = k @ sT[0, 0]
        rhs = (1 - b * nk) * (k @ (np.exp(c["g"][t, 0])[:, None] * S)) + b * nk * c["v"][t, 0]
        if not np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12):
            return False
        S = sT[0, 0]
    return True


def pin_linearity_and_segment_map(impl):
    c1 = rand_case(5, [11, 4], H=2, DK=6, DV=4)
    c2 = rand_case(6, [11, 4], H=2, DK=6, DV=4)
    mix = dict(c1)
    mix["v"] = c1["v"] + 2.0 * c2["v"]
    mix["initial_state"] = c1["initial_state"] + 2.0 * c2["initial_state"]
    c2s = dict(c1, v=c2["v"], initial_state=c2["initial_state"])
    o1, s1 = call(impl, c1)
    o2, s2 = call(impl, c2s)
    om, sm = call(impl, mix)
    if not (np.allclose(om, o1 + 2 * o2, rtol=1e-11, atol=1e-12)
            and np.allclose(sm, s1 + 2 * s2, rtol=1e-11, atol=1e-12)):
        return False
    # segment map: M from (V = 0, S0 = I), C from S0 = 0; S_T = M S0 + C
    N, H, DK, DV = 2, 2, 6, 6
    cs = rand_case(7, [13, 3], H=H, DK=DK, DV=DV)
    eye = np.broadcast_to(np.eye(DK), (N, H, DK, DK)).copy()
    _, M = call(impl, dict(cs, v=np.zeros_like(cs["v"]), initial_state=eye))
    _, C = call(impl, dict(cs, initial_state=np.zeros_like(cs["initial_state"])))
    _, S = call(impl, cs)
    return bool(np.allclose(S, M @ cs["initial_state"] + C, rtol=1e-11, atol=1e-12))


def pin_split_invariance(impl):
    c = rand_case(8, [23], H=2, DK=5, DV=4)
    o_full, s_full = call(impl, c)
    T1 = 9
    a = {key: (c[key][:T1] if key in ("q", "k", "v", "g", "beta") else c[key]) for key in c}
    a["cu_seqlens"] = np.array([0, T1])
    oa, sa = call(impl, a)
    b = {key: (c[key][T1:] if key in ("q", "k", "v", "g", "beta") else c[key]) for key in c}
    b["cu_seqlens"] = np.array([0, 23 - T1])
    b["initial_state"] = sa
    ob, sb = call(impl, b)
    return bool(np.array_equal(np.concatenate([oa, ob]), o_full) and np.array_equal(sb, s_full))


def pin_chunked_twin(impl):
    for chunk in (16, 64):
        for gate_lo in (-5.0, -1.0):
            c = rand_case(9, [130, 0, 64, 17], H=2, DK=8, DV=6, gate_lo=gate_lo)
            o, sT = call(impl, c)
            oc, sc = chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], c["initial_state"],
                             c["cu_seqlens"], chunk=chunk)
            if oracle.rel_l2(oc, o) > 1e-12 or oracle.rel_l2(sc, sT) > 1e-12:
                return False
    return True


def pin_packing_independence(impl):
    lengths = [6, 0, 13, 1]
    c = rand_case(10, lengths, H=3, DK=4, DV=5)
    o, sT = call(impl, c)
    cu = c["cu_seqlens"]
    for n in range(len(lengths)):
        sl = slice(cu[n], cu[n + 1])
        one = {key: (c[key][sl] if key in ("q", "k", "v", "g", "beta") else None) for key in c}
        one["initial_state"] = c["initial_state"][n:n + 1]
        one["cu_seqlens"] = np.array([0, lengths[n]])
        o1, s1 = call(impl, one)
        if not (np.array_equal(o1, o[sl]) and np.array_equal(s1[0], sT[n])):
            return False
    perm = [2, 0, 1]
    cp = {key: (c[key][:, perm] if key in ("q", "k", "v", "g", "beta") else c[key]) for key in c}
    cp["initial_state"] = c["initial_state"][:, perm]
    op, sp = call(impl, cp)
    return bool(np.array_equal(op, o[:, perm]) and np.array_equal(sp, sT[:, perm]))


PINS = {
    "P1_beta_zero": pin_beta_zero,
    "P2_orthonormal_delta_rule": pin_orthonormal_delta_rule,
    "P3_hand_worked_d2": pin_hand_worked_d2,
    "P4_step_identity": pin_step_identity,
    "P5_linearity_segment_map": pin_linearity_and_segment_map,
    "P6_split_invariance": pin_split_invariance,
    "P7_chunked_twin": pin_chunked_twin,
    "P8_packing_independence": pin_packing_independence,
}


def c_oracle(*args):
    return oracle.run_c(*args, threads=2)


IMPLS = {"numpy": oracle.recurrence, "c": c_oracle}


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("pin", sorted(PINS))
def test_pin(pin, impl, oracle_lib):
    assert PINS[pin](IMPLS[impl]), f"oracle ({impl}) fails {pin}"


# ------------------------------------------------- planted mistakes -------

def _mutant(kind):
    """A copy of the numpy recurrence with one planted mistake."""
    def impl(q, k, v, g, beta, initial_state=None, cu_seqlens=None):
        q, k, v, g, beta, s0, cu = oracle._packed(q, k, v, g, beta, initial_state, cu_seqlens)
        T, H, DK = q.shape
        DV = v.shape[-1]
        N = len(cu) - 1
        o = np.zeros((T, H, DV))
        sT = np.zeros((N, H, DK, DV))
        for n in range(N):
            for h in range(H):
                S = np.zeros((DK, DV)) if s0 is None else s0[n, h].copy()
                for t in range(cu[n], cu[n + 1]):
                    gt = g[t - 1, h] if (kind == "gate_index" and t > cu[n]) else g[t, h]
                    bt = 1.0 if kind == "dropped_beta" else beta[t, h]
                    if kind == "decay_after_delta":
                        S = S + bt * np.outer(k[t, h], v[t, h] - k[t, h] @ S)
                        S = np.exp(gt)[:, None] * S
                    else:
                        S_prev = S
                        S = np.exp(gt)[:, None] * S
                        r = k[t, h] @ (S_prev if kind == "undecayed_read" else S)
                        sign = -1.0 if kind == "sign" else 1.0
                        S = S + bt * np.outer(k[t, h], v[t, h] - sign * r)
                    if kind == "transposed_output":
                        o[t, h] = S @ q[t, h]
                    elif kind == "pre_update_output":
                        o[t, h] = (np.exp(gt)[:, None] * S_prev).T @ q[t, h]
                    else:
                        o[t, h] = S.T @ q[t, h]
                sT[n, h] = S
        return o, sT
    return impl


MUTANTS = ["gate_index", "dropped_beta", "decay_after_delta", "undecayed_read", "sign",
           "transposed_output", "pre_update_output"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    results = {}
    for name, pin in PINS.items():
        try:
            results[name] = pin(_mutant(kind))
        except ValueError:          # a shape error is also a caught mistake
            results[name] = False
    assert not all(results.values()), f"no pin catches the '{kind}' mistake: {results}"


def test_c_matches_numpy_on_random_case(oracle_lib):
    c = rand_case(11, [70, 3, 0, 40], H=3, DK=16, DV=12)
    o1, s1 = call(oracle.recurrence, c)
    o2, s2 = call(c_oracle, c)
    assert oracle.rel_l2(o2, o1) < 1e-13 and oracle.rel_l2(s2, s1) < 1e-13


def test_gate_floor_finite(oracle_lib):
    c = rand_case(12, [200], H=2, DK=16, DV=16)
    c["g"] = np.full_like(c["g"], -5.0)
    o, sT = call(c_oracle, c)
    assert np.isfinite(o).all() and np.isfinite(sT).all()
    oc, sc = chunked(c["q"], c["k"], c["v"], c["g"], c["beta"], c["initial_state"],
                     c["cu_seqlens"], chunk=64)
    assert oracle.rel_l2(oc, o) < 1e-12 and oracle.rel_l2(sc, sT) < 1e-12


def test_zero_length_sequence_keeps_state(oracle_lib):
    c = rand_case(13, [0, 5, 0], H=2, DK=4, DV=4)
    o, sT = call(c_oracle, c)
    assert np.array_equal(sT[0], c["initial_state"][0])
    assert np.array_equal(sT[2], c["initial_state"][2])


def test_tiny_workload_runs(oracle_lib):
    import workloads
    w = workloads.WORKLOADS["tiny"]
    x = workloads.make_inputs(w)
    o, sT = oracle.run_c(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    assert o.shape == (256, 2, 64) and sT.shape == (1, 2, 64, 64)
    assert np.isfinite(o).all()
    # the recorded oracle output for this workload must not drift
    import json, os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_summary.json")
    ref = json.load(open(path))
    assert abs(float(np.linalg.norm(o)) - ref["o_norm"]) <= 1e-9 * ref["o_norm"]
    assert abs(float(np.linalg.norm(sT)) - ref["state_norm"]) <= 1e-9 * ref["state_norm"]
    np.testing.assert_allclose(o[::37, :, ::13].ravel(), ref["o_samples"], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------- activations (NEXT-1)
def _activation_closed_forms(act):
    x = np.array([0.0, np.log(3.0), -np.log(3.0), 800.0, -800.0])
    g, b = act(x, x, lower_bound=-5.0)
    np.testing.assert_allclose(g, [-2.5, -3.75, -1.25, -5.0, 0.0], rtol=1e-15, atol=0)
    np.testing.assert_allclose(b, [0.5, 0.75, 0.25, 1.0, 0.0], rtol=1e-15, atol=0)


def test_activations_closed_forms():
    """g = lb * sigmoid(x), beta = sigmoid(b) at points with exact values:
    sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4; the limits
    lb (x -> +inf) and 0 (x -> -inf); and sigmoid(x) + sigmoid(-x) = 1."""
    _activation_closed_forms(oracle.activations)
    rng = np.random.default_rng(3)
    y = rng.normal(size=1000) * 4
    _, b1 = oracle.activations(None, y)
    _, b2 = oracle.activations(None, -y)
    np.testing.assert_allclose(b1 + b2, 1.0, rtol=0, atol=1e-15)
    gz, _ = oracle.activations(y, None, lower_bound=0.0)
    assert np.all(gz == 0.0)


def test_activations_match_library_logistic():
    """The activation is the logistic function of scipy.special.expit (a library
    routine), scaled by the lower bound."""
    from scipy.special import expit
    rng = np.random.default_rng(4)
    x = rng.normal(size=(64, 3, 16)) * 3
    g, b = oracle.activations(x, x[..., 0], lower_bound=-3.5)
    np.testing.assert_allclose(g, -3.5 * expit(x), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(b, expit(x[..., 0]), rtol=1e-14, atol=1e-300)


def test_activations_with_zero_beta_reduce_to_pure_decay(oracle_lib):
    """beta logits at -inf give beta = 0: the recurrence is pure decay (pin P1),
    S_T = Diag(e^{sum g}) S0 with g = lb * sigmoid(x)."""
    rng = np.random.default_rng(5)
    T, H, D = 7, 1, 3
    q, k, v = (rng.normal(size=(T, H, D)) for _ in range(3))
    x = rng.normal(size=(T, H, D))
    g, beta = oracle.activations(x, np.full((T, H), -1e4), lower_bound=-2.0)
    s0 = rng.normal(size=(1, H, D, D))
    _, sT = oracle.recurrence(q, k, v, g, beta, s0, np.array([0, T]))
    want = np.exp(g.sum(axis=0))[0][:, None] * s0[0, 0]
    np.testing.assert_allclose(sT[0, 0], want, rtol=1e-13)


@pytest.mark.parametrize("kind", ["sign", "no_bound", "exp_not_logistic"])
def test_activation_pins_catch_planted_mistake(kind):
    """A plausible slip in the activation (a sign, the bound dropped, e^x in
    place of the logistic) fails the closed-form pin."""
    def bad(gx, bx, lower_bound=-5.0):
        def f(x):
            x = np.asarray(x, dtype=np.float64)
            if kind == "sign":
                return 1.0 / (1.0 + np.exp(x))
            if kind == "exp_not_logistic":
                return np.exp(np.minimum(x, 0.0))
            return 1.0 / (1.0 + np.exp(-x))
        return (f(gx) * (1.0 if kind == "no_bound" else lower_bound)), f(bx)
    with pytest.raises(AssertionError):
        _activation_closed_forms(bad)


# ----------------------------------------------------------- gated RMSNorm epilogue (NEXT-4)
def _gated_rmsnorm_pins(fn):
    rng = np.random.default_rng(7)
    o = rng.normal(size=(5, 3, 16))
    z = rng.normal(size=(5, 3, 16))
    w = rng.normal(size=16)
    # a constant row c * 1 has mean square c^2: with eps = 0 the row maps to sign(c) * w * sigmoid(z)
    c = np.full((2, 16), -3.0)
    y = fn(c, np.zeros((2, 16)), np.ones(16), 0.0)
    np.testing.assert_allclose(y, -0.5, rtol=1e-15)
    # scale invariance at eps = 0
    np.testing.assert_allclose(fn(7.5 * o, z, w, 0.0), fn(o, z, w, 0.0), rtol=1e-13)
    # an open gate (z -> +inf) leaves the library RMS norm (torch, float64) times the weight
    import torch
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), weight=torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(fn(o, np.full_like(z, 800.0), w, 1e-6), ref, rtol=1e-12, atol=1e-15)
    # the gate is the logistic function: z = 0 halves the open-gate result
    np.testing.assert_allclose(fn(o, np.zeros_like(z), w, 1e-6), 0.5 * ref, rtol=1e-12, atol=1e-15)


def test_gated_rmsnorm_pins():
    """Closed forms (a constant row; scale invariance), the library RMS norm
    (torch.nn.functional.rms_norm in float64) for an open gate, and the logistic
    gate at z = 0."""
    _gated_rmsnorm_pins(oracle.gated_rmsnorm)


@pytest.mark.parametrize("kind", ["mean_not_rms", "no_eps_inside_root", "gate_sign", "sum_not_mean"])
def test_gated_rmsnorm_pins_catch_planted_mistake(kind):
    def bad(o, z, w, eps):
        o, z, w = (np.asarray(a, dtype=np.float64) for a in (o, z, w))
        ms = np.mean(o * o, axis=-1, keepdims=True)
        if kind == "mean_not_rms":
            r = 1.0 / (np.abs(np.mean(o, axis=-1, keepdims=True)) + eps)
        elif kind == "no_eps_inside_root":
            r = 1.0 / (np.sqrt(ms) + eps)
        elif kind == "sum_not_mean":
            r = 1.0 / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps)
        else:
            r = 1.0 / np.sqrt(ms + eps)
        gate = 1.0 / (1.0 + np.exp(z if kind == "gate_sign" else -z))
        return o * r * w * gate
    with pytest.raises(AssertionError):
        _gated_rmsnorm_pins(bad)


# ----------------------------------------------------------- the parity metric itself
def _rel_l2_pins(fn):
    """Hand-computed values of the whole-tensor relative L2 error ||x - ref|| / ||ref||."""
    ref = np.array([2.0, 3.0, 6.0])                       # ||ref|| = 7
    # a difference of norm 0.07 (0.02, 0.03, -0.06) gives 0.01
    assert abs(fn(ref + np.array([0.02, 0.03, -0.06]), ref) - 0.01) <= 1e-15
    # x = ref (1 + eps) gives eps, at several scales of eps
    for eps in (1e-1, 4e-3, 1e-6):
        assert abs(fn(ref * (1.0 + eps), ref) - eps) <= 1e-12 * max(eps, 1e-3)
    assert fn(np.zeros(3), ref) == 1.0                    # x = 0: the whole reference is error
    assert fn(ref, ref) == 0.0
    # the denominator is the reference's norm, not x's: x = 2 ref gives 1, ref against 2 ref 1/2
    assert fn(2.0 * ref, ref) == 1.0
    assert fn(ref, 2.0 * ref) == 0.5
    # whole tensor, not a mean of per-row ratios: rows of norm 7 and 700 with errors of norm
    # 0.07 and 0 give 0.07 / sqrt(7^2 + 700^2), not (0.01 + 0) / 2
    big = np.stack([ref, 100.0 * ref])
    err = np.stack([ref + np.array([0.02, 0.03, -0.06]), 100.0 * ref])
    assert abs(fn(err, big) - 0.07 / np.sqrt(49.0 + 490000.0)) <= 1e-15
    # any shape and dtype is flattened: a 3-D float32 tensor of 3-4-5 triangles
    x3 = np.zeros((2, 2, 2), dtype=np.float32)
    r3 = np.zeros((2, 2, 2), dtype=np.float32)
    r3[0, 0, 0], r3[1, 1, 1] = 3.0, 4.0                   # ||r3|| = 5
    x3[0, 0, 0], x3[1, 1, 1] = 3.0, 4.0
    x3[0, 1, 0] = 0.5                                      # error norm 0.5
    assert abs(fn(x3, r3) - 0.1) <= 1e-15


def test_rel_l2_pins():
    """The metric every parity verdict uses, against values worked by hand (a 2-3-6-7
    quadruple, x = ref (1 + eps), x = 0, the asymmetry of the denominator, whole-tensor
    rather than per-row aggregation, and a float32 3-D tensor)."""
    _rel_l2_pins(oracle.rel_l2)
    import torch
    assert abs(oracle.rel_l2(torch.tensor([2.0, 3.0, 6.0]) * 1.004, torch.tensor([2.0, 3.0, 6.0])) - 4e-3) < 1e-6   # float32 inputs
    # a zero reference: exact agreement is 0, anything else infinite
    assert oracle.rel_l2(np.zeros(4), np.zeros(4)) == 0.0
    assert oracle.rel_l2(np.ones(4), np.zeros(4)) == float("inf")


@pytest.mark.parametrize("kind", ["no_sqrt", "swapped_arguments", "mean_of_rows", "max_abs", "l1"])
def test_rel_l2_pins_catch_planted_mistake(kind):
    """Plausible slips in the metric each fail the pins: a missing square root (which would
    turn a 4e-3 error into 1.6e-5), the arguments swapped (dividing by ||x||), a mean of
    per-row ratios, a max-abs ratio and an L1 ratio."""
    def bad(x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        d = x - ref
        if kind == "no_sqrt":
            return float(np.sum(d * d) / np.sum(ref * ref))
        if kind == "swapped_arguments":
            return float(np.linalg.norm(d) / np.linalg.norm(x)) if np.linalg.norm(x) else 1.0
        if kind == "mean_of_rows":
            d2, r2 = d.reshape(-1, d.shape[-1]), ref.reshape(-1, ref.shape[-1])
            return float(np.mean(np.linalg.norm(d2, axis=-1) / np.linalg.norm(r2, axis=-1)))
        if kind == "max_abs":
            return float(np.abs(d).max() / np.abs(ref).max())
        return float(np.abs(d).sum() / np.abs(ref).sum())
    with pytest.raises(AssertionError):
        _rel_l2_pins(bad)


# ----------------------------------------------------------- the dense [B, T, H, D] layout
@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_dense_layout_equals_packed(impl, oracle_lib):
    """A dense [B, T, H, D] call gives, bit for bit, the packed call on the same values laid
    out sequence after sequence (built here by concatenating the batch entries, not by the
    oracle's own reshape) with cu = [0, T, 2T, ...]; a packed call with 4-D [1, T, H, D]
    tensors gives the 3-D packed call's bits."""
    fn = IMPLS[impl]
    rng = np.random.default_rng(17)
    B, T, H, DK, DV = 3, 11, 2, 5, 4
    q, k = rng.standard_normal((B, T, H, DK)), rng.standard_normal((B, T, H, DK))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, DK))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.1 * rng.standard_normal((B, H, DK, DV))
    od, sd = fn(q, k, v, g, beta, s0, None)
    cat = lambda a: np.concatenate([a[b] for b in range(B)], axis=0)
    cu = np.arange(B + 1, dtype=np.int64) * T
    op, sp = fn(cat(q), cat(k), cat(v), cat(g), cat(beta), s0, cu)
    assert od.shape == (B * T, H, DV) and sd.shape == (B, H, DK, DV)
    assert np.array_equal(od, op) and np.array_equal(sd, sp)
    o4, s4 = fn(cat(q)[None], cat(k)[None], cat(v)[None], cat(g)[None], cat(beta)[None], s0, cu)
    assert np.array_equal(o4, op) and np.array_equal(s4, sp)
    # and each batch entry alone is the same as its rows of the batched call
    for b in range(B):
        ob, sb = fn(q[b], k[b], v[b], g[b], beta[b], s0[b:b + 1], np.array([0, T]))
        assert np.array_equal(ob, od[b * T:(b + 1) * T]) and np.array_equal(sb[0], sd[b])


@pytest.mark.parametrize("kind", ["time_major", "batch_head_swap"])
def test_dense_layout_pin_catches_planted_mistake(kind):
    """A dense reshape that interleaves the batch and token axes, or swaps batch and head,
    fails the dense-layout pin."""
    def bad(q, k, v, g, beta, s0=None, cu=None):
        if q.ndim == 4 and cu is None:
            if kind == "time_major":
                fix = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1)).reshape(a.shape[0] * a.shape[1], *a.shape[2:])
            else:
                fix = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 2)).reshape(a.shape[2] * a.shape[1], *a.shape[2:]) \
                    if a.ndim == 4 else np.ascontiguousarray(np.swapaxes(a, 0, 2)).reshape(a.shape[2] * a.shape[1], a.shape[0])
            B, T = q.shape[:2]
            try:
                return oracle.recurrence(fix(q), fix(k), fix(v), fix(g), fix(beta), s0, np.arange(B + 1) * T)
            except (ValueError, IndexError):
                return np.zeros(1), np.zeros(1)
        return oracle.recurrence(q, k, v, g, beta, s0, cu)
    saved = dict(IMPLS)
    IMPLS["bad"] = bad
    try:
        with pytest.raises(AssertionError):
            test_dense_layout_equals_packed("bad", None)
    finally:
        IMPLS.clear()
        IMPLS.update(saved)
