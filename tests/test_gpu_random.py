"""Seeded random configurations of the prefill against the float64 oracle.

Each case draws a batch layout (dense or packed, with empty and ragged sequences),
a head count, the head size and I/O dtype (d = 128 bf16 or the d = 64 fp32 debug
mode), a segment count (the planner's or forced), the kernel variant, the state
dtypes (fp32 or bf16), logit inputs and, on the pipelined kernel, the gated RMS
norm epilogue — and checks every output and final state with the tolerances of
the other parity tests.  The cases are drawn once, from a fixed seed, so the set
is the same on every run.  KDA_RANDOM_CASES=n widens the sweep to the first n
cases (24 by default).
"""
import os
import sys

import numpy as np
import pytest

import normcheck
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 5e-3, "f32": 1e-4}


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    fp32 = rng.random() < 0.25
    D = 64 if fp32 else 128
    dense = rng.random() < 0.3
    n = int(rng.integers(1, 6))
    if dense:
        L = int(rng.integers(1, 700))
        lengths = [L] * n
    else:
        lengths = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 900, n)]
    H = int(rng.integers(1, 4))
    variant = 1 if fp32 else int(rng.choice([0, 0, 1, 2]))
    nseg = int(rng.choice([0, 0, 1, 2, 3, 5]))
    pipelined = not fp32 and variant != 1
    return dict(case=i, fp32=fp32, D=D, dense=dense, lengths=lengths, H=H, variant=variant, nseg=nseg,
                zero_state=bool(rng.random() < 0.2), bf16_state=bool(rng.random() < 0.3),
                logits=bool(rng.random() < 0.3), norm=bool(pipelined and rng.random() < 0.3),
                gate=str(rng.choice(["none", "none", "none", "mild", "floor"])),
                lb=float(rng.choice([-5.0, -5.0, -3.0, -1.0, -0.25])))      # gate lower bound with logits


CASES = [_draw(i) for i in range(int(os.environ.get("KDA_RANDOM_CASES", "24")))]


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as k
    k.load_library()
    return k


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['case']}" for c in CASES])
def test_random_configuration(kda, c):
    import torch
    print("[case]", c, file=sys.stderr, flush=True)
    w = workloads.custom(c["lengths"], H=c["H"], D=c["D"], dtype="f32" if c["fp32"] else "bf16", dense=c["dense"],
                         zero_state=c["zero_state"], seed=2000 + c["case"])
    gate = None if c["gate"] == "none" else c["gate"]
    x = workloads.make_inputs(w, device="cuda", gate=gate)
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    s0 = x["initial_state"]
    if s0 is not None and c["bf16_state"]:
        s0 = s0.to(torch.bfloat16)
    N = len(c["lengths"])
    fin = torch.empty((N, c["H"], c["D"], c["D"]), device="cuda",
                      dtype=torch.bfloat16 if c["bf16_state"] else torch.float32)
    kw = dict(nseg=c["nseg"], variant=c["variant"], gate_logits=logits, beta_logits=logits, gate_lower_bound=c["lb"])
    z = nw = None
    if c["norm"]:
        gen = torch.Generator(device="cuda").manual_seed(3000 + c["case"])
        z = torch.randn(x["v"].shape, generator=gen, device="cuda").to(x["v"].dtype)
        nw = 1.0 + 0.1 * torch.randn(c["D"], generator=gen, device="cuda")
        kw.update(out_gate=z, norm_weight=nw, norm_eps=1e-6)
    out, _ = kda.prefill(x["q"], x["k"], x["v"], g_in, b_in, s0, x["cu_seqlens"], final_state=fin, **kw)
    torch.cuda.synchronize()
    if logits:
        g64, b64 = oracle.activations(x["g_logits"].cpu(), x["beta_logits"].cpu(), c["lb"])
    else:
        g64, b64 = x["g"].cpu(), x["beta"].cpu()
    o_ref, s_ref = oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), g64, b64,
                                None if s0 is None else s0.float().cpu(),
                                None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu())
    tol = TOL["f32"] if c["fp32"] else TOL["bf16"]
    o_gpu = out.float().cpu().numpy().reshape(o_ref.shape)
    s_gpu = fin.float().cpu().numpy()
    assert np.isfinite(o_gpu).all() and np.isfinite(s_gpu).all()
    es = oracle.rel_l2(s_gpu, s_ref) if np.abs(s_ref).sum() > 0 else float(np.abs(s_gpu).max())
    tol_s = TOL["bf16"] if (c["bf16_state"] or not c["fp32"]) else TOL["f32"]
    assert es <= tol_s, f"rel-L2 state {es:.3e}"
    if c["norm"]:
        # the three checks of the normalised output (tests/normcheck.py): o from the same
        # call without the epilogue against the oracle, y against the exact norm of that o,
        # and y against the oracle's y with rows weighted by their oracle RMS of o
        plain = {k: v for k, v in kw.items() if k not in ("out_gate", "norm_weight", "norm_eps")}
        o_plain, _ = kda.prefill(x["q"], x["k"], x["v"], g_in, b_in, s0, x["cu_seqlens"], **plain)
        y_ref = oracle.gated_rmsnorm(o_ref, z.float().cpu().numpy().reshape(o_ref.shape), nw.cpu().numpy(), 1e-6)
        og = o_plain.float().cpu().numpy().reshape(o_ref.shape)
        y_own = oracle.gated_rmsnorm(og, z.float().cpu().numpy().reshape(o_ref.shape), nw.cpu().numpy(), 1e-6)
        e_o = oracle.rel_l2(og, o_ref) if np.abs(o_ref).sum() > 0 else 0.0
        e_epi = oracle.rel_l2(o_gpu, y_own) if np.abs(y_own).sum() > 0 else 0.0
        e_w = normcheck.weighted_rel_l2(o_gpu, y_ref, o_ref)
        assert e_o <= tol and e_epi <= tol and e_w <= normcheck.TOL_Y_WEIGHTED, \
            f"o {e_o:.3e}, epilogue {e_epi:.3e}, y weighted {e_w:.3e}"
    else:
        eo = oracle.rel_l2(o_gpu, o_ref) if o_ref.size and np.abs(o_ref).sum() > 0 else 0.0
        assert eo <= tol, f"rel-L2 out {eo:.3e}"


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['case']}" for c in CASES])
def test_random_configuration_stalled_wave(kda, c):
    """The same configurations with one wave (chosen by the case) stalled ~20 us after
    every workgroup barrier give the unstalled bits: outputs and final states."""
    import torch
    w = workloads.custom(c["lengths"], H=c["H"], D=c["D"], dtype="f32" if c["fp32"] else "bf16", dense=c["dense"],
                         zero_state=c["zero_state"], seed=2000 + c["case"])
    x = workloads.make_inputs(w, device="cuda", gate=None if c["gate"] == "none" else c["gate"])
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    s0 = x["initial_state"]
    if s0 is not None and c["bf16_state"]:
        s0 = s0.to(torch.bfloat16)
    kw = dict(nseg=c["nseg"], variant=c["variant"], gate_logits=logits, beta_logits=logits, gate_lower_bound=c["lb"])
    if c["norm"]:
        gen = torch.Generator(device="cuda").manual_seed(3000 + c["case"])
        kw.update(out_gate=torch.randn(x["v"].shape, generator=gen, device="cuda").to(x["v"].dtype),
                  norm_weight=1.0 + 0.1 * torch.randn(c["D"], generator=gen, device="cuda"), norm_eps=1e-6)
    waves = 8 if (not c["fp32"] and c["variant"] != 1) else 4
    wave = c["case"] % waves
    print("[case]", c, "stalled wave", wave, file=sys.stderr, flush=True)
    fins = [torch.empty((len(c["lengths"]), c["H"], c["D"], c["D"]), device="cuda",
                        dtype=torch.bfloat16 if c["bf16_state"] else torch.float32) for _ in range(2)]
    o0, _ = kda.prefill(x["q"], x["k"], x["v"], g_in, b_in, s0, x["cu_seqlens"], final_state=fins[0], **kw)
    o1, _ = kda.prefill(x["q"], x["k"], x["v"], g_in, b_in, s0, x["cu_seqlens"], final_state=fins[1],
                        stall_wave=wave, stall_cycles=127 * 6, **kw)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(bits(o0), bits(o1)) and torch.equal(bits(fins[0]), bits(fins[1]))


def _padded(t, rng, align):
    """The same values in a view with padded strides: every dimension but the last gets
    a larger stride (extra channels per row, extra heads per token, ...), each a multiple
    of `align` elements so that vector rows stay aligned."""
    import torch
    shape = list(t.shape)
    pad = [int(rng.integers(0, 3)) * align for _ in shape]
    pad[-1] = int(rng.integers(0, 3)) * align
    big = torch.full([s + p for s, p in zip(shape, pad)], float("nan"), dtype=t.dtype, device=t.device)
    view = big[tuple(slice(0, s) for s in shape)]
    view.copy_(t)
    return view


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['case']}" for c in CASES])
def test_random_configuration_padded_views(kda, c):
    """The same configurations with every tensor (q, k, v, g, beta, states, out, output
    gate) passed as a view with padded strides give the bits of the contiguous call;
    the padding holds NaN, so any read of it would show."""
    import torch
    w = workloads.custom(c["lengths"], H=c["H"], D=c["D"], dtype="f32" if c["fp32"] else "bf16", dense=c["dense"],
                         zero_state=c["zero_state"], seed=2000 + c["case"])
    x = workloads.make_inputs(w, device="cuda", gate=None if c["gate"] == "none" else c["gate"])
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    s0 = x["initial_state"]
    if s0 is not None and c["bf16_state"]:
        s0 = s0.to(torch.bfloat16)
    kw = dict(nseg=c["nseg"], variant=c["variant"], gate_logits=logits, beta_logits=logits, gate_lower_bound=c["lb"])
    z = nw = None
    if c["norm"]:
        gen = torch.Generator(device="cuda").manual_seed(3000 + c["case"])
        z = torch.randn(x["v"].shape, generator=gen, device="cuda").to(x["v"].dtype)
        nw = 1.0 + 0.1 * torch.randn(c["D"], generator=gen, device="cuda")
        kw.update(norm_weight=nw, norm_eps=1e-6)
    print("[case]", c, "padded views", file=sys.stderr, flush=True)
    N = len(c["lengths"])
    sdt = torch.bfloat16 if c["bf16_state"] else torch.float32
    fin0 = torch.empty((N, c["H"], c["D"], c["D"]), device="cuda", dtype=sdt)
    o0, _ = kda.prefill(x["q"], x["k"], x["v"], g_in, b_in, s0, x["cu_seqlens"], final_state=fin0, out_gate=z, **kw)
    rng = np.random.default_rng(4000 + c["case"])
    P = lambda t, a=4: None if t is None else _padded(t, rng, a)
    out1 = P(torch.empty_like(x["v"]))
    fin1 = P(torch.empty((N, c["H"], c["D"], c["D"]), device="cuda", dtype=sdt), 1)
    o1, _ = kda.prefill(P(x["q"]), P(x["k"]), P(x["v"]), P(g_in), P(b_in, 1), P(s0, 1), x["cu_seqlens"],
                        out=out1, final_state=fin1, out_gate=P(z), **kw)
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)
    assert torch.equal(bits(o0), bits(o1)) and torch.equal(bits(fin0), bits(fin1))


@pytest.mark.parametrize("c", [c for c in CASES if not c["dense"] and not c["fp32"] and c["variant"] != 1],
                         ids=lambda c: f"case{c['case']}")
def test_random_configuration_longest_first(kda, c, monkeypatch):
    """The packed pipelined configurations as one segment, with the chains started longest
    sequence first (KDA_ORDER=longest) and in launch order: the same bits."""
    import torch
    w = workloads.custom(c["lengths"], H=c["H"], D=c["D"], dtype="bf16", dense=False,
                         zero_state=c["zero_state"], seed=2000 + c["case"])
    x = workloads.make_inputs(w, device="cuda", gate=None if c["gate"] == "none" else c["gate"])
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    s0 = x["initial_state"]
    if s0 is not None and c["bf16_state"]:
        s0 = s0.to(torch.bfloat16)
    kw = dict(nseg=1, variant=c["variant"], gate_logits=logits, beta_logits=logits, gate_lower_bound=c["lb"])
    if c["norm"]:
        gen = torch.Generator(device="cuda").manual_seed(3000 + c["case"])
        kw.update(out_gate=torch.randn(x["v"].shape, generator=gen, device="cuda").to(x["v"].dtype),
                  norm_weight=1.0 + 0.1 * torch.randn(c["D"], generator=gen, device="cuda"), norm_eps=1e-6)
    print("[case]", c, "longest first", file=sys.stderr, flush=True)
    res = []
    for order in ("natural", "longest"):
        monkeypatch.setenv("KDA_ORDER", order)
        fin = torch.empty((len(c["lengths"]), c["H"], c["D"], c["D"]), device="cuda",
                          dtype=torch.bfloat16 if c["bf16_state"] else torch.float32)
        o, _ = kda.prefill(x["q"], x["k"], x["v"], g_in, b_in, s0, x["cu_seqlens"], final_state=fin, **kw)
        res.append((o, fin))
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(bits(res[0][0]), bits(res[1][0])) and torch.equal(bits(res[0][1]), bits(res[1][1]))
