"""GPU parity of the HIP KDA prefill (called through the C ABI) against the
float64 oracle, plus the bit-stability properties the pages ask for.

Tolerances (whole-tensor relative L2, outputs and final states separately):
5e-3 with bf16 q/k/v, 1e-4 in the fp32 debug mode.  Small cases compare every
element with the oracle; the full-size workloads compare every element of a
seeded sample of (sequence, head) chains that the oracle runs one by one, in
the same launch configuration the bench times.
"""
import sys

import numpy as np
import pytest

import normcheck
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 5e-3, "f32": 1e-4}


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as k
    k.load_library()
    return k


def gen(w, gate=None):
    return workloads.make_inputs(w, device="cuda", gate=gate)


def run(kda, x, **kw):
    return kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"], **kw)


def chain_slice(x, n, h):
    """Host float64-ready copies of chain (n, h)'s inputs, packed [L, 1, D]."""
    if x["cu_seqlens"] is None:
        sel = lambda t: t[n, :, h:h + 1]
        bsel = lambda t: t[n, :, h:h + 1]
    else:
        cu = x["cu_seqlens"].cpu()
        a, b = int(cu[n]), int(cu[n + 1])
        sel = lambda t: t[a:b, h:h + 1]
        bsel = sel
    s0 = None if x["initial_state"] is None else x["initial_state"][n:n + 1, h:h + 1].cpu()
    return (sel(x["q"]).cpu(), sel(x["k"]).cpu(), sel(x["v"]).cpu(), sel(x["g"]).cpu(), bsel(x["beta"]).cpu(), s0)


def out_slice(x, out, n, h):
    if x["cu_seqlens"] is None:
        return out[n, :, h:h + 1]
    cu = x["cu_seqlens"].cpu()
    return out[int(cu[n]):int(cu[n + 1]), h:h + 1]


def check_chains(x, out, sT, chains, tol):
    worst = 0.0
    for n, h in chains:
        q, k, v, g, b, s0 = chain_slice(x, n, h)
        L = q.shape[0]
        o_ref, s_ref = oracle.run_c(q, k, v, g, b, s0, np.array([0, L]))
        o_gpu = out_slice(x, out, n, h).float().cpu().numpy().reshape(o_ref.shape)
        s_gpu = sT[n:n + 1, h:h + 1].cpu().numpy()
        assert np.isfinite(o_gpu).all() and np.isfinite(s_gpu).all(), (n, h)
        eo = oracle.rel_l2(o_gpu, o_ref) if L else 0.0
        es = oracle.rel_l2(s_gpu, s_ref)
        worst = max(worst, eo, es)
        assert eo <= tol and es <= tol, f"chain {(n, h)}: rel-L2 out {eo:.3e} state {es:.3e}"
    return worst


def check_full(x, out, sT, tol):
    o_ref, s_ref = oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                                None if x["initial_state"] is None else x["initial_state"].cpu(),
                                None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu())
    o_gpu = out.float().cpu().numpy().reshape(o_ref.shape)
    s_gpu = sT.cpu().numpy()
    assert np.isfinite(o_gpu).all() and np.isfinite(s_gpu).all()
    eo, es = oracle.rel_l2(o_gpu, o_ref), oracle.rel_l2(s_gpu, s_ref)
    assert eo <= tol and es <= tol, f"rel-L2 out {eo:.3e} state {es:.3e}"
    return eo, es


# ------------------------------------------------------------ parity ----

def test_tiny_fp32_debug_mode(kda):
    w = workloads.WORKLOADS["tiny"]
    say("tiny fp32", w.describe())
    x = gen(w)
    out, sT = run(kda, x)
    eo, es = check_full(x, out, sT, TOL["f32"])
    say(f"tiny rel-L2 out {eo:.2e} state {es:.2e}")


EDGE = [
    ([17, 0, 16], 2, 128), ([1025, 0, 31], 2, 128), ([1024], 4, 128), ([1], 2, 128), ([64], 2, 128),
    ([63, 65, 128, 1, 0], 3, 128), ([300, 5], 2, 64), ([0], 2, 128), ([0, 0], 1, 64),
]


@pytest.mark.parametrize("lengths,H,D", EDGE)
def test_edge_shapes_bf16(kda, lengths, H, D):
    w = workloads.custom(lengths, H=H, D=D, dtype="bf16", dense=False, seed=3)
    say("edge", lengths, H, D)
    x = gen(w)
    out, sT = run(kda, x)
    check_full(x, out, sT, TOL["bf16"])
    if D == 128:     # the single-role 64-token kernel on the same inputs
        out1, sT1 = run(kda, x, variant=1)
        check_full(x, out1, sT1, TOL["bf16"])


@pytest.mark.parametrize("lengths,H", [([130, 7], 2), ([64, 1, 200], 1)])
def test_edge_shapes_fp32(kda, lengths, H):
    w = workloads.custom(lengths, H=H, D=64, dtype="f32", dense=False, seed=4)
    say("edge fp32", lengths, H)
    x = gen(w)
    out, sT = run(kda, x)
    check_full(x, out, sT, TOL["f32"])


def test_zero_length_keeps_initial_state_bits(kda):
    w = workloads.custom([0, 40, 0], H=2, D=128, seed=5)
    x = gen(w)
    out, sT = run(kda, x)
    s0 = x["initial_state"]
    assert torch_equal(sT[0], s0[0]) and torch_equal(sT[2], s0[2])


@pytest.mark.parametrize("gate", ["floor", "zero"])
def test_gate_extremes(kda, gate):
    """Every g at the -5 floor (a chunk-wide exp(-Gamma) would overflow) and g = 0."""
    w = workloads.custom([200, 64, 33], H=2, D=128, seed=6)
    say("gate", gate)
    x = gen(w, gate=gate)
    out, sT = run(kda, x)
    check_full(x, out, sT, TOL["bf16"])


def _sample(w, count, seed=0):
    """The first and last chains, on a dense layout the chains on either side of the 2^31-byte
    offset of g (the first whose g rows start at or past it, the last wholly below it: where a
    32-bit byte offset would wrap) and the one of the highest offset, then seeded random ones."""
    rng = np.random.default_rng(seed)
    chains = {(w.n_seq - 1, w.H - 1), (0, 0)}
    if w.dense:
        T, H, D = w.lengths[0], w.H, w.D
        lo = lambda n, h: ((n * T) * H + h) * D * 4
        live = [(n, h) for n in range(w.n_seq) for h in range(H)]
        above = [c for c in live if lo(*c) >= 1 << 31]
        if above:
            chains.add(min(above, key=lambda c: lo(*c)))
            chains.add(max((c for c in live if lo(*c) < 1 << 31), key=lambda c: lo(*c)))
    while len(chains) < min(count, w.n_seq * w.H):
        chains.add((int(rng.integers(w.n_seq)), int(rng.integers(w.H))))
    return sorted(chains)


@pytest.mark.parametrize("name,count", [("eqlen", 8), ("varlen", 12), ("varlen_padded", 6), ("long", 8),
                                        ("large", 16), ("eqlen288", 8)])
def test_workload_sampled_chains(kda, name, count):
    import torch
    w = workloads.WORKLOADS[name]
    say("workload", w.describe())
    x = gen(w)
    out, sT = run(kda, x)
    torch.cuda.synchronize()
    worst = check_chains(x, out, sT, _sample(w, count), TOL[w.dtype])
    say(f"{name}: worst sampled rel-L2 {worst:.2e}")
    del x, out, sT
    torch.cuda.empty_cache()


# -------------------------------------------------- bit-stability ----

def torch_equal(a, b):
    import torch
    return bool(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                            b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)))


def test_repeat_runs_bitwise(kda):
    w = workloads.custom([1000, 64, 300], H=4, D=128, seed=7)
    x = gen(w)
    o0, s0 = run(kda, x)
    for _ in range(9):
        o1, s1 = run(kda, x)
        assert torch_equal(o0, o1) and torch_equal(s0, s1)


STALLS = [(2, w) for w in range(8)] + [(1, w) for w in range(4)]


@pytest.mark.parametrize("layout", ["padded_eqlen", "varlen"])
@pytest.mark.parametrize("variant,wave", STALLS)
def test_stalled_wave_gives_same_bits(kda, layout, variant, wave):
    """A copy of the kernel with one wave stalled ~20 us after every barrier must
    reproduce the unstalled bits (the warp-timing test of TensorRT-LLM PR #19826).
    Variant 2 (pipelined) has 8 waves: 4 consumers, 4 producers; variant 1 has 4."""
    if layout == "padded_eqlen":
        w = workloads.custom([200] * 3, H=2, D=128, dense=True, seed=8)
    else:
        w = workloads.custom([130, 1, 77, 64], H=2, D=128, seed=8)
    x = gen(w)
    say("stall", layout, "variant", variant, "wave", wave)
    o0, s0 = run(kda, x, nseg=1, variant=variant)
    o1, s1 = run(kda, x, nseg=1, variant=variant, stall_wave=wave, stall_cycles=127 * 6)
    assert torch_equal(o0, o1) and torch_equal(s0, s1)
    o2, s2 = run(kda, x, nseg=3, variant=variant)
    o3, s3 = run(kda, x, nseg=3, variant=variant, stall_wave=wave, stall_cycles=127 * 6)
    assert torch_equal(o2, o3) and torch_equal(s2, s3)


def test_poisoned_outputs_and_workspace(kda):
    import torch
    w = workloads.custom([333, 64, 5], H=3, D=128, seed=9)
    x = gen(w)
    o0, s0 = run(kda, x, nseg=2)
    out = torch.full_like(o0, float("nan"))
    fin = torch.full_like(s0, float("nan"))
    ws_bytes = kda.workspace_size(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"],
                                  nseg=2)
    ws = torch.full((ws_bytes // 4 + 64,), float("nan"), device="cuda")
    o1, s1 = run(kda, x, out=out, final_state=fin, nseg=2, workspace=ws.view(torch.uint8))
    assert torch_equal(o0, o1) and torch_equal(s0, s1)


def test_row_padded_views_same_bits(kda):
    """Q backed by [T, H, 256] viewed [..., :128] and the initial state with row
    stride 256 (the strided probe of the cudnn-frontend PR review)."""
    import torch
    w = workloads.custom([17, 0, 16], H=2, D=128, seed=10)
    x = gen(w)
    o0, s0 = run(kda, x)
    qb = torch.zeros(x["q"].shape[0], 2, 256, dtype=x["q"].dtype, device="cuda")
    qb[..., :128] = x["q"]
    sb = torch.zeros(3, 2, 128, 256, device="cuda")
    sb[..., :128] = x["initial_state"]
    y = dict(x, q=qb[..., :128], initial_state=sb[..., :128])
    o1, s1 = run(kda, y)
    assert torch_equal(o0, o1) and torch_equal(s0, s1)


def test_dense_equals_packed(kda):
    w = workloads.custom([200] * 3, H=2, D=128, dense=True, seed=11)
    x = gen(w)
    o0, s0 = run(kda, x)
    y = {kk: (workloads.to_packed(t) if kk in ("q", "k", "v", "g", "beta") else t) for kk, t in x.items()}
    import torch
    y["cu_seqlens"] = torch.tensor([0, 200, 400, 600], dtype=torch.int32, device="cuda")
    o1, s1 = run(kda, y)
    assert torch_equal(workloads.to_packed(o0), o1) and torch_equal(s0, s1)


@pytest.mark.parametrize("variant", [1, 2])
@pytest.mark.parametrize("nseg", [1, 2, 4, 8, 64])
def test_forced_segments_match_oracle(kda, nseg, variant):
    """Forced segment counts up to the maximum (64): chains shorter than nseg chunks get
    empty segments, whose maps are the identity (M = I, C = 0)."""
    w = workloads.custom([700, 64, 1, 300], H=2, D=128, seed=12)
    x = gen(w)
    say("nseg", nseg, "variant", variant)
    out, sT = run(kda, x, nseg=nseg, variant=variant)
    check_full(x, out, sT, TOL["bf16"])


@pytest.mark.parametrize("nseg", [1, 4])
@pytest.mark.parametrize("variant", [1, 2])
def test_standalone_prep_equals_fused_scan(kda, variant, nseg):
    w = workloads.custom([700, 64, 1, 300], H=2, D=128, seed=13)
    x = gen(w)
    say("nseg", nseg, "variant", variant)
    o1, s1 = run(kda, x, nseg=nseg, prep=1, variant=variant)
    o2, s2 = run(kda, x, nseg=nseg, prep=2, variant=variant)
    assert torch_equal(o1, o2) and torch_equal(s1, s2)


@pytest.mark.parametrize("gate", [None, "mild", "zero"])
@pytest.mark.parametrize("nseg", [3, 8])
def test_forced_segments_fp32_d64(kda, nseg, gate):
    """The fp32 debug mode (d = 64) through the segment maps and the d = 64 COMBINE."""
    w = workloads.custom([700, 64, 1, 300], H=2, D=64, dtype="f32", dense=False, seed=15)
    x = gen(w, gate=gate)
    say("nseg", nseg, "fp32 d=64 gate", gate)
    out, sT = run(kda, x, nseg=nseg)
    check_full(x, out, sT, TOL["f32"])


@pytest.mark.parametrize("variant", [1, 2])
@pytest.mark.parametrize("gate", ["mild", "zero"])
@pytest.mark.parametrize("nseg", [2, 5, 16])
def test_forced_segments_slow_decay(kda, nseg, gate, variant):
    """Segment maps M that are far from zero: with the drawn gates a state decays to
    nothing within a segment (M underflows to 0), so slow and absent decay are what
    exercise the M S_start term of COMBINE."""
    w = workloads.custom([1500, 64, 1, 700], H=2, D=128, seed=16)
    x = gen(w, gate=gate)
    say("nseg", nseg, "gate", gate, "variant", variant)
    out, sT = run(kda, x, nseg=nseg, variant=variant)
    check_full(x, out, sT, TOL["bf16"])


def test_in_place_state(kda):
    import torch
    w = workloads.custom([150, 20], H=2, D=128, seed=14)
    x = gen(w)
    o0, s0 = run(kda, x)
    st = x["initial_state"].clone()
    y = dict(x, initial_state=st)
    o1, s1 = run(kda, y, final_state=st)
    assert s1.data_ptr() == st.data_ptr()
    assert torch_equal(o0, o1) and torch_equal(s0, st)


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("dense", [True, False])
def test_prep_kernel_bit_exact(kda, dense, chunk):
    """PREP output equals a float32 sequential cumsum restarted every `chunk`
    tokens of every sequence."""
    import torch
    if dense:
        w = workloads.custom([130] * 2, H=3, D=128, dense=True, seed=15)
    else:
        w = workloads.custom([130, 0, 64, 1, 65], H=3, D=128, seed=15)
    x = gen(w)
    gam = kda.prep(x["g"], x["cu_seqlens"], chunk=chunk)
    g = x["g"].cpu().numpy()
    got = gam.cpu().numpy()
    if dense:
        g = g.reshape(-1, *g.shape[2:])
        got = got.reshape(-1, *got.shape[2:])
        cu = np.arange(3) * 130
    else:
        cu = x["cu_seqlens"].cpu().numpy()
    want = np.zeros_like(g)
    for n in range(len(cu) - 1):
        for c0 in range(cu[n], cu[n + 1], chunk):
            acc = np.zeros(g.shape[1:], dtype=np.float32)
            for t in range(c0, min(c0 + chunk, cu[n + 1])):
                acc = (acc + g[t]).astype(np.float32)
                want[t] = acc
    assert np.array_equal(want.view(np.int32), got.view(np.int32))


def test_graph_replay_with_changed_q(kda):
    """kda_prefill_ws captured in a HIP graph; q changes between replays and
    each replay must equal a fresh eager call bit for bit."""
    import torch
    w = workloads.custom([300, 77], H=2, D=128, seed=16)
    x = gen(w)
    ws_bytes = kda.workspace_size(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"],
                                  nseg=2)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device="cuda")
    qbuf = x["q"].clone()
    out = torch.empty_like(x["v"])
    fin = torch.empty_like(x["initial_state"])
    y = dict(x, q=qbuf)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(kda, y, out=out, final_state=fin, nseg=2, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(kda, y, out=out, final_state=fin, nseg=2, workspace=ws)
    gen_ = torch.Generator(device="cuda")
    for rep in range(4):
        gen_.manual_seed(100 + rep)
        newq = torch.randn(qbuf.shape, generator=gen_, device="cuda")
        newq = (newq / newq.norm(dim=-1, keepdim=True)).to(qbuf.dtype)
        qbuf.copy_(newq)
        graph.replay()
        torch.cuda.synchronize()
        o_ref, s_ref = run(kda, dict(x, q=newq.clone()), nseg=2)
        torch.cuda.synchronize()
        assert torch_equal(out, o_ref) and torch_equal(fin, s_ref), f"replay {rep}"


# ------------------------------------------------ activations fused into the gate scan
def _oracle_with_activations(x, lower_bound=-5.0):
    g64, b64 = oracle.activations(x["g_logits"].cpu(), x["beta_logits"].cpu(), lower_bound)
    return oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), g64, b64,
                        None if x["initial_state"] is None else x["initial_state"].cpu(),
                        None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu())


@pytest.mark.parametrize("nseg", [1, 4])
@pytest.mark.parametrize("variant", [1, 2])
def test_logit_inputs_match_oracle(kda, variant, nseg):
    """g and beta given as logits (g = -5 sigmoid(x), beta = sigmoid(b)), the
    activations fused into the gate scan, against the float64 oracle applied to
    the float64 activations of the same logits."""
    w = workloads.custom([700, 0, 64, 1, 300], H=2, D=128, seed=21)
    x = gen(w)
    say("nseg", nseg, "variant", variant, "logits")
    out, sT = kda.prefill(x["q"], x["k"], x["v"], x["g_logits"], x["beta_logits"], x["initial_state"],
                          x["cu_seqlens"], nseg=nseg, variant=variant, gate_logits=True, beta_logits=True)
    o_ref, s_ref = _oracle_with_activations(x)
    eo = oracle.rel_l2(out.float().cpu().numpy().reshape(o_ref.shape), o_ref)
    es = oracle.rel_l2(sT.cpu().numpy(), s_ref)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], f"rel-L2 out {eo:.3e} state {es:.3e}"


def test_logit_inputs_fp32_d64(kda):
    w = workloads.custom([130, 7, 0, 64], H=2, D=64, dtype="f32", dense=False, seed=22)
    x = gen(w)
    out, sT = kda.prefill(x["q"], x["k"], x["v"], x["g_logits"], x["beta_logits"], x["initial_state"],
                          x["cu_seqlens"], gate_logits=True, beta_logits=True)
    o_ref, s_ref = _oracle_with_activations(x)
    eo = oracle.rel_l2(out.cpu().numpy().reshape(o_ref.shape), o_ref)
    es = oracle.rel_l2(sT.cpu().numpy(), s_ref)
    assert eo <= TOL["f32"] and es <= TOL["f32"], f"rel-L2 out {eo:.3e} state {es:.3e}"


@pytest.mark.parametrize("variant", [1, 2])
def test_fused_activations_match_unfused(kda, variant):
    """Fused activations against the same kernel fed values activated by torch on
    the device beforehand (the fused-vs-unfused check of the TensorRT-LLM KDA
    prefill fix PR #19826).  Only the rounding of the two sigmoids differs."""
    import torch
    w = workloads.custom([300, 64, 45], H=2, D=128, seed=23)
    x = gen(w)
    o1, s1 = kda.prefill(x["q"], x["k"], x["v"], x["g_logits"], x["beta_logits"], x["initial_state"],
                         x["cu_seqlens"], variant=variant, gate_logits=True, beta_logits=True)
    g = -5.0 * torch.sigmoid(x["g_logits"])
    b = torch.sigmoid(x["beta_logits"])
    o2, s2 = kda.prefill(x["q"], x["k"], x["v"], g, b, x["initial_state"], x["cu_seqlens"], variant=variant)
    do = ((o1.float() - o2.float()).norm() / o2.float().norm()).item()
    ds = ((s1 - s2).norm() / s2.norm()).item()
    assert do <= 1e-3 and ds <= 1e-3, f"fused vs unfused: out {do:.2e} state {ds:.2e}"


@pytest.mark.parametrize("variant", [1, 2])
def test_standalone_prep_with_gate_logits_equals_fused(kda, variant):
    """The standalone PREP kernel applies the same gate activation as the fused
    scans: the two plans give the same bits."""
    w = workloads.custom([400, 33], H=2, D=128, seed=24)
    x = gen(w)
    kw = dict(variant=variant, gate_logits=True, gate_lower_bound=-3.0, beta_logits=True)
    o1, s1 = kda.prefill(x["q"], x["k"], x["v"], x["g_logits"], x["beta_logits"], x["initial_state"],
                         x["cu_seqlens"], prep=1, **kw)
    o2, s2 = kda.prefill(x["q"], x["k"], x["v"], x["g_logits"], x["beta_logits"], x["initial_state"],
                         x["cu_seqlens"], prep=2, **kw)
    assert torch_equal(o1, o2) and torch_equal(s1, s2)


# ------------------------------------------------ bf16 state I/O (fp32 arithmetic inside)
@pytest.mark.parametrize("nseg", [1, 4])
@pytest.mark.parametrize("variant", [1, 2])
def test_bf16_states_match_oracle(kda, variant, nseg):
    """bf16 initial and final states: the oracle starts from the bf16 values (widened
    exactly) and the final state is compared after its one rounding to bf16.  A
    zero-length sequence keeps its bf16 state bit for bit."""
    import torch
    w = workloads.custom([700, 0, 64, 1, 300], H=2, D=128, seed=31)
    x = gen(w)
    s0 = x["initial_state"].to(torch.bfloat16)
    fin = torch.empty_like(s0)
    say("bf16 states nseg", nseg, "variant", variant)
    out, _ = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, x["cu_seqlens"], final_state=fin,
                         nseg=nseg, variant=variant)
    o_ref, s_ref = oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                                s0.float().cpu(), x["cu_seqlens"].cpu())
    eo = oracle.rel_l2(out.float().cpu().numpy().reshape(o_ref.shape), o_ref)
    es = oracle.rel_l2(fin.float().cpu().numpy(), s_ref)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], f"rel-L2 out {eo:.3e} state {es:.3e}"
    assert torch.equal(fin[1].view(torch.int16), s0[1].view(torch.int16))


def test_bf16_state_in_place_and_mixed(kda):
    """In-place bf16 state update gives the bits of a separate final state; a bf16
    final state is the fp32 final state rounded once (same arithmetic, one store)."""
    import torch
    w = workloads.custom([300, 45], H=2, D=128, seed=32)
    x = gen(w)
    s0 = x["initial_state"].to(torch.bfloat16)
    fin = torch.empty_like(s0)
    o1, _ = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, x["cu_seqlens"], final_state=fin)
    f32 = torch.empty(s0.shape, dtype=torch.float32, device="cuda")
    o2, _ = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, x["cu_seqlens"], final_state=f32)
    st = s0.clone()
    o3, _ = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], st, x["cu_seqlens"], final_state=st)
    torch.cuda.synchronize()
    assert torch_equal(o1, o2) and torch_equal(o1, o3)
    assert torch.equal(fin.view(torch.int16), st.view(torch.int16))
    assert torch.equal(fin.view(torch.int16), f32.to(torch.bfloat16).view(torch.int16))


def test_bf16_states_fp32_d64(kda):
    import torch
    w = workloads.custom([130, 7, 0, 64], H=2, D=64, dtype="f32", dense=False, seed=33)
    x = gen(w)
    s0 = x["initial_state"].to(torch.bfloat16)
    fin = torch.empty_like(s0)
    out, _ = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, x["cu_seqlens"], final_state=fin, nseg=3)
    o_ref, s_ref = oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                                s0.float().cpu(), x["cu_seqlens"].cpu())
    eo = oracle.rel_l2(out.cpu().numpy().reshape(o_ref.shape), o_ref)
    es = oracle.rel_l2(fin.float().cpu().numpy(), s_ref)
    assert eo <= TOL["f32"] and es <= TOL["bf16"], f"rel-L2 out {eo:.3e} state {es:.3e}"


# ------------------------------------------------ gated RMS norm output epilogue
# How the normalised output y is checked (three checks, each able to fail on its own):
# the same call without the epilogue gives o within 5e-3 of the oracle; y is within 5e-3
# of the float64 norm of that o (the epilogue's own arithmetic); and y against the
# oracle's y, each row weighted by its oracle RMS of o (normcheck.weighted_rel_l2: a
# plain relative L2 of y would weight rows of tiny |o| as much as the rest, and those
# carry relative errors far above o's), within o's budget plus one bf16 rounding of y.


def check_norm(y, o, y_ref, o_ref, z, nw):
    """The two-part check of a normalised output (torch y, o on the GPU; float64 refs)."""
    og = o.float().cpu().numpy().reshape(o_ref.shape)
    yg = y.float().cpu().numpy().reshape(y_ref.shape)
    y_own = oracle.gated_rmsnorm(og, z.float().cpu().numpy().reshape(o_ref.shape), nw.cpu().numpy(), 1e-6)
    e_o, e_epi = oracle.rel_l2(og, o_ref), oracle.rel_l2(yg, y_own)
    e_w = normcheck.weighted_rel_l2(yg, y_ref, o_ref)
    say(f"norm check: o {e_o:.3e}, epilogue {e_epi:.3e}, y weighted {e_w:.3e}")
    assert e_o <= TOL["bf16"], f"o (no epilogue) against the oracle {e_o:.3e}"
    assert e_epi <= TOL["bf16"], f"epilogue against the norm of the kernel's own o {e_epi:.3e}"
    assert e_w <= normcheck.TOL_Y_WEIGHTED, f"y against the oracle, rows weighted by |o|: {e_w:.3e}"


def _norm_inputs(x, seed):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    z = torch.randn(x["v"].shape, generator=gen, device="cuda").to(x["v"].dtype)
    w = 1.0 + 0.1 * torch.randn(x["v"].shape[-1], generator=gen, device="cuda")
    return z, w


@pytest.mark.parametrize("layout", ["varlen", "padded_eqlen"])
@pytest.mark.parametrize("nseg", [1, 4])
def test_output_norm_matches_oracle(kda, nseg, layout):
    """out = o * rsqrt(mean(o^2) + eps) * w * sigmoid(z) per (token, head), fused into
    the pipelined kernel's output store, against the float64 oracle's o passed
    through the float64 gated RMS norm."""
    if layout == "varlen":
        w = workloads.custom([700, 0, 64, 1, 300], H=2, D=128, seed=41)
    else:
        w = workloads.custom([200] * 3, H=2, D=128, dense=True, seed=41)
    x = gen(w)
    z, nw = _norm_inputs(x, 41)
    say("output norm", layout, "nseg", nseg)
    out, sT = run(kda, x, nseg=nseg, out_gate=z, norm_weight=nw, norm_eps=1e-6)
    o_ref, s_ref = oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                                x["initial_state"].cpu(), None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu())
    y_ref = oracle.gated_rmsnorm(o_ref, z.float().cpu().numpy().reshape(o_ref.shape), nw.cpu().numpy(), 1e-6)
    es = oracle.rel_l2(sT.cpu().numpy(), s_ref)
    assert es <= TOL["bf16"], f"state {es:.3e}"
    o, _ = run(kda, x, nseg=nseg)
    check_norm(out, o, y_ref, o_ref, z, nw)


def test_output_norm_fused_matches_unfused(kda):
    """The fused epilogue against torch's gated RMS norm (float32) of the kernel's
    own bf16 output: they differ by the rounding of o to bf16 before the norm."""
    import torch
    w = workloads.custom([300, 64, 45], H=2, D=128, seed=42)
    x = gen(w)
    z, nw = _norm_inputs(x, 42)
    y1, _ = run(kda, x, out_gate=z, norm_weight=nw, norm_eps=1e-6)
    o, _ = run(kda, x)
    of = o.float()
    y2 = of * torch.rsqrt(of.pow(2).mean(-1, keepdim=True) + 1e-6) * nw * torch.sigmoid(z.float())
    d = ((y1.float() - y2).norm() / y2.norm()).item()
    assert d <= TOL["bf16"], f"fused vs unfused {d:.2e}"


@pytest.mark.parametrize("wave", list(range(8)))
def test_output_norm_stalled_wave_gives_same_bits(kda, wave):
    """The epilogue's per-token sums cross the 4 consumer waves through LDS: a wave
    stalled after every barrier must not change a bit."""
    w = workloads.custom([130, 1, 77, 64], H=2, D=128, seed=43)
    x = gen(w)
    z, nw = _norm_inputs(x, 43)
    say("output norm stall wave", wave)
    o0, s0 = run(kda, x, nseg=1, out_gate=z, norm_weight=nw)
    o1, s1 = run(kda, x, nseg=1, out_gate=z, norm_weight=nw, stall_wave=wave, stall_cycles=127 * 6)
    assert torch_equal(o0, o1) and torch_equal(s0, s1)


# ------------------------------------------------ KDA_CHECK (device check of cu_seqlens)
def test_check_rejects_bad_cu_seqlens(kda, monkeypatch):
    """With KDA_CHECK=1 an offset array that runs past the tokens, or goes backwards, is
    refused before any prefill kernel runs (outputs untouched); a valid one gives the
    bits of an unchecked call.  The bad arrays only ever reach the device check."""
    import torch
    w = workloads.custom([100, 50, 30], H=2, D=128, seed=60)
    x = gen(w)
    o_ref, s_ref = run(kda, x)
    monkeypatch.setenv("KDA_CHECK", "1")
    o_chk, s_chk = run(kda, x)
    assert torch_equal(o_ref, o_chk) and torch_equal(s_ref, s_chk)
    for kind in ("past_end", "backwards", "nonzero_start"):
        bad = x["cu_seqlens"].clone()
        if kind == "past_end":
            bad[-1] += 7
        elif kind == "backwards":
            bad[1], bad[2] = bad[2].clone(), bad[1].clone()
        else:
            bad[0] = 1
        out = torch.full_like(x["v"], -512.0)
        say("KDA_CHECK", kind)
        with pytest.raises(kda.KdaError) as e:
            kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], bad, out=out)
        assert e.value.status == 2 and "cu_seqlens" in str(e.value)
        assert torch.all(out.float() == -512.0)
        with pytest.raises(kda.KdaError):
            kda.prep(x["g"], bad, chunk=32)


def test_cached_workspace_per_stream(kda):
    """Plain kda_prefill calls on two streams at once, both on the segmented path (so
    both need the library's cached workspace), give the bits of the same calls made
    one after the other: each stream has a workspace of its own."""
    import torch
    xs = [gen(workloads.custom([600, 200], H=2, D=128, seed=70 + i)) for i in range(2)]
    refs = []
    for x in xs:
        refs.append(run(kda, x))
        torch.cuda.synchronize()
    kda.release_cached_workspace()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    res = [None, None]
    for rep in range(3):
        for i, (x, s) in enumerate(zip(xs, streams)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                res[i] = run(kda, x)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch_equal(res[i][0], refs[i][0]) and torch_equal(res[i][1], refs[i][1]), f"rep {rep} stream {i}"


def test_cached_workspace_threads(kda):
    """Two host threads calling plain kda_prefill on one stream, with workspace needs
    that grow and shrink from call to call (segment counts 2 to 18), give the bits of
    the same calls made from one thread: a call that replaces the cached buffer waits
    until the other thread's call has enqueued its kernels."""
    import threading
    import torch
    lens = [[600, 200], [1200, 100], [2400, 50], [4800, 10]]
    xs = [gen(workloads.custom(L, H=2, D=128, seed=80 + i)) for i, L in enumerate(lens)]
    refs = []
    for x in xs:
        refs.append(run(kda, x))
    torch.cuda.synchronize()
    kda.release_cached_workspace()
    results = {0: [], 1: []}
    errors = []

    def worker(tid):
        try:
            order = list(range(len(xs))) if tid == 0 else list(range(len(xs)))[::-1]
            for _ in range(4):
                for i in order:
                    results[tid].append((i, run(kda, xs[i])))
        except Exception as e:      # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "worker threads did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for tid in (0, 1):
        assert len(results[tid]) == 4 * len(xs)
        for n, (i, (o, s)) in enumerate(results[tid]):
            assert torch_equal(o, refs[i][0]) and torch_equal(s, refs[i][1]), f"thread {tid} call {n} workload {i}"


def test_longest_first_order_same_bits(kda, monkeypatch):
    """Longest-first chain order (packed, one segment) changes only which workgroup runs
    which chain: outputs and final states are the bits of the natural order.  A batch of
    mixed lengths with more chains than CUs takes it by default; smaller batches are forced
    with KDA_ORDER=longest, also with bf16 states, the output norm and a stalled wave (the
    ranking adds barriers before the main loop)."""
    import torch
    big = workloads.custom([700, 5, 0, 1300, 64, 2100], H=48, D=128, seed=90)     # 288 chains
    small = workloads.custom([130, 0, 64, 1, 300], H=2, D=128, seed=91)
    for w, forced in ((big, None), (small, "longest")):
        x = gen(w)
        z, nw = _norm_inputs(x, 92)
        for kw in (dict(nseg=1), dict(nseg=1, out_gate=z, norm_weight=nw, norm_eps=1e-6),
                   dict(nseg=1, stall_wave=3, stall_cycles=127 * 6)):
            say("longest first", w.lengths, w.H, sorted(kw))
            monkeypatch.setenv("KDA_ORDER", "natural")
            o0, s0 = run(kda, x, **kw)
            if forced:
                monkeypatch.setenv("KDA_ORDER", forced)
            else:
                monkeypatch.delenv("KDA_ORDER")
            o1, s1 = run(kda, x, **kw)
            torch.cuda.synchronize()
            assert torch_equal(o0, o1) and torch_equal(s0, s1)
    # the reordered big batch against the oracle on its longest and shortest sequences
    x = gen(big)
    monkeypatch.delenv("KDA_ORDER", raising=False)
    out, sT = run(kda, x)
    check_chains(x, out, sT, [(5, 47), (1, 0), (3, 20), (2, 5)], TOL["bf16"])


@pytest.mark.parametrize("N", [512, 600])
def test_many_short_sequences(kda, monkeypatch, N):
    """Packed batches of many short ragged sequences (one head, lengths 0 to 160, about one in
    eight empty): 512 sequences, the most the workgroups rank longest first (512 chains on
    256 CUs take that order by default), and 600, past it (natural order).  Same bits as the
    natural order, and the longest, a one-token and an empty sequence, the first and the last
    against the oracle."""
    import torch
    rng = np.random.default_rng(8000 + N)
    lengths = [int(x) if rng.random() > 0.12 else 0 for x in rng.integers(1, 161, N)]
    lengths[N // 2] = 1
    x = gen(workloads.custom(lengths, H=1, D=128, seed=8100 + N))
    say("many short sequences", N, sum(lengths))
    monkeypatch.setenv("KDA_ORDER", "natural")
    o0, s0 = run(kda, x)
    monkeypatch.delenv("KDA_ORDER")
    o1, s1 = run(kda, x)
    torch.cuda.synchronize()
    assert torch_equal(o0, o1) and torch_equal(s0, s1)
    empty = lengths.index(0)
    check_chains(x, o1, s1, [(int(np.argmax(lengths)), 0), (N // 2, 0), (empty, 0), (0, 0), (N - 1, 0)],
                 TOL["bf16"])


def test_capped_concurrency_same_bits(kda, monkeypatch):
    """The capped schedule (packed, one segment, more chains than the 160-chain cap, every
    chain resident) only delays when some workgroups start: outputs and final states are the
    bits of the uncapped launch (KDA_CAP=0).  On the varlen lengths the packing leaves the
    longest sequence as the bound, so the short sequences queue; on equal lengths it would
    lengthen the call and nothing waits.  Each also with every wait cut short by a 1 us bound
    (KDA_CAP_WAIT_US=1), a stalled wave and the output norm; then the capped varlen batch
    against the oracle on its longest, shortest and queued sequences."""
    import torch
    varl = workloads.custom(workloads.varlen_lengths(), H=32, D=128, seed=95)    # 256 chains
    eq = workloads.custom([1000] * 8, H=32, D=128, seed=96)
    for w in (varl, eq):
        x = gen(w)
        z, nw = _norm_inputs(x, 97)
        for kw, env in ((dict(nseg=1), {}), (dict(nseg=1), {"KDA_CAP_WAIT_US": "1"}),
                        (dict(nseg=1, stall_wave=3, stall_cycles=127 * 2), {}),
                        (dict(nseg=1, out_gate=z, norm_weight=nw, norm_eps=1e-6), {})):
            say("capped", w.lengths, w.H, sorted(kw), env)
            monkeypatch.setenv("KDA_CAP", "0")
            o0, s0 = run(kda, x, **kw)
            monkeypatch.delenv("KDA_CAP")
            for k, v in env.items():
                monkeypatch.setenv(k, v)
            o1, s1 = run(kda, x, **kw)
            for k in env:
                monkeypatch.delenv(k)
            torch.cuda.synchronize()
            assert torch_equal(o0, o1) and torch_equal(s0, s1)
    x = gen(varl)
    out, sT = run(kda, x)
    check_chains(x, out, sT, [(7, 0), (7, 31), (4, 5), (0, 17), (6, 31), (3, 2)], TOL["bf16"])


def test_capped_concurrency_in_graph(kda, monkeypatch):
    """Capped calls captured in HIP graphs on one workspace, which holds the chains' flags.  A
    graph of two calls (different q) is replayed three times, with eager work and
    synchronisations between the replays, and a graph of one call likewise (its chains find
    the captured call's value in their own flags and count replays): every replay gives the
    bits of eager uncapped calls."""
    import torch
    w = workloads.custom(workloads.varlen_lengths(), H=32, D=128, seed=98)    # 256 chains
    x = gen(w)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(99)
    q2 = torch.randn(x["q"].shape, generator=gq, device="cuda")
    x2 = dict(x, q=(q2 / q2.norm(dim=-1, keepdim=True)).to(x["q"].dtype))
    monkeypatch.setenv("KDA_CAP", "0")
    refs = [run(kda, x), run(kda, x2)]
    monkeypatch.delenv("KDA_CAP")
    torch.cuda.synchronize()
    ws_bytes = kda.workspace_size(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device="cuda")
    outs = [(torch.empty_like(x["v"]), torch.empty_like(x["initial_state"])) for _ in range(2)]
    for ncalls in (2, 1):
        say("capped graph of", ncalls, "calls")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in range(ncalls):
                run(kda, (x, x2)[c], out=outs[c][0], final_state=outs[c][1], workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in range(ncalls):
                run(kda, (x, x2)[c], out=outs[c][0], final_state=outs[c][1], workspace=ws)
        for rep in range(3):
            for o, f in outs:
                o.fill_(float("nan"))
                f.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            for c in range(ncalls):
                assert torch_equal(outs[c][0], refs[c][0]) and torch_equal(outs[c][1], refs[c][1]), (ncalls, rep, c)
            run(kda, x2)              # eager work between the replays
            torch.cuda.synchronize()
        del graph


def _capped_case(i):
    rng = np.random.default_rng(7000 + i)
    H = int(rng.choice([16, 32, 64]))
    N = int(rng.integers(161 // H + 1, 256 // H + 1))
    lengths = [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, 2500, N)]
    return lengths, H


@pytest.mark.parametrize("i", range(8))
def test_capped_concurrency_random_batches(kda, monkeypatch, i):
    """Seeded packed batches of 161 to 256 chains (mixed lengths, some empty sequences, 16 to
    64 heads: 10, 5 or 2 groups): the capped schedule gives the uncapped bits, and sampled
    chains match the oracle."""
    import torch
    lengths, H = _capped_case(i)
    say("capped random", i, lengths, H)
    x = gen(workloads.custom(lengths, H=H, D=128, seed=7100 + i))
    monkeypatch.setenv("KDA_CAP", "0")
    o0, s0 = run(kda, x)
    monkeypatch.delenv("KDA_CAP")
    o1, s1 = run(kda, x)
    torch.cuda.synchronize()
    assert torch_equal(o0, o1) and torch_equal(s0, s1)
    N = len(lengths)
    longest = int(np.argmax(lengths))
    shortest = int(np.argmin([L if L > 0 else 10 ** 9 for L in lengths]))
    check_chains(x, o1, s1, [(longest, 0), (shortest, H - 1), (N - 1, H // 2)], TOL["bf16"])


@pytest.mark.parametrize("as_handle", [False, True])
def test_explicit_stream_argument(kda, as_handle):
    """prefill(stream=...) on a stream other than torch's current one, given as a
    torch.cuda.Stream or as a raw handle, on a segmented plan (the binding allocates the
    workspace): the outputs and workspace are allocated on that stream, so memory that
    the current stream allocates and fills meanwhile never lands in them; results are
    the bits of the same call on the current stream."""
    import torch
    w = workloads.custom([600, 200], H=2, D=128, seed=75)
    x = gen(w)
    o_ref, s_ref = run(kda, x, nseg=3)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for rep in range(3):
        s.wait_stream(torch.cuda.current_stream())
        o, st = run(kda, x, nseg=3, stream=s.cuda_stream if as_handle else s)
        # the current stream allocates and poisons memory while the call may still run on s
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(8)]
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        del junk
        assert torch_equal(o, o_ref) and torch_equal(st, s_ref), f"rep {rep}"


def test_check_rejects_gates_out_of_range(kda, monkeypatch):
    """With KDA_CHECK=1 a g holding one value below the -5 floor (or above 0, or NaN) is
    refused with KDA_ERR_RANGE before any prefill kernel runs (outputs untouched); with
    logit inputs only NaN is refused.  In-range inputs give the bits of an unchecked call,
    on the dense and the packed layout, including a padded g view."""
    import torch
    for dense in (False, True):
        w = workloads.custom([100, 100, 100] if dense else [100, 50, 30], H=2, D=128, dense=dense, seed=61)
        x = gen(w)
        o_ref, s_ref = run(kda, x)
        monkeypatch.setenv("KDA_CHECK", "1")
        o_chk, s_chk = run(kda, x)
        assert torch_equal(o_ref, o_chk) and torch_equal(s_ref, s_chk)
        gpad = torch.full(x["g"].shape[:-1] + (160,), float("nan"), device="cuda")[..., :128]
        gpad.copy_(x["g"])
        o_pad, _ = run(kda, dict(x, g=gpad))
        assert torch_equal(o_ref, o_pad)          # the padding (NaN) is not part of the view
        for bad_value in (-5.5, 1e-3, float("nan")):
            g = x["g"].clone()
            g.view(-1)[g.numel() // 2 + 5] = bad_value
            out = torch.full_like(x["v"], -512.0)
            say("KDA_CHECK g", bad_value, "dense", dense)
            with pytest.raises(kda.KdaError) as e:
                kda.prefill(x["q"], x["k"], x["v"], g, x["beta"], x["initial_state"], x["cu_seqlens"], out=out)
            assert e.value.status == 9 and "g holds" in str(e.value)
            assert torch.all(out.float() == -512.0)
        # logits: any finite or infinite value is a valid input; NaN is not
        gl = x["g_logits"].clone()
        gl.view(-1)[7] = 1e6
        kda.prefill(x["q"], x["k"], x["v"], gl, x["beta_logits"], x["initial_state"], x["cu_seqlens"],
                    gate_logits=True, beta_logits=True)
        gl.view(-1)[7] = float("nan")
        with pytest.raises(kda.KdaError) as e:
            kda.prefill(x["q"], x["k"], x["v"], gl, x["beta_logits"], x["initial_state"], x["cu_seqlens"],
                        gate_logits=True, beta_logits=True)
        assert e.value.status == 9
        monkeypatch.delenv("KDA_CHECK")


@pytest.mark.parametrize("dense", [True, False])
@pytest.mark.parametrize("nseg,split", [(3, 2), (8, 1), (4, 5)])
def test_split_plan_matches_oracle_and_whole_chains_keep_their_bits(kda, dense, nseg, split):
    """A split plan cuts only the last `split` chains into segments; their segment outputs and
    the other chains, run whole, share one launch.  Everything matches the oracle, and the
    chains run whole give exactly the bits of the one-segment plan."""
    import torch
    if dense:
        w = workloads.custom([300] * 3, H=2, D=128, dense=True, seed=80)
    else:
        w = workloads.custom([700, 64, 1, 300], H=2, D=128, seed=80)
    x = gen(w)
    say("split plan", "dense" if dense else "packed", "nseg", nseg, "split", split)
    out, sT = run(kda, x, nseg=nseg, split_chains=split)
    check_full(x, out, sT, TOL["bf16"])
    o1, s1 = run(kda, x, nseg=1)
    chains = w.n_seq * w.H
    whole = [(c // w.H, c % w.H) for c in range(chains - split)]
    for n, h in whole:
        assert torch_equal(out_slice(x, out, n, h), out_slice(x, o1, n, h)), (n, h)
        assert torch_equal(sT[n, h], s1[n, h]), (n, h)


@pytest.mark.parametrize("wave", [0, 3, 4, 7])
def test_split_plan_stalled_wave_gives_same_bits(kda, wave):
    w = workloads.custom([300] * 3, H=2, D=128, dense=True, seed=81)
    x = gen(w)
    o0, s0 = run(kda, x, nseg=3, split_chains=2)
    o1, s1 = run(kda, x, nseg=3, split_chains=2, stall_wave=wave, stall_cycles=127 * 6)
    assert torch_equal(o0, o1) and torch_equal(s0, s1)


def test_planner_split_on_288_chains(kda):
    """288 equal chains: the planner segments only 32 of them; sampled chains of both kinds
    (whole and segmented) against the oracle, including the first and last of each kind."""
    import torch
    w = workloads.WORKLOADS["eqlen288"]
    x = gen(w)
    out, sT = run(kda, x)
    torch.cuda.synchronize()
    chains = [(0, 0), (7, 31), (3, 17), (8, 0), (8, 31), (8, 13)]     # chains 256..287 are n = 8
    worst = check_chains(x, out, sT, chains, TOL["bf16"])
    say(f"eqlen288 worst sampled rel-L2 {worst:.2e}")



@pytest.mark.parametrize("name", ["varlen", "eqlen", "long"])
def test_full_size_bits_stable_under_repeat_and_stall(kda, name):
    """The full-size workloads in the bench's launch configuration (one launch on varlen; map
    pass, COMBINE and segment outputs on eqlen and long): a second call, and calls with a
    consumer wave or a producer wave stalled after every barrier, give the first call's bits."""
    import torch
    w = workloads.WORKLOADS[name]
    x = gen(w)
    o0, s0 = run(kda, x)
    o1, s1 = run(kda, x)
    torch.cuda.synchronize()
    assert torch_equal(o0, o1) and torch_equal(s0, s1)
    for wave in (0, 5):          # the options leave the segment count to the planner: the same plan
        say(name, "full size, stalled wave", wave)
        o2, s2 = run(kda, x, stall_wave=wave, stall_cycles=127 * 2)
        torch.cuda.synchronize()
        assert torch_equal(o0, o2) and torch_equal(s0, s2), f"wave {wave}"
    del x, o0, o1, s0, s1
    torch.cuda.empty_cache()

