"""GPU parity of the recurrent decode / draft-verify kernel (kda_decode, called
through the C ABI) against the float64 oracle.

The oracle is the same token recurrence the prefill tests use: request r starts
from the pool slot it names (widened to float64 from the stored fp32 or bf16
values) and runs over its first n_r tokens.  Tolerances (whole-tensor relative
L2): 1e-4 with fp32 inputs and an fp32 pool; 5e-3 when q/k/v/out or the pool
are bf16 (a bf16 pool slot is rounded once when written back).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


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


def make_case(R, T, H, D, dtype, pool_dtype, seed, P=None):
    """Decode inputs in the workload recipe: R requests of T tokens ([R, T, H, D],
    a dense workload of R equal-length sequences), a pool of P random states
    (N(0, 0.1^2)), a permutation of slots with one request skipped (index -1) and
    per-request token counts in [0, T]."""
    import torch
    w = workloads.custom([T] * R, H=H, D=D, dtype=dtype, dense=True, seed=seed)
    x = workloads.make_inputs(w, device="cuda")
    P = P or R + 3
    gen = torch.Generator().manual_seed(seed + 1000)
    pool = (0.1 * torch.randn(P, H, D, D, generator=gen)).to({"f32": torch.float32, "bf16": torch.bfloat16}[pool_dtype])
    idx = torch.randperm(P, generator=gen)[:R].to(torch.int32)
    idx[R // 2] = -1
    ntok = torch.randint(0, T + 1, (R,), generator=gen, dtype=torch.int32)
    ntok[0] = T
    return x, pool.cuda(), idx.cuda(), ntok.cuda()


def oracle_decode(x, pool, idx, ntok, g=None, beta=None):
    """Per request: the float64 recurrence from pool[idx[r]] over its first n_r
    tokens.  Returns ({r: out rows [n_r, H, D]}, {r: final state [H, D, D]})."""
    import torch
    idx_h, n_h = idx.cpu().numpy(), ntok.cpu().numpy()
    g = x["g"].cpu() if g is None else torch.as_tensor(g)
    beta = x["beta"].cpu() if beta is None else torch.as_tensor(beta)
    reqs = [r for r in range(len(idx_h)) if idx_h[r] >= 0]
    cat = lambda t: torch.cat([t[r, : int(n_h[r])].double() for r in reqs])
    q, k, v = (cat(x[n].cpu()) for n in ("q", "k", "v"))
    gg, bb = cat(g), cat(beta)
    s0 = torch.stack([pool[int(idx_h[r])].cpu().double() for r in reqs])
    cu = np.concatenate([[0], np.cumsum([int(n_h[r]) for r in reqs])]).astype(np.int64)
    o, s = oracle.run_c(q, k, v, gg, bb, s0, cu)
    outs = {r: o[cu[i]:cu[i + 1]] for i, r in enumerate(reqs)}
    states = {r: s[i] for i, r in enumerate(reqs)}
    return outs, states


def check(x, out, pool_before, pool_after, idx, ntok, tol, update=True, **kw):
    import torch
    outs, states = oracle_decode(x, pool_before, idx, ntok, **kw)
    o_gpu = out.float().cpu().numpy()
    got = np.concatenate([o_gpu[r, : outs[r].shape[0]] for r in outs])
    want = np.concatenate([outs[r] for r in outs])
    eo = oracle.rel_l2(got, want) if want.size else 0.0
    idx_h, n_h = idx.cpu().numpy(), ntok.cpu().numpy()
    # rows past each request's count, and skipped requests, keep the sentinel
    for r in range(len(idx_h)):
        n = int(n_h[r]) if idx_h[r] >= 0 else 0
        assert torch.all(out[r, n:].float() == -512.0), f"request {r}: rows past {n} written"
    used = {int(idx_h[r]) for r in outs}
    for sl in range(pool_before.shape[0]):
        if sl not in used or not update:
            assert torch.equal(pool_after[sl].cpu(), pool_before[sl].cpu()), f"slot {sl} changed"
    es = 0.0
    if update and states:
        s_gpu = np.stack([pool_after[int(idx_h[r])].float().cpu().numpy() for r in states])
        s_ref = np.stack([states[r] for r in states])
        es = oracle.rel_l2(s_gpu, s_ref)
    assert eo <= tol and es <= tol, f"rel-L2 out {eo:.3e} state {es:.3e}"
    return eo, es


@pytest.mark.parametrize("pool_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_matches_oracle(kda, T, D, dtype, pool_dtype):
    import torch
    say("decode T", T, "D", D, dtype, "pool", pool_dtype)
    x, pool, idx, ntok = make_case(R=7, T=T, H=3, D=D, dtype=dtype, pool_dtype=pool_dtype, seed=40 + T + D)
    before = pool.clone()
    out = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, idx, ntok, out=out)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "f32" and pool_dtype == "f32" else 5e-3
    check(x, out, before, pool, idx, ntok, tol)


def test_decode_all_tokens_and_repeat_bitwise(kda):
    """num_tokens = NULL runs every token; two runs from the same pool give the same bits."""
    import torch
    x, pool, idx, _ = make_case(R=5, T=3, H=2, D=128, dtype="bf16", pool_dtype="f32", seed=51)
    ntok = torch.full((5,), 3, dtype=torch.int32, device="cuda")
    p1, p2 = pool.clone(), pool.clone()
    o1 = torch.full_like(x["v"], -512.0)
    o2 = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], p1, idx, None, out=o1)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], p2, idx, None, out=o2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(p1, p2)
    check(x, o1, pool, p1, idx, ntok, 5e-3)


def test_verify_then_replay_commit(kda):
    """The draft-verify flow: a verify pass over T drafts reads the pool only; a
    replay-only commit of the accepted count per request then writes the state
    the oracle reaches after those tokens, and the verify outputs of the accepted
    tokens are the oracle's."""
    import torch
    x, pool, idx, acc = make_case(R=6, T=4, H=2, D=128, dtype="bf16", pool_dtype="bf16", seed=52)
    before = pool.clone()
    out = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, idx, None, out=out, update_state=False)
    torch.cuda.synchronize()
    assert torch.equal(pool, before), "the verify pass wrote the pool"
    full = torch.full((6,), 4, dtype=torch.int32, device="cuda")
    check(x, out, before, pool, idx, full, 5e-3, update=False)
    r = kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, idx, acc, update_state=True, write_out=False)
    torch.cuda.synchronize()
    assert r is None
    _, states = oracle_decode(x, before, idx, acc)
    idx_h = idx.cpu().numpy()
    s_gpu = np.stack([pool[int(idx_h[r])].float().cpu().numpy() for r in states])
    s_ref = np.stack([states[r] for r in states])
    assert oracle.rel_l2(s_gpu, s_ref) <= 5e-3
    # verify outputs equal a committing decode's outputs bit for bit (one kernel, same order)
    p3 = before.clone()
    o3 = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], p3, idx, None, out=o3, update_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.int16), out.view(torch.int16))


def test_decode_continues_prefill(kda):
    """Prefill L tokens (chunked kernel) into a pool slot, then decode the next T
    tokens (recurrent kernel): the decode outputs match a prefill of all L + T
    tokens within the tolerance (two different kernels, same recurrence)."""
    import torch
    H, D, L, T = 2, 128, 200, 4
    w = workloads.custom([L + T], H=H, D=D, dtype="bf16", dense=True, seed=53)
    x = workloads.make_inputs(w, device="cuda")
    o_all, s_all = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"])
    cut = lambda t, a, b: t[:, a:b].contiguous()
    _, s_mid = kda.prefill(cut(x["q"], 0, L), cut(x["k"], 0, L), cut(x["v"], 0, L), cut(x["g"], 0, L),
                           cut(x["beta"], 0, L), x["initial_state"])
    pool = torch.zeros(3, H, D, D, device="cuda")
    pool[2] = s_mid[0]
    idx = torch.tensor([2], dtype=torch.int32, device="cuda")
    out = kda.decode(cut(x["q"], L, L + T), cut(x["k"], L, L + T), cut(x["v"], L, L + T), cut(x["g"], L, L + T),
                     cut(x["beta"], L, L + T), pool, idx)
    torch.cuda.synchronize()
    ref = o_all[:, L:].float()
    assert ((out.float() - ref).norm() / ref.norm()).item() <= 5e-3
    assert ((pool[2] - s_all[0]).norm() / s_all[0].norm()).item() <= 5e-3


def test_decode_logit_inputs(kda):
    import torch
    x, pool, idx, ntok = make_case(R=5, T=4, H=2, D=128, dtype="bf16", pool_dtype="f32", seed=54)
    before = pool.clone()
    out = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g_logits"], x["beta_logits"], pool, idx, ntok, out=out,
               gate_logits=True, beta_logits=True, gate_lower_bound=-5.0)
    torch.cuda.synchronize()
    g64, b64 = oracle.activations(x["g_logits"].cpu(), x["beta_logits"].cpu(), -5.0)
    check(x, out, before, pool, idx, ntok, 5e-3, g=g64, beta=b64)


@pytest.mark.parametrize("pool_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("wave", [0, 1, 2, 3])
def test_decode_stalled_wave_gives_same_bits(kda, wave, pool_dtype):
    """A copy of the decode kernel with one of its 4 waves stalled ~20 us after every
    barrier reproduces the unstalled bits (its cross-wave reductions go through LDS)."""
    import torch
    x, pool, idx, ntok = make_case(R=5, T=4, H=2, D=128, dtype="bf16", pool_dtype=pool_dtype, seed=55)
    say("decode stall wave", wave, pool_dtype)
    p1, p2 = pool.clone(), pool.clone()
    o1 = torch.full_like(x["v"], -512.0)
    o2 = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], p1, idx, ntok, out=o1)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], p2, idx, ntok, out=o2, stall_wave=wave,
               stall_cycles=127 * 6)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(p1.view(torch.int16) if p1.dtype == torch.bfloat16 else p1.view(torch.int32),
                       p2.view(torch.int16) if p2.dtype == torch.bfloat16 else p2.view(torch.int32))


@pytest.mark.parametrize("name", ["decode", "decode_bf16", "verify4"])
def test_decode_bench_workloads(kda, name):
    """The bench's decode workloads at full size (256 requests x 32 heads), every
    request against the float64 oracle, in the launch the bench times."""
    import torch
    w = workloads.DECODE_WORKLOADS[name]
    x = workloads.make_decode_inputs(w, device="cuda")
    say("decode workload", name)
    pool = x["pool"].clone()
    out = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, x["idx"], None, out=out)
    torch.cuda.synchronize()
    ntok = torch.full((w.R,), w.T, dtype=torch.int32, device="cuda")
    check(x, out, x["pool"], pool, x["idx"], ntok, 5e-3)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_output_norm(kda, D):
    """The gated RMS norm epilogue in decode: outputs equal the float64 oracle's
    outputs through the float64 gated RMS norm; the pool update is unchanged."""
    import torch
    x, pool, idx, ntok = make_case(R=6, T=3, H=2, D=D, dtype="bf16", pool_dtype="f32", seed=56)
    gen = torch.Generator(device="cuda").manual_seed(57)
    z = torch.randn(x["v"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn(D, generator=gen, device="cuda")
    before = pool.clone()
    out = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, idx, ntok, out=out, out_gate=z, norm_weight=nw,
               norm_eps=1e-6)
    torch.cuda.synchronize()
    outs, states = oracle_decode(x, before, idx, ntok)
    zc, o_gpu = z.float().cpu().numpy(), out.float().cpu().numpy()
    got = np.concatenate([o_gpu[r, : outs[r].shape[0]] for r in outs])
    want = np.concatenate([oracle.gated_rmsnorm(outs[r], zc[r, : outs[r].shape[0]], nw.cpu().numpy(), 1e-6)
                           for r in outs])
    assert oracle.rel_l2(got, want) <= 5e-3
    idx_h = idx.cpu().numpy()
    s_gpu = np.stack([pool[int(idx_h[r])].cpu().numpy() for r in states])
    assert oracle.rel_l2(s_gpu, np.stack([states[r] for r in states])) <= 5e-3


def test_decode_graph_replay(kda):
    """kda_decode captured in a HIP graph (one launch, nothing allocated): q changes
    between replays and each replay of the verify pass equals a fresh eager call bit
    for bit; a committing replay advances the pool exactly as an eager call does."""
    import torch
    x, pool, idx, ntok = make_case(R=6, T=4, H=2, D=128, dtype="bf16", pool_dtype="f32", seed=58)
    qbuf = x["q"].clone()
    out = torch.full_like(x["v"], -512.0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.decode(qbuf, x["k"], x["v"], x["g"], x["beta"], pool, idx, ntok, out=out, update_state=False)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.decode(qbuf, x["k"], x["v"], x["g"], x["beta"], pool, idx, ntok, out=out, update_state=False)
    gen_ = torch.Generator(device="cuda")
    for rep in range(4):
        gen_.manual_seed(200 + rep)
        newq = torch.randn(qbuf.shape, generator=gen_, device="cuda")
        qbuf.copy_((newq / newq.norm(dim=-1, keepdim=True)).to(qbuf.dtype))
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.full_like(x["v"], -512.0)
        kda.decode(qbuf.clone(), x["k"], x["v"], x["g"], x["beta"], pool, idx, ntok, out=ref, update_state=False)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
    # a committing graph: two replays advance the pool as two eager calls do
    p_graph, p_eager = pool.clone(), pool.clone()
    o_g = torch.empty_like(x["v"])
    with torch.cuda.stream(s):
        kda.decode(qbuf, x["k"], x["v"], x["g"], x["beta"], p_graph.clone(), idx, ntok, out=o_g)
    torch.cuda.current_stream().wait_stream(s)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        kda.decode(qbuf, x["k"], x["v"], x["g"], x["beta"], p_graph, idx, ntok, out=o_g)
    for _ in range(2):
        g2.replay()
        torch.cuda.synchronize()
        o_e = torch.empty_like(x["v"])
        kda.decode(qbuf, x["k"], x["v"], x["g"], x["beta"], p_eager, idx, ntok, out=o_e)
        torch.cuda.synchronize()
        assert torch.equal(p_graph, p_eager)


# ------------------------------------------------ seeded random configurations
def _draw_decode(i):
    rng = np.random.default_rng(5000 + i)
    return dict(case=i, R=int(rng.integers(1, 12)), T=int(rng.integers(1, 9)), H=int(rng.integers(1, 5)),
                D=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "bf16", "f32"])),
                pool_dtype=str(rng.choice(["f32", "bf16"])), extra_slots=int(rng.integers(0, 6)),
                bad_idx=bool(rng.random() < 0.5), ntok_null=bool(rng.random() < 0.25),
                update=bool(rng.random() < 0.8), write_out=bool(rng.random() < 0.85),
                logits=bool(rng.random() < 0.3), norm=bool(rng.random() < 0.25),
                gate=str(rng.choice(["none", "none", "mild", "floor"])),
                lb=float(rng.choice([-5.0, -5.0, -3.0, -1.0, -0.25])))      # gate lower bound with logits


DECODE_CASES = [_draw_decode(i) for i in range(int(__import__("os").environ.get("KDA_RANDOM_CASES", "24")))]


@pytest.mark.parametrize("c", DECODE_CASES, ids=[f"case{c['case']}" for c in DECODE_CASES])
def test_decode_random_configuration(kda, c):
    """Seeded random decode calls: request and token counts (including requests with no
    tokens), head size, I/O and pool dtypes, slot indices below 0 or past the pool
    (skipped), verify (no state update) or commit, outputs written or not, logit inputs,
    the output norm, and the gate distributions; every output row, every pool slot
    (written or required unchanged) and the rows left alone are checked."""
    import torch
    say("decode random", c)
    R, T, H, D = c["R"], c["T"], c["H"], c["D"]
    w = workloads.custom([T] * R, H=H, D=D, dtype=c["dtype"], dense=True, seed=6000 + c["case"])
    x = workloads.make_inputs(w, device="cuda", gate=None if c["gate"] == "none" else c["gate"])
    P = R + c["extra_slots"]
    gen = torch.Generator().manual_seed(7000 + c["case"])
    pool = (0.1 * torch.randn(P, H, D, D, generator=gen)).to(
        {"f32": torch.float32, "bf16": torch.bfloat16}[c["pool_dtype"]]).cuda()
    idx = torch.randperm(P, generator=gen)[:R].to(torch.int32)
    if c["bad_idx"] and R > 1:
        idx[R - 1] = -3
        idx[0] = P + 2 if R > 2 else idx[0]
    ntok = None if c["ntok_null"] else torch.randint(0, T + 1, (R,), generator=gen, dtype=torch.int32)
    n_eff = torch.full((R,), T, dtype=torch.int32) if ntok is None else ntok
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    z = nw = None
    norm = c["norm"] and c["write_out"]      # the norm needs out
    if norm:
        gz = torch.Generator(device="cuda").manual_seed(8000 + c["case"])
        z = torch.randn(x["v"].shape, generator=gz, device="cuda").to(x["v"].dtype)
        nw = 1.0 + 0.1 * torch.randn(D, generator=gz, device="cuda")
    before = pool.clone()
    out = torch.full_like(x["v"], -512.0) if c["write_out"] else None
    kda.decode(x["q"], x["k"], x["v"], g_in, b_in, pool, idx.cuda(), None if ntok is None else ntok.cuda(), out=out,
               update_state=c["update"], write_out=c["write_out"], gate_logits=logits, beta_logits=logits,
               gate_lower_bound=c["lb"],
               out_gate=z, norm_weight=nw, norm_eps=1e-6)
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx < P)
    idx_o = torch.where(valid, idx, torch.full_like(idx, -1))
    g64, b64 = (oracle.activations(x["g_logits"].cpu(), x["beta_logits"].cpu(), c["lb"]) if logits else (None, None))
    outs, states = oracle_decode(x, before, idx_o, n_eff, g=g64, beta=b64)
    tol = 1e-4 if c["dtype"] == "f32" and c["pool_dtype"] == "f32" else 5e-3
    if out is not None:
        o_gpu = out.float().cpu().numpy()
        for r in range(R):
            n = int(n_eff[r]) if valid[r] else 0
            assert torch.all(out[r, n:].float() == -512.0), f"request {r}: rows past {n} written"
        if outs and sum(v.shape[0] for v in outs.values()):
            want = np.concatenate([outs[r] for r in outs])
            if norm:
                zc = z.float().cpu().numpy()
                want = np.concatenate([oracle.gated_rmsnorm(outs[r], zc[r, : outs[r].shape[0]], nw.cpu().numpy(), 1e-6)
                                       for r in outs])
            got = np.concatenate([o_gpu[r, : outs[r].shape[0]] for r in outs])
            eo = oracle.rel_l2(got, want) if np.abs(want).sum() > 0 else float(np.abs(got).max())
            assert eo <= tol, f"out {eo:.3e}"
    written = {int(idx[r]) for r in states} if c["update"] else set()
    for sl in range(P):
        if sl not in written:
            assert torch.equal(pool[sl].cpu(), before[sl].cpu()), f"slot {sl} changed"
    if written:
        s_gpu = np.stack([pool[int(idx[r])].float().cpu().numpy() for r in states])
        s_ref = np.stack([states[r] for r in states])
        es = oracle.rel_l2(s_gpu, s_ref)
        assert es <= tol, f"state {es:.3e}"


def _padded(t, rng, align):
    """The same values in a view with padded strides (NaN in the padding), each stride a
    multiple of `align` elements."""
    import torch
    shape = list(t.shape)
    pad = [int(rng.integers(0, 3)) * align for _ in shape]
    big = torch.full([s + p for s, p in zip(shape, pad)], float("nan"), dtype=t.dtype, device=t.device)
    view = big[tuple(slice(0, s) for s in shape)]
    view.copy_(t)
    return view


@pytest.mark.parametrize("c", DECODE_CASES, ids=[f"case{c['case']}" for c in DECODE_CASES])
def test_decode_random_padded_views(kda, c):
    """The random decode configurations with q, k, v, g, beta, out, the output gate and
    the state pool passed as NaN-padded strided views give the contiguous call's bits,
    in the outputs and in every pool slot."""
    import torch
    R, T, H, D = c["R"], c["T"], c["H"], c["D"]
    w = workloads.custom([T] * R, H=H, D=D, dtype=c["dtype"], dense=True, seed=6000 + c["case"])
    x = workloads.make_inputs(w, device="cuda", gate=None if c["gate"] == "none" else c["gate"])
    P = R + c["extra_slots"]
    gen = torch.Generator().manual_seed(7000 + c["case"])
    pool = (0.1 * torch.randn(P, H, D, D, generator=gen)).to(
        {"f32": torch.float32, "bf16": torch.bfloat16}[c["pool_dtype"]]).cuda()
    idx = torch.randperm(P, generator=gen)[:R].to(torch.int32).cuda()
    ntok = None if c["ntok_null"] else torch.randint(0, T + 1, (R,), generator=gen, dtype=torch.int32).cuda()
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    z = nw = None
    if c["norm"]:
        gz = torch.Generator(device="cuda").manual_seed(8000 + c["case"])
        z = torch.randn(x["v"].shape, generator=gz, device="cuda").to(x["v"].dtype)
        nw = 1.0 + 0.1 * torch.randn(D, generator=gz, device="cuda")
    say("decode padded views", c)
    kw = dict(update_state=c["update"], gate_logits=logits, beta_logits=logits, gate_lower_bound=c["lb"],
              norm_weight=nw, norm_eps=1e-6)
    p0 = pool.clone()
    o0 = torch.full_like(x["v"], -512.0)
    kda.decode(x["q"], x["k"], x["v"], g_in, b_in, p0, idx, ntok, out=o0, out_gate=z, **kw)
    rng = np.random.default_rng(9000 + c["case"])
    pad = lambda t, a=4: None if t is None else _padded(t, rng, a)
    p1 = pad(pool)
    o1 = pad(torch.full_like(x["v"], -512.0))
    kda.decode(pad(x["q"]), pad(x["k"]), pad(x["v"]), pad(g_in), pad(b_in, 1), p1, idx, ntok, out=o1, out_gate=pad(z), **kw)
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous().view(torch.int32)
    assert torch.equal(bits(o0), bits(o1)) and torch.equal(bits(p0), bits(p1))


@pytest.mark.parametrize("c", DECODE_CASES, ids=[f"case{c['case']}" for c in DECODE_CASES])
def test_decode_random_stalled_wave(kda, c):
    """The random decode configurations with one of the 4 waves (chosen by the case)
    stalled after every barrier give the unstalled bits, in the outputs and the pool."""
    import torch
    R, T, H, D = c["R"], c["T"], c["H"], c["D"]
    w = workloads.custom([T] * R, H=H, D=D, dtype=c["dtype"], dense=True, seed=6000 + c["case"])
    x = workloads.make_inputs(w, device="cuda", gate=None if c["gate"] == "none" else c["gate"])
    P = R + c["extra_slots"]
    gen = torch.Generator().manual_seed(7000 + c["case"])
    pool = (0.1 * torch.randn(P, H, D, D, generator=gen)).to(
        {"f32": torch.float32, "bf16": torch.bfloat16}[c["pool_dtype"]]).cuda()
    idx = torch.randperm(P, generator=gen)[:R].to(torch.int32).cuda()
    ntok = None if c["ntok_null"] else torch.randint(0, T + 1, (R,), generator=gen, dtype=torch.int32).cuda()
    logits = c["logits"] and x["g_logits"] is not None
    g_in, b_in = (x["g_logits"], x["beta_logits"]) if logits else (x["g"], x["beta"])
    z = nw = None
    if c["norm"]:
        gz = torch.Generator(device="cuda").manual_seed(8000 + c["case"])
        z = torch.randn(x["v"].shape, generator=gz, device="cuda").to(x["v"].dtype)
        nw = 1.0 + 0.1 * torch.randn(D, generator=gz, device="cuda")
    wave = c["case"] % 4
    say("decode stalled wave", wave, c)
    kw = dict(update_state=c["update"], gate_logits=logits, beta_logits=logits, gate_lower_bound=c["lb"], out_gate=z,
              norm_weight=nw, norm_eps=1e-6)
    res = []
    for stall in (dict(), dict(stall_wave=wave, stall_cycles=127 * 6)):
        p = pool.clone()
        o = torch.full_like(x["v"], -512.0)
        kda.decode(x["q"], x["k"], x["v"], g_in, b_in, p, idx, ntok, out=o, **kw, **stall)
        res.append((o, p))
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(bits(res[0][0]), bits(res[1][0])) and torch.equal(bits(res[0][1]), bits(res[1][1]))


def test_check_rejects_duplicate_slots_and_bad_gates(kda, monkeypatch):
    """With KDA_CHECK=1 kda_decode refuses, before its kernel runs, two requests naming
    the same slot when the state update is on (KDA_ERR_ALIAS), and a g outside [-5, 0]
    (KDA_ERR_RANGE); the pool and out stay untouched.  Repeated slots are fine for the
    verify pass and for skipped (out-of-range) indices; valid calls give the unchecked
    bits."""
    import torch
    x, pool, idx, ntok = make_case(R=300, T=2, H=2, D=128, dtype="bf16", pool_dtype="f32", seed=71, P=400)
    args = lambda p, i, g=None: (x["q"], x["k"], x["v"], x["g"] if g is None else g, x["beta"], p, i, ntok)
    # rows past each request's token count are left untouched: both outputs start as the sentinel
    p0 = pool.clone()
    o0 = kda.decode(*args(p0, idx), out=torch.full_like(x["v"], -512.0))
    monkeypatch.setenv("KDA_CHECK", "1")
    p1 = pool.clone()
    o1 = kda.decode(*args(p1, idx), out=torch.full_like(x["v"], -512.0))
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(p0.view(torch.int32), p1.view(torch.int32))
    dup = idx.clone()
    dup[250] = dup[3]                  # two live requests on one slot
    say("KDA_CHECK decode duplicate slots")
    p2 = pool.clone()
    out = torch.full_like(x["v"], -512.0)
    with pytest.raises(kda.KdaError) as e:
        kda.decode(*args(p2, dup), out=out)
    assert e.value.status == 5 and "slot" in str(e.value)
    assert torch.all(out.float() == -512.0) and torch.equal(p2.view(torch.int32), pool.view(torch.int32))
    kda.decode(*args(p2, dup), out=out, update_state=False)      # verify pass: repeats allowed
    skip = idx.clone()
    skip[10], skip[20] = -7, -7        # repeated out-of-range indices are skipped requests
    kda.decode(*args(pool.clone(), skip))
    g = x["g"].clone()
    g[5, 1, 1, 3] = -6.0
    with pytest.raises(kda.KdaError) as e:
        kda.decode(*args(pool.clone(), idx, g))
    assert e.value.status == 9
