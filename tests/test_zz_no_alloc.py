"""The no-alloc entry point (kda_prefill_noalloc) against kda_prefill_ws, through the C ABI.

kda_prefill_noalloc keeps its scratch in a fixed device array of the library's (one per GPU,
kept until the process ends) and allocates nothing.  On plans that fit the array it must give
kda_prefill_ws's bits: two calls in a row on segmented plans (the scratch holds the segment
maps and start states), the second with a smaller input; a single-segment plan (no scratch);
standalone PREP (the gate sums in the scratch).  A forced plan that does not fit is refused
before anything is launched; an automatic one is planned with fewer segments and stays within
the oracle tolerance.
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


def bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def both(kda, x, **kw):
    """(out, final_state) of kda_prefill_ws (torch workspace) and of kda_prefill_noalloc, each
    into NaN-filled outputs."""
    import torch
    res = []
    for fn in (kda.prefill, kda.prefill_noalloc):
        out = torch.full_like(x["v"], float("nan"))
        N = x["initial_state"].shape[0]
        fin = torch.full((N,) + x["initial_state"].shape[1:], float("nan"), device="cuda")
        fn(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"], out=out, final_state=fin,
           **kw)
        res.append((out, fin))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("forced", [False, True])
def test_noalloc_matches_ws_two_calls_second_smaller(kda, forced):
    """Two calls in a row on segmented plans, the second on a smaller input (it sees the
    first call's scratch contents), each equal to kda_prefill_ws bit for bit."""
    import torch
    for i, (lengths, H) in enumerate((([3000, 0, 1700, 64], 3), ([1200, 5, 130], 2))):
        w = workloads.custom(lengths, H=H, D=128, seed=500 + i)
        x = workloads.make_inputs(w, device="cuda")
        kw = dict(nseg=4 if forced else 0)
        need = kda.workspace_size(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"], **kw)
        say("noalloc call", i, lengths, H, kw, "scratch", need)
        assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES
        (o_ws, s_ws), (o_na, s_na) = both(kda, x, **kw)
        assert torch.equal(bits(o_ws), bits(o_na)) and torch.equal(bits(s_ws), bits(s_na)), f"call {i}"
        o_ref, s_ref = oracle.run_c(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                                    x["initial_state"].cpu(), x["cu_seqlens"].cpu())
        assert oracle.rel_l2(o_na.float().cpu().numpy(), o_ref) <= 5e-3
        assert oracle.rel_l2(s_na.cpu().numpy(), s_ref) <= 5e-3


def test_noalloc_split_plan_matches(kda):
    """288 equal chains (B=9, H=32, T=1024): the planner splits the 32 chains past the CU
    count into segments and runs the other 256 whole; the no-alloc call plans the same (its
    scratch holds the 32 chains' maps and start states) and gives the same bits."""
    import torch
    w = workloads.custom([1024] * 9, H=32, D=128, dense=True, seed=520)
    x = workloads.make_inputs(w, device="cuda")
    need = kda.workspace_size(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], None)
    dd = 128 * 128 * 4
    say("noalloc split plan", "scratch", need)
    assert 0 < need <= kda.NOALLOC_SCRATCH_BYTES and need % (32 * dd) == 0     # 32 segmented chains only
    (o_ws, s_ws), (o_na, s_na) = both(kda, x)
    assert torch.equal(bits(o_ws), bits(o_na)) and torch.equal(bits(s_ws), bits(s_na))
    assert not torch.isnan(o_na.float()).any() and not torch.isnan(s_na).any()


def test_noalloc_capped_plan_matches(kda):
    """A packed batch of mixed lengths whose 256 chains fit the CUs runs the capped schedule
    (short sequences queue behind others, their flags in the scratch): the no-alloc call gives
    kda_prefill's bits, twice in a row (the flags of the first call are left in the
    scratch)."""
    import torch
    w = workloads.custom(workloads.varlen_lengths(), H=32, D=128, seed=530)
    x = workloads.make_inputs(w, device="cuda")
    need = kda.workspace_size(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    say("noalloc capped plan", "scratch", need)
    assert need == 256 * 8                                    # one flag per chain
    for i in range(2):
        (o_ws, s_ws), (o_na, s_na) = both(kda, x)
        assert torch.equal(bits(o_ws), bits(o_na)) and torch.equal(bits(s_ws), bits(s_na)), f"call {i}"


def test_noalloc_single_segment_and_standalone_prep(kda):
    import torch
    w = workloads.custom([900, 1, 77], H=2, D=128, seed=510)
    x = workloads.make_inputs(w, device="cuda")
    for kw in (dict(nseg=1), dict(nseg=1, prep=1), dict(nseg=3, prep=1), dict(nseg=2, variant=1)):
        say("noalloc", kw)
        (o_ws, s_ws), (o_na, s_na) = both(kda, x, **kw)
        assert torch.equal(bits(o_ws), bits(o_na)) and torch.equal(bits(s_ws), bits(s_na)), kw


def test_noalloc_refuses_forced_plan_beyond_scratch(kda):
    """nseg = 64 on 64 chains of 16K tokens needs 64 x 64 x 192 KB = 768 MiB of scratch:
    refused with KDA_ERR_WORKSPACE and the outputs untouched; the automatic plan for the same
    input fits by using fewer segments and matches the oracle on sampled chains."""
    import torch
    w = workloads.custom([16384] * 8, H=8, D=128, dense=True, seed=520)
    x = workloads.make_inputs(w, device="cuda")
    out = torch.full_like(x["v"], -512.0)
    fin = torch.empty_like(x["initial_state"])
    with pytest.raises(kda.KdaError) as e:
        kda.prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], None, out=out,
                            final_state=fin, nseg=64)
    assert e.value.status == 7 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out.float() == -512.0)
    kda.prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], None, out=out, final_state=fin)
    torch.cuda.synchronize()
    for n, h in ((0, 0), (7, 7), (3, 5)):
        o_ref, s_ref = oracle.run_c(x["q"][n, :, h:h + 1].cpu(), x["k"][n, :, h:h + 1].cpu(),
                                    x["v"][n, :, h:h + 1].cpu(), x["g"][n, :, h:h + 1].cpu(),
                                    x["beta"][n, :, h:h + 1].cpu(), x["initial_state"][n:n + 1, h:h + 1].cpu(),
                                    np.array([0, 16384]))
        assert oracle.rel_l2(out[n, :, h:h + 1].float().cpu().numpy().reshape(o_ref.shape), o_ref) <= 5e-3
        assert oracle.rel_l2(fin[n:n + 1, h:h + 1].cpu().numpy(), s_ref) <= 5e-3
