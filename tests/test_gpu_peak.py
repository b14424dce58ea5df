"""The measurement probes behind `bench.py --peak` compute what they claim, so the practical
ceilings they report are for real work: the stream probe's output is the XOR of its five
inputs bit for bit (every byte read and written once), and the MFMA loop accumulates the
same product every iteration in every wave (twice the iterations give exactly twice the
sum: doubling is exact in floating point)."""
import sys

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_38_amd as k
    k.load_library()
    return k


@pytest.mark.parametrize("n16", [1, 255, 256, 257, 100003])
def test_stream_probe_xors_its_inputs(kda, n16):
    import torch
    print("[case] stream probe n16", n16, file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(n16)
    ins = [torch.randint(-2**31, 2**31 - 1, (n16, 4), dtype=torch.int32, device="cuda", generator=g) for _ in range(5)]
    out = torch.full((n16, 4), 7, dtype=torch.int32, device="cuda")
    kda.peak_stream(ins, out)
    torch.cuda.synchronize()
    ref = ins[0] ^ ins[1] ^ ins[2] ^ ins[3] ^ ins[4]
    assert torch.equal(out, ref)


def test_mfma_probe_accumulates_the_same_product(kda):
    import torch
    wg = 300
    outs = []
    for iters in (1, 2, 4):
        o = torch.full((wg * 4,), float("nan"), dtype=torch.float32, device="cuda")
        kda.peak_mfma(o, wg, iters)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    one = outs[0]
    assert torch.isfinite(one).all() and one[0] != 0
    assert torch.equal(one, torch.full_like(one, float(one[0])))        # every wave the same
    assert torch.equal(outs[1], 2 * one) and torch.equal(outs[2], 4 * one)
