"""White-box checks of the segmented path through the caller's workspace.

After a forced-nseg call of ``kda_prefill_ws`` the workspace holds, for every chain and
segment s < nseg - 1, the segment maps the chunk kernel's map roles wrote (M_s: the end
state of segment s from V = 0 and start state I; C_s: from start state 0), then every
start state COMBINE wrote.  Two checks, each independent of the other kernels' rounding:

* the maps against the float64 oracle run over the segment's own tokens with those start
  states and values (the definition of the two maps: S_end = M_s S_start + C_s);
* COMBINE's arithmetic: start[0] is the initial state bit for bit, and every start[s+1]
  equals M_s start[s] + C_s computed in float64 from the stored M_s, C_s and start[s],
  element by element within a bound proportional to |M_s| |start[s]| + |C_s| (the split
  bf16 product keeps about 16 bits: 2^-14; fp32 MFMAs over 128 terms: 2^-16).

The workspace layout is the library's own (maps, then start states, 256-byte aligned; M
in the order COMBINE reads it, split into two bf16 parts on bf16 I/O; C and the start
states row-major fp32).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 5e-3          # the bf16 path's gate against the oracle (fp32 I/O: 1e-4)


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


def _m_index(D, split):
    """Index of element (row, k) of a stored M: bf16 elements of the high part (split) or
    floats."""
    r, k = np.meshgrid(np.arange(D), np.arange(D), indexing="ij")
    if split:
        return (((r >> 4) * (D >> 4) + 2 * (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (r & 15)) * 8 + (k & 7)
    return (((r >> 4) * (D >> 4) + (k >> 4)) * 64 + ((k & 15) >> 2) * 16 + (r & 15)) * 4 + (k & 3)


def _bf16(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _decode_m(raw, D, split):
    idx = _m_index(D, split)
    if split:
        h = raw.view(np.uint16)
        return _bf16(h[idx]) + _bf16(h[idx + 512])
    return raw.view(np.float32)[idx].astype(np.float64)


@pytest.mark.parametrize("dtype,D,variant,chunk", [
    ("bf16", 128, 0, 32),       # pipelined kernel: merged M/C workgroups, split maps
    ("bf16", 128, 1, 64),       # single-role kernel at d = 128: separate M and C, split maps
    ("bf16", 64, 0, 64),        # single-role kernel at d = 64
    ("f32", 64, 0, 64),         # fp32 debug mode: fp32 maps, fp32 COMBINE
])
def test_segment_maps_and_combine_in_the_workspace(kda, dtype, D, variant, chunk):
    import torch
    nseg, H = 4, 2
    lengths = [700, 450]
    say("segment maps", dtype, D, "variant", variant, "lengths", lengths, "nseg", nseg)
    w = workloads.custom(lengths, H=H, D=D, dtype=dtype, dense=False, seed=5)
    x = workloads.make_inputs(w, device="cuda", gate="mild")
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    need = kda.workspace_size(*args, nseg=nseg, variant=variant)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert ws.data_ptr() % 256 == 0
    kda.prefill(*args, nseg=nseg, variant=variant, workspace=ws)
    torch.cuda.synchronize()

    chains, dd = len(lengths) * H, D * D * 4
    maps_bytes = chains * (nseg - 1) * 2 * dd
    off_start = (maps_bytes + 255) // 256 * 256
    assert need == off_start + chains * nseg * dd
    raw = ws.cpu().numpy()
    maps = raw[:maps_bytes].reshape(chains, nseg - 1, 2, dd)
    start = raw[off_start:off_start + chains * nseg * dd].view(np.float32).reshape(chains, nseg, D, D)
    split = dtype == "bf16"

    cat = lambda t: t.detach().cpu().double().numpy()
    q, k, v, g, beta = (cat(x[n]) for n in ("q", "k", "v", "g", "beta"))
    s0 = cat(x["initial_state"])
    cu = workloads.cu_from_lengths(lengths)
    eye = np.broadcast_to(np.eye(D), (1, H, D, D)).copy()
    tol_maps = TOL if split else 1e-4
    tol_scan = 2.0 ** -14 if split else 2.0 ** -16
    for n, L in enumerate(lengths):
        nck = -(-L // chunk)
        cps = -(-nck // nseg)
        for s in range(nseg - 1):
            t0, t1 = min(s * cps * chunk, L), min((s + 1) * cps * chunk, L)
            sl = slice(cu[n] + t0, cu[n] + t1)
            seg_cu = np.array([0, t1 - t0], dtype=np.int64)
            if t1 > t0:
                _, m_ref = oracle.run_c(q[sl], k[sl], np.zeros_like(v[sl]), g[sl], beta[sl], eye, seg_cu)
                _, c_ref = oracle.run_c(q[sl], k[sl], v[sl], g[sl], beta[sl], None, seg_cu)
            else:                           # an empty segment: the identity map
                m_ref, c_ref = eye, np.zeros_like(eye)
            for h in range(H):
                c = n * H + h
                M = _decode_m(maps[c, s, 0], D, split)
                C = maps[c, s, 1].view(np.float32).reshape(D, D).astype(np.float64)
                em, ec = oracle.rel_l2(M, m_ref[0, h]), oracle.rel_l2(C, c_ref[0, h])
                assert em <= tol_maps and ec <= tol_maps, (n, s, h, em, ec)
        for h in range(H):
            c = n * H + h
            assert np.array_equal(start[c, 0], x["initial_state"][n, h].cpu().numpy())
            for s in range(nseg - 1):
                M = _decode_m(maps[c, s, 0], D, split)
                C = maps[c, s, 1].view(np.float32).reshape(D, D).astype(np.float64)
                S = start[c, s].astype(np.float64)
                ref = M @ S + C
                bound = tol_scan * (np.abs(M) @ np.abs(S) + np.abs(C)) + 1e-30
                worst = float(np.max(np.abs(start[c, s + 1] - ref) / bound))
                assert worst <= 1.0, (n, h, s, worst)
