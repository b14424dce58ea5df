"""Host-side logic of bench.py: the algorithmic byte counts behind the roofline
figures (counted here from the tensors the workloads actually build), the CU
load balance of the single-segment plan (by simulating the schedule), the
staleness rule for committed traffic figures, and the one-GPU refusal."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def _nbytes(t):
    return t.numel() * t.element_size()


@pytest.mark.parametrize("w", [
    workloads.custom([5, 70, 33], H=3, D=128, seed=1),
    workloads.custom([40, 40], H=2, D=64, dtype="f32", dense=True, seed=2),
])
def test_algorithmic_bytes_are_the_tensors_bytes(w):
    """Inputs read once (q, k, v, g, beta, initial state) and outputs written once
    (out shaped like v, final state shaped like the initial state)."""
    x = workloads.make_inputs(w)
    read = sum(_nbytes(x[n]) for n in ("q", "k", "v", "g", "beta", "initial_state"))
    written = _nbytes(x["v"]) + _nbytes(x["initial_state"])
    bytes_, _, per_th = bench.algorithmic(w)
    assert bytes_ == read + written
    assert per_th * w.tokens * w.H + 2 * _nbytes(x["initial_state"]) == bytes_


def test_decode_algorithmic_bytes_are_the_tensors_bytes():
    w = workloads.DecodeWorkload("t", R=5, T=3, H=2, D=64, pool_dtype="bf16", P=9)
    x = workloads.make_decode_inputs(w)
    slot_bytes = _nbytes(x["pool"]) // w.P
    read = sum(_nbytes(x[n]) for n in ("q", "k", "v", "g", "beta", "idx")) + w.R * slot_bytes
    written = _nbytes(x["v"]) + w.R * slot_bytes
    assert bench.decode_algorithmic(w)[0] == read + written


def _simulate(lengths, H, cus, chunk, longest_first=False):
    """Chains start in launch order (or longest sequence first) on the first free CU and
    run to the end."""
    free = [0] * cus
    seqs = sorted(lengths, key=lambda L: -L) if longest_first else list(lengths)
    for L in seqs:
        for _ in range(H):
            i = min(range(cus), key=lambda c: free[c])
            free[i] += math.ceil(L / chunk)
    busy = [f for f in free if f]
    return max(free), sum(busy) / len(busy)


@pytest.mark.parametrize("name", ["varlen", "varlen_padded", "varlen_h64", "large", "long"])
def test_work_balance_matches_a_simulated_schedule(name):
    w = workloads.WORKLOADS[name]
    wb = bench.work_balance(w)
    lpt = (not w.dense) and w.n_seq * w.H > 256 and 1 < w.n_seq <= 512
    makespan, mean_busy = _simulate(w.lengths, w.H, 256, 32, lpt)
    assert wb["chains"] == w.n_seq * w.H
    assert wb["order"] == ("longest-first" if lpt else "launch")
    assert wb["makespan_chunks"] == makespan
    assert wb["mean_chunks_per_cu"] == pytest.approx(mean_busy)
    assert wb["occupancy_bound"] == pytest.approx(mean_busy / makespan)


def test_varlen_balance_figures():
    wb = bench.work_balance(workloads.WORKLOADS["varlen"])
    assert (wb["chains"], wb["longest_chain_chunks"], wb["makespan_chunks"]) == (256, 221, 221)
    assert wb["occupancy_bound"] == pytest.approx(1027 * 32 / 256 / 221)
    # the same lengths at 64 heads: 389 chunk-steps in launch order, 270 longest first
    w = workloads.WORKLOADS["varlen_h64"]
    assert _simulate(w.lengths, w.H, 256, 32, False)[0] == 389
    assert bench.work_balance(w)["makespan_chunks"] == 270


def test_traffic_figure_is_dropped_when_the_kernel_source_changes(monkeypatch):
    for kernel, config in (("chunk_kernel", "varlen"), ("decode_kernel", "decode")):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.json")))
        assert rec["kernel"] in ("chunk_pipe_kernel", "decode_kernel")
        if rec["kernel_source_sha"] == bench.source_sha(kernel):
            assert bench.traffic_from_profile(config, kernel) == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_sha", lambda kernel="chunk_kernel": "0" * 16)
    assert bench.traffic_from_profile("varlen") is None
    assert bench.traffic_from_profile("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_sampled_chains_cross_the_2gib_offset_of_g():
    """On the large workload g is 2^32 bytes: the sample holds the last chain whose g rows
    all lie below 2^31 bytes, the first at or past it, and the chain of the highest offset,
    besides the first and the last; 16 distinct chains in all."""
    w = workloads.WORKLOADS["large"]
    ch = bench.sample_chains(w, 16)
    assert len(ch) == 16 and len(set(ch)) == 16
    T, H, D = 8192, 64, 128
    lo = lambda n, h: ((n * T) * H + h) * D * 4
    assert (8, 0) in ch and lo(8, 0) == 1 << 31           # first chain at 2^31
    assert (7, 63) in ch and lo(7, 63) < 1 << 31          # last chain below it
    assert (15, 63) in ch and (0, 0) in ch
    # a small workload has no such chains: first, last and random ones
    v = bench.sample_chains(workloads.WORKLOADS["varlen"], 16)
    assert len(v) == 16 and v[0] == (0, 0) and v[1] == (7, 31)


def test_whole_call_roofline_from_a_multi_launch_profile():
    """A segmented call's roofline divides the call's algorithmic bytes by the sum of all its
    launches (segment build, COMBINE, segment output) per step, not by the chunk launches
    alone; the split gives each kernel's share."""
    w = workloads.WORKLOADS["eqlen"]
    steps = 4
    prof = {"kda_chunk_segbuild": (steps, 0.080 * steps), "kda_combine": (steps, 0.020 * steps),
            "kda_chunk_segout": (steps, 0.050 * steps)}
    roof, mfma, kern = bench.kernel_record(w, prof, steps)
    bytes_, flops, _ = bench.algorithmic(w)
    assert kern["launches_per_step"] == 3 and kern["avg_ms"] == pytest.approx(0.150)
    assert roof["achieved"] == pytest.approx(bytes_ / 0.150e-3 / 1e9)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0)
    assert mfma["achieved"] == pytest.approx(flops / 0.150e-3 / 1e12)
    shares = {s["name"]: s["share"] for s in kern["split"]}
    assert shares == pytest.approx({"kda_chunk_segbuild": 0.08 / 0.15, "kda_combine": 0.02 / 0.15,
                                    "kda_chunk_segout": 0.05 / 0.15})
    # one launch: the kernel's own duration
    roof1, _, kern1 = bench.kernel_record(workloads.WORKLOADS["varlen"], {"kda_chunk": (steps, 0.46 * steps)}, steps)
    assert kern1["launches_per_step"] == 1 and kern1["name"] == "kda_chunk"
    assert roof1["achieved"] == pytest.approx(bench.algorithmic(workloads.WORKLOADS["varlen"])[0] / 0.46e-3 / 1e9)


def test_timing_statistics():
    st = bench._stats([5.0, 1.0, 3.0, 2.0, 4.0, 6.0, 7.0])
    assert st["median"] == 4.0 and st["groups"] == 7
    assert st["p10"] == pytest.approx(1.6) and st["p90"] == pytest.approx(6.4)


def test_host_info_fields():
    info = bench._host_info()
    assert set(info) == {"cpu_model", "nproc", "affinity"} and info["nproc"] >= 1


def test_whole_call_timed_by_bracketing_events():
    """With several launches per call the roofline uses the call's duration from events
    bracketing the timed steps (gaps between launches included), and the split still gives
    each kernel's share of the launches' summed durations."""
    w = workloads.WORKLOADS["long"]
    prof = {"kda_chunk_segbuild": (2, 0.30), "kda_combine": (2, 0.15), "kda_chunk_segout": (2, 0.31)}
    roof, _, kern = bench.kernel_record(w, prof, 2, call_ms=0.40)
    assert kern["avg_ms"] == 0.40 and kern["kernels_ms_per_step"] == pytest.approx(0.38)
    assert roof["achieved"] == pytest.approx(bench.algorithmic(w)[0] / 0.40e-3 / 1e9)
    assert sum(s["share"] for s in kern["split"]) == pytest.approx(1.0)


def test_committed_traffic_figures_match_the_current_kernel_sources():
    """Every committed HBM-traffic figure was taken on the kernel sources as they stand (the
    bench reports null for a stale one): a kernel edit without a fresh counter pass shows up
    here.  The figure itself sits within a few per cent of the algorithmic bytes (single
    launches) or above them by the segmented path's maps and second input pass."""
    import glob
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")))
    assert len(files) >= 7
    for f in files:
        rec = json.load(open(f))
        kernel = os.path.basename(f)[: -len("_" + rec["workload"] + "_traffic.json")]
        assert kernel in bench.KERNEL_SOURCES, f
        assert rec["kernel_source_sha"] == bench.source_sha(kernel), f"{f}: taken on other kernel sources"
        assert os.path.exists(os.path.join(ROOT, "profiles", rec["source"])), f
        ratio = rec["hbm_bytes_per_launch"] / rec.get("algorithmic_bytes", rec.get("algorithmic_bytes_per_launch"))
        assert (0.99 <= ratio <= 1.05) if kernel != "whole_call" else (1.5 <= ratio <= 2.2), (f, ratio)


def test_power_sample_reads_one_gpu_from_amdsmi_json():
    """The amd-smi JSON (`metric -p -c --json`, the layout printed on MI355X) gives the socket
    power and the lowest and highest GFX clock of the XCDs; a listing of several GPUs gives
    None, since the record could not say which one ran the call."""
    one = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 1400, "unit": "W"}, "gfx_voltage": "N/A"},
                         "clock": {"gfx_0": {"clk": {"value": 1729, "unit": "MHz"}, "clk_locked": "DISABLED"},
                                   "gfx_1": {"clk": {"value": 1847, "unit": "MHz"}},
                                   "gfx_2": {"clk": {"value": 1780, "unit": "MHz"}},
                                   "mem_0": {"clk": {"value": 2000, "unit": "MHz"}}}}]}
    assert bench.parse_amdsmi_metric(json.dumps(one)) == (1400.0, 1729.0, 1847.0)
    two = {"gpu_data": one["gpu_data"] * 2}
    assert bench.parse_amdsmi_metric(json.dumps(two)) is None
