"""KDA chunked-prefill benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config varlen|large|eqlen|long|varlen_padded|varlen_h64|tiny]
    python bench.py --config decode|decode_bf16|verify4        (the recurrent decode kernel)
    python bench.py --peak                                     (practical HBM and MFMA ceilings)

One step is one kda_prefill call over the whole workload (every kernel of the
hot path), with inputs already resident in HBM.  Before anything is timed the
call is checked against the float64 oracle on sampled chains (outputs poisoned
first; a second call into differently poisoned outputs must give the same
bits; a HIP-graph replay with a changed q is checked against the oracle on the
new q).  Then the step runs untimed for at least 0.2 s (`settle`: the GPU
returns to steady clocks after the host-side oracle), W warm-up steps, and K
timed steps: `value` is their back-to-back ("pipelined") rate.  `roofline` and
`mfma` come from HIP events on the launch stream over those K steps: around
the one launch of a single-segment plan (the library's own events), or
bracketing the K steps when a call makes several launches (segment build,
COMBINE and segment output on a segmented plan; events around each of them
would add gaps of their own), with the per-kernel split in `kernel.split` from
a second, profiled pass.  `timing_modes` gives the three modes of
the cudnn-frontend KDA PR (pipelined, per call, HIP graph of 8 calls), each
over 7 timing groups as median / p10 / p90.  `cpu_baseline` is the float64
oracle on the host's cores (and on one thread) over a bounded sample.  The
default (varlen, the H = 32 workload of the headline metric) also measures the
large workload (B=16, H=64, T=8192; the roofline workload) the same way, in
`large`, and the two segmented-plan workloads (eqlen: B=2, H=16, T=4096; long:
B=1, H=8, T=65536) in `segmented`.  After the timings of varlen and large, `power`
holds the socket power and GFX clocks amd-smi reports while the same call runs
back to back for 1.5 s (null without amd-smi; `--no-power` skips it).  Prints
ONE JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded synthetic inputs; no step of the method)

METRIC = "KDA prefill tokens/sec at H=32,d=128 bf16; MFMA util % and HBM GB/s"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3


def algorithmic(w):
    """Bytes and flops the method itself must move / compute for workload w:
    per token-head q, k, v, out (D elements each in the I/O dtype), g (D fp32),
    beta (one fp32); per chain the initial and final fp32 D x D states.
    Flops per token-head: the three dense state contractions (6 D^2) plus the
    triangular in-chunk work (A, P, Ut, W, P U: 64 * 5 D)."""
    es = 2 if w.dtype == "bf16" else 4
    D, H = w.D, w.H
    th = w.tokens * H
    chains = w.n_seq * H
    per_th = 4 * D * es + D * 4 + 4
    bytes_ = th * per_th + chains * 2 * D * D * 4
    flops = th * (6 * D * D + 64 * 5 * D)
    return bytes_, flops, per_th


KERNEL_SOURCES = {"chunk_kernel": ("kda_chunk_pipe.hip", "kda_device.hpp"),
                  "decode_kernel": ("kda_decode.hip", "kda_device.hpp"),
                  # a segmented call: both chunk-kernel passes and COMBINE
                  "whole_call": ("kda_chunk_pipe.hip", "kda_combine.hip", "kda_device.hpp")}


def source_sha(kernel="chunk_kernel"):
    """Hash of the sources a kernel is built from: a traffic figure taken on other
    sources is stale."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_delta_rule_38_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(config, kernel="chunk_kernel"):
    """HBM bytes per launch of the kernel (per call for "whole_call") from the committed
    rocprofv3 PMC summary, or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _host_info():
    """Host CPU facts for the baseline record: the model name, the logical CPU count and the
    CPUs this process may run on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": affinity}


def _gather_chains(x, w, picked):
    """The picked (sequence, head) chains as one packed float64-ready problem with H = 1."""
    import numpy as np
    import torch
    qs, ks, vs, gs, bs, ss, lens = [], [], [], [], [], [], []
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu()
    for n, h in picked:
        if cu is None:
            sl = lambda t: t[n, :, h]
        else:
            a, b = int(cu[n]), int(cu[n + 1])
            sl = lambda t: t[a:b, h]
        qs.append(sl(x["q"]).cpu()); ks.append(sl(x["k"]).cpu()); vs.append(sl(x["v"]).cpu())
        gs.append(sl(x["g"]).cpu()); bs.append(sl(x["beta"]).cpu())
        ss.append(x["initial_state"][n, h].cpu() if x["initial_state"] is not None else torch.zeros(w.D, w.D))
        lens.append(w.lengths[n])
    cat = lambda lst: torch.cat(lst)[:, None]
    cuh = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return (cat(qs), cat(ks), cat(vs), cat(gs), cat(bs), torch.stack(ss)[:, None]), cuh, int(sum(lens))


def cpu_baseline(x, w, budget_s):
    """The float64 oracle (C, OpenMP over chains) on a bounded sample of the workload's
    chains, on the host's cores (OMP_NUM_THREADS when set, else every logical CPU), and
    on one thread over a smaller sample; tokens/s scaled to the whole workload's H."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    per_th = 7.0 * w.D * w.D             # ~1.5 GFLOP/s per core for the scalar fp64 loop

    def pick(seconds, nthreads, seed):
        target_th = seconds * nthreads * 1.5e9 / per_th
        rng = np.random.default_rng(seed)
        order = [(n, h) for n in range(w.n_seq) for h in range(w.H) if w.lengths[n]]
        rng.shuffle(order)
        picked, th = [], 0
        for n, h in order:
            if th >= target_th:
                break
            picked.append((n, h))
            th += w.lengths[n]
        return picked

    picked = pick(budget_s, threads, 0)
    args, cuh, token_heads = _gather_chains(x, w, picked)
    t = time.perf_counter()
    _, _, used = oracle.run_c(*args, cuh, threads=threads, return_threads=True)
    dt = time.perf_counter() - t
    one = pick(max(1.0, budget_s / 4), 1, 1)
    args1, cuh1, th1 = _gather_chains(x, w, one)
    t = time.perf_counter()
    oracle.run_c(*args1, cuh1, threads=1)
    dt1 = time.perf_counter() - t
    rec = {"value": token_heads / w.H / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"{len(picked)} of {w.n_seq * w.H} (sequence, head) chains, {token_heads} token-heads, "
                     f"float64 C recurrence, {dt:.1f} s on {used} threads; tokens/s = token-heads / H / seconds",
           "one_thread": {"value": th1 / w.H / dt1, "unit": "tokens/s",
                          "sample": f"{len(one)} chains, {th1} token-heads, {dt1:.1f} s"}}
    rec.update(_host_info())
    return rec


def work_balance(w, cus=256, chunk=32):
    """How evenly the single-segment plan loads the CUs: one workgroup runs each
    (sequence, head) chain start to end, chunk after chunk, and a workgroup starts on the
    first CU to free up, in launch order -- longest sequence first when the library orders
    them (packed, more chains than CUs, at most 512 sequences).  The makespan is simulated;
    occupancy_bound = mean chunks per busy CU / makespan is the fraction of the roofline
    that the imbalance alone leaves."""
    import heapq
    chunks = [-(-L // chunk) for L in w.lengths]
    chains = w.n_seq * w.H
    order = list(range(w.n_seq))
    longest_first = (not w.dense) and chains > cus and 1 < w.n_seq <= 512
    if longest_first:
        order.sort(key=lambda n: (-chunks[n], n))
    free = [0] * min(cus, chains) if chains else []
    heapq.heapify(free)
    for n in order:
        for _ in range(w.H):
            heapq.heappush(free, heapq.heappop(free) + chunks[n])
    makespan = max(free) if free else 0
    total = sum(chunks) * w.H
    per_cu = total / min(cus, chains) if chains else 0.0
    return {"chains": chains, "chunk_tokens": chunk, "longest_chain_chunks": max(chunks) if chunks else 0,
            "order": "longest-first" if longest_first else "launch", "makespan_chunks": makespan,
            "mean_chunks_per_cu": per_cu, "occupancy_bound": (per_cu / makespan) if makespan else None}


def sample_chains(w, count, seed=0):
    """(sequence, head) chains the oracle checks: the first and the last, the chains on either
    side of the 2^31-byte offset of g (the first whose g rows start at or past it and the
    last wholly below it, where 32-bit byte offsets would wrap) and the chain of the highest
    g offset, then seeded random ones up to `count`."""
    import numpy as np
    H, D = w.H, w.D
    def g_range(n, h):          # byte range of chain (n, h) in a contiguous fp32 g
        if w.dense:
            T = w.lengths[0]
            lo = ((n * T) * H + h) * D * 4
            hi = ((n * T + T - 1) * H + h) * D * 4 + D * 4
        else:
            t0 = int(sum(w.lengths[:n]))
            lo = (t0 * H + h) * D * 4
            hi = ((t0 + max(w.lengths[n], 1) - 1) * H + h) * D * 4 + D * 4
        return lo, hi
    live = [(n, h) for n in range(w.n_seq) for h in range(H) if w.lengths[n]]
    chains = [live[0], live[-1]]
    ranges = {c: g_range(*c) for c in live}
    above = [c for c in live if ranges[c][0] >= 1 << 31]
    below = [c for c in live if ranges[c][0] < 1 << 31]
    if above:
        chains.append(min(above, key=lambda c: ranges[c][0]))
        chains.append(max(below, key=lambda c: ranges[c][0]))
    chains.append(max(live, key=lambda c: ranges[c][1]))
    rng = np.random.default_rng(seed)
    out = list(dict.fromkeys(chains))
    while len(out) < min(count, len(live)):
        c = live[int(rng.integers(len(live)))]
        if c not in out:
            out.append(c)
    return out


def chain_errors(x, w, out, fin, chains, q=None):
    """Worst rel-L2 (out, final state) against the oracle over the given chains."""
    import numpy as np
    import oracle
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu()
    q_src = x["q"] if q is None else q
    worst_o = worst_s = 0.0
    for n, h in chains:
        if cu is None:
            sl = lambda t: t[n, :, h:h + 1]
        else:
            a, b = int(cu[n]), int(cu[n + 1])
            sl = lambda t: t[a:b, h:h + 1]
        s0 = None if x["initial_state"] is None else x["initial_state"][n:n + 1, h:h + 1].cpu()
        qq = sl(q_src).cpu()
        o_ref, s_ref = oracle.run_c(qq, sl(x["k"]).cpu(), sl(x["v"]).cpu(), sl(x["g"]).cpu(), sl(x["beta"]).cpu(),
                                    s0, np.array([0, qq.shape[0]]))
        og = sl(out).float().cpu().numpy().reshape(o_ref.shape)
        sg = fin[n:n + 1, h:h + 1].float().cpu().numpy()
        if not (np.isfinite(og).all() and np.isfinite(sg).all()):
            return float("inf"), float("inf")
        worst_o = max(worst_o, oracle.rel_l2(og, o_ref) if o_ref.size else 0.0)
        worst_s = max(worst_s, oracle.rel_l2(sg, s_ref))
    return worst_o, worst_s


def bits_equal(a, b):
    import torch
    view = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    return bool(torch.equal(view(a), view(b)))


def pre_timing_checks(kda, x, w, out, fin, chains):
    """Correctness before anything is timed (the method of the cudnn-frontend KDA PR's review:
    an fp64 oracle, poisoned outputs and a changed-q replay):
      1. outputs poisoned with NaN, one call, the sampled chains against the float64 oracle;
      2. outputs poisoned with another pattern, one more call: the same bits as (1);
      3. kda_prefill_ws captured in a HIP graph over a q buffer, the buffer refilled with a
         new q, the graph replayed: its sampled chains against the oracle on the new q."""
    import torch
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    out.fill_(float("nan"))
    fin.fill_(float("nan"))
    kda.prefill(*args, out=out, final_state=fin)
    torch.cuda.synchronize()
    eo, es = chain_errors(x, w, out, fin, chains)
    tol = 5e-3 if w.dtype == "bf16" else 1e-4
    out2 = torch.full_like(out, -3.0e38)
    fin2 = torch.full_like(fin, 7.0)
    kda.prefill(*args, out=out2, final_state=fin2)
    torch.cuda.synchronize()
    repeat_bits = bits_equal(out, out2) and bits_equal(fin, fin2)
    # changed-q replay of a captured call
    qbuf = x["q"].clone()
    ws_bytes = kda.workspace_size(qbuf, *args[1:], out=out2, final_state=fin2)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=out.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.prefill(qbuf, *args[1:], out=out2, final_state=fin2, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.prefill(qbuf, *args[1:], out=out2, final_state=fin2, workspace=ws)
    gen = torch.Generator(device=out.device).manual_seed(12345)
    newq = torch.randn(qbuf.shape, generator=gen, device=out.device, dtype=torch.float32)
    qbuf.copy_((newq / torch.linalg.vector_norm(newq, dim=-1, keepdim=True)).to(qbuf.dtype))
    del newq
    out2.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    ro, rs = chain_errors(x, w, out2, fin2, chains[:4], q=qbuf)
    del graph, qbuf, out2, fin2, ws
    torch.cuda.empty_cache()
    ok = eo <= tol and es <= tol and repeat_bits and ro <= tol and rs <= tol
    rec = {"oracle_chains": len(chains), "rel_l2_out_max": eo, "rel_l2_state_max": es, "tolerance": tol,
           "poisoned_repeat_bit_identical": repeat_bits, "changed_q_graph_replay": {"chains": min(4, len(chains)),
           "rel_l2_out_max": ro, "rel_l2_state_max": rs}}
    if not ok:
        raise SystemExit(f"correctness checks failed before timing: {json.dumps(rec)}")
    return rec


DECODE_METRIC = "KDA decode tokens/sec at H=32,d=128 bf16 against a state pool; HBM GB/s"


def decode_algorithmic(w):
    """Bytes the decode method must move per call: every request's state slot read
    and written back (pool dtype), q, k, v, out (bf16) and g (fp32), beta (fp32) per
    token-head, and the slot index; flops: 7 D^2 per token-head."""
    es = 2 if w.pool_dtype == "bf16" else 4
    th = w.R * w.T * w.H
    bytes_ = w.R * w.H * 2 * w.D * w.D * es + th * (4 * w.D * 2 + w.D * 4 + 4) + w.R * 4
    return bytes_, th * 7 * w.D * w.D


def decode_main(a, w):
    import numpy as np
    import torch
    import gated_delta_rule_38_amd as kda
    import oracle
    import workloads
    dev = torch.device("cuda:0")
    x = workloads.make_decode_inputs(w, device=dev)
    out = torch.empty_like(x["v"])
    step = lambda pool: kda.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, x["idx"], None, out=out)
    # correctness gate on a copy of the pool: every request against the float64 oracle
    pool0 = x["pool"].clone()
    step(pool0)
    torch.cuda.synchronize()
    idx = x["idx"].cpu().numpy()
    cat = lambda t: t.cpu().double().reshape(w.R * w.T, w.H, -1) if t.dim() == 4 else t.cpu().double().reshape(w.R * w.T, w.H)
    s0 = x["pool"].cpu().double()[idx]
    cu = np.arange(w.R + 1, dtype=np.int64) * w.T
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(16, os.cpu_count() or 1)
    t = time.perf_counter()
    o_ref, s_ref, used = oracle.run_c(cat(x["q"]), cat(x["k"]), cat(x["v"]), cat(x["g"]), cat(x["beta"]), s0, cu,
                                      threads=threads, return_threads=True)
    dt = time.perf_counter() - t
    eo = oracle.rel_l2(out.float().cpu().numpy().reshape(o_ref.shape), o_ref)
    es = oracle.rel_l2(pool0.float().cpu().numpy()[idx], s_ref)
    if not max(eo, es) <= 5e-3:
        raise SystemExit(f"correctness gate failed: rel-L2 out {eo:.3e} state {es:.3e}")
    pool = x["pool"]
    settle(lambda: step(pool))
    for _ in range(a.warmup):
        step(pool)
    torch.cuda.synchronize()
    kda.profile_read()
    kda.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(pool)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kda.profile_enable(False)
    k_ms, k_n = kda.profile_read("kda_decode")
    kern_ms = k_ms / max(1, k_n)
    bytes_, flops = decode_algorithmic(w)
    achieved = bytes_ / (kern_ms * 1e-3) / 1e9
    rec = {
        "metric": DECODE_METRIC, "value": w.tokens * a.steps / (t1 - t0), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": (t1 - t0) / a.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded; see workloads.py)",
        "config": w.describe(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profile(w.name, "decode_kernel")},
        "kernel": {"name": "kda_decode", "avg_ms": kern_ms, "launches_per_step": k_n // max(1, a.steps),
                   "algorithmic_bytes_per_launch": bytes_, "flops_per_launch": flops,
                   "kernel_source_sha": source_sha("decode_kernel")},
        "correctness": {"rel_l2_out": eo, "rel_l2_state": es},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = {"value": w.tokens / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
                               "sample": f"all {w.R} requests x {w.H} heads, float64 C recurrence from the pool "
                                         f"slots, {dt:.2f} s (the correctness gate's run)"}
    print(json.dumps(rec))


def _stats(vals):
    import numpy as np
    v = np.asarray(vals, dtype=np.float64)
    return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)), "p90": float(np.percentile(v, 90)),
            "groups": len(vals)}


def timing_modes(kda, x, w, out, fin, steps, groups=7, calls=8):
    """The three timing modes the cudnn-frontend KDA PR quotes, each over `groups` timing
    groups, as median / p10 / p90 of the per-call milliseconds:
      pipelined -- `steps` calls back to back, timed by events on the stream around the group;
      per_call  -- `calls` calls each synchronised (host dispatch included), the group's median;
      graph     -- `calls` kda_prefill_ws launches captured in one HIP graph, replayed back to back
                   max(1, steps // calls) times per group (so that a group holds about as many calls
                   as a pipelined one and times neither the first launch nor an idle GPU's clock)."""
    import statistics
    import torch
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    pipelined, per_call, per_graph = [], [], []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            kda.prefill(*args, out=out, final_state=fin)
        e1.record()
        torch.cuda.synchronize()
        pipelined.append(e0.elapsed_time(e1) / steps)
        one = []
        for _ in range(calls):
            t = time.perf_counter()
            kda.prefill(*args, out=out, final_state=fin)
            torch.cuda.synchronize()
            one.append((time.perf_counter() - t) * 1e3)
        per_call.append(statistics.median(one))
    ws_bytes = kda.workspace_size(*args, out=out, final_state=fin)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=out.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.prefill(*args, out=out, final_state=fin, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            kda.prefill(*args, out=out, final_state=fin, workspace=ws)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // calls)
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per_graph.append(e0.elapsed_time(e1) / (calls * reps))
    return {"pipelined_ms": _stats(pipelined), "per_call_ms": _stats(per_call), "graph_ms": _stats(per_graph),
            "graph_calls": calls, "graph_replays_per_group": reps, "pipelined_calls_per_group": steps,
            "per_call_calls_per_group": calls}


def parse_amdsmi_metric(text):
    """(socket power W, lowest GFX clock MHz, highest GFX clock MHz) from the JSON of
    `amd-smi metric -p -c --json` for a box that shows exactly one GPU; None otherwise."""
    d = json.loads(text)
    gpus = d.get("gpu_data") if isinstance(d, dict) else d
    if not isinstance(gpus, list) or len(gpus) != 1:
        return None
    g = gpus[0]
    pw = float(g["power"]["socket_power"]["value"])
    clks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
            if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
    if not clks:
        return None
    return pw, min(clks), max(clks)


def power_sample(step, seconds=1.5):
    """Socket power and GFX clocks while `step` runs back to back for `seconds` (after the timed
    steps, so the timing is not affected): `amd-smi metric -p -c --json` polled from a second
    thread, medians over the samples taken after the first 0.4 s.  None when amd-smi is absent,
    fails or reports anything but one GPU: the record is context, not a measurement of ours."""
    import shutil
    import statistics
    import subprocess
    import threading
    import torch
    if seconds <= 0 or shutil.which("amd-smi") is None:
        return None
    samples, stop = [], threading.Event()

    def poll():
        t_start = time.perf_counter()
        while not stop.is_set():
            try:
                p = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=5)
                v = parse_amdsmi_metric(p.stdout)
            except Exception:
                v = None
            if v is None:
                samples.append(None)
                return
            if time.perf_counter() - t_start > 0.4:
                samples.append(v)
            stop.wait(0.2)

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds and th.is_alive():
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=10)
    if not samples or any(v is None for v in samples):
        return None
    return {"socket_power_w": statistics.median(v[0] for v in samples),
            "gfx_clock_mhz_lowest_xcd": statistics.median(v[1] for v in samples),
            "gfx_clock_mhz_highest_xcd": statistics.median(v[2] for v in samples),
            "samples": len(samples), "seconds": seconds, "source": "amd-smi metric -p -c"}


def settle(step, seconds=0.2):
    """Untimed steps for at least `seconds` of wall time (GPU back to steady state)."""
    import torch
    t = time.perf_counter()
    while time.perf_counter() - t < seconds:
        step()
        torch.cuda.synchronize()


def kernel_record(w, prof, steps, call_ms=None):
    """Roofline, matrix-core rate and per-kernel split of one step from the library's own
    HIP events: {kernel name: (launches, summed ms)} over `steps` steps.  One launch: its
    average duration.  Several launches (segment build, COMBINE and segment output on a
    segmented plan): the whole call, `call_ms` (events bracketing the timed steps, the gaps
    between launches included) when given, else the launches' summed durations; the split
    gives each kernel's share of the summed durations."""
    bytes_, flops, per_th = algorithmic(w)
    kernels_ms = sum(ms for _, ms in prof.values()) / steps
    launches = sum(n for n, _ in prof.values()) // steps
    total_ms = kernels_ms if (launches == 1 or call_ms is None) else call_ms
    achieved = bytes_ / (total_ms * 1e-3) / 1e9
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    tflops = flops / (total_ms * 1e-3) / 1e12
    split = [{"name": name, "launches_per_step": n // steps, "avg_ms": ms / max(1, n), "ms_per_step": ms / steps,
              "share": (ms / steps) / kernels_ms} for name, (n, ms) in prof.items()]
    tr = traffic_from_profile(w.name) if launches == 1 else traffic_from_profile(w.name, "whole_call")
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": tr}
    mfma = {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s", "frac": tflops / mfma_peak,
            "flops_per_call": flops,
            # the most the matrix cores can be fed when the call moves its algorithmic bytes at the
            # HBM peak (flops / bytes x 8 TB/s)
            "frac_ceiling_at_hbm_peak": (flops / bytes_) * HBM_PEAK_GBS * 1e9 / (mfma_peak * 1e12)}
    kern = {"name": "kda_chunk" if launches == 1 else "whole call", "scope": "one launch" if launches == 1 else
            f"{launches} launches per call" + (", timed by events bracketing the steps" if call_ms else ""),
            "avg_ms": total_ms, "kernels_ms_per_step": kernels_ms, "launches_per_step": launches,
            "algorithmic_bytes_per_launch" if launches == 1 else "algorithmic_bytes_per_call": bytes_,
            "bytes_per_token_head": per_th, "kernel_source_sha": source_sha("chunk_kernel"), "split": split}
    return roof, mfma, kern


def prefill_record(kda, w, steps, warmup, groups, checks_count, power_seconds=0.0):
    """Everything measured on one prefill workload: the pre-timing checks, the K timed steps
    (wall clock, and the library's HIP events for the roofline), and the timing groups."""
    import torch
    dev = torch.device("cuda:0")
    x = workloads.make_inputs(w, device=dev)
    out = torch.empty_like(x["v"])
    fin = torch.empty((w.n_seq, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    step = lambda: kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"],
                               out=out, final_state=fin)
    torch.cuda.synchronize()
    checks = pre_timing_checks(kda, x, w, out, fin, sample_chains(w, checks_count))
    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # launches per call (a one-step profile)
    kda.profile_read()
    kda.profile_enable(True)
    step()
    torch.cuda.synchronize()
    kda.profile_enable(False)
    launches = sum(n for n, _ in kda.profile_read_kernels().values())
    settle(step, 0.05)
    if launches == 1:
        # one launch per call: the library's HIP events around every launch of the timed steps
        kda.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kda.profile_enable(False)
        prof = kda.profile_read_kernels()
        roof, mfma, kern = kernel_record(w, prof, steps)
    else:
        # several launches per call: events around every launch would add their own gaps between
        # the launches, so the timed steps are bracketed by two events on the launch stream (the
        # whole call, gaps included); the per-kernel split comes from a second, profiled pass
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        call_ms = e0.elapsed_time(e1) / steps
        kda.profile_enable(True)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        kda.profile_enable(False)
        prof = kda.profile_read_kernels()
        roof, mfma, kern = kernel_record(w, prof, steps, call_ms=call_ms)
    modes = timing_modes(kda, x, w, out, fin, steps, groups)
    power = power_sample(step, power_seconds)
    return {"x": x, "elapsed": t1 - t0, "roofline": roof, "mfma": mfma, "kernel": kern, "checks": checks,
            "timing_modes": modes, "power": power}


def peak_main(a):
    """The practical ceilings: the HBM stream with the chunk kernel's read/write mix, sized
    like the large workload's traffic, and the bf16 MFMA loop, each timed over 7 groups."""
    import torch
    import gated_delta_rule_38_amd as kda
    kda.load_library()
    dev = torch.device("cuda:0")
    bytes_large = algorithmic(workloads.WORKLOADS["large"])[0]
    n16 = int(bytes_large // (6 * 16))
    ins = [torch.full((n16 * 4,), i + 1, dtype=torch.int32, device=dev) for i in range(5)]
    out = torch.empty((n16 * 4,), dtype=torch.int32, device=dev)
    kda.peak_stream(ins, out)
    torch.cuda.synchronize()
    assert int(out[0]) == (1 ^ 2 ^ 3 ^ 4 ^ 5) and int(out[-1]) == (1 ^ 2 ^ 3 ^ 4 ^ 5)
    reps, groups = 5, 7
    gbs = []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            kda.peak_stream(ins, out)
        e1.record()
        torch.cuda.synchronize()
        gbs.append(6 * n16 * 16 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9)
    del ins, out
    torch.cuda.empty_cache()
    wgs, iters = 256 * 2, 4000
    mo = torch.zeros(wgs * 4, device=dev)
    kda.peak_mfma(mo, wgs, iters)
    torch.cuda.synchronize()
    tf = []
    flops = wgs * 4 * iters * 8 * 32768
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kda.peak_mfma(mo, wgs, iters)
        e1.record()
        torch.cuda.synchronize()
        tf.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    st, mf = _stats(gbs), _stats(tf)
    print(json.dumps({
        "metric": "practical ceilings of one MI355X: HBM stream at the chunk kernel's 5:1 read/write mix; bf16 MFMA loop",
        "stream": {"bytes_per_launch": 6 * n16 * 16, "read_write_ratio": 5, "GB_s": st,
                   "frac_of_peak_median": st["median"] / HBM_PEAK_GBS, "peak": HBM_PEAK_GBS},
        "mfma_bf16": {"flops_per_launch": flops, "workgroups": wgs, "TFLOP_s": mf,
                      "frac_of_peak_median": mf["median"] / MFMA_BF16_PEAK_TFLOPS, "peak": MFMA_BF16_PEAK_TFLOPS}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="varlen")
    ap.add_argument("--groups", type=int, default=7, help="timing groups per mode (median / p10 / p90)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the large-workload sub-record of the default run")
    ap.add_argument("--no-segmented", action="store_true",
                    help="skip the segmented-plan sub-records (eqlen, long) of the default run")
    ap.add_argument("--peak", action="store_true", help="measure the practical HBM and MFMA ceilings instead")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the 1.5 s amd-smi power and clock sample after the varlen and large timings")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="instead of the bench, copy this many MiB device-to-device 5 times (PMC calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_38_amd as kda
    kda.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs the GPU")
    dev = torch.device("cuda:0")

    if a.copy_calib:
        n = a.copy_calib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_each_way": n * 4, "copies": 5}))
        return
    if a.peak:
        return peak_main(a)
    if a.config in workloads.DECODE_WORKLOADS:
        return decode_main(a, workloads.DECODE_WORKLOADS[a.config])
    w = workloads.WORKLOADS[a.config]
    r = prefill_record(kda, w, a.steps, a.warmup, a.groups, 16 if w.name in ("varlen", "large") else 8,
                       0.0 if a.no_power else 1.5)
    elapsed = r["elapsed"]
    rec = {
        "metric": METRIC, "value": w.tokens * a.steps / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": elapsed / a.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded; see workloads.py)",
        "config": w.describe(), "roofline": r["roofline"], "mfma": r["mfma"], "kernel": r["kernel"],
        "correctness": r["checks"],
        "work_balance": work_balance(w) if r["kernel"]["launches_per_step"] == 1 else None,
        "timing_modes": r["timing_modes"],
        "power": r["power"],
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(r["x"], w, a.cpu_budget)
    r = None                # the sub-records below allocate their own inputs
    if a.config == "varlen" and not a.no_large:
        # the roofline workload (B=16, H=64, T=8192), timed the same way in the same run
        torch.cuda.empty_cache()
        wl = workloads.WORKLOADS["large"]
        steps_l = max(3, min(a.steps, 10))
        rl = prefill_record(kda, wl, steps_l, min(a.warmup, 5), a.groups, 16, 0.0 if a.no_power else 1.5)
        rec["large"] = {"config": wl.describe(), "steps": steps_l, "ms_per_step": rl["elapsed"] / steps_l * 1e3,
                        "tokens_per_s": wl.tokens * steps_l / rl["elapsed"], "roofline": rl["roofline"],
                        "mfma": rl["mfma"], "kernel": rl["kernel"], "correctness": rl["checks"],
                        "timing_modes": rl["timing_modes"], "power": rl["power"]}
    if a.config == "varlen" and not a.no_segmented:
        # the workloads with too few chains to fill the CUs, on segmented plans (map pass, COMBINE,
        # segment outputs): whole-call roofline and the per-kernel split, timed the same way
        rec["segmented"] = {}
        rl = None
        for name in ("eqlen", "long"):
            rs = None
            torch.cuda.empty_cache()
            ws = workloads.WORKLOADS[name]
            rs = prefill_record(kda, ws, a.steps, min(a.warmup, 5), a.groups, 8)
            rec["segmented"][name] = {
                "config": ws.describe(), "steps": a.steps, "ms_per_step": rs["elapsed"] / a.steps * 1e3,
                "tokens_per_s": ws.tokens * a.steps / rs["elapsed"], "roofline": rs["roofline"], "mfma": rs["mfma"],
                "kernel": rs["kernel"], "correctness": rs["checks"], "timing_modes": rs["timing_modes"]}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
