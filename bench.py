"""KDA chunked-prefill benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config varlen|large|eqlen|long|varlen_padded|varlen_h64|tiny]
    python bench.py --config decode|decode_bf16|verify4        (the recurrent decode kernel)

One step is one kda_prefill call over the whole workload (every kernel of the
hot path), with inputs already resident in HBM; `value` is the back-to-back
("pipelined") rate, and `timing_modes` adds per-call (synchronised, host
dispatch included) and HIP-graph times.  The correctness gate runs the oracle
on the host while the GPU idles; afterwards the step runs untimed for at least
0.2 s (`settle`) so that the GPU is back in its steady state before the W
warm-up steps and the K timed steps (with only a few steps of warm-up, the
first milliseconds after the idle ran ~13% slower on the varlen workload).  Prints ONE JSON line:
throughput in tokens/s, the roofline of the dominant kernel (its duration from
HIP events recorded by the library on the launch stream over the timed region),
and the float64 oracle timed on the host cores on a bounded sample of the same
workload.  Correctness is checked against the oracle on sampled chains before
anything is timed.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

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
                  "decode_kernel": ("kda_decode.hip", "kda_device.hpp")}


def source_sha(kernel="chunk_kernel"):
    """Hash of the sources a kernel is built from: a traffic figure taken on other
    sources is stale."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_delta_rule_38_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(config, kernel="chunk_kernel"):
    """HBM bytes per launch of the kernel from the committed rocprofv3 PMC
    summary, or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(x, w, budget_s):
    """The float64 oracle (C, OpenMP over chains) on a bounded sample of the
    workload's chains; returns tokens/s scaled to the whole workload's H."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(16, os.cpu_count() or 1)
    # ~1.5 GFLOP/s per core for the scalar fp64 loop: pick chains worth ~budget_s
    per_th = 7.0 * w.D * w.D
    target_th = budget_s * threads * 1.5e9 / per_th
    rng = np.random.default_rng(0)
    order = [(n, h) for n in range(w.n_seq) for h in range(w.H)]
    rng.shuffle(order)
    picked, th = [], 0
    for n, h in order:
        if th >= target_th:
            break
        picked.append((n, h))
        th += w.lengths[n]
    # gather the picked chains as one packed problem with H = 1
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
    s0 = torch.stack(ss)[:, None]
    cuh = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    args = (cat(qs), cat(ks), cat(vs), cat(gs), cat(bs), s0)
    t = time.perf_counter()
    _, _, used = oracle.run_c(*args, cuh, threads=threads, return_threads=True)
    dt = time.perf_counter() - t
    token_heads = int(sum(lens))
    return {"value": token_heads / w.H / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{len(picked)} of {w.n_seq * w.H} (sequence, head) chains, {token_heads} token-heads, "
                      f"float64 C recurrence, {dt:.1f} s; tokens/s = token-heads / H / seconds"}


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


def correctness_gate(kda, x, w, out, fin):
    import numpy as np
    import oracle
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu()
    worst = 0.0
    for n, h in [(0, 0), (w.n_seq - 1, w.H - 1)]:
        if cu is None:
            sl, osl = (lambda t: t[n, :, h:h + 1]), (lambda t: t[n, :, h:h + 1])
        else:
            a, b = int(cu[n]), int(cu[n + 1])
            sl = osl = (lambda t: t[a:b, h:h + 1])
        s0 = None if x["initial_state"] is None else x["initial_state"][n:n + 1, h:h + 1].cpu()
        q = sl(x["q"]).cpu()
        o_ref, s_ref = oracle.run_c(q, sl(x["k"]).cpu(), sl(x["v"]).cpu(), sl(x["g"]).cpu(), sl(x["beta"]).cpu(),
                                    s0, np.array([0, q.shape[0]]))
        eo = oracle.rel_l2(osl(out).float().cpu().numpy().reshape(o_ref.shape), o_ref)
        es = oracle.rel_l2(fin[n:n + 1, h:h + 1].cpu().numpy(), s_ref)
        worst = max(worst, eo, es)
    tol = 5e-3 if w.dtype == "bf16" else 1e-4
    if not worst <= tol:
        raise SystemExit(f"correctness gate failed: sampled rel-L2 {worst:.3e} > {tol}")
    return worst


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


def timing_modes(kda, x, w, out, fin, calls=8, reps=5):
    """The other two timing modes the cudnn-frontend KDA PR quotes beside the
    back-to-back one: per call (each call synchronised, host dispatch included) and a
    HIP graph of `calls` kda_prefill_ws launches replayed as one.  Medians in ms."""
    import statistics
    import torch
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    per_call = []
    for _ in range(calls * reps):
        t = time.perf_counter()
        kda.prefill(*args, out=out, final_state=fin)
        torch.cuda.synchronize()
        per_call.append((time.perf_counter() - t) * 1e3)
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
    per_graph = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per_graph.append(e0.elapsed_time(e1) / calls)
    return {"per_call_ms": statistics.median(per_call), "graph_ms": statistics.median(per_graph),
            "graph_calls": calls}


def settle(step, seconds=0.2):
    """Untimed steps for at least `seconds` of wall time (GPU back to steady state)."""
    import torch
    t = time.perf_counter()
    while time.perf_counter() - t < seconds:
        step()
        torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="varlen")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="instead of the bench, copy this many MiB device-to-device 5 times (PMC calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_38_amd as kda
    import workloads
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

    if a.config in workloads.DECODE_WORKLOADS:
        return decode_main(a, workloads.DECODE_WORKLOADS[a.config])
    w = workloads.WORKLOADS[a.config]
    x = workloads.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    step = lambda: kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"],
                               out=out, final_state=fin)
    out = torch.empty_like(x["v"])
    fin = torch.empty((w.n_seq, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    step()
    torch.cuda.synchronize()
    gate = correctness_gate(kda, x, w, out, fin)
    settle(step)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    kda.profile_read()            # drop anything recorded so far
    kda.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kda.profile_enable(False)
    chunk_ms, chunk_n = kda.profile_read("kda_chunk")
    elapsed = t1 - t0
    ms_step = elapsed / a.steps * 1e3
    tokens_s = w.tokens * a.steps / elapsed

    bytes_, flops, per_th = algorithmic(w)
    launches_per_step = max(1, chunk_n // a.steps)
    kern_ms = chunk_ms / max(1, chunk_n)                 # average chunk-kernel launch
    # algorithmic bytes of one chunk-kernel launch: the single-segment plan does
    # the whole workload in one launch
    bytes_launch = bytes_ / launches_per_step
    achieved = bytes_launch / (kern_ms * 1e-3) / 1e9
    tr = traffic_from_profile(a.config) if launches_per_step == 1 else None
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    tflops = flops / launches_per_step / (kern_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": tokens_s, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded; see workloads.py)",
        "config": w.describe(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": tr},
        "mfma": {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s", "frac": tflops / mfma_peak,
                 "flops_per_launch": flops / launches_per_step,
                 # the most the matrix cores can be fed when the launch moves its
                 # algorithmic bytes at the HBM peak (flops / bytes x 8 TB/s)
                 "frac_ceiling_at_hbm_peak": (flops / bytes_) * HBM_PEAK_GBS * 1e9 / (mfma_peak * 1e12)},
        "kernel": {"name": "kda_chunk", "avg_ms": kern_ms, "launches_per_step": launches_per_step,
                   "algorithmic_bytes_per_launch": bytes_launch, "bytes_per_token_head": per_th,
                   "kernel_source_sha": source_sha("chunk_kernel")},
        "correctness": {"sampled_rel_l2_max": gate},
        "work_balance": work_balance(w) if launches_per_step == 1 else None,
        "timing_modes": dict(timing_modes(kda, x, w, out, fin), pipelined_ms=ms_step),
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, w, a.cpu_budget)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
