#!/usr/bin/env python3
"""Throughput of the batch-invariant fused linear log-probability forward on
one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]
                    [--no-cpu-baseline] [--no-backward] [--no-det-gemm]
                    [--no-invariance-cost] [--no-shard-share] [--no-library-context]

One step is one full pass of the hot path over one batch: bilogp_partials
(fused bf16-MFMA projection + per-split online softmax) followed by
bilogp_merge (ascending split merge), i.e. exactly bilogp_forward_ex with a
caller workspace.  Inputs are synthetic, seeded, and resident in HBM before
timing starts.  W untimed warmup steps, then K timed steps between device
synchronisations.  HIP events recorded on the launch stream bracket each
kernel so the projection kernel's own average duration is measured live.

Prints ONE JSON line with the throughput (tokens/s), the roofline of the
projection kernel (bf16 MFMA bound) and the fp64 CPU oracle timed on a
bounded row sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s + TFLOP/s (MFMA %peak), linear-logp N=4096 H=4096 V=128256 bf16"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0

# L2-miss (fabric) bytes per launch of proj_lse_kernel on the headline workload, from
# two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by what the same
# counter reads for a plain 1 GiB device copy (x2.000 and x1.000).  These are the bytes
# the L2 exchanges with the memory side (the 256 MB Infinity Cache or HBM); no counter
# available on gfx950 separates the HBM share.  Keyed by projection_digest() of the code
# the counters were taken on (the kernel and its launch code, comments and whitespace
# stripped): any change to that code reports null.
MEASURED_TRAFFIC = {
    ("headline", "a64480087dff0507"): {"fetch_bytes": 6_356_370_368, "write_bytes": 22_868_176},
}
TRAFFIC_KIND = ("L2-miss (fabric) bytes per launch: FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                "served by the Infinity Cache or HBM - HBM bytes alone are not separable with "
                "the counters available on gfx950")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-det-gemm", action="store_true",
                    help="skip timing the deterministic GEMM (forward, dA, dB)")
    ap.add_argument("--no-shard-share", action="store_true",
                    help="skip timing one GPU's share of an 8-way vocabulary or row sharding")
    ap.add_argument("--no-library-context", action="store_true",
                    help="skip timing torch's matmul (hipBLASLt) and the unfused matmul + "
                         "logsumexp path at the workload's shape")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the deterministic backward")
    ap.add_argument("--no-invariance-cost", action="store_true",
                    help="skip timing the throughput split policy beside the invariant one")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other single-GPU configurations (medium, sweep, peaky)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the board clock / power sample under sustained load")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the workload the CPU oracle is timed on")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 device copies of MIB MiB (a plain copy kernel of known "
                         "size, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


def algorithmic_bytes(N, H, V, S, bias_bytes):
    """Bytes the forward must move at least once: W, hidden, targets, bias,
    the partials written and read back, target logits, and the outputs."""
    return (V * H * 2 + N * H * 2 + N * 8 + bias_bytes + 2 * N * S * 8 + 2 * N * 4 + 2 * N * 4)


def code_digest(*paths):
    """sha256 prefix of C++/HIP sources with comments and whitespace removed
    (concatenated in the order given): edits to comments alone keep it, any
    change to the code changes it."""
    import hashlib
    import re
    text = ""
    for path in paths:
        with open(path) as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def projection_digest():
    """code_digest of what decides the projection kernel's memory traffic: the
    kernel source and the host code that picks its launch (row blocks, split
    runs)."""
    csrc = os.path.join(ROOT, "invariant_linear_log_amd", "csrc")
    return code_digest(os.path.join(csrc, "proj_fwd.hip"), os.path.join(csrc, "bilogp_host.cpp"))


def measured_traffic(workload):
    rec = MEASURED_TRAFFIC.get((workload, projection_digest()))
    return None if rec is None else rec["fetch_bytes"] + rec["write_bytes"]


def time_forward(h, t, w, b, steps, warmup, stream):
    """Full forward steps (bilogp_partials + bilogp_merge, i.e. bilogp_forward_ex
    with a caller workspace) on resident inputs; HIP events on the launch stream
    around each kernel.  Returns per-step projection / merge / step times (ms)."""
    import torch
    import invariant_linear_log_amd as ila
    N = h.shape[0]
    V = w.shape[0]
    logp = torch.empty(N, dtype=torch.float32, device=h.device)
    lse = torch.empty(N, dtype=torch.float32, device=h.device)
    ws = ila.workspace_for(N, V, h.device)
    for _ in range(warmup):
        ila.bilogp_partials(h, w, t, b, ws, stream=stream)
        ila.bilogp_merge(t, ws, logp, lse, V, stream=stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        ila.bilogp_partials(h, w, t, b, ws, stream=stream)
        e[1].record(stream)
        ila.bilogp_merge(t, ws, logp, lse, V, stream=stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    proj = [e[0].elapsed_time(e[1]) for e in evs]
    merge = [e[1].elapsed_time(e[2]) for e in evs]
    step = [e[0].elapsed_time(e[2]) for e in evs]
    ok = bool(torch.all(torch.isfinite(lse))) and bool(torch.all(logp <= 0))
    return proj, merge, step, ok


def launch_plan(N, H, V):
    """The projection launch the library makes on this device: row-block height,
    splits per workgroup of the longest runs, workgroups over all launches, and
    the split schedule (where single splits begin, where the 128-token second
    launch begins; both = S when there is none)."""
    import torch
    import invariant_linear_log_amd as ila
    cu = ila.device_cu_count(torch.device("cuda:0"))
    inv = ila.BILOGP_SPLITS_INVARIANT
    rows, spg, wgs = ila.bilogp_launch_plan(N, H, V, inv, cu)
    sa, st = ila.bilogp_launch_schedule(N, H, V, inv, cu)
    return {"rows_per_block": rows, "splits_per_workgroup": spg, "workgroups": wgs,
            "split_a": sa, "split_t": st, "splits": ila.bilogp_num_vocab_splits(V),
            "compute_units": cu}


def config_legs(steps=10, warmup=3, names=("medium", "sweep", "peaky")):
    """The other single-GPU configurations, each timed like the headline (full
    forward step on resident inputs).  medium: N=512, H=1024, V=32000, fp32 bias;
    sweep: N=4096, H=4096, V=151936, bf16 bias (the bias kernel, a 128-column
    vocabulary tail); peaky: N=16384, H=8192, V=152064, hidden x8.  Targets are
    the workloads' own (for peaky the uniform half; which tile holds a row's
    target moves one 4-byte write, not the timing)."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    out = {}
    for name in names:
        inp = synth.make_inputs(name, device=dev)
        wl = inp["workload"]
        h = inp["hidden"].reshape(-1, wl.H).contiguous()
        t = inp["target"].reshape(-1).contiguous()
        w, b = inp["weight"], inp["bias"]
        torch.cuda.synchronize()
        proj, merge, step, ok = time_forward(h, t, w, b, steps, warmup, stream)
        flops = 2.0 * wl.N * wl.H * wl.V
        pm = sorted(proj)[len(proj) // 2]
        sm = sorted(step)[len(step) // 2]
        out[name] = {"N": wl.N, "H": wl.H, "V": wl.V, "bias": wl.bias,
                     "step_ms": sm, "proj_lse_ms": pm,
                     "merge_ms": sorted(merge)[len(merge) // 2],
                     "tokens_per_s": wl.N / sm * 1e3, "tflops": flops / sm / 1e9,
                     "proj_lse_tflops": flops / pm / 1e9,
                     "frac": flops / pm / 1e9 / PEAK_BF16_TFLOPS, "outputs_sane": ok,
                     "launch": launch_plan(wl.N, wl.H, wl.V)}
        del inp, h, t, w, b
        torch.cuda.empty_cache()
    return out


def clock_sample(run_step, seconds=3.0):
    """Board clock and power while the headline step runs back to back for a few
    seconds: `amd-smi metric` samples taken on a side thread (the timed region
    itself is shorter than one sample).  The GFX clock is averaged over the
    XCDs of each sample.  None if amd-smi is unavailable."""
    import shutil
    import subprocess
    import threading
    import torch
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run([exe, "metric", "-g", "0", "-p", "-c", "--json"],
                                   capture_output=True, text=True, timeout=10)
                d = json.loads(r.stdout)
                g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                clk = [v["clk"]["value"] for k, v in g["clock"].items()
                       if k.startswith("gfx_") and isinstance(v, dict)]
                samples.append((float(sum(clk)) / len(clk), float(g["power"]["socket_power"]["value"])))
            except Exception:  # pragma: no cover - a missing field skips the sample
                pass
    th = threading.Thread(target=sampler)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            run_step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if len(samples) < 2:
        return None
    warm = samples[1:]                 # the first sample may predate the load
    clks = [c for c, _ in warm]
    pw = [p for _, p in warm]
    cap = None
    try:
        import glob
        for f in glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_cap"):
            cap = int(open(f).read()) / 1e6
            break
    except Exception:  # pragma: no cover
        pass
    # a sample can land in the short idle gap of a host synchronisation: the
    # medians describe the loaded board, the means include such gaps
    return {"gfx_mhz_median": statistics.median(clks), "gfx_mhz_mean": sum(clks) / len(clks),
            "gfx_mhz_min": min(clks), "gfx_mhz_max": max(clks),
            "power_w_median": statistics.median(pw), "power_w_mean": sum(pw) / len(pw),
            "power_w_max": max(pw), "power_cap_w": cap,
            "samples": len(warm), "seconds": seconds,
            "source": "amd-smi metric -p -c during back-to-back headline steps"}


def invariance_cost(h, t, w, b, steps=10, warmup=3, repeats=3):
    """ms per full forward step under the invariant and the throughput split
    policies, at the workload's N and at its first 512 and 64 rows (fewer row
    blocks: the throughput policy then adds splits to fill the device).  The
    two policies alternate, `repeats` times, and each reports its fastest
    repeat, so neither is timed only on a board the other has warmed."""
    import torch
    import invariant_linear_log_amd as ila
    dev = h.device
    cu = ila.device_cu_count(dev)
    stream = torch.cuda.Stream(device=dev)
    res = {"cu_count": cu, "repeats": repeats}
    for n in (h.shape[0], 512, 64):
        hn, tn = h[:n].contiguous(), t[:n].contiguous()
        V = w.shape[0]
        logp = torch.empty(n, dtype=torch.float32, device=dev)
        lse = torch.empty(n, dtype=torch.float32, device=dev)
        modes = (("invariant", ila.BILOGP_SPLITS_INVARIANT),
                 ("throughput", ila.BILOGP_SPLITS_THROUGHPUT))
        wss = {name: ila.workspace_for(n, V, dev, name, cu) for name, _ in modes}
        for _ in range(repeats):
            for name, mode in modes:
                ws = wss[name]

                def run():
                    ila.bilogp_forward_mode(hn, w, tn, b, logp, lse, mode, cu, ws,
                                            stream=stream)
                for _ in range(warmup):
                    run()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(steps):
                    run()
                e1.record(stream)
                e1.synchronize()
                key = f"n{n}_{name}_ms"
                res[key] = min(res.get(key, float("inf")), e0.elapsed_time(e1) / steps)
                res[f"n{n}_{name}_splits"] = ila.bilogp_num_vocab_splits_mode(n, V, mode, cu)
    return res


def det_gemm_leg(steps=10, warmup=3, reps=5):
    """The deterministic GEMM (forward, dA, dB, and forward + dA + dB) at M = N = K
    = 4096 and at the three shapes of the page's own table (M x K x N = 128 x 128
    x 128, 256 x 512 x 512, 512 x 1024 x 1024), with torch's bf16 matmul
    (hipBLASLt, not deterministic by contract) beside them.  Per shape, the five
    runs alternate in `reps` rounds of `steps` calls; ms = median over the rounds."""
    import torch
    import invariant_linear_log_amd as ila
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    out = {"peak_tflops": PEAK_BF16_TFLOPS,
           "protocol": f"per shape, the runs alternate in {reps} rounds of {steps} calls after "
                       f"{warmup} warmup calls each; ms = median over the rounds"}
    for (M, N, K) in ((4096, 4096, 4096), (128, 128, 128), (256, 512, 512), (512, 1024, 1024)):
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        b = torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16)
        dc = torch.randn((M, N), generator=g, device=dev).to(torch.bfloat16)
        bt = b.t().contiguous()              # [K, N] once, outside the timed calls
        flops = 2.0 * M * N * K

        def fwd_bwd():
            ila.det_gemm(a, b)
            ila.det_gemm_da(dc, b)
            ila.det_gemm_db(a, dc)
        runs = {"fwd": lambda: ila.det_gemm(a, b), "da": lambda: ila.det_gemm_da(dc, b),
                "db": lambda: ila.det_gemm_db(a, dc), "fwd_bwd": fwd_bwd,
                "torch_matmul_fwd": lambda: torch.matmul(a, bt)}
        for fn in runs.values():
            for _ in range(warmup):
                fn()
        times = {name: [] for name in runs}
        for _ in range(reps):                    # the runs alternate, round by round
            for name, fn in runs.items():
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                e1.synchronize()
                times[name].append(e0.elapsed_time(e1) / steps)
        rec = {}
        for name, v in times.items():
            ms = statistics.median(v)
            f = 3 * flops if name == "fwd_bwd" else flops
            rec[name] = {"ms": ms, "ms_min": min(v), "tflops": f / ms / 1e9}
        rec["fwd"]["frac"] = rec["fwd"]["tflops"] / PEAK_BF16_TFLOPS
        out[f"M{M}_N{N}_K{K}"] = rec
    return out


def backward_leg(h, t, w, b, lse, steps=10, warmup=3):
    """The deterministic backward (bilogp_backward: softmax-gradient
    projection kernel, grad_hidden and grad_weight GEMMs, bias row sums) on
    the workload's own shapes with seeded upstream gradients; 6 N H V flops
    per call (z recomputed, then two products of the same size)."""
    import torch
    import invariant_linear_log_amd as ila
    import synth
    dev = h.device
    N, H = h.shape
    V = w.shape[0]
    up = synth.make_upstream_grads(N, 12, device=dev)
    gh = torch.empty((N, H), dtype=torch.float32, device=dev)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    gb = None if b is None else torch.empty(V, dtype=torch.float32, device=dev)
    ws = ila.backward_workspace_for(N, V, dev)
    stream = torch.cuda.Stream(device=dev)

    def run():
        ila.bilogp_backward(h, w, t, b, lse, up["grad_logp"], up["grad_lse"], gh, gw, gb, ws,
                            stream=stream)
    for _ in range(warmup):
        run()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 6.0 * N * H * V
    return {"ms": ms, "tflops": flops / ms / 1e9, "frac": flops / ms / 1e9 / PEAK_BF16_TFLOPS,
            "tokens_per_s": N / ms * 1e3, "flops": flops,
            "finite": bool(torch.isfinite(gh).all()) and bool(torch.isfinite(gw).all())}


def shard_share_leg(h, t, w, b, ranks=8, steps=10, warmup=3):
    """One GPU's share of the workload sharded over `ranks` GPUs, at its real
    shape: (a) vocabulary sharding - rank 0's contiguous split range of the
    full V (bilogp_partials_range on its own weight columns), (b) row sharding
    - the full step on N / ranks rows.  No exchange is timed (one GPU)."""
    import torch
    import invariant_linear_log_amd as ila
    dev = h.device
    N, H = h.shape
    V = w.shape[0]
    S = ila.bilogp_num_vocab_splits(V)
    per = -(-S // ranks)
    c0, c1 = ila.vocab_split_columns(V, 0, per)
    w_slice = w[c0:c1].clone()
    b_slice = None if b is None else b[c0:c1].clone()
    ws = ila.workspace_for(N, V, dev)
    stream = torch.cuda.Stream(device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / steps

    vs_ms = timed(lambda: ila.bilogp_partials_range(h, w_slice, t, b_slice, V, 0, per, ws,
                                                    stream=stream))
    n = -(-N // ranks)
    hn, tn = h[:n].contiguous(), t[:n].contiguous()
    lp = torch.empty(n, device=dev)
    ls = torch.empty(n, device=dev)
    wsn = ila.workspace_for(n, V, dev)
    ns_ms = timed(lambda: ila.bilogp_forward_ex(hn, w, tn, b, lp, ls, wsn, stream=stream))
    fv = 2.0 * N * H * (c1 - c0)
    fn_ = 2.0 * n * H * V
    return {"ranks": ranks,
            "vocab_shard": {"splits": [0, per], "columns": [c0, c1], "ms": vs_ms,
                            "tflops": fv / vs_ms / 1e9, "frac": fv / vs_ms / 1e9 / PEAK_BF16_TFLOPS},
            "row_shard": {"rows": n, "ms": ns_ms, "tflops": fn_ / ns_ms / 1e9,
                          "frac": fn_ / ns_ms / 1e9 / PEAK_BF16_TFLOPS}}


def library_context_leg(h, t, w, b, step, stream, reps=5, steps=10, warmup=3):
    """Context, not the product: the same contraction through torch's bf16 matmul
    (hipBLASLt; z = hidden . W^T materialised as bf16 [N, V], no softmax), and the
    unfused path a caller would otherwise run (that matmul, the bias added in
    float32, a float32 logsumexp over V and a gather of the target logit).  Neither is batch-
    invariant by contract.  The fused step and the library GEMM alternate on one
    stream, `reps` rounds of `steps` calls each, so both see the same clock and
    power state; medians and minima over the rounds."""
    import torch
    h2 = h.reshape(-1, h.shape[-1])
    t2 = t.reshape(-1)
    N, H = h2.shape
    V = w.shape[0]
    flops = 2.0 * N * H * V

    def gemm():
        return torch.matmul(h2, w.t())

    def unfused():
        z = torch.matmul(h2, w.t()).float()
        if b is not None:
            z = z + b.float()
        lse = torch.logsumexp(z, dim=-1)
        return z.gather(1, t2[:, None])[:, 0] - lse, lse

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    alternating = {"fused_step": step, "hipblaslt_gemm": gemm}
    times = {name: [] for name in alternating}
    with torch.cuda.stream(stream):
        for fn in alternating.values():
            for _ in range(warmup):
                fn()
        for _ in range(reps):
            for name, fn in alternating.items():
                times[name].append(timed(fn, steps))
        for _ in range(warmup):
            unfused()
        unfused_ms = timed(unfused, steps)
    rec = {}
    for name, v in times.items():
        v = sorted(v)
        rec[name] = {"ms": statistics.median(v), "ms_min": v[0],
                     "tflops": flops / statistics.median(v) / 1e9}
    rec["unfused_matmul_logsumexp"] = {"ms": unfused_ms, "tflops": flops / unfused_ms / 1e9}
    rec["protocol"] = (f"fused_step and hipblaslt_gemm alternate on one stream, {reps} rounds "
                       f"of {steps} calls each after {warmup} warmup calls; ms = median over "
                       f"the rounds; the unfused path once, {steps} calls")
    torch.cuda.empty_cache()
    return rec


def device_info(dev):
    import torch
    prop = torch.cuda.get_device_properties(dev)
    return {"name": prop.name, "arch": getattr(prop, "gcnArchName", ""),
            "compute_units": prop.multi_processor_count,
            "hbm_gib": round(prop.total_memory / 2 ** 30, 1)}


def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas = ""
    try:
        from threadpoolctl import threadpool_info
        blas = ",".join(sorted({i.get("internal_api", "") for i in threadpool_info()
                                if i.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover
        pass
    return model, blas


def cpu_baseline(inp, rows_n, seed=7):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("internal_api") in ("openblas", "mkl", "blis")] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    h = inp["hidden"].reshape(-1, inp["hidden"].shape[-1]).cpu()
    t = inp["target"].reshape(-1).cpu()
    w = inp["weight"].cpu()
    b = None if inp["bias"] is None else inp["bias"].cpu()
    N = h.shape[0]
    g = np.random.default_rng(seed)
    rows = np.sort(g.choice(N, size=min(rows_n, N), replace=False))
    t0 = time.perf_counter()
    oracle.linear_logp(h, w, t, b, rows=rows)
    dt = time.perf_counter() - t0
    model, blas = cpu_info()
    flops = 2.0 * len(rows) * h.shape[1] * w.shape[0]
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} seeded rows of the {N}-row workload (fp64 numpy/BLAS, "
                      f"bf16 decode included), {dt:.1f} s",
            "fp64_gflops": flops / dt / 1e9, "cpu": model, "blas": blas}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); rows are independent, "
              "so N GPUs would each run this same single-GPU step on their own rows.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_linear_log_amd as ila
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_inputs(args.workload, device=dev)
    wl = inp["workload"]
    h = inp["hidden"].reshape(-1, wl.H).contiguous()
    t = inp["target"].reshape(-1).contiguous()
    w = inp["weight"]
    b = inp["bias"]
    N, H, V = wl.N, wl.H, wl.V
    S = ila.bilogp_num_vocab_splits(V)
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    ws = ila.workspace_for(N, V, dev)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    def step(ev0=None, ev1=None, ev2=None):
        if ev0 is not None:
            ev0.record(stream)
        ila.bilogp_partials(h, w, t, b, ws, stream=stream)
        if ev1 is not None:
            ev1.record(stream)
        ila.bilogp_merge(t, ws, logp, lse, V, stream=stream)
        if ev2 is not None:
            ev2.record(stream)

    for _ in range(args.warmup):
        step()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(*evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    proj_ms = [e[0].elapsed_time(e[1]) for e in evs]
    merge_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)
    avg_proj_s = sum(proj_ms) / K / 1e3
    avg_merge_s = sum(merge_ms) / K / 1e3
    flops = 2.0 * N * H * V
    tflops_proj = flops / avg_proj_s / 1e12
    ms_per_step = elapsed / K * 1e3
    tokens_per_s = N * K / elapsed
    tflops_step = flops / (elapsed / K) / 1e12
    ok = bool(torch.all(torch.isfinite(lse))) and bool(torch.all(logp <= 0))
    bias_bytes = 0 if b is None else V * b.element_size()

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "H": H, "V": V,
                   "lead_shape": list(wl.lead_shape),
                   "bias": wl.bias, "splits": S, "tokens_per_step": N},
        "tflops": tflops_step,
        "mfma_peak_frac": tflops_step / PEAK_BF16_TFLOPS,
        "kernel_ms": {"proj_lse": avg_proj_s * 1e3, "merge": avg_merge_s * 1e3,
                      "proj_lse_median": sorted(proj_ms)[K // 2], "proj_lse_min": min(proj_ms),
                      "step_median": step_ms[K // 2], "step_min": step_ms[0]},
        "device": device_info(dev),
        "outputs_sane": ok,
        "launch": launch_plan(N, H, V),
        "roofline": {"bound": "mfma", "kernel": "proj_lse_kernel",
                     "achieved": tflops_proj, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops_proj / PEAK_BF16_TFLOPS,
                     "algorithmic_flops": flops,
                     "algorithmic_bytes": algorithmic_bytes(N, H, V, S, bias_bytes),
                     "algorithmic_hbm_gbps": algorithmic_bytes(N, H, V, S, bias_bytes)
                     / avg_proj_s / 1e9,
                     "traffic": measured_traffic(wl.name),
                     "traffic_unit": "bytes per launch",
                     "traffic_kind": TRAFFIC_KIND},
    }
    if not args.no_clock:
        out["clock"] = clock_sample(step)
    if not args.no_configs:
        out["configs"] = config_legs()
    if not args.no_invariance_cost:
        out["invariance_cost"] = invariance_cost(h, t, w, b)
    if not args.no_backward:
        out["backward"] = backward_leg(h, t, w, b, lse)
    if not args.no_shard_share:
        out["shard_share"] = shard_share_leg(h, t, w, b)
    if not args.no_det_gemm:
        out["det_gemm"] = det_gemm_leg()
    if not args.no_library_context:
        out["library_context"] = library_context_leg(h, t, w, b, step, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
