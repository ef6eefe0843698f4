"""Benchmark of the Beam MoE block on one MI355X.

A step is one forward of the whole block (router, permutation, experts,
combine) over one batch of synthetic tokens already resident in HBM.  The
default workload is the Beam-shape decode layer (64 bf16 tokens, hidden 5120,
256 experts in 8 groups of 32, top-4 groups, top-8 experts, SwiGLU 2560),
the HBM-bound half of the metric; the default run also times the MFMA-bound
half, the 16,384-token prefill with skewed routing, in the same process and
reports it under "prefill" in the same line.

Prints one JSON line: throughput (tokens/s), the dominant kernel's roofline
(its average duration from HIP events recorded around it on its own stream
inside the timed region) and the CPU oracle timed on a bounded sample of the
same workload on this host's cores.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % of roofline (MFMA prefill, HBM GB/s decode), 1 GPU"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5033.2        # MI355X dense fp8 MFMA
FP32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode64")
    ap.add_argument("--prefill-workload", default="prefill16k_skew",
                    help="second workload timed in the default run (the MFMA-bound "
                         "prefill); 'none' skips it.  Runs only with the default "
                         "--workload and no --tokens")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count (decode/verify sweep)")
    ap.add_argument("--path", choices=["auto", "stream", "grouped"], default="auto")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time K replays of the step captured in a HIP graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 4 GiB device copy instead (the known-size "
                         "kernel that scales HBM byte counters)")
    ap.add_argument("--dense-ref", action="store_true",
                    help="time the library GEMM (torch.matmul, hipBLASLt) on dense "
                         "bf16 products of the expert shapes instead: the reference "
                         "the grouped GEMMs are compared with")
    return ap.parse_args()


def kernel_bytes_flops(name, T, S, H, I, E, touched, wbytes):
    """Algorithmic bytes and flops of one launch of a kernel.  Weights of
    touched experts are read once; activations once; outputs written once."""
    if name in ("stream_gate_up_bf16", "grouped_gate_up_bf16"):
        return (touched * 2 * I * H * wbytes + T * H * 2 + S * I * 2,
                2.0 * S * 2 * I * H)
    if name in ("stream_down_bf16", "grouped_down_bf16"):
        ybytes = 4 if name.startswith("stream") else 2
        return (touched * H * I * wbytes + S * I * 2 + S * H * ybytes,
                2.0 * S * H * I)
    # e4m3 codes with fp32 scales per 128x128 weight block and per 128
    # activation channels; gate/up writes h as codes + scales
    if name == "gate_up_fp8":
        return (touched * 2 * I * H * (1 + 4 / 16384) + T * H * (1 + 4 / 128)
                + S * I * (1 + 4 / 128), 2.0 * S * 2 * I * H)
    if name == "down_fp8":
        return (touched * H * I * (1 + 4 / 16384) + S * I * (1 + 4 / 128) + S * H * 2,
                2.0 * S * H * I)
    # MXFP4 weights (wbytes includes the E8M0 bytes), MXFP8 activations
    if name == "stream_gate_up_mx":
        return (touched * 2 * I * H * wbytes + T * H * (1 + 1 / 32) + S * I * 2,
                2.0 * S * 2 * I * H)
    if name == "stream_down_mx":
        return (touched * H * I * wbytes + S * I * (1 + 1 / 32) + S * H * 4,
                2.0 * S * H * I)
    if name == "grouped_gate_up_mx":  # writes h as MXFP8 codes + E8M0 bytes
        return (touched * 2 * I * H * wbytes + T * H * (1 + 1 / 32) + S * I * (1 + 1 / 32),
                2.0 * S * 2 * I * H)
    if name == "grouped_down_mx":
        return (touched * H * I * wbytes + S * I * (1 + 1 / 32) + S * H * 4,
                2.0 * S * H * I)
    return None, None


def sources_sha256(paths):
    """SHA-256 over the listed source files (repository-relative), in order."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    try:
        h = sources_sha256(rec["sources"])
    except (OSError, KeyError):
        return None
    return rec["bytes_per_launch"] if h == rec["sources_sha256"] else None


def traffic_source(kernel, workload, value):
    """Where the roofline's traffic figure comes from (it is not counted in
    this run: HBM counters need profiler passes of their own)."""
    if value is None:
        return ("none: no counter run on the current kernel sources "
                f"(profiles/traffic_{kernel}_{workload}.json absent or stale)")
    return (f"replayed from profiles/traffic_{kernel}_{workload}.json: rocprofv3 "
            "FETCH_SIZE and WRITE_SIZE runs on the same kernel sources (SHA-256 "
            "checked), scaled by the copy calibration")


def calibrate_copy(steps):
    """A plain device copy of 4 GiB (torch's copy kernel): reads and writes
    known byte counts, so HBM counters of other kernels can be scaled."""
    import torch
    n = 4 * 2**30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n,
                      "ms": ms, "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}),
          flush=True)


def dense_reference(steps, warmup):
    """torch.matmul (hipBLASLt on ROCm) on dense bf16 products with the Beam
    expert shapes: 16,384 rows (the 16K-token prefill's rows if one expert
    held them all) times the gate/up matrix [2I, H] and the down matrix
    [H, I], and about the hot experts' rows in the skewed 16K layer (10,680 to 10,928: 10,880).
    Reports TFLOP/s per shape."""
    import torch
    H, I = 5120, 2560
    g = torch.Generator(device="cuda:0").manual_seed(0)
    out = []
    for name, M, N, K in (("gate_up", 16384, 2 * I, H), ("down", 16384, H, I),
                          ("gate_up_hot_expert", 10880, 2 * I, H)):
        a = torch.randn(M, K, generator=g, device="cuda:0").to(torch.bfloat16)
        w = torch.randn(N, K, generator=g, device="cuda:0").to(torch.bfloat16)
        wt = w.t()                      # nn.Linear layout: x @ W^T
        for _ in range(warmup):
            torch.matmul(a, wt)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            torch.matmul(a, wt)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out.append({"shape": name, "M": M, "N": N, "K": K, "ms": ms, "TFLOPs": tf,
                    "frac_bf16_peak": tf / BF16_PEAK_TFLOPS})
        del a, w, wt
    print(json.dumps({"dense_reference": "torch.matmul bf16", "results": out}), flush=True)


def read_sclk():
    """Current shader clock level in MHz from the amdgpu sysfs table, or None."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().rstrip("*").strip()
                               .lower().rstrip("mhz").strip())
        except (OSError, ValueError, IndexError):
            continue
    return None


def cpu_baseline(inp, shape, seconds):
    """The oracle (logits, routing, experts, combine in binary64) timed on
    this host's cores over a bounded sample of the workload's tokens: about
    `seconds` of oracle work, repeating passes over the sample when the whole
    workload is shorter.  Copies of the touched experts to host memory are
    made outside the timed region."""
    import numpy as np
    import torch
    import oracle

    T = inp.x.shape[0]
    rng = np.random.default_rng(0)
    threads = oracle.max_threads()
    bias = inp.bias.cpu().numpy()
    w_router = inp.w_router.cpu()
    cache = {}

    def experts(need):
        missing = [int(e) for e in need if int(e) not in cache]
        if missing:
            sel = torch.as_tensor(missing, device=inp.x.device)
            wgu = inp.w_gate_up.index_select(0, sel).cpu()
            wd = inp.w_down.index_select(0, sel).cpu()
            sgu = sd = None
            if inp.s_gate_up is not None:
                sgu = inp.s_gate_up.index_select(0, sel).cpu()
                sd = inp.s_down.index_select(0, sel).cpu()
            for j, e in enumerate(missing):
                cache[e] = (wgu[j], wd[j], None if sgu is None else sgu[j],
                            None if sd is None else sd[j])
        parts = [cache[int(e)] for e in need]
        stack = lambda i: (None if parts[0][i] is None
                           else torch.stack([q[i] for q in parts]))
        return stack(0), stack(1), stack(2), stack(3)

    def run(tokens, passes=1):
        xs = inp.x[torch.as_tensor(tokens, device=inp.x.device)].cpu()
        busy = 0.0
        for _ in range(passes):
            t0 = time.perf_counter()
            lg = oracle.logits(shape, xs, w_router).astype(np.float32)
            idx, w, _ = oracle.route(shape, lg, bias)
            busy += time.perf_counter() - t0
            need = np.unique(idx)
            remap = np.full(shape.n_experts, -1, np.int64)
            remap[need] = np.arange(need.size)
            wgu, wd, sgu, sd = experts(need)          # host copies, untimed
            t0 = time.perf_counter()
            oracle.forward_tokens(shape, np.arange(len(tokens)), xs,
                                  remap[idx].astype(np.int32), w, wgu, wd, sgu, sd,
                                  act_quant=sgu is not None)
            busy += time.perf_counter() - t0
        return busy

    probe = rng.choice(T, min(T, threads), replace=False)
    per_tok = run(probe) / len(probe)
    want = max(len(probe), int(seconds / max(per_tok, 1e-9)))
    if want <= T:
        n = max(threads, (want // threads) * threads) if want >= threads else want
        toks, passes = rng.choice(T, min(n, T), replace=False), 1
    else:
        toks, passes = np.arange(T), int(np.ceil(want / T))
    t = run(toks, passes)
    done = len(toks) * passes
    what = (f"{len(toks)} of {T} tokens (random, seed 0)" if passes == 1 else
            f"all {T} tokens, {passes} passes")
    return {"value": done / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}: binary64 logits, routing, {shape.top_k} SwiGLU experts "
                      f"and combine per token; {t:.1f} s of oracle work on {threads} "
                      f"threads (host copies of the touched experts excluded)"}


def graph_timing(step, stream, steps, T):
    """Capture one step in a HIP graph (torch.cuda.CUDAGraph) and time `steps`
    replays on `stream` with events, as the eager steps are timed."""
    import numpy as np
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    med = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    return {"ms_per_step": ms, "value": T / (ms * 1e-3), "step_ms_median": med}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported: "
              "the library has no multi-GPU path (the block runs whole on one "
              "MI355X).", file=sys.stderr)
        sys.exit(2)
    if a.calibrate_copy:
        calibrate_copy(max(a.steps, 1))
        return
    if a.dense_ref:
        dense_reference(max(a.steps, 1), a.warmup)
        return
    res = run_workload(a, a.workload, a.tokens)
    if (a.prefill_workload != "none" and a.workload == "decode64" and a.tokens is None):
        import torch
        torch.cuda.empty_cache()
        pre = run_workload(a, a.prefill_workload, None)
        res["prefill"] = {k: pre[k] for k in (
            "value", "unit", "ms_per_step", "step_ms", "dtype", "config", "roofline",
            "layer", "sclk_mhz", "routing", "kernels_ms", "cpu_baseline", "graph")
            if k in pre}
    print(json.dumps(res), flush=True)


def run_workload(a, workload, tokens):
    """Times a.steps forwards of one workload; returns its result dict."""
    import numpy as np
    import torch

    import group_limited_routing_sigmoid_amd as gl
    from synth import WORKLOADS, make_inputs, FP8, MXFP4

    w = WORKLOADS[workload]
    sh = w.shape
    dev = torch.device("cuda:0")
    inp = make_inputs(w, device=dev, tokens=tokens)
    T, H, I, E, K = inp.x.shape[0], sh.hidden, sh.intermediate, sh.n_experts, sh.top_k
    S = T * K
    flags = {"auto": 0, "stream": gl.PATH_STREAM, "grouped": gl.PATH_GROUPED}[a.path]
    wdt = {FP8: gl.FP8_E4M3, MXFP4: gl.MXFP4, "f32": gl.F32}.get(w.weight_dtype, gl.BF16)
    act = gl.F32 if w.act_dtype == "f32" else gl.BF16
    d = gl.make_desc(sh, act, wdt, flags)
    ws = gl.Workspace(dev)
    out = torch.empty(T, H, dtype=inp.x.dtype, device=dev)

    def step(timer=None):
        gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                   inp.s_gate_up, inp.s_down, out=out, workspace=ws, timer=timer)

    # routing statistics of this batch (touched experts set the byte count)
    idx, _, _ = gl.route(d, inp.x, inp.w_router, inp.bias, workspace=ws)
    counts = torch.bincount(idx.flatten().long(), minlength=E).cpu().numpy()
    touched = int((counts > 0).sum())
    for _ in range(a.warmup):
        step()
    timer = gl.Timer(capacity=64 * max(a.steps, 1))
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(a.steps):
        step(timer)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / a.steps
    step_ms = np.sort([ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)])
    graph = graph_timing(step, stream, a.steps, T) if a.graph else None
    sclk = read_sclk()
    per = {}
    for name, kms in timer.records():
        per.setdefault(name, []).append(kms)
    kern_ms = {k: sum(v) / len(v) for k, v in per.items()}
    launches = {k: len(v) / a.steps for k, v in per.items()}
    dom = max(kern_ms, key=lambda k: kern_ms[k] * launches[k])
    wbytes = {FP8: 1, MXFP4: 0.5 + 1 / 32, "f32": 4}.get(w.weight_dtype, 2)
    kb, kf = kernel_bytes_flops(dom, T, S, H, I, E, touched, wbytes)
    # the e4m3 x E2M1 products of the MXFP4 path are priced at the fp8 rate
    peak = FP8_PEAK_TFLOPS if w.weight_dtype in (FP8, MXFP4) else (
        FP32_PEAK_TFLOPS if w.weight_dtype == "f32" else BF16_PEAK_TFLOPS)
    # the kernel's bound is the larger of its memory time and its compute time
    mem_bound = kf is None or kb / (HBM_PEAK_GBS * 1e9) >= kf / (peak * 1e12)
    if mem_bound:
        ach = kb / (kern_ms[dom] * 1e-3) / 1e9 if kb else None
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS if ach else None,
                "traffic": traffic_for(dom, workload), "kernel": dom,
                "kernel_ms": kern_ms[dom], "algorithmic_bytes": kb}
    else:
        ach = kf / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": traffic_for(dom, workload),
                "kernel": dom, "kernel_ms": kern_ms[dom], "algorithmic_flops": kf}
    roof["traffic_source"] = traffic_source(dom, workload, roof["traffic"])
    layer_bytes = touched * 3 * H * I * wbytes + E * H * 4 + 2 * T * H * inp.x.element_size()
    layer_flops = 2.0 * S * 3 * H * I
    roof_ms = max(layer_bytes / (HBM_PEAK_GBS * 1e9), layer_flops / (peak * 1e12)) * 1e3
    res = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "step_ms": {"median": float(np.median(step_ms)), "min": float(step_ms[0]),
                    "p90": float(step_ms[min(len(step_ms) - 1, int(0.9 * len(step_ms)))])},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8", "f32": "f32", "mxfp4": "mxfp4"}.get(w.weight_dtype, "bf16"),
        "data": "synthetic",
        "config": {"workload": workload, "tokens": T, "hidden": H,
                   "intermediate": I, "experts": E, "groups": sh.n_groups,
                   "topk_groups": sh.topk_groups, "top_k": K,
                   "routed_scale": sh.routed_scale, "path": a.path,
                   "weights": w.weight_dtype, "bias": w.bias, "seed": w.seed},
        "roofline": roof,
        "layer": {"hbm_GBps": layer_bytes / (ms * 1e-3) / 1e9,
                  "hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "mfma_TFLOPs": layer_flops / (ms * 1e-3) / 1e12,
                  "mfma_frac": layer_flops / (ms * 1e-3) / 1e12 / peak,
                  "bound": "hbm" if layer_bytes / (HBM_PEAK_GBS * 1e9) >=
                           layer_flops / (peak * 1e12) else "mfma",
                  "roofline_ms": roof_ms, "roofline_frac": roof_ms / ms,
                  "algorithmic_bytes": layer_bytes, "expert_flops": layer_flops},
        "sclk_mhz": sclk,
        "routing": {"touched_experts": touched,
                    "max_over_mean_load": float(counts.max() / counts.mean())},
        "kernels_ms": kern_ms,
    }
    if graph is not None:
        res["graph"] = graph
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, sh, a.cpu_seconds)
    del inp, ws, out
    return res


if __name__ == "__main__":
    main()
