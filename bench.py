#!/usr/bin/env python3
"""Benchmark of the KDA chunked forward on one MI355X.

One step = one kda_fwd call (both kernels: intra-chunk stage and scan) over
the T=8192, H=96, D=128 fixed-length workload with a bf16 initial state and
an fp32 final state, inputs already resident in HBM.  Prints ONE JSON line.
The same run times the other T=8192 workloads of the pages (fixed H=64,
uniform varlen 8 x 1024, mixed varlen at H=96 and H=64) and reports them
under path.workloads; `value` is the headline workload's.

Roofline accounting (algorithmic bytes, i.e. what the operation must move):
  per (token, head): q, k, g, v 4 x 256 B, beta 2 B, out 256 B   = 1282 B
  per (sequence, head): initial state (bf16 32 KiB) if given, final state
  (fp32 64 KiB) if requested.
  Split per kernel: the intra-chunk kernel must read q, k, g, beta (770 B);
  the scan must read v and write out (512 B) plus the states.  The hand-off
  records between the two kernels are design overhead, not algorithmic.
The timed steps run with nothing between the kernels; a second pass of the
same number of steps takes each kernel's duration from HIP events the
library records around it (kda_set_stage_events) on the stream the kernels
run on (those events cost a few microseconds per step, so they stay out of
the timed pass).

`--head-dim 256` measures the same workload at K = V = 256.

`--scalar-gate` measures the Gated DeltaNet form (kda_fwd_scalar_gate) on
the same workload with g [B, T, H] and dt_bias [H]: g then moves 2 B per
(token, head) instead of 256; with `--backward`, its backward
(kda_bwd_scalar_gate).

`--head-dim 64` measures the same workload at K = V = 64.

`--backward` measures the backward pass (kda_bwd, five kernels) on the same
workload: gradients of every input for an incoming bf16 d_out and fp32
d_final_state.  Algorithmic bytes per (token, head): q, k, v, g, beta, d_out
read and dq, dk, dv, dg, dbeta written (2308 B); per (sequence, head): the
initial state and d_final_state read, the initial-state gradient written.

`--decode-batch N` instead measures the decode step (kda_decode, one kernel
on the current stream): N one-token sequences x H heads with an fp32 state
updated in place, algorithmic bytes per (sequence, head) = the state read and
written (2 x 64 KiB) + q, k, g, v, beta, out (1282 B).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "KDA fwd tokens/s @T=8192,H=96,D=128 (fixed+varlen); % of MFMA/HBM roofline"
CHUNK = 16           # tokens per chunk of the forward
BWD_CHUNK = 16       # the backward's chunk factors


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, has_init=True, has_final=True, scalar_gate=False):
    th = w.tokens * w.H
    n_units = w.num_seqs * w.H
    state_in = n_units * w.K * w.V * 2 if (has_init and w.initial_state) else 0
    state_out = n_units * w.K * w.V * 4 if has_final else 0
    intra = th * ((2 * w.K * 2 + 2 + 2) if scalar_gate else (3 * w.K * 2 + 2))
    scan = th * (2 * w.V * 2) + state_in + state_out
    # MACs per token-head of the chunkwise algorithm at chunk C: three state
    # products, the two in-chunk Gram products at triangular useful size, the
    # T-apply and Aqk E products, and the C x C inverse.
    C = CHUNK
    macs = 3 * w.K * w.V + C * w.K + (C + 1) * w.V + C * C / 6.0
    return {"intra_bytes": intra, "scan_bytes": scan, "total_bytes": intra + scan,
            "flops": 2.0 * macs * th}


def stored_traffic(workload: str, kernel: str, backward: bool = False):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/hbm_traffic_[bwd_]<workload>.json: FETCH_SIZE and WRITE_SIZE
    runs scaled by a plain copy of known size), or None when there is none or
    the kernel sources changed since the counters were taken."""
    import kimi_delta_attention_04_amd as kda
    tag = "bwd_" if backward else ""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{tag}{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sources = kda.BACKWARD_KERNEL_SOURCES if backward else kda.FORWARD_KERNEL_SOURCES
    if rec.get("source_digest") != kda.source_digest(sources) or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return {"read_bytes": k["read_bytes"], "write_bytes": k["write_bytes"],
            "total_bytes": k["read_bytes"] + k["write_bytes"]}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, w, heads: int):
    import oracle
    sel = list(range(min(heads, w.H)))
    t0 = time.perf_counter()
    oracle.cref_forward(inp, heads=sel, want_final=True)
    dt = time.perf_counter() - t0
    # the whole workload takes H / len(sel) times as long (heads are independent)
    tok_s = w.tokens / (dt * w.H / len(sel))
    return {"value": tok_s, "unit": "tokens/s", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{w.name}: heads 0..{len(sel) - 1} of {w.H}, all {w.tokens} tokens, "
                      f"fp64 C/OpenMP token recurrence, {dt:.2f} s wall"}


def bench_decode(args, torch, kda, kda_inputs):
    N, H, D = args.decode_batch, args.decode_heads, args.head_dim
    log(f"[bench] decode: generating N={N} H={H} D={D} ...")
    inp = kda_inputs.random_small(2, B=N, T=1, H=H, K=D, V=D)
    gen = torch.Generator().manual_seed(2)
    state0 = (torch.randn(N, H, D, D, generator=gen) * 0.05).float()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flat = lambda t: t.reshape(N, H, -1).contiguous().to(dev)
    q, k, v, g = (flat(inp[x]) for x in ("q", "k", "v", "g"))
    beta = inp["beta"].reshape(N, H).contiguous().to(dev)
    A_log, dtb = inp["A_log"].to(dev), inp["dt_bias"].to(dev)
    state = state0.to(dev)
    out = torch.empty(N, H, D, dtype=torch.bfloat16, device=dev)

    def step():
        kda.decode(q, k, v, g, beta, inp["scale"], out, A_log, dtb, inp["lower_bound"], state)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    units = N * H
    # per (sequence, head): the fp32 state read and written; q, k, v, g and
    # o (bf16, D each) and beta
    bytes_ = units * (2 * D * D * 4 + 10 * D + 2)
    achieved = bytes_ / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "kda_decode",
                "bytes_per_launch": bytes_, "avg_launch_ms": ms}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        inp["initial_state"] = state0
        t0 = time.perf_counter()
        oracle.cref_forward(inp, want_final=True)
        dt = time.perf_counter() - t0
        cpu = {"value": N / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
               "sample": f"the whole step: {N} sequences x {H} heads, fp64 C/OpenMP, {dt:.3f} s wall"}
    rec = {"metric": f"KDA decode step tokens/s (one token per sequence) @N={N},H={H},D={D}, fp32 state",
           "value": N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp32", "data": "synthetic (seeded)",
           "config": {"workload": f"decode_N{N}_H{H}" + ("" if D == 128 else f"_D{D}"), "N": N, "H": H,
                      "K": D, "V": D,
                      "state": "fp32, in place"},
           "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def bench_backward(args, torch, kda, kda_inputs):
    """One step = one kda_bwd call over the workload (all five kernels)."""
    name = args.workload or kda_inputs.HEADLINE
    w = kda_inputs.WORKLOADS[name]
    if args.head_dim != w.K:
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}_D{args.head_dim}", K=args.head_dim, V=args.head_dim)
        name = w.name
    log(f"[bench] backward: generating {name} ...")
    inp = kda_inputs.generate(w)
    d_out, d_final = kda_inputs.output_grads(w.seed + 1, w.B, w.T, w.H, V=w.V, N=w.num_seqs, K=w.K)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    dO, dF = d_out.to(dev), d_final.to(dev)
    bf = torch.bfloat16
    shp = (w.B, w.T, w.H, w.K)
    dq, dk, dg = (torch.empty(shp, dtype=bf, device=dev) for _ in range(3))
    dv = torch.empty(w.B, w.T, w.H, w.V, dtype=bf, device=dev)
    dbeta = torch.empty(w.B, w.T, w.H, dtype=bf, device=dev)
    dA = torch.empty(w.H, device=dev)
    ddtb = torch.empty(w.H * w.K, device=dev)
    dinit = torch.empty(w.num_seqs, w.H, w.K, w.V, device=dev)
    bwd = kda.bwd
    if args.scalar_gate:
        # the Gated DeltaNet form: one gate value per (token, head), channel 0
        # of the workload's gate, and dt_bias per head
        d["g"] = d["g"][..., 0].contiguous()
        d["dt_bias"] = d["dt_bias"].view(w.H, w.K)[:, 0].contiguous()
        dg = torch.empty(w.B, w.T, w.H, dtype=bf, device=dev)
        ddtb = torch.empty(w.H, device=dev)
        bwd = kda.bwd_scalar_gate

    def step():
        bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d["dt_bias"],
            d["lower_bound"], dO, dq, dk, dv, dg, dbeta, dA, ddt_bias=ddtb,
            initial_state=d["initial_state"], d_final_state=dF, d_initial_state=dinit,
            cu_seqlens=d["cu_seqlens"])

    log(f"[bench] backward warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    names = ["kda_bwd_prep", "kda_bwd_states", "kda_bwd_dstates", "kda_bwd_chunk", "kda_bwd_reduce"]
    evs = []
    for _ in range(args.steps):
        six = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in six:
            e.record()
        evs.append(six)
    torch.cuda.synchronize()
    # as the forward: an uninstrumented timed pass, then a pass with the
    # per-kernel events
    log(f"[bench] backward timing {args.steps} steps")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    for i in range(args.steps):
        kda.set_bwd_stage_events([e.cuda_event for e in evs[i]])
        step()
    kda.set_bwd_stage_events(None)
    torch.cuda.synchronize()
    stage = {n: statistics.mean(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps))
             for j, n in enumerate(names)}

    # algorithmic bytes: per (token, head) the inputs q, k, v, g, beta and
    # d_out read once and dq, dk, dv, dg, dbeta written once (2308 B); per
    # (sequence, head) the initial state, d_final read and the initial-state
    # gradient written.  Per kernel, the part of that each kernel must move.
    th, units = w.tokens * w.H, w.num_seqs * w.H
    st_in = units * w.K * w.V * 2 if w.initial_state else 0
    st32 = units * w.K * w.V * 4
    kb = {"kda_bwd_prep": th * 770, "kda_bwd_states": th * 256 + st_in,
          "kda_bwd_dstates": th * 512 + 2 * st32, "kda_bwd_chunk": th * (1282 + 770),
          "kda_bwd_reduce": 0}
    total_bytes = th * 2308 + st_in + 2 * st32
    dom = max(names, key=lambda n: stage[n])
    achieved = kb[dom] / (stage[dom] * 1e-3) / 1e9
    tr = None if args.scalar_gate else stored_traffic(name, dom, backward=True)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": tr["total_bytes"] if tr else None,
                "traffic_x_algorithmic": tr["total_bytes"] / kb[dom] if tr else None,
                "kernel": dom, "bytes_per_launch": kb[dom], "avg_launch_ms": stage[dom]}
    path_gbs = total_bytes / (ms * 1e-3) / 1e9
    path = {"algorithmic_bytes": total_bytes, "hbm_achieved_GBs": path_gbs,
            "hbm_frac": path_gbs / HBM_PEAK_GBS, "stage_ms": stage,
            "stage_traffic_bytes": {k: (t["total_bytes"] if t else None) for k, t in
                                    ((k, None if args.scalar_gate else
                                      stored_traffic(name, k, backward=True)) for k in names)},
            # per (chunk slot, head): the two scans' records (5 + 7, 9 + 13 or
            # 17 + 26 KB at K = 64, 128, 256), S0 and dS1 (bf16 K x V), X
            # (bf16 16 x V), the partial sums (max(K, 128) + 1 floats)
            "workspace_bytes": int(w.H * (w.tokens // BWD_CHUNK + w.num_seqs) *
                                   ({64: 5120 + 7168, 128: 9216 + 13312, 256: 17408 + 26624}[w.K] +
                                    2 * w.K * w.V * 2 + BWD_CHUNK * w.V * 2 +
                                    (max(w.K, 128) + 1) * 4))}
    cpu = None
    if not args.no_cpu_baseline and not args.scalar_gate:
        import oracle
        # every head at K <= 128 (about 10 s on 16 threads at 128), a quarter
        # of them at 256 (four times the work per head)
        heads = list(range(w.H if w.K <= 128 else max(1, w.H // 4)))
        log(f"[bench] gradient oracle CPU baseline on heads 0..{heads[-1]}")
        t0 = time.perf_counter()
        oracle.cref_backward(inp, d_out, d_final, heads=heads)
        dt = time.perf_counter() - t0
        cpu = {"value": w.tokens / (dt * w.H / len(heads)), "unit": "tokens/s",
               "cores": oracle.max_threads(), "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"{w.name}: heads {heads[0]}..{heads[-1]} of {w.H}, all {w.tokens} "
                         f"tokens, fp64 C/OpenMP reverse-mode token recurrence, {dt:.2f} s wall"}
    form = " (Gated DeltaNet form)" if args.scalar_gate else ""
    rec = {"metric": f"KDA bwd tokens/s @T={w.T},H={w.H},D={w.K} (gradients of every input){form}",
           "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
           "data": "synthetic (seeded; shapes of the pages' workloads)",
           "config": dict(w.describe(), d_out="bf16", d_final_state="fp32"),
           "roofline": roofline, "cpu_baseline": cpu, "path": path}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the T=8192 H=96 fixed one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (default: all five T=8192 workloads)")
    ap.add_argument("--cpu-heads", type=int, default=96, help="heads in the oracle's timed sample")
    ap.add_argument("--head-dim", type=int, default=128, choices=(64, 128, 256),
                    help="K = V of the measured workload")
    ap.add_argument("--scalar-gate", action="store_true",
                    help="measure the Gated DeltaNet form (one gate value per token and head)")
    ap.add_argument("--decode-batch", type=int, default=0, metavar="N",
                    help="measure the decode step on N one-token sequences instead")
    ap.add_argument("--decode-heads", type=int, default=96)
    ap.add_argument("--backward", action="store_true",
                    help="measure the backward pass (kda_bwd) on the workload instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times): the "
                         "reference kernel for scaling the HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the KDA forward here runs on a single "
              "MI355X and no multi-GPU path is built (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return

    import kda_inputs
    import kimi_delta_attention_04_amd as kda

    kda.load()
    if args.decode_batch:
        bench_decode(args, torch, kda, kda_inputs)
        return
    if args.backward:
        bench_backward(args, torch, kda, kda_inputs)
        return
    name = args.workload or kda_inputs.HEADLINE
    w = kda_inputs.WORKLOADS[name]
    if args.head_dim != w.K:
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}_D{args.head_dim}", K=args.head_dim, V=args.head_dim)
    rec = bench_forward(args, torch, kda, kda_inputs, w, want_cpu=True)
    # The default run also times the other benchmark workloads of the pages
    # (T = 8192: fixed H = 64, uniform varlen 8 x 1024, mixed varlen at
    # H = 96 and H = 64) with the same kernels and step count; the headline
    # `value` stays the fixed-length H = 96 workload.
    if args.workload is None and args.head_dim == 128 and not args.scalar_gate and not args.headline_only:
        others = {}
        for other in kda_inputs.BENCH_WORKLOADS:
            if other == w.name:
                continue
            r = bench_forward(args, torch, kda, kda_inputs, kda_inputs.WORKLOADS[other], want_cpu=False)
            others[other] = {"ms_per_step": r["ms_per_step"], "tokens_per_s": r["value"],
                             "hbm_frac": r["path"]["hbm_frac"],
                             "algorithmic_bytes": r["path"]["algorithmic_bytes"],
                             "stage_ms": r["path"]["stage_ms"], "roofline": r["roofline"],
                             "config": r["config"]}
        rec["path"]["workloads"] = others
    print(json.dumps(rec), flush=True)


def bench_forward(args, torch, kda, kda_inputs, w, want_cpu):
    """Time args.steps kda_fwd calls on workload w; returns the JSON record."""
    name = w.name
    log(f"[bench] generating {name} ...")
    inp = kda_inputs.generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = torch.empty(w.B, w.T, w.H, w.V, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(w.num_seqs, w.H, w.K, w.V, dtype=torch.float32, device=dev)

    if args.scalar_gate:
        # one gate value per (token, head): channel 0 of the workload's gate
        d["g"] = d["g"][..., 0].contiguous()
        d["dt_bias"] = d["dt_bias"].view(w.H, w.K)[:, 0].contiguous()
        fwd = kda.fwd_scalar_gate
    else:
        fwd = kda.fwd

    def step():
        fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"],
            d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"],
            final_state=fin, cu_seqlens=d["cu_seqlens"])

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-step stage events (created by recording once)
    evs = []
    for _ in range(args.steps):
        trip = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for e in trip:
            e.record()
        evs.append(trip)
    torch.cuda.synchronize()

    # Pass 1: the timed steps themselves, no instrumentation between the
    # kernels.  Pass 2: the same number of steps with the library's per-kernel
    # events, for each kernel's average duration (the events add a few
    # microseconds per step, so they stay out of pass 1).
    log(f"[bench] timing {args.steps} steps of {name}")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    log(f"[bench] per-kernel timing over {args.steps} more steps")
    for i in range(args.steps):
        kda.set_stage_events(evs[i][0].cuda_event, evs[i][1].cuda_event, evs[i][2].cuda_event)
        step()
    kda.set_stage_events(None, None, None)
    torch.cuda.synchronize()
    intra_ms = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]
    kern_ms = [evs[i][0].elapsed_time(evs[i][2]) for i in range(args.steps)]
    scan_ms = [evs[i][1].elapsed_time(evs[i][2]) for i in range(args.steps)]
    intra_avg = statistics.mean(intra_ms)
    scan_avg = statistics.mean(scan_ms)

    alg = algorithmic(w, scalar_gate=args.scalar_gate)
    tok_s = w.tokens / (ms * 1e-3)
    kernels = {
        "kda_intra": {"ms": intra_avg, "bytes": alg["intra_bytes"]},
        "kda_scan": {"ms": scan_avg, "bytes": alg["scan_bytes"]},
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["ms"])
    dom = kernels[dom_name]
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    tr = None if args.scalar_gate else stored_traffic(name, dom_name)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": tr["total_bytes"] if tr else None,
                "traffic_x_algorithmic": tr["total_bytes"] / dom["bytes"] if tr else None,
                "kernel": dom_name, "bytes_per_launch": dom["bytes"], "avg_launch_ms": dom["ms"]}
    path_gbs = alg["total_bytes"] / (ms * 1e-3) / 1e9
    path_tflops = alg["flops"] / (ms * 1e-3) / 1e12
    path = {"algorithmic_bytes": alg["total_bytes"], "hbm_achieved_GBs": path_gbs,
            "hbm_frac": path_gbs / HBM_PEAK_GBS, "algorithmic_flops": alg["flops"],
            "mfma_achieved_TFLOPs": path_tflops, "mfma_frac": path_tflops / BF16_PEAK_TFLOPS,
            "stage_ms": {k: v["ms"] for k, v in kernels.items()},
            "stage_traffic_bytes": {k: (t["total_bytes"] if t else None) for k, t in
                                    ((k, None if args.scalar_gate else stored_traffic(name, k))
                                     for k in kernels)},
            "stage_ms_min": {"kda_intra": min(intra_ms), "kda_scan": min(scan_ms)},
            # first kernel start to last kernel end of each instrumented step
            # (no gap between calls)
            "kernels_ms_per_step": {"median": statistics.median(kern_ms), "min": min(kern_ms),
                                    "mean": statistics.mean(kern_ms)}}

    cpu = None
    if want_cpu and not args.no_cpu_baseline and not args.scalar_gate and w.K == 128:
        log(f"[bench] oracle CPU baseline on {args.cpu_heads} heads")
        cpu = cpu_baseline(inp, w, args.cpu_heads)

    cfg = w.describe()
    metric = METRIC
    if w.K != 128:
        metric = f"KDA fwd tokens/s @T={w.T},H={w.H},D={w.K}"
    if args.scalar_gate:
        metric = "KDA fwd, scalar (Gated DeltaNet) gate, tokens/s @T=8192,H=96,D=128"
        cfg = dict(cfg, gate="scalar per (token, head)")
    return {"metric": metric, "value": tok_s, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded; shapes of the pages' workloads)",
            "config": cfg, "roofline": roofline, "cpu_baseline": cpu, "path": path}

if __name__ == "__main__":
    main()
