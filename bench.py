"""Throughput of the relation-KL hot path (forward + backward of Q/Q, K/K and V/V) on one GPU.

    python bench.py [--steps K] [--warmup W] [--workload llama2_32k] [--no-cpu-baseline]

A step is one pass of the whole path over one batch: for each of the three relations the
forward (LSE statistics + KL) and the backward (recompute + gradient) kernels.  Inputs are
seeded synthetic activations of the workload's shape, resident in HBM before timing.
Prints ONE JSON line.  The dominant kernel (the backward) is timed per launch with HIP
events on the stream it runs on; its algorithmic FLOP count gives the roofline fraction.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "relation-KL fwd+bwd tokens/s at 32 heads,d=128,N=32K; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0


def alg_flops(B, H, N, d, causal):
    """Algorithmic FLOPs of one relation call: (fwd, bwd).

    Forward: the two score contractions (teacher, student) over the kept entries.
    Backward: the two score recomputations plus the two gradient contractions dZ X_s and
    dZ^T X_s over the same entries.  Kept entries: N(N+1)/2 causal, N^2 otherwise.
    """
    kept = N * (N + 1) / 2 if causal else float(N) * N
    per = 2.0 * d * kept  # one contraction over the kept entries
    return B * H * 2 * per, B * H * 4 * per


def cpu_baseline(rel, causal, rows):
    """Time the float64 oracle on a bounded sample: forward and gradient of the last
    `rows` rows of one unit (batch 0, head 0).  For a causal relation these rows are
    self-contained (their column terms only involve rows j >= i of the same sample)."""
    import numpy as np
    import oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    x_t = rel.x_t[0, 0].double().numpy()
    x_s = rel.x_s[0, 0].double().numpy()
    n = x_t.shape[0]
    r0 = n - rows
    sel = np.arange(r0, n)
    s = oracle.default_scale(x_t.shape[1])
    t0 = time.perf_counter()
    lt, ls, kl = oracle.forward_unit(x_t, x_s, s, causal, chunk=1024, rows=sel)
    full_lt = np.full(n, np.nan)
    full_ls = np.full(n, np.nan)
    full_lt[sel], full_ls[sel] = lt, ls
    oracle.backward_unit(x_t, x_s, s, causal, 1.0, lse_t=full_lt, lse_s=full_ls, rows=sel,
                         chunk=1024)
    dt = time.perf_counter() - t0
    return dt, cores


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama2_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the relation-KL "
              "path is single-GPU in this build", file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_relation_distillation_amd import relkl, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[args.workload]
    causal = wl.masks[0]
    t_gen = time.perf_counter()
    rels = workloads.make_inputs(wl)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] inputs generated in {t_gen:.1f}s", file=sys.stderr, flush=True)
    gpu = []
    for r in rels:
        gpu.append((r.name, r.x_t.to(dev), r.x_s.to(dev)))
    gl = torch.ones((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev_log = []

    def step(record):
        for name, xt, xs in gpu:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e2 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            f = relkl.relkl_fwd(xt, xs, causal=causal)
            if record:
                e1.record(stream)
            relkl.relkl_bwd(xt, xs, f["reserve"], gl, causal=causal)
            if record:
                e2.record(stream)
                ev_log.append((name, e0, e1, e2))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # timed region: bracketed by synchronize on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    fwd_ms = sum(e0.elapsed_time(e1) for _, e0, e1, _ in ev_log) / args.steps
    bwd_launch_ms = [e1.elapsed_time(e2) for _, _, e1, e2 in ev_log]
    bwd_ms = sum(bwd_launch_ms) / args.steps
    per_rel = {}
    for name, e0, e1, e2 in ev_log:
        a = per_rel.setdefault(name, [0.0, 0.0])
        a[0] += e0.elapsed_time(e1) / args.steps
        a[1] += e1.elapsed_time(e2) / args.steps

    tokens = wl.B * wl.N
    value = tokens / (ms_per_step / 1e3)
    fl_f = fl_b = 0.0
    bwd_flops_per_launch = []
    for r in rels:
        h = r.x_t.shape[1]
        f_, b_ = alg_flops(wl.B, h, wl.N, wl.d, causal)
        fl_f += f_
        fl_b += b_
        bwd_flops_per_launch.append(b_)
    # dominant kernel: the backward; achieved = its algorithmic FLOPs per launch divided by
    # its mean launch duration, averaged over launches (one per relation per step)
    n_rel = len(rels)
    ach = []
    for k, ms in enumerate(bwd_launch_ms):
        ach.append(bwd_flops_per_launch[k % n_rel] / (ms / 1e3) / 1e12)
    achieved = sum(ach) / len(ach)
    total_tflops = (fl_f + fl_b) / (ms_per_step / 1e3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H_q": wl.Hq, "H_kv": wl.Hkv, "N": wl.N,
                   "d": wl.d, "relations": ",".join(r.name for r in rels), "causal": causal,
                   "input_dtype": wl.dtype},
        "roofline": {"bound": "mfma", "kernel": "relkl_bwd_kernel",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "alg_tflops_total": round(total_tflops, 1),
        "frac_of_bf16_peak_total": round(total_tflops / PEAK_BF16_TFLOPS, 4),
        "fwd_ms": round(fwd_ms, 3),
        "bwd_ms": round(bwd_ms, 3),
        "per_relation_ms": {k: [round(v[0], 3), round(v[1], 3)] for k, v in per_rel.items()},
        "peak_mem_gb": round(torch.cuda.max_memory_allocated(dev) / 1e9, 3),
        "device": torch.cuda.get_device_name(dev),
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        rows = min(args.cpu_rows, wl.N)
        rel0 = rels[0]
        dt, cores = cpu_baseline(rel0, causal, rows)
        # the oracle's cost is proportional to rows x N (it evaluates full rows), so one
        # unit costs N / rows samples and the step has sum over relations of B * H units
        units = sum(wl.B * r.x_t.shape[1] for r in rels)
        est_step_s = dt * (wl.N / rows) * units
        out["cpu_baseline"] = {
            "value": round(tokens / est_step_s, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"float64 oracle forward+gradient of the last {rows} rows of one "
                       f"{rel0.name} head at N={wl.N} ({dt:.2f}s), extrapolated x{wl.N // rows} "
                       f"rows x {units} units; host {platform.processor() or platform.machine()}"),
            "sample_seconds": round(dt, 3),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
