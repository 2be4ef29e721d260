"""Throughput of the relation-KL hot path (forward + backward of Q/Q, K/K and V/V) on one GPU.

    python bench.py [--steps K] [--warmup W] [--workload llama2_32k] [--no-cpu-baseline]
                    [--no-mem-sweep] [--calibrate-copy MIB]

A step is one pass of the whole path over one batch: for each of the three relations the
forward (LSE statistics + KL) and the backward (recompute + gradient) kernels.  Inputs are
seeded synthetic activations of the workload's shape, resident in HBM before timing.
Prints ONE JSON line.  The dominant kernel (the backward) is timed per launch with HIP
events on the stream it runs on; its algorithmic FLOP count gives the roofline fraction.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "relation-KL fwd+bwd tokens/s at 32 heads,d=128,N=32K; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("attention_relation_distillation_amd/csrc/relkl_kernels.hip",
                  "attention_relation_distillation_amd/csrc/relkl_internal.h")
TRAFFIC_PROFILE = "profiles/relkl_bwd_kernel_llama2_32k_hbm_traffic.md"


def kernel_source_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per backward launch from the committed counter summary, or None when the
    summary is missing, covers another workload, or was taken on other kernel sources."""
    try:
        with open(os.path.join(ROOT, TRAFFIC_PROFILE)) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"traffic: workload=(\S+) bytes_per_launch=(\d+) source_sha256=([0-9a-f]+)",
                  text)
    if not m or m.group(1) != workload or m.group(3) != kernel_source_digest():
        return None
    return int(m.group(2))


COUNTER_PROFILE = "profiles/relkl_kernels_llama2_32k_mfma_valu_counters.md"


def measured_counters(workload):
    """Executed MFMA utilisation and vector / transcendental pressure per kept element of both
    kernels from the committed counter summary (rocprofv3 --pmc), or None when it is missing,
    covers another workload, or was taken on other kernel sources."""
    try:
        with open(os.path.join(ROOT, COUNTER_PROFILE)) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"counters: workload=(\S+) (.*) source_sha256=([0-9a-f]+)", text)
    if not m or m.group(1) != workload or m.group(3) != kernel_source_digest():
        return None
    out = {}
    for kv in m.group(2).split():
        k, v = kv.split("=")
        out[k] = float(v)
    out["source"] = COUNTER_PROFILE
    return out


def alg_flops(B, H, N, d, causal):
    """Algorithmic FLOPs of one relation call: (fwd, bwd).

    Forward: the two score contractions (teacher, student) over the kept entries.
    Backward: the two score recomputations plus the two gradient contractions dZ X_s and
    dZ^T X_s over the same entries.  Kept entries: N(N+1)/2 causal, N^2 otherwise.
    """
    kept = N * (N + 1) / 2 if causal else float(N) * N
    per = 2.0 * d * kept  # one contraction over the kept entries
    return B * H * 2 * per, B * H * 4 * per


def executed_bwd_flops(B, H, N, d):
    """MFMA flops the backward kernel executes per launch (2-byte inputs): every workgroup of 8
    waves owns 256 rows and runs one matrix phase per 32-key block of the whole key range plus
    one (2 key_tiles + 1); a wave's phase issues d/8 score MFMAs (teacher and student) and d/16
    gradient MFMAs of 32x32x16.  Full-row ownership scores every (row, key) pair of the causal
    relation twice, so this is 6/4 of the algorithmic count."""
    row_tiles = -(-N // 256)
    key_tiles = -(-N // 64)
    per_phase = d // 8 + d // 16
    return B * H * row_tiles * (2 * key_tiles + 1) * 8 * per_phase * 2.0 * 32 * 32 * 16


def mfma_ceiling(relkl, torch, dev, iters=2000, reps=5):
    """Dense bf16 MFMA rate the part sustains under a full matrix load (lard_probe_mfma), with
    and without the backward's vector work beside it: TFLOP/s over `reps` timed launches."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * relkl.PROBE_THREADS, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = cus * 8 * iters * relkl.PROBE_MFMA_PER_ITER * relkl.PROBE_FLOPS_PER_MFMA
    out = {}
    for vec in (False, True):
        relkl.probe_mfma(vec, iters, cus, sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            relkl.probe_mfma(vec, iters, cus, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) / reps / 1e3
        out["with_vector_work_tflops" if vec else "pure_tflops"] = round(flops / s / 1e12, 1)
    out["workgroups"] = cus
    return out


_CPU_UNIT = {}


def _cpu_init(x_t, x_s, scale, causal):
    """Pool initializer of cpu_baseline: the unit's inputs, handed to each worker once."""
    _CPU_UNIT.update(x_t=x_t, x_s=x_s, scale=scale, causal=causal)


def _oracle_fwd_rows(rows):
    """Pool task of cpu_baseline: the oracle's forward of some rows of the unit."""
    import oracle
    u = _CPU_UNIT
    lt, ls, kl = oracle.forward_unit(u["x_t"], u["x_s"], u["scale"], u["causal"], chunk=256,
                                     rows=rows)
    return rows, lt, ls


def _oracle_bwd_rows(args):
    """Pool task of cpu_baseline: the oracle's gradient of some rows of the unit."""
    import oracle
    lt, ls, rows = args
    u = _CPU_UNIT
    oracle.backward_unit(u["x_t"], u["x_s"], u["scale"], u["causal"], 1.0, lse_t=lt, lse_s=ls,
                         rows=rows, chunk=256)
    return rows.size


def cpu_baseline(rel, causal, bwd_rows=1024):
    """Time the float64 oracle, as it stands, on the host cores: the forward of one whole
    unit (batch 0, head 0; every row, so the causal mix of row lengths is the real one) and
    the gradient of a uniform sample of `bwd_rows` of its rows (evenly spaced over the
    unit, given the LSE vectors of that forward).  Rows are spread over a process pool
    (fresh interpreters: nothing of this process's GPU state is inherited) sized by the
    cores available to this process (at most 16, the box's share of one GPU) and by host
    RAM, with one BLAS thread per worker.  Returns (unit seconds estimate, details)."""
    import multiprocessing as mp

    import numpy as np
    import oracle

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    host = host_info(avail)
    mem_gb = host.get("ram_gb", 16.0)
    x_t = np.ascontiguousarray(rel.x_t[0, 0].double().numpy())
    x_s = np.ascontiguousarray(rel.x_s[0, 0].double().numpy())
    n = x_t.shape[0]
    scale = oracle.default_scale(x_t.shape[1])
    # ~2 GB per worker at N = 32768 (a few 256 x N float64 blocks plus the inputs)
    workers = int(max(1, min(avail, 16, mem_gb // 2)))
    # forward: 256-row blocks dealt round-robin so that every task mixes short and long rows
    blocks = [np.arange(r0, min(n, r0 + 256)) for r0 in range(0, n, 256)]
    fwd_tasks = [np.concatenate(blocks[k::workers * 2])
                 for k in range(min(len(blocks), workers * 2))]
    sample = np.unique(np.linspace(0, n - 1, min(n, bwd_rows)).round().astype(np.int64))
    env_keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                               "MKL_NUM_THREADS")}
    for k in env_keep:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(workers, initializer=_cpu_init,
                                          initargs=(x_t, x_s, scale, causal)) as pool:
            pool.map(_oracle_fwd_rows, [np.arange(4)] * workers)  # start-up, untimed
            t0 = time.perf_counter()
            parts = pool.map(_oracle_fwd_rows, fwd_tasks, chunksize=1)
            t_fwd = time.perf_counter() - t0
            lt, ls = np.empty(n), np.empty(n)
            for rows, a, b_ in parts:
                lt[rows], ls[rows] = a, b_
            bwd_tasks = [(lt, ls, sample[k::workers]) for k in range(workers)]
            t0 = time.perf_counter()
            pool.map(_oracle_bwd_rows, bwd_tasks, chunksize=1)
            t_bwd = time.perf_counter() - t0
    finally:
        for k, v in env_keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    unit_s = t_fwd + t_bwd * (n / sample.size)
    return unit_s, {"workers": workers, "fwd_unit_s": round(t_fwd, 3),
                    "bwd_sample_rows": int(sample.size), "bwd_sample_s": round(t_bwd, 3),
                    "bwd_scale": round(n / sample.size, 3), "host": host}


def host_info(avail):
    """CPU model, cores available to this process and host RAM, from /proc."""
    info = {"cores_available": avail}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    info["ram_gb"] = round(int(line.split()[1]) / 1e6, 1)
                    break
    except OSError:
        pass
    return info


def mem_sweep(relkl, torch, dev, d=128, H=32, ns=(4096, 8192, 16384, 32768)):
    """Extra device memory of one causal bf16 relation call (fwd + bwd) against N: the peak
    allocation during the call beyond the inputs and the gradient it returns (the forward's
    per-row state, its loss partials and the backward's workspace), next to a materialised
    fp32 relation (H N^2 4 B)."""
    rows = []
    for n in ns:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        g = torch.Generator(device=dev).manual_seed(n)
        xt = torch.randn((1, H, n, d), generator=g, device=dev, dtype=torch.float32).bfloat16()
        xs = (xt.float() + 0.05 * torch.randn(xt.shape, generator=g, device=dev)).bfloat16()
        gl = torch.ones((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        f = relkl.relkl_fwd(xt, xs, causal=True)
        dx = relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], f["diag_delta"], gl, causal=True)
        torch.cuda.synchronize()
        extra = torch.cuda.max_memory_allocated(dev) - base - dx.numel() * dx.element_size()
        state = sum(f[k].numel() * 4 for k in ("lse_t", "lse_s", "diag_delta"))
        rows.append({"N": n, "extra_mb": round(extra / 1e6, 2),
                     "state_mb": round(state / 1e6, 2),
                     "bwd_workspace_mb": round(relkl.workspace_size(xt, xs, pass_=1) / 1e6, 2),
                     "materialised_fp32_gb": round(H * n * n * 4 / 1e9, 2)})
        del xt, xs, f, dx
    # least-squares slope / intercept of extra bytes against N
    xs_ = [r["N"] for r in rows]
    ys_ = [r["extra_mb"] * 1e6 for r in rows]
    mx, my = sum(xs_) / len(xs_), sum(ys_) / len(ys_)
    slope = (sum((x - mx) * (y - my) for x, y in zip(xs_, ys_))
             / sum((x - mx) ** 2 for x in xs_))
    return {"H": H, "d": d, "points": rows, "fit_bytes_per_token": round(slope, 1),
            "fit_intercept_mb": round((my - slope * mx) / 1e6, 3)}


def rope_fused_timing(relkl, workloads, wl, dev, causal, steps, tokens, plain_ms):
    """The RoPE-fused path on the same workload: activations before the rotation and the
    teacher's / student's fp32 tables (Q/Q and K/K; V/V without), forward + backward of
    every relation per step, timed like the main line after one untimed step."""
    import torch
    rels = workloads.make_rope_inputs(wl)
    gpu = []
    for r in rels:
        tabs = [None if t is None else t.to(dev) for t in (r.cos_t, r.sin_t, r.cos_s, r.sin_s)]
        gpu.append((r.name, r.x_t.to(dev), r.x_s.to(dev), tabs))
    gl = torch.ones((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    log = []

    def step(record):
        for name, xt, xs, tabs in gpu:
            if record:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                ev[0].record(stream)
            f = relkl.rope_relkl_fwd(xt, xs, *tabs, causal=causal)
            if record:
                ev[1].record(stream)
            relkl.rope_relkl_bwd(xs, f["reserve"], f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                                 *tabs, causal=causal)
            if record:
                ev[2].record(stream)
                log.append(ev)

    step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    fwd = sum(e[0].elapsed_time(e[1]) for e in log) / steps
    bwd = sum(e[1].elapsed_time(e[2]) for e in log) / steps
    return {"metric": "relation-KL fwd+bwd tokens/s with RoPE applied inside the operation",
            "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "steps": steps,
            "ms_per_step": round(ms, 3), "fwd_ms": round(fwd, 3), "bwd_ms": round(bwd, 3),
            "vs_plain_step": round(ms / plain_ms, 4),
            "rotated": [r.name for r in rels if r.cos_t is not None]}


def cross_timing(relkl, workloads, wl, dev, causal, steps, tokens):
    """The cross relation on the same workload: the attention maps softmax(Q K^T / sqrt(d))
    of teacher and student from the pre-RoPE Q and K draws, rotated inside the call (teacher
    native RoPE, student the workload's), gradients to the student's Q and K; one call per
    step over all heads, timed like the main line after one untimed step."""
    import torch
    rels = {r.name: r for r in workloads.make_rope_inputs(wl, relations=("qq", "kk"))}
    q, k = rels["qq"], rels["kk"]
    if q.x_t.shape != k.x_t.shape:
        return {"skipped": "query and key head counts differ"}
    a_t, b_t = q.x_t.to(dev), k.x_t.to(dev)
    a_s, b_s = q.x_s.to(dev), k.x_s.to(dev)
    tabs = [t.to(dev) for t in (q.cos_t, q.sin_t, q.cos_s, q.sin_s)]
    gl = torch.ones((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    log = []

    def step(record):
        if record:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
        f = relkl.cross_relkl_fwd(a_t, b_t, a_s, b_s, rope=tabs, causal=causal)
        if record:
            ev[1].record(stream)
        relkl.cross_relkl_bwd(a_s, b_s, f["reserve"], f["lse_t"], f["lse_s"], gl, rope=tabs,
                              causal=causal)
        if record:
            ev[2].record(stream)
            log.append(ev)

    step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    fwd = sum(e[0].elapsed_time(e[1]) for e in log) / steps
    bwd = sum(e[1].elapsed_time(e[2]) for e in log) / steps
    h = q.x_t.shape[1]
    fl_f, fl_b = alg_flops(wl.B, h, wl.N, wl.d, causal)
    ach = fl_b / (bwd / 1e3) / 1e12
    return {"metric": "cross-relation (Q K^T attention map, RoPE inside) fwd+bwd tokens/s",
            "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "steps": steps,
            "ms_per_step": round(ms, 3), "fwd_ms": round(fwd, 3), "bwd_ms": round(bwd, 3),
            "roofline": {"bound": "mfma", "kernel": "relkl_bwd_kernel (dA and dB passes)",
                         "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                         "alg_flops_per_call": fl_b}}


def group_timing(relkl, workloads, dev, steps):
    """Every relation of a layer in one grouped call (one launch of each kernel) against one
    call per relation, fwd + bwd per step: on the GQA shapes (Q/Q on 32 query heads, K/K and
    V/V on 8 KV heads, N = 16384) and on the 4K LLaMA2 shapes, where each relation's grid is
    small.  Two interleaved rounds of `steps` steps each; the faster round of each counts."""
    import torch
    gl = torch.ones((), dtype=torch.float32, device=dev)
    res = {}
    for name in ("gqa_16k", "llama2_4k"):
        wl = workloads.WORKLOADS[name]
        causal = wl.masks[0]
        pairs = [(r.x_t.to(dev), r.x_s.to(dev)) for r in workloads.make_inputs(wl)]

        def separate():
            for xt, xs in pairs:
                f = relkl.relkl_fwd(xt, xs, causal=causal)
                relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                                causal=causal)

        def grouped():
            f = relkl.group_relkl_fwd(pairs, causal=causal)
            relkl.group_relkl_bwd(pairs, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                                  causal=causal)

        best = {}
        for fn, label in ((separate, "separate"), (grouped, "group")) * 2:
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            best[label] = min(ms, best.get(label, float("inf")))
        tokens = wl.B * wl.N
        res[name] = {"heads": [p[0].shape[1] for p in pairs], "N": wl.N, "steps": steps,
                     "separate_ms_per_step": round(best["separate"], 3),
                     "group_ms_per_step": round(best["group"], 3),
                     "group_tokens_per_s": round(tokens / (best["group"] / 1e3), 1),
                     "separate_tokens_per_s": round(tokens / (best["separate"] / 1e3), 1),
                     "speedup": round(best["separate"] / best["group"], 4)}
        del pairs
    return {"metric": "relation-KL fwd+bwd tokens/s, all relations of a layer in one grouped "
                      "call vs one call per relation", **res}


def stats_ms(v):
    return {"median": round(statistics.median(v), 3), "min": round(min(v), 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time the oracle sample is sized to")
    ap.add_argument("--no-mem-sweep", action="store_true")
    ap.add_argument("--rope-steps", type=int, default=5,
                    help="timed steps of the RoPE-fused path on the same workload (0: skip)")
    ap.add_argument("--cross-steps", type=int, default=5,
                    help="timed steps of the cross relation (attention maps Q K^T with RoPE "
                         "inside) on the same workload (0: skip)")
    ap.add_argument("--group-steps", type=int, default=10,
                    help="timed steps of the grouped call against per-relation calls on the "
                         "GQA 16K and LLaMA2 4K shapes (0: skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the steps, copy a MIB-MiB buffer three times (a plain copy "
                         "kernel of known size, for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the relation-KL "
              "library runs on a single GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_relation_distillation_amd import relkl, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    relkl.load_library()
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

    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {args.calibrate_copy} MiB", file=sys.stderr,
              flush=True)
        del src, dst

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
            relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], f["diag_delta"], gl, causal=causal)
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
    print("[bench] timed steps done", file=sys.stderr, flush=True)

    fwd_launch_ms = [e0.elapsed_time(e1) for _, e0, e1, _ in ev_log]
    bwd_launch_ms = [e1.elapsed_time(e2) for _, _, e1, e2 in ev_log]
    fwd_ms = sum(fwd_launch_ms) / args.steps
    bwd_ms = sum(bwd_launch_ms) / args.steps
    n_rel_launch = len(gpu)
    step_gpu_ms = [sum(e0.elapsed_time(e2) for _, e0, _, e2 in ev_log[k:k + n_rel_launch])
                   for k in range(0, len(ev_log), n_rel_launch)]
    per_rel = {}
    for name, e0, e1, e2 in ev_log:
        a = per_rel.setdefault(name, ([], []))
        a[0].append(e0.elapsed_time(e1))
        a[1].append(e1.elapsed_time(e2))

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
    # its mean launch duration (launches of all relations pooled; equal shapes here)
    n_rel = len(rels)
    mean_bwd_flops = sum(bwd_flops_per_launch) / n_rel
    mean_bwd_s = sum(bwd_launch_ms) / len(bwd_launch_ms) / 1e3
    achieved = mean_bwd_flops / mean_bwd_s / 1e12
    total_tflops = (fl_f + fl_b) / (ms_per_step / 1e3) / 1e12
    traffic = measured_traffic(wl.name)
    counters = measured_counters(wl.name)

    props = torch.cuda.get_device_properties(dev)
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
                     "traffic": traffic,
                     "alg_flops_per_launch": mean_bwd_flops,
                     "mean_launch_ms": round(mean_bwd_s * 1e3, 3)},
        "executed_counters": counters,
        "mfma_ceiling": None,
        "alg_tflops_total": round(total_tflops, 1),
        "frac_of_bf16_peak_total": round(total_tflops / PEAK_BF16_TFLOPS, 4),
        "fwd_ms": round(fwd_ms, 3),
        "bwd_ms": round(bwd_ms, 3),
        "step_kernel_ms": stats_ms(step_gpu_ms),
        "per_relation_ms": {k: {"fwd": stats_ms(v[0]), "bwd": stats_ms(v[1])}
                            for k, v in per_rel.items()},
        "peak_mem_gb": round(torch.cuda.max_memory_allocated(dev) / 1e9, 3),
        "device": f"{props.name} ({getattr(props, 'gcnArchName', '?')}, "
                  f"{props.multi_processor_count} CUs)",
        "kernel_sources": kernel_source_digest(),
        "cpu_baseline": None,
    }

    # the dense bf16 rate the part sustains beside the published peak, and the backward's
    # executed MFMA rate against it (full-row ownership executes 6/4 of the algorithmic work)
    ceil = mfma_ceiling(relkl, torch, dev)
    ex_b = sum(executed_bwd_flops(wl.B, r.x_t.shape[1], wl.N, wl.d) for r in rels) / n_rel
    ceil["bwd_executed_tflops"] = round(ex_b / mean_bwd_s / 1e12, 1)
    ceil["bwd_executed_frac_of_pure"] = round(ex_b / mean_bwd_s / 1e12 / ceil["pure_tflops"], 4)
    out["mfma_ceiling"] = ceil
    print("[bench] MFMA ceiling probe done", file=sys.stderr, flush=True)

    if args.rope_steps > 0:
        out["next_rows"] = {"rope_fused": rope_fused_timing(relkl, workloads, wl, dev, causal,
                                                             args.rope_steps, tokens, ms_per_step)}
        print("[bench] RoPE-fused timing done", file=sys.stderr, flush=True)
    if args.cross_steps > 0:
        out.setdefault("next_rows", {})["cross_attention_map"] = cross_timing(
            relkl, workloads, wl, dev, causal, args.cross_steps, tokens)
        print("[bench] cross-relation timing done", file=sys.stderr, flush=True)

    if args.group_steps > 0:
        out.setdefault("next_rows", {})["single_launch_group"] = group_timing(
            relkl, workloads, dev, args.group_steps)
        print("[bench] grouped-call timing done", file=sys.stderr, flush=True)

    if not args.no_mem_sweep:
        del gpu
        out["extra_memory_vs_N"] = mem_sweep(relkl, torch, dev)
        print("[bench] memory sweep done", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        rel0 = rels[0]
        unit_s, det = cpu_baseline(rel0, causal)
        units = sum(wl.B * r.x_t.shape[1] for r in rels)
        est_step_s = unit_s * units
        out["cpu_baseline"] = {
            "value": round(tokens / est_step_s, 3), "unit": "tokens/s",
            "cores": det["workers"], "kind": "oracle",
            "sample": (f"float64 oracle on {det['workers']} host processes: forward of one whole "
                       f"{rel0.name} unit at N={wl.N} ({det['fwd_unit_s']:.2f}s) plus the "
                       f"gradient of {det['bwd_sample_rows']} evenly spaced rows of it "
                       f"({det['bwd_sample_s']:.2f}s, x{det['bwd_scale']:.1f} to the unit); "
                       f"extrapolated (labelled as such) x{units} units of a step"),
            "unit_seconds": round(unit_s, 3),
            "extrapolated": True,
            "extrapolation_factor": units,
            "host": det["host"],
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
