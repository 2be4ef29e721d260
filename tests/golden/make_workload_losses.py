"""Write tests/golden/workload_losses.json: the float64 oracle's loss of every relation of
the full-size workloads, per (batch, head) unit and in total, plus LSE and row KL of a fixed
sample of rows of two units per relation.

    python tests/golden/make_workload_losses.py [--workers 6] [--only llama2_32k ...]

Calls only ``oracle`` (the plain float64 definition, materialising every row in blocks of
rows) on the seeded inputs of ``attention_relation_distillation_amd.workloads``; nothing
here touches the GPU library.  The full-size oracle takes tens of CPU minutes, which is why
its results are stored: the GPU tests compare against these numbers.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, "1")

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from attention_relation_distillation_amd import workloads  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "workload_losses.json")
CASES = [("llama2_32k", True), ("batched_8k", True), ("batched_8k", False), ("gqa_16k", True)]
CHUNK = 512

_INPUTS = {}  # filled in the parent before the pool forks


def sample_rows(n: int) -> list:
    """Fixed rows (first, tile and half boundaries, last) plus a seeded spread."""
    r = np.random.default_rng(n)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 255, 256, n // 2, n - 2, n - 1]
    spread = r.integers(0, n, size=10).tolist()
    return sorted(set(v for v in fixed + spread if 0 <= v < n))


def sample_units(B: int, H: int) -> list:
    return [(0, 0), (B - 1, H - 1)]


def unit_task(args):
    key, rel, b, h, causal, want_rows = args
    x_t, x_s, scale = _INPUTS[(key, rel)]
    ut = x_t[b, h].double().numpy()
    us = x_s[b, h].double().numpy()
    lt, ls, kl = oracle.forward_unit(ut, us, scale, causal, chunk=CHUNK)
    out = {"b": b, "h": h, "loss": float(kl.sum())}
    if want_rows:
        rows = sample_rows(ut.shape[0])
        out["rows"] = rows
        out["lse_t"] = [float(v) for v in lt[rows]]
        out["lse_s"] = [float(v) for v in ls[rows]]
        out["row_kl"] = [float(v) for v in kl[rows]]
    return out


def run_case(name: str, causal: bool, workers: int) -> dict:
    wl = workloads.WORKLOADS[name]
    t0 = time.time()
    rels = workloads.make_inputs(wl)
    scale = oracle.default_scale(wl.d)
    key = f"{name}/{'causal' if causal else 'noncausal'}"
    tasks = []
    for r in rels:
        _INPUTS[(key, r.name)] = (r.x_t, r.x_s, scale)
        B, H = r.x_t.shape[0], r.x_t.shape[1]
        picks = sample_units(B, H)
        for b in range(B):
            for h in range(H):
                tasks.append((key, r.name, b, h, causal, (b, h) in picks))
    print(f"[golden] {key}: {len(tasks)} units, inputs in {time.time() - t0:.1f}s", flush=True)
    with mp.get_context("fork").Pool(workers) as pool:
        results = pool.map(unit_task, tasks, chunksize=1)
    entry = {"N": wl.N, "d": wl.d, "B": wl.B, "scale": scale, "causal": causal,
             "chunk_rows": CHUNK, "relations": {}}
    for r in rels:
        mine = [res for task, res in zip(tasks, results) if task[1] == r.name]
        H = r.x_t.shape[1]
        units = sorted(mine, key=lambda u: (u["b"], u["h"]))
        entry["relations"][r.name] = {
            "H": H,
            "loss": float(sum(u["loss"] for u in units)),
            "unit_loss": [u["loss"] for u in units],
            "samples": [{k: u[k] for k in ("b", "h", "rows", "lse_t", "lse_s", "row_kl")}
                        for u in units if "rows" in u],
        }
        del _INPUTS[(key, r.name)]
    print(f"[golden] {key}: done in {time.time() - t0:.1f}s; losses "
          + ", ".join(f"{k} {v['loss']:.9g}" for k, v in entry["relations"].items()), flush=True)
    return key, entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=6)
    ap.add_argument("--only", nargs="*", default=None, help="workload names to (re)compute")
    args = ap.parse_args()
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    data.setdefault("about", (
        "float64 oracle (oracle.forward_unit, rows materialised in blocks of "
        f"{CHUNK}) on the seeded full-size workloads of workloads.make_inputs (seed 0); "
        "written by tests/golden/make_workload_losses.py"))
    data.setdefault("cases", {})
    for name, causal in CASES:
        if args.only and name not in args.only:
            continue
        key, entry = run_case(name, causal, args.workers)
        data["cases"][key] = entry
        with open(OUT, "w") as f:  # saved after every case
            json.dump(data, f, indent=1)
    print(f"[golden] wrote {OUT}", flush=True)


if __name__ == "__main__":
    main()
