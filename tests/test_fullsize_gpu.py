"""Full-size parity on the workload shapes, in the launch configuration bench.py times.

The float64 oracle's loss of every relation at full size -- per (batch, head) unit and in
total -- and its LSE and row KL on a fixed sample of rows are stored in
tests/golden/workload_losses.json (written by tests/golden/make_workload_losses.py, which
calls only the oracle; the full-size oracle takes tens of CPU minutes).  Here every
relation's loss and every unit's loss are held to the bf16 loss gate against those values,
the sampled rows to the LSE and row-KL gates, and sampled gradient rows of one unit per
relation to the gradient gate (computed here by the oracle row by row: O(N d) per row once
the LSE of the rows they touch is known).  Properties that hold at any size are checked on
every output: finite values, KL >= 0 up to fp32 noise, loss equal to the sum of the row KLs.
Each relation prints one "[table]" line (repeated in the session summary): loss error, max |dLSE| and row-KL relative L2 on
the sampled rows, gradient relative L2 on the sampled gradient rows."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import (GRAD_RL2, LOSS_RTOL, ROW_KL_RL2, banner, device, diag_delta_ref,
                        diag_delta_tol, np64, rel_l2, table)

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "workload_losses.json")


def golden(key):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert key in cases, f"{key} missing from {GOLDEN}"
    return cases[key]


def grad_rows(n, causal, seed):
    r = np.random.default_rng(seed)
    if causal and n > 4096:
        # long causal rows: the last 1024 rows; their column terms involve rows j >= i only,
        # so only those rows' LSE is needed
        rows = [n - 1024, n - 513, n - 257, n - 1] + r.integers(n - 1024, n, 4).tolist()
        return np.array(sorted(set(rows))), np.arange(n - 1024, n)
    rows = [0, 1, 255, 256, n // 2, n - 1] + r.integers(0, n, 4).tolist()
    return np.array(sorted(set(rows))), np.arange(n)


def check_workload(name, causal):
    key = f"{name}/{'causal' if causal else 'noncausal'}"
    ref = golden(key)
    wl = workloads.WORKLOADS[name]
    banner(f"full-size {key}: generating inputs")
    rels = workloads.make_inputs(wl)
    dev = device()
    scale = oracle.default_scale(wl.d)
    assert ref["N"] == wl.N and ref["scale"] == scale
    for rel in rels:
        r_ref = ref["relations"][rel.name]
        banner(f"{key} {rel.name}: GPU fwd+bwd")
        xt, xs = rel.x_t.to(dev), rel.x_s.to(dev)
        f = relkl.relkl_fwd(xt, xs, causal=causal, want_row_kl=True)
        gl = torch.ones((), dtype=torch.float32, device=dev)
        dx = relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], f["diag_delta"], gl, causal=causal)
        torch.cuda.synchronize()
        loss = float(f["loss"].item())
        row_kl = np64(f["row_kl"])
        lse_t, lse_s = np64(f["lse_t"]), np64(f["lse_s"])
        assert np.isfinite(loss) and loss > 0
        assert np.all(np.isfinite(row_kl)) and np.all(np.isfinite(lse_t))
        assert row_kl.min() >= -1e-5, row_kl.min()
        assert abs(loss - row_kl.sum()) <= 1e-6 * abs(loss) + 1e-6
        assert torch.isfinite(dx.float()).all()
        B, H, N = row_kl.shape
        # the relation's loss and every unit's loss against the stored float64 oracle
        loss_rel = abs(loss - r_ref["loss"]) / r_ref["loss"]
        unit_got = row_kl.sum(axis=-1).reshape(-1)
        unit_ref = np.array(r_ref["unit_loss"])
        unit_rel = np.abs(unit_got - unit_ref) / unit_ref
        # sampled rows: LSE, row KL and diag_delta = R_s(i,i) - R_t(i,i), the last from its
        # definition with the stored oracle LSE
        dlse, kl_got, kl_ref, ddiff = 0.0, [], [], 0.0
        dd = np64(f["diag_delta"])
        assert rel.head_map is None  # the calls above read every input head
        for smp in r_ref["samples"]:
            b, h, rows = smp["b"], smp["h"], np.array(smp["rows"])
            dlse = max(dlse, float(np.max(np.abs(lse_t[b, h, rows] - smp["lse_t"]))),
                       float(np.max(np.abs(lse_s[b, h, rows] - smp["lse_s"]))))
            kl_got.append(row_kl[b, h, rows])
            kl_ref.append(np.array(smp["row_kl"]))
            xt_r = rel.x_t[b, h, rows].double().numpy()
            xs_r = rel.x_s[b, h, rows].double().numpy()
            dd_ref = (np.exp(scale * np.sum(xs_r * xs_r, axis=1) - np.array(smp["lse_s"]))
                      - np.exp(scale * np.sum(xt_r * xt_r, axis=1) - np.array(smp["lse_t"])))
            ddiff = max(ddiff, float(np.max(np.abs(dd[b, h, rows] - dd_ref))))
        # the gate of diag_delta_tol, with max |x|^2 taken in fp32 over the full-size tensors
        sq = max(float(rel.x_t.float().square().sum(-1).max()),
                 float(rel.x_s.float().square().sum(-1).max()))
        dd_tol = 1e-7 + 4.0 * 2.0 ** -24 * scale * sq * (1 + 1e-5)
        kl_rl2 = rel_l2(np.concatenate(kl_got), np.concatenate(kl_ref))
        lse_max = max(abs(v) for smp in r_ref["samples"] for v in smp["lse_t"] + smp["lse_s"])
        # sampled gradient rows of the first unit
        banner(f"{key} {rel.name}: oracle gradient of sampled rows")
        ut = rel.x_t[0, 0].double().numpy()
        us = rel.x_s[0, 0].double().numpy()
        rows, need = grad_rows(N, causal, seed=3)
        flt, fls = np.full(N, np.nan), np.full(N, np.nan)
        flt[need], fls[need], _ = oracle.forward_unit(ut, us, scale, causal, chunk=1024,
                                                       rows=need)
        g_ref = oracle.backward_unit(ut, us, scale, causal, 1.0, lse_t=flt, lse_s=fls,
                                     rows=rows, chunk=1024)
        g_rl2 = rel_l2(np64(dx[0, 0])[rows], g_ref)
        table(f"{key} {rel.name} loss_rel {loss_rel:.2e} unit_rel_max "
              f"{unit_rel.max():.2e} max_dlse {dlse:.2e} row_kl_rl2 {kl_rl2:.2e} "
              f"grad_rl2 {g_rl2:.2e} max_ddiag {ddiff:.2e}")
        assert loss_rel <= LOSS_RTOL[torch.bfloat16]
        assert np.all(unit_rel <= LOSS_RTOL[torch.bfloat16]), unit_rel.max()
        assert dlse <= 5e-5 * max(1.0, lse_max)
        assert kl_rl2 <= ROW_KL_RL2
        assert g_rl2 <= GRAD_RL2[torch.bfloat16]
        assert ddiff <= dd_tol, (ddiff, dd_tol)
        del xt, xs, f, dx


def test_llama2_4k_full():
    """The 4K workload: every output against the oracle in full (it fits in seconds)."""
    wl = workloads.WORKLOADS["llama2_4k"]
    dev = device()
    scale = oracle.default_scale(wl.d)
    for rel in workloads.make_inputs(wl):
        banner(f"llama2_4k {rel.name}: GPU fwd+bwd")
        xt, xs = rel.x_t.to(dev), rel.x_s.to(dev)
        f = relkl.relkl_fwd(xt, xs, causal=True, want_row_kl=True)
        gl = torch.ones((), dtype=torch.float32, device=dev)
        dx = relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], f["diag_delta"], gl, causal=True,
                             dx_dtype=torch.float32)
        torch.cuda.synchronize()
        banner(f"llama2_4k {rel.name}: full oracle")
        x_t, x_s = rel.x_t.double().numpy(), rel.x_s.double().numpy()
        fo = oracle.forward(x_t, x_s, scale, True, chunk=1024)
        loss_rel = abs(float(f["loss"].item()) - fo["loss"]) / fo["loss"]
        dlse = max(float(np.max(np.abs(np64(f["lse_t"]) - fo["lse_t"]))),
                   float(np.max(np.abs(np64(f["lse_s"]) - fo["lse_s"]))))
        kl_rl2 = rel_l2(np64(f["row_kl"]), fo["row_kl"])
        dd_err = float(np.max(np.abs(np64(f["diag_delta"])
                                     - diag_delta_ref(x_t, x_s, scale, fo["lse_t"], fo["lse_s"]))))
        # gradient of two whole heads (the oracle's full backward per unit)
        g_err = []
        for h in (0, wl.Hq - 1):
            g_ref = oracle.backward_unit(x_t[0, h], x_s[0, h], scale, True, 1.0,
                                         lse_t=fo["lse_t"][0, h], lse_s=fo["lse_s"][0, h],
                                         chunk=1024)
            g_err.append(rel_l2(np64(dx[0, h]), g_ref))
        table(f"llama2_4k/causal {rel.name} loss_rel {loss_rel:.2e} max_dlse "
              f"{dlse:.2e} row_kl_rl2 {kl_rl2:.2e} grad_rl2 {max(g_err):.2e} (fp32 output) "
              f"max_ddiag {dd_err:.2e}")
        assert dd_err <= diag_delta_tol(x_t, x_s, scale), dd_err
        assert loss_rel <= LOSS_RTOL[torch.bfloat16]
        assert dlse <= 5e-5 * max(1.0, float(np.max(np.abs(fo["lse_t"]))))
        assert kl_rl2 <= ROW_KL_RL2
        assert max(g_err) <= GRAD_RL2[torch.bfloat16]
        del xt, xs, f, dx


def test_llama2_32k_full_loss():
    check_workload("llama2_32k", True)


def test_batched_8k_causal_full_loss():
    check_workload("batched_8k", True)


def test_batched_8k_noncausal_full_loss():
    check_workload("batched_8k", False)


def test_gqa_16k_full_loss():
    check_workload("gqa_16k", True)
