"""Shared helpers of the GPU parity tests (no test functions here)."""

import os

import numpy as np
import pytest
import torch

import oracle
from attention_relation_distillation_amd import relkl

# Gates (loss: relative error; gradient: relative L2 error) by input dtype.
LOSS_RTOL = {torch.bfloat16: 1e-4, torch.float32: 1e-5}
GRAD_RL2 = {torch.bfloat16: 2e-3, torch.float32: 1e-4}


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def banner(msg: str):
    print(f"[case] {msg}", flush=True)


def gpu_fwd_bwd(x_t, x_s, causal, head_map=None, dx_dtype=None, scale=None, g=1.0):
    dev = device()
    xt, xs = x_t.to(dev), x_s.to(dev)
    f = relkl.relkl_fwd(xt, xs, causal=causal, head_map=head_map, want_row_kl=True, scale=scale)
    gl = torch.tensor(g, dtype=torch.float32, device=dev)
    dx = relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], gl, causal=causal, head_map=head_map,
                         dx_dtype=dx_dtype, scale=scale)
    torch.cuda.synchronize()
    return f, dx


def oracle_fwd_bwd(x_t, x_s, causal, head_map=None, scale=None, g=1.0):
    d = x_t.shape[-1]
    s = oracle.default_scale(d) if scale is None else scale
    xt, xs = np64(x_t), np64(x_s)
    f = oracle.forward(xt, xs, s, causal, head_map=head_map)
    dx = oracle.backward(xt, xs, s, causal, g, head_map=head_map)
    return f, dx


def assert_parity(f, dx, fo, dxo, dtype, label="", dx_out_dtype=None):
    """Compare GPU outputs with the oracle at the dtype's gates; returns diagnostics."""
    loss = float(f["loss"].item())
    loss_err = abs(loss - fo["loss"]) / max(abs(fo["loss"]), 1e-30)
    lse_err = max(float(np.max(np.abs(np64(f["lse_t"]) - fo["lse_t"]))),
                  float(np.max(np.abs(np64(f["lse_s"]) - fo["lse_s"]))))
    kl_err = rel_l2(np64(f["row_kl"]), fo["row_kl"])
    g_err = rel_l2(np64(dx), dxo)
    diag = dict(loss=loss, loss_ref=fo["loss"], loss_rel=loss_err, lse_abs=lse_err,
                row_kl_rl2=kl_err, grad_rl2=g_err)
    print(f"[parity] {label} {diag}", flush=True)
    assert loss_err <= LOSS_RTOL[dtype], diag
    gate = GRAD_RL2[dtype]
    assert g_err <= gate, diag
    assert lse_err <= 5e-5 * max(1.0, float(np.max(np.abs(fo["lse_t"])))), diag
    return diag
