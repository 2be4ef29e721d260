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
# The row-KL vector (relative L2), for either dtype (the forward's arithmetic is fp32 for
# both).  A row's KL is formed from lambda_t - lambda_s (lambda: the row's off-diagonal mass
# relative to its diagonal), two fp32 sums that each carry a few units of 2^-24 relative
# error, against a KL of about lambda Var(delta) / 2 (delta: the teacher-student logit gap
# along the row): a relative error of about 4 2^-24 sqrt(2) 2 / Var(delta), i.e. ~1.4e-4
# for V/V rows (Var(delta) ~ 0.005), far less for Q/Q and K/K.  The loss sums many rows.
ROW_KL_RL2 = 3e-4


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


TABLE_LINES = []  # repeated at the end of the session by the terminal-summary hook


def table(line: str):
    """Print one per-workload parity line and keep it for the session's closing summary."""
    line = f"[table] {line}"
    print(line, flush=True)
    TABLE_LINES.append(line)


def state(f):
    """The forward's per-row state the backward takes: (lse_t, lse_s, diag_delta)."""
    return f["lse_t"], f["lse_s"], f["diag_delta"]


def gpu_fwd_bwd(x_t, x_s, causal, head_map=None, dx_dtype=None, scale=None, g=1.0):
    dev = device()
    xt, xs = x_t.to(dev), x_s.to(dev)
    f = relkl.relkl_fwd(xt, xs, causal=causal, head_map=head_map, want_row_kl=True, scale=scale)
    gl = torch.tensor(g, dtype=torch.float32, device=dev)
    dx = relkl.relkl_bwd(xt, xs, *state(f), gl, causal=causal, head_map=head_map,
                         dx_dtype=dx_dtype, scale=scale)
    torch.cuda.synchronize()
    return f, dx


def diag_delta_ref(xt, xs, scale, lse_t, lse_s, head_map=None):
    """R_s(i,i) - R_t(i,i) from its definition: R_m(i,i) = exp(scale |x_m,i|^2 - LSE_m(i)), in
    float64 on the inputs' exact values and the oracle's LSE vectors ([B, H, N])."""
    if head_map is not None:
        xt, xs = xt[:, head_map], xs[:, head_map]
    zt = scale * np.einsum("bhnd,bhnd->bhn", xt, xt)
    zs = scale * np.einsum("bhnd,bhnd->bhn", xs, xs)
    return np.exp(zs - lse_s) - np.exp(zt - lse_t)


def diag_delta_tol(xt, xs, scale):
    """Absolute gate of diag_delta = R_s(i,i) - R_t(i,i) = 1/(1 + lam_s) - 1/(1 + lam_t), lam the
    row's off-diagonal mass relative to its diagonal.  Every off-diagonal exponential carries the
    fp32 rounding of its score S, a relative error of about ln2 scale log2(e) 2^-24 |S| (a few
    times that over the accumulation), and the error of 1/(1 + lam) is at most a quarter of lam's
    relative error; |S| <= max |x|^2 by Cauchy-Schwarz.  Hence 1e-7 + 4 2^-24 scale max |x|^2:
    about 4e-6 on the workloads (d = 128, N(0, 1) rows), more where rows carry large norms."""
    sq = max(float(np.max(np.einsum("...d,...d->...", xt, xt))),
             float(np.max(np.einsum("...d,...d->...", xs, xs))))
    return 1e-7 + 4.0 * 2.0 ** -24 * scale * sq


def oracle_fwd_bwd(x_t, x_s, causal, head_map=None, scale=None, g=1.0):
    d = x_t.shape[-1]
    s = oracle.default_scale(d) if scale is None else scale
    xt, xs = np64(x_t), np64(x_s)
    f = oracle.forward(xt, xs, s, causal, head_map=head_map)
    f["diag_delta"] = diag_delta_ref(xt, xs, s, f["lse_t"], f["lse_s"], head_map)
    f["diag_delta_tol"] = diag_delta_tol(xt, xs, s)
    dx = oracle.backward(xt, xs, s, causal, g, head_map=head_map)
    return f, dx


def tiny_n_floor(fo, x_s, scale):
    """Absolute error floors of fp32 arithmetic for rows with only a handful of entries
    (N < 64 in the edge-size tests; also the closed-form goldens, whose rows are all alike):
    there a row's KL is a difference of terms of size |LSE| (the diagonal's nearly-one
    probability against a few tiny off-diagonal ones), and the fp32 LSE that normalises
    every probability carries a relative error of a few ulps of |LSE|.

    Loss: 2^-24 (1 + max|LSE|) per row.  Gradient: each probability is exp(z - LSE) with
    LSE in fp32, so its relative error is eta = 2^-20 (1 + max|LSE|), and a gradient row
    sums |R| |x| over at most 4 units of probability (row and transposed terms)."""
    lse_max = float(max(np.max(np.abs(fo["lse_t"])), np.max(np.abs(fo["lse_s"]))))
    eta = 2.0 ** -20 * (1.0 + lse_max)
    rows = fo["row_kl"].size
    loss_floor = 2.0 ** -24 * (1.0 + lse_max) * rows
    xs = np64(x_s)
    row_norm_max = float(np.sqrt(np.max(np.sum(xs * xs, axis=-1))))
    grad_floor = 4.0 * eta * scale * row_norm_max * np.sqrt(xs.shape[0] * xs.shape[1] * xs.shape[2])
    return loss_floor, grad_floor


def assert_parity(f, dx, fo, dxo, dtype, label="", floor=None, row_kl_rl2=ROW_KL_RL2,
                  grad_dtype=None):
    """Compare GPU outputs with the oracle at the dtype's gates; returns diagnostics.

    floor: None, or (loss_floor, grad_floor) from tiny_n_floor for the named tiny-N edge
    cases, added to the gates there.  row_kl_rl2: the row-KL gate (a named case may
    derive its own).  grad_dtype: the gradient output's dtype when it differs from the
    inputs' (its gate is that dtype's)."""
    loss = float(f["loss"].item())
    loss_abs = abs(loss - fo["loss"])
    loss_err = loss_abs / max(abs(fo["loss"]), 1e-30)
    lse_err = max(float(np.max(np.abs(np64(f["lse_t"]) - fo["lse_t"]))),
                  float(np.max(np.abs(np64(f["lse_s"]) - fo["lse_s"]))))
    kl_got = np64(f["row_kl"])
    kl_abs = float(np.linalg.norm(kl_got - fo["row_kl"]))
    kl_err = rel_l2(kl_got, fo["row_kl"])
    g_abs = float(np.linalg.norm(np64(dx) - dxo))
    g_err = rel_l2(np64(dx), dxo)
    diag = dict(loss=loss, loss_ref=fo["loss"], loss_rel=loss_err, lse_abs=lse_err,
                row_kl_rl2=kl_err, grad_rl2=g_err)
    if "diag_delta" in fo and "diag_delta" in f:
        diag["diag_delta_abs"] = float(np.max(np.abs(np64(f["diag_delta"]) - fo["diag_delta"])))
    loss_floor = grad_floor = 0.0
    if floor is not None:
        loss_floor, grad_floor = floor
        diag.update(loss_floor=loss_floor, grad_floor=grad_floor, grad_abs=g_abs)
    print(f"[parity] {label} {diag}", flush=True)
    assert loss_abs <= LOSS_RTOL[dtype] * abs(fo["loss"]) + loss_floor, diag
    assert kl_abs <= row_kl_rl2 * float(np.linalg.norm(fo["row_kl"])) + loss_floor, diag
    gd = dtype if grad_dtype is None else grad_dtype  # the gradient's output dtype's gate
    assert g_abs <= GRAD_RL2[gd] * float(np.linalg.norm(dxo)) + grad_floor, diag
    assert lse_err <= 5e-5 * max(1.0, float(np.max(np.abs(fo["lse_t"])))), diag
    if "diag_delta_abs" in diag:  # gate derived in diag_delta_tol
        assert diag["diag_delta_abs"] <= fo["diag_delta_tol"], diag
    return diag
