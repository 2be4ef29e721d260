"""Float64 CPU oracle for the attention-relation KL loss of LinearARD and its gradient.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports nothing from it.

What it computes (page "LinearARD ... verdict" on pith.science, fields
``pith_extraction.key_machinery`` and ``core_discovery``; arXiv abstract on mlsanity.com):

* For one attention head and one relation X in {Q, K, V}, teacher (t) and student (s)
  each form logits Z_m = scale * X_m X_m^T + M, with M the mask, and the masked
  row-softmax relation R_m = softmax_rows(Z_m).
* Per row i, the forward KL divergence KL_i = sum_j R_t(i,j) (log R_t(i,j) - log R_s(i,j)).
* The loss returned here is the plain SUM of KL_i over rows (and over batch and heads in
  the batched helpers).  The pages' 1/n mean is the same quantity times 1/n; a caller gets
  it by passing g = 1/n as the upstream gradient.
* The gradient of the loss with respect to a student logit is g * (R_s(i,j) - R_t(i,j))
  (the identity stated in key_machinery; there with the 1/n factor).  The student
  matrix X_s appears on both sides of X_s X_s^T, so
  dL/dX_s = scale * (dZ + dZ^T) X_s with dZ = g * (R_s - R_t), zero where masked.
  The teacher is frozen and gets no gradient (the abstract describes the teacher as a
  fixed model with native RoPE).

Readings where the pages are silent (all listed in the design notes):
* causal mask keeps j <= i (diagonal included); non-causal keeps everything;
  excluded entries contribute exactly 0 to the KL (0 log 0 = 0) and to dZ;
* the scale is whatever value the caller gives (normally the float32 rounding of
  1/sqrt(d)), used unchanged for teacher and student;
* KL in nats (natural log).

Every function below is the plain definition: the N x N logit matrices are materialised
(optionally a block of rows at a time, which changes nothing in the arithmetic of any
single row), numpy float64 throughout, BLAS matmul as the only library step.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "default_scale",
    "keep_mask",
    "logits",
    "row_lse",
    "forward_unit",
    "backward_unit",
    "forward",
    "backward",
]


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32, returned as the exact float64 of that float32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def keep_mask(rows: np.ndarray, cols: np.ndarray, causal: bool) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: True where entry (i, j) takes part (j <= i if causal)."""
    if not causal:
        return np.ones((rows.size, cols.size), dtype=bool)
    return cols[None, :] <= rows[:, None]


def logits(x_rows: np.ndarray, x_cols: np.ndarray, scale: float) -> np.ndarray:
    """Z[i, j] = scale * <x_rows[i], x_cols[j]>."""
    return scale * (x_rows @ x_cols.T)


def row_lse(z: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """log sum_{j kept} exp(z[i, j]) per row, with the usual max shift."""
    zm = np.where(keep, z, -np.inf)
    m = zm.max(axis=1)
    return m + np.log(np.exp(zm - m[:, None]).sum(axis=1))


def _chunks(n: int, chunk: int | None):
    step = n if not chunk else max(1, int(chunk))
    for r0 in range(0, n, step):
        yield np.arange(r0, min(n, r0 + step))


def forward_unit(x_t, x_s, scale: float, causal: bool, chunk: int | None = None, rows=None):
    """Forward for one (batch, head) unit.

    x_t, x_s: [N, d].  Returns (lse_t, lse_s, row_kl), each float64 [N] (or, when ``rows``
    is given, float64 [len(rows)] for those rows only: every row is its own definition).
    """
    x_t = _f64(x_t)
    x_s = _f64(x_s)
    n = x_t.shape[0]
    cols = np.arange(n)
    sel = cols if rows is None else np.asarray(rows, dtype=np.int64)
    lse_t = np.empty(sel.size)
    lse_s = np.empty(sel.size)
    row_kl = np.empty(sel.size)
    for pos in _chunks(sel.size, chunk):
        rows = sel[pos]
        # causal rows never keep a column beyond their own index: leave those out
        hi = int(rows.max()) + 1 if causal else n
        cols = np.arange(hi)
        keep = keep_mask(rows, cols, causal)
        z_t = logits(x_t[rows], x_t[:hi], scale)
        z_s = logits(x_s[rows], x_s[:hi], scale)
        lt = row_lse(z_t, keep)
        ls = row_lse(z_s, keep)
        logp_t = z_t - lt[:, None]
        logp_s = z_s - ls[:, None]
        p_t = np.where(keep, np.exp(np.where(keep, logp_t, -np.inf)), 0.0)
        term = np.where(keep, p_t * (logp_t - logp_s), 0.0)
        lse_t[pos] = lt
        lse_s[pos] = ls
        row_kl[pos] = term.sum(axis=1)
    return lse_t, lse_s, row_kl


def _probs(x_rows, rows, x_all, lse_rows, scale, causal, cols):
    """R[rows, cols] = exp(Z - LSE_row), zero where masked."""
    keep = keep_mask(rows, cols, causal)
    z = logits(x_rows, x_all, scale)
    return np.where(keep, np.exp(np.where(keep, z - lse_rows[:, None], -np.inf)), 0.0)


def backward_unit(x_t, x_s, scale: float, causal: bool, g: float = 1.0,
                  lse_t=None, lse_s=None, rows=None, chunk: int | None = None):
    """Gradient of g * sum_i KL_i with respect to x_s for one unit.

    dX_s = scale * (dZ + dZ^T) X_s,  dZ = g * (R_s - R_t) (0 where masked).
    Returns float64 [len(rows), d] (all rows when ``rows`` is None).  The LSE vectors, if
    not given, are computed here with ``forward_unit``.
    """
    x_t = _f64(x_t)
    x_s = _f64(x_s)
    n = x_t.shape[0]
    if lse_t is None or lse_s is None:
        lse_t, lse_s, _ = forward_unit(x_t, x_s, scale, causal, chunk)
    lse_t = _f64(lse_t)
    lse_s = _f64(lse_s)
    all_idx = np.arange(n)
    rows = all_idx if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, x_s.shape[1]))
    step = rows.size if not chunk else max(1, int(chunk))
    for c0 in range(0, rows.size, step):
        r = rows[c0:c0 + step]
        # causal: row r keeps columns <= r, and column r is kept by rows >= r only
        hi = int(r.max()) + 1 if causal else n
        lo = int(r.min()) if causal else 0
        left, right = all_idx[:hi], all_idx[lo:]
        # dZ[r, :]  (row r of the loss, normalised by the LSE of row r)
        dz_rows = g * (_probs(x_s[r], r, x_s[:hi], lse_s[r], scale, causal, left)
                       - _probs(x_t[r], r, x_t[:hi], lse_t[r], scale, causal, left))
        # dZ[:, r]  (column r: rows j normalised by the LSE of row j); Z is symmetric
        # in its two indices, so Z[:, r] = scale * X X[r]^T
        dz_cols = g * (_probs(x_s[lo:], right, x_s[r], lse_s[lo:], scale, causal, r)
                       - _probs(x_t[lo:], right, x_t[r], lse_t[lo:], scale, causal, r))
        out[c0:c0 + step] = scale * (dz_rows @ x_s[:hi] + dz_cols.T @ x_s[lo:])
    return out


def _unit_views(x, head_map):
    """Iterate (b, h, h_in) over the relation heads of a [B, H_in, N, d] array."""
    b_n, h_in_n = x.shape[0], x.shape[1]
    hm = list(range(h_in_n)) if head_map is None else [int(v) for v in head_map]
    for b in range(b_n):
        for h, hi in enumerate(hm):
            yield b, h, hi


def forward(x_t, x_s, scale: float, causal: bool, head_map=None, chunk: int | None = None):
    """Batched forward over [B, H_in, N, d] inputs.

    Returns dict with lse_t, lse_s, row_kl (float64 [B, H, N]) and loss (float), where
    H = len(head_map) (or H_in) and loss = sum of row_kl.
    """
    x_t = np.asarray(x_t)
    x_s = np.asarray(x_s)
    b_n, _, n, _ = x_t.shape
    h_n = x_t.shape[1] if head_map is None else len(head_map)
    lse_t = np.empty((b_n, h_n, n))
    lse_s = np.empty((b_n, h_n, n))
    row_kl = np.empty((b_n, h_n, n))
    for b, h, hi in _unit_views(x_t, head_map):
        lse_t[b, h], lse_s[b, h], row_kl[b, h] = forward_unit(x_t[b, hi], x_s[b, hi], scale,
                                                              causal, chunk)
    return {"lse_t": lse_t, "lse_s": lse_s, "row_kl": row_kl, "loss": float(row_kl.sum())}


def backward(x_t, x_s, scale: float, causal: bool, g: float = 1.0, head_map=None,
             chunk: int | None = None):
    """Batched gradient: float64 [B, H_in, N, d]; heads not in head_map stay zero."""
    x_t = np.asarray(x_t)
    x_s = np.asarray(x_s)
    out = np.zeros(x_s.shape, dtype=np.float64)
    for b, _, hi in _unit_views(x_t, head_map):
        out[b, hi] = backward_unit(x_t[b, hi], x_s[b, hi], scale, causal, g, chunk=chunk)
    return out
