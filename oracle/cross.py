"""Float64 CPU oracle for the cross-relation KL: row-softmax(scale * A B^T) of two different
matrices per side (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

What it computes.  The relation KL of LinearARD compares row-softmax relations of one
matrix with itself (Q Q^T, K K^T, V V^T; verdict page on pith.science,
``pith_extraction.key_machinery``).  The same row-wise KL applies to a relation between
two different matrices -- the attention map softmax(Q K^T / sqrt(d)) being the usual one --
which the pages' own inference on the method's scope points to.  With A (rows, "queries")
and B (columns, "keys") given per side m = t, s:

* Z_m = scale * A_m B_m^T + M (M: the mask), R_m = softmax_rows(Z_m);
* KL_i = sum_j R_t(i,j) (log R_t(i,j) - log R_s(i,j)), loss = sum over rows (and batch,
  heads);
* with dZ = g (R_s - R_t) (zero where masked), the gradients of the student's two inputs
  are dA_s = scale * dZ B_s and dB_s = scale * dZ^T A_s.  With A = B = X their sum is the
  relation gradient scale (dZ + dZ^T) X of ``oracle.relkl``.  The teacher is frozen.

The readings of the relation case apply unchanged (causal keeps j <= i, sums, nats).
Every function is the plain definition with the N x N matrices materialised.
"""

from __future__ import annotations

import numpy as np

from .relkl import _chunks, _f64, keep_mask, row_lse

__all__ = ["forward_unit", "backward_unit", "forward", "backward"]


def forward_unit(a_t, b_t, a_s, b_s, scale: float, causal: bool, chunk: int | None = None,
                 rows=None):
    """(lse_t, lse_s, row_kl) float64 [N] (or for the given rows) of one unit."""
    a_t, b_t, a_s, b_s = (_f64(v) for v in (a_t, b_t, a_s, b_s))
    n = a_t.shape[0]
    sel = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    lse_t, lse_s, row_kl = np.empty(sel.size), np.empty(sel.size), np.empty(sel.size)
    for pos in _chunks(sel.size, chunk):
        r = sel[pos]
        hi = int(r.max()) + 1 if causal else n
        keep = keep_mask(r, np.arange(hi), causal)
        z_t = scale * (a_t[r] @ b_t[:hi].T)
        z_s = scale * (a_s[r] @ b_s[:hi].T)
        lt, ls = row_lse(z_t, keep), row_lse(z_s, keep)
        logp_t, logp_s = z_t - lt[:, None], z_s - ls[:, None]
        p_t = np.where(keep, np.exp(np.where(keep, logp_t, -np.inf)), 0.0)
        lse_t[pos], lse_s[pos] = lt, ls
        row_kl[pos] = np.where(keep, p_t * (logp_t - logp_s), 0.0).sum(axis=1)
    return lse_t, lse_s, row_kl


def _dz(a_t, b_t, a_s, b_s, rows, cols, lse_t, lse_s, scale, causal, g):
    """dZ[rows, cols] = g (R_s - R_t), zero where masked (rows normalised by their LSE)."""
    keep = keep_mask(rows, cols, causal)

    def probs(a, b, lse):
        z = scale * (a[rows] @ b[cols].T)
        return np.where(keep, np.exp(np.where(keep, z - lse[rows][:, None], -np.inf)), 0.0)

    return g * (probs(a_s, b_s, lse_s) - probs(a_t, b_t, lse_t))


def backward_unit(a_t, b_t, a_s, b_s, scale: float, causal: bool, g: float = 1.0,
                  lse_t=None, lse_s=None, rows_a=None, rows_b=None, chunk: int | None = None):
    """(dA_s [len(rows_a), d], dB_s [len(rows_b), d]) of g * loss for one unit (all rows by
    default).  dA_s rows need their own row's LSE; dB_s row j needs the LSE of every row
    i that keeps column j (i >= j when causal)."""
    a_t, b_t, a_s, b_s = (_f64(v) for v in (a_t, b_t, a_s, b_s))
    n = a_t.shape[0]
    if lse_t is None or lse_s is None:
        lse_t, lse_s, _ = forward_unit(a_t, b_t, a_s, b_s, scale, causal, chunk)
    lse_t, lse_s = _f64(lse_t), _f64(lse_s)
    idx = np.arange(n)
    ra = idx if rows_a is None else np.asarray(rows_a, dtype=np.int64)
    rb = idx if rows_b is None else np.asarray(rows_b, dtype=np.int64)
    da = np.empty((ra.size, a_s.shape[1]))
    db = np.empty((rb.size, b_s.shape[1]))
    step_a = ra.size if not chunk else max(1, int(chunk))
    for c0 in range(0, ra.size, step_a):
        r = ra[c0:c0 + step_a]
        hi = int(r.max()) + 1 if causal else n
        cols = idx[:hi]
        da[c0:c0 + step_a] = scale * (_dz(a_t, b_t, a_s, b_s, r, cols, lse_t, lse_s, scale,
                                          causal, g) @ b_s[:hi])
    step_b = rb.size if not chunk else max(1, int(chunk))
    for c0 in range(0, rb.size, step_b):
        c = rb[c0:c0 + step_b]
        lo = int(c.min()) if causal else 0
        rows = idx[lo:]
        dz = _dz(a_t, b_t, a_s, b_s, rows, c, lse_t, lse_s, scale, causal, g)  # [rows, c]
        db[c0:c0 + step_b] = scale * (dz.T @ a_s[lo:])
    return da, db


def _units(x, head_map):
    hm = list(range(x.shape[1])) if head_map is None else [int(v) for v in head_map]
    for b in range(x.shape[0]):
        for h, hi in enumerate(hm):
            yield b, h, hi


def forward(a_t, b_t, a_s, b_s, scale: float, causal: bool, head_map=None,
            chunk: int | None = None):
    """Batched forward over [B, H_in, N, d] inputs (one head map for all four); returns
    lse_t, lse_s, row_kl float64 [B, H, N] and the summed loss."""
    a_t = np.asarray(a_t)
    bsz, _, n, _ = a_t.shape
    h_n = a_t.shape[1] if head_map is None else len(head_map)
    out = {k: np.empty((bsz, h_n, n)) for k in ("lse_t", "lse_s", "row_kl")}
    for b, h, hi in _units(a_t, head_map):
        lt, ls, kl = forward_unit(a_t[b, hi], np.asarray(b_t)[b, hi], np.asarray(a_s)[b, hi],
                                  np.asarray(b_s)[b, hi], scale, causal, chunk)
        out["lse_t"][b, h], out["lse_s"][b, h], out["row_kl"][b, h] = lt, ls, kl
    out["loss"] = float(out["row_kl"].sum())
    return out


def backward(a_t, b_t, a_s, b_s, scale: float, causal: bool, g: float = 1.0, head_map=None,
             chunk: int | None = None):
    """Batched (dA_s, dB_s), float64 [B, H_in, N, d] each; unmapped heads stay zero."""
    a_t, b_t, a_s, b_s = (np.asarray(v) for v in (a_t, b_t, a_s, b_s))
    da = np.zeros(a_s.shape)
    db = np.zeros(b_s.shape)
    for b, _, hi in _units(a_t, head_map):
        da[b, hi], db[b, hi] = backward_unit(a_t[b, hi], b_t[b, hi], a_s[b, hi], b_s[b, hi],
                                             scale, causal, g, chunk=chunk)
    return da, db
