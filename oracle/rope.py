"""Float64 CPU oracle for the relation KL with the rotary position embedding applied
inside the operation (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

What it computes.  The LinearARD pages distil the attention relations of queries, keys
and values *after* the rotary embedding: the teacher keeps its native RoPE, the student
runs a rescaled one (position interpolation or a larger base), and the gradient flows back
to the student's Q/K/V projections (verdict page on pith.science,
``pith_extraction.key_machinery``; arXiv abstract on mlsanity.com).  Here the rotation is
part of the operation:

* ``X_m = rope(Xpre_m; cos_m, sin_m)`` for teacher m = t and student m = s, where the
  tables give, for token p and frequency k < d/2, the cosine and sine of that token's
  angle.  The pages do not spell the rotation out; the reading taken is the rotate-half
  pairing of dimension k with k + d/2:
      X[p, k]       = Xpre[p, k] cos[p, k] - Xpre[p, k + d/2] sin[p, k]
      X[p, k + d/2] = Xpre[p, k + d/2] cos[p, k] + Xpre[p, k] sin[p, k]
  (the complex product (Xpre[p, k] + i Xpre[p, k + d/2]) e^{i angle}).  A side without
  tables is not rotated (the V relation).
* The rotated rows are the relation inputs in the activations' own dtype, as when the
  model applies RoPE itself and hands the result to the plain relation KL: the exact
  rotation (float64 here; the products of a bf16 or fp32 value with an fp32 table entry
  are exact in float64, and the sum of two of them is off by at most one float64 rounding)
  rounded once to the input dtype, to nearest with ties to even.  ``dtype=None`` keeps the
  exact float64 rotation (used by the pins that differentiate through it).
* The loss is the relation KL of ``oracle.relkl`` on the rotated inputs.
* The gradient with respect to the student's pre-rotation input is the transposed
  rotation of the gradient with respect to X_s (the rounding to the dtype passes the
  gradient through unchanged, as a dtype cast does under automatic differentiation):
      dXpre[p, k]       = dX[p, k] cos[p, k] + dX[p, k + d/2] sin[p, k]
      dXpre[p, k + d/2] = dX[p, k + d/2] cos[p, k] - dX[p, k] sin[p, k]

The tables are inputs, like the activations: the caller builds them from its own recipe
(base, positions), and the oracle uses exactly the values it is given.
"""

from __future__ import annotations

import numpy as np

from . import relkl

__all__ = ["rotate", "rotate_back", "round_bf16", "round_fp32", "rotate_in_dtype", "forward",
           "backward"]


def _tab(t):
    return None if t is None else np.asarray(t, dtype=np.float64)


def rotate(x, cos, sin) -> np.ndarray:
    """Rotate-half RoPE of [..., N, d] rows with [N, d/2] tables (None: unrotated)."""
    x = np.asarray(x, dtype=np.float64)
    if cos is None and sin is None:
        return x.copy()
    cos, sin = _tab(cos), _tab(sin)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate((x1 * cos - x2 * sin, x2 * cos + x1 * sin), axis=-1)


def rotate_back(g, cos, sin) -> np.ndarray:
    """Transpose of ``rotate``: maps a gradient w.r.t. the rotated rows to the inputs."""
    g = np.asarray(g, dtype=np.float64)
    if cos is None and sin is None:
        return g.copy()
    cos, sin = _tab(cos), _tab(sin)
    h = g.shape[-1] // 2
    g1, g2 = g[..., :h], g[..., h:]
    return np.concatenate((g1 * cos + g2 * sin, g2 * cos - g1 * sin), axis=-1)


def round_bf16(v) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even, for values in
    the normal range: v = m 2^e with 1/2 <= |m| < 1, m rounded to a multiple of 2^-8."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_fp32(v) -> np.ndarray:
    """Round to the nearest fp32 value, ties to even (numpy's float64 -> float32 cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def rotate_in_dtype(x, cos, sin, dtype) -> np.ndarray:
    """The rotated rows as the operation uses them: the exact rotation rounded once to
    ``dtype`` ("bf16" or "fp32"); dtype None gives the exact rotation unrounded.  A side
    without tables is returned as given (its values are already of the dtype)."""
    y = rotate(x, cos, sin)
    if dtype is None or (cos is None and sin is None):
        return y
    if dtype == "bf16":
        return round_bf16(y)
    if dtype == "fp32":
        return round_fp32(y)
    raise ValueError(f"unknown dtype {dtype!r}")


def forward(x_t, x_s, scale: float, causal: bool, cos_t=None, sin_t=None, cos_s=None,
            sin_s=None, head_map=None, chunk: int | None = None, dtype=None):
    """Forward on pre-rotation [B, H_in, N, d] inputs; same outputs as ``relkl.forward``.
    ``dtype`` ("bf16" / "fp32") rounds the rotated rows as the operation does."""
    return relkl.forward(rotate_in_dtype(x_t, cos_t, sin_t, dtype),
                         rotate_in_dtype(x_s, cos_s, sin_s, dtype), scale, causal,
                         head_map=head_map, chunk=chunk)


def backward(x_t, x_s, scale: float, causal: bool, g: float = 1.0, cos_t=None, sin_t=None,
             cos_s=None, sin_s=None, head_map=None, chunk: int | None = None, dtype=None):
    """Gradient of g * loss w.r.t. the student's pre-rotation input, float64 [B, H_in, N, d]
    (heads outside head_map stay zero)."""
    d_rot = relkl.backward(rotate_in_dtype(x_t, cos_t, sin_t, dtype),
                           rotate_in_dtype(x_s, cos_s, sin_s, dtype), scale, causal,
                           g, head_map=head_map, chunk=chunk)
    return rotate_back(d_rot, cos_s, sin_s)
