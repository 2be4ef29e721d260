"""Closed-form values of the relation KL and its gradient for a family of structured inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This is an independent derivation,
done by hand from the definitions (pith.science verdict page, key_machinery field:
R_m = softmax(X_m X_m^T / sqrt(d) + M), forward KL per row, gradient R_s - R_t), and
evaluated in 50-digit decimal arithmetic.  It does not call the matrix oracle, so it can
pin it.

Inputs: X_t = a * E and X_s = b * E, where E is N x d with E[i] = e_i (unit vector) for
i < m = min(N, d) and E[i] = 0 for i >= m.  With c_t = scale * a^2, c_s = scale * b^2 and
n_i the number of kept entries of row i (i + 1 causal, N otherwise):

* rows i < m: the logit row is c on the diagonal and 0 elsewhere, so
  LSE_i = log(e^c + n_i - 1), R(i,i) = e^c / (e^c + n_i - 1) and every other kept entry
  is (1 - R(i,i)) / (n_i - 1).  The row KL collapses to the Bernoulli KL of the
  diagonal probabilities.
* rows i >= m: the logit row is all zeros, R is uniform, LSE_i = log(n_i), KL_i = 0.
* dX_s[i, k] = scale * b * (dZ[i,k] + dZ[k,i]) for k < m and 0 for k >= m, because
  column k of X_s is b * e_k.
"""

from __future__ import annotations

from decimal import Decimal, getcontext

getcontext().prec = 50

__all__ = ["structured_case"]


def _row_probs(c: Decimal, n_kept: int):
    """(diagonal prob, off-diagonal prob, lse) of a row with one logit c and n_kept-1 zeros."""
    ec = c.exp()
    denom = ec + Decimal(n_kept - 1)
    return ec / denom, (Decimal(1) / denom if n_kept > 1 else Decimal(0)), denom.ln()


def structured_case(n: int, d: int, a: float, b: float, scale: float, causal: bool,
                    g: float = 1.0):
    """Return dict(lse_t, lse_s, row_kl: list[N]; loss: float; dx: list[N][d]) as floats."""
    m = min(n, d)
    s = Decimal(scale)
    ct = s * Decimal(a) * Decimal(a)
    cs = s * Decimal(b) * Decimal(b)
    gd = Decimal(g)
    lse_t, lse_s, row_kl = [], [], []
    diag_t, diag_s, off_t, off_s = [], [], [], []
    for i in range(n):
        nk = i + 1 if causal else n
        if i < m:
            pt, ot, lt = _row_probs(ct, nk)
            ps, os_, ls = _row_probs(cs, nk)
            kl = pt * (pt / ps).ln()
            if nk > 1:
                kl += (1 - pt) * ((1 - pt) / (1 - ps)).ln()
        else:
            lt = ls = Decimal(nk).ln()
            pt = ps = ot = os_ = Decimal(1) / Decimal(nk)
            kl = Decimal(0)
        lse_t.append(lt)
        lse_s.append(ls)
        row_kl.append(kl)
        diag_t.append(pt)
        diag_s.append(ps)
        off_t.append(ot)
        off_s.append(os_)

    def dz(i: int, j: int) -> Decimal:
        if causal and j > i:
            return Decimal(0)
        if i == j:
            return gd * (diag_s[i] - diag_t[i])
        return gd * (off_s[i] - off_t[i])

    bd = Decimal(b)
    dx = [[0.0] * d for _ in range(n)]
    for i in range(n):
        for k in range(m):
            dx[i][k] = float(s * bd * (dz(i, k) + dz(k, i)))
    return {
        "lse_t": [float(v) for v in lse_t],
        "lse_s": [float(v) for v in lse_s],
        "row_kl": [float(v) for v in row_kl],
        "loss": float(sum(row_kl)),
        "dx": dx,
    }
