"""Pins of the float64 oracle against things other than itself.

Each test below ties the oracle to an independent fact: a closed form derived by hand
(stored under tests/golden/), central finite differences of the loss (which pins the
gradient, including the reading that both occurrences of X_s in X_s X_s^T are
differentiated), the Gibbs inequality, a torch float64 log_softmax / kl_div / autograd
computation, orthogonal and permutation invariances, causality of the mask, and the
quadratic memory of a materialising implementation.
"""

import math
import tracemalloc

import numpy as np
import pytest
import torch

import oracle
from oracle import closed_form

RNG = np.random.default_rng(1234)


def rand_pair(n, d, noise=0.3, seed=0):
    r = np.random.default_rng(seed)
    x_t = r.standard_normal((n, d))
    x_s = x_t + noise * r.standard_normal((n, d))
    return x_t, x_s


def loss_of(x_t, x_s, scale, causal):
    return oracle.forward_unit(x_t, x_s, scale, causal)[2].sum()


# --------------------------------------------------------------------------- closed form
def test_golden_closed_form(golden):
    for case in golden["cases"]:
        n, d = case["N"], case["d"]
        e = np.zeros((n, d))
        m = min(n, d)
        e[np.arange(m), np.arange(m)] = 1.0
        x_t, x_s = case["a"] * e, case["b"] * e
        lt, ls, kl = oracle.forward_unit(x_t, x_s, case["scale"], case["causal"])
        np.testing.assert_allclose(lt, case["lse_t"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(ls, case["lse_s"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(kl, case["row_kl"], rtol=1e-11, atol=1e-15)
        assert kl.sum() == pytest.approx(case["loss"], rel=1e-12)
        rows = np.array(case["dx_rows"])
        dx = oracle.backward_unit(x_t, x_s, case["scale"], case["causal"], case["g"], rows=rows)
        np.testing.assert_allclose(dx, np.array(case["dx"]), rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d,a,b", [(1, 4, 2.0, 3.0), (6, 6, 1.5, 2.5), (9, 4, 3.0, 1.0),
                                     (16, 32, 2.0, 2.0)])
def test_closed_form_direct(n, d, a, b, causal):
    scale = 1.0 / math.sqrt(d)
    ref = closed_form.structured_case(n, d, a, b, scale, causal, g=0.7)
    e = np.zeros((n, d))
    m = min(n, d)
    e[np.arange(m), np.arange(m)] = 1.0
    lt, ls, kl = oracle.forward_unit(a * e, b * e, scale, causal)
    np.testing.assert_allclose(lt, ref["lse_t"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ls, ref["lse_s"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(kl, ref["row_kl"], rtol=1e-11, atol=1e-15)
    dx = oracle.backward_unit(a * e, b * e, scale, causal, 0.7)
    np.testing.assert_allclose(dx, np.array(ref["dx"]), rtol=1e-11, atol=1e-15)
    if a == b:
        assert np.all(kl == 0.0)


# --------------------------------------------------------------------- finite differences
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(2, 2), (3, 4), (5, 2), (8, 4)])
def test_finite_differences(n, d, causal):
    x_t, x_s = rand_pair(n, d, seed=n * 10 + d)
    scale = 1.0 / math.sqrt(d)
    g = 1.3
    grad = oracle.backward_unit(x_t, x_s, scale, causal, g)
    eps = 1e-6
    fd = np.zeros_like(x_s)
    for i in range(n):
        for k in range(d):
            xp = x_s.copy()
            xm = x_s.copy()
            xp[i, k] += eps
            xm[i, k] -= eps
            fd[i, k] = g * (loss_of(x_t, xp, scale, causal) - loss_of(x_t, xm, scale, causal)) / (2 * eps)
    err = np.linalg.norm(grad - fd) / np.linalg.norm(fd)
    assert err < 1e-7, err
    # the teacher gets no gradient: the loss is not symmetric in (t, s), so swapping the
    # roles must change the result (guards against differentiating the wrong tensor)
    swapped = oracle.backward_unit(x_s, x_t, scale, causal, g)
    assert np.linalg.norm(swapped - grad) > 1e-3 * np.linalg.norm(grad)


def test_finite_differences_one_sided_only_would_fail():
    """A gradient that kept only dZ X_s (dropping dZ^T X_s) is far from the differences."""
    n, d = 6, 3
    x_t, x_s = rand_pair(n, d, seed=5)
    scale = 0.5
    lt, ls, _ = oracle.forward_unit(x_t, x_s, scale, True)
    full = oracle.backward_unit(x_t, x_s, scale, True, 1.0)
    keep = np.tril(np.ones((n, n), dtype=bool))
    zt = scale * x_t @ x_t.T
    zs = scale * x_s @ x_s.T
    dz = np.where(keep, np.exp(np.where(keep, zs - ls[:, None], -np.inf))
                  - np.exp(np.where(keep, zt - lt[:, None], -np.inf)), 0.0)
    half = scale * dz @ x_s
    assert np.linalg.norm(full - half) > 0.1 * np.linalg.norm(full)


# ------------------------------------------------------------------------------ Gibbs
@pytest.mark.parametrize("causal", [True, False])
def test_gibbs_nonnegative_and_zero_at_equality(causal):
    for seed in range(4):
        x_t, x_s = rand_pair(40, 8, noise=1.0, seed=seed)
        _, _, kl = oracle.forward_unit(x_t, x_s, 0.35, causal)
        assert np.all(kl >= -1e-15)
        assert kl.sum() > 0
        lt, ls, kl0 = oracle.forward_unit(x_t, x_t.copy(), 0.35, causal)
        np.testing.assert_array_equal(lt, ls)
        assert np.all(np.abs(kl0) == 0.0)
        dx0 = oracle.backward_unit(x_t, x_t.copy(), 0.35, causal, 1.0)
        assert np.all(dx0 == 0.0)


def test_single_token_and_first_causal_row():
    x_t, x_s = rand_pair(1, 4, seed=3)
    for causal in (True, False):
        lt, ls, kl = oracle.forward_unit(x_t, x_s, 0.5, causal)
        assert kl[0] == 0.0
        # one kept entry: LSE is the logit itself
        assert lt[0] == pytest.approx(0.5 * x_t[0] @ x_t[0], rel=1e-15)
        assert np.all(oracle.backward_unit(x_t, x_s, 0.5, causal) == 0.0)
    x_t, x_s = rand_pair(10, 4, seed=4)
    _, _, kl = oracle.forward_unit(x_t, x_s, 0.5, True)
    assert kl[0] == 0.0 and kl[1] > 0.0


# ------------------------------------------------------------- library cross-check (torch)
def torch_reference(x_t, x_s, scale, causal, g):
    """log_softmax + kl_div (log_target) per row slice, gradient by torch.autograd."""
    xt = torch.tensor(x_t, dtype=torch.float64)
    xs = torch.tensor(x_s, dtype=torch.float64, requires_grad=True)
    zt = scale * xt @ xt.T
    zs = scale * xs @ xs.T
    n = xt.shape[0]
    rows = []
    for i in range(n):
        hi = i + 1 if causal else n
        lt = torch.log_softmax(zt[i, :hi], dim=0)
        ls = torch.log_softmax(zs[i, :hi], dim=0)
        rows.append(torch.nn.functional.kl_div(ls, lt, reduction="sum", log_target=True))
    row_kl = torch.stack(rows)
    (g * row_kl.sum()).backward()
    return row_kl.detach().numpy(), xs.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(7, 3), (33, 16), (64, 8)])
def test_torch_autograd_crosscheck(n, d, causal):
    x_t, x_s = rand_pair(n, d, noise=0.5, seed=n + d)
    scale = 1.0 / math.sqrt(d)
    kl_ref, dx_ref = torch_reference(x_t, x_s, scale, causal, 0.8)
    _, _, kl = oracle.forward_unit(x_t, x_s, scale, causal)
    dx = oracle.backward_unit(x_t, x_s, scale, causal, 0.8)
    np.testing.assert_allclose(kl, kl_ref, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dx, dx_ref, rtol=1e-10, atol=1e-13)


# -------------------------------------------------------------------------- invariances
def _orth(d, seed):
    q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((d, d)))
    return q


@pytest.mark.parametrize("causal", [True, False])
def test_orthogonal_invariance(causal):
    x_t, x_s = rand_pair(30, 6, seed=7)
    r1, r2 = _orth(6, 1), _orth(6, 2)
    a = oracle.forward_unit(x_t, x_s, 0.4, causal)
    b = oracle.forward_unit(x_t @ r1, x_s @ r2, 0.4, causal)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-10, atol=1e-13)
    dx = oracle.backward_unit(x_t, x_s, 0.4, causal)
    dxr = oracle.backward_unit(x_t @ r1, x_s @ r2, 0.4, causal)
    np.testing.assert_allclose(dxr, dx @ r2, rtol=1e-9, atol=1e-12)


def test_permutation_equivariance_noncausal():
    x_t, x_s = rand_pair(25, 5, seed=8)
    perm = np.random.default_rng(9).permutation(25)
    lt, ls, kl = oracle.forward_unit(x_t, x_s, 0.45, False)
    lt2, ls2, kl2 = oracle.forward_unit(x_t[perm], x_s[perm], 0.45, False)
    np.testing.assert_allclose(kl2, kl[perm], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lt2, lt[perm], rtol=1e-13)
    dx = oracle.backward_unit(x_t, x_s, 0.45, False)
    dx2 = oracle.backward_unit(x_t[perm], x_s[perm], 0.45, False)
    np.testing.assert_allclose(dx2, dx[perm], rtol=1e-10, atol=1e-13)


def test_causal_mask_direction():
    """Row i of a causal relation depends only on tokens 0..i."""
    x_t, x_s = rand_pair(20, 4, seed=11)
    lt, ls, kl = oracle.forward_unit(x_t, x_s, 0.5, True)
    y_t, y_s = x_t.copy(), x_s.copy()
    y_t[12:] += 1.0
    y_s[12:] -= 0.7
    lt2, ls2, kl2 = oracle.forward_unit(y_t, y_s, 0.5, True)
    np.testing.assert_array_equal(kl2[:12], kl[:12])
    np.testing.assert_array_equal(lt2[:12], lt[:12])
    assert np.all(kl2[12:] != kl[12:])
    # non-causal rows see everything
    _, _, kln = oracle.forward_unit(x_t, x_s, 0.5, False)
    _, _, kln2 = oracle.forward_unit(y_t, y_s, 0.5, False)
    assert np.all(kln2[:12] != kln[:12])


def test_row_chunking_is_exact():
    x_t, x_s = rand_pair(50, 8, seed=12)
    for causal in (True, False):
        a = oracle.forward_unit(x_t, x_s, 0.3, causal)
        b = oracle.forward_unit(x_t, x_s, 0.3, causal, chunk=7)
        for u, v in zip(a, b):
            np.testing.assert_allclose(u, v, rtol=1e-14, atol=1e-15)
        rows = np.array([0, 3, 17, 49])
        for u, v in zip(oracle.forward_unit(x_t, x_s, 0.3, causal, rows=rows, chunk=3), a):
            np.testing.assert_allclose(u, v[rows], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(oracle.backward_unit(x_t, x_s, 0.3, causal, rows=rows, chunk=3),
                                   oracle.backward_unit(x_t, x_s, 0.3, causal)[rows],
                                   rtol=1e-12, atol=1e-14)


def test_batched_head_map():
    r = np.random.default_rng(13)
    x_t = r.standard_normal((2, 4, 9, 3))
    x_s = x_t + 0.2 * r.standard_normal((2, 4, 9, 3))
    hm = [3, 0]
    f = oracle.forward(x_t, x_s, 0.5, True, head_map=hm)
    assert f["row_kl"].shape == (2, 2, 9)
    for b in range(2):
        for h, hi in enumerate(hm):
            _, _, kl = oracle.forward_unit(x_t[b, hi], x_s[b, hi], 0.5, True)
            np.testing.assert_array_equal(f["row_kl"][b, h], kl)
    dx = oracle.backward(x_t, x_s, 0.5, True, 1.0, head_map=hm)
    assert np.all(dx[:, [1, 2]] == 0.0)
    assert np.all(dx[:, [0, 3]] != 0.0)
    assert f["loss"] == pytest.approx(f["row_kl"].sum(), rel=1e-15)


def test_oracle_memory_is_quadratic():
    """A materialising implementation holds N x N matrices: peak memory ~ N^2."""
    peaks = []
    for n in (256, 512):
        x_t, x_s = rand_pair(n, 8, seed=n)
        tracemalloc.start()
        oracle.forward_unit(x_t, x_s, 0.3, True)
        peaks.append(tracemalloc.get_traced_memory()[1])
        tracemalloc.stop()
    ratio = peaks[1] / peaks[0]
    assert 3.0 < ratio < 5.0, ratio


# ------------------------------------------------------------- pure-Python brute force
def brute_force(x_t, x_s, scale, causal):
    n = len(x_t)
    out = []
    for i in range(n):
        js = range(i + 1) if causal else range(n)
        zt = [scale * sum(a * b for a, b in zip(x_t[i], x_t[j])) for j in js]
        zs = [scale * sum(a * b for a, b in zip(x_s[i], x_s[j])) for j in js]
        st = sum(math.exp(v) for v in zt)
        ss = sum(math.exp(v) for v in zs)
        kl = 0.0
        for a, b in zip(zt, zs):
            pt = math.exp(a) / st
            ps = math.exp(b) / ss
            kl += pt * math.log(pt / ps)
        out.append((math.log(st), math.log(ss), kl))
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_pure_python_brute_force(causal):
    for n, d in ((1, 1), (4, 3), (12, 4)):
        x_t, x_s = rand_pair(n, d, seed=n)
        ref = brute_force(x_t.tolist(), x_s.tolist(), 0.6, causal)
        lt, ls, kl = oracle.forward_unit(x_t, x_s, 0.6, causal)
        np.testing.assert_allclose(lt, [r[0] for r in ref], rtol=1e-12)
        np.testing.assert_allclose(ls, [r[1] for r in ref], rtol=1e-12)
        np.testing.assert_allclose(kl, [r[2] for r in ref], rtol=1e-9, atol=1e-15)
