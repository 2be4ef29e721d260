"""Pins of the cross-relation oracle (``oracle.cross``) against facts other than itself:
the relation oracle when A = B (loss, and dA + dB equals the relation gradient), central
finite differences of both gradients, a torch float64 log_softmax / kl_div / autograd
computation, invariances of A B^T, the causal direction, and the frozen teacher."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import cross


def rand_quad(n, d, noise=0.3, seed=0):
    r = np.random.default_rng(seed)
    a_t = r.standard_normal((n, d))
    b_t = r.standard_normal((n, d))
    return a_t, b_t, a_t + noise * r.standard_normal((n, d)), b_t + noise * r.standard_normal((n, d))


@pytest.mark.parametrize("causal", [True, False])
def test_equal_operands_reduce_to_relation(causal):
    r = np.random.default_rng(1)
    x_t = r.standard_normal((30, 6))
    x_s = x_t + 0.3 * r.standard_normal((30, 6))
    a = cross.forward_unit(x_t, x_t, x_s, x_s, 0.4, causal)
    b = oracle.forward_unit(x_t, x_s, 0.4, causal)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-14)
    da, db = cross.backward_unit(x_t, x_t, x_s, x_s, 0.4, causal, 0.8)
    np.testing.assert_allclose(da + db, oracle.backward_unit(x_t, x_s, 0.4, causal, 0.8),
                               rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(3, 4), (5, 2), (6, 3)])
def test_finite_differences(n, d, causal):
    a_t, b_t, a_s, b_s = rand_quad(n, d, seed=10 * n + d)
    scale, g = 1.0 / math.sqrt(d), 1.2

    def loss(a, b):
        return cross.forward_unit(a_t, b_t, a, b, scale, causal)[2].sum()

    da, db = cross.backward_unit(a_t, b_t, a_s, b_s, scale, causal, g)
    eps = 1e-6
    for which, got in (("a", da), ("b", db)):
        fd = np.zeros((n, d))
        for i in range(n):
            for k in range(d):
                p, m = (a_s.copy(), b_s.copy()), (a_s.copy(), b_s.copy())
                idx = 0 if which == "a" else 1
                p[idx][i, k] += eps
                m[idx][i, k] -= eps
                fd[i, k] = g * (loss(*p) - loss(*m)) / (2 * eps)
        err = np.linalg.norm(got - fd) / np.linalg.norm(fd)
        assert err < 1e-7, (which, err)


def torch_reference(a_t, b_t, a_s, b_s, scale, causal, g):
    t = [torch.tensor(v, dtype=torch.float64) for v in (a_t, b_t, a_s, b_s)]
    t[2].requires_grad_(True)
    t[3].requires_grad_(True)
    n = t[0].shape[0]
    mask = torch.ones(n, n, dtype=torch.bool)
    if causal:
        mask = torch.tril(mask)
    z_t = (scale * t[0] @ t[1].T).masked_fill(~mask, float("-inf"))
    z_s = (scale * t[2] @ t[3].T).masked_fill(~mask, float("-inf"))
    lp_t = torch.log_softmax(z_t, dim=1)
    lp_s = torch.log_softmax(z_s, dim=1)
    p_t = lp_t.exp()
    terms = torch.where(mask, p_t * (lp_t - lp_s), torch.zeros_like(p_t))
    loss = terms.sum()
    (g * loss).backward()
    return float(loss.detach()), t[2].grad.numpy(), t[3].grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_torch_autograd_crosscheck(causal):
    a_t, b_t, a_s, b_s = rand_quad(40, 8, seed=3)
    loss, ga, gb = torch_reference(a_t, b_t, a_s, b_s, 0.3, causal, 0.6)
    got = cross.forward_unit(a_t, b_t, a_s, b_s, 0.3, causal)[2].sum()
    assert abs(got - loss) <= 1e-12 * abs(loss)
    da, db = cross.backward_unit(a_t, b_t, a_s, b_s, 0.3, causal, 0.6)
    np.testing.assert_allclose(da, ga, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(db, gb, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_invariances_of_the_product(causal):
    """Z depends on A B^T only: (A R, B R) for an orthogonal R and (c A, B / c) leave the
    loss unchanged, and the gradients transform covariantly; swapping A and B transposes
    Z, which changes a causal or non-symmetric loss."""
    a_t, b_t, a_s, b_s = rand_quad(25, 6, seed=4)
    q, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((6, 6)))
    base = cross.forward_unit(a_t, b_t, a_s, b_s, 0.4, causal)[2].sum()
    rot = cross.forward_unit(a_t, b_t, a_s @ q, b_s @ q, 0.4, causal)[2].sum()
    sc = cross.forward_unit(a_t, b_t, 2.0 * a_s, 0.5 * b_s, 0.4, causal)[2].sum()
    assert abs(rot - base) <= 1e-10 * base and abs(sc - base) <= 1e-10 * base
    da, db = cross.backward_unit(a_t, b_t, a_s, b_s, 0.4, causal)
    dar, dbr = cross.backward_unit(a_t, b_t, a_s @ q, b_s @ q, 0.4, causal)
    np.testing.assert_allclose(dar, da @ q, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dbr, db @ q, rtol=1e-9, atol=1e-12)
    swapped = cross.forward_unit(b_t, a_t, b_s, a_s, 0.4, causal)[2].sum()
    assert abs(swapped - base) > 1e-3 * base


def test_causal_direction_and_zero_at_equality():
    a_t, b_t, a_s, b_s = rand_quad(12, 4, seed=6)
    kl = cross.forward_unit(a_t, b_t, a_s, b_s, 0.5, True)[2]
    b2 = b_s.copy()
    b2[-1] += 1.0  # the last key is kept by the last row only
    kl2 = cross.forward_unit(a_t, b_t, a_s, b2, 0.5, True)[2]
    np.testing.assert_array_equal(kl[:-1], kl2[:-1])
    assert kl2[-1] != kl[-1]
    assert kl[0] == 0.0  # row 0 keeps one column: both relations are the point mass
    z = cross.forward_unit(a_t, b_t, a_t, b_t, 0.5, True)[2]
    assert np.all(z == 0.0) and np.all(kl >= -1e-15)
    da, db = cross.backward_unit(a_t, b_t, a_t, b_t, 0.5, True)
    assert not np.any(da) and not np.any(db)
    # the teacher is frozen: swapping roles changes the gradient
    da2, _ = cross.backward_unit(a_s, b_s, a_t, b_t, 0.5, True)
    da1, _ = cross.backward_unit(a_t, b_t, a_s, b_s, 0.5, True)
    assert np.linalg.norm(da1 + da2) > 1e-6 and np.linalg.norm(da1 - da2) > 1e-6


def test_batched_head_map():
    r = np.random.default_rng(7)
    shp = (2, 3, 10, 4)
    a_t, b_t = r.standard_normal(shp), r.standard_normal(shp)
    a_s, b_s = a_t + 0.2 * r.standard_normal(shp), b_t + 0.2 * r.standard_normal(shp)
    out = cross.forward(a_t, b_t, a_s, b_s, 0.5, True, head_map=[2, 0])
    assert out["row_kl"].shape == (2, 2, 10)
    u = cross.forward_unit(a_t[1, 0], b_t[1, 0], a_s[1, 0], b_s[1, 0], 0.5, True)
    np.testing.assert_array_equal(out["row_kl"][1, 1], u[2])
    da, db = cross.backward(a_t, b_t, a_s, b_s, 0.5, True, head_map=[2, 0])
    assert not np.any(da[:, 1]) and not np.any(db[:, 1])
    ua, ub = cross.backward_unit(a_t[0, 2], b_t[0, 2], a_s[0, 2], b_s[0, 2], 0.5, True)
    np.testing.assert_array_equal(da[0, 2], ua)
    np.testing.assert_array_equal(db[0, 2], ub)
