"""Pins of the RoPE-fused oracle (``oracle.rope``) against facts other than itself.

* the rotation equals the complex product (x_k + i x_{k+d/2}) e^{i angle} (the textbook
  form of rotate-half RoPE), and rotating back inverts it;
* identity tables reduce the fused loss and gradient to the plain oracle;
* tables that give every token the same angles rotate all rows by one orthogonal map, so
  the loss and the pre-rotation gradient equal the plain ones on the unrotated inputs;
* central finite differences of the fused loss pin the pre-rotation gradient (and with it
  the transposed rotation of the chain rule);
* with equal activations, equal tables give a zero loss and unequal ones a positive loss
  that changes when the tables swap sides (each side uses its own tables);
* the harness's RoPE recipe and the tables it builds give the same rotation.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from attention_relation_distillation_amd import workloads


def rand_tables(n, d, seed):
    ang = np.random.default_rng(seed).uniform(-math.pi, math.pi, (n, d // 2))
    return np.cos(ang), np.sin(ang)


def rand_pair(n, d, noise=0.3, seed=0):
    r = np.random.default_rng(seed)
    x_t = r.standard_normal((1, 1, n, d))
    x_s = x_t + noise * r.standard_normal((1, 1, n, d))
    return x_t, x_s


def test_rotation_is_complex_product():
    n, d = 7, 8
    x = np.random.default_rng(3).standard_normal((n, d))
    ang = np.random.default_rng(4).uniform(-3, 3, (n, d // 2))
    got = rope.rotate(x, np.cos(ang), np.sin(ang))
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * ang)
    np.testing.assert_allclose(got[:, : d // 2], z.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[:, d // 2:], z.imag, rtol=0, atol=1e-14)
    np.testing.assert_allclose(rope.rotate_back(got, np.cos(ang), np.sin(ang)), x, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_identity_tables_reduce_to_plain_oracle(causal):
    x_t, x_s = rand_pair(20, 6, seed=1)
    one, zero = np.ones((20, 3)), np.zeros((20, 3))
    a = rope.forward(x_t, x_s, 0.4, causal, one, zero, one, zero)
    b = oracle.forward(x_t, x_s, 0.4, causal)
    assert a["loss"] == b["loss"]
    np.testing.assert_array_equal(a["row_kl"], b["row_kl"])
    ga = rope.backward(x_t, x_s, 0.4, causal, 0.7, one, zero, one, zero)
    gb = oracle.backward(x_t, x_s, 0.4, causal, 0.7)
    np.testing.assert_array_equal(ga, gb)


@pytest.mark.parametrize("causal", [True, False])
def test_position_independent_rotation_is_invisible(causal):
    """One rotation for every token (different for teacher and student) leaves X X^T of
    each side unchanged: the fused loss equals the plain loss on the unrotated inputs, and
    the pre-rotation gradient equals the plain gradient."""
    n, d = 25, 8
    x_t, x_s = rand_pair(n, d, seed=2)
    at = np.random.default_rng(5).uniform(-3, 3, d // 2)
    as_ = np.random.default_rng(6).uniform(-3, 3, d // 2)
    ct, st = np.tile(np.cos(at), (n, 1)), np.tile(np.sin(at), (n, 1))
    cs, ss = np.tile(np.cos(as_), (n, 1)), np.tile(np.sin(as_), (n, 1))
    a = rope.forward(x_t, x_s, 0.35, causal, ct, st, cs, ss)
    b = oracle.forward(x_t, x_s, 0.35, causal)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * abs(b["loss"])
    ga = rope.backward(x_t, x_s, 0.35, causal, 1.1, ct, st, cs, ss)
    gb = oracle.backward(x_t, x_s, 0.35, causal, 1.1)
    np.testing.assert_allclose(ga, gb, rtol=1e-10, atol=1e-12)
    # a position-dependent rotation does change the loss (the test above is not vacuous)
    ct2, st2 = rand_tables(n, d, 9)
    c = rope.forward(x_t, x_s, 0.35, causal, ct2, st2, cs, ss)
    assert abs(c["loss"] - b["loss"]) > 1e-3 * abs(b["loss"])


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(3, 4), (5, 4), (6, 2)])
def test_finite_differences_pre_rotation(n, d, causal):
    x_t, x_s = rand_pair(n, d, seed=10 * n + d)
    ct, st = rand_tables(n, d, 11)
    cs, ss = rand_tables(n, d, 12)
    scale, g = 1.0 / math.sqrt(d), 0.9

    def loss(xs):
        return rope.forward(x_t, xs, scale, causal, ct, st, cs, ss)["loss"]

    grad = rope.backward(x_t, x_s, scale, causal, g, ct, st, cs, ss)
    eps = 1e-6
    fd = np.zeros_like(x_s)
    for i in range(n):
        for k in range(d):
            xp, xm = x_s.copy(), x_s.copy()
            xp[0, 0, i, k] += eps
            xm[0, 0, i, k] -= eps
            fd[0, 0, i, k] = g * (loss(xp) - loss(xm)) / (2 * eps)
    err = np.linalg.norm(grad - fd) / np.linalg.norm(fd)
    assert err < 1e-7, err
    # the untransposed rotation (a plausible slip) is far from the differences
    wrong = rope.rotate(oracle.backward(rope.rotate(x_t, ct, st), rope.rotate(x_s, cs, ss),
                                        scale, causal, g), cs, ss)
    assert np.linalg.norm(wrong - fd) > 1e-2 * np.linalg.norm(fd)


def test_harness_recipe_matches_tables():
    n, d = 40, 16
    x = torch.randn((1, 2, n, d), generator=torch.Generator().manual_seed(0))
    for base, div in [(10000.0, 1.0), (10000.0, 8.0), (500000.0, 4.0)]:
        cos, sin = workloads.rope_tables(n, d, base, div, dtype=torch.float64)
        got = rope.rotate(x.numpy(), cos.numpy(), sin.numpy())
        ref = workloads.rope(x, base, div).numpy()
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_each_side_takes_its_own_tables(causal):
    """Same activations on both sides: equal tables give a zero loss and gradient, unequal
    tables a positive loss (which fails if one side took the other's tables or neither was
    rotated), and swapping the tables between the sides changes it."""
    n, d = 18, 8
    x = np.random.default_rng(13).standard_normal((1, 1, n, d))
    ca, sa = rand_tables(n, d, 14)
    cb, sb = rand_tables(n, d, 15)
    same = rope.forward(x, x, 0.4, causal, ca, sa, ca, sa)
    assert same["loss"] == 0.0
    assert not np.any(rope.backward(x, x, 0.4, causal, 1.0, ca, sa, ca, sa))
    diff = rope.forward(x, x, 0.4, causal, ca, sa, cb, sb)
    swap = rope.forward(x, x, 0.4, causal, cb, sb, ca, sa)
    assert diff["loss"] > 1e-3 and swap["loss"] > 1e-3
    assert abs(diff["loss"] - swap["loss"]) > 1e-6 * diff["loss"]  # KL is not symmetric
    only_t = rope.forward(x, x, 0.4, causal, ca, sa, None, None)
    assert only_t["loss"] > 1e-3


def test_round_bf16_matches_torch_on_fp32_values():
    """Nearest-even rounding to bf16 agrees with torch's float32 -> bfloat16 conversion,
    including constructed halfway cases (which round to the even neighbour)."""
    r = np.random.default_rng(20)
    v = (r.standard_normal(200000) * np.exp(r.uniform(-8, 8, 200000))).astype(np.float32)
    bits = v.view(np.uint32)
    half = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)  # exact ties
    for arr in (v, half):
        ref = torch.from_numpy(arr.copy()).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(rope.round_bf16(arr.astype(np.float64)), ref)
    # ties go to the even significand
    assert rope.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert rope.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_rotation_in_dtype_is_the_rounded_exact_rotation():
    """The rows the operation uses are the exact rotation rounded once to the dtype: fp32
    equals torch's float64 -> float32 cast of a float64 rotation computed by torch, and
    every bf16 element is a bf16 value no further from the exact rotation than half a
    bf16 step (the nearest one)."""
    n, d = 400, 64
    r = np.random.default_rng(21)
    x = torch.from_numpy(r.standard_normal((n, d))).to(torch.bfloat16).double().numpy()
    ang = r.uniform(-3, 3, (n, d // 2))
    c = np.cos(ang).astype(np.float32).astype(np.float64)
    s = np.sin(ang).astype(np.float32).astype(np.float64)
    xt, ct, st = torch.from_numpy(x), torch.from_numpy(c), torch.from_numpy(s)
    h = d // 2
    ref64 = torch.cat((xt[:, :h] * ct - xt[:, h:] * st, xt[:, h:] * ct + xt[:, :h] * st), -1)
    f32 = rope.rotate_in_dtype(x, c, s, "fp32")
    np.testing.assert_array_equal(f32, ref64.to(torch.float32).double().numpy())
    exact = rope.rotate(x, c, s)
    b16 = rope.rotate_in_dtype(x, c, s, "bf16")
    assert np.all(b16 == torch.from_numpy(b16).to(torch.bfloat16).double().numpy())
    half_ulp = np.ldexp(1.0, np.frexp(exact)[1] - 9)
    assert np.all(np.abs(b16 - exact) <= half_ulp)
    # and it is not simply the identity or an unrotated copy
    assert np.mean(b16 != x) > 0.9
    # without tables a side is returned as given
    assert np.array_equal(rope.rotate_in_dtype(x, None, None, "bf16"), x)


def test_bf16_fused_loss_equals_unfused_pipeline():
    """The fused loss in bf16 equals the plain loss on the same pre-RoPE bf16 activations
    rotated the way a model does it outside the operation (torch fp32 products and sums,
    then a cast to bf16), up to the rare elements where that fp32 evaluation and the exact
    rotation round to different bf16 neighbours."""
    (r,) = workloads.make_rope_inputs("llama2_4k", N=300, Hq=1, Hkv=1, relations=("qq",))

    def model_rope(x, c, s_):
        x = x.float()
        h = x.shape[-1] // 2
        y = torch.cat((x[..., :h] * c - x[..., h:] * s_, x[..., h:] * c + x[..., :h] * s_), -1)
        return y.to(torch.bfloat16).double().numpy()

    ut = model_rope(r.x_t, r.cos_t, r.sin_t)
    us = model_rope(r.x_s, r.cos_s, r.sin_s)
    fused_t = rope.rotate_in_dtype(r.x_t.double().numpy(), r.cos_t.double().numpy(),
                                   r.sin_t.double().numpy(), "bf16")
    assert (fused_t != ut).mean() < 1e-3  # the roundings agree almost everywhere
    tabs = [t.double().numpy() for t in (r.cos_t, r.sin_t, r.cos_s, r.sin_s)]
    sc = oracle.default_scale(128)
    a = rope.forward(r.x_t.double().numpy(), r.x_s.double().numpy(), sc, True, *tabs, dtype="bf16")
    b = oracle.forward(ut, us, sc, True)
    # a bf16 step on under 1e-3 of the elements moves the loss by about 1e-7 relative
    assert abs(a["loss"] - b["loss"]) <= 1e-6 * b["loss"]
