"""GPU parity at the size limits: a sequence four times the longest workload, the largest
number of relation heads one call computes (through a head map), and a launch of many
small units.  All through the C ABI, against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import (GRAD_RL2, LOSS_RTOL, ROW_KL_RL2, assert_parity, banner, device,
                        gpu_fwd_bwd, np64, oracle_fwd_bwd, rel_l2, state)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rel_name", ["qq", "vv"])
def test_long_sequence_131k_sampled(rel_name):
    """N = 131072 (the 32K recipe at four times the length, one head): the oracle computes
    sampled rows one by one.  LSE and row KL of the first, middle and last rows; gradient of
    the last 256 rows, whose column terms involve only rows after them; the loss equals the
    sum of the row KLs at any size."""
    n = 131072
    banner(f"N={n} {rel_name}: inputs")
    (rel,) = workloads.make_inputs("llama2_32k", N=n, Hq=1, Hkv=1, relations=(rel_name,))
    dev = device()
    xt, xs = rel.x_t.to(dev), rel.x_s.to(dev)
    banner(f"N={n} {rel_name}: GPU fwd+bwd")
    f = relkl.relkl_fwd(xt, xs, causal=True, want_row_kl=True)
    gl = torch.ones((), dtype=torch.float32, device=dev)
    dx = relkl.relkl_bwd(xt, xs, *state(f), gl, causal=True)
    torch.cuda.synchronize()
    loss = float(f["loss"].item())
    row_kl = np64(f["row_kl"])[0, 0]
    assert np.isfinite(loss) and loss > 0 and np.all(np.isfinite(row_kl))
    assert row_kl.min() >= -1e-5
    assert abs(loss - row_kl.sum()) <= 1e-6 * loss
    assert torch.isfinite(dx.float()).all()
    assert row_kl[0] == 0.0  # causal row 0: one entry

    banner(f"N={n} {rel_name}: oracle rows")
    ut = rel.x_t[0, 0].double().numpy()
    us = rel.x_s[0, 0].double().numpy()
    scale = oracle.default_scale(ut.shape[1])
    r = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(8), r.integers(8, n - 256, 24),
                                     np.arange(n - 256, n)]))
    lt, ls, kl = oracle.forward_unit(ut, us, scale, True, chunk=256, rows=rows)
    dlse = max(float(np.max(np.abs(np64(f["lse_t"])[0, 0, rows] - lt))),
               float(np.max(np.abs(np64(f["lse_s"])[0, 0, rows] - ls))))
    kl_rl2 = rel_l2(row_kl[rows], kl)
    last = np.arange(n - 256, n)
    flt, fls = np.full(n, np.nan), np.full(n, np.nan)
    sel = np.searchsorted(rows, last)
    flt[last], fls[last] = lt[sel], ls[sel]
    g_ref = oracle.backward_unit(ut, us, scale, True, 1.0, lse_t=flt, lse_s=fls, rows=last,
                                 chunk=256)
    g_rl2 = rel_l2(np64(dx[0, 0])[last], g_ref)
    print(f"[sizes] N={n} {rel_name} max_dlse {dlse:.2e} row_kl_rl2 {kl_rl2:.2e} "
          f"grad_rl2 {g_rl2:.2e}", flush=True)
    assert dlse <= 5e-5 * max(1.0, float(np.max(np.abs(lt))))
    assert kl_rl2 <= ROW_KL_RL2
    assert g_rl2 <= GRAD_RL2[torch.bfloat16]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_max_relation_heads_through_head_map(dtype):
    """LARD_MAX_HEADS relation heads selected (in a scrambled order) from 300 input heads; the
    unselected input heads of dx keep their contents.  One more head is refused."""
    h_in, h = 300, relkl.LARD_MAX_HEADS
    banner(f"{h} heads of {h_in}, {dtype}")
    g = torch.Generator().manual_seed(21)
    x = torch.randn((1, h_in, 70, 64), generator=g)
    x_s = x + 0.1 * torch.randn((1, h_in, 70, 64), generator=g)
    x_t, x_s = x.to(dtype), x_s.to(dtype)
    hm = np.random.default_rng(3).permutation(h_in)[:h].tolist()
    dev = device()
    xt, xs = x_t.to(dev), x_s.to(dev)
    f = relkl.relkl_fwd(xt, xs, causal=True, head_map=hm, want_row_kl=True)
    sentinel = torch.full(xs.shape, 3.0, dtype=torch.float32, device=dev)
    relkl.relkl_bwd(xt, xs, *state(f), torch.ones((), device=dev), causal=True, head_map=hm,
                    dx=sentinel)
    torch.cuda.synchronize()
    fo, dxo = oracle_fwd_bwd(x_t, x_s, True, head_map=hm)
    got = np64(sentinel)
    assert abs(float(f["loss"].item()) - fo["loss"]) <= LOSS_RTOL[dtype] * fo["loss"]
    assert rel_l2(np64(f["row_kl"]), fo["row_kl"]) <= ROW_KL_RL2
    assert dxo.shape == got.shape  # the oracle places each head's gradient at its input head
    assert rel_l2(got[:, hm], dxo[:, hm]) <= GRAD_RL2[dtype]
    untouched = sorted(set(range(h_in)) - set(hm))
    assert np.all(got[:, untouched] == 3.0)
    with pytest.raises(relkl.LardError):
        relkl.relkl_fwd(xt, xs, causal=True, head_map=hm + [sorted(untouched)[0]])


@pytest.mark.parametrize("causal", [True, False])
def test_many_small_units(causal):
    """B = 64, H = 32 (2048 units) of N = 70: a grid of many short units, one row tile and
    two key tiles (the second ragged) each."""
    banner(f"2048 units of N=70, causal={causal}")
    g = torch.Generator().manual_seed(22)
    x = torch.randn((64, 32, 70, 128), generator=g)
    x_s = x + 0.05 * torch.randn((64, 32, 70, 128), generator=g)
    x_t, x_s = x.to(torch.bfloat16), x_s.to(torch.bfloat16)
    f, dx = gpu_fwd_bwd(x_t, x_s, causal)
    fo, dxo = oracle_fwd_bwd(x_t, x_s, causal)
    assert_parity(f, dx, fo, dxo, torch.bfloat16, f"2048 units causal={causal}")
