"""Seeded sweep of random problems through the RoPE-fused entry points (lard_relkl_rope_fwd /
_bwd through the C ABI) against the float64 oracle (``oracle.rope``): batch, heads, length
(1 to 500, ragged), head dimension, dtype, mask, head map and upstream gradient are drawn per
case, and each side's rotation is a random cos / sin table or none (a side without tables is
used as given).  Each case is held to the plain gates (below 64 rows, plus the named floor of
tiny_n_floor).  LARD_ROPE_RANDOM_CASES widens the sweep."""

import os

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import assert_parity, banner, tiny_n_floor
from tests.test_rope_gpu import gpu_rope, oracle_rope, rand_tables

pytestmark = pytest.mark.gpu
CASES = int(os.environ.get("LARD_ROPE_RANDOM_CASES", "24"))


@pytest.mark.parametrize("seed", range(CASES))
def test_random_rope_case(seed):
    r = np.random.default_rng(9000 + seed)
    B, H_in = int(r.integers(1, 3)), int(r.integers(1, 4))
    N = int(r.integers(1, 64)) if r.random() < 0.25 else int(r.integers(64, 501))
    d = int(r.choice([64, 128]))
    dtype = torch.bfloat16 if r.random() < 0.6 else torch.float32
    causal = bool(r.random() < 0.6)
    g = float(r.choice([1.0, 0.37, -2.0]))
    noise = float(r.choice([0.06, 0.1, 0.3]))
    head_map = None
    if r.random() < 0.4:
        k = int(r.integers(1, H_in + 1))
        head_map = [int(v) for v in r.permutation(H_in)[:k]]
    sides = r.choice(["both", "both", "teacher", "student"])
    tabs_t = rand_tables(N, d, 2 * seed + 1) if sides in ("both", "teacher") else (None, None)
    tabs_s = rand_tables(N, d, 2 * seed + 2) if sides in ("both", "student") else (None, None)
    tabs = (*tabs_t, *tabs_s)
    banner(f"random rope {seed}: B={B} H_in={H_in} N={N} d={d} {dtype} causal={causal} "
           f"map={head_map} rotated={sides} g={g}")
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn((B, H_in, N, d), generator=gen)
    x_s = x + noise * torch.randn(x.shape, generator=gen)
    x_t, x_s = x.to(dtype), x_s.to(dtype)
    dx_dtype = torch.float32 if r.random() < 0.6 else dtype
    f, dx = gpu_rope(x_t, x_s, tabs, causal, head_map=head_map, dx_dtype=dx_dtype, g=g)
    fo, dxo = oracle_rope(x_t, x_s, tabs, causal, head_map=head_map, g=g)
    floor = tiny_n_floor(fo, x_s, oracle.default_scale(d)) if N < 64 else None
    if floor is not None:  # the gradient floor scales with |g|
        floor = (floor[0], floor[1] * abs(g))
    grad_dtype = torch.bfloat16 if dx_dtype == torch.bfloat16 else dtype
    assert_parity(f, dx, fo, dxo, dtype, f"random rope {seed}", floor=floor,
                  grad_dtype=grad_dtype)
