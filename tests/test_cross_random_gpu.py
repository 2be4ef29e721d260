"""Seeded sweep of random problems through the cross-relation entry points
(lard_relkl_cross_fwd / _bwd through the C ABI) against the float64 oracle (``oracle.cross``):
batch, heads, length (1 to 500, ragged), head dimension, dtype, mask, head map, noise and
upstream gradient are drawn per case, and the call rotates A and B inside it with random
cos / sin tables on both sides, on one side, or on neither.  Each case is held to the
relation path's gates on the loss and on each of dA_s and dB_s (below 64 rows, plus the named
floor of tiny_n_floor).  LARD_CROSS_RANDOM_CASES widens the sweep."""

import os

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import banner, tiny_n_floor
from tests.test_cross_gpu import check, gpu_cross, oracle_cross, quad
from tests.test_rope_gpu import rand_tables

pytestmark = pytest.mark.gpu
CASES = int(os.environ.get("LARD_CROSS_RANDOM_CASES", "24"))


@pytest.mark.parametrize("seed", range(CASES))
def test_random_cross_case(seed):
    r = np.random.default_rng(13000 + seed)
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
    sides = r.choice(["none", "both", "both", "teacher", "student"])
    tabs = None
    if sides != "none":
        tabs_t = rand_tables(N, d, 2 * seed + 1) if sides in ("both", "teacher") else (None, None)
        tabs_s = rand_tables(N, d, 2 * seed + 2) if sides in ("both", "student") else (None, None)
        tabs = (*tabs_t, *tabs_s)
    dx_dtype = torch.float32 if r.random() < 0.6 else dtype
    banner(f"random cross {seed}: B={B} H_in={H_in} N={N} d={d} {dtype} causal={causal} "
           f"map={head_map} rotated={sides} g={g} dx={dx_dtype}")
    a_t, b_t, a_s, b_s = quad(B, H_in, N, d, dtype, seed=20000 + seed, noise=noise)
    f, da, db = gpu_cross(a_t, b_t, a_s, b_s, causal, tabs=tabs, head_map=head_map,
                          dx_dtype=dx_dtype, g=g)
    fo, dao, dbo = oracle_cross(a_t, b_t, a_s, b_s, causal, tabs=tabs, head_map=head_map, g=g)
    floors = tiny_n_floor(fo, a_s, oracle.default_scale(d)) if N < 64 else None
    if floors is not None:  # the gradient floor scales with |g|
        floors = (floors[0], floors[1] * abs(g))
    check(f, da, db, fo, dao, dbo, dtype, f"random {seed}", floors)
