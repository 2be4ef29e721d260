"""Seeded sweep of random grouped launches (lard_relkl_group_fwd / _bwd through the C ABI): one
to four members of one dtype, head dimension and mask, each with its own batch, heads, length
(1 to 400, ragged), head map, logit scale and noise, and one upstream gradient.  Every member is
held to the plain gates against the float64 oracle (below 64 rows, plus the named floor of
tiny_n_floor), the group's loss to the loss gate, and every member's forward outputs must equal
those of a single call on the same inputs bit for bit (the forward does not depend on how the
launch is shared).  LARD_GROUP_RANDOM_CASES widens the sweep."""

import os

import numpy as np
import pytest
import torch

import oracle
from attention_relation_distillation_amd import relkl
from tests._gpu import LOSS_RTOL, assert_parity, banner, device, oracle_fwd_bwd, tiny_n_floor

pytestmark = pytest.mark.gpu
CASES = int(os.environ.get("LARD_GROUP_RANDOM_CASES", "24"))


def draw_group(seed):
    r = np.random.default_rng(5000 + seed)
    d = int(r.choice([64, 128]))
    c = dict(d=d, dtype=torch.bfloat16 if r.random() < 0.6 else torch.float32,
             causal=bool(r.random() < 0.6), g=float(r.choice([1.0, 0.37, -2.0])),
             members=[])
    c["dx_dtype"] = torch.float32 if r.random() < 0.6 else c["dtype"]
    for _ in range(int(r.integers(1, relkl_max_group() + 1))):
        m = dict(B=int(r.integers(1, 3)), H_in=int(r.integers(1, 5)),
                 N=int(r.integers(1, 64)) if r.random() < 0.25 else int(r.integers(64, 401)),
                 noise=float(r.choice([0.06, 0.1, 0.3])),
                 scale=oracle.default_scale(d) if r.random() < 0.7 else float(r.uniform(0.1, 0.2)))
        if r.random() < 0.4:
            k = int(r.integers(1, m["H_in"] + 1))
            m["head_map"] = [int(v) for v in r.permutation(m["H_in"])[:k]]
        else:
            m["head_map"] = None
        c["members"].append(m)
    return c


def relkl_max_group():
    return 4  # LARD_MAX_GROUP


@pytest.mark.parametrize("seed", range(CASES))
def test_random_group(seed):
    c = draw_group(seed)
    banner(f"random group {seed}: d={c['d']} {c['dtype']} causal={c['causal']} g={c['g']} "
           f"members={c['members']}")
    dev = device()
    gen = torch.Generator().manual_seed(77 + seed)
    pairs, pairs_dev = [], []
    for m in c["members"]:
        x = torch.randn((m["B"], m["H_in"], m["N"], c["d"]), generator=gen)
        x_s = x + m["noise"] * torch.randn(x.shape, generator=gen)
        x_t, x_s = x.to(c["dtype"]), x_s.to(c["dtype"])
        pairs.append((x_t, x_s))
        pairs_dev.append((x_t.to(dev), x_s.to(dev)))
    maps = [m["head_map"] for m in c["members"]]
    scales = [m["scale"] for m in c["members"]]
    f = relkl.group_relkl_fwd(pairs_dev, causal=c["causal"], scale=scales, head_maps=maps,
                              want_row_kl=True)
    gl = torch.tensor(c["g"], dtype=torch.float32, device=dev)
    dx = relkl.group_relkl_bwd(pairs_dev, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                               causal=c["causal"], scale=scales, head_maps=maps,
                               dx_dtype=c["dx_dtype"])
    torch.cuda.synchronize()
    total, floor_total = 0.0, 0.0
    grad_dtype = torch.bfloat16 if c["dx_dtype"] == torch.bfloat16 else c["dtype"]
    for k, (m, (x_t, x_s), (xt_d, xs_d)) in enumerate(zip(c["members"], pairs, pairs_dev)):
        fs = relkl.relkl_fwd(xt_d, xs_d, causal=c["causal"], scale=m["scale"],
                             head_map=m["head_map"], want_row_kl=True)
        torch.cuda.synchronize()
        for key in ("lse_t", "lse_s", "diag_delta", "row_kl"):
            assert torch.equal(f[key][k], fs[key]), (seed, k, key)
        assert torch.equal(f["member_loss"][k], fs["loss"]), (seed, k)
        fo, dxo = oracle_fwd_bwd(x_t, x_s, c["causal"], head_map=m["head_map"],
                                 scale=m["scale"], g=c["g"])
        total += fo["loss"]
        floor = tiny_n_floor(fo, x_s, m["scale"]) if m["N"] < 64 else None
        if floor is not None:  # the gradient floor scales with |g|
            floor_total += floor[0]
            floor = (floor[0], floor[1] * abs(c["g"]))
        mem = {"loss": f["member_loss"][k], "lse_t": f["lse_t"][k], "lse_s": f["lse_s"][k],
               "diag_delta": f["diag_delta"][k], "row_kl": f["row_kl"][k]}
        assert_parity(mem, dx[k], fo, dxo, c["dtype"], f"group {seed} member {k}", floor=floor,
                      grad_dtype=grad_dtype)
        if m["head_map"] is not None:  # heads outside the map stay zero in the new gradient
            rest = [h for h in range(m["H_in"]) if h not in m["head_map"]]
            assert not torch.any(dx[k][:, rest])
    got = float(f["loss"].item())
    assert abs(got - total) <= LOSS_RTOL[c["dtype"]] * abs(total) + floor_total, (got, total)
