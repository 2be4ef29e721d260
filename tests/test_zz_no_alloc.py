"""The allocation-free forward (lard_relkl_fwd_noalloc, through the C ABI) against the
workspace forward (lard_relkl_fwd): bitwise equal outputs on two calls in a row, the second
on a smaller input (the library's per-GPU scratch keeps the first call's partials)."""

import pytest
import torch

from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import banner, device

pytestmark = pytest.mark.gpu


def outputs(x, want_row_kl=True):
    b, h, n, _ = x.shape
    vec = lambda: torch.empty((b, h, n), dtype=torch.float32, device=x.device)  # noqa: E731
    return vec(), vec(), vec(), (vec() if want_row_kl else None), torch.empty(
        (), dtype=torch.float32, device=x.device)


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_forward_matches_workspace_forward(causal):
    dev = device()
    for n, h, seed in ((1000, 4, 0), (300, 1, 1)):
        banner(f"no-alloc forward N={n} H={h} causal={causal}")
        (rel,) = workloads.make_inputs("llama2_4k", seed=seed, N=n, Hq=h, Hkv=h,
                                       relations=("vv",))
        xt, xs = rel.x_t.to(dev), rel.x_s.to(dev)
        ref = relkl.relkl_fwd(xt, xs, causal=causal, want_row_kl=True)
        lt, ls, dg, kl, loss = outputs(xt)
        relkl.relkl_fwd_noalloc(xt, xs, lt, ls, dg, kl, loss, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(loss, ref["loss"]), (float(loss), float(ref["loss"]))
        assert torch.equal(lt, ref["lse_t"]) and torch.equal(ls, ref["lse_s"])
        assert torch.equal(dg, ref["diag_delta"]) and torch.equal(kl, ref["row_kl"])


def test_noalloc_rejects_sizes_beyond_its_scratch():
    dev = device()
    # 3 x 86 units x ceil(32768 / 128) row tiles = 66048 > LARD_NOALLOC_MAX_PARTIALS = 65536
    x = torch.zeros((3, 86, 32768, 64), dtype=torch.bfloat16, device=dev)
    lt, ls, dg, kl, loss = outputs(x, want_row_kl=False)
    with pytest.raises(relkl.LardError) as ei:
        relkl.relkl_fwd_noalloc(x, x, lt, ls, dg, kl, loss, causal=True)
    assert ei.value.status == 3  # LARD_ERR_WORKSPACE_TOO_SMALL, before any launch
