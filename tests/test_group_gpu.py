"""GPU parity of the grouped entry points (lard_relkl_group_fwd / _bwd through the C ABI):
several relation problems -- Q/Q on the query heads, K/K and V/V on the KV heads of a GQA
layer -- in one launch per kernel.  Every member is checked against the float64 oracle at
the dtype's gates, and against the single-problem entry points on the same inputs: forward
outputs bitwise, gradients bitwise when both use the same split count."""

import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import (GRAD_RL2, LOSS_RTOL, assert_parity, banner, device, np64, state,
                        oracle_fwd_bwd, rel_l2)

pytestmark = pytest.mark.gpu


def to_dev(pairs, tabs=None):
    dev = device()
    ps = [(a.to(dev), b.to(dev)) for a, b in pairs]
    rp = None
    if tabs is not None:
        rp = [None if t is None else [v.to(dev).contiguous() for v in t] for t in tabs]
    return ps, rp


def gpu_group(pairs, causal, head_maps=None, tabs=None, dx_dtype=None, g=1.0):
    dev = device()
    ps, rp = to_dev(pairs, tabs)
    f = relkl.group_relkl_fwd(ps, causal=causal, head_maps=head_maps, rope=rp, want_row_kl=True)
    gl = torch.tensor(g, dtype=torch.float32, device=dev)
    dx = relkl.group_relkl_bwd(ps, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                               reserve=f["reserve"], causal=causal, head_maps=head_maps,
                               rope=rp, dx_dtype=dx_dtype)
    torch.cuda.synchronize()
    return f, dx


def gpu_group_scaled(pairs, causal, head_maps, scales):
    dev = device()
    ps, _ = to_dev(pairs)
    f = relkl.group_relkl_fwd(ps, causal=causal, head_maps=head_maps, scale=scales,
                              want_row_kl=True)
    gl = torch.ones((), dtype=torch.float32, device=dev)
    dx = relkl.group_relkl_bwd(ps, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                               causal=causal, head_maps=head_maps, scale=scales)
    torch.cuda.synchronize()
    return f, dx


def gpu_single(x_t, x_s, causal, head_map=None, tabs=None, dx_dtype=None):
    dev = device()
    xt, xs = x_t.to(dev), x_s.to(dev)
    gl = torch.ones((), dtype=torch.float32, device=dev)
    if tabs is None:
        f = relkl.relkl_fwd(xt, xs, causal=causal, head_map=head_map, want_row_kl=True)
        dx = relkl.relkl_bwd(xt, xs, *state(f), gl, causal=causal, head_map=head_map,
                             dx_dtype=dx_dtype)
    else:
        tg = [None if t is None else t.to(dev).contiguous() for t in tabs]
        f = relkl.rope_relkl_fwd(xt, xs, *tg, causal=causal, head_map=head_map, want_row_kl=True)
        dx = relkl.rope_relkl_bwd(xs, f["reserve"], *state(f), gl, *tg, causal=causal,
                                  head_map=head_map, dx_dtype=dx_dtype)
    torch.cuda.synchronize()
    return f, dx


def member(f, k):
    return {"loss": f["member_loss"][k], "lse_t": f["lse_t"][k], "lse_s": f["lse_s"][k],
            "diag_delta": f["diag_delta"][k], "row_kl": f["row_kl"][k]}


def assert_same_as_single(f, dx, k, fs, dxs, label):
    for key in ("lse_t", "lse_s", "diag_delta", "row_kl"):
        assert torch.equal(f[key][k], fs[key]), (label, key)
    assert torch.equal(f["member_loss"][k], fs["loss"]), label
    assert torch.equal(dx[k], dxs), label


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n", [333, 777])
def test_group_gqa_layer_matches_oracle(n, causal, dtype):
    """Q/Q on 4 query heads, K/K and V/V on 2 KV heads, ragged tiles, one group; the V/V
    row KL is about 5e-5 per row at these lengths."""
    banner(f"group GQA layer N={n} causal={causal} {dtype}")
    rels = workloads.make_inputs("gqa_16k", N=n, Hq=4, Hkv=2)
    pairs = [(r.x_t.to(dtype), r.x_s.to(dtype)) for r in rels]
    f, dx = gpu_group(pairs, causal, dx_dtype=torch.float32)
    total = 0.0
    for k, (r, (x_t, x_s)) in enumerate(zip(rels, pairs)):
        fo, dxo = oracle_fwd_bwd(x_t, x_s, causal)
        total += fo["loss"]
        assert_parity(member(f, k), dx[k], fo, dxo, dtype, f"group {r.name} c{int(causal)}")
    got = float(f["loss"].item())
    print(f"[parity] group total {got} oracle {total}", flush=True)
    assert abs(got - total) <= LOSS_RTOL[dtype] * abs(total)


def test_group_equals_single_calls(monkeypatch):
    """Members of different B, H, N and head maps: each member's outputs are bitwise those
    of a single call with the same split count; with the default split counts (which
    depend on the group's total work) the gradients agree to rounding."""
    banner("group vs single calls")
    g = torch.Generator().manual_seed(5)

    def pair(b, h, n, noise=0.3):
        x = torch.randn((b, h, n, 128), generator=g)
        return x.to(torch.bfloat16), (x + noise * torch.randn(x.shape, generator=g)).to(torch.bfloat16)

    pairs = [pair(1, 4, 300), pair(2, 3, 517), pair(1, 2, 64)]
    maps = [None, [2, 0], [1]]
    for splits in ("3", None):
        if splits is None:
            monkeypatch.delenv("LARD_SPLITK", raising=False)
        else:
            monkeypatch.setenv("LARD_SPLITK", splits)
        f, dx = gpu_group(pairs, True, head_maps=maps)
        total = 0.0
        for k, ((x_t, x_s), hm) in enumerate(zip(pairs, maps)):
            fs, dxs = gpu_single(x_t, x_s, True, head_map=hm)
            total += float(fs["loss"].item())
            if splits is not None:
                assert_same_as_single(f, dx, k, fs, dxs, f"member {k}")
            else:
                for key in ("lse_t", "lse_s", "row_kl"):
                    assert torch.equal(f[key][k], fs[key]), (k, key)
                e = rel_l2(np64(dx[k]), np64(dxs))
                print(f"[parity] member {k} default splits: grad rl2 vs single {e:.2e}", flush=True)
                assert e <= 1e-5
            if hm is not None:  # heads outside the map stay zero in the new gradient
                rest = [h for h in range(x_s.shape[1]) if h not in hm]
                assert not torch.any(dx[k][:, rest])
        assert abs(float(f["loss"].item()) - total) <= 1e-6 * total


def test_group_rope_layer(monkeypatch):
    """The RoPE-fused group: Q/Q and K/K rotated with their tables, V/V without, inputs
    before the rotation; against the oracle and bitwise against single fused calls."""
    banner("group RoPE layer")
    monkeypatch.setenv("LARD_SPLITK", "2")
    rels = workloads.make_rope_inputs("gqa_16k", N=777, Hq=4, Hkv=2)
    pairs = [(r.x_t, r.x_s) for r in rels]
    tabs = [None if r.cos_t is None else (r.cos_t, r.sin_t, r.cos_s, r.sin_s) for r in rels]
    f, dx = gpu_group(pairs, True, tabs=tabs)
    s = oracle.default_scale(128)
    for k, r in enumerate(rels):
        if tabs[k] is None:
            # no tables: the fused single call copies the rows unrotated, as the group does
            fs, dxs = gpu_single(r.x_t, r.x_s, True, tabs=(None, None, None, None))
            fo, dxo = oracle_fwd_bwd(r.x_t, r.x_s, True)
        else:
            fs, dxs = gpu_single(r.x_t, r.x_s, True, tabs=tabs[k])
            ct, st, cs, ss = [t.double().numpy() for t in tabs[k]]
            xt, xs = np64(r.x_t), np64(r.x_s)
            fo = rope.forward(xt, xs, s, True, ct, st, cs, ss, dtype="bf16")
            dxo = rope.backward(xt, xs, s, True, 1.0, ct, st, cs, ss, dtype="bf16")
        assert_same_as_single(f, dx, k, fs, dxs, f"rope member {r.name}")
        assert_parity(member(f, k), dx[k], fo, dxo, torch.bfloat16, f"group rope {r.name}")


def test_group_autograd_with_gqa_head_maps():
    """group_relation_kl over Q/Q and the distinct KV heads of repeated K / V tensors
    (head maps), fp32: the gradients of 1.5 x loss against the oracle; repeated heads get
    none."""
    banner("group autograd GQA maps")
    dev = device()
    g = torch.Generator().manual_seed(9)
    n, d = 200, 64
    q = torch.randn((1, 4, n, d), generator=g)
    kv = [torch.randn((1, 2, n, d), generator=g) for _ in range(2)]
    rep = [t.repeat_interleave(2, dim=1) for t in kv]  # [1, 4, n, d]: KV heads repeated
    noisy = [t + 0.2 * torch.randn(t.shape, generator=g) for t in [q] + rep]
    teach = [q] + rep
    xs = [t.clone().to(dev).requires_grad_(True) for t in noisy]
    maps = [None, [0, 2], [0, 2]]
    loss = relkl.group_relation_kl([(t.to(dev), x) for t, x in zip(teach, xs)], causal=True,
                                   head_maps=maps)
    (1.5 * loss).backward()
    total = 0.0
    for k in range(3):
        fo, dxo = oracle_fwd_bwd(teach[k], noisy[k], True, head_map=maps[k], g=1.5)
        total += fo["loss"]
        e = rel_l2(np64(xs[k].grad), dxo)
        print(f"[parity] autograd member {k}: grad rl2 {e:.2e}", flush=True)
        assert e <= GRAD_RL2[torch.float32]
        if maps[k] is not None:
            assert not torch.any(xs[k].grad[:, [1, 3]])
    assert float(loss.item()) == pytest.approx(total, rel=1e-5)


def test_group_fullsize_gqa_16k():
    """The GQA workload at full size (Q/Q on 32 heads, K/K and V/V on 8, N = 16384) in one
    group: bitwise equal to the three single calls (no split at this size), which the
    full-size tests check against the oracle on sampled rows."""
    banner("group gqa_16k full size")
    rels = workloads.make_inputs("gqa_16k")
    pairs = [(r.x_t, r.x_s) for r in rels]
    f, dx = gpu_group(pairs, True)
    total = 0.0
    for k, r in enumerate(rels):
        fs, dxs = gpu_single(r.x_t, r.x_s, True)
        total += float(fs["loss"].item())
        assert_same_as_single(f, dx, k, fs, dxs, f"gqa_16k {r.name}")
        del fs, dxs
    print(f"[parity] gqa_16k group loss {float(f['loss'].item())} sum of singles {total}",
          flush=True)
    assert abs(float(f["loss"].item()) - total) <= 1e-6 * total


def test_group_of_four_members_mixed_scale_and_length():
    """LARD_MAX_GROUP members with their own scale, length, batch and head map, non-causal,
    fp32 (d = 64): each against the oracle at its own scale."""
    banner("group of four, fp32, non-causal")
    g = torch.Generator().manual_seed(13)
    shapes = [(1, 2, 129), (2, 1, 300), (1, 3, 64), (1, 2, 517)]
    pairs = []
    for b, h, n in shapes:
        x = torch.randn((b, h, n, 64), generator=g)
        pairs.append((x, x + 0.3 * torch.randn(x.shape, generator=g)))
    scales = [0.125, 0.09375, 0.1875, 0.125]  # fp32-exact, one per member
    maps = [None, None, [2, 0], [1]]
    f, dx = gpu_group_scaled(pairs, False, maps, scales)
    for k, ((x_t, x_s), hm, sc) in enumerate(zip(pairs, maps, scales)):
        fo, dxo = oracle_fwd_bwd(x_t, x_s, False, head_map=hm, scale=sc)
        assert_parity(member(f, k), dx[k], fo, dxo, torch.float32, f"four/{k}")


def test_group_rope_fullsize_gqa_16k():
    """The GQA workload at full size handed over before the rotation, Q/Q and K/K rotated
    inside one group call, V/V not: bitwise equal to three single fused calls."""
    banner("group RoPE gqa_16k full size")
    rels = workloads.make_rope_inputs("gqa_16k")
    pairs = [(r.x_t, r.x_s) for r in rels]
    tabs = [None if r.cos_t is None else (r.cos_t, r.sin_t, r.cos_s, r.sin_s) for r in rels]
    f, dx = gpu_group(pairs, True, tabs=tabs)
    for k, r in enumerate(rels):
        t = tabs[k] if tabs[k] is not None else (None, None, None, None)
        fs, dxs = gpu_single(r.x_t, r.x_s, True, tabs=t)
        assert_same_as_single(f, dx, k, fs, dxs, f"rope gqa_16k {r.name}")
        del fs, dxs


def test_group_rope_fp32_members(monkeypatch):
    """A RoPE-fused group of fp32 members (fp32 rotated copies in the reserve, members of
    different N and heads, one without tables): bitwise equal to single fused calls, and
    against the RoPE oracle at the fp32 gates."""
    banner("group RoPE fp32")
    monkeypatch.setenv("LARD_SPLITK", "2")
    g = torch.Generator().manual_seed(17)
    specs = [(3, 300, True), (2, 517, True), (2, 200, False)]  # heads, N, rotated
    pairs, tabs = [], []
    for h, n, rot in specs:
        x = torch.randn((1, h, n, 64), generator=g)
        pairs.append((x, x + 0.3 * torch.randn(x.shape, generator=g)))
        if rot:
            ct, st = workloads.rope_tables(n, 64, 10000.0, 1.0)
            cs, ss = workloads.rope_tables(n, 64, 10000.0, 4.0)
            tabs.append((ct, st, cs, ss))
        else:
            tabs.append(None)
    f, dx = gpu_group(pairs, True, tabs=tabs)
    s = oracle.default_scale(64)
    for k, ((x_t, x_s), t) in enumerate(zip(pairs, tabs)):
        tt = t if t is not None else (None, None, None, None)
        fs, dxs = gpu_single(x_t, x_s, True, tabs=tt)
        assert_same_as_single(f, dx, k, fs, dxs, f"rope fp32 member {k}")
        if t is None:
            fo, dxo = oracle_fwd_bwd(x_t, x_s, True)
        else:
            ct, st, cs, ss = [v.double().numpy() for v in t]
            xt, xs = np64(x_t), np64(x_s)
            fo = rope.forward(xt, xs, s, True, ct, st, cs, ss, dtype="fp32")
            dxo = rope.backward(xt, xs, s, True, 1.0, ct, st, cs, ss, dtype="fp32")
        assert_parity(member(f, k), dx[k], fo, dxo, torch.float32, f"group rope fp32 {k}")
