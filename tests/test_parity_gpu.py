"""GPU parity of the HIP relation-KL path (called through the C ABI) with the float64
oracle, on the seeded workload recipes at sizes the oracle finishes in seconds, with
ragged tails over several row tiles (256 rows) and key tiles (64 rows)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import (GRAD_RL2, LOSS_RTOL, ROW_KL_RL2, assert_parity, banner, device,
                        gpu_fwd_bwd, np64, oracle_fwd_bwd, rel_l2, state, table,
                        tiny_n_floor)

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tiny_workload_full():
    """The tiny fp32 Q/Q workload at its full size (N=256, d=64, causal)."""
    banner("tiny fp32 N=256 d=64 causal")
    (rel,) = workloads.make_inputs("tiny")
    f, dx = gpu_fwd_bwd(rel.x_t, rel.x_s, True)
    fo, dxo = oracle_fwd_bwd(rel.x_t, rel.x_s, True)
    d = assert_parity(f, dx, fo, dxo, torch.float32, "tiny")
    table(f"tiny/causal qq loss_rel {d['loss_rel']:.2e} max_dlse {d['lse_abs']:.2e} "
          f"row_kl_rl2 {d['row_kl_rl2']:.2e} grad_rl2 {d['grad_rl2']:.2e}")
    err = np.abs(np64(f["row_kl"]) - fo["row_kl"])
    print(f"[parity] tiny row_kl max abs err {err.max():.3e}", flush=True)
    np.testing.assert_allclose(np64(f["row_kl"]), fo["row_kl"], rtol=1e-4, atol=1e-7)
    assert float(f["row_kl"][0, 0, 0].item()) == 0.0  # causal row 0: one entry, KL exactly 0


@pytest.mark.parametrize("name,n,hq,hkv,b", [
    ("llama2_4k", 1000, 2, 2, 1),
    ("gqa_16k", 777, 4, 2, 1),
    ("batched_8k", 600, 2, 2, 2),
])
def test_workload_recipes_reduced(name, n, hq, hkv, b):
    """bf16 relations of each recipe at a reduced size, every mask the workload runs."""
    wl = workloads.WORKLOADS[name]
    rels = workloads.make_inputs(wl, N=n, Hq=hq, Hkv=hkv, B=b)
    for causal in wl.masks:
        for rel in rels:
            banner(f"{name} {rel.name} N={n} causal={causal}")
            f, dx = gpu_fwd_bwd(rel.x_t, rel.x_s, causal)
            fo, dxo = oracle_fwd_bwd(rel.x_t, rel.x_s, causal)
            assert_parity(f, dx, fo, dxo, torch.bfloat16, f"{name}/{rel.name}/c{int(causal)}")
            # fp32 gradient output isolates the kernel's own error from bf16 output rounding
            _, dx32 = gpu_fwd_bwd(rel.x_t, rel.x_s, causal, dx_dtype=torch.float32)
            e32 = rel_l2(np64(dx32), dxo)
            print(f"[parity] fp32-out grad rl2 {e32:.3e}", flush=True)
            assert e32 <= 1e-3


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 63, 64, 65, 255, 256, 257, 513])
def test_edge_sizes(n, causal, d, dtype):
    """Ragged and tiny sizes.  N >= 64 is held to the plain gates; below that a row has
    only a few entries and the named fp32 floor of tiny_n_floor applies."""
    banner(f"edge N={n} d={d} causal={causal} {dtype}")
    g = torch.Generator().manual_seed(n * 7 + d)
    x = torch.randn((1, 2, n, d), generator=g)
    x_t = x.to(dtype)
    x_s = (x + 0.2 * torch.randn((1, 2, n, d), generator=g)).to(dtype)
    f, dx = gpu_fwd_bwd(x_t, x_s, causal, dx_dtype=torch.float32)
    fo, dxo = oracle_fwd_bwd(x_t, x_s, causal)
    scale = oracle.default_scale(d)
    floor = tiny_n_floor(fo, x_s, scale) if n < 64 else None
    assert_parity(f, dx, fo, dxo, dtype, f"edge N={n}", floor=floor)
    if causal:  # row 0 keeps one entry: R_t = R_s = 1, KL exactly 0
        assert torch.all(f["row_kl"][..., 0] == 0)
        assert torch.all(f["diag_delta"][..., 0] == 0)
    if n == 1:  # one entry per row: loss and gradient exactly 0
        assert np.all(fo["row_kl"] == 0.0) and not np.any(dxo)
        assert float(f["loss"].item()) == 0.0
        assert torch.all(f["row_kl"] == 0)
        assert torch.all(dx == 0)


@pytest.mark.parametrize("n", [200, 333, 400, 777])
def test_vv_small_kl_loss(n):
    """The V/V relation of the GQA recipe (student V = V + 0.05 noise), whose row KL is
    about 1e-4 of its LSE, at short lengths where the diagonal carries nearly all of each
    row's mass: loss and row KL at the plain bf16 gate, five draws each."""
    for seed in range(5):
        banner(f"V/V N={n} seed={seed}")
        (rel,) = workloads.make_inputs("gqa_16k", seed=seed, N=n, Hq=2, Hkv=2,
                                       relations=("vv",))
        f, dx = gpu_fwd_bwd(rel.x_t, rel.x_s, True, dx_dtype=torch.float32)
        fo, dxo = oracle_fwd_bwd(rel.x_t, rel.x_s, True)
        assert_parity(f, dx, fo, dxo, torch.bfloat16, f"vv N={n} seed={seed}")


def test_golden_closed_form():
    """Structured inputs whose relation KL has a closed form (tests/golden)."""
    with open(os.path.join(ROOT, "tests", "golden", "closed_form.json")) as fh:
        gold = json.load(fh)
    for case in gold["cases"]:
        if case["d"] not in (64, 128):
            continue
        n, d = case["N"], case["d"]
        for dtype in (torch.float32, torch.bfloat16):
            banner(f"golden {case['name']} {dtype}")
            e = torch.zeros((1, 1, n, d))
            m = min(n, d)
            e[0, 0, torch.arange(m), torch.arange(m)] = 1.0
            x_t, x_s = (case["a"] * e).to(dtype), (case["b"] * e).to(dtype)
            f, dx = gpu_fwd_bwd(x_t, x_s, case["causal"], dx_dtype=torch.float32,
                                scale=case["scale"], g=case["g"])
            np.testing.assert_allclose(np64(f["lse_t"])[0, 0], case["lse_t"], rtol=2e-6, atol=2e-6)
            np.testing.assert_allclose(np64(f["lse_s"])[0, 0], case["lse_s"], rtol=2e-6, atol=2e-6)
            err = abs(float(f["loss"].item()) - case["loss"])
            # Every row of these structured inputs is alike, so a row's fp32 rounding is
            # repeated by every row instead of averaging out; where the diagonal carries a
            # small part of the row (N > d leaves zero rows; non-causal rows of 200
            # entries) the row KL is a difference of terms of size |LSE|.  For fp32 inputs
            # the gate therefore adds the per-row fp32 floor of tiny_n_floor (named case:
            # the closed-form goldens); bf16's gate is far above it.
            ref = {k: np.array(case[k]) for k in ("lse_t", "lse_s", "row_kl")}
            floor = tiny_n_floor(ref, x_s, case["scale"])[0] if dtype == torch.float32 else 0.0
            print(f"[parity] golden {case['name']} loss rel err {err / max(case['loss'], 1e-30):.3e}"
                  f" floor {floor / max(case['loss'], 1e-30):.3e}")
            assert err <= LOSS_RTOL[dtype] * case["loss"] + floor
            np.testing.assert_allclose(np64(f["row_kl"])[0, 0], case["row_kl"],
                                       rtol=ROW_KL_RL2, atol=floor / n)
            rows = case["dx_rows"]
            got = np64(dx)[0, 0][rows]
            ref = np.array(case["dx"])
            assert rel_l2(got, ref) <= 1e-3, rel_l2(got, ref)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_student_equals_teacher_is_exactly_zero(causal, dtype):
    banner(f"exact zero causal={causal} {dtype}")
    g = torch.Generator().manual_seed(3)
    x = torch.randn((2, 3, 300, 128), generator=g).to(dtype)
    f, dx = gpu_fwd_bwd(x, x.clone(), causal, dx_dtype=torch.float32)
    assert float(f["loss"].item()) == 0.0
    assert torch.all(f["row_kl"] == 0)
    assert torch.equal(f["lse_t"], f["lse_s"])
    assert torch.all(f["diag_delta"] == 0)
    assert torch.all(dx == 0)


def test_deterministic_and_split_invariant(monkeypatch):
    banner("determinism / split-K")
    (rel,) = workloads.make_inputs("llama2_4k", N=700, Hq=2, Hkv=2, relations=("qq",))
    f1, dx1 = gpu_fwd_bwd(rel.x_t, rel.x_s, True, dx_dtype=torch.float32)
    f2, dx2 = gpu_fwd_bwd(rel.x_t, rel.x_s, True, dx_dtype=torch.float32)
    assert torch.equal(f1["loss"], f2["loss"]) and torch.equal(dx1, dx2)
    assert torch.equal(f1["lse_t"], f2["lse_t"]) and torch.equal(f1["row_kl"], f2["row_kl"])
    outs = []
    for s in ("1", "3", "11"):
        monkeypatch.setenv("LARD_SPLITK", s)
        _, dx = gpu_fwd_bwd(rel.x_t, rel.x_s, True, dx_dtype=torch.float32)
        outs.append(np64(dx))
    for o in outs[1:]:
        assert rel_l2(o, outs[0]) < 1e-6


def test_head_map_and_untouched_heads():
    """GQA: K expanded to 8 query-head slots (repeat 4x); head_map picks the distinct KV
    heads.  Unmapped heads of dx keep their previous contents."""
    banner("head_map")
    dev = device()
    g = torch.Generator().manual_seed(5)
    k = torch.randn((1, 2, 333, 128), generator=g)
    k_s = k + 0.1 * torch.randn((1, 2, 333, 128), generator=g)
    rep_t = k.repeat_interleave(4, dim=1).to(torch.bfloat16).to(dev)
    rep_s = k_s.repeat_interleave(4, dim=1).to(torch.bfloat16).to(dev)
    hm = [0, 4]
    f = relkl.relkl_fwd(rep_t, rep_s, causal=True, head_map=hm, want_row_kl=True)
    sentinel = torch.full(rep_s.shape, 7.0, dtype=torch.float32, device=dev)
    relkl.relkl_bwd(rep_t, rep_s, *state(f), torch.ones((), device=dev),
                    causal=True, head_map=hm, dx=sentinel)
    torch.cuda.synchronize()
    base_t, base_s = k.to(torch.bfloat16), k_s.to(torch.bfloat16)
    fo, dxo = oracle_fwd_bwd(base_t, base_s, True)
    assert abs(float(f["loss"].item()) - fo["loss"]) <= 1e-4 * fo["loss"]
    got = np64(sentinel)
    assert rel_l2(got[:, [0, 4]], dxo) <= 1e-3
    untouched = [h for h in range(8) if h not in hm]
    assert np.all(got[:, untouched] == 7.0)


def test_strided_inputs_match_contiguous():
    """Inputs taken as views of a [B, N, H, d] buffer (stride over n = H * d)."""
    banner("strided")
    dev = device()
    g = torch.Generator().manual_seed(6)
    buf_t = torch.randn((2, 300, 3, 128), generator=g).to(torch.bfloat16).to(dev)
    buf_s = (buf_t.float() + 0.1 * torch.randn((2, 300, 3, 128), generator=g).to(dev)).to(torch.bfloat16)
    v_t, v_s = buf_t.permute(0, 2, 1, 3), buf_s.permute(0, 2, 1, 3)
    assert not v_t.is_contiguous()
    f1 = relkl.relkl_fwd(v_t, v_s, causal=True)
    f2 = relkl.relkl_fwd(v_t.contiguous(), v_s.contiguous(), causal=True)
    gl = torch.ones((), device=dev)
    d1 = relkl.relkl_bwd(v_t, v_s, *state(f1), gl, causal=True)
    d2 = relkl.relkl_bwd(v_t.contiguous(), v_s.contiguous(), *state(f2), gl, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(f1["loss"], f2["loss"])
    assert torch.equal(d1.contiguous(), d2)


def test_autograd_function():
    banner("autograd")
    dev = device()
    g = torch.Generator().manual_seed(8)
    x_t = torch.randn((1, 2, 200, 64), generator=g).to(dev)
    x_s = (x_t + 0.3 * torch.randn((1, 2, 200, 64), generator=g).to(dev)).requires_grad_(True)
    loss = relkl.relation_kl(x_t, x_s, causal=True)
    (2.5 * loss).backward()
    fo, dxo = oracle_fwd_bwd(x_t.cpu(), x_s.detach().cpu(), True, g=2.5)
    assert float(loss.item()) == pytest.approx(fo["loss"], rel=1e-5)
    assert rel_l2(np64(x_s.grad), dxo) <= GRAD_RL2[torch.float32]
    # the pages' mean over rows: loss / N, gradient scaled alike
    x_s.grad = None
    mean = relkl.relation_kl(x_t, x_s, causal=True, reduction="mean_rows")
    (2.5 * mean).backward()
    assert float(mean.item()) == pytest.approx(fo["loss"] / 200, rel=1e-5)
    assert rel_l2(np64(x_s.grad), dxo / 200) <= GRAD_RL2[torch.float32]


def test_side_stream_matches_default_stream():
    """Forward and backward issued on a side stream (outputs and workspaces allocated on
    it) give bitwise the results of the default stream."""
    banner("side stream")
    dev = device()
    (rel,) = workloads.make_inputs("llama2_4k", N=600, Hq=2, Hkv=2, relations=("kk",))
    xt, xs = rel.x_t.to(dev), rel.x_s.to(dev)
    gl = torch.ones((), device=dev)
    f0 = relkl.relkl_fwd(xt, xs, causal=True)
    d0 = relkl.relkl_bwd(xt, xs, *state(f0), gl, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    f1 = relkl.relkl_fwd(xt, xs, causal=True, stream=side)
    d1 = relkl.relkl_bwd(xt, xs, *state(f1), gl, causal=True, stream=side)
    side.synchronize()
    assert torch.equal(f0["loss"], f1["loss"]) and torch.equal(f0["lse_t"], f1["lse_t"])
    assert torch.equal(f0["diag_delta"], f1["diag_delta"])
    assert torch.equal(d0, d1)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_growing_row_maximum(causal, d, dtype):
    """Token norms that grow along the sequence: every row's maximum logit keeps rising
    across key blocks by far more than 64 in log2 units, so the forward's fast update
    (which keeps a row's exponent bias) must keep handing blocks to its exact rescaling
    path.  Rows are alpha_j u + noise with alpha_j rising from 1 to 40."""
    n = 700
    banner(f"growing maxima N={n} d={d} causal={causal} {dtype}")
    gen = torch.Generator().manual_seed(7)
    u = torch.randn(d, generator=gen, dtype=torch.float64)
    u = u / u.norm()
    alpha = 1.0 + 39.0 * (torch.arange(n, dtype=torch.float64) / (n - 1)) ** 2
    noise = torch.randn((1, 2, n, d), generator=gen, dtype=torch.float64)
    x_t = alpha[None, None, :, None] * u + 0.3 * noise
    x_s = x_t + 0.05 * torch.randn((1, 2, n, d), generator=gen, dtype=torch.float64)
    x_t, x_s = x_t.to(dtype), x_s.to(dtype)
    f, dx = gpu_fwd_bwd(x_t, x_s, causal)
    fo, dxo = oracle_fwd_bwd(x_t, x_s, causal)
    # These rows are dominated by entries far above their own diagonal (scores up to
    # alpha_max^2 ~ 1600, LSE up to ~140 nats), so the row KL (~3e-3) is formed from
    # quantities of size LSE whose fp32 ulp is ~1e-5: a per-row precision of about
    # 2^-23 LSE / KL ~ 5e-3 at worst; the row-KL gate here is 1e-3 (the loss and gradient
    # keep the plain gates).
    assert_parity(f, dx, fo, dxo, dtype, "growing", row_kl_rl2=1e-3)


def test_relations_in_one_call_through_a_fused_qkv_buffer():
    """Q/Q, K/K and V/V of equal head counts in one launch: a fused projection buffer
    [N, 3, H, d] viewed as [3, H, N, d] (the batch index selects the relation) gives, in one
    call, the sum of the three relation losses and each relation's gradient, bitwise equal
    to three separate calls."""
    banner("fused QKV buffer, one call")
    dev = device()
    rels = workloads.make_inputs("llama2_4k", N=500, Hq=2, Hkv=2)
    H, N, d = 2, 500, 128
    buf_t = torch.empty((N, 3, H, d), dtype=torch.bfloat16, device=dev)
    buf_s = torch.empty_like(buf_t)
    for k, r in enumerate(rels):
        buf_t[:, k] = r.x_t[0].permute(1, 0, 2).to(dev)
        buf_s[:, k] = r.x_s[0].permute(1, 0, 2).to(dev)
    v_t, v_s = buf_t.permute(1, 2, 0, 3), buf_s.permute(1, 2, 0, 3)  # [3, H, N, d] views
    assert v_t.stride() == (H * d, d, 3 * H * d, 1)
    gl = torch.ones((), device=dev)
    f = relkl.relkl_fwd(v_t, v_s, causal=True)
    dx = relkl.relkl_bwd(v_t, v_s, *state(f), gl, causal=True, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    total, parts = 0.0, []
    for k, r in enumerate(rels):
        xt, xs = r.x_t.to(dev), r.x_s.to(dev)
        fk = relkl.relkl_fwd(xt, xs, causal=True)
        dk = relkl.relkl_bwd(xt, xs, *state(fk), gl, causal=True, dx_dtype=torch.float32)
        torch.cuda.synchronize()
        total += float(fk["loss"].item())
        assert torch.equal(dx[k], dk[0]), k
    assert abs(float(f["loss"].item()) - total) <= 1e-6 * total
