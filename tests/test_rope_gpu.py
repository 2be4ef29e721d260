"""GPU parity of the RoPE-fused entry points (lard_relkl_rope_fwd / _bwd through the C ABI)
with the float64 oracle (``oracle.rope``), on the workload recipes handed over before the
rotation: reduced sizes with ragged tails, edge sizes, head maps, the autograd function,
and the full-size 4K and 32K shapes on sampled rows.

The fused path rounds the rotated rows to the input dtype, as a model that applies RoPE
itself would; the oracle takes the exact rotation of the same bytes and tables rounded once
to that dtype.  The kernel forms the same value (exact products in fp64, one rounding of
their sum or difference, one rounding to the dtype), so the rotated rows it keeps in the
reserve equal the oracle's bit for bit; the other outputs are held to the plain path's
gates."""

import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import (GRAD_RL2, LOSS_RTOL, assert_parity, banner, device, np64, rel_l2,
                        state, tiny_n_floor)

pytestmark = pytest.mark.gpu


def tables_of(rel):
    return (rel.cos_t, rel.sin_t, rel.cos_s, rel.sin_s)


def np_tables(tabs):
    return [None if t is None else t.double().numpy() for t in tabs]


def gpu_rope(x_t, x_s, tabs, causal, head_map=None, dx_dtype=None, g=1.0, dx=None):
    dev = device()
    xt, xs = x_t.to(dev), x_s.to(dev)
    tg = [None if t is None else t.to(dev).contiguous() for t in tabs]
    f = relkl.rope_relkl_fwd(xt, xs, *tg, causal=causal, head_map=head_map, want_row_kl=True)
    gl = torch.tensor(g, dtype=torch.float32, device=dev)
    out = relkl.rope_relkl_bwd(xs, f["reserve"], *state(f), gl, *tg, causal=causal,
                               head_map=head_map, dx_dtype=dx_dtype, dx=dx)
    torch.cuda.synchronize()
    return f, out


def dtype_name(t):
    return "bf16" if t == torch.bfloat16 else "fp32"


def oracle_rope(x_t, x_s, tabs, causal, head_map=None, g=1.0):
    s = oracle.default_scale(x_t.shape[-1])
    ct, st, cs, ss = np_tables(tabs)
    xt, xs = np64(x_t), np64(x_s)
    dt = dtype_name(x_t.dtype)
    fo = rope.forward(xt, xs, s, causal, ct, st, cs, ss, head_map=head_map, dtype=dt)
    dxo = rope.backward(xt, xs, s, causal, g, ct, st, cs, ss, head_map=head_map, dtype=dt)
    return fo, dxo


def rand_tables(n, d, seed):
    ang = torch.rand((n, d // 2), generator=torch.Generator().manual_seed(seed),
                     dtype=torch.float64) * 6.0 - 3.0
    return torch.cos(ang).float(), torch.sin(ang).float()


@pytest.mark.parametrize("name,n,hq,hkv,b", [
    ("llama2_4k", 1000, 2, 2, 1),
    ("gqa_16k", 777, 4, 2, 1),
    ("batched_8k", 600, 2, 2, 2),
])
def test_rope_recipes_reduced(name, n, hq, hkv, b):
    wl = workloads.WORKLOADS[name]
    rels = workloads.make_rope_inputs(wl, N=n, Hq=hq, Hkv=hkv, B=b)
    for causal in wl.masks:
        for rel in rels:
            banner(f"rope {name} {rel.name} N={n} causal={causal}")
            f, dx = gpu_rope(rel.x_t, rel.x_s, tables_of(rel), causal)
            fo, dxo = oracle_rope(rel.x_t, rel.x_s, tables_of(rel), causal)
            assert_parity(f, dx, fo, dxo, torch.bfloat16, f"rope {name}/{rel.name}/c{int(causal)}")
            _, dx32 = gpu_rope(rel.x_t, rel.x_s, tables_of(rel), causal, dx_dtype=torch.float32)
            e32 = rel_l2(np64(dx32), dxo)
            print(f"[parity] rope fp32-out grad rl2 {e32:.3e}", flush=True)
            assert e32 <= 1e-3


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n", [1, 2, 3, 65, 257])
def test_rope_edge_sizes(n, causal, d, dtype):
    banner(f"rope edge N={n} d={d} causal={causal} {dtype}")
    g = torch.Generator().manual_seed(n * 11 + d)
    x = torch.randn((1, 2, n, d), generator=g)
    x_t = x.to(dtype)
    x_s = (x + 0.2 * torch.randn((1, 2, n, d), generator=g)).to(dtype)
    tabs = (*rand_tables(n, d, 1), *rand_tables(n, d, 2))
    f, dx = gpu_rope(x_t, x_s, tabs, causal, dx_dtype=torch.float32)
    fo, dxo = oracle_rope(x_t, x_s, tabs, causal)
    floor = tiny_n_floor(fo, x_s, oracle.default_scale(d)) if n < 64 else None
    assert_parity(f, dx, fo, dxo, dtype, f"rope edge N={n}", floor=floor)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rope_without_tables_is_plain_path(dtype):
    """No tables on either side: the fused path runs the plain kernels on copies of the
    inputs, bitwise the plain path.  Identity tables give bitwise the same results as no
    tables (x cos - y sin = x exactly)."""
    banner(f"rope null tables {dtype}")
    g = torch.Generator().manual_seed(21)
    x = torch.randn((1, 2, 300, 128), generator=g)
    x_t, x_s = x.to(dtype), (x + 0.1 * torch.randn(x.shape, generator=g)).to(dtype)
    none = (None, None, None, None)
    one, zero = torch.ones((300, 64)), torch.zeros((300, 64))
    f0, d0 = gpu_rope(x_t, x_s, none, True, dx_dtype=torch.float32)
    f1, d1 = gpu_rope(x_t, x_s, (one, zero, one, zero), True, dx_dtype=torch.float32)
    assert torch.equal(f0["loss"], f1["loss"]) and torch.equal(d0, d1)
    dev = device()
    fp = relkl.relkl_fwd(x_t.to(dev), x_s.to(dev), causal=True)
    dp = relkl.relkl_bwd(x_t.to(dev), x_s.to(dev), *state(fp), torch.ones((), device=dev),
                         causal=True, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(f0["loss"], fp["loss"]) and torch.equal(f0["lse_t"], fp["lse_t"])
    assert torch.equal(d0, dp)


def test_rope_head_map_and_untouched_heads():
    banner("rope head_map")
    dev = device()
    g = torch.Generator().manual_seed(9)
    k = torch.randn((1, 2, 300, 128), generator=g)
    rep = k.repeat_interleave(4, dim=1).to(torch.bfloat16)
    ct, st = workloads.rope_tables(300, 128, 500000.0, 1.0)
    cs, ss = workloads.rope_tables(300, 128, 500000.0, 4.0)
    tabs = (ct, st, cs, ss)
    hm = [1, 6]
    sentinel = torch.full(rep.shape, 3.0, dtype=torch.float32, device=dev)
    f, _ = gpu_rope(rep, rep, tabs, True, head_map=hm, dx=sentinel)
    fo, dxo = oracle_rope(rep[:, hm], rep[:, hm], tabs, True)
    assert abs(float(f["loss"].item()) - fo["loss"]) <= 1e-4 * fo["loss"]
    got = np64(sentinel)
    assert rel_l2(got[:, hm], dxo) <= 1e-3
    assert np.all(got[:, [h for h in range(8) if h not in hm]] == 3.0)


def test_rope_autograd_function():
    banner("rope autograd")
    dev = device()
    g = torch.Generator().manual_seed(12)
    x = torch.randn((1, 2, 200, 64), generator=g)
    ct, st = workloads.rope_tables(200, 64, 10000.0, 1.0)
    cs, ss = workloads.rope_tables(200, 64, 10000.0, 8.0)
    xs = x.clone().to(dev).requires_grad_(True)
    loss = relkl.rope_relation_kl(x.to(dev), xs, ct.to(dev), st.to(dev), cs.to(dev), ss.to(dev),
                                  causal=True)
    (0.5 * loss).backward()
    fo, dxo = oracle_rope(x, x, (ct, st, cs, ss), True, g=0.5)
    assert float(loss.item()) == pytest.approx(fo["loss"], rel=1e-5)
    assert rel_l2(np64(xs.grad), dxo) <= GRAD_RL2[torch.float32]


def sample_rows(n, seed):
    r = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 255, 256, n // 2, n - 2, n - 1]
    return np.array(sorted(set(v for v in fixed + r.integers(0, n, 6).tolist() if 0 <= v < n)))


def check_rope_full(name, full_loss):
    wl = workloads.WORKLOADS[name]
    banner(f"rope full-size {name}: generating inputs")
    rels = workloads.make_rope_inputs(wl)
    dev = device()
    scale = oracle.default_scale(wl.d)
    causal = True
    for rel in rels:
        banner(f"rope {name} {rel.name}: GPU fwd+bwd")
        tabs = tables_of(rel)
        f, dx = gpu_rope(rel.x_t, rel.x_s, tabs, causal)
        loss = float(f["loss"].item())
        row_kl, lse_t = np64(f["row_kl"]), np64(f["lse_t"])
        assert np.isfinite(loss) and loss > 0 and np.all(np.isfinite(row_kl))
        assert row_kl.min() >= -1e-5
        assert abs(loss - row_kl.sum()) <= 1e-6 * abs(loss) + 1e-6
        assert torch.isfinite(dx.float()).all()
        ct, st, cs, ss = np_tables(tabs)
        B, H, N = row_kl.shape
        for k, (b, h) in enumerate([(0, 0), (B - 1, H - 1)]):
            ut = rope.rotate_in_dtype(rel.x_t[b, h].double().numpy(), ct, st, "bf16")
            us = rope.rotate_in_dtype(rel.x_s[b, h].double().numpy(), cs, ss, "bf16")
            rows = sample_rows(N, k)
            lt, ls, kl = oracle.forward_unit(ut, us, scale, causal, chunk=512, rows=rows)
            assert np.max(np.abs(lse_t[b, h, rows] - lt)) <= 5e-5 * max(1.0, np.max(np.abs(lt)))
            assert np.all(np.abs(row_kl[b, h, rows] - kl) <= 1e-3 * np.abs(kl) + 2e-6)
            if k == 0:
                banner(f"rope {name} {rel.name}: oracle gradient of sampled rows")
                if N > 4096:
                    rows = np.array(sorted(set([N - 1024, N - 257, N - 1]
                                               + np.random.default_rng(3).integers(N - 1024, N, 4).tolist())))
                    need = np.arange(rows.min(), N)
                else:
                    need = np.arange(N)
                flt, fls = np.full(N, np.nan), np.full(N, np.nan)
                flt[need], fls[need], _ = oracle.forward_unit(ut, us, scale, causal, chunk=1024,
                                                               rows=need)
                g_rot = oracle.backward_unit(ut, us, scale, causal, 1.0, lse_t=flt, lse_s=fls,
                                             rows=rows, chunk=1024)
                g_ref = rope.rotate_back(g_rot, None if cs is None else cs[rows],
                                         None if ss is None else ss[rows])
                e = rel_l2(np64(dx[b, h])[rows], g_ref)
                print(f"[parity] rope {name}/{rel.name} sampled-row grad rel-L2 {e:.3e}",
                      flush=True)
                assert e <= GRAD_RL2[torch.bfloat16]
        if full_loss:
            banner(f"rope {name} {rel.name}: full oracle loss")
            fo = rope.forward(rel.x_t.double().numpy(), rel.x_s.double().numpy(), scale, causal,
                              ct, st, cs, ss, chunk=1024, dtype="bf16")
            e = abs(loss - fo["loss"]) / fo["loss"]
            print(f"[parity] rope {name}/{rel.name} full loss rel err {e:.3e}", flush=True)
            assert e <= LOSS_RTOL[torch.bfloat16]


def test_rope_llama2_4k_full():
    check_rope_full("llama2_4k", full_loss=True)


def test_rope_llama2_32k_sampled():
    check_rope_full("llama2_32k", full_loss=False)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_reserve_is_the_rounded_rotation_bit_for_bit(d, dtype):
    """The reserve's rotated rows (dense [units][N][d] per side, each copy starting on a
    256-byte boundary) against rope.rotate_in_dtype of the same bytes and tables, compared
    as bit patterns; the teacher side rotated, the student side with other tables, and a
    head map that picks heads out of order."""
    n, h_in = 301, 3
    hm = [2, 0]
    banner(f"rope reserve bits d={d} {dtype}")
    g = torch.Generator().manual_seed(40 + d)
    x = torch.randn((2, h_in, n, d), generator=g) * 3.0
    x_t = x.to(dtype)
    x_s = (x + 0.1 * torch.randn((2, h_in, n, d), generator=g)).to(dtype)
    ct, st = rand_tables(n, d, 1)
    cs, ss = rand_tables(n, d, 2)
    f, _ = gpu_rope(x_t, x_s, (ct, st, cs, ss), True, head_map=hm)
    e = 2 if dtype == torch.bfloat16 else 4
    units = 2 * len(hm)
    copy = units * n * d * e
    stride = (copy + 255) // 256 * 256
    res = f["reserve"].cpu()
    view = torch.int16 if dtype == torch.bfloat16 else torch.int32
    got_t = res[:copy].view(view).reshape(2, len(hm), n, d)
    got_s = res[stride:stride + copy].view(view).reshape(2, len(hm), n, d)
    dt = dtype_name(dtype)
    ref_t = rope.rotate_in_dtype(np64(x_t)[:, hm], ct.double().numpy(), st.double().numpy(), dt)
    ref_s = rope.rotate_in_dtype(np64(x_s)[:, hm], cs.double().numpy(), ss.double().numpy(), dt)
    want_t = torch.from_numpy(ref_t).to(dtype).view(view)
    want_s = torch.from_numpy(ref_s).to(dtype).view(view)
    assert torch.equal(got_t, want_t), int((got_t != want_t).sum())
    assert torch.equal(got_s, want_s), int((got_s != want_s).sum())
