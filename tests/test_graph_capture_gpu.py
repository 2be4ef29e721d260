"""The library's calls inside a captured HIP graph: the entry points only launch kernels on
the given stream (no allocation, no memset, no synchronisation), so a forward + backward
can be captured once and replayed.  Every replay, with eager work and synchronisations in
between, must match the eager result bitwise.  The allocation-free forward is captured into
outputs allocated beforehand, as a caller that cannot allocate would use it."""

import pytest
import torch

from attention_relation_distillation_amd import relkl, workloads
from tests._gpu import banner, device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", ["plain", "rope", "cross", "group", "noalloc"])
def test_capture_and_replay(path):
    banner(f"graph capture {path}")
    dev = device()
    q, k = workloads.make_rope_inputs("llama2_4k", N=700, Hq=2, Hkv=2, relations=("qq", "kk"))
    xt, xs = q.x_t.to(dev), q.x_s.to(dev)
    kt, ks = k.x_t.to(dev), k.x_s.to(dev)
    tabs = [t.to(dev) for t in (q.cos_t, q.sin_t, q.cos_s, q.sin_s)]
    gl = torch.ones((), dtype=torch.float32, device=dev)
    # outputs of the allocation-free forward and its backward, allocated before any capture
    rows = (xt.shape[0], xt.shape[1], xt.shape[2])
    na = [torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(3)]
    na_loss = torch.empty((), dtype=torch.float32, device=dev)
    na_dx = torch.empty_like(xs)

    def run():
        if path == "noalloc":
            relkl.relkl_fwd_noalloc(xt, xs, na[0], na[1], na[2], None, na_loss, causal=True)
            relkl.relkl_bwd(xt, xs, na[0], na[1], na[2], gl, causal=True, dx=na_dx)
            return na_loss, na_dx
        if path == "plain":
            f = relkl.relkl_fwd(xt, xs, causal=True)
            return f["loss"], relkl.relkl_bwd(xt, xs, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                                              causal=True)
        if path == "rope":
            f = relkl.rope_relkl_fwd(xt, xs, *tabs, causal=True)
            return f["loss"], relkl.rope_relkl_bwd(xs, f["reserve"], f["lse_t"], f["lse_s"],
                                                   f["diag_delta"], gl, *tabs, causal=True)
        if path == "cross":
            f = relkl.cross_relkl_fwd(xt, kt, xs, ks, rope=tabs, causal=True)
            da, db = relkl.cross_relkl_bwd(xs, ks, f["reserve"], f["lse_t"], f["lse_s"], gl,
                                           rope=tabs, causal=True)
            return f["loss"], torch.cat((da, db), dim=1)
        # grouped: Q/Q on two heads and K/K on one (a head view), both rotated inside the call
        pairs = [(xt, xs), (kt[:, :1], ks[:, :1])]
        f = relkl.group_relkl_fwd(pairs, causal=True, rope=[tabs, tabs])
        dq, dk = relkl.group_relkl_bwd(pairs, f["lse_t"], f["lse_s"], f["diag_delta"], gl,
                                       reserve=f["reserve"], causal=True, rope=[tabs, tabs])
        loss = torch.stack((f["loss"], f["member_loss"][0], f["member_loss"][1]))
        return loss, torch.cat((dq, dk), dim=1)

    ref_loss, ref_dx = run()
    torch.cuda.synchronize()
    ref_loss, ref_dx = ref_loss.clone(), ref_dx.clone()
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        run()  # warm-up on the side stream before capture
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_loss, g_dx = run()
    for rep in range(3):
        junk = torch.randn((1024, 1024), device=dev) @ torch.randn((1024, 1024), device=dev)
        g_dx.fill_(float("nan"))  # the replay must rewrite everything it returns
        g_loss.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_loss, ref_loss), rep
        assert torch.equal(g_dx, ref_dx), rep
        del junk
