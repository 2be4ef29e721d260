"""C-ABI tests that need no GPU: the library loads, exports what include/lard.h declares,
and rejects invalid requests on the host before any HIP call (no compute is launched)."""

import ctypes
import os
import re

import pytest
import torch

from attention_relation_distillation_amd import relkl
from attention_relation_distillation_amd.relkl import (_CrossDesc, _Desc, _GradDesc, _Member,
                                                       _RopeDesc)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WS_SMALL, HIP = 0, 1, 2, 3, 4
FAKE = 0x100000  # 16-byte-aligned fake device address; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    return relkl.load_library()


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    """Every call here uses fake device addresses: with the launch wrapper told to fail, a
    call that passes validation returns LARD_ERR_HIP instead of reaching a GPU."""
    monkeypatch.setenv("LARD_FAULT_INJECT", "1")


def declared_functions():
    src = open(os.path.join(ROOT, "include", "lard.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lard_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"lard_relkl_fwd", "lard_relkl_bwd", "lard_relkl_workspace_size",
                          "lard_status_string", "lard_version",
                          "lard_relkl_rope_reserve_size", "lard_relkl_rope_fwd",
                          "lard_relkl_rope_bwd", "lard_relkl_cross_reserve_size",
                          "lard_relkl_cross_fwd", "lard_relkl_cross_bwd",
                          "lard_relkl_group_reserve_size", "lard_relkl_group_workspace_size",
                          "lard_relkl_group_fwd", "lard_relkl_group_bwd"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.lard_version() >= 20000


def test_status_strings(lib):
    for code, name in relkl._STATUS_NAMES.items():
        assert lib.lard_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.lard_status_string(99)


def good_desc(**kw):
    base = dict(dtype=1, B=1, H_in=4, N=100, d=128, t_stride_b=4 * 100 * 128,
                t_stride_h=100 * 128, t_stride_n=128, s_stride_b=4 * 100 * 128,
                s_stride_h=100 * 128, s_stride_n=128, H=4, causal=1,
                head_map=ctypes.POINTER(ctypes.c_int32)(), scale=128 ** -0.5)
    base.update(kw)
    return _Desc(**base)


def ws_query(lib, desc, pass_=0):
    st = ctypes.c_int(-1)
    n = lib.lard_relkl_workspace_size(ctypes.byref(desc), pass_, ctypes.byref(st))
    return n, st.value


def fwd(lib, desc, xt=FAKE, xs=FAKE, lt=FAKE, ls=FAKE, dg=FAKE, kl=None, loss=FAKE, ws=FAKE,
        nws=1 << 20):
    return lib.lard_relkl_fwd(ctypes.byref(desc) if desc is not None else None, xt, xs, lt, ls,
                              dg, kl, loss, ws, nws, None)


def bwd(lib, desc, g=None, xt=FAKE, xs=FAKE, lt=FAKE, ls=FAKE, dg=FAKE, gl=FAKE, dx=FAKE,
        ws=FAKE, nws=1 << 30):
    g = g or _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128,
                       stride_n=128)
    return lib.lard_relkl_bwd(ctypes.byref(desc), xt, xs, lt, ls, dg, gl, ctypes.byref(g), dx,
                              ws, nws, None)


def test_workspace_sizes(lib):
    n0, st = ws_query(lib, good_desc(), 0)
    assert st == OK and n0 >= 8 and n0 % 256 == 0
    n1, st = ws_query(lib, good_desc(), 1)
    # 4 units x 1 row tile: the backward splits its key range (2 tiles) in two
    assert st == OK and n1 == 2 * 4 * 256 * 128 * 4
    big = good_desc(N=32768, H_in=32, H=32, t_stride_h=32768 * 128, t_stride_b=32 * 32768 * 128,
                    s_stride_h=32768 * 128, s_stride_b=32 * 32768 * 128)
    n1, st = ws_query(lib, big, 1)
    # the grid fills the chip: no split, no workspace (the state is the forward's outputs)
    assert st == OK and n1 == 0
    n0, st = ws_query(lib, big, 0)
    assert st == OK and n0 < 32 * 32768  # O(B * H * N / 128) partial sums
    _, st = ws_query(lib, good_desc(), 2)
    assert st == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), INVALID),
    (dict(B=0), INVALID),
    (dict(N=0), INVALID),
    (dict(d=32), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED),
    (dict(causal=2), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(H=3), INVALID),                 # no head map: H must equal H_in
    (dict(H=0), INVALID),
    (dict(t_stride_n=100), INVALID),      # not a multiple of 8 bf16 elements
    (dict(s_stride_h=-128), INVALID),
    (dict(t_stride_n=64), INVALID),       # rows overlap (stride over n < d)
    (dict(s_stride_n=1 << 23), UNSUPPORTED),  # bf16 row stride of 16 MiB: beyond 24-bit offsets
    (dict(t_stride_n=(1 << 23) - 8, s_stride_n=128), "ok"),  # just below the limit
    (dict(N=(1 << 30) + 1), UNSUPPORTED),  # beyond LARD_MAX_N (32-bit row indices in the kernels)
    (dict(N=0x7fffffff), UNSUPPORTED),     # no overflow in the sizing of the largest int32 N
])
def test_descriptor_validation(lib, kw, code):
    desc = good_desc(**kw)
    _, st = ws_query(lib, desc, 0)
    if code == "ok":  # valid: the calls get as far as the (injected) launch failure
        assert st == OK
        assert fwd(lib, desc) == HIP
        assert bwd(lib, desc) == HIP
        return
    assert st == code
    assert fwd(lib, desc) == code
    assert bwd(lib, desc) == code


def test_longest_sequence_is_sized_without_overflow(lib):
    n = 1 << 30  # LARD_MAX_N
    desc = good_desc(N=n, H_in=1, H=1, t_stride_h=n * 128, s_stride_h=n * 128,
                     t_stride_b=n * 128, s_stride_b=n * 128)
    ws, st = ws_query(lib, desc, 0)
    assert st == OK
    assert ws == 8 * (n // 128)  # one fp64 loss partial per 128-row forward workgroup


def test_head_map_validation(lib):
    def with_map(vals, h_in=4):
        arr = (ctypes.c_int32 * len(vals))(*vals)
        d = good_desc(H=len(vals), H_in=h_in,
                      head_map=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
        return d, arr

    d, keep = with_map([0, 2])
    assert ws_query(lib, d)[1] == OK
    d, keep = with_map([0, 4])
    assert ws_query(lib, d)[1] == INVALID   # out of range
    d, keep = with_map([1, 1])
    assert ws_query(lib, d)[1] == INVALID   # not injective
    d, keep = with_map([-1])
    assert ws_query(lib, d)[1] == INVALID
    d, keep = with_map(list(range(257)), h_in=300)
    assert ws_query(lib, d)[1] == UNSUPPORTED  # more than LARD_MAX_HEADS
    del keep


def test_pointer_and_workspace_validation(lib):
    d = good_desc()
    assert fwd(lib, d, dg=None) == HIP             # diag_delta is optional in the forward
    assert fwd(lib, d, dg=FAKE + 2) == INVALID     # misaligned state vector
    assert fwd(lib, d, lt=None) == INVALID
    assert bwd(lib, d, dg=None) == INVALID         # the backward needs the forward's state
    assert bwd(lib, d, ls=None) == INVALID
    assert bwd(lib, d, lt=FAKE + 1) == INVALID
    assert bwd(lib, d, gl=None) == INVALID
    assert bwd(lib, d, ws=FAKE + 8) == INVALID     # workspace must be 16-byte aligned
    assert fwd(lib, None) == INVALID
    assert fwd(lib, d, xt=None) == INVALID
    assert fwd(lib, d, loss=None) == INVALID
    assert fwd(lib, d, xs=FAKE + 2) == INVALID     # misaligned
    assert fwd(lib, d, nws=0) == WS_SMALL
    assert bwd(lib, d, dx=None) == INVALID
    assert bwd(lib, d, nws=0) == WS_SMALL
    g = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=130)
    assert bwd(lib, d, g=g) == INVALID
    # fp32 inputs cannot produce a bf16 gradient
    d32 = good_desc(dtype=0)
    g = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=128)
    assert bwd(lib, d32, g=g) == UNSUPPORTED


def test_noalloc_forward_validation(lib):
    def call(desc, lt=FAKE, loss=FAKE):
        return lib.lard_relkl_fwd_noalloc(ctypes.byref(desc), FAKE, FAKE, lt, FAKE, FAKE, None,
                                          loss, None)
    assert call(good_desc(N=0)) == INVALID
    assert call(good_desc(), lt=None) == INVALID
    assert call(good_desc(), loss=None) == INVALID
    # 3 x 86 units x 256 row tiles of 128 = 66048 loss partials > LARD_NOALLOC_MAX_PARTIALS
    big = good_desc(B=3, H_in=86, H=86, N=32768, d=64, t_stride_n=64, s_stride_n=64,
                    t_stride_h=32768 * 64, s_stride_h=32768 * 64, t_stride_b=86 * 32768 * 64,
                    s_stride_b=86 * 32768 * 64)
    assert call(big) == WS_SMALL
    # a valid request reaches the device side (no GPU here, or the injected fault)
    assert call(good_desc()) == HIP


def test_fault_injection_maps_to_hip_error(lib, monkeypatch):
    """A failed launch is reported as LARD_ERR_HIP (the launch wrapper is told to fail
    before it calls HIP), and the Python layer turns it into an exception."""
    monkeypatch.setenv("LARD_FAULT_INJECT", "1")
    assert fwd(lib, good_desc()) == HIP
    assert bwd(lib, good_desc()) == HIP
    with pytest.raises(relkl.LardError) as ei:
        relkl._check(HIP)
    assert ei.value.status == HIP


def test_mfma_probe_validation(lib):
    """The throughput probe checks its arguments on the host; a valid request reaches the
    launch wrapper, which the fixture tells to fail."""
    assert lib.lard_probe_mfma(0, 10, 256, None, None) == INVALID
    assert lib.lard_probe_mfma(2, 10, 256, FAKE, None) == INVALID
    assert lib.lard_probe_mfma(0, 0, 256, FAKE, None) == INVALID
    assert lib.lard_probe_mfma(0, (1 << 20) + 1, 256, FAKE, None) == INVALID
    assert lib.lard_probe_mfma(1, 10, 0, FAKE, None) == INVALID
    assert lib.lard_probe_mfma(1, 10, (1 << 16) + 1, FAKE, None) == INVALID
    assert lib.lard_probe_mfma(0, 10, 256, FAKE + 2, None) == INVALID  # misaligned sink
    assert lib.lard_probe_mfma(0, 10, 256, FAKE, None) == HIP
    assert lib.lard_probe_mfma(1, 1 << 20, 1 << 16, FAKE, None) == HIP
    with pytest.raises(RuntimeError, match="GPU"):
        relkl.probe_mfma(False, 10, 1, torch.zeros(512))


def test_python_layer_range_checks_head_map():
    """Head indices beyond int32 would wrap into valid ones in the ctypes array: the binding
    rejects every entry outside [0, H_in) itself."""
    x = torch.zeros(1, 4, 8, 64)
    for bad in ([2 ** 32], [-1], [4], [0, 2 ** 33 + 1]):
        with pytest.raises(relkl.LardError):
            relkl._make_desc(x, x, True, None, bad)
    desc, keep = relkl._make_desc(x, x, True, None, [3, 1])
    assert desc.H == 2 and desc.head_map[0] == 3 and desc.head_map[1] == 1


def test_python_layer_refuses_cpu_tensors():
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(RuntimeError, match="GPU"):
        relkl.relkl_fwd(x, x)
    with pytest.raises(relkl.LardError):
        relkl.relkl_fwd(torch.zeros(1, 8, 64), torch.zeros(1, 8, 64))
    with pytest.raises(relkl.LardError):
        relkl.relkl_fwd(torch.zeros(1, 1, 8, 64, dtype=torch.float16),
                        torch.zeros(1, 1, 8, 64, dtype=torch.float16))


# ------------------------------------------------------------------ RoPE-fused entry points
def rope_fwd(lib, desc, rope, rs=FAKE, nrs=1 << 30):
    return lib.lard_relkl_rope_fwd(ctypes.byref(desc), ctypes.byref(rope) if rope else None,
                                   FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, rs, nrs, FAKE,
                                   1 << 20, None)


def rope_bwd(lib, desc, rope, rs=FAKE, nrs=1 << 30, dg=FAKE):
    g = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=128)
    return lib.lard_relkl_rope_bwd(ctypes.byref(desc), ctypes.byref(rope) if rope else None,
                                   rs, nrs, FAKE, FAKE, dg, FAKE, ctypes.byref(g), FAKE, FAKE,
                                   1 << 30, None)


def test_rope_reserve_size(lib):
    st = ctypes.c_int(-1)
    n = lib.lard_relkl_rope_reserve_size(ctypes.byref(good_desc()), ctypes.byref(st))
    # the rotated rows of both sides in the input dtype, nothing else
    assert st.value == OK and n == 2 * (((4 * 100 * 128 * 2) + 255) // 256 * 256)
    n = lib.lard_relkl_rope_reserve_size(ctypes.byref(good_desc(dtype=0)), ctypes.byref(st))
    assert st.value == OK and n == 2 * (((4 * 100 * 128 * 4) + 255) // 256 * 256)
    assert lib.lard_relkl_rope_reserve_size(ctypes.byref(good_desc(N=0)), ctypes.byref(st)) == 0
    assert st.value == INVALID


def test_rope_validation(lib):
    d = good_desc()
    both = _RopeDesc(FAKE, FAKE, FAKE, FAKE)
    assert rope_fwd(lib, d, None) == INVALID                          # no rope descriptor
    assert rope_fwd(lib, d, _RopeDesc(FAKE, None, None, None)) == INVALID  # cos without sin
    assert rope_fwd(lib, d, _RopeDesc(None, None, None, FAKE)) == INVALID
    assert rope_fwd(lib, d, _RopeDesc(FAKE + 4, FAKE, None, None)) == INVALID  # misaligned
    assert rope_bwd(lib, d, _RopeDesc(None, None, FAKE, FAKE + 8)) == INVALID
    need = lib.lard_relkl_rope_reserve_size(ctypes.byref(d), None)
    assert rope_fwd(lib, d, both, nrs=need - 1) == WS_SMALL
    assert rope_bwd(lib, d, both, nrs=need - 1) == WS_SMALL
    assert rope_fwd(lib, d, both, rs=FAKE + 64) == INVALID            # reserve alignment
    assert rope_fwd(lib, d, both, rs=None) == INVALID
    assert rope_bwd(lib, d, both, dg=None) == INVALID                 # needs the diag state


def test_rope_fault_injection_maps_to_hip_error(lib, monkeypatch):
    monkeypatch.setenv("LARD_FAULT_INJECT", "1")
    both = _RopeDesc(FAKE, FAKE, FAKE, FAKE)
    assert rope_fwd(lib, good_desc(), both) == HIP
    assert rope_bwd(lib, good_desc(), both) == HIP
    assert rope_fwd(lib, good_desc(), _RopeDesc(None, None, None, None)) == HIP


def test_rope_python_layer_checks_tables():
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(RuntimeError, match="GPU"):
        relkl.rope_relkl_fwd(x, x)
    with pytest.raises(relkl.LardError):
        relkl.rope_relkl_fwd(x, x, torch.zeros(8, 31), torch.zeros(8, 31))


# ------------------------------------------------------------------ cross-relation entry points
def good_keys(**kw):
    base = dict(bt_stride_b=4 * 100 * 128, bt_stride_h=100 * 128, bt_stride_n=128,
                bs_stride_b=4 * 100 * 128, bs_stride_h=100 * 128, bs_stride_n=128)
    base.update(kw)
    return _CrossDesc(**base)


def cross_fwd(lib, desc, keys, rope=None, rs=FAKE, nrs=1 << 30):
    return lib.lard_relkl_cross_fwd(ctypes.byref(desc), ctypes.byref(keys) if keys else None,
                                    ctypes.byref(rope) if rope else None, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, None, FAKE, rs, nrs, FAKE, 1 << 20, None)


def cross_bwd(lib, desc, ga=None, gb=None, rope=None, rs=FAKE, nrs=1 << 30, da=FAKE, db=FAKE,
              lt=FAKE):
    g = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=128)
    ga = ga or g
    gb = gb or g
    return lib.lard_relkl_cross_bwd(ctypes.byref(desc), ctypes.byref(rope) if rope else None,
                                    rs, nrs, lt, FAKE, FAKE, ctypes.byref(ga), da,
                                    ctypes.byref(gb), db, FAKE, 1 << 30, None)


def test_cross_reserve_size(lib):
    st = ctypes.c_int(-1)
    n = lib.lard_relkl_cross_reserve_size(ctypes.byref(good_desc()), ctypes.byref(st))
    assert st.value == OK and n == 4 * (((4 * 100 * 128 * 2) + 255) // 256 * 256)
    n = lib.lard_relkl_cross_reserve_size(ctypes.byref(good_desc(dtype=0)), ctypes.byref(st))
    assert st.value == OK and n == 4 * (((4 * 100 * 128 * 4) + 255) // 256 * 256)


def test_cross_validation(lib):
    d = good_desc()
    assert cross_fwd(lib, d, None) == INVALID                             # no key strides
    assert cross_fwd(lib, d, good_keys(bt_stride_n=100)) == INVALID       # not 16-byte rows
    assert cross_fwd(lib, d, good_keys(bs_stride_n=64)) == INVALID        # overlapping rows
    assert cross_fwd(lib, d, good_keys(), rope=_RopeDesc(FAKE, None, None, None)) == INVALID
    need = lib.lard_relkl_cross_reserve_size(ctypes.byref(d), None)
    assert cross_fwd(lib, d, good_keys(), nrs=need - 1) == WS_SMALL
    assert cross_bwd(lib, d, nrs=need - 1) == WS_SMALL
    assert cross_bwd(lib, d, db=None) == INVALID
    assert cross_bwd(lib, d, lt=None) == INVALID                          # needs the LSE state
    assert cross_bwd(lib, d, da=FAKE + 8) == INVALID                      # misaligned gradient
    bad = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=130)
    assert cross_bwd(lib, d, gb=bad) == INVALID
    g16 = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=128)
    assert cross_bwd(lib, good_desc(dtype=0), ga=g16) == UNSUPPORTED      # fp32 -> bf16 grad


def test_cross_fault_injection_maps_to_hip_error(lib, monkeypatch):
    monkeypatch.setenv("LARD_FAULT_INJECT", "1")
    assert cross_fwd(lib, good_desc(), good_keys()) == HIP
    assert cross_bwd(lib, good_desc()) == HIP


def test_cross_python_layer_checks_shapes():
    a = torch.zeros(1, 1, 8, 64)
    with pytest.raises(relkl.LardError):
        relkl.cross_relkl_fwd(a, torch.zeros(1, 1, 9, 64), a, a)
    with pytest.raises(RuntimeError, match="GPU"):
        relkl.cross_relkl_fwd(a, a, a, a)


# ------------------------------------------------------------------ grouped entry points
def members_of(*descs, rope=None):
    ms = (_Member * len(descs))()
    for k, d in enumerate(descs):
        ms[k].desc = d
        ms[k].x_teacher = ms[k].x_student = FAKE
        ms[k].lse_teacher = ms[k].lse_student = ms[k].diag_delta = ms[k].loss = FAKE
        ms[k].row_kl = None
        if rope is not None:
            ms[k].rope = rope
    return ms


def kv_desc(**kw):  # 2 KV heads of a GQA layer, N = 100
    base = dict(H_in=2, H=2, t_stride_b=2 * 100 * 128, s_stride_b=2 * 100 * 128)
    base.update(kw)
    return good_desc(**base)


def group_query(lib, fn, ms, arg):
    st = ctypes.c_int(-1)
    n = getattr(lib, fn)(len(ms), ms, arg, ctypes.byref(st))
    return n, st.value


def group_fwd(lib, ms, with_rope=0, rs=FAKE, nrs=1 << 30, n=None):
    return lib.lard_relkl_group_fwd(len(ms) if n is None else n, ms, with_rope, FAKE, rs, nrs,
                                    FAKE, 1 << 20, None)


def group_bwd(lib, ms, grads=None, with_rope=0, nrs=1 << 30):
    # (the reserve is read only with with_rope = 1)
    k = len(ms)
    if grads is None:
        grads = [_GradDesc(dtype=1, reserved=0, stride_b=m.desc.t_stride_b,
                           stride_h=m.desc.t_stride_h, stride_n=128) for m in ms]
    g = (_GradDesc * k)(*grads)
    dx = (ctypes.c_void_p * k)(*([FAKE] * k))
    return lib.lard_relkl_group_bwd(k, ms, with_rope, FAKE, nrs, FAKE, g, dx, FAKE, 1 << 30,
                                    None)


def test_group_sizes_are_the_sums_of_the_members(lib):
    q, kv = good_desc(), kv_desc()
    ms = members_of(q, kv, kv)
    n, st = group_query(lib, "lard_relkl_group_reserve_size", ms, 0)
    assert st == OK and n == 0  # the plain path keeps no reserve
    n, st = group_query(lib, "lard_relkl_group_reserve_size", ms, 1)
    one = [lib.lard_relkl_rope_reserve_size(ctypes.byref(d), None) for d in (q, kv, kv)]
    assert st == OK and n == sum(one)
    # forward: one fp64 partial per workgroup of 128 rows, all members back to back
    n, st = group_query(lib, "lard_relkl_group_workspace_size", ms, 0)
    assert st == OK and n == ((8 * (4 + 2 + 2)) + 255) // 256 * 256
    # backward: 8 (unit, row tile) workgroups in total -> the key range (2 tiles) is split
    # in two, fp32 partials of 256 padded rows per unit
    n, st = group_query(lib, "lard_relkl_group_workspace_size", ms, 1)
    assert st == OK and n == 2 * (4 + 2 + 2) * 256 * 128 * 4
    big = good_desc(N=32768, H_in=32, H=32, t_stride_h=32768 * 128, t_stride_b=32 * 32768 * 128,
                    s_stride_h=32768 * 128, s_stride_b=32 * 32768 * 128)
    n, st = group_query(lib, "lard_relkl_group_workspace_size", members_of(big, big), 1)
    assert st == OK and n == 0
    _, st = group_query(lib, "lard_relkl_group_workspace_size", ms, 2)
    assert st == INVALID


def test_group_validation(lib):
    q, kv = good_desc(), kv_desc()
    assert group_fwd(lib, members_of(q), n=0) == INVALID
    five = members_of(q, q, q, q, q)
    assert group_fwd(lib, five) == UNSUPPORTED                   # more than LARD_MAX_GROUP
    assert group_fwd(lib, members_of(q, kv_desc(dtype=0))) == INVALID   # mixed dtype
    assert group_fwd(lib, members_of(q, kv_desc(causal=0))) == INVALID  # mixed mask
    d64 = kv_desc(d=64, t_stride_n=64, s_stride_n=64, t_stride_h=6400, s_stride_h=6400,
                  t_stride_b=12800, s_stride_b=12800)
    assert group_fwd(lib, members_of(q, d64)) == INVALID         # mixed d
    assert group_fwd(lib, members_of(q, kv_desc(N=0))) == INVALID  # an invalid member
    assert group_bwd(lib, members_of(q, kv_desc(d=96))) == UNSUPPORTED
    assert group_fwd(lib, members_of(q, kv), with_rope=2) == INVALID
    # with_rope = 1 checks every member's tables; with_rope = 0 does not read them
    half = _RopeDesc(FAKE, None, None, None)
    both = _RopeDesc(FAKE, FAKE, FAKE, FAKE)
    assert group_fwd(lib, members_of(q, kv, rope=half), with_rope=1, nrs=16) == INVALID
    assert group_fwd(lib, members_of(q, kv, rope=both), with_rope=1, nrs=16) == WS_SMALL
    assert group_fwd(lib, members_of(q, kv, rope=both), with_rope=1, rs=None) == INVALID
    # head maps of one group: at most 512 entries together
    arr = (ctypes.c_int32 * 200)(*range(200))
    hm = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    wide = good_desc(H_in=256, H=200, head_map=hm, t_stride_b=256 * 100 * 128,
                     s_stride_b=256 * 100 * 128)
    n, st = group_query(lib, "lard_relkl_group_reserve_size", members_of(wide, wide), 0)
    assert st == OK
    n, st = group_query(lib, "lard_relkl_group_reserve_size", members_of(wide, wide, wide), 0)
    assert st == UNSUPPORTED and n == 0
    # reserve too small (with rope), gradients of two dtypes, missing pointers
    need, _ = group_query(lib, "lard_relkl_group_reserve_size", members_of(q, kv), 1)
    assert group_bwd(lib, members_of(q, kv, rope=both), with_rope=1, nrs=need - 1) == WS_SMALL
    g16 = _GradDesc(dtype=1, reserved=0, stride_b=4 * 100 * 128, stride_h=100 * 128, stride_n=128)
    g32 = _GradDesc(dtype=0, reserved=0, stride_b=2 * 100 * 128, stride_h=100 * 128, stride_n=128)
    assert group_bwd(lib, members_of(q, kv), grads=[g16, g32]) == INVALID
    ms = members_of(q, kv)
    ms[1].lse_student = None
    assert group_fwd(lib, ms) == INVALID
    assert group_bwd(lib, ms) == INVALID
    ms = members_of(q, kv)
    ms[1].diag_delta = None
    assert group_bwd(lib, ms) == INVALID         # the backward needs every member's state
    ms = members_of(q, kv)
    ms[0].x_teacher = FAKE + 8
    assert group_fwd(lib, ms) == INVALID
    assert group_bwd(lib, ms) == INVALID         # the plain backward reads the inputs
    ms = members_of(q, kv, rope=both)
    ms[0].x_teacher = FAKE + 8
    assert group_bwd(lib, ms, with_rope=1, nrs=16) == WS_SMALL  # the fused one does not
    del arr


def test_group_fault_injection_maps_to_hip_error(lib, monkeypatch):
    monkeypatch.setenv("LARD_FAULT_INJECT", "1")
    ms = members_of(good_desc(), kv_desc(), kv_desc())
    assert group_fwd(lib, ms) == HIP
    assert group_bwd(lib, ms) == HIP
    assert group_fwd(lib, members_of(good_desc(), kv_desc(), rope=_RopeDesc(None, None, None, None)),
                     with_rope=1) == HIP


def test_group_python_layer_checks_members():
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(relkl.LardError):
        relkl.group_relkl_fwd([(x, x)] * 5)
    with pytest.raises(relkl.LardError):
        relkl.group_relkl_fwd([])
    with pytest.raises(relkl.LardError):
        relkl.group_relkl_fwd([(x, x), (x, x)], head_maps=[None])
    with pytest.raises(RuntimeError, match="GPU"):
        relkl.group_relkl_fwd([(x, x), (x, x)])
