"""Python binding of the relation-KL C ABI (include/lard.h).

Argument marshalling only: output buffers and the workspace come from PyTorch's caching
allocator, the stream is PyTorch's current stream, and every arithmetic step runs in the
HIP kernels of liblard.so.  There is no CPU fallback: without the built library or a GPU
these functions raise.

    loss = relation_kl(x_t, x_s, causal=True)          # sum over rows, heads, batch
    loss.backward()                                      # gradient reaches x_s only

Workspaces and outputs are allocated on the stream the call runs on (the ``stream``
argument, else the current stream), so PyTorch's caching allocator never hands them to
other work before that stream has finished with them.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = ["LardError", "library_path", "load_library", "relkl_fwd", "relkl_fwd_noalloc",
           "relkl_bwd",
           "relation_kl", "workspace_size", "rope_reserve_size",
           "rope_relkl_fwd", "rope_relkl_bwd", "rope_relation_kl", "cross_reserve_size",
           "cross_relkl_fwd", "cross_relkl_bwd", "cross_relation_kl", "group_reserve_size",
           "group_workspace_size", "group_relkl_fwd", "group_relkl_bwd", "group_relation_kl",
           "LARD_MAX_HEADS", "LARD_MAX_GROUP"]

LARD_FP32 = 0
LARD_BF16 = 1
LARD_MAX_HEADS = 256
LARD_MAX_GROUP = 4
_STATUS_NAMES = {0: "LARD_OK", 1: "LARD_ERR_INVALID_ARGUMENT", 2: "LARD_ERR_UNSUPPORTED",
                 3: "LARD_ERR_WORKSPACE_TOO_SMALL", 4: "LARD_ERR_HIP"}


class LardError(RuntimeError):
    """A non-zero lard_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H_in", ctypes.c_int32), ("N", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("t_stride_b", ctypes.c_int64), ("t_stride_h", ctypes.c_int64),
        ("t_stride_n", ctypes.c_int64),
        ("s_stride_b", ctypes.c_int64), ("s_stride_h", ctypes.c_int64),
        ("s_stride_n", ctypes.c_int64),
        ("H", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("head_map", ctypes.POINTER(ctypes.c_int32)),
        ("scale", ctypes.c_float),
    ]


class _RopeDesc(ctypes.Structure):
    _fields_ = [
        ("cos_teacher", ctypes.c_void_p), ("sin_teacher", ctypes.c_void_p),
        ("cos_student", ctypes.c_void_p), ("sin_student", ctypes.c_void_p),
    ]


class _CrossDesc(ctypes.Structure):
    _fields_ = [
        ("bt_stride_b", ctypes.c_int64), ("bt_stride_h", ctypes.c_int64),
        ("bt_stride_n", ctypes.c_int64),
        ("bs_stride_b", ctypes.c_int64), ("bs_stride_h", ctypes.c_int64),
        ("bs_stride_n", ctypes.c_int64),
    ]


class _Member(ctypes.Structure):
    _fields_ = [
        ("desc", _Desc),
        ("x_teacher", ctypes.c_void_p), ("x_student", ctypes.c_void_p),
        ("lse_teacher", ctypes.c_void_p), ("lse_student", ctypes.c_void_p),
        ("diag_delta", ctypes.c_void_p),
        ("row_kl", ctypes.c_void_p), ("loss", ctypes.c_void_p),
        ("rope", _RopeDesc),
    ]


class _GradDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("stride_n", ctypes.c_int64),
    ]


_LIB = None


def library_path() -> str:
    """The in-tree liblard.so (LARD_LIBRARY overrides it, e.g. for a host sanitizer build of
    the C-ABI layer in the CPU tests)."""
    return os.environ.get("LARD_LIBRARY") or os.path.join(
        os.path.dirname(os.path.abspath(__file__)), "liblard.so")


def load_library():
    """Load liblard.so (built in-tree by ``__graft_entry__.build()``); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                           "(python -m attention_relation_distillation_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.lard_relkl_workspace_size.restype = sz
    lib.lard_relkl_workspace_size.argtypes = [ctypes.POINTER(_Desc), ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_int)]
    lib.lard_relkl_fwd.restype = ctypes.c_int
    lib.lard_relkl_fwd.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lard_probe_mfma.restype = ctypes.c_int
    lib.lard_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.lard_relkl_fwd_noalloc.restype = ctypes.c_int
    lib.lard_relkl_fwd_noalloc.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lard_relkl_bwd.restype = ctypes.c_int
    lib.lard_relkl_bwd.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp,
                                   ctypes.POINTER(_GradDesc), vp, vp, sz, vp]
    lib.lard_relkl_rope_reserve_size.restype = sz
    lib.lard_relkl_rope_reserve_size.argtypes = [ctypes.POINTER(_Desc),
                                                 ctypes.POINTER(ctypes.c_int)]
    lib.lard_relkl_rope_fwd.restype = ctypes.c_int
    lib.lard_relkl_rope_fwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_RopeDesc), vp,
                                        vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.lard_relkl_rope_bwd.restype = ctypes.c_int
    lib.lard_relkl_rope_bwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_RopeDesc), vp,
                                        sz, vp, vp, vp, vp, ctypes.POINTER(_GradDesc), vp, vp,
                                        sz, vp]
    lib.lard_relkl_cross_reserve_size.restype = sz
    lib.lard_relkl_cross_reserve_size.argtypes = [ctypes.POINTER(_Desc),
                                                  ctypes.POINTER(ctypes.c_int)]
    lib.lard_relkl_cross_fwd.restype = ctypes.c_int
    lib.lard_relkl_cross_fwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_CrossDesc),
                                         ctypes.POINTER(_RopeDesc), vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp, sz, vp]
    lib.lard_relkl_cross_bwd.restype = ctypes.c_int
    lib.lard_relkl_cross_bwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_RopeDesc), vp,
                                         sz, vp, vp, vp, ctypes.POINTER(_GradDesc), vp,
                                         ctypes.POINTER(_GradDesc), vp, vp, sz, vp]
    mp, ci = ctypes.POINTER(_Member), ctypes.c_int
    lib.lard_relkl_group_reserve_size.restype = sz
    lib.lard_relkl_group_reserve_size.argtypes = [ci, mp, ci, ctypes.POINTER(ctypes.c_int)]
    lib.lard_relkl_group_workspace_size.restype = sz
    lib.lard_relkl_group_workspace_size.argtypes = [ci, mp, ci, ctypes.POINTER(ctypes.c_int)]
    lib.lard_relkl_group_fwd.restype = ctypes.c_int
    lib.lard_relkl_group_fwd.argtypes = [ci, mp, ci, vp, vp, sz, vp, sz, vp]
    lib.lard_relkl_group_bwd.restype = ctypes.c_int
    lib.lard_relkl_group_bwd.argtypes = [ci, mp, ci, vp, sz, vp, ctypes.POINTER(_GradDesc),
                                         ctypes.POINTER(ctypes.c_void_p), vp, sz, vp]
    lib.lard_status_string.restype = ctypes.c_char_p
    lib.lard_status_string.argtypes = [ctypes.c_int]
    lib.lard_version.restype = ctypes.c_int
    lib.lard_version.argtypes = []
    _LIB = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().lard_status_string(status).decode()
        raise LardError(status, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return LARD_BF16
    if t == torch.float32:
        return LARD_FP32
    raise LardError(2, f"unsupported dtype {t} (bfloat16 or float32)")


def _make_desc(x_t: torch.Tensor, x_s: torch.Tensor, causal: bool, scale: Optional[float],
               head_map: Optional[Sequence[int]]):
    if x_t.dim() != 4 or x_s.dim() != 4:
        raise LardError(1, "inputs must be [B, H, N, d]")
    if x_t.shape != x_s.shape or x_t.dtype != x_s.dtype:
        raise LardError(1, "teacher and student must have the same shape and dtype")
    if x_t.device != x_s.device:
        raise LardError(1, "teacher and student must be on the same device")
    if x_t.stride(-1) != 1 or x_s.stride(-1) != 1:
        raise LardError(1, "the last dimension (d) must be contiguous")
    b, h_in, n, d = x_t.shape
    keep = []
    if head_map is not None:
        vals = [int(v) for v in head_map]
        if any(v < 0 or v >= h_in for v in vals):
            # checked here too: ctypes would wrap values beyond int32 into valid head indices
            raise LardError(1, f"head_map entries must lie in [0, {h_in})")
        arr = (ctypes.c_int32 * len(vals))(*vals)
        keep.append(arr)
        hm_ptr = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        h = len(head_map)
    else:
        hm_ptr = ctypes.POINTER(ctypes.c_int32)()
        h = h_in
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
    desc = _Desc(dtype=_dtype_code(x_t.dtype), B=b, H_in=h_in, N=n, d=d,
                 t_stride_b=x_t.stride(0), t_stride_h=x_t.stride(1), t_stride_n=x_t.stride(2),
                 s_stride_b=x_s.stride(0), s_stride_h=x_s.stride(1), s_stride_n=x_s.stride(2),
                 H=h, causal=1 if causal else 0, head_map=hm_ptr, scale=scale)
    return desc, keep


def _stream_of(dev: torch.device, stream):
    return torch.cuda.current_stream(dev) if stream is None else stream


def _stream_handle(dev: torch.device, stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(_stream_of(dev, stream).cuda_stream)


def _row_vector(b, h, n, dev):
    return torch.empty((b, h, n), dtype=torch.float32, device=dev)


def _check_state(name, t, shape, dev):
    if (t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
            or t.device != dev):
        raise LardError(1, f"{name} must be a contiguous fp32 {tuple(shape)} tensor on the "
                           "inputs' device, as the forward returned it")


def _check_grad_loss(grad_loss, dev):
    if (grad_loss.dtype != torch.float32 or grad_loss.numel() != 1 or grad_loss.device != dev):
        raise LardError(1, "grad_loss must be a one-element fp32 tensor on the inputs' device")
    return grad_loss.contiguous()


def _require_gpu(x: torch.Tensor):
    if x.device.type != "cuda":
        raise RuntimeError("the relation-KL library runs on a ROCm GPU only; got a tensor on "
                           f"{x.device}")


def workspace_size(x_t, x_s, *, causal=True, scale=None, head_map=None, pass_: int = 0) -> int:
    lib = load_library()
    desc, _keep = _make_desc(x_t, x_s, causal, scale, head_map)
    st = ctypes.c_int(0)
    n = lib.lard_relkl_workspace_size(ctypes.byref(desc), pass_, ctypes.byref(st))
    _check(st.value)
    return int(n)


def _workspace(lib, desc, pass_, dev):
    st = ctypes.c_int(0)
    nbytes = lib.lard_relkl_workspace_size(ctypes.byref(desc), pass_, ctypes.byref(st))
    _check(st.value)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def relkl_fwd(x_t: torch.Tensor, x_s: torch.Tensor, *, causal: bool = True,
              scale: Optional[float] = None, head_map: Optional[Sequence[int]] = None,
              want_row_kl: bool = False, stream=None):
    """Forward: returns dict(loss: 0-d fp32, lse_t, lse_s, diag_delta: fp32 [B, H, N] -- the
    state the backward takes --, row_kl: fp32 [B, H, N] or None)."""
    lib = load_library()
    desc, keep = _make_desc(x_t, x_s, causal, scale, head_map)
    _require_gpu(x_t)
    b, n = desc.B, desc.N
    dev = x_t.device
    with torch.cuda.stream(_stream_of(dev, stream)):
        lse_t = _row_vector(b, desc.H, n, dev)
        lse_s = _row_vector(b, desc.H, n, dev)
        diag = _row_vector(b, desc.H, n, dev)
        row_kl = _row_vector(b, desc.H, n, dev) if want_row_kl else None
        loss = torch.empty((), dtype=torch.float32, device=dev)
        ws = _workspace(lib, desc, 0, dev)
        _check(lib.lard_relkl_fwd(ctypes.byref(desc), x_t.data_ptr(), x_s.data_ptr(),
                                  lse_t.data_ptr(), lse_s.data_ptr(), diag.data_ptr(),
                                  row_kl.data_ptr() if row_kl is not None else None,
                                  loss.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream_handle(dev, stream)))
    del keep
    return {"loss": loss, "lse_t": lse_t, "lse_s": lse_s, "diag_delta": diag, "row_kl": row_kl}


def relkl_fwd_noalloc(x_t: torch.Tensor, x_s: torch.Tensor, lse_t: torch.Tensor,
                      lse_s: torch.Tensor, diag_delta: Optional[torch.Tensor],
                      row_kl: Optional[torch.Tensor], loss: torch.Tensor, *,
                      causal: bool = True, scale: Optional[float] = None,
                      head_map: Optional[Sequence[int]] = None, stream=None):
    """The forward into caller-given outputs (fp32 [B, H, N] row vectors, a 0-d fp32 loss)
    with no allocation by the library or by this binding: the loss partials live in the
    library's per-GPU scratch.  Calls that overlap on one GPU race on that scratch."""
    lib = load_library()
    desc, keep = _make_desc(x_t, x_s, causal, scale, head_map)
    _require_gpu(x_t)
    dev = x_t.device
    shape = (desc.B, desc.H, desc.N)
    for name, t in (("lse_t", lse_t), ("lse_s", lse_s), ("diag_delta", diag_delta),
                    ("row_kl", row_kl)):
        if t is not None:
            _check_state(name, t, shape, dev)
    if loss.dtype != torch.float32 or loss.numel() != 1 or loss.device != dev:
        raise LardError(1, "loss must be a one-element fp32 tensor on the inputs' device")
    _check(lib.lard_relkl_fwd_noalloc(ctypes.byref(desc), x_t.data_ptr(), x_s.data_ptr(),
                                      lse_t.data_ptr(), lse_s.data_ptr(),
                                      diag_delta.data_ptr() if diag_delta is not None else None,
                                      row_kl.data_ptr() if row_kl is not None else None,
                                      loss.data_ptr(), _stream_handle(dev, stream)))
    del keep


def relkl_bwd(x_t: torch.Tensor, x_s: torch.Tensor, lse_t: torch.Tensor, lse_s: torch.Tensor,
              diag_delta: torch.Tensor, grad_loss: torch.Tensor, *, causal: bool = True,
              scale: Optional[float] = None, head_map: Optional[Sequence[int]] = None,
              dx: Optional[torch.Tensor] = None, dx_dtype: Optional[torch.dtype] = None,
              stream=None) -> torch.Tensor:
    """Backward: gradient of grad_loss * loss with respect to x_s (teacher is frozen), from
    the inputs and the forward's lse_t, lse_s and diag_delta.

    dx (optional) receives the result; heads outside head_map are left untouched.  A new
    dx is zero-filled when head_map selects a subset of heads.
    """
    lib = load_library()
    desc, keep = _make_desc(x_t, x_s, causal, scale, head_map)
    _require_gpu(x_t)
    dev = x_t.device
    shape = (desc.B, desc.H, desc.N)
    for name, t in (("lse_t", lse_t), ("lse_s", lse_s), ("diag_delta", diag_delta)):
        _check_state(name, t, shape, dev)
    grad_loss = _check_grad_loss(grad_loss, dev)
    with torch.cuda.stream(_stream_of(dev, stream)):
        dx, gdesc = _new_grad(x_s, head_map, desc.H_in, dx, dx_dtype)
        ws = _workspace(lib, desc, 1, dev)
        _check(lib.lard_relkl_bwd(ctypes.byref(desc), x_t.data_ptr(), x_s.data_ptr(),
                                  lse_t.data_ptr(), lse_s.data_ptr(), diag_delta.data_ptr(),
                                  grad_loss.data_ptr(), ctypes.byref(gdesc), dx.data_ptr(),
                                  ws.data_ptr(), ws.numel(), _stream_handle(dev, stream)))
    del keep
    return dx


PROBE_THREADS = 512       # LARD_PROBE_THREADS
PROBE_MFMA_PER_ITER = 24  # LARD_PROBE_MFMA_PER_ITER
PROBE_FLOPS_PER_MFMA = 2 * 32 * 32 * 16


def probe_mfma(vector_work: bool, iters: int, workgroups: int, sink: torch.Tensor, stream=None):
    """Enqueue the matrix-core throughput probe (lard_probe_mfma; measurement only).  It
    issues workgroups * 8 waves * iters * PROBE_MFMA_PER_ITER bf16 MFMAs; sink: fp32 device
    tensor of at least workgroups * PROBE_THREADS elements."""
    lib = load_library()
    _require_gpu(sink)
    if sink.dtype != torch.float32 or not sink.is_contiguous() or \
            sink.numel() < workgroups * PROBE_THREADS:
        raise ValueError("sink: contiguous fp32 tensor of workgroups * PROBE_THREADS elements")
    _check(lib.lard_probe_mfma(1 if vector_work else 0, int(iters), int(workgroups),
                               ctypes.c_void_p(sink.data_ptr()),
                               _stream_handle(sink.device, stream)))


def _mean_rows_factor(x: torch.Tensor, reduction: str) -> Optional[float]:
    if reduction == "sum":
        return None
    if reduction == "mean_rows":
        return 1.0 / x.shape[2]
    raise LardError(1, f"reduction must be 'sum' or 'mean_rows', not {reduction!r}")


class _RelationKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x_t, x_s, causal, scale, head_map, factor):
        out = relkl_fwd(x_t, x_s, causal=causal, scale=scale, head_map=head_map)
        ctx.save_for_backward(x_t, x_s, out["lse_t"], out["lse_s"], out["diag_delta"])
        ctx.causal, ctx.scale, ctx.head_map, ctx.factor = causal, scale, head_map, factor
        return out["loss"] if factor is None else out["loss"] * factor

    @staticmethod
    def backward(ctx, grad):
        x_t, x_s, lse_t, lse_s, diag = ctx.saved_tensors
        g = grad if grad.dtype == torch.float32 else grad.float()
        if ctx.factor is not None:
            g = g * ctx.factor
        dx = relkl_bwd(x_t, x_s, lse_t, lse_s, diag, g, causal=ctx.causal, scale=ctx.scale,
                       head_map=ctx.head_map)
        return None, dx, None, None, None, None


def relation_kl(x_t: torch.Tensor, x_s: torch.Tensor, *, causal: bool = True,
                scale: Optional[float] = None, head_map: Optional[Sequence[int]] = None,
                reduction: str = "sum"):
    """KL(R_teacher || R_student) summed over batch, relation heads and rows (a 0-d fp32
    tensor); reduction="mean_rows" divides by N, the pages' mean over the rows of a head
    (the gradient is scaled alike).  Differentiable with respect to x_s; the teacher is
    treated as frozen."""
    return _RelationKL.apply(x_t.detach(), x_s, causal, scale,
                             None if head_map is None else tuple(int(v) for v in head_map),
                             _mean_rows_factor(x_t, reduction))


# ------------------------------------------------------------------ RoPE-fused entry points
def _rope_desc(x: torch.Tensor, tables) -> _RopeDesc:
    """tables: (cos_t, sin_t, cos_s, sin_s), each an fp32 [N, d/2] device tensor or None."""
    n, d = x.shape[2], x.shape[3]
    ptrs = []
    for t in tables:
        if t is None:
            ptrs.append(None)
            continue
        if (t.dtype != torch.float32 or tuple(t.shape) != (n, d // 2) or not t.is_contiguous()
                or t.device != x.device):
            raise LardError(1, f"RoPE tables must be contiguous fp32 [{n}, {d // 2}] tensors "
                               "on the inputs' device")
        ptrs.append(t.data_ptr())
    return _RopeDesc(*ptrs)


def rope_reserve_size(x_t, x_s, *, causal=True, scale=None, head_map=None) -> int:
    lib = load_library()
    desc, _keep = _make_desc(x_t, x_s, causal, scale, head_map)
    st = ctypes.c_int(0)
    n = lib.lard_relkl_rope_reserve_size(ctypes.byref(desc), ctypes.byref(st))
    _check(st.value)
    return int(n)


def _reserve(nbytes, dev):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def _check_reserve(reserve, dev, what):
    if reserve.dtype != torch.uint8 or not reserve.is_contiguous() or reserve.device != dev:
        raise LardError(1, f"reserve must be the uint8 device buffer returned by {what}")


def rope_relkl_fwd(x_t: torch.Tensor, x_s: torch.Tensor, cos_t=None, sin_t=None, cos_s=None,
                   sin_s=None, *, causal: bool = True, scale: Optional[float] = None,
                   head_map: Optional[Sequence[int]] = None, want_row_kl: bool = False,
                   stream=None):
    """RoPE-fused forward on pre-rotation inputs; returns the dict of relkl_fwd plus
    "reserve" (the rotated rows, which rope_relkl_bwd reads)."""
    lib = load_library()
    desc, keep = _make_desc(x_t, x_s, causal, scale, head_map)
    rdesc = _rope_desc(x_t, (cos_t, sin_t, cos_s, sin_s))
    _require_gpu(x_t)
    b, n = desc.B, desc.N
    dev = x_t.device
    st = ctypes.c_int(0)
    rs_bytes = lib.lard_relkl_rope_reserve_size(ctypes.byref(desc), ctypes.byref(st))
    _check(st.value)
    with torch.cuda.stream(_stream_of(dev, stream)):
        lse_t = _row_vector(b, desc.H, n, dev)
        lse_s = _row_vector(b, desc.H, n, dev)
        diag = _row_vector(b, desc.H, n, dev)
        row_kl = _row_vector(b, desc.H, n, dev) if want_row_kl else None
        loss = torch.empty((), dtype=torch.float32, device=dev)
        ws = _workspace(lib, desc, 0, dev)
        reserve = _reserve(rs_bytes, dev)
        _check(lib.lard_relkl_rope_fwd(ctypes.byref(desc), ctypes.byref(rdesc), x_t.data_ptr(),
                                       x_s.data_ptr(), lse_t.data_ptr(), lse_s.data_ptr(),
                                       diag.data_ptr(),
                                       row_kl.data_ptr() if row_kl is not None else None,
                                       loss.data_ptr(), reserve.data_ptr(), reserve.numel(),
                                       ws.data_ptr(), ws.numel(), _stream_handle(dev, stream)))
    del keep
    return {"loss": loss, "lse_t": lse_t, "lse_s": lse_s, "diag_delta": diag, "row_kl": row_kl,
            "reserve": reserve}


def rope_relkl_bwd(x_s: torch.Tensor, reserve: torch.Tensor, lse_t: torch.Tensor,
                   lse_s: torch.Tensor, diag_delta: torch.Tensor, grad_loss: torch.Tensor,
                   cos_t=None, sin_t=None, cos_s=None, sin_s=None, *, causal: bool = True,
                   scale: Optional[float] = None, head_map: Optional[Sequence[int]] = None,
                   dx: Optional[torch.Tensor] = None, dx_dtype: Optional[torch.dtype] = None,
                   stream=None) -> torch.Tensor:
    """RoPE-fused backward: gradient of grad_loss * loss with respect to the student's
    pre-rotation input x_s (x_s gives the shape, dtype and device; its values are not
    read: the rotated operands come from the reserve)."""
    lib = load_library()
    desc, keep = _make_desc(x_s, x_s, causal, scale, head_map)
    rdesc = _rope_desc(x_s, (cos_t, sin_t, cos_s, sin_s))
    _require_gpu(x_s)
    dev = x_s.device
    _check_reserve(reserve, dev, "rope_relkl_fwd")
    shape = (desc.B, desc.H, desc.N)
    for name, t in (("lse_t", lse_t), ("lse_s", lse_s), ("diag_delta", diag_delta)):
        _check_state(name, t, shape, dev)
    grad_loss = _check_grad_loss(grad_loss, dev)
    with torch.cuda.stream(_stream_of(dev, stream)):
        dx, gdesc = _new_grad(x_s, head_map, desc.H_in, dx, dx_dtype)
        ws = _workspace(lib, desc, 1, dev)
        _check(lib.lard_relkl_rope_bwd(ctypes.byref(desc), ctypes.byref(rdesc),
                                       reserve.data_ptr(), reserve.numel(), lse_t.data_ptr(),
                                       lse_s.data_ptr(), diag_delta.data_ptr(),
                                       grad_loss.data_ptr(), ctypes.byref(gdesc),
                                       dx.data_ptr(), ws.data_ptr(), ws.numel(),
                                       _stream_handle(dev, stream)))
    del keep
    return dx


class _RopeRelationKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x_t, x_s, cos_t, sin_t, cos_s, sin_s, causal, scale, head_map):
        out = rope_relkl_fwd(x_t, x_s, cos_t, sin_t, cos_s, sin_s, causal=causal, scale=scale,
                             head_map=head_map)
        ctx.save_for_backward(x_s, out["reserve"], out["lse_t"], out["lse_s"],
                              out["diag_delta"])
        ctx.tables = (cos_t, sin_t, cos_s, sin_s)
        ctx.causal, ctx.scale, ctx.head_map = causal, scale, head_map
        return out["loss"]

    @staticmethod
    def backward(ctx, grad):
        x_s, reserve, lse_t, lse_s, diag = ctx.saved_tensors
        g = grad if grad.dtype == torch.float32 else grad.float()
        dx = rope_relkl_bwd(x_s, reserve, lse_t, lse_s, diag, g, *ctx.tables,
                            causal=ctx.causal, scale=ctx.scale, head_map=ctx.head_map)
        return None, dx, None, None, None, None, None, None, None


def rope_relation_kl(x_t: torch.Tensor, x_s: torch.Tensor, cos_t=None, sin_t=None, cos_s=None,
                     sin_s=None, *, causal: bool = True, scale: Optional[float] = None,
                     head_map: Optional[Sequence[int]] = None):
    """relation_kl with each side's rotate-half RoPE applied inside the operation: x_t and
    x_s are the activations before the rotation, the tables fp32 [N, d/2] cos / sin per
    token (None: that side is not rotated).  Differentiable with respect to x_s."""
    return _RopeRelationKL.apply(x_t.detach(), x_s, cos_t, sin_t, cos_s, sin_s, causal, scale,
                                 None if head_map is None else tuple(int(v) for v in head_map))


# ------------------------------------------------------------------ cross-relation entry points
def _cross_desc(a_t, a_s, b_t, b_s) -> _CrossDesc:
    if b_t.shape != a_t.shape or b_s.shape != a_s.shape:
        raise LardError(1, "A and B must have the same shape [B, H, N, d]")
    if b_t.dtype != a_t.dtype or b_s.dtype != a_s.dtype:
        raise LardError(1, "A and B must have the same dtype")
    if b_t.stride(-1) != 1 or b_s.stride(-1) != 1:
        raise LardError(1, "the last dimension (d) of B must be contiguous")
    if b_t.device != a_t.device or b_s.device != a_t.device:
        raise LardError(1, "all inputs must be on the same device")
    return _CrossDesc(bt_stride_b=b_t.stride(0), bt_stride_h=b_t.stride(1),
                      bt_stride_n=b_t.stride(2), bs_stride_b=b_s.stride(0),
                      bs_stride_h=b_s.stride(1), bs_stride_n=b_s.stride(2))


def _rope_ptr(x, tables):
    if tables is None or all(t is None for t in tables):
        return None
    return ctypes.byref(_rope_desc(x, tables))


def cross_reserve_size(a_t, a_s, *, causal=True, scale=None, head_map=None) -> int:
    lib = load_library()
    desc, _keep = _make_desc(a_t, a_s, causal, scale, head_map)
    st = ctypes.c_int(0)
    n = lib.lard_relkl_cross_reserve_size(ctypes.byref(desc), ctypes.byref(st))
    _check(st.value)
    return int(n)


def cross_relkl_fwd(a_t: torch.Tensor, b_t: torch.Tensor, a_s: torch.Tensor, b_s: torch.Tensor,
                    *, rope=None, causal: bool = True, scale: Optional[float] = None,
                    head_map: Optional[Sequence[int]] = None, want_row_kl: bool = False,
                    stream=None):
    """Forward of the cross relation softmax(scale A B^T) per side (A: queries, B: keys);
    rope: None or (cos_t, sin_t, cos_s, sin_s) rotating each side's A and B.  Returns
    dict(loss, lse_t, lse_s, row_kl, reserve); the reserve and the LSE vectors are what
    cross_relkl_bwd needs."""
    lib = load_library()
    desc, keep = _make_desc(a_t, a_s, causal, scale, head_map)
    kdesc = _cross_desc(a_t, a_s, b_t, b_s)
    rptr = _rope_ptr(a_t, rope)
    _require_gpu(a_t)
    b, n = desc.B, desc.N
    dev = a_t.device
    st = ctypes.c_int(0)
    rs_bytes = lib.lard_relkl_cross_reserve_size(ctypes.byref(desc), ctypes.byref(st))
    _check(st.value)
    with torch.cuda.stream(_stream_of(dev, stream)):
        lse_t = _row_vector(b, desc.H, n, dev)
        lse_s = _row_vector(b, desc.H, n, dev)
        row_kl = _row_vector(b, desc.H, n, dev) if want_row_kl else None
        loss = torch.empty((), dtype=torch.float32, device=dev)
        ws = _workspace(lib, desc, 0, dev)
        reserve = _reserve(rs_bytes, dev)
        _check(lib.lard_relkl_cross_fwd(ctypes.byref(desc), ctypes.byref(kdesc), rptr,
                                        a_t.data_ptr(), b_t.data_ptr(), a_s.data_ptr(),
                                        b_s.data_ptr(), lse_t.data_ptr(), lse_s.data_ptr(),
                                        row_kl.data_ptr() if row_kl is not None else None,
                                        loss.data_ptr(), reserve.data_ptr(), reserve.numel(),
                                        ws.data_ptr(), ws.numel(), _stream_handle(dev, stream)))
    del keep
    return {"loss": loss, "lse_t": lse_t, "lse_s": lse_s, "row_kl": row_kl, "reserve": reserve}


def _new_grad(x, head_map, n_in, dx, dx_dtype):
    if dx is None:
        out_dtype = x.dtype if dx_dtype is None else dx_dtype
        subset = head_map is not None and sorted(int(v) for v in head_map) != list(range(n_in))
        dx = (torch.zeros if subset else torch.empty)(x.shape, dtype=out_dtype, device=x.device)
    if dx.shape != x.shape or dx.stride(-1) != 1 or dx.device != x.device:
        raise LardError(1, "gradients must match their input in shape, with a contiguous last "
                           "dimension")
    return dx, _GradDesc(dtype=_dtype_code(dx.dtype), reserved=0, stride_b=dx.stride(0),
                         stride_h=dx.stride(1), stride_n=dx.stride(2))


def cross_relkl_bwd(a_s: torch.Tensor, b_s: torch.Tensor, reserve: torch.Tensor,
                    lse_t: torch.Tensor, lse_s: torch.Tensor, grad_loss: torch.Tensor, *,
                    rope=None, causal: bool = True, scale: Optional[float] = None,
                    head_map: Optional[Sequence[int]] = None, da: Optional[torch.Tensor] = None,
                    db: Optional[torch.Tensor] = None, dx_dtype: Optional[torch.dtype] = None,
                    stream=None):
    """(dA_s, dB_s) of grad_loss * loss; a_s / b_s give shapes, dtypes and the device (their
    values are not read: the operands come from the reserve)."""
    lib = load_library()
    desc, keep = _make_desc(a_s, a_s, causal, scale, head_map)
    rptr = _rope_ptr(a_s, rope)
    _require_gpu(a_s)
    dev = a_s.device
    _check_reserve(reserve, dev, "cross_relkl_fwd")
    shape = (desc.B, desc.H, desc.N)
    for name, t in (("lse_t", lse_t), ("lse_s", lse_s)):
        _check_state(name, t, shape, dev)
    grad_loss = _check_grad_loss(grad_loss, dev)
    with torch.cuda.stream(_stream_of(dev, stream)):
        da, gda = _new_grad(a_s, head_map, desc.H_in, da, dx_dtype)
        db, gdb = _new_grad(b_s, head_map, desc.H_in, db, dx_dtype)
        ws = _workspace(lib, desc, 1, dev)
        _check(lib.lard_relkl_cross_bwd(ctypes.byref(desc), rptr, reserve.data_ptr(),
                                        reserve.numel(), lse_t.data_ptr(), lse_s.data_ptr(),
                                        grad_loss.data_ptr(), ctypes.byref(gda), da.data_ptr(),
                                        ctypes.byref(gdb), db.data_ptr(), ws.data_ptr(),
                                        ws.numel(), _stream_handle(dev, stream)))
    del keep
    return da, db


class _CrossRelationKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a_t, b_t, a_s, b_s, rope, causal, scale, head_map):
        out = cross_relkl_fwd(a_t, b_t, a_s, b_s, rope=rope, causal=causal, scale=scale,
                              head_map=head_map)
        ctx.save_for_backward(a_s, b_s, out["reserve"], out["lse_t"], out["lse_s"])
        ctx.rope, ctx.causal, ctx.scale, ctx.head_map = rope, causal, scale, head_map
        return out["loss"]

    @staticmethod
    def backward(ctx, grad):
        a_s, b_s, reserve, lse_t, lse_s = ctx.saved_tensors
        g = grad if grad.dtype == torch.float32 else grad.float()
        da, db = cross_relkl_bwd(a_s, b_s, reserve, lse_t, lse_s, g, rope=ctx.rope,
                                 causal=ctx.causal, scale=ctx.scale, head_map=ctx.head_map)
        return None, None, da, db, None, None, None, None


def cross_relation_kl(a_t: torch.Tensor, b_t: torch.Tensor, a_s: torch.Tensor,
                      b_s: torch.Tensor, *, rope=None, causal: bool = True,
                      scale: Optional[float] = None, head_map: Optional[Sequence[int]] = None):
    """Sum over rows of KL(softmax(scale A_t B_t^T) || softmax(scale A_s B_s^T)) (e.g. the
    attention maps of queries A and keys B), differentiable with respect to a_s and b_s.
    rope: None or (cos_t, sin_t, cos_s, sin_s) applied to each side's A and B inside the
    call."""
    return _CrossRelationKL.apply(a_t.detach(), b_t.detach(), a_s, b_s,
                                  None if rope is None else tuple(rope), causal, scale,
                                  None if head_map is None else tuple(int(v) for v in head_map))


# ------------------------------------------------------------------ grouped entry points
def _group(pairs, causal, scale, head_maps, rope):
    """ctypes members for [(x_t, x_s), ...]; head_maps and rope: None or one entry per member
    (rope entries: None -- not rotated -- or (cos_t, sin_t, cos_s, sin_s))."""
    pairs = [tuple(p) for p in pairs]
    n = len(pairs)
    if n < 1:
        raise LardError(1, "a group needs at least one member")
    if n > LARD_MAX_GROUP:
        raise LardError(2, f"a group holds at most {LARD_MAX_GROUP} members")
    if head_maps is not None and len(head_maps) != n:
        raise LardError(1, "head_maps needs one entry per member")
    if rope is not None and len(rope) != n:
        raise LardError(1, "rope needs one entry per member")
    scales = list(scale) if isinstance(scale, (list, tuple)) else [scale] * n
    if len(scales) != n:
        raise LardError(1, "scale needs one value, or one per member")
    members = (_Member * n)()
    keep = []
    for k, (x_t, x_s) in enumerate(pairs):
        desc, kk = _make_desc(x_t, x_s, causal, scales[k],
                              None if head_maps is None else head_maps[k])
        keep.extend(kk)
        members[k].desc = desc
        members[k].x_teacher = x_t.data_ptr()
        members[k].x_student = x_s.data_ptr()
        if rope is not None and rope[k] is not None:
            members[k].rope = _rope_desc(x_t, rope[k])
    return members, keep, (0 if rope is None else 1)


def group_reserve_size(pairs, *, causal=True, scale=None, head_maps=None, rope=None) -> int:
    lib = load_library()
    members, _keep, with_rope = _group(pairs, causal, scale, head_maps, rope)
    st = ctypes.c_int(0)
    n = lib.lard_relkl_group_reserve_size(len(members), members, with_rope, ctypes.byref(st))
    _check(st.value)
    return int(n)


def group_workspace_size(pairs, *, causal=True, scale=None, head_maps=None, pass_: int = 0) -> int:
    lib = load_library()
    members, _keep, _ = _group(pairs, causal, scale, head_maps, None)
    st = ctypes.c_int(0)
    n = lib.lard_relkl_group_workspace_size(len(members), members, pass_, ctypes.byref(st))
    _check(st.value)
    return int(n)


def group_relkl_fwd(pairs, *, causal: bool = True, scale: Optional[float] = None,
                    head_maps=None, rope=None, want_row_kl: bool = False, stream=None):
    """Forward of up to LARD_MAX_GROUP relation problems in one launch per kernel.

    pairs: [(x_t, x_s), ...] with a shared dtype and d (B, H, N may differ); head_maps:
    None or one head map (or None) per member; rope: None (post-rotation inputs) or one
    entry per member, None or (cos_t, sin_t, cos_s, sin_s), rotating inside the call.
    Returns dict(loss: 0-d fp32 sum over the members, member_loss: list of 0-d fp32,
    lse_t, lse_s, diag_delta, row_kl: lists per member, reserve: the rotated rows, or None
    without rope).  scale: None (1/sqrt(d)), one value for every member, or one per
    member."""
    lib = load_library()
    members, keep, with_rope = _group(pairs, causal, scale, head_maps, rope)
    _require_gpu(pairs[0][0])
    dev = pairs[0][0].device
    n = len(members)
    sizes = [m.desc.B * m.desc.H * m.desc.N for m in members]
    per = 4 if want_row_kl else 3
    st = ctypes.c_int(0)
    ws_bytes = lib.lard_relkl_group_workspace_size(n, members, 0, ctypes.byref(st))
    _check(st.value)
    rs_bytes = lib.lard_relkl_group_reserve_size(n, members, with_rope, ctypes.byref(st))
    _check(st.value)
    out = {"lse_t": [], "lse_s": [], "diag_delta": [], "row_kl": [], "member_loss": []}
    with torch.cuda.stream(_stream_of(dev, stream)):
        # one allocation for all members' row vectors and losses; views per member
        flat = torch.empty(per * sum(sizes) + n, dtype=torch.float32, device=dev)
        loss = torch.empty((), dtype=torch.float32, device=dev)
        off = 0
        for k, m in enumerate(members):
            shape = (m.desc.B, m.desc.H, m.desc.N)
            views = []
            for _ in range(per):
                views.append(flat[off:off + sizes[k]].view(shape))
                off += sizes[k]
            lt, ls, dg = views[0], views[1], views[2]
            kl = views[3] if want_row_kl else None
            m.lse_teacher, m.lse_student = lt.data_ptr(), ls.data_ptr()
            m.diag_delta = dg.data_ptr()
            m.row_kl = kl.data_ptr() if kl is not None else None
            out["lse_t"].append(lt)
            out["lse_s"].append(ls)
            out["diag_delta"].append(dg)
            out["row_kl"].append(kl)
        for k, m in enumerate(members):
            ml = flat[off + k]
            m.loss = ml.data_ptr()
            out["member_loss"].append(ml)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        reserve = _reserve(rs_bytes, dev) if with_rope else None
        _check(lib.lard_relkl_group_fwd(n, members, with_rope, loss.data_ptr(),
                                        reserve.data_ptr() if reserve is not None else None,
                                        reserve.numel() if reserve is not None else 0,
                                        ws.data_ptr(), ws.numel(),
                                        _stream_handle(dev, stream)))
    del keep
    out["loss"] = loss
    out["reserve"] = reserve
    return out


def group_relkl_bwd(pairs, lse_t, lse_s, diag_delta, grad_loss: torch.Tensor, *,
                    reserve: Optional[torch.Tensor] = None, causal: bool = True,
                    scale: Optional[float] = None, head_maps=None, rope=None, dx=None,
                    dx_dtype: Optional[torch.dtype] = None, stream=None):
    """Gradients of grad_loss * (group loss) with respect to every member's x_s (a list).
    lse_t, lse_s, diag_delta: the per-member lists group_relkl_fwd returned; reserve: its
    reserve (with rope); the other arguments as given to group_relkl_fwd.  dx (optional):
    one output tensor per member."""
    lib = load_library()
    members, keep, with_rope = _group(pairs, causal, scale, head_maps, rope)
    _require_gpu(pairs[0][0])
    dev = pairs[0][0].device
    if with_rope:
        if reserve is None:
            raise LardError(1, "a RoPE-fused group backward needs the forward's reserve")
        _check_reserve(reserve, dev, "group_relkl_fwd")
    grad_loss = _check_grad_loss(grad_loss, dev)
    n = len(members)
    if len(lse_t) != n or len(lse_s) != n or len(diag_delta) != n:
        raise LardError(1, "lse_t, lse_s and diag_delta need one tensor per member")
    if dx is not None and len(dx) != n:
        raise LardError(1, "dx needs one tensor per member")
    for k, m in enumerate(members):
        shape = (m.desc.B, m.desc.H, m.desc.N)
        for name, t in (("lse_t", lse_t[k]), ("lse_s", lse_s[k]), ("diag_delta", diag_delta[k])):
            _check_state(name, t, shape, dev)
        m.lse_teacher, m.lse_student = lse_t[k].data_ptr(), lse_s[k].data_ptr()
        m.diag_delta = diag_delta[k].data_ptr()
    st = ctypes.c_int(0)
    ws_bytes = lib.lard_relkl_group_workspace_size(n, members, 1, ctypes.byref(st))
    _check(st.value)
    outs = []
    gdescs = (_GradDesc * n)()
    ptrs = (ctypes.c_void_p * n)()
    with torch.cuda.stream(_stream_of(dev, stream)):
        for k, (_, x_s) in enumerate(pairs):
            hm = None if head_maps is None else head_maps[k]
            g, gd = _new_grad(x_s, hm, members[k].desc.H_in, None if dx is None else dx[k],
                              dx_dtype)
            outs.append(g)
            gdescs[k] = gd
            ptrs[k] = g.data_ptr()
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        _check(lib.lard_relkl_group_bwd(n, members, with_rope,
                                        reserve.data_ptr() if with_rope else None,
                                        reserve.numel() if with_rope else 0,
                                        grad_loss.data_ptr(), gdescs, ptrs, ws.data_ptr(),
                                        ws.numel(), _stream_handle(dev, stream)))
    del keep
    return outs


class _GroupRelationKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, causal, scale, head_maps, rope, *xs):
        pairs = [(xs[2 * k], xs[2 * k + 1]) for k in range(len(xs) // 2)]
        out = group_relkl_fwd(pairs, causal=causal, scale=scale, head_maps=head_maps, rope=rope)
        n = len(pairs)
        saved = list(xs) + out["lse_t"] + out["lse_s"] + out["diag_delta"]
        if out["reserve"] is not None:
            saved.append(out["reserve"])
        ctx.save_for_backward(*saved)
        ctx.n = n
        ctx.causal, ctx.scale, ctx.head_maps, ctx.rope = causal, scale, head_maps, rope
        return out["loss"]

    @staticmethod
    def backward(ctx, grad):
        saved = ctx.saved_tensors
        n = ctx.n
        xs = saved[:2 * n]
        lse_t, lse_s = list(saved[2 * n:3 * n]), list(saved[3 * n:4 * n])
        diag = list(saved[4 * n:5 * n])
        reserve = saved[5 * n] if len(saved) > 5 * n else None
        pairs = [(xs[2 * k], xs[2 * k + 1]) for k in range(n)]
        g = grad if grad.dtype == torch.float32 else grad.float()
        dxs = group_relkl_bwd(pairs, lse_t, lse_s, diag, g, reserve=reserve, causal=ctx.causal,
                              scale=ctx.scale, head_maps=ctx.head_maps, rope=ctx.rope)
        grads = [None, None, None, None]
        for dx in dxs:
            grads.extend([None, dx])
        return tuple(grads)


def group_relation_kl(pairs, *, causal: bool = True, scale: Optional[float] = None,
                      head_maps=None, rope=None):
    """Sum of relation_kl over up to LARD_MAX_GROUP members [(x_t, x_s), ...] -- e.g. the
    Q/Q, K/K and V/V relations of one layer, with GQA head counts -- computed by one launch
    per kernel.  head_maps / rope: None or one entry per member (see group_relkl_fwd).
    Differentiable with respect to every x_s."""
    hm = None if head_maps is None else tuple(None if h is None else tuple(int(v) for v in h)
                                              for h in head_maps)
    if isinstance(scale, list):
        scale = tuple(scale)
    rp = None if rope is None else tuple(None if r is None else tuple(r) for r in rope)
    flat = []
    for x_t, x_s in pairs:
        flat.extend([x_t.detach(), x_s])
    return _GroupRelationKL.apply(causal, scale, hm, rp, *flat)
