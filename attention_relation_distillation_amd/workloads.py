"""Seeded synthetic workloads for the relation-KL path (input generation only).

This module holds none of the loss arithmetic: it only draws the teacher and student
relation inputs (Q, K, V after RoPE) that both the HIP library and the float64 oracle
consume, so both sides see identical bytes.

The shapes follow the models the LinearARD pages name (LLaMA2-7B: 32 heads of d = 128,
4K -> 32K with position interpolation 8x; Llama-3-8B: 32 query / 8 KV heads, RoPE base
500000).  No weights or text are available, so the activations are N(0, 1) draws:
* the teacher's Q and K carry native RoPE (positions 0..N-1);
* the student's Q and K carry the scaled RoPE of the workload (positions / factor for
  position interpolation, or a larger base for the NTK-style variant);
* V has no RoPE; the student's V is the teacher's V plus 0.05 * N(0, 1).
RoPE uses the rotate-half pairing (k, k + d/2) with theta_k = base^(-2k/d); angles and
rotation are computed in float64 and then rounded to the workload dtype.

Draw order with one CPU ``torch.Generator`` seeded once, float32 ``randn``:
x_q, x_k, x_v, noise_v (the tiny workload: x, noise).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["Workload", "Relation", "RopeRelation", "WORKLOADS", "make_inputs",
           "make_rope_inputs", "rope", "rope_tables", "default_scale"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str                      # "fp32" | "bf16"
    masks: tuple                    # tuple of bool (causal flags that are run)
    relations: tuple                # subset of ("qq", "kk", "vv")
    teacher_rope: Optional[tuple]   # (base, position divisor) or None
    student_rope: Optional[tuple]
    noise: float                    # std of the student perturbation (V, or the tiny X)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


@dataclasses.dataclass
class Relation:
    name: str            # "qq" | "kk" | "vv"
    x_t: torch.Tensor    # [B, H_in, N, d]
    x_s: torch.Tensor
    head_map: Optional[list] = None


@dataclasses.dataclass
class RopeRelation:
    """Inputs of the RoPE-fused call: activations before the rotation and the fp32
    [N, d/2] cos / sin tables of each side (None: that side is not rotated)."""
    name: str
    x_t: torch.Tensor    # [B, H_in, N, d], before RoPE
    x_s: torch.Tensor
    cos_t: Optional[torch.Tensor] = None
    sin_t: Optional[torch.Tensor] = None
    cos_s: Optional[torch.Tensor] = None
    sin_s: Optional[torch.Tensor] = None


WORKLOADS = {
    # Q/Q only, fp32, student = teacher + 0.1 N(0,1), no RoPE.
    "tiny": Workload("tiny", 1, 1, 1, 256, 64, "fp32", (True,), ("qq",), None, None, 0.1),
    # LLaMA2-7B-shaped layer at 4K, student RoPE = position interpolation 8x.
    "llama2_4k": Workload("llama2_4k", 1, 32, 32, 4096, 128, "bf16", (True,),
                          ("qq", "kk", "vv"), (10000.0, 1.0), (10000.0, 8.0), 0.05),
    # Same recipe at 32K (the linear-memory stress case).
    "llama2_32k": Workload("llama2_32k", 1, 32, 32, 32768, 128, "bf16", (True,),
                           ("qq", "kk", "vv"), (10000.0, 1.0), (10000.0, 8.0), 0.05),
    # Batched 8K, causal and non-causal, student RoPE = NTK-style base 80000.
    "batched_8k": Workload("batched_8k", 8, 32, 32, 8192, 128, "bf16", (True, False),
                           ("qq", "kk", "vv"), (10000.0, 1.0), (80000.0, 1.0), 0.05),
    # Llama-3-8B-like GQA: 32 query heads, 8 KV heads, base 500000, student PI 4x.
    "gqa_16k": Workload("gqa_16k", 1, 32, 8, 16384, 128, "bf16", (True,),
                        ("qq", "kk", "vv"), (500000.0, 1.0), (500000.0, 4.0), 0.05),
}


def default_scale(d: int) -> float:
    """float32 rounding of 1/sqrt(d), as a Python float."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def rope_tables(n: int, d: int, base: float, pos_div: float, dtype=torch.float32):
    """Cosine and sine tables [n, d/2] of the RoPE recipe: token p at position p / pos_div,
    frequency k at base^(-2k/d); angles and cos/sin in float64, then cast to ``dtype``."""
    k = torch.arange(d // 2, dtype=torch.float64)
    inv_freq = base ** (-2.0 * k / d)
    pos = torch.arange(n, dtype=torch.float64) / pos_div
    ang = pos[:, None] * inv_freq[None, :]
    return torch.cos(ang).to(dtype), torch.sin(ang).to(dtype)


def rope(x: torch.Tensor, base: float, pos_div: float) -> torch.Tensor:
    """Rotate-half RoPE in float64 at positions arange(N) / pos_div; returns float64."""
    n, d = x.shape[-2], x.shape[-1]
    half = d // 2
    cos, sin = rope_tables(n, d, base, pos_div, dtype=torch.float64)
    x64 = x.to(torch.float64)
    x1, x2 = x64[..., :half], x64[..., half:]
    return torch.cat((x1 * cos - x2 * sin, x2 * cos + x1 * sin), dim=-1)


def make_inputs(wl: Workload | str, seed: int = 0, *, B: Optional[int] = None,
                Hq: Optional[int] = None, Hkv: Optional[int] = None,
                N: Optional[int] = None, relations: Optional[tuple] = None):
    """Draw the workload's relations (CPU tensors in the workload dtype).

    B / Hq / Hkv / N override the shape (same recipe at another size, for tests).
    Returns a list of Relation in the order of ``wl.relations`` (or ``relations``).
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    b = wl.B if B is None else B
    hq = wl.Hq if Hq is None else Hq
    hkv = wl.Hkv if Hkv is None else Hkv
    n = wl.N if N is None else N
    d = wl.d
    dt = wl.torch_dtype
    rels = wl.relations if relations is None else relations
    gen = torch.Generator().manual_seed(seed)

    def draw(h):
        return torch.randn((b, h, n, d), generator=gen, dtype=torch.float32)

    out = []
    if wl.teacher_rope is None:
        x = draw(hq)
        noise = draw(hq)
        x_t = x.to(dt)
        x_s = (x.to(torch.float64) + wl.noise * noise.to(torch.float64)).to(dt)
        out.append(Relation("qq", x_t.contiguous(), x_s.contiguous()))
        return [r for r in out if r.name in rels]

    x_q, x_k, x_v, noise_v = draw(hq), draw(hkv), draw(hkv), draw(hkv)
    tb, tdiv = wl.teacher_rope
    sb, sdiv = wl.student_rope
    for name in rels:
        if name == "qq":
            x_t = rope(x_q, tb, tdiv).to(dt)
            x_s = rope(x_q, sb, sdiv).to(dt)
        elif name == "kk":
            x_t = rope(x_k, tb, tdiv).to(dt)
            x_s = rope(x_k, sb, sdiv).to(dt)
        elif name == "vv":
            x_t = x_v.to(dt)
            x_s = (x_v.to(torch.float64) + wl.noise * noise_v.to(torch.float64)).to(dt)
        else:
            raise ValueError(f"unknown relation {name!r}")
        out.append(Relation(name, x_t.contiguous(), x_s.contiguous()))
    return out


def make_rope_inputs(wl: Workload | str, seed: int = 0, *, B: Optional[int] = None,
                     Hq: Optional[int] = None, Hkv: Optional[int] = None,
                     N: Optional[int] = None, relations: Optional[tuple] = None):
    """The same draws as ``make_inputs``, handed over before the rotation: Q/K relations
    carry the teacher's and the student's RoPE tables (fp32), V and the tiny workload none.
    The teacher's and student's Q (and K) are the same pre-RoPE activations."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    b = wl.B if B is None else B
    hq = wl.Hq if Hq is None else Hq
    hkv = wl.Hkv if Hkv is None else Hkv
    n = wl.N if N is None else N
    d = wl.d
    dt = wl.torch_dtype
    rels = wl.relations if relations is None else relations
    gen = torch.Generator().manual_seed(seed)

    def draw(h):
        return torch.randn((b, h, n, d), generator=gen, dtype=torch.float32)

    if wl.teacher_rope is None:
        x = draw(hq)
        noise = draw(hq)
        x_t = x.to(dt)
        x_s = (x.to(torch.float64) + wl.noise * noise.to(torch.float64)).to(dt)
        return [r for r in [RopeRelation("qq", x_t.contiguous(), x_s.contiguous())]
                if r.name in rels]

    x_q, x_k, x_v, noise_v = draw(hq), draw(hkv), draw(hkv), draw(hkv)
    ct, st = rope_tables(n, d, *wl.teacher_rope)
    cs, ss = rope_tables(n, d, *wl.student_rope)
    out = []
    for name in rels:
        if name in ("qq", "kk"):
            x = (x_q if name == "qq" else x_k).to(dt).contiguous()
            out.append(RopeRelation(name, x, x, ct, st, cs, ss))
        elif name == "vv":
            x_t = x_v.to(dt)
            x_s = (x_v.to(torch.float64) + wl.noise * noise_v.to(torch.float64)).to(dt)
            out.append(RopeRelation(name, x_t.contiguous(), x_s.contiguous()))
        else:
            raise ValueError(f"unknown relation {name!r}")
    return out
