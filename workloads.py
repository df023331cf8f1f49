"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and names shapes; it holds none of the
attention arithmetic, so both the fp64 oracle's tests and the GPU path's
tests and benchmark can take their inputs from it.

Recipe (the pages give no dataset and no seeds; these are choices of this
implementation): one ``torch.Generator('cpu')`` per workload, seeded as
listed below; draws in the order q, k, v, then (for a masked workload) the
mask bias and the drop decisions.  Each tensor is drawn as fp32 standard
normal, multiplied by the workload's factor, then rounded to bf16/fp16.  The
shapes mirror the pages' own examples: iid ``randn`` tensors in the SDPA
layout [B, H, N, D] (ffpa-attn README, "Quick Start" example with B=1, H=32,
N=8192, D=512).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import torch

SWEEP_D = (64, 128, 256, 320, 384, 448, 512, 640, 768, 1024)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: torch.dtype = torch.bfloat16
    seed: int = 0
    factor: float = 1.0          # multiplies the N(0,1) draws before rounding
    causal: bool = False
    mask: Optional[str] = None   # None or "add_f32_drop10"

    @property
    def flops(self) -> float:
        """4*B*Hq*Nq*Nkv*D, halved for causal (the metric's FLOP count)."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.D
        return f / 2 if self.causal else f

    def describe(self) -> dict:
        d = dict(workload=self.name, B=self.B, Hq=self.Hq, Hkv=self.Hkv, Nq=self.Nq, Nkv=self.Nkv, D=self.D,
                 dtype=str(self.dtype).replace("torch.", ""), causal=self.causal, mask=self.mask or "none",
                 seed=self.seed)
        if self.factor != 1.0:
            d["input_factor"] = self.factor
        return d


def tiny() -> Workload:
    return Workload("tiny_B1_H1_N256_D320", 1, 1, 1, 256, 256, 320, seed=1)


def large_d_self() -> Workload:
    return Workload("self_B1_H8_N4096_D512", 1, 8, 8, 4096, 4096, 512, seed=2)


def gqa_causal() -> Workload:
    return Workload("gqa_causal_B2_Hq32_Hkv8_N8192_D512", 2, 32, 8, 8192, 8192, 512, seed=3, factor=0.5, causal=True)


def cross_mask() -> Workload:
    return Workload("cross_mask_B4_H16_Nq1024_Nkv4096_D1024", 4, 16, 16, 1024, 4096, 1024, seed=4,
                    mask="add_f32_drop10")


def sweep(D: int, dtype: torch.dtype = torch.bfloat16) -> Workload:
    idx = SWEEP_D.index(D)
    seed = 100 + idx + (1000 if dtype == torch.float16 else 0)
    tag = "bf16" if dtype == torch.bfloat16 else "fp16"
    return Workload(f"sweep_B1_H16_N8192_D{D}_{tag}", 1, 16, 16, 8192, 8192, D, dtype=dtype, seed=seed)


def all_workloads() -> List[Workload]:
    ws = [tiny(), large_d_self(), gqa_causal(), cross_mask()]
    for dt in (torch.bfloat16, torch.float16):
        ws += [sweep(D, dt) for D in SWEEP_D]
    return ws


def scaled(w: Workload, **changes) -> Workload:
    """The same recipe at other sizes (for oracle-sized parity cases)."""
    return dataclasses.replace(w, **changes)


def make_inputs(w: Workload) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Host tensors q [B,Hq,Nq,D], k/v [B,Hkv,Nkv,D] and the optional mask, drawn by the recipe."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)

    def draw(*shape):
        x = torch.randn(*shape, generator=g, dtype=torch.float32)
        if w.factor != 1.0:
            x.mul_(w.factor)
        return x.to(w.dtype)

    q = draw(w.B, w.Hq, w.Nq, w.D)
    k = draw(w.B, w.Hkv, w.Nkv, w.D)
    v = draw(w.B, w.Hkv, w.Nkv, w.D)
    mask = None
    if w.mask == "add_f32_drop10":
        mask = additive_mask(g, w.B, w.Nq, w.Nkv, drop=0.10)
    elif w.mask is not None:
        raise ValueError(f"unknown mask recipe {w.mask}")
    return q, k, v, mask


def additive_mask(g: torch.Generator, B: int, Nq: int, Nkv: int, drop: float = 0.10) -> torch.Tensor:
    """fp32 [B, 1, Nq, Nkv]: N(0,1) bias, a `drop` fraction set to -inf, >= 1 finite key per row."""
    bias = torch.randn(B, 1, Nq, Nkv, generator=g, dtype=torch.float32)
    dropped = torch.rand(B, 1, Nq, Nkv, generator=g) < drop
    dead = dropped.all(dim=-1)
    if bool(dead.any()):
        keep = torch.randint(0, Nkv, dead.shape, generator=g)
        rows = dead.nonzero(as_tuple=False)
        for b, h, r in rows.tolist():
            dropped[b, h, r, keep[b, h, r]] = False
    bias[dropped] = float("-inf")
    return bias


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch (ffpa-attn "API Reference", ffpa_attn_varlen_func): sequence b has lens_q[b]
    query tokens and lens_k[b] key tokens; tensors [T, H, D]."""
    name: str
    lens_q: Tuple[int, ...]
    lens_k: Tuple[int, ...]
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype = torch.bfloat16
    seed: int = 0
    causal: bool = False

    @property
    def flops(self) -> float:
        """Sum over sequences of 4*Hq*Nq_b*Nkv_b*D, halved for causal (the metric's convention)."""
        f = sum(4.0 * self.Hq * nq * nk * self.D for nq, nk in zip(self.lens_q, self.lens_k))
        return f / 2 if self.causal else f

    def describe(self) -> dict:
        return dict(workload=self.name, B=len(self.lens_q), Hq=self.Hq, Hkv=self.Hkv, Tq=sum(self.lens_q),
                    Tk=sum(self.lens_k), max_seqlen_q=max(self.lens_q), max_seqlen_k=max(self.lens_k), D=self.D,
                    dtype=str(self.dtype).replace("torch.", ""), causal=self.causal, seed=self.seed,
                    lens_q=list(self.lens_q))


def varlen_causal() -> VarlenWorkload:
    """Packed causal self-attention (a prefill batch): 8 sequences, lengths drawn uniformly from
    256..8192 with seed 6, Hq = Hkv = 16, D = 512, bf16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(6)
    lens = tuple(int(x) for x in torch.randint(256, 8193, (8,), generator=g).tolist())
    return VarlenWorkload("varlen_causal_B8_H16_D512", lens, lens, 16, 16, 512, seed=6, causal=True)


def make_varlen_inputs(w: VarlenWorkload):
    """Host tensors q [Tq, Hq, D], k/v [Tk, Hkv, D] (drawn by the recipe above, in the order q, k, v)
    and the int32 offsets cu_q, cu_k [B+1]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 1)

    def draw(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32).to(w.dtype)

    Tq, Tk = sum(w.lens_q), sum(w.lens_k)
    q = draw(Tq, w.Hq, w.D)
    k = draw(Tk, w.Hkv, w.D)
    v = draw(Tk, w.Hkv, w.D)
    cu_q = torch.tensor([0] + list(torch.tensor(w.lens_q).cumsum(0).tolist()), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(torch.tensor(w.lens_k).cumsum(0).tolist()), dtype=torch.int32)
    return q, k, v, cu_q, cu_k


def sample_tokens(lens: Tuple[int, ...], seed: int, bucket: int = 64) -> List[int]:
    """Packed query tokens to compare at full size: per sequence, one seeded token per `bucket`-token
    bucket plus its first, second and last tokens."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7907)
    out, base = [], 0
    for n in lens:
        picked = {r for r in (0, 1, n - 1) if 0 <= r < n}
        nb = (n + bucket - 1) // bucket
        for i, o in enumerate(torch.randint(0, bucket, (nb,), generator=g).tolist()):
            if i * bucket + o < n:
                picked.add(i * bucket + o)
        out.extend(base + r for r in sorted(picked))
        base += n
    return out


def random_qkv(B: int, Hq: int, Hkv: int, Nq: int, Nkv: int, D: int, dtype=torch.bfloat16, seed: int = 0,
               factor: float = 1.0):
    """Small ad-hoc cases for tests, same recipe."""
    w = Workload("adhoc", B, Hq, Hkv, Nq, Nkv, D, dtype=dtype, seed=seed, factor=factor)
    q, k, v, _ = make_inputs(w)
    return q, k, v


def sample_rows(B: int, Hq: int, Nq: int, seed: int, bucket: int = 64) -> List[int]:
    """Flat row indices to compare at full size: per (b, h), one seeded row per `bucket`-row bucket
    plus the boundary rows 0, 1, 63, 64, 127, 128 and Nq-1 (those that exist)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7919)
    fixed = sorted({r for r in (0, 1, 63, 64, 127, 128, Nq - 1) if 0 <= r < Nq})
    out = []
    nb = (Nq + bucket - 1) // bucket
    for bh in range(B * Hq):
        offs = torch.randint(0, bucket, (nb,), generator=g).tolist()
        rows = set(fixed)
        for i, o in enumerate(offs):
            r = i * bucket + o
            if r < Nq:
                rows.add(r)
        out.extend(bh * Nq + r for r in sorted(rows))
    return out
