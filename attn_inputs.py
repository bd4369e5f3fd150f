"""Seeded synthetic inputs for the attention backward workloads.

This module only draws random numbers and names the workload shapes. It holds
none of the attention arithmetic, so both the CPU oracle (``oracle/``) and the
HIP path's tests and benchmark can draw identical inputs from it without
sharing any of the method's code.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws Q, K, V
and dO in that order, each ``torch.randn(B, H, S, D)`` in float32 (standard
normal), and each is rounded to bfloat16 (round-to-nearest-even) for the
bf16 path. The float32 draws are kept for the oracle-only rounding study.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    """One attention-backward workload: shape, mask and seed."""

    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    seed: int
    tile: int = 0  # 0 = let the library choose the KV/Q tile edge
    note: str = ""
    Hkv: int = 0   # K/V heads when query heads share them (0: one per query head)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Backward FLOP convention: 2.5 x 4*B*H*S^2*D, halved for causal."""
        f = 2.5 * 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2.0 if self.causal else f

    def describe(self) -> str:
        mask = "causal" if self.causal else "full"
        kv = f",Hkv={self.Hkv}" if self.Hkv and self.Hkv != self.H else ""
        return f"B={self.B},H={self.H}{kv},S={self.S},D={self.D},{mask}"


# The pages give no shapes; these stand in for their workloads (head shapes of
# the 7-8B-class models and of a long-sequence full-mask case).
WORKLOADS = {
    "C1": Workload("C1", 1, 2, 256, 64, False, 1, tile=64,
                   note="small full-mask correctness case, 64x64 tiles"),
    "C2": Workload("C2", 4, 16, 2048, 128, False, 2),
    "C3": Workload("C3", 4, 32, 4096, 128, True, 3, note="8B-LLM head shape, causal"),
    "C3F": Workload("C3F", 4, 32, 4096, 128, False, 3, note="C3's shape with a full mask"),
    "C4": Workload("C4", 2, 16, 8192, 64, True, 4),
    "C5": Workload("C5", 1, 16, 16384, 128, False, 5, note="long-sequence full mask"),
    "C3G": Workload("C3G", 4, 32, 4096, 128, True, 3, Hkv=8,
                    note="C3 with 8 shared K/V heads (grouped-query attention of 8B-class models)"),
}


def draw(B: int, H: int, S: int, D: int, seed: int):
    """Draw Q, K, V, dO (float32, standard normal) from one seeded generator.

    Returns a dict with float32 tensors ``q32, k32, v32, do32`` and their
    bfloat16 roundings ``q, k, v, do`` (all CPU, contiguous [B, H, S, D]).
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = {}
    for name in ("q", "k", "v", "do"):
        t = torch.randn(B, H, S, D, generator=g, dtype=torch.float32)
        out[name + "32"] = t
        out[name] = t.to(torch.bfloat16)
    return out


def draw_grouped(B: int, H: int, Hkv: int, S: int, D: int, seed: int):
    """Like draw, with K and V over Hkv heads (query heads sharing K/V heads).

    Q and dO are [B, H, S, D], K and V [B, Hkv, S, D]; same dict keys as draw.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = {}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv), ("do", H)):
        t = torch.randn(B, heads, S, D, generator=g, dtype=torch.float32)
        out[name + "32"] = t
        out[name] = t.to(torch.bfloat16)
    return out


def draw_workload(w: Workload):
    if w.kv_heads != w.H:
        return draw_grouped(w.B, w.H, w.kv_heads, w.S, w.D, w.seed)
    return draw(w.B, w.H, w.S, w.D, w.seed)


def to_f64(t: torch.Tensor):
    """Exact lift of a CPU tensor (bf16/fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
