"""torch.autograd wrapper and a synthetic attention block over the library.

    out = attention(q, k, v, causal=True, schedule="descending")   # differentiable
    block = AttentionBlock(hidden=4096, heads=32, kv_heads=8, head_dim=128)

The forward runs the library's attention forward (O and the log-sum-exp it
saves for the backward); the backward runs the deterministic attention
backward with the chosen schedule (or the atomic-dQ variant when
schedule=None). Both are the library's HIP kernels; this module only wires
them into autograd. q, k, v are bf16 [B, H, S, D] and [B, Hkv, S, D] CUDA
tensors (contiguous copies are taken when needed).

AttentionBlock is the attention half of a decoder layer shaped like the
8B-class models the DASH pages time end to end (hidden 4096, 32 query heads,
8 shared K/V heads, head size 128): RMS norm, Q/K/V projections, rotary
position embedding, attention, output projection and the residual add. Its
weights are random (there are no trained weights here); it exists to time
the attention backward inside the surrounding work, not to model a network.
"""

from __future__ import annotations

import math

import torch

from . import bwd, bwd_nondeterministic, fwd


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, schedule, scale):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = fwd(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.schedule, ctx.scale = causal, schedule, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        do = do.contiguous()
        if ctx.schedule is None:
            dq, dk, dv = bwd_nondeterministic(q, k, v, o, do, lse, ctx.causal, ctx.scale)
        else:
            dq, dk, dv = bwd(q, k, v, o, do, lse, ctx.causal, ctx.schedule, ctx.scale)
        return dq, dk, dv, None, None, None


def attention(q, k, v, causal: bool = True, schedule="descending", scale: float | None = None):
    """Differentiable softmax attention; schedule=None uses the atomic-dQ backward.

    The default, Descending, measured fastest on the causal shapes timed (4k
    and 8k, also with grouped K/V heads) and on the 16k full mask, and 3-6%
    behind Shift on the 2k and 4k full masks."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _Attention.apply(q, k, v, causal, schedule, float(scale))


def rotary(x, base: float = 500000.0):
    """Rotary position embedding over [B, H, S, D] (pairs (i, i + D/2) rotated by position * base^(-2i/D))."""
    S, D = x.shape[-2], x.shape[-1]
    inv = base ** (-torch.arange(0, D, 2, device=x.device, dtype=torch.float32) / D)
    ang = torch.arange(S, device=x.device, dtype=torch.float32)[:, None] * inv[None, :]
    cos, sin = ang.cos(), ang.sin()
    x1, x2 = x[..., : D // 2].float(), x[..., D // 2:].float()
    return torch.cat((x1 * cos - x2 * sin, x1 * sin + x2 * cos), dim=-1).to(x.dtype)


class AttentionBlock(torch.nn.Module):
    """x + Wo . attention(rope(Wq n(x)), rope(Wk n(x)), Wv n(x)), n = RMS norm; random bf16 weights."""

    def __init__(self, hidden=4096, heads=32, kv_heads=8, head_dim=128, causal=True, schedule="descending", seed=0,
                 device="cuda"):
        super().__init__()
        g = torch.Generator(device="cpu").manual_seed(seed)
        init = lambda o, i: torch.nn.Parameter(
            (torch.randn(o, i, generator=g) / math.sqrt(i)).to(torch.bfloat16).to(device))
        self.heads, self.kv_heads, self.head_dim = heads, kv_heads, head_dim
        self.causal, self.schedule = causal, schedule
        self.norm = torch.nn.Parameter(torch.ones(hidden, dtype=torch.bfloat16, device=device))
        self.wq = init(heads * head_dim, hidden)
        self.wk = init(kv_heads * head_dim, hidden)
        self.wv = init(kv_heads * head_dim, hidden)
        self.wo = init(hidden, heads * head_dim)

    def forward(self, x):
        B, S, _ = x.shape
        n = (x.float() * torch.rsqrt(x.float().pow(2).mean(-1, keepdim=True) + 1e-5)).to(x.dtype) * self.norm
        split = lambda t, h: t.view(B, S, h, self.head_dim).transpose(1, 2).contiguous()
        lin = torch.nn.functional.linear
        q = rotary(split(lin(n, self.wq), self.heads))
        k = rotary(split(lin(n, self.wk), self.kv_heads))
        v = split(lin(n, self.wv), self.kv_heads)
        o = attention(q, k, v, self.causal, self.schedule)
        return x + lin(o.transpose(1, 2).reshape(B, S, -1), self.wo)
