"""Phase-1 context encoding through a stack of Llama-3 attention layers.

Each layer is out = x + Attn(rope(RMSNorm(x) Wqkv^T)) Wo^T, with Phase-1
attention (anchor block + own block, causal).  On one device every token's
q/k/v is computed once per layer and the anchor's K/V are block 1's rows of
that layer: the anchor is causal and first in every augmented block, so its
hidden states equal host 1's at every layer (Pith review of Star Attention,
"What carries the argument").

Layout: the fused projection output qkv [B*L, (Hq + 2 Hkv) * D] is read by
RoPE and by the flash kernel as strided [B, H, L, D] views, and the flash
kernel writes the attention output straight into the [B*L, Hq * D] input of
the output projection: no transposes.  The projections run in rocBLAS
(star_linear), RMSNorm, RoPE and the attention in this library's kernels.
"""
from __future__ import annotations

import math

import torch

from . import (Context, linear, phase1_blocklocal, phase1_rope, rmsnorm, rope_apply,
               sched_workspace)


class AttentionLayers:
    """Weights (device, bf16) and buffers of a stack of attention layers.

    ``layers`` is a list of dicts with ``gamma`` [H], ``wq`` [Hq*D, H],
    ``wk``/``wv`` [Hkv*D, H] and ``wo`` [H, Hq*D] device tensors, H = Hq*D.
    """

    def __init__(self, B, Hq, Hkv, D, L, b, layers, anchor=None, rope=True,
                 base=500000.0, eps=1e-5, device="cuda"):
        self.B, self.Hq, self.Hkv, self.D, self.L, self.b = B, Hq, Hkv, D, L, b
        self.a = b if anchor is None else anchor
        self.rope, self.base, self.eps = rope, base, eps
        self.scale = 1.0 / math.sqrt(D)
        H = Hq * D
        self.H, self.N = H, (Hq + 2 * Hkv) * D
        self.ctx = Context()
        self.w = []
        for w in layers:
            wqkv = torch.cat([w["wq"], w["wk"], w["wv"]], dim=0).contiguous()
            self.w.append((w["gamma"].contiguous(), wqkv, w["wo"].contiguous()))
        bf = torch.bfloat16
        dev = torch.device(device)
        M = B * L
        self.h = torch.empty((M, H), dtype=bf, device=dev)
        self.qkv = torch.empty((M, self.N), dtype=bf, device=dev)
        self.attn = torch.empty((M, Hq * D), dtype=bf, device=dev)
        self.xs = [torch.empty((M, H), dtype=bf, device=dev) for _ in range(2)]
        self.sched = sched_workspace(dev)   # Phase-1 work queues (one stream)

    def heads(self, t, first, n):
        """[B, n, L, D] view of heads first..first+n-1 of a [B*L, cols] buffer."""
        B, L, D = self.B, self.L, self.D
        cols = t.shape[1]
        return t.view(B, L, cols)[:, :, first * D:(first + n) * D].view(B, L, n, D).transpose(1, 2)

    def forward(self, x, mark=None):
        """x [B, L, H] bf16 -> the stack's output [B, L, H] (a view of an
        internal buffer, valid until the next call).  ``mark(name)``, if
        given, is called after each stage is enqueued (for event timing)."""
        B, L, H = x.shape
        mark = mark or (lambda name: None)
        cur = x.reshape(B * L, H)
        for i, (gamma, wqkv, wo) in enumerate(self.w):
            rmsnorm(cur, gamma, self.eps, out=self.h)
            mark("rmsnorm")
            linear(self.ctx, self.h, wqkv, out=self.qkv)
            mark("qkv_proj")
            q = self.heads(self.qkv, 0, self.Hq)
            k = self.heads(self.qkv, self.Hq, self.Hkv)
            v = self.heads(self.qkv, self.Hq + self.Hkv, self.Hkv)
            # Phase 1 rotates q itself (bf16, D = 128): only k gets its own pass
            fused = self.rope and self.D == 128
            if self.rope:
                if not fused:
                    rope_apply(q, pos0=0, base=self.base)
                rope_apply(k, pos0=0, base=self.base)
            mark("rope")
            if fused:
                phase1_rope(q, k, v, self.b, self.a, self.base, self.scale,
                            out=self.heads(self.attn, 0, self.Hq), sched=self.sched)
            else:
                phase1_blocklocal(q, k, v, self.b, self.a, self.scale,
                                  out=self.heads(self.attn, 0, self.Hq), sched=self.sched)
            mark("phase1")
            nxt = self.xs[i % 2]
            linear(self.ctx, self.attn, wo, residual=cur, out=nxt)
            mark("o_proj")
            cur = nxt
        return cur.view(B, L, H)

    def gemm_flops(self) -> float:
        """Projection FLOPs of one layer (2 M K N for q/k/v and output)."""
        M = self.B * self.L
        return 2.0 * M * self.H * self.N + 2.0 * M * self.Hq * self.D * self.H
