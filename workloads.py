"""Seeded synthetic inputs for routed block-sparse attention.

This module only draws random tensors; it holds none of the attention
method's arithmetic (no pooling, scoring, selection or softmax).  Both the
CPU oracle tests and the GPU path are fed from the same tensors made here.

Shapes follow the packed video-DiT layout described on the page
"Sol-Attn and Spark for MiniMax-H3" (Install: contiguous BF16
[batch, tokens, heads, 128]; H3 pipeline integration: the target video grid
comes first in raster (frame, height, width) order and conditioning tokens are
packed after it as exact K/V sinks).

Recipes (the pages give no data; these stand in for H3-shaped activations):

* ``tiny``:   X = 0.6 * u_X[block, head] + 0.8 * N(0,1) per token, with an
  independent per-(block, head) N(0,1) vector u_X for each of Q, K, V.
* ``video``:  for each (batch, head, channel) a low-resolution N(0,1) field on
  a (ceil(F/2), 8, 8) grid is upsampled trilinearly (align_corners=False) to
  (F, 32, 32).  Q and K of video tokens are 0.5 * field + N(0,1), the field
  shared by Q and K, the noise independent.  Context (sink) tokens get
  Q, K ~ N(0,1).  V ~ N(0,1) everywhere.
* key_bias:   float32 [B, T]: 0 on video keys, U(-2, 0) on context keys.

All values are drawn in float32 from ``torch.Generator().manual_seed(seed)``
and rounded once to bfloat16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch
import torch.nn.functional as F

HEAD_DIM = 128


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor            # bf16 [B, T, H, 128], CPU
    k: torch.Tensor
    v: torch.Tensor
    sink_start: int            # number of video tokens (first in packed order)
    topk_ratio: float
    local_radius: int
    key_bias: Optional[torch.Tensor] = None   # float32 [B, T] natural log, CPU
    tail_mode: str = "dense"   # video tail mode: "dense" or "pad"

    @property
    def shape(self):
        B, T, H, D = self.q.shape
        return B, T, H, D


def tiny_qkv(B=1, H=2, T=1024, seed=0, block=64):
    """Block-clustered tokens: 0.6 * shared per-block vector + 0.8 * noise."""
    g = torch.Generator().manual_seed(seed)
    nb = -(-T // block)
    out = []
    for _ in range(3):
        u = torch.randn(B, nb, H, HEAD_DIM, generator=g)
        u_tok = u.repeat_interleave(block, dim=1)[:, :T]
        x = 0.6 * u_tok + 0.8 * torch.randn(B, T, H, HEAD_DIM, generator=g)
        out.append(x.to(torch.bfloat16).contiguous())
    return tuple(out)


def video_qkv(B, H, frames, ctx_tokens, seed, height=32, width=32):
    """Smooth-field + noise Q/K over a (frames, height, width) raster grid,
    followed by ``ctx_tokens`` context tokens; V ~ N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    tv = frames * height * width
    T = tv + ctx_tokens
    low = (max(1, math.ceil(frames / 2)), max(1, height // 4), max(1, width // 4))
    field = torch.randn(B * H * HEAD_DIM, 1, *low, generator=g)
    field = F.interpolate(field, size=(frames, height, width), mode="trilinear",
                          align_corners=False)
    # [B, H, D, F, Y, X] -> [B, F*Y*X, H, D] (raster order t = f*Y*X + y*X + x)
    field = field.reshape(B, H, HEAD_DIM, tv).permute(0, 3, 1, 2)
    q = torch.empty(B, T, H, HEAD_DIM)
    k = torch.empty(B, T, H, HEAD_DIM)
    q[:, :tv] = 0.5 * field + torch.randn(B, tv, H, HEAD_DIM, generator=g)
    k[:, :tv] = 0.5 * field + torch.randn(B, tv, H, HEAD_DIM, generator=g)
    if ctx_tokens:
        q[:, tv:] = torch.randn(B, ctx_tokens, H, HEAD_DIM, generator=g)
        k[:, tv:] = torch.randn(B, ctx_tokens, H, HEAD_DIM, generator=g)
    v = torch.randn(B, T, H, HEAD_DIM, generator=g)
    to = lambda x: x.to(torch.bfloat16).contiguous()
    return to(q), to(k), to(v), tv


def sink_key_bias(B, T, sink_start, seed):
    """Natural-log per-key bias: 0 on video keys, U(-2, 0) on context keys."""
    g = torch.Generator().manual_seed(seed)
    bias = torch.zeros(B, T, dtype=torch.float32)
    n = T - sink_start
    if n > 0:
        bias[:, sink_start:] = -2.0 * torch.rand(B, n, generator=g)
    return bias.contiguous()


def random_qkv(B, T, H, seed, scale=1.0):
    """Plain i.i.d. N(0, scale^2) Q/K/V (edge-case tests)."""
    g = torch.Generator().manual_seed(seed)
    mk = lambda: (scale * torch.randn(B, T, H, HEAD_DIM, generator=g)).to(torch.bfloat16).contiguous()
    return mk(), mk(), mk()


# ---------------------------------------------------------------------------
# Named workloads (sizes of the H3-shaped pipeline and its neighbours)
# ---------------------------------------------------------------------------

def tiny():
    q, k, v = tiny_qkv(B=1, H=2, T=1024, seed=0)
    return Workload("tiny_B1_H2_T1024", q, k, v, sink_start=1024,
                    topk_ratio=0.25, local_radius=0)


def mid():
    q, k, v, tv = video_qkv(B=1, H=8, frames=8, ctx_tokens=256, seed=1)
    return Workload("mid_B1_H8_T8448", q, k, v, sink_start=tv,
                    topk_ratio=0.1, local_radius=1)


def h3(with_bias=False):
    q, k, v, tv = video_qkv(B=1, H=56, frames=9, ctx_tokens=289, seed=2)
    bias = sink_key_bias(1, q.shape[1], tv, seed=3) if with_bias else None
    name = "h3_B1_H56_T9505" + ("_keybias" if with_bias else "")
    return Workload(name, q, k, v, sink_start=tv, topk_ratio=0.1,
                    local_radius=0, key_bias=bias)


def long():
    q, k, v, tv = video_qkv(B=1, H=24, frames=32, ctx_tokens=512, seed=4)
    return Workload("long_B1_H24_T33280", q, k, v, sink_start=tv,
                    topk_ratio=0.1, local_radius=1)


def max_blocks():
    """The widest routing the library accepts: 1024 video blocks (64 frames
    of 32 x 32 tokens) and 200 context tokens, two heads, ratio 0.1 with
    radius 1 and key_bias.  Lists hold 103 + 3 + 4 = 110 entries, so the
    attention kernel walks them in two 64-entry chunks."""
    q, k, v, tv = video_qkv(B=1, H=2, frames=64, ctx_tokens=200, seed=30)
    bias = sink_key_bias(1, q.shape[1], tv, seed=31)
    return Workload("maxblocks_B1_H2_T65736_keybias", q, k, v, sink_start=tv, topk_ratio=0.1,
                    local_radius=1, key_bias=bias)


def h3_heads(H, seed=2, with_bias=False):
    """H3 sequence shape (9 x 32 x 32 video + 289 context) with fewer heads."""
    q, k, v, tv = video_qkv(B=1, H=H, frames=9, ctx_tokens=289, seed=seed)
    bias = sink_key_bias(1, q.shape[1], tv, seed=3) if with_bias else None
    return Workload(f"h3_B1_H{H}_T9505", q, k, v, sink_start=tv, topk_ratio=0.1,
                    local_radius=0, key_bias=bias)


def h3_share():
    """One GPU's share of the H3 call split by head over eight GPUs: the H3
    sequence shape and recipe with 7 heads (56 / 8)."""
    w = h3_heads(7)
    return Workload("h3_share_B1_H7_T9505", w.q, w.k, w.v, sink_start=w.sink_start,
                    topk_ratio=w.topk_ratio, local_radius=w.local_radius)


NAMED = {"tiny": tiny, "mid": mid, "h3": h3,
         "h3_bias": lambda: h3(with_bias=True), "long": long, "max_blocks": max_blocks,
         "h3_share": h3_share}
