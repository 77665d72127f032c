"""Plain CPU oracle: Spark virtual summaries and the approximate branch.

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

What is computed, and where the pages define it
-----------------------------------------------
Page "Sol-Attn and Spark for MiniMax-H3":

1. ``global_anchor`` - one query representative per (batch, head): the mean
   of all target-video query rows, stored in BF16 (Spark inference
   integration: one global representative per head, formed by averaging all
   target-video queries; the default stored anchor dtype is BF16).  Spark
   averages after its reblocking permutation; a mean does not depend on the
   order of the rows, so no permutation is needed here.
2. ``virtual_summaries`` - for each anchor a and each physical 64-token K/V
   block (the last may be partial and then only its real keys count), the
   softmax weights w_s of the logits scale * a.k_s over the block's keys, the
   weighted key and value ak = sum w_s k_s, av = sum w_s v_s, and the log-mass
   correction lm = logsumexp_s(scale * a.k_s) - scale * a.ak (Spark
   primitives, the spark_reweight paragraph).  ak and av are stored in BF16,
   lm in FP32, and by default lm subtracts the stored BF16 summary key
   (Spark inference integration, the reweight ablation paragraph: log-mass
   subtraction uses the stored BF16 summary key unless "pre_round" is asked
   for).
3. ``approx_block_output`` / ``routed_attention_spark`` - the approximate
   branch merged with exact attention (Spark inference integration: global
   anchor K/V and log-mass summaries merged with exact attention, exact and
   approximate tiles in one FP32 online-softmax accumulator; the component
   ablation paragraph: a skipped block's mass is its summary's log-mass in
   place of the ordinary log(block length)).  Each video block that a query
   block's exact list leaves out becomes one virtual key: key ak_j, value
   av_j and additive logit lm_j, so its logit for query row t is
   scale * q_t.ak_j + lm_j.  Sink blocks are always exact and never
   summarised (page "Add key bias to chunked Sol-Attn producers", Tests and
   source audit: sink blocks are excluded from the pooled tail).  Context
   (dense) rows see every key exactly and no summaries.

Readings taken where the pages are silent: one anchor per (batch, head) (the
pages' default); the approximate branch uses the same softmax scale as the
summaries; the anchor mean is the float64 quotient rounded to fp32 and then
to BF16.  With lm computed from the unrounded key, a query row equal to the
anchor reproduces each skipped block's exact softmax mass and weighted value
(the identity the pins check).

Precision: float64 throughout; BF16 storage is modelled by rounding to fp32
and then to BF16, round to nearest even, as a device computing in fp32
stores it.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from oracle.sparse_attention import (BLOCK, HEAD_DIM, Route, block_counts, key_bias_vector,
                                     pad_query_block, route, attend)

__all__ = ["to_bf16", "global_anchor", "virtual_summaries", "log_mass",
           "approx_block_output", "routed_attention_spark"]


def to_bf16(x) -> np.ndarray:
    """fp64/fp32 -> fp32 -> bf16 (round to nearest even), returned as fp32."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float64).astype(np.float32))
    return t.to(torch.bfloat16).float().numpy()


def _scale(scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(HEAD_DIM) if not scale else float(scale)


def global_anchor(q: np.ndarray, sink_start: int) -> np.ndarray:
    """Mean of the video query rows [0, sink_start) per (batch, head),
    float64 sum divided by the row count, rounded to fp32, stored as bf16.
    Returns [B, 1, H, D] (fp32 holding bf16 values)."""
    if sink_start <= 0:
        raise ValueError("the anchor needs at least one video row")
    x = np.asarray(q, dtype=np.float64)[:, :sink_start]
    mean = x.sum(axis=1) / sink_start                        # [B, H, D]
    return to_bf16(mean.astype(np.float32))[:, None]


def log_mass(a: np.ndarray, keys: np.ndarray, key_for_shift: np.ndarray, scale: float) -> float:
    """logsumexp_s(scale * a.k_s) - scale * a.key_for_shift (float64)."""
    z = scale * (np.asarray(keys, np.float64) @ np.asarray(a, np.float64))
    m = z.max()
    lse = m + math.log(np.exp(z - m).sum())
    return lse - scale * float(np.dot(np.asarray(a, np.float64), np.asarray(key_for_shift, np.float64)))


def virtual_summaries(a: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None,
                      logmass_key: str = "stored", store: str = "bf16"):
    """Per anchor and physical 64-token block: (ak, av, lm).

    a: [B, P, H, D]; k, v: [B, T, H, D].  Returns ak, av [B, P, H, NB, D]
    and lm [B, P, H, NB] (float64).  ``store``: "bf16" rounds ak and av as
    they are stored (the pages' default), "f64" keeps them unrounded.
    ``logmass_key``: "stored" subtracts scale * a.ak with ak as stored,
    "pre_round" with the unrounded weighted key.
    """
    if logmass_key not in ("stored", "pre_round"):
        raise ValueError("logmass_key must be 'stored' or 'pre_round'")
    if store not in ("bf16", "f64"):
        raise ValueError("store must be 'bf16' or 'f64'")
    rnd = to_bf16 if store == "bf16" else (lambda x: np.asarray(x, np.float64))
    s = _scale(scale)
    a64 = np.asarray(a, np.float64)
    k64 = np.asarray(k, np.float64)
    v64 = np.asarray(v, np.float64)
    B, P, H, D = a64.shape
    T = k64.shape[1]
    nb = -(-T // BLOCK)
    ak = np.zeros((B, P, H, nb, D), np.float64)
    av = np.zeros((B, P, H, nb, D), np.float64)
    lm = np.zeros((B, P, H, nb), np.float64)
    for b in range(B):
        for p in range(P):
            for h in range(H):
                for j in range(nb):
                    keys = k64[b, j * BLOCK:min(T, j * BLOCK + BLOCK), h]
                    vals = v64[b, j * BLOCK:min(T, j * BLOCK + BLOCK), h]
                    z = s * (keys @ a64[b, p, h])
                    w = np.exp(z - z.max())
                    w = w / w.sum()
                    ak64 = w @ keys
                    ak[b, p, h, j] = rnd(ak64)
                    av[b, p, h, j] = rnd(w @ vals)
                    shift = ak[b, p, h, j] if logmass_key == "stored" else ak64
                    lm[b, p, h, j] = log_mass(a64[b, p, h], keys, shift, s)
    return ak, av, lm


def approx_block_output(q, k, v, b: int, h: int, i: int, blocks, ak, av, lm,
                        key_bias=None, nvb: int = 0, scale=None, qrows=None):
    """Rows of query block i (or ``qrows``) over the exact keys of
    ``blocks`` plus one virtual key per skipped video block (anchor 0)."""
    T = q.shape[1]
    idx = np.concatenate([np.arange(j * BLOCK, min(j * BLOCK + BLOCK, T)) for j in blocks])
    kb = key_bias_vector(key_bias, b, T, nvb)
    exact_bias = np.zeros(len(idx)) if kb is None else kb[idx]
    skipped = [j for j in range(nvb) if j not in set(blocks)]
    keys = np.concatenate([np.asarray(k[b, idx, h], np.float64),
                           np.asarray(ak[b, 0, h, skipped], np.float64).reshape(-1, k.shape[-1])])
    vals = np.concatenate([np.asarray(v[b, idx, h], np.float64),
                           np.asarray(av[b, 0, h, skipped], np.float64).reshape(-1, v.shape[-1])])
    bias = np.concatenate([exact_bias, np.asarray(lm[b, 0, h, skipped], np.float64)])
    if qrows is None:
        qrows = q[b, i * BLOCK:min(i * BLOCK + BLOCK, T), h]
    return attend(qrows, keys, vals, bias, _scale(scale))


def routed_attention_spark(q, k, v, sink_start: int, ratio: float, radius: int, summaries,
                           key_bias=None, scale=None, rt: Optional[Route] = None,
                           tail_mode: str = "dense"):
    """Routed attention with the approximate branch: sparse rows over their
    exact lists plus virtual keys for the skipped video blocks; dense rows
    over all keys exactly.  ``summaries`` = (ak, av, lm) with one anchor.
    Returns (out float64 [B,T,H,D], lse [B,H,T], Route)."""
    ak, av, lm = summaries
    q = np.asarray(q)
    B, T, H, D = q.shape
    if rt is None:
        rt = route(q, k, sink_start, ratio, radius, tail_mode)
    nvb = rt.nvb
    nvq = nvb if rt.nvq < 0 else rt.nvq
    end = nvb * BLOCK if rt.sparse_end < 0 else rt.sparse_end
    s = _scale(scale)
    out = np.zeros((B, T, H, D), np.float64)
    lse = np.zeros((B, H, T), np.float64)
    dense = np.arange(end, T)
    for b in range(B):
        for h in range(H):
            for i in range(nvq):
                r0, r1 = i * BLOCK, min(i * BLOCK + BLOCK, end)
                padded = pad_query_block(q, b, h, i, end) if r1 - r0 < BLOCK else None
                o, l = approx_block_output(q, k, v, b, h, i, rt.rows[b][h][i].blocks, ak, av, lm,
                                           key_bias, nvb, s, qrows=padded)
                out[b, r0:r1, h] = o[:r1 - r0]
                lse[b, h, r0:r1] = l[:r1 - r0]
            if len(dense):
                kb = key_bias_vector(key_bias, b, T, nvb)
                o, l = attend(q[b, dense, h], k[b, :, h], v[b, :, h], kb, s)
                out[b, dense, h] = o
                lse[b, h, dense] = l
    return out, lse, rt
