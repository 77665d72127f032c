"""Plain CPU oracle: mean-pooled Top-K block-routed sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed, and where the pages define it
-----------------------------------------------
Tensors are packed ``[B, T, H, 128]`` (page "Sol-Attn and Spark for
MiniMax-H3", section Install).  Tokens ``[0, sink_start)`` are the target
video grid, tokens ``[sink_start, T)`` are conditioning tokens packed after it
as exact K/V sinks (same page, "H3 pipeline integration" and "Direct
Sol-Attn": ``sink_start=video_tokens``).  Blocks are 64 tokens (same page,
"Spark primitives": 64-token leaves, ``T // 64`` blocks).

1. ``pool_means``     - one mean vector per complete 64-token video block, for
   Q and K ("native mean" Top-K routing, "Spark inference integration"; the
   producers' pooled K sums are taken from the unweighted activations,
   page "Add key bias to chunked Sol-Attn producers", Summary).
2. ``route_scores``   - pooled query-block x key-block scores, computed once
   outside attention ("packed route ... avoids recomputing route QK",
   "Spark inference integration"), in FP32 (its boundary selection is an
   exact FP32 selection, same section, last paragraph).
3. ``topk_budget`` / ``select_row`` - fixed-ratio Top-K (ratio 0.1 by
   default) among the routed candidates; forced self/neighbour blocks are added
   outside the budget ("H3 pipeline integration", fixed Top-K routing
   paragraph); sink blocks go straight into the exact list and are excluded
   from the routed candidates (PR page, "Tests and source audit").
4. ``block_lists``    - the exact list of each query block.
5. ``attend``         - softmax attention of a set of query rows over a set of
   keys, with the per-key natural-log ``key_bias`` added to the logits of sink
   keys only (PR page, Summary and Contract: the bias is consumed by the
   exact branch only, biased key blocks must be sink-routed).
6. ``routed_attention`` - sparse rows ``[0, 64*NVB)`` over their exact lists,
   dense rows ``[64*NVB, T)`` (context query rows and a video tail block split
   by the video boundary) over all keys ("H3 pipeline integration": context
   query rows and the mixed final block are computed densely with the
   complete K/V).
7. Video tail modes (same page, "H3 pipeline integration", the paragraph on
   the video tail mode, and "Spark inference integration", last paragraph).
   ``"dense"`` is item 6.  ``"pad"`` also routes the video block split by the
   boundary (block NVB, real video rows ``[64*NVB, sink_start)``): its other
   query slots are filled with the mean Q of its real rows (``pad_query_block``),
   so its routing centroid is that mean; it is routed and attended like a
   complete video block and only its real rows are kept.  Context rows
   ``[sink_start, T)`` stay dense; K/V are the unmodified full sequence for
   both paths.  The context suffix must fill the rest of that block
   (``T >= 64*(NVB+1)``).

Readings taken where the pages are silent (each also listed in the design
notes): budget ``k = max(1, ceil(ratio*NVB - 1e-6))`` clamped to the number of
candidates; forced blocks are excluded from the candidates; neighbours are
block index +-r clipped to the video blocks; ties go to the lower block index;
every block holding a token >= 64*NVB is a sink block; softmax scale
``1/sqrt(128)``; scores are unscaled (a positive scale cannot reorder them).
In pad mode the key side does not change: candidates are still the NVB
complete video blocks (budget over NVB), block NVB stays a sink block, and
the padded block's forced neighbours are the video blocks within the radius
below it.

Precision: pooled means are the float64 quotient of the exact float64 block
sum (sums of bf16 inputs are exact there) by the number of rows, rounded to
fp32; for a complete block the division by 64 is exact, so that is the
correctly rounded mean.  Route scores are fp32 values of a float64 dot
product of those fp32 means; attention runs in float64 throughout.

Parity pins (tests/test_oracle_pins.py): every function above is pinned by a
brute-force, closed-form or library check that does not reuse its code.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 64
HEAD_DIM = 128
NEAR_TIE_REL = 1e-5

TAIL_MODES = ("dense", "pad")

__all__ = [
    "BLOCK", "HEAD_DIM", "NEAR_TIE_REL", "TAIL_MODES", "block_counts",
    "query_blocks", "sparse_rows_end", "topk_budget", "forced_blocks",
    "max_selected", "pool_means", "pad_query_block", "route_scores",
    "select_row", "RowSelection", "list_accepted", "Route", "route", "attend", "key_bias_vector",
    "sparse_block_output", "dense_rows_output", "routed_attention",
    "effective_flops",
]


# ---------------------------------------------------------------------------
# Shapes
# ---------------------------------------------------------------------------

def block_counts(T: int, sink_start: int) -> Tuple[int, int]:
    """(NB, NVB): all 64-token blocks (the last may be partial) and complete
    video blocks.  A block that holds any token >= 64*NVB is a sink block."""
    if not (0 <= sink_start <= T):
        raise ValueError("sink_start must lie in [0, T]")
    nb = -(-T // BLOCK)
    nvb = sink_start // BLOCK
    return nb, nvb


def query_blocks(T: int, sink_start: int, tail_mode: str = "dense") -> int:
    """NVQ, the routed query blocks: NVB, plus the block split by the video
    boundary in pad mode.  Pad mode needs the context suffix to complete that
    block (``T >= 64*(NVB+1)``), else ValueError."""
    if tail_mode not in TAIL_MODES:
        raise ValueError("tail_mode must be 'dense' or 'pad'")
    _, nvb = block_counts(T, sink_start)
    if tail_mode == "dense" or sink_start % BLOCK == 0:
        return nvb
    if T < (nvb + 1) * BLOCK:
        raise ValueError("pad mode needs the context suffix to complete the split video block")
    return nvb + 1


def sparse_rows_end(T: int, sink_start: int, tail_mode: str = "dense") -> int:
    """Query rows [0, end) take the sparse path, rows [end, T) the dense one."""
    nvq = query_blocks(T, sink_start, tail_mode)
    _, nvb = block_counts(T, sink_start)
    return sink_start if nvq > nvb else nvb * BLOCK


def topk_budget(nvb: int, ratio: float) -> int:
    """Fixed-ratio budget before clamping to the candidate count.

    ``ratio`` is the fp32 value the caller passes; the product is formed in
    double.  The 1e-6 guard keeps products such as 0.1*30 from rounding up.
    """
    r = float(np.float32(ratio))
    if not (0.0 < r <= 1.0):
        raise ValueError("topk ratio must lie in (0, 1]")
    if nvb <= 0:
        return 0
    return max(1, int(math.ceil(r * nvb - 1e-6)))


def forced_blocks(i: int, nvb: int, radius: int) -> List[int]:
    """Blocks forced exact for query block i: radius 0 -> the block itself,
    radius 1 -> itself and its two immediate neighbours, clipped to the video
    blocks."""
    return [j for j in range(i - radius, i + radius + 1) if 0 <= j < nvb]


def max_selected(T: int, sink_start: int, ratio: float, radius: int,
                 tail_mode: str = "dense") -> int:
    """Upper bound of any exact list's length: budget + forced + sinks."""
    nb, nvb = block_counts(T, sink_start)
    if query_blocks(T, sink_start, tail_mode) == 0:
        return 0
    return min(nvb, topk_budget(nvb, ratio) + 2 * radius + 1) + (nb - nvb)


# ---------------------------------------------------------------------------
# Step 1-2: pooling and route scores
# ---------------------------------------------------------------------------

def pool_means(x: np.ndarray, nblocks: int, end: Optional[int] = None) -> np.ndarray:
    """Mean over the video rows of each of the first ``nblocks`` blocks.

    Block i holds rows [64i, min(64i+64, end)); ``end`` defaults to
    64*nblocks (complete blocks only).  x: [B, T, H, D] holding bf16 values
    (any float dtype).  Returns fp32 [B, H, nblocks, D]: the float64 row sum
    (exact for bf16 inputs of ordinary range) divided by the row count in
    float64, rounded to fp32.
    """
    B, T, H, D = x.shape
    end = nblocks * BLOCK if end is None else end
    out = np.zeros((B, H, nblocks, D), dtype=np.float32)
    x64 = np.asarray(x, dtype=np.float64)
    for i in range(nblocks):
        r0, r1 = i * BLOCK, min(i * BLOCK + BLOCK, end)
        s = x64[:, r0:r1].sum(axis=1)                          # [B, H, D]
        out[:, :, i, :] = (s / (r1 - r0)).astype(np.float32)
    return out


def pad_query_block(q: np.ndarray, b: int, h: int, i: int, sink_start: int) -> np.ndarray:
    """The 64 query rows that pad mode runs for block i, which the video
    boundary splits: the real video rows [64i, sink_start) and, in the other
    slots, the float64 mean Q of those real rows.  float64 [64, D]."""
    r0 = i * BLOCK
    real = np.asarray(q[b, r0:sink_start, h], dtype=np.float64)
    if not (0 < len(real) < BLOCK):
        raise ValueError("block i is not split by the video boundary")
    out = np.empty((BLOCK, real.shape[1]), dtype=np.float64)
    out[:len(real)] = real
    out[len(real):] = real.mean(axis=0)
    return out


def route_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s[b,h,i,j] = qbar_i . kbar_j as fp32 (float64 dot of fp32 values,
    rounded once).  Unscaled: a positive softmax scale cannot reorder it."""
    s = np.matmul(qbar.astype(np.float64), np.swapaxes(kbar.astype(np.float64), -1, -2))
    return s.astype(np.float32)


# ---------------------------------------------------------------------------
# Step 3-4: selection
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class RowSelection:
    routed: List[int]          # R(i): the Top-K among the candidates
    forced: List[int]          # F(i)
    blocks: List[int]          # S(i) = sorted(R u F u sinks)
    near_tie: bool             # k-th and (k+1)-th scores within 1e-5 rel
    band: Tuple[float, float]  # scores inside this closed band may swap


def select_row(scores_row: np.ndarray, i: int, nvb: int, nb: int,
               budget: int, radius: int) -> RowSelection:
    """Top-K of one query block.

    Candidates are the video blocks minus the forced ones.  They are ordered
    by (score descending, block index ascending); the first
    ``min(budget, #candidates)`` are routed.  Sink blocks [nvb, nb) are always
    in the list and never candidates.
    """
    forced = forced_blocks(i, nvb, radius)
    fset = set(forced)
    cand = np.array([j for j in range(nvb) if j not in fset], dtype=np.int64)
    k = min(budget, len(cand))
    s = np.asarray(scores_row, dtype=np.float32)[cand] if len(cand) else np.zeros(0, np.float32)
    # lexsort: last key is primary.  Negating fp32 is exact; -0.0 == +0.0.
    order = np.lexsort((cand, -s.astype(np.float64))) if len(cand) else np.zeros(0, np.int64)
    routed = sorted(int(j) for j in cand[order[:k]])
    near, band = False, (math.inf, -math.inf)
    if 0 < k < len(cand):
        a = float(s[order[k - 1]])   # k-th best score
        b = float(s[order[k]])       # (k+1)-th best score
        tol = NEAR_TIE_REL * max(abs(a), abs(b))
        if abs(a - b) <= tol:
            near = True
            lo, hi = min(a, b), max(a, b)
            band = (lo - tol, hi + tol)
    blocks = sorted(set(routed) | fset | set(range(nvb, nb)))
    return RowSelection(routed, forced, blocks, near, band)


def list_accepted(got: Sequence[int], sel: RowSelection, scores_row: np.ndarray, nvb: int) -> bool:
    """Whether a block list computed elsewhere is a correct selection for
    the row that ``sel`` describes (several lists are correct only in a
    near-tie row).

    The list must equal ``sel.blocks``; in a near-tie row it may differ, but
    only by routed candidates whose scores (``scores_row``, the fp32 route
    scores of this row) lie inside ``sel.band``: same length, ascending, the
    forced and sink blocks unchanged.  This is the selection rule of
    ``select_row`` read with the k-th and (k+1)-th scores treated as equal
    (the boundary selection is an exact FP32 one, page "Sol-Attn and Spark
    for MiniMax-H3", Spark inference integration; two roundings of the same
    sum may land one ulp apart)."""
    got = [int(j) for j in got]
    if got == sel.blocks:
        return True
    if not sel.near_tie or len(got) != len(sel.blocks):
        return False
    if any(a >= b for a, b in zip(got, got[1:])):
        return False
    lo, hi = sel.band
    fixed = set(sel.forced)
    for j in set(got) ^ set(sel.blocks):
        if not (0 <= j < nvb) or j in fixed or not (lo <= float(scores_row[j]) <= hi):
            return False
    return True


@dataclasses.dataclass
class Route:
    nb: int
    nvb: int
    budget: int
    qbar: np.ndarray                     # fp32 [B, H, NVQ, D]
    kbar: np.ndarray                     # fp32 [B, H, NVB, D]
    scores: np.ndarray                   # fp32 [B, H, NVQ, NVB]
    rows: List[List[List[RowSelection]]]  # [B][H][NVQ]
    nvq: int = -1                        # routed query blocks (NVB, +1 in pad mode)
    sparse_end: int = -1                 # query rows [0, sparse_end) are sparse

    def lists(self) -> List[List[List[List[int]]]]:
        return [[[r.blocks for r in hrow] for hrow in brow] for brow in self.rows]


def route(q: np.ndarray, k: np.ndarray, sink_start: int, ratio: float,
          radius: int, tail_mode: str = "dense") -> Route:
    """Pool, score and select for every (batch, head, routed query block).

    In pad mode the query block split by the video boundary is pooled over
    its real video rows (the mean that its padded slots carry) and selects
    among the same NVB candidates as every other query block."""
    B, T, H, D = q.shape
    nb, nvb = block_counts(T, sink_start)
    nvq = query_blocks(T, sink_start, tail_mode)
    budget = topk_budget(nvb, ratio)
    qbar = pool_means(q, nvq, end=sink_start if nvq > nvb else None)
    kbar = pool_means(k, nvb)
    scores = route_scores(qbar, kbar)
    rows = [[[select_row(scores[b, h, i], i, nvb, nb, budget, radius)
              for i in range(nvq)] for h in range(H)] for b in range(B)]
    return Route(nb, nvb, budget, qbar, kbar, scores, rows, nvq,
                 sparse_rows_end(T, sink_start, tail_mode))


# ---------------------------------------------------------------------------
# Step 5-6: attention
# ---------------------------------------------------------------------------

def attend(qrows: np.ndarray, keys: np.ndarray, vals: np.ndarray,
           bias: Optional[np.ndarray], scale: float):
    """Softmax attention in float64.

    logits[t, j] = scale * (q_t . k_j) + bias_j; out_t = sum_j softmax_j * v_j.
    Returns (out [n, D], natural-log logsumexp [n]).
    """
    qf = np.asarray(qrows, dtype=np.float64)
    kf = np.asarray(keys, dtype=np.float64)
    vf = np.asarray(vals, dtype=np.float64)
    logits = (qf @ kf.T) * scale
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    denom = p.sum(axis=1, keepdims=True)
    out = (p @ vf) / denom
    lse = m[:, 0] + np.log(denom[:, 0])
    return out, lse


def key_bias_vector(key_bias: Optional[np.ndarray], b: int, T: int,
                    nvb: int) -> Optional[np.ndarray]:
    """Per-key natural-log bias of batch b as seen by the exact branch: the
    given value on sink keys (tokens >= 64*NVB), zero elsewhere."""
    if key_bias is None:
        return None
    kb = np.asarray(key_bias, dtype=np.float64).reshape(-1, T)[b].copy()
    kb[: nvb * BLOCK] = 0.0
    return kb


def _scale(scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(HEAD_DIM) if not scale else float(scale)


def sparse_block_output(q, k, v, b: int, h: int, i: int, blocks: Sequence[int],
                        key_bias=None, nvb: Optional[int] = None, scale=None,
                        qrows: Optional[np.ndarray] = None):
    """Rows [64i, 64i+64) of head h (or the given ``qrows``) over the keys
    of ``blocks`` (keys >= T do not exist)."""
    T = q.shape[1]
    if nvb is None:
        raise ValueError("nvb required")
    idx = np.concatenate([np.arange(j * BLOCK, min(j * BLOCK + BLOCK, T)) for j in blocks])
    kb = key_bias_vector(key_bias, b, T, nvb)
    bias = None if kb is None else kb[idx]
    if qrows is None:
        qrows = q[b, i * BLOCK:min(i * BLOCK + BLOCK, T), h]
    return attend(qrows, k[b, idx, h], v[b, idx, h], bias, _scale(scale))


def dense_rows_output(q, k, v, b: int, h: int, rows: np.ndarray,
                      key_bias=None, nvb: int = 0, scale=None):
    """Given query rows of head h over all T keys."""
    T = q.shape[1]
    kb = key_bias_vector(key_bias, b, T, nvb)
    return attend(q[b, rows, h], k[b, :, h], v[b, :, h], kb, _scale(scale))


def routed_attention(q, k, v, sink_start: int, ratio: float, radius: int,
                     key_bias=None, scale=None, rt: Optional[Route] = None,
                     tail_mode: str = "dense"):
    """Full forward: returns (out float64 [B,T,H,D], lse [B,H,T], Route)."""
    q = np.asarray(q)
    B, T, H, D = q.shape
    if D != HEAD_DIM:
        raise ValueError("head dim must be 128")
    if rt is None:
        rt = route(q, k, sink_start, ratio, radius, tail_mode)
    nvb = rt.nvb
    nvq = nvb if rt.nvq < 0 else rt.nvq
    end = nvb * BLOCK if rt.sparse_end < 0 else rt.sparse_end
    out = np.zeros((B, T, H, D), dtype=np.float64)
    lse = np.zeros((B, H, T), dtype=np.float64)
    dense = np.arange(end, T)
    for b in range(B):
        for h in range(H):
            for i in range(nvq):
                r0, r1 = i * BLOCK, min(i * BLOCK + BLOCK, end)
                padded = pad_query_block(q, b, h, i, end) if r1 - r0 < BLOCK else None
                o, l = sparse_block_output(q, k, v, b, h, i, rt.rows[b][h][i].blocks,
                                           key_bias, nvb, scale, qrows=padded)
                out[b, r0:r1, h] = o[:r1 - r0]
                lse[b, h, r0:r1] = l[:r1 - r0]
            if len(dense):
                o, l = dense_rows_output(q, k, v, b, h, dense, key_bias, nvb, scale)
                out[b, dense, h] = o
                lse[b, h, dense] = l
    return out, lse, rt


def effective_flops(T: int, H: int, B: int, lists: Sequence, nvb: int,
                    D: int = HEAD_DIM, sparse_end: Optional[int] = None) -> int:
    """4*D FLOPs per (query row, valid key) pair scored exactly: QK^T and PV
    each take 2*D.  ``lists`` is [B][H][NVQ] of block lists; query rows
    [0, sparse_end) (default 64*NVB) are sparse, the rest dense.  Padded
    query slots are not counted."""
    end = nvb * BLOCK if sparse_end is None else sparse_end
    nvq = -(-end // BLOCK)
    pairs = 0
    for b in range(B):
        for h in range(H):
            for i in range(nvq):
                nk = sum(min(BLOCK, T - j * BLOCK) for j in lists[b][h][i])
                pairs += min(BLOCK, end - i * BLOCK) * nk
    pairs += B * H * (T - end) * T
    return 4 * D * pairs
