"""Pins of the CPU oracle against facts that do not come from the oracle.

Each ``check_*`` raises AssertionError when the oracle disagrees with:
exact rational arithmetic, brute-force enumeration, closed forms, PyTorch's
scaled_dot_product_attention (a library routine) or an independent
token-mask formulation.  The checks look the oracle's functions up on the
module at call time, so the mutation tests can swap one of them for a
plausible mistake and see a check fail.
"""
import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle.sparse_attention as ra
import oracle.spark_summaries as sp
import workloads
from _exact import exact_block_means, exact_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(x):
    return x.float().numpy()


def _sdpa(q, k, v, mask=None, scale=None):
    """Reference attention over [B, T, H, D] numpy arrays, float64, CPU."""
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64)).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=np.float64))
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m,
                                       scale=scale if scale else 1.0 / math.sqrt(q.shape[-1]))
    return o.permute(0, 2, 1, 3).numpy()


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _varied_bf16(shape, seed):
    """bf16 values spread over many binades (stresses exact summation)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g) * torch.exp2(torch.randint(-12, 4, shape, generator=g).float())
    return x.to(torch.bfloat16)


# ---------------------------------------------------------------- pooling ---

def check_pool_exact():
    x = _np(_varied_bf16((1, 256, 2, 128), seed=11))
    got = ra.pool_means(x, 4)
    want = exact_block_means(x, 4)
    assert got.dtype == np.float32 and got.shape == (1, 2, 4, 128)
    assert np.array_equal(_bits(got), _bits(want)), "pooled means are not the correctly rounded exact means"


def check_pool_permutation_invariant():
    x = _np(_varied_bf16((1, 320, 3, 128), seed=12))
    rng = np.random.default_rng(5)
    y = x.copy()
    for i in range(5):
        perm = rng.permutation(64) + 64 * i
        y[:, 64 * i:64 * i + 64] = x[:, perm]
    assert np.array_equal(_bits(ra.pool_means(x, 5)), _bits(ra.pool_means(y, 5)))


# ----------------------------------------------------------------- scores ---

def check_scores_exact():
    x = _np(_varied_bf16((1, 384, 2, 128), seed=13))
    z = _np(_varied_bf16((1, 384, 2, 128), seed=14))
    qbar = exact_block_means(x, 6)
    kbar = exact_block_means(z, 6)
    got = ra.route_scores(qbar, kbar)
    want = exact_scores(qbar, kbar)
    assert got.dtype == np.float32 and got.shape == (1, 2, 6, 6)
    assert np.array_equal(_bits(got), _bits(want)), "scores are not fp32 of the exact dot products"


# ----------------------------------------------------------------- budget ---

def check_budget():
    # closed forms of ceil(ratio * NVB) for the workloads' sizes
    f = ra.topk_budget
    assert f(16, 0.25) == 4
    assert f(128, 0.1) == 13
    assert f(144, 0.1) == 15
    assert f(512, 0.1) == 52
    assert f(30, 0.1) == 3          # 0.1*30 is 3.0000000000000004 in double
    assert f(10, 0.1) == 1
    assert f(144, 1.0) == 144
    assert f(7, 1e-4) == 1          # at least one routed block
    assert f(0, 0.1) == 0
    for bad in (0.0, -0.5, 1.5):
        try:
            f(10, bad)
        except ValueError:
            pass
        else:
            raise AssertionError("invalid ratio accepted")


# -------------------------------------------------------------- selection ---

def _brute_topk(scores, cand, k):
    """The unique k-subset whose every member beats every non-member under
    (score descending, index ascending)."""
    def beats(a, b):
        return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)
    found = []
    for sub in itertools.combinations(cand, k):
        s = set(sub)
        rest = [b for b in cand if b not in s]
        if all(beats(a, b) for a in sub for b in rest):
            found.append(sorted(sub))
    assert len(found) == 1, "brute force must find exactly one subset"
    return found[0]


def check_topk_bruteforce():
    rng = np.random.default_rng(21)
    for nvb in range(1, 9):
        for radius in (0, 1, 2):
            for ratio in (0.1, 0.3, 0.5, 1.0):
                nb = nvb + int(rng.integers(0, 3))
                budget = ra.topk_budget(nvb, ratio)
                # coarse values -> many exact ties; include signed zeros
                row_vals = rng.integers(-3, 4, size=nvb).astype(np.float32)
                row_vals[row_vals == 0] = np.where(rng.random((row_vals == 0).sum()) < 0.5, -0.0, 0.0)
                for i in range(nvb):
                    sel = ra.select_row(row_vals, i, nvb, nb, budget, radius)
                    forced = [j for j in range(nvb) if abs(j - i) <= radius]
                    cand = [j for j in range(nvb) if j not in forced]
                    k = min(budget, len(cand))
                    want = _brute_topk({j: float(row_vals[j]) for j in cand}, cand, k) if k else []
                    assert sel.routed == want, (nvb, radius, ratio, i, sel.routed, want)
                    assert sel.forced == forced
                    assert sel.blocks == sorted(set(want) | set(forced) | set(range(nvb, nb)))


def check_signed_zero_tie():
    row = np.array([5.0, -0.0, 0.0, -1.0], dtype=np.float32)
    # i=0, radius 0: candidates 1,2,3; budget 1 -> -0.0 and +0.0 tie, index 1 wins
    sel = ra.select_row(row, 0, 4, 4, 1, 0)
    assert sel.routed == [1]
    row2 = np.array([5.0, 0.0, -0.0, -1.0], dtype=np.float32)
    assert ra.select_row(row2, 0, 4, 4, 1, 0).routed == [1]


def check_near_tie_flag():
    budget = ra.topk_budget(6, 1.0 / 3.0)
    assert budget == 2
    tied = np.array([9.0, 3.0, 1.0, np.float32(1.0000001), -2.0, 0.5], dtype=np.float32)
    sel = ra.select_row(tied, 0, 6, 6, budget, 0)
    assert sel.routed == [1, 3] and sel.near_tie
    lo, hi = sel.band
    assert lo <= 1.0 <= hi and lo <= float(np.float32(1.0000001)) <= hi and hi < 1.001
    apart = np.array([9.0, 3.0, 1.0, 1.5, -2.0, 0.5], dtype=np.float32)
    sel2 = ra.select_row(apart, 0, 6, 6, budget, 0)
    assert sel2.routed == [1, 3] and not sel2.near_tie


def check_list_accepted():
    """Which lists from elsewhere count as correct: only the oracle's own list
    in an ordinary row; in a near-tie row also a list that swaps blocks whose
    scores lie inside the band, and nothing else."""
    budget = ra.topk_budget(6, 1.0 / 3.0)
    tied = np.array([9.0, 3.0, 1.0, np.float32(1.0000001), -2.0, 0.5], dtype=np.float32)
    sel = ra.select_row(tied, 0, 6, 8, budget, 0)       # blocks 6, 7 are sinks
    assert sel.blocks == [0, 1, 3, 6, 7] and sel.near_tie
    assert ra.list_accepted([0, 1, 3, 6, 7], sel, tied, 6)
    assert ra.list_accepted([0, 1, 2, 6, 7], sel, tied, 6)        # 1.0 for 1.0000001
    assert not ra.list_accepted([0, 1, 5, 6, 7], sel, tied, 6)    # 0.5 is outside the band
    assert not ra.list_accepted([0, 2, 3, 6, 7], sel, tied, 6)    # drops the clear winner 1
    assert not ra.list_accepted([1, 2, 3, 6, 7], sel, tied, 6)    # drops the forced block 0
    assert not ra.list_accepted([0, 1, 2, 3, 6, 7], sel, tied, 6)  # too long
    assert not ra.list_accepted([0, 1, 2, 6], sel, tied, 6)       # drops a sink
    assert not ra.list_accepted([0, 2, 1, 6, 7], sel, tied, 6)    # not ascending
    # the forced block 0 scores inside the band too: it still may not be swapped out
    forced_tied = tied.copy()
    forced_tied[0] = 1.0
    sel3 = ra.select_row(forced_tied, 0, 6, 8, budget, 0)
    assert sel3.blocks == [0, 1, 3, 6, 7] and sel3.near_tie
    assert not ra.list_accepted([1, 2, 3, 6, 7], sel3, forced_tied, 6)
    apart = np.array([9.0, 3.0, 1.0, 1.5, -2.0, 0.5], dtype=np.float32)
    sel2 = ra.select_row(apart, 0, 6, 8, budget, 0)
    assert ra.list_accepted(sel2.blocks, sel2, apart, 6)
    assert not ra.list_accepted([0, 1, 2, 6, 7], sel2, apart, 6)  # no leniency without a tie


def check_list_structure():
    rng = np.random.default_rng(22)
    nvb, nb = 20, 24
    for radius in (0, 1, 2):
        for ratio in (0.1, 0.25, 1.0):
            budget = ra.topk_budget(nvb, ratio)
            row = rng.standard_normal(nvb).astype(np.float32)
            for i in range(nvb):
                sel = ra.select_row(row, i, nvb, nb, budget, radius)
                S = sel.blocks
                F_ = [j for j in range(max(0, i - radius), min(nvb, i + radius + 1))]
                assert set(F_) <= set(S) and set(range(nvb, nb)) <= set(S)
                assert all(a < b for a, b in zip(S, S[1:]))
                assert not (set(sel.routed) & set(F_))
                k = min(budget, nvb - len(F_))
                assert len(S) == k + len(F_) + (nb - nvb)
                assert len(S) <= ra.max_selected(nb * 64, nvb * 64, ratio, radius)


def check_route_glue():
    """route() = pool(Q), pool(K), score(qbar, kbar), select - against the
    exact rational path and the brute-force selection."""
    q, k, _ = workloads.random_qkv(1, 448, 2, seed=23)
    q, k = _np(q), _np(k)
    rt = ra.route(q, k, sink_start=420, ratio=0.34, radius=1)
    nvb = 6
    assert (rt.nb, rt.nvb) == (7, nvb)
    s = exact_scores(exact_block_means(q, nvb), exact_block_means(k, nvb))
    budget = ra.topk_budget(nvb, 0.34)
    for h in range(2):
        for i in range(nvb):
            forced = [j for j in range(nvb) if abs(j - i) <= 1]
            cand = [j for j in range(nvb) if j not in forced]
            want = _brute_topk({j: float(s[0, h, i, j]) for j in cand}, cand, min(budget, len(cand)))
            assert rt.rows[0][h][i].routed == want
            assert rt.rows[0][h][i].blocks == sorted(set(want) | set(forced) | {6})


# -------------------------------------------------------------- attention ---

def _case(T, H, seed, sink_start):
    q, k, v = workloads.random_qkv(1, T, H, seed=seed)
    return _np(q), _np(k), _np(v), sink_start


def _sink_bias_mask(T, nvb, bias):
    m = np.zeros((T, T))
    if bias is not None:
        kb = np.asarray(bias, dtype=np.float64).reshape(-1)[:T].copy()
        kb[: nvb * 64] = 0.0
        m = m + kb[None, :]
    return m


def check_ratio_one_equals_sdpa():
    q, k, v, ss = _case(200, 2, 31, 150)          # NVB=2, split video block, partial last block
    bias = workloads.sink_key_bias(1, 200, ss, seed=32).numpy()
    out, lse, rt = ra.routed_attention(q, k, v, ss, 1.0, 0, key_bias=bias)
    want = _sdpa(q, k, v, mask=_sink_bias_mask(200, rt.nvb, bias)[None, None])
    assert np.abs(out - want).max() < 1e-12
    # natural-log LSE against torch.logsumexp of the biased, scaled logits
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    logits = torch.einsum("bthd,bshd->bhts", qt, kt) / math.sqrt(128) + torch.from_numpy(_sink_bias_mask(200, 2, bias))
    assert np.abs(lse - torch.logsumexp(logits, dim=-1).numpy()).max() < 1e-10


def check_all_dense_when_no_video_block():
    q, k, v, ss = _case(150, 2, 33, 40)           # sink_start < 64 -> NVB = 0
    out, _, rt = ra.routed_attention(q, k, v, ss, 0.1, 1)
    assert rt.nvb == 0
    assert np.abs(out - _sdpa(q, k, v)).max() < 1e-12


def check_token_mask_path():
    """Block lists expanded to a token mask over the dense score matrix."""
    T, ss = 1000, 900                              # NVB=14, sinks {14, 15}, last block 40 keys
    q, k, v, _ = _case(T, 2, 34, ss)
    bias = workloads.sink_key_bias(1, T, ss, seed=35).numpy()
    out, _, rt = ra.routed_attention(q, k, v, ss, 0.25, 1, key_bias=bias)
    nvb = rt.nvb
    mask = np.full((2, T, T), -np.inf)
    for h in range(2):
        for t in range(T):
            if t < nvb * 64:
                for j in rt.rows[0][h][t // 64].blocks:
                    mask[h, t, j * 64:min(T, j * 64 + 64)] = 0.0
            else:
                mask[h, t, :] = 0.0
    mask = mask + _sink_bias_mask(T, nvb, bias)[None]
    want = _sdpa(q, k, v, mask=mask[None])
    assert np.abs(out - want).max() < 1e-12


def check_zero_bias_is_no_bias():
    q, k, v, ss = _case(400, 2, 36, 300)
    a, la, _ = ra.routed_attention(q, k, v, ss, 0.25, 0)
    b, lb, _ = ra.routed_attention(q, k, v, ss, 0.25, 0, key_bias=np.zeros((1, 400), np.float32))
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def check_bias_ln_m_duplicates_key():
    """Bias ln(m) on a sink key weighs it like m copies of that key."""
    T, ss, j0, m = 200, 128, 150, 3
    q, k, v, _ = _case(T, 2, 37, ss)
    bias = np.zeros((1, T), np.float32)
    bias[0, j0] = np.float32(math.log(m))
    out, _, _ = ra.routed_attention(q, k, v, ss, 1.0, 0, key_bias=bias)
    extra = [j0] * (m - 1)
    k2 = np.concatenate([k, k[:, extra]], axis=1)
    v2 = np.concatenate([v, v[:, extra]], axis=1)
    # fp32(ln 3) is ln 3 to 1e-8 relative, so the weights agree to ~1e-8
    want = _sdpa(q, k2, v2)
    assert np.abs(out - want).max() < 1e-6


def check_bias_removes_key():
    T, ss, j0 = 200, 128, 170
    q, k, v, _ = _case(T, 2, 38, ss)
    bias = np.zeros((1, T), np.float32)
    bias[0, j0] = -1e4
    out, _, _ = ra.routed_attention(q, k, v, ss, 1.0, 0, key_bias=bias)
    keep = [j for j in range(T) if j != j0]
    want = _sdpa(q, k[:, keep], v[:, keep])
    assert np.abs(out - want).max() < 1e-12


def check_bias_changes_output():
    q, k, v, ss = _case(400, 2, 39, 300)
    bias = workloads.sink_key_bias(1, 400, ss, seed=40).numpy()
    a, _, _ = ra.routed_attention(q, k, v, ss, 0.25, 0)
    b, _, _ = ra.routed_attention(q, k, v, ss, 0.25, 0, key_bias=bias)
    assert np.abs(a - b).max() > 1e-3


def check_bias_ignored_on_video_keys():
    """Only the exact sink branch consumes the bias: a bias on video keys
    leaves the output unchanged."""
    q, k, v, ss = _case(400, 2, 41, 300)
    bias = np.zeros((1, 400), np.float32)
    bias[0, :256] = -1.5                               # blocks 0..3 are video blocks
    a, _, _ = ra.routed_attention(q, k, v, ss, 0.25, 1)
    b, _, _ = ra.routed_attention(q, k, v, ss, 0.25, 1, key_bias=bias)
    assert np.array_equal(a, b)


def check_constant_v():
    q, k, v, ss = _case(330, 2, 42, 260)
    v = np.full_like(v, 0.75)
    out, _, _ = ra.routed_attention(q, k, v, ss, 0.2, 1)
    assert np.abs(out - 0.75).max() < 1e-12


def check_convex_hull():
    T, ss = 330, 260
    q, k, v, _ = _case(T, 2, 43, ss)
    out, _, rt = ra.routed_attention(q, k, v, ss, 0.2, 1)
    for h in range(2):
        for t in range(T):
            if t < rt.nvb * 64:
                idx = np.concatenate([np.arange(j * 64, min(T, j * 64 + 64)) for j in rt.rows[0][h][t // 64].blocks])
            else:
                idx = np.arange(T)
            vv = v[0, idx, h].astype(np.float64)
            assert np.all(out[0, t, h] >= vv.min(0) - 1e-12) and np.all(out[0, t, h] <= vv.max(0) + 1e-12)


def check_effective_flops_h3():
    # H3: 144 video blocks, 5 sink blocks (the last has 33 keys), ratio 0.1 -> 15 routed + self
    nvb, T, H = 144, 9505, 56
    lists = [[[list(range(nvb - 1))[:15] + [nvb - 1] + list(range(144, 149))] * nvb for _ in range(H)]]
    want = 4 * 128 * (H * nvb * 64 * (20 * 64 + 33) + H * (T - nvb * 64) * T)
    assert want == 425_709_039_616
    assert ra.effective_flops(T, H, 1, lists, nvb) == want


def check_golden_pages_numbers():
    with open(os.path.join(GOLDEN, "pages_numbers.json")) as f:
        items = {it["name"]: it["value"] for it in json.load(f)["items"]}
    assert ra.HEAD_DIM == items["head_dim"] and ra.BLOCK == items["block_tokens"]
    T, H = items["h3_tokens"], items["h3_heads"]
    # ~20 GB of scores for the dense matrix: fp32 [1, 56, 9505, 9505]
    gb = T * T * H * 4 / 1e9
    assert abs(gb - items["h3_dense_score_gigabytes"]) / items["h3_dense_score_gigabytes"] < 0.05
    nb, nvb = ra.block_counts(T, 9 * 32 * 32)
    assert (nb, nvb) == (T // 64 + 1, 144) and T % 64 == 33
    assert len(ra.forced_blocks(10, nvb, 0)) == items["exact_radius_0_forced_blocks"]
    assert len(ra.forced_blocks(10, nvb, 1)) == items["exact_radius_1_forced_blocks"]
    assert ra.topk_budget(nvb, items["default_topk_ratio"]) == 15
    # the pages keep sequences below the crossover dense; every configured
    # routed workload (Mid 8448, H3 9505, Long 33280 tokens) lies above it
    # and the small parity case (1024 tokens) below
    cross = items["dense_crossover_tokens"]
    assert cross == 8192 and 1024 < cross < min(8192 + 256, T, 32 * 1024 + 512)


# ------------------------------------------------------- pad video tail ---
# Page "Sol-Attn and Spark for MiniMax-H3", H3 pipeline integration (video
# tail mode) and Spark inference integration (last paragraph).

def check_pad_tail_means_exact():
    """The split block's centroid is the exact mean of its real video rows,
    rounded to fp32; complete blocks are unchanged."""
    x = _np(_varied_bf16((1, 320, 2, 128), seed=51))
    got = ra.pool_means(x, 5, end=300)              # block 4 holds rows 256..299
    want = exact_block_means(x, 5, end=300)
    assert np.array_equal(_bits(got), _bits(want)), "tail mean is not the mean of the real rows"
    assert np.array_equal(_bits(got[:, :, :4]), _bits(ra.pool_means(x, 4)))


def check_pad_centroid_preserved():
    """The padded 64-row block keeps the real rows and its plain mean is the
    routing centroid of the split block."""
    T, ss = 1000, 900
    q, k, _, _ = _case(T, 2, 52, ss)
    rt = ra.route(q, k, ss, 0.25, 1, tail_mode="pad")
    assert (rt.nvb, rt.nvq, rt.sparse_end) == (14, 15, 900)
    for h in range(2):
        blk = ra.pad_query_block(q, 0, h, 14, ss)
        assert blk.shape == (64, 128)
        assert np.array_equal(blk[:4], q[0, 896:900, h].astype(np.float64))
        scale = np.abs(q[0, 896:900, h]).max()
        assert np.abs(blk.mean(axis=0) - rt.qbar[0, h, 14]).max() <= 2.0 ** -23 * scale + 1e-12 * scale


def check_pad_route_and_mask():
    """Pad mode against an independent path: exact centroids and scores,
    brute-force Top-K for the split block, then a token mask over the dense
    score matrix in which rows < sink_start use their block's list."""
    T, ss = 1000, 900                                  # NVB=14, block 14 split at 4 rows
    q, k, v, _ = _case(T, 2, 53, ss)
    bias = workloads.sink_key_bias(1, T, ss, seed=54).numpy()
    out, lse, rt = ra.routed_attention(q, k, v, ss, 0.25, 1, key_bias=bias, tail_mode="pad")
    nvb, nb = 14, 16
    s = exact_scores(exact_block_means(q, 15, end=ss), exact_block_means(k, nvb))
    budget = ra.topk_budget(nvb, 0.25)
    for h in range(2):
        cand = list(range(nvb - 1))                    # block 13 is forced (radius 1)
        want = _brute_topk({j: float(s[0, h, 14, j]) for j in cand}, cand, budget)
        assert rt.rows[0][h][14].routed == want
        assert rt.rows[0][h][14].blocks == sorted(set(want) | {13, 14, 15})
    mask = np.full((2, T, T), -np.inf)
    for h in range(2):
        for t in range(T):
            if t < ss:
                for j in rt.rows[0][h][t // 64].blocks:
                    mask[h, t, j * 64:min(T, j * 64 + 64)] = 0.0
            else:
                mask[h, t, :] = 0.0
    mask = mask + _sink_bias_mask(T, nvb, bias)[None]
    assert np.abs(out - _sdpa(q, k, v, mask=mask[None])).max() < 1e-12
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    logits = torch.einsum("bthd,bshd->bhts", qt, kt) / math.sqrt(128) + torch.from_numpy(mask[None])
    assert np.abs(lse - torch.logsumexp(logits, dim=-1).numpy()).max() < 1e-10


def check_pad_modes_agree_where_they_must():
    """Aligned boundary: the modes are identical.  Split boundary: context
    rows are the same dense rows in both modes; the real tail rows change
    from dense to sparse."""
    q, k, v, ss = _case(400, 2, 55, 320)
    a, la, ra_ = ra.routed_attention(q, k, v, ss, 0.25, 1)
    b, lb, rb = ra.routed_attention(q, k, v, ss, 0.25, 1, tail_mode="pad")
    assert np.array_equal(a, b) and np.array_equal(la, lb) and ra_.lists() == rb.lists()
    q, k, v, ss = _case(1000, 2, 56, 900)
    a, la, _ = ra.routed_attention(q, k, v, ss, 0.25, 1)
    b, lb, _ = ra.routed_attention(q, k, v, ss, 0.25, 1, tail_mode="pad")
    assert np.abs(a[:, 900:] - b[:, 900:]).max() < 1e-12
    assert np.abs(la[:, :, 900:] - lb[:, :, 900:]).max() < 1e-12
    assert np.array_equal(a[:, :896], b[:, :896])
    assert np.abs(a[:, 896:900] - b[:, 896:900]).max() > 1e-4


def check_pad_ratio_one_and_no_complete_block():
    """Ratio 1 reaches every key, so pad mode is full attention; with no
    complete video block the split block's list is every (sink) block."""
    q, k, v, ss = _case(200, 2, 57, 150)               # NVB=2, block 2 split at 22 rows
    bias = workloads.sink_key_bias(1, 200, ss, seed=58).numpy()
    out, _, rt = ra.routed_attention(q, k, v, ss, 1.0, 0, key_bias=bias, tail_mode="pad")
    assert rt.nvq == 3
    assert np.abs(out - _sdpa(q, k, v, mask=_sink_bias_mask(200, 2, bias)[None, None])).max() < 1e-12
    q, k, v, ss = _case(150, 2, 59, 40)                # NVB=0, block 0 split at 40 rows
    out, _, rt = ra.routed_attention(q, k, v, ss, 0.1, 1, tail_mode="pad")
    assert (rt.nvb, rt.nvq) == (0, 1) and rt.rows[0][1][0].blocks == [0, 1, 2]
    assert np.abs(out - _sdpa(q, k, v)).max() < 1e-12
    assert ra.max_selected(150, 40, 0.1, 1, "pad") == 3 and ra.max_selected(150, 40, 0.1, 1) == 0


def check_pad_needs_context_slots():
    for T, ss in ((930, 900), (100, 70)):              # suffix cannot complete the block
        for fn in (lambda: ra.query_blocks(T, ss, "pad"),
                   lambda: ra.route(*_case(T, 1, 60, ss)[:2], ss, 0.1, 0, tail_mode="pad")):
            try:
                fn()
            except ValueError:
                pass
            else:
                raise AssertionError("pad mode accepted an incomplete tail block")
    assert ra.query_blocks(930, 900) == 14 and ra.query_blocks(960, 900, "pad") == 15
    try:
        ra.query_blocks(960, 900, "Pad")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown tail mode accepted")


def check_pad_effective_flops():
    """Closed form: real tail rows count, padded slots do not."""
    T, ss, nvb = 1000, 900, 14
    lists = [[[[0, 14, 15]] * nvb + [[13, 14, 15]]]]
    nk = 64 + 64 + 40
    want = 4 * 128 * (nvb * 64 * nk + 4 * nk + 100 * T)
    assert ra.effective_flops(T, 1, 1, lists, nvb, sparse_end=ss) == want


# ------------------------------------------------ Spark virtual summaries ---
# Page "Sol-Attn and Spark for MiniMax-H3", Spark primitives (spark_reweight)
# and Spark inference integration (global anchor, summaries merged with exact
# attention).

def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def check_anchor_exact():
    """The anchor is the exact mean of the video query rows, rounded to fp32
    then bf16; context rows do not count."""
    from fractions import Fraction
    from _exact import round_fraction_to_f32
    q = _np(_varied_bf16((1, 200, 2, 128), seed=61))
    got = sp.global_anchor(q, 150)
    assert got.shape == (1, 1, 2, 128)
    want = np.zeros((1, 1, 2, 128), np.float32)
    for h in range(2):
        for d in range(128):
            m = sum(Fraction(float(q[0, t, h, d])) for t in range(150)) / 150
            want[0, 0, h, d] = round_fraction_to_f32(m)
    assert np.array_equal(_bits(got), _bits(_bf16(want)))


def check_summaries_explicit_softmax():
    """ak, av, lm against torch.softmax / logsumexp over each block's keys,
    a partial final block included (its missing keys do not count)."""
    T, H, P = 200, 2, 2                                  # blocks of 64, 64, 64, 8
    _, k, v = (_np(x) for x in workloads.random_qkv(1, T, H, seed=62))
    a = _np(_varied_bf16((1, P, H, 128), seed=63))
    ak, av, lm = sp.virtual_summaries(a, k, v, logmass_key="pre_round", store="f64")
    akr, avr, lmr = sp.virtual_summaries(a, k, v)        # stored bf16, stored-key log-mass
    assert ak.shape == (1, P, H, 4, 128) and lm.shape == (1, P, H, 4)
    s = 1.0 / math.sqrt(128)
    for p in range(P):
        for h in range(H):
            for j in range(4):
                kt = torch.from_numpy(k[0, 64 * j:min(T, 64 * j + 64), h].astype(np.float64))
                vt = torch.from_numpy(v[0, 64 * j:min(T, 64 * j + 64), h].astype(np.float64))
                at = torch.from_numpy(a[0, p, h].astype(np.float64))
                z = (kt @ at) * s
                w = torch.softmax(z, dim=0)
                wk, wv = (w @ kt).numpy(), (w @ vt).numpy()
                assert np.abs(ak[0, p, h, j] - wk).max() < 1e-12
                assert np.abs(av[0, p, h, j] - wv).max() < 1e-12
                lse = float(torch.logsumexp(z, dim=0))
                assert abs(lm[0, p, h, j] - (lse - s * float(at @ torch.from_numpy(wk)))) < 1e-10
                # stored: bf16 of the weighted key/value, log-mass shifted by the stored key
                assert np.array_equal(_bits(akr[0, p, h, j]), _bits(_bf16(wk)))
                assert np.array_equal(_bits(avr[0, p, h, j]), _bits(_bf16(wv)))
                shift = s * float(at @ torch.from_numpy(_bf16(wk).astype(np.float64)))
                assert abs(lmr[0, p, h, j] - (lse - shift)) < 1e-10


def check_log_mass_closed_forms():
    """A block of n identical keys: ak is that key and lm = ln n (64 for a
    full block, 8 for the partial final block of T = 200)."""
    T, H = 200, 1
    _, k, v = (_np(x) for x in workloads.random_qkv(1, T, H, seed=64))
    for j in range(4):
        k[0, 64 * j:min(T, 64 * j + 64)] = k[0, 64 * j]
    a = _np(_varied_bf16((1, 1, H, 128), seed=65))
    ak, _, lm = sp.virtual_summaries(a, k, v)
    for j, n in enumerate((64, 64, 64, 8)):
        assert np.array_equal(ak[0, 0, 0, j], k[0, 64 * j, 0].astype(np.float64))
        assert abs(lm[0, 0, 0, j] - math.log(n)) < 1e-9


def _anchor_rows_case(seed):
    """Q whose query block 2 rows all equal the anchor, plus unrounded
    summaries shifted by the unrounded key."""
    T, H, ss = 600, 2, 512                               # NVB = 8, sinks 8, 9 (last partial)
    q, k, v = (_np(x) for x in workloads.random_qkv(1, T, H, seed=seed))
    a = sp.global_anchor(q, ss)
    q[0, 128:192] = a[0, 0][None]
    summ = sp.virtual_summaries(a, k, v, logmass_key="pre_round", store="f64")
    return q, k, v, ss, summ


def check_spark_anchor_rows_are_exact():
    """For a query row equal to the anchor, every skipped block's virtual key
    carries that block's exact softmax mass and weighted value, so the row
    equals full attention over all keys (with the sink bias)."""
    q, k, v, ss, summ = _anchor_rows_case(66)
    bias = workloads.sink_key_bias(1, 600, ss, seed=67).numpy()
    out, lse, rt = sp.routed_attention_spark(q, k, v, ss, 0.25, 1, summ, key_bias=bias)
    assert len(rt.rows[0][0][2].blocks) < rt.nb             # some blocks are skipped
    want = _sdpa(q, k, v, mask=_sink_bias_mask(600, 8, bias)[None, None])
    assert np.abs(out[0, 128:192] - want[0, 128:192]).max() < 1e-10
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    logits = torch.einsum("bthd,bshd->bhts", qt, kt) / math.sqrt(128) + torch.from_numpy(_sink_bias_mask(600, 8, bias))
    assert np.abs(lse[0, :, 128:192] - torch.logsumexp(logits, dim=-1).numpy()[0, :, 128:192]).max() < 1e-10
    # and the other rows do differ from full attention
    assert np.abs(out[0, :128] - want[0, :128]).max() > 1e-4


def check_spark_ratio_one_is_exact():
    """Ratio 1 leaves no block skipped: the approximate branch adds nothing."""
    q, k, v, ss = _case(600, 2, 68, 512)
    a = sp.global_anchor(q, ss)
    summ = sp.virtual_summaries(a, k, v)
    o1, l1, _ = sp.routed_attention_spark(q, k, v, ss, 1.0, 0, summ)
    o2, l2, _ = ra.routed_attention(q, k, v, ss, 1.0, 0)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def check_spark_token_mask_path():
    """Against one dense formulation: every row sees all T keys plus NVB
    virtual keys; a mask keeps, for sparse rows, the keys of its exact
    blocks and the virtual keys of its skipped blocks (with bias lm), and
    for dense rows the real keys only."""
    T, ss, H = 1000, 900, 2                              # NVB = 14, split tail (pad mode)
    q, k, v, _ = _case(T, H, 69, ss)
    bias = workloads.sink_key_bias(1, T, ss, seed=70).numpy()
    a = sp.global_anchor(q, ss)
    ak, av, lm = sp.virtual_summaries(a, k, v)
    out, _, rt = sp.routed_attention_spark(q, k, v, ss, 0.25, 1, (ak, av, lm), key_bias=bias,
                                           tail_mode="pad")
    nvb = 14
    k2 = np.concatenate([k, np.transpose(ak[:, 0, :, :nvb], (0, 2, 1, 3))], axis=1)
    v2 = np.concatenate([v, np.transpose(av[:, 0, :, :nvb], (0, 2, 1, 3))], axis=1)
    mask = np.full((H, T, T + nvb), -np.inf)
    for h in range(H):
        for t in range(T):
            if t < ss:
                blocks = rt.rows[0][h][t // 64].blocks
                for j in blocks:
                    mask[h, t, j * 64:min(T, j * 64 + 64)] = 0.0
                for j in range(nvb):
                    if j not in blocks:
                        mask[h, t, T + j] = lm[0, 0, h, j]
            else:
                mask[h, t, :T] = 0.0
    sb = np.zeros(T + nvb)
    sb[:T] = bias[0]
    sb[: nvb * 64] = 0.0
    mask = mask + sb[None, None, :]
    want = _sdpa(q, k2, v2, mask=mask[None])
    assert np.abs(out - want).max() < 1e-12


ALL_CHECKS = [
    check_pool_exact, check_pool_permutation_invariant, check_scores_exact,
    check_budget, check_topk_bruteforce, check_signed_zero_tie, check_near_tie_flag,
    check_list_accepted,
    check_list_structure, check_route_glue, check_ratio_one_equals_sdpa,
    check_all_dense_when_no_video_block, check_token_mask_path,
    check_zero_bias_is_no_bias, check_bias_ln_m_duplicates_key, check_bias_removes_key,
    check_bias_changes_output, check_bias_ignored_on_video_keys, check_constant_v,
    check_convex_hull, check_effective_flops_h3, check_golden_pages_numbers,
    check_pad_tail_means_exact, check_pad_centroid_preserved, check_pad_route_and_mask,
    check_pad_modes_agree_where_they_must, check_pad_ratio_one_and_no_complete_block,
    check_pad_needs_context_slots, check_pad_effective_flops,
    check_anchor_exact, check_summaries_explicit_softmax, check_log_mass_closed_forms,
    check_spark_anchor_rows_are_exact, check_spark_ratio_one_is_exact, check_spark_token_mask_path,
]
