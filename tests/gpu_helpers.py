"""Helpers for the GPU parity tests: run the HIP path through the C-ABI
binding, run the oracle on the same bf16 inputs, compare."""
import sys

import numpy as np
import torch

import oracle.sparse_attention as ora

# Output tolerance against the oracle (fp32/fp64 reference, bf16 output).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy()


def run_gpu(wl, *, key_bias=None, ratio=None, radius=None, scores=True, lse=True, check_bias=True):
    import block_sparse_attention_05_amd as sa
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (wl.q, wl.k, wl.v))
    B, T, H, _ = q.shape
    ratio = wl.topk_ratio if ratio is None else ratio
    radius = wl.local_radius if radius is None else radius
    kb = key_bias if key_bias is not None else wl.key_bias
    kb = None if kb is None else kb.to(dev)
    mode = wl.tail_mode
    nb, nvb = ora.block_counts(T, wl.sink_start)
    nvq = ora.query_blocks(T, wl.sink_start, mode)
    sc = torch.full((B, H, nvq, nvb), float("nan"), device=dev) if (scores and nvb) else None
    idx, cnt = sa.sparse_attn_route(q, k, wl.sink_start, ratio, radius, video_tail_mode=mode,
                                    route_scores=sc)
    out = torch.full_like(q, float("nan"))
    ls = torch.full((B, H, T), float("nan"), device=dev) if lse else None
    sa.sparse_attn_fwd(q, k, v, wl.sink_start, idx, cnt, video_tail_mode=mode, key_bias=kb,
                       out=out, lse=ls, check_bias=check_bias)
    sa.dense_sink_fwd(q, k, v, wl.sink_start, video_tail_mode=mode, key_bias=kb, out=out, lse=ls,
                      check_bias=check_bias)
    torch.cuda.synchronize()
    return dict(out=out.cpu(), lse=None if ls is None else ls.cpu(), idx=idx.cpu(), cnt=cnt.cpu(),
                scores=None if sc is None else sc.cpu())


def compare_lists(idx, cnt, rt):
    """Lists must equal the oracle's except in near-tie rows, where every
    differing block must have an oracle score inside the tie band
    (``oracle.list_accepted``).  Returns (rows, mismatched rows, near-tie
    rows, unexplained rows)."""
    idx = idx.numpy() if hasattr(idx, "numpy") else np.asarray(idx)
    cnt = cnt.numpy() if hasattr(cnt, "numpy") else np.asarray(cnt)
    B, H, nvq, max_sel = idx.shape
    rows = mism = ties = unexplained = 0
    for b in range(B):
        for h in range(H):
            for i in range(nvq):
                rows += 1
                sel = rt.rows[b][h][i]
                c = int(cnt[b, h, i])
                got = idx[b, h, i, :c].tolist()
                assert all(x == -1 for x in idx[b, h, i, c:]), "padding must be -1"
                assert got == sorted(set(got)), "lists must be strictly ascending"
                ties += sel.near_tie
                if got == sel.blocks:
                    continue
                mism += 1
                if not ora.list_accepted(got, sel, rt.scores[b, h, i], rt.nvb):
                    unexplained += 1
    return rows, mism, ties, unexplained


def adopt_lists(idx, cnt, rt):
    """Point the oracle's route at the GPU's lists (after compare_lists has
    accepted them), so that attention is compared on the same key sets."""
    idx = idx.numpy() if hasattr(idx, "numpy") else np.asarray(idx)
    cnt = cnt.numpy() if hasattr(cnt, "numpy") else np.asarray(cnt)
    for b, brow in enumerate(rt.rows):
        for h, hrow in enumerate(brow):
            for i, sel in enumerate(hrow):
                sel.blocks = idx[b, h, i, :cnt[b, h, i]].tolist()


def err_stats(got, want):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(d.max()), float(d.mean())


def pad_lists(idx, cnt, front, back, width):
    """Lists with the entries `front` before and `back` after every list's
    own entries (all ascending), -1 beyond, `width` entries per list."""
    B, H, nq, ms = idx.shape
    wide = torch.full((B, H, nq, width), -1, dtype=torch.int32, device=idx.device)
    c = cnt.long()
    nf = len(front)
    for j, x in enumerate(front):
        wide[..., j] = x
    pos = torch.arange(ms, device=idx.device).view(1, 1, 1, ms)
    ok = pos < c.unsqueeze(-1)
    tgt = torch.where(ok, pos + nf, torch.full_like(pos, width - 1)).expand(B, H, nq, ms)
    vals = torch.where(ok, idx, torch.full_like(idx, -1))
    wide.scatter_(-1, tgt, vals)
    for j, x in enumerate(back):
        wide.scatter_(-1, (c + nf + j).unsqueeze(-1), torch.full_like(c.unsqueeze(-1), x, dtype=torch.int32))
    wide[..., width - 1] = torch.where(c + nf + len(back) > width - 1, wide[..., width - 1],
                                       torch.full_like(cnt, -1))
    return wide, (cnt + nf + len(back)).to(torch.int32)
