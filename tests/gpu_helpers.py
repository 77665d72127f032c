"""Helpers for the GPU parity tests: run the HIP path through the C-ABI
binding, run the oracle on the same bf16 inputs, compare."""
import sys
import time

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


def check_route(res, rt, wl):
    B, T, H, _ = wl.q.shape
    nvb, nvq = rt.nvb, rt.nvq
    if nvq == 0:
        return
    rows, mism, ties, unexp = compare_lists(res["idx"], res["cnt"], rt)
    log(f"[{wl.name}] lists: rows={rows} mismatched={mism} near_ties={ties} unexplained={unexp}")
    assert unexp == 0
    if res["scores"] is not None and nvb > 0:
        g = res["scores"].numpy()
        # fp32 of an fp64 dot product on both sides: equal except where the two
        # fp64 sums straddle an fp32 rounding boundary (1 ulp)
        gi = g.view(np.int32).astype(np.int64)
        oi = rt.scores.view(np.int32).astype(np.int64)
        ulps = np.abs(gi - oi)
        log(f"[{wl.name}] scores: bit-equal={np.mean(ulps == 0):.6f} max_ulp={ulps.max()}")
        assert ulps.max() <= 1
    # forced and sink blocks always present
    idx, cnt = res["idx"].numpy(), res["cnt"].numpy()
    nb = rt.nb
    for b in range(B):
        for h in range(H):
            for i in range(nvq):
                s = set(idx[b, h, i, :cnt[b, h, i]].tolist())
                assert set(ora.forced_blocks(i, nvb, wl.local_radius)) <= s
                assert set(range(nvb, nb)) <= s


def full_parity(wl, key_bias=None):
    q, k, v = (to_np(x) for x in (wl.q, wl.k, wl.v))
    kb = key_bias if key_bias is not None else wl.key_bias
    kbn = None if kb is None else kb.numpy()
    log(f"[{wl.name}] GPU run")
    res = run_gpu(wl, key_bias=kb)
    t0 = time.perf_counter()
    log(f"[{wl.name}] oracle route")
    rt = ora.route(q, k, wl.sink_start, wl.topk_ratio, wl.local_radius, tail_mode=wl.tail_mode)
    check_route(res, rt, wl)
    adopt_lists(res["idx"], res["cnt"], rt)
    log(f"[{wl.name}] oracle attention ({time.perf_counter() - t0:.1f} s so far)")
    want, want_lse, _ = ora.routed_attention(q, k, v, wl.sink_start, wl.topk_ratio,
                                             wl.local_radius, key_bias=kbn, rt=rt)
    got = to_np(res["out"])
    assert np.isfinite(got).all()
    mx, mean = err_stats(got, want)
    lmx, _ = err_stats(res["lse"].numpy(), want_lse)
    worst = np.unravel_index(np.argmax(np.abs(got - want)), got.shape)
    log(f"[{wl.name}] every element: out max_abs={mx:.3e} (oracle value there {want[worst]:.4f}) "
        f"mean_abs={mean:.3e} |out|max={np.abs(want).max():.3f} lse max_abs={lmx:.3e} "
        f"(oracle {time.perf_counter() - t0:.1f} s)")
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    assert lmx <= 1e-2
    return res, rt
