"""Spark virtual summaries and the approximate branch: HIP path vs the CPU
oracle (oracle/spark_summaries.py) on the same seeded bf16 inputs (needs a
GPU; every call goes through the C ABI).

Anchor: bit-exact.  Summaries: each ak / av value within one bf16 ulp of the
oracle's or within 1e-3 absolute (both sides round a value they computed in
different precision; near zero one ulp is tiny), lm within 1e-4
of the oracle's log-mass taken against the GPU's own stored key, for every
head.  Lists: equal to the oracle's except inside near-tie bands.
Attention: every element of out and LSE, max-abs <= 2e-2 and mean-abs
<= 2e-3, with the oracle fed the GPU's lists and summaries (so the check
isolates the merge), including the full H3 size.
"""
import time

import numpy as np
import pytest
import torch

import oracle.sparse_attention as ora
import oracle.spark_summaries as osp
import workloads
from gpu_helpers import MAX_ABS, MEAN_ABS, adopt_lists, compare_lists, err_stats, log, to_np

pytestmark = pytest.mark.gpu


def _bf16_ulp(x):
    """Spacing of bf16 values at |x| (normal range)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _check_summaries(got_ak, got_av, got_lm, a, k, v, heads, name, logmass_key="stored"):
    """Oracle summaries for the given heads; returns the worst deviations."""
    a_n = to_np(a)[:, :, heads]
    k_n, v_n = to_np(k)[:, :, heads], to_np(v)[:, :, heads]
    ak, av, lm = osp.virtual_summaries(a_n, k_n, v_n, logmass_key=logmass_key)
    gak = to_np(got_ak)[:, :, heads]
    gav = to_np(got_av)[:, :, heads]
    glm = got_lm.cpu().numpy()[:, :, heads]
    dk = np.abs(gak - ak) / (_bf16_ulp(ak) + 1e-30)
    dv = np.abs(gav - av) / (_bf16_ulp(av) + 1e-30)
    small_k = np.abs(gak - ak) <= 1e-3
    small_v = np.abs(gav - av) <= 1e-3
    assert np.all((dk <= 1.0) | small_k), f"ak off by {dk.max():.2f} ulp"
    assert np.all((dv <= 1.0) | small_v), f"av off by {dv.max():.2f} ulp"
    # log-mass against the GPU's own key: isolates lm from a bf16 rounding flip
    B, P, H, NB, _ = gak.shape
    T = k_n.shape[1]
    lm_own = np.zeros_like(glm, dtype=np.float64)
    s = 1.0 / np.sqrt(128)
    for b in range(B):
        for p in range(P):
            for h in range(H):
                for j in range(NB):
                    keys = k_n[b, 64 * j:min(T, 64 * j + 64), h]
                    shift = gak[b, p, h, j] if logmass_key == "stored" else ak[b, p, h, j]
                    lm_own[b, p, h, j] = osp.log_mass(a_n[b, p, h], keys, shift, s)
    tol = 1e-4 if logmass_key == "stored" else 5e-3
    e_own = np.abs(glm - lm_own).max()
    e_ora = np.abs(glm - lm).max()
    log(f"[{name}] summaries: ak max {dk.max():.2f} ulp, av max {dv.max():.2f} ulp, "
        f"lm vs own-key {e_own:.2e}, vs oracle {e_ora:.2e}")
    assert e_own <= tol and e_ora <= 5e-3


def _split_case(seed=7):
    q, k, v, tv = workloads.video_qkv(B=1, H=3, frames=2, ctx_tokens=150, seed=seed, height=16, width=32)
    return q, k, v, tv - 17


def test_anchor_bit_exact():
    import block_sparse_attention_05_amd as sa
    for (q, ss) in ((_split_case()[0], 1007), (workloads.mid().q, 8192)):
        got = sa.spark_global_anchor(q.cuda(), ss)
        torch.cuda.synchronize()
        want = osp.global_anchor(to_np(q), ss)
        assert np.array_equal(to_np(got).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("key", ["stored", "pre_round"])
def test_reweight_matches_oracle(key):
    import block_sparse_attention_05_amd as sa
    q, k, v, ss = _split_case()                      # T = 1174: partial final block of 22 keys
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    g = torch.Generator().manual_seed(21)
    anchors = torch.cat([sa.spark_global_anchor(qc, ss),
                         torch.randn(1, 1, 3, 128, generator=g).to(torch.bfloat16).cuda()], dim=1)
    ak, av, lm = sa.spark_reweight(anchors.contiguous(), kc, vc, logmass_key=key)
    torch.cuda.synchronize()
    assert ak.shape == (1, 2, 3, 19, 128) and lm.shape == (1, 2, 3, 19)
    _check_summaries(ak, av, lm, anchors.cpu(), k, v, [0, 1, 2], f"reweight_{key}", key)


def _spark_parity(q, k, v, ss, ratio, radius, name, key_bias=None, tail_mode="dense"):
    """The whole Spark call against the oracle: anchor (bit-exact), the
    summaries of every head, every list (tie bands), every output and LSE
    element."""
    import block_sparse_attention_05_amd as sa
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    kb = None if key_bias is None else key_bias.cuda()
    log(f"[{name}] GPU run")
    out, lse, parts = sa.routed_attention_spark(qc, kc, vc, ss, ratio, radius, video_tail_mode=tail_mode,
                                                key_bias=kb, return_lse=True, return_parts=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    anchor = parts["anchor"].cpu()
    assert np.array_equal(to_np(anchor).view(np.uint32), osp.global_anchor(to_np(q), ss).view(np.uint32))
    ak, av, lm = (x.cpu() for x in parts["summaries"])
    _check_summaries(ak, av, lm, anchor, k, v, list(range(q.shape[2])), name)
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    rt = ora.route(qn, kn, ss, ratio, radius, tail_mode=tail_mode)
    rows, mism, ties, unexp = compare_lists(parts["block_idx"].cpu(), parts["block_cnt"].cpu(), rt)
    log(f"[{name}] lists: rows={rows} mismatched={mism} near_ties={ties} unexplained={unexp}")
    assert unexp == 0
    adopt_lists(parts["block_idx"].cpu(), parts["block_cnt"].cpu(), rt)
    log(f"[{name}] oracle attention ({time.perf_counter() - t0:.1f} s so far)")
    want, want_lse, _ = osp.routed_attention_spark(
        qn, kn, vn, ss, ratio, radius, (to_np(ak), to_np(av), lm.numpy().astype(np.float64)),
        key_bias=None if key_bias is None else key_bias.numpy(), rt=rt, tail_mode=tail_mode)
    got = to_np(out)
    assert np.isfinite(got).all()
    mx, mean = err_stats(got, want)
    lmx, _ = err_stats(lse.cpu().numpy(), want_lse)
    log(f"[{name}] spark every element: out max_abs={mx:.3e} mean_abs={mean:.3e} lse max_abs={lmx:.3e} "
        f"(oracle {time.perf_counter() - t0:.1f} s)")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lmx <= 1e-2
    return out, parts


def test_spark_split_block_with_bias():
    q, k, v, ss = _split_case()
    bias = workloads.sink_key_bias(1, q.shape[1], ss, seed=8)
    _spark_parity(q, k, v, ss, 0.2, 1, "spark_split", key_bias=bias)


def test_spark_pad_mode():
    q, k, v, ss = _split_case(seed=9)
    bias = workloads.sink_key_bias(1, q.shape[1], ss, seed=10)
    _spark_parity(q, k, v, ss, 0.2, 1, "spark_pad", key_bias=bias, tail_mode="pad")


def test_spark_many_virtual_tiles_odd_count():
    # NVB = 200, budget 10 + the self block: 189 skipped blocks pack into
    # three virtual tiles (an odd count, the last one partial)
    q, k, v = workloads.random_qkv(1, 64 * 200 + 100, 2, seed=11)
    _spark_parity(q, k, v, 64 * 200, 0.05, 0, "spark_nvb200")


def test_spark_no_bias_whole_sink_blocks():
    """Without key_bias the complete sink tiles run ahead of the virtual
    tiles; here T is a multiple of 64, so no partial block follows them."""
    q, k, v = workloads.random_qkv(1, 64 * 40, 2, seed=23)
    _spark_parity(q, k, v, 64 * 36, 0.1, 0, "spark_nobias_T64")


def test_spark_no_bias_split_block():
    """Without key_bias, with the video boundary inside a block and a
    partial last block (the only tile after the virtual ones)."""
    q, k, v, ss = _split_case(seed=24)
    for mode in ("dense", "pad"):
        _spark_parity(q, k, v, ss, 0.2, 1, f"spark_nobias_split_{mode}", tail_mode=mode)


def test_spark_ratio_one_equals_exact():
    """Nothing skipped: no virtual tile, so the approximate branch walks the
    exact path's tiles in the same order on the same paired kernel and
    gives the same bits.  One leaked virtual key would carry about a
    block's worth of mass and move LSE and outputs by several hundredths."""
    import block_sparse_attention_05_amd as sa
    q, k, v, ss = _split_case(seed=12)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    bias = workloads.sink_key_bias(1, q.shape[1], ss, seed=13).cuda()
    idx, cnt = sa.sparse_attn_route(qc, kc, ss, 1.0, 0)
    summ = sa.spark_reweight(sa.spark_global_anchor(qc, ss), kc, vc)
    lse_a = torch.zeros(1, 3, q.shape[1], device="cuda")
    lse_b = torch.zeros(1, 3, q.shape[1], device="cuda")
    a = sa.sparse_attn_fwd(qc, kc, vc, ss, idx, cnt, key_bias=bias, lse=lse_a)
    b = sa.sparse_attn_fwd_spark(qc, kc, vc, ss, idx, cnt, summ, key_bias=bias, lse=lse_b)
    torch.cuda.synchronize()
    rows = 64 * (ss // 64)
    d = (a[:, :rows].float() - b[:, :rows].float()).abs().max().item()
    dl = (lse_a[:, :, :rows] - lse_b[:, :, :rows]).abs().max().item()
    log(f"[spark ratio 1] vs exact path: out max_abs={d:.3e} lse max_abs={dl:.3e}")
    assert torch.equal(a[:, :rows], b[:, :rows]) and torch.equal(lse_a[:, :, :rows], lse_b[:, :, :rows])


def test_spark_one_block_kernel_wide_lists():
    """Lists wider than the paired kernel takes with the approximate branch
    (the same entries, -1 up to 512 per list) run on the one-block kernel:
    every output and LSE element of the sparse rows against the oracle, and
    within the tolerance of the paired kernel's."""
    import block_sparse_attention_05_amd as sa
    from gpu_helpers import pad_lists
    q, k, v, ss = _split_case(seed=31)
    bias = workloads.sink_key_bias(1, q.shape[1], ss, seed=32)
    qc, kc, vc, kb = q.cuda(), k.cuda(), v.cuda(), bias.cuda()
    ratio, radius = 0.2, 1
    pair_out, pair_lse, parts = sa.routed_attention_spark(qc, kc, vc, ss, ratio, radius, key_bias=kb,
                                                         return_lse=True, return_parts=True)
    idx, cnt, summ = parts["block_idx"], parts["block_cnt"], parts["summaries"]
    wide, wcnt = pad_lists(idx, cnt, [], [], 512)
    lse = torch.zeros_like(pair_lse)
    out = sa.sparse_attn_fwd_spark(qc, kc, vc, ss, wide, wcnt, summ, key_bias=kb, lse=lse)
    torch.cuda.synchronize()
    rows = 64 * (ss // 64)
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    rt = ora.route(qn, kn, ss, ratio, radius)
    adopt_lists(idx.cpu(), cnt.cpu(), rt)
    ak, av, lm = (x.cpu() for x in summ)
    want, want_lse, _ = osp.routed_attention_spark(qn, kn, vn, ss, ratio, radius,
                                                   (to_np(ak), to_np(av), lm.numpy().astype(np.float64)),
                                                   key_bias=bias.numpy(), rt=rt)
    mx, mean = err_stats(to_np(out)[:, :rows], want[:, :rows])
    lmx, _ = err_stats(lse.cpu().numpy()[:, :, :rows], want_lse[:, :, :rows])
    d = (out[:, :rows].float() - pair_out[:, :rows].float()).abs().max().item()
    log(f"[spark one-block] out max_abs={mx:.3e} mean_abs={mean:.3e} lse max_abs={lmx:.3e}; "
        f"vs paired kernel max_abs={d:.3e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lmx <= 1e-2 and d <= MAX_ABS


def test_spark_h3_full():
    """Full H3 size with key_bias: the summaries of all 56 heads and every
    output element against the oracle."""
    wl = workloads.h3(with_bias=True)
    _spark_parity(wl.q, wl.k, wl.v, wl.sink_start, wl.topk_ratio, wl.local_radius, "spark_h3",
                  key_bias=wl.key_bias)


def test_spark_max_route_blocks_full():
    """NVB = 1024: about 918 skipped blocks per row packed into 15 virtual
    tiles, lists of 110 entries."""
    wl = workloads.max_blocks()
    _spark_parity(wl.q, wl.k, wl.v, wl.sink_start, wl.topk_ratio, wl.local_radius, "spark_maxblocks",
                  key_bias=wl.key_bias)


def test_spark_batch2_radius2_pad_with_bias():
    q, k, v = workloads.random_qkv(2, 1100, 3, seed=19)
    bias = workloads.sink_key_bias(2, 1100, 1000, seed=20)
    _spark_parity(q, k, v, 1000, 0.3, 2, "spark_B2_pad", key_bias=bias, tail_mode="pad")


def test_spark_invalid_entries_are_skipped():
    """The approximate branch with lists padded by entries outside [0, NB)
    (-7, -1 in front; NB, NB + 3 behind) gives the same bits as the plain
    lists, with and without key_bias: the virtual keys are the video blocks
    the valid entries skip."""
    import block_sparse_attention_05_amd as sa
    from gpu_helpers import pad_lists
    wl = workloads.mid()
    q, k, v = (x.cuda() for x in (wl.q, wl.k, wl.v))
    T = q.shape[1]
    nb = -(-T // 64)
    ss = wl.sink_start
    bias = workloads.sink_key_bias(1, T, ss, seed=12).cuda()
    out, parts = sa.routed_attention_spark(q, k, v, ss, wl.topk_ratio, wl.local_radius, return_parts=True)
    idx, cnt = parts["block_idx"], parts["block_cnt"]
    summ = parts["summaries"]
    wide, wcnt = pad_lists(idx, cnt, [-7, -1], [nb, nb + 3], idx.shape[-1] + 4)
    for kb in (None, bias):
        ref = sa.sparse_attn_fwd_spark(q, k, v, ss, idx, cnt, summ, key_bias=kb)
        got = sa.sparse_attn_fwd_spark(q, k, v, ss, wide, wcnt, summ, key_bias=kb)
        torch.cuda.synchronize()
        assert torch.equal(got[:, :ss], ref[:, :ss]), kb is None
