"""HIP path vs the CPU oracle on the same seeded bf16 inputs (needs a GPU).

Selections: bit-exact lists except rows the oracle reports as near-ties
(there a differing block must score inside the tie band).  Outputs: every
element of out and LSE, max-abs <= 2e-2 and mean-abs <= 2e-3 against the
oracle, at every size including the full H3, H3 + key_bias, Long and
1024-block workloads.
"""
import time

import numpy as np
import pytest
import torch

import oracle.sparse_attention as ora
import workloads
from gpu_helpers import (MAX_ABS, MEAN_ABS, adopt_lists, check_route, compare_lists, err_stats,
                         full_parity, log, pad_lists, run_gpu, to_np)

pytestmark = pytest.mark.gpu


def test_tiny_full():
    full_parity(workloads.tiny())


def test_tiny_batch2_radius2():
    q, k, v = workloads.tiny_qkv(B=2, H=3, T=1024, seed=5)
    wl = workloads.Workload("tiny_B2_H3_r2", q, k, v, sink_start=1024, topk_ratio=0.3, local_radius=2)
    full_parity(wl)


def test_mid_full():
    full_parity(workloads.mid())


def test_split_video_block_and_bias():
    # video boundary inside a 64-token block: that block is a sink block and
    # its rows take the dense path; last block partial
    q, k, v, tv = workloads.video_qkv(B=1, H=3, frames=2, ctx_tokens=150, seed=7, height=16, width=32)
    tv2 = tv - 17                          # 1024 - 17: boundary splits block 15
    bias = workloads.sink_key_bias(1, q.shape[1], tv2, seed=8)
    wl = workloads.Workload("split_block", q, k, v, sink_start=tv2, topk_ratio=0.2, local_radius=1,
                            key_bias=bias)
    full_parity(wl)


# ---- pad video tail mode ---------------------------------------------------

def _split_workload(mode, name="split_block"):
    q, k, v, tv = workloads.video_qkv(B=1, H=3, frames=2, ctx_tokens=150, seed=7, height=16, width=32)
    tv2 = tv - 17                          # 1024 - 17: boundary splits block 15
    bias = workloads.sink_key_bias(1, q.shape[1], tv2, seed=8)
    return workloads.Workload(f"{name}_{mode}", q, k, v, sink_start=tv2, topk_ratio=0.2,
                              local_radius=1, key_bias=bias, tail_mode=mode)


def test_pad_split_video_block_and_bias():
    # block 15 (47 real video rows) is routed and sparse, context rows dense
    res, rt = full_parity(_split_workload("pad"))
    assert rt.nvq == rt.nvb + 1 and res["cnt"].shape[2] == rt.nvq


def test_pad_h3_shape_split_tail():
    # H3 sequence with the video boundary 17 rows before a block edge
    q, k, v, tv = workloads.video_qkv(B=1, H=4, frames=9, ctx_tokens=289, seed=13)
    bias = workloads.sink_key_bias(1, q.shape[1], tv - 17, seed=14)
    wl = workloads.Workload("h3_H4_pad", q, k, v, sink_start=tv - 17, topk_ratio=0.1,
                            local_radius=1, key_bias=bias, tail_mode="pad")
    full_parity(wl)


def test_pad_without_complete_video_block():
    # NVB = 0: the split block 0 is the only query block; its list is every block
    q, k, v = workloads.random_qkv(1, 700, 2, seed=15)
    wl = workloads.Workload("pad_nvb0", q, k, v, sink_start=40, topk_ratio=0.1, local_radius=1,
                            tail_mode="pad")
    res, rt = full_parity(wl)
    assert res["cnt"].flatten().tolist() == [11, 11]


def test_pad_and_dense_modes_share_bits_where_they_must():
    """Where the two modes run the same computation they give the same bits:
    the lists of the complete video blocks, the outputs of the query-block
    pairs that are the same in both modes (blocks 0-13; block 14 is alone in
    dense mode and paired with the split block in pad mode, so its tiles are
    summed in another order) and the context rows.  With a block-aligned
    boundary the whole call is equal."""
    a = run_gpu(_split_workload("dense"))
    b = run_gpu(_split_workload("pad"))
    ss = 1024 - 17
    assert torch.equal(a["idx"], b["idx"][:, :, :-1]) and torch.equal(a["cnt"], b["cnt"][:, :, :-1])
    assert torch.equal(a["out"][:, :896], b["out"][:, :896])
    d = (a["out"][:, 896:960].float() - b["out"][:, 896:960].float()).abs().max().item()
    log(f"[pad vs dense] block 14 max_abs={d:.3e}")
    assert d <= 1e-2
    assert torch.equal(a["out"][:, ss:], b["out"][:, ss:])
    assert torch.equal(a["lse"][:, :, ss:], b["lse"][:, :, ss:])
    assert not torch.equal(a["out"][:, 960:ss], b["out"][:, 960:ss])
    wl = workloads.mid()
    c = run_gpu(wl)
    wl.tail_mode = "pad"
    d = run_gpu(wl)
    for key in ("out", "lse", "idx", "cnt", "scores"):
        assert torch.equal(c[key], d[key]), key


def test_pad_pooled_tail_mean_bit_exact():
    import block_sparse_attention_05_amd as sa
    wl = _split_workload("pad")
    q, k = wl.q.cuda(), wl.k.cuda()
    B, T, H, _ = q.shape
    ss = wl.sink_start
    nvb, nvq = ss // 64, ss // 64 + 1
    ws = torch.zeros(sa.sa_route_workspace_bytes(B, T, H, ss, "pad"), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_route(q, k, ss, 0.2, 1, video_tail_mode="pad", workspace=ws)
    torch.cuda.synchronize()
    ntq, ntk = -(-nvq // 16), -(-nvb // 16)
    nq, nk = B * H * ntq * 16 * 128, B * H * ntk * 16 * 128
    raw = ws.cpu()
    qt = raw[: 8 * nq].view(torch.float64).numpy().reshape(B, H, ntq, 16, 64, 2)
    kt = raw[8 * nq: 8 * nq + 4 * nk].view(torch.float32).numpy().reshape(B, H, ntk, 8, 64, 4)
    d = np.arange(128)[None, :]
    iq = np.arange(nvq)[:, None]
    ik = np.arange(nvb)[:, None]
    qm = qt[:, :, iq // 16, (d % 32) // 2, 16 * (d // 32) + iq % 16, d % 2]
    km = kt[:, :, ik // 16, (d % 32) // 4, 16 * (d // 32) + ik % 16, d % 4]
    qo = ora.pool_means(to_np(wl.q), nvq, end=ss)
    assert np.array_equal(qm.astype(np.float32).view(np.uint32), qo.view(np.uint32))
    assert np.array_equal(km.view(np.uint32), ora.pool_means(to_np(wl.k), nvb).view(np.uint32))


def _tied_keys(nvb, copies, seed):
    """K whose blocks in `copies` repeat block 0 token for token: their pooled
    means, hence their scores against every query block, are bit-identical."""
    q, k, v = workloads.random_qkv(1, 64 * nvb, 2, seed=seed)
    k = k.clone()
    for j in copies:
        k[:, 64 * j:64 * j + 64] = k[:, 0:64]
    return q, k, v


@pytest.mark.parametrize("nvb,ratio,radius,copies", [
    (20, 0.25, 0, range(20)),             # all scores equal, small budget
    (20, 0.6, 1, range(0, 20, 2)),        # half the blocks tied
    (80, 0.5, 0, range(80)),              # budget 40: the large-budget selection path
    (80, 0.6, 1, range(3, 80, 3)),
])
def test_exact_ties_break_to_lower_index(nvb, ratio, radius, copies):
    """Exactly equal scores: the lower block index wins, on both selection
    paths (small and large budgets).  No near-tie leniency here."""
    import block_sparse_attention_05_amd as sa
    q, k, v = _tied_keys(nvb, copies, seed=30 + nvb)
    qn, kn = to_np(q), to_np(k)
    rt = ora.route(qn, kn, 64 * nvb, ratio, radius)
    idx, cnt = sa.sparse_attn_route(q.cuda(), k.cuda(), 64 * nvb, ratio, radius)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for h in range(2):
        for i in range(nvb):
            assert idx[0, h, i, :cnt[0, h, i]].tolist() == rt.rows[0][h][i].blocks, (h, i)


def test_no_video_blocks_all_dense():
    q, k, v = workloads.random_qkv(1, 700, 2, seed=9)
    wl = workloads.Workload("all_dense", q, k, v, sink_start=40, topk_ratio=0.1, local_radius=1)
    full_parity(wl)


def test_single_video_block():
    q, k, v = workloads.random_qkv(1, 200, 2, seed=10)
    wl = workloads.Workload("one_block", q, k, v, sink_start=100, topk_ratio=0.1, local_radius=0)
    full_parity(wl)


def test_ratio_one_is_dense_and_matches_oracle():
    q, k, v = workloads.random_qkv(1, 1000, 2, seed=11)
    wl = workloads.Workload("ratio_one", q, k, v, sink_start=900, topk_ratio=1.0, local_radius=0)
    full_parity(wl)


def test_ratio_one_sparse_bit_identical_to_dense_kernel():
    """At ratio 1.0 every list is all blocks in ascending order: the sparse
    path must reproduce the dense path bit for bit (same kernel, same tile
    order)."""
    import block_sparse_attention_05_amd as sa
    q, k, v = (x.cuda() for x in workloads.random_qkv(1, 1088, 2, seed=12))
    T = q.shape[1]
    idx, cnt = sa.sparse_attn_route(q, k, T, 1.0, 0)
    a = sa.sparse_attn_fwd(q, k, v, T, idx, cnt)
    b = sa.dense_sink_fwd(q, k, v, 0, workspace=None)   # NVB = 0: all rows dense, no key split
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dense_split_and_unsplit_agree_with_oracle():
    """The dense rows with and without the split-KV workspace."""
    import block_sparse_attention_05_amd as sa
    wl = workloads.mid()
    q, k, v = (x.cuda() for x in (wl.q, wl.k, wl.v))
    T = q.shape[1]
    bias = workloads.sink_key_bias(1, T, wl.sink_start, seed=3)
    assert sa.sa_dense_workspace_bytes(1, T, 8, wl.sink_start) > 0
    a = sa.dense_sink_fwd(q, k, v, wl.sink_start, key_bias=bias.cuda())
    b = sa.dense_sink_fwd(q, k, v, wl.sink_start, key_bias=bias.cuda(), workspace=None)
    torch.cuda.synchronize()
    rows = np.arange(wl.sink_start, T)
    qn, kn, vn = (to_np(x) for x in (wl.q, wl.k, wl.v))
    for h in (0, 5):
        want, _ = ora.dense_rows_output(qn, kn, vn, 0, h, rows, bias.numpy(), wl.sink_start // 64)
        for got in (a, b):
            mx, mean = err_stats(to_np(got[0, wl.sink_start:, h]), want)
            log(f"[dense split/unsplit] h={h} max_abs={mx:.3e} mean_abs={mean:.3e}")
            assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_dense_rows_odd_block_count_batch2():
    """Seven dense query blocks per head (odd: the last pair of every head
    has no block B) and five heads, batch 2.  Every dense row of every head
    and batch, out and LSE, with and without the split-KV workspace."""
    import block_sparse_attention_05_amd as sa
    B, T, H, ss = 2, 1000, 5, 576
    assert (sa.sa_num_blocks(T) - ss // 64) % 2 == 1
    q, k, v = (x.cuda() for x in workloads.random_qkv(B, T, H, seed=41))
    bias = workloads.sink_key_bias(B, T, ss, seed=42)
    assert sa.sa_dense_workspace_bytes(B, T, H, ss) > 0
    lse_a = torch.full((B, H, T), float("nan"), device="cuda")
    lse_b = torch.full((B, H, T), float("nan"), device="cuda")
    a = sa.dense_sink_fwd(q, k, v, ss, key_bias=bias.cuda(), lse=lse_a)
    b = sa.dense_sink_fwd(q, k, v, ss, key_bias=bias.cuda(), lse=lse_b, workspace=None)
    torch.cuda.synchronize()
    rows = np.arange(ss, T)
    qn, kn, vn = (to_np(x) for x in (q, k, v))
    for bb in range(B):
        for h in range(H):
            want, want_lse = ora.dense_rows_output(qn, kn, vn, bb, h, rows, bias.numpy(), ss // 64)
            for got, gl in ((a, lse_a), (b, lse_b)):
                mx, mean = err_stats(to_np(got[bb, ss:, h]), want)
                lmx, _ = err_stats(to_np(gl[bb, h, ss:]), want_lse)
                assert mx <= MAX_ABS and mean <= MEAN_ABS, (bb, h, mx, mean)
                assert lmx <= 1e-2, (bb, h, lmx)
    log(f"[dense odd blocks, B{B} H{H}] every row within tolerance, split and unsplit")


def test_zero_bias_bit_identical_to_no_bias():
    wl = workloads.mid()
    a = run_gpu(wl, scores=False)
    b = run_gpu(wl, key_bias=torch.zeros(1, wl.q.shape[1]), scores=False)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])


def test_bias_changes_output_and_only_on_sinks():
    """A sink-key bias changes the output.  A bias on a routed (video) key
    breaks the pages' precondition: the binding rejects it before anything
    runs, and with the check switched off the library ignores it (only the
    exact sink branch reads the bias)."""
    import block_sparse_attention_05_amd as sa
    wl = workloads.mid()
    T = wl.q.shape[1]
    a = run_gpu(wl, scores=False)
    bias = workloads.sink_key_bias(1, T, wl.sink_start, seed=3)
    b = run_gpu(wl, key_bias=bias, scores=False)
    assert (a["out"].float() - b["out"].float()).abs().max() > 1e-3
    video_bias = bias.clone()
    video_bias[:, :wl.sink_start] = -1.0
    with pytest.raises(ValueError, match="sink blocks"):
        run_gpu(wl, key_bias=video_bias, scores=False)
    q, k, v = (x.cuda() for x in (wl.q, wl.k, wl.v))
    with pytest.raises(ValueError, match="sink blocks"):
        sa.routed_attention(q, k, v, wl.sink_start, wl.topk_ratio, wl.local_radius,
                            key_bias=video_bias.cuda())
    c = run_gpu(wl, key_bias=video_bias, scores=False, check_bias=False)
    assert torch.equal(b["out"], c["out"]) and torch.equal(b["lse"], c["lse"])


def test_deterministic_repeat():
    wl = workloads.mid()
    a = run_gpu(wl)
    b = run_gpu(wl)
    for key in ("out", "lse", "idx", "cnt", "scores"):
        assert torch.equal(a[key], b[key]), key


def test_pooled_means_bit_exact():
    import block_sparse_attention_05_amd as sa
    wl = workloads.mid()
    q, k = wl.q.cuda(), wl.k.cuda()
    B, T, H, _ = q.shape
    ws = torch.zeros(sa.sa_route_workspace_bytes(B, T, H, wl.sink_start), dtype=torch.uint8, device="cuda")
    sa.sparse_attn_route(q, k, wl.sink_start, 0.1, 1, workspace=ws)
    torch.cuda.synchronize()
    nvb = wl.sink_start // 64
    nt = -(-nvb // 16)
    n = B * H * nt * 16 * 128
    raw = ws.cpu()
    # operand order of the route kernel: tile of 16 blocks, step st = d % 32,
    # lane 16*(d // 32) + block % 16; q pieces hold 2 steps, k pieces 4
    qt = raw[: 8 * n].view(torch.float64).numpy().reshape(B, H, nt, 16, 64, 2)
    kt = raw[8 * n: 12 * n].view(torch.float32).numpy().reshape(B, H, nt, 8, 64, 4)
    i = np.arange(nvb)[:, None]
    d = np.arange(128)[None, :]
    lane = 16 * (d // 32) + i % 16
    qm = qt[:, :, i // 16, (d % 32) // 2, lane, d % 2]
    km = kt[:, :, i // 16, (d % 32) // 4, lane, d % 4]
    qo = ora.pool_means(to_np(wl.q), nvb)
    assert np.array_equal(qm, qo.astype(np.float64))       # fp64 copies of the fp32 means
    assert np.array_equal(qm.astype(np.float32).view(np.uint32), qo.view(np.uint32))
    assert np.array_equal(km.view(np.uint32), ora.pool_means(to_np(wl.k), nvb).view(np.uint32))


# ---- full-size workloads: every list, every output and LSE element --------

def test_h3_full():
    full_parity(workloads.h3())


def test_h3_keybias_full():
    full_parity(workloads.h3(with_bias=True))


def test_long_full():
    full_parity(workloads.long())


def test_max_route_blocks_full():
    """NVB = 1024 (the widest route row): lists of 110 entries, walked in two
    chunks."""
    full_parity(workloads.max_blocks())


def test_h3_deterministic_repeat():
    """Full-size call repeated: outputs, LSE and lists must be bit-identical
    (catches races between tile loads and LDS reads)."""
    wl = workloads.h3(with_bias=True)
    runs = [run_gpu(wl, scores=False) for _ in range(3)]
    for r in runs[1:]:
        for key in ("out", "lse", "idx", "cnt"):
            assert torch.equal(runs[0][key], r[key]), key


def test_h3_dense_stream_overlap_bit_identical():
    """Dense rows on a second stream, concurrent with routing and the sparse
    rows (the schedule the benchmark times): the same bits as one stream."""
    import block_sparse_attention_05_amd as sa
    wl = workloads.h3(with_bias=True)
    q, k, v, kb = wl.q.cuda(), wl.k.cuda(), wl.v.cuda(), wl.key_bias.cuda()
    args = (q, k, v, wl.sink_start, wl.topk_ratio, wl.local_radius)
    ref_out, ref_lse = sa.routed_attention(*args, key_bias=kb, return_lse=True)
    side = torch.cuda.Stream()
    for _ in range(3):
        out, lse = sa.routed_attention(*args, key_bias=kb, return_lse=True, dense_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)


def test_h3_graph_capture_replays_match_eager():
    """The whole call (route, sparse rows, dense rows on a forked stream)
    captured in one HIP graph.  The library records no memset and allocates
    nothing, so every replay must give the eager call's bits; the outputs are
    cleared by eager kernels, with synchronisations, between replays."""
    import block_sparse_attention_05_amd as sa
    wl = workloads.h3(with_bias=True)
    dev = torch.device("cuda:0")
    q, k, v, kb = (x.to(dev) for x in (wl.q, wl.k, wl.v, wl.key_bias))
    B, T, H, _ = q.shape
    ss, ratio, radius = wl.sink_start, wl.topk_ratio, wl.local_radius
    nvb = sa.sa_num_sparse_blocks(T, ss)
    max_sel = sa.sa_max_selected(T, ss, ratio, radius)
    idx = torch.empty((B, H, nvb, max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, nvb), dtype=torch.int32, device=dev)
    ws = torch.empty(sa.sa_route_workspace_bytes(B, T, H, ss), dtype=torch.uint8, device=dev)
    dws = torch.empty(sa.sa_dense_workspace_bytes(B, T, H, ss), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(dev)

    sa.check_key_bias(kb, B, T, ss)     # once, eagerly: no host sync inside the graph

    def call():
        cur = torch.cuda.current_stream(dev)
        side.wait_stream(cur)
        sa.sparse_attn_route(q, k, ss, ratio, radius, block_idx=idx, block_cnt=cnt, workspace=ws)
        with torch.cuda.stream(side):
            sa.dense_sink_fwd(q, k, v, ss, key_bias=kb, out=out, lse=lse, workspace=dws, check_bias=False)
        sa.sparse_attn_fwd(q, k, v, ss, idx, cnt, key_bias=kb, out=out, lse=lse, check_bias=False)
        cur.wait_stream(side)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, idx, cnt)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (out, lse, idx, cnt):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "idx", "cnt"), (out, lse, idx, cnt), ref):
            assert torch.equal(got, want), (rep, name)
        log(f"[graph] replay {rep} equals the eager call")


def test_pad_batch2_radius2_with_bias():
    # B = 2: both batch elements share sink_start (split at 40 rows of block 15)
    q, k, v = workloads.random_qkv(2, 1100, 3, seed=17)
    bias = workloads.sink_key_bias(2, 1100, 1000, seed=18)
    wl = workloads.Workload("pad_B2_H3_r2", q, k, v, sink_start=1000, topk_ratio=0.3, local_radius=2,
                            key_bias=bias, tail_mode="pad")
    full_parity(wl)


def _mid_lists():
    import block_sparse_attention_05_amd as sa
    wl = workloads.mid()
    q, k, v = (x.cuda() for x in (wl.q, wl.k, wl.v))
    idx, cnt = sa.sparse_attn_route(q, k, wl.sink_start, wl.topk_ratio, wl.local_radius)
    return sa, wl, q, k, v, idx, cnt


def test_invalid_entries_are_skipped():
    """Entries outside [0, NB) are skipped and counts above max_sel are
    clamped: lists padded with -7, -1 in front and NB, NB + 3 and 1 << 30
    behind give the same bits as the plain lists (paired kernel)."""
    sa, wl, q, k, v, idx, cnt = _mid_lists()
    T = q.shape[1]
    nb = -(-T // 64)
    ss = wl.sink_start
    ref = sa.sparse_attn_fwd(q, k, v, ss, idx, cnt)
    wide, wcnt = pad_lists(idx, cnt, [-7, -1], [nb, nb + 3, 1 << 30], idx.shape[-1] + 5)
    got = sa.sparse_attn_fwd(q, k, v, ss, wide, wcnt)
    # counts past max_sel: the clamped list is the whole padded row
    got2 = sa.sparse_attn_fwd(q, k, v, ss, wide, torch.full_like(wcnt, 1 << 20))
    torch.cuda.synchronize()
    rows = slice(0, ss)
    assert torch.equal(got[:, rows], ref[:, rows])
    assert torch.equal(got2[:, rows], ref[:, rows])


def test_invalid_entries_are_skipped_long_lists():
    """Lists wider than the paired kernel's 512 entries take the one-block
    kernel: 300 negative entries in front (the first tile past the first
    64-entry chunk) and NB, NB + 1 behind give the same bits as the same
    width without them."""
    sa, wl, q, k, v, idx, cnt = _mid_lists()
    T = q.shape[1]
    nb = -(-T // 64)
    ss = wl.sink_start
    width = 520
    plain, pcnt = pad_lists(idx, cnt, [], [], width)
    ref = sa.sparse_attn_fwd(q, k, v, ss, plain, pcnt)
    front = list(range(-300, 0))
    wide, wcnt = pad_lists(idx, cnt, front, [nb, nb + 1], width)
    got = sa.sparse_attn_fwd(q, k, v, ss, wide, wcnt)
    torch.cuda.synchronize()
    rows = slice(0, ss)
    assert torch.equal(got[:, rows], ref[:, rows])
    # and the one-block kernel agrees with the paired one within rounding
    pair = sa.sparse_attn_fwd(q, k, v, ss, idx, cnt)
    torch.cuda.synchronize()
    err = (got[:, rows].float() - pair[:, rows].float()).abs().max().item()
    assert err <= 2e-2, err


def test_unsorted_lists_stay_in_bounds():
    """Lists outside the contract (not ascending, repeated entries) give
    unspecified values but must not disturb anything else: the workgroups
    whose two lists are ascending give the same bits, the others finite
    values."""
    sa, wl, q, k, v, idx, cnt = _mid_lists()
    ss = wl.sink_start
    ref = sa.sparse_attn_fwd(q, k, v, ss, idx, cnt)
    bad = idx.clone()
    # head 0: query block 4 reversed, block 9 with a repeated first entry
    c4, c9 = int(cnt[0, 0, 4]), int(cnt[0, 0, 9])
    bad[0, 0, 4, :c4] = idx[0, 0, 4, :c4].flip(0)
    bad[0, 0, 9, 1] = idx[0, 0, 9, 0]
    got = sa.sparse_attn_fwd(q, k, v, ss, bad, cnt)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    same = torch.ones(q.shape[2], ss // 64, dtype=torch.bool)
    same[0, 4:6] = False   # the pair of block 4
    same[0, 8:10] = False  # the pair of block 9
    for h in range(q.shape[2]):
        for i in range(ss // 64):
            if same[h, i]:
                r = slice(64 * i, 64 * i + 64)
                assert torch.equal(got[0, r, h], ref[0, r, h]), (h, i)
