"""The benchmark's host-side pieces (CPU): the one-GPU guard and the
effective-FLOP count the headline divides by."""
import os
import subprocess
import sys

import numpy as np
import torch

import oracle.sparse_attention as ora
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _lists_as_arrays(rt, B, H):
    ms = max(len(rt.rows[b][h][i].blocks) for b in range(B) for h in range(H) for i in range(rt.nvq))
    idx = np.full((B, H, rt.nvq, ms), -1, dtype=np.int32)
    cnt = np.zeros((B, H, rt.nvq), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(rt.nvq):
                bl = list(rt.rows[b][h][i].blocks)
                idx[b, h, i, :len(bl)] = bl
                cnt[b, h, i] = len(bl)
    return torch.from_numpy(idx), torch.from_numpy(cnt)


def test_effective_flops_match_the_oracle_count():
    """Sparse plus dense effective FLOPs from the lists (partial last block
    counted by its real keys) equal the oracle's definition."""
    q, k, v, tv = workloads.video_qkv(B=1, H=2, frames=2, ctx_tokens=150, seed=7, height=16, width=32)
    B, T, H, _ = q.shape
    rt = ora.route(q.float().numpy(), k.float().numpy(), tv, 0.2, 1)
    idx, cnt = _lists_as_arrays(rt, B, H)
    sp, dn = bench.effective_flops_from_lists(cnt, idx, T, rt.nvb, H, B)
    want = ora.effective_flops(T, H, B, rt.lists(), rt.nvb)
    assert sp + dn == want
    # the dense part is every key for every context row
    assert dn == 4 * 128 * B * H * (T - 64 * rt.nvb) * T
