"""sparse_attn_route_noalloc (pooled means in the library's static device
scratch) against sparse_attn_route with a caller workspace, both called
through the raw C ABI on the same stream: three calls in a row, each smaller
than the one before, and each must give the same lists, counts and route
scores bit for bit (integer outputs, and fp32 scores from the same kernels).
"""
import ctypes

import pytest
import torch

import workloads
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(L, wl, mode):
    dev = torch.device("cuda:0")
    q, k = wl.q.to(dev), wl.k.to(dev)
    B, T, H, D = q.shape
    ss = wl.sink_start
    nvb = L.sa_num_sparse_blocks(T, ss)
    nvq = L.sa_num_query_blocks(T, ss, mode)
    max_sel = L.sa_max_selected(T, ss, mode, wl.topk_ratio, wl.local_radius)
    outs = []
    for _ in range(2):
        outs.append((torch.full((B, H, nvq, max_sel), -7, dtype=torch.int32, device=dev),
                     torch.full((B, H, nvq), -7, dtype=torch.int32, device=dev),
                     torch.full((B, H, nvq, nvb), float("nan"), device=dev)))
    ws_bytes = L.sa_route_workspace_bytes(B, T, H, ss, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    (ia, ca, sa_), (ib, cb, sb) = outs
    args = (_p(q), _p(k), B, T, H, D, ss, T - ss, mode, ctypes.c_float(wl.topk_ratio), wl.local_radius)
    assert L.sparse_attn_route(*args, _p(ia), max_sel, _p(ca), _p(sa_), _p(ws), ws_bytes, stream) == 0
    rc = L.sparse_attn_route_noalloc(*args, _p(ib), max_sel, _p(cb), _p(sb), stream)
    assert rc == 0, L.sa_last_error().decode()
    torch.cuda.synchronize()
    log(f"[noalloc {wl.name}] means {ws_bytes} B: lists equal {torch.equal(ia, ib)}, "
        f"scores equal {torch.equal(sa_, sb)}")
    assert torch.equal(ia, ib) and torch.equal(ca, cb)
    assert torch.equal(sa_.view(torch.int32), sb.view(torch.int32))
    assert int((ca >= 0).sum()) == B * H * nvq
    return ws_bytes


def test_route_noalloc_matches_route_on_calls_of_shrinking_size():
    from block_sparse_attention_05_amd import _lib
    L = _lib.lib()
    q, k, v, tv = workloads.video_qkv(B=1, H=3, frames=2, ctx_tokens=150, seed=7, height=16, width=32)
    pad = workloads.Workload("split_pad", q, k, v, sink_start=tv - 17, topk_ratio=0.2,
                             local_radius=1, tail_mode="pad")
    sizes = [_both(L, workloads.h3(), 0), _both(L, workloads.mid(), 0), _both(L, pad, 1)]
    assert sizes[0] > sizes[1] > sizes[2] > 0
