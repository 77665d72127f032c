"""ctypes binding of libsparse_attn.so (include/sparse_attn.h).

Argument marshalling only: tensors supply device pointers and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

# SA_LIBRARY selects another build of the same library (the sanitizer
# build of the host validation tests); by default the in-tree one.
LIB_PATH = os.environ.get("SA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libsparse_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
HEAD_DIM = 128
BLOCK = 64
# video tail modes: where the real rows of a video block split by the video
# boundary are computed (dense path, or routed and sparse)
VIDEO_TAIL_MODES = {"dense": 0, "pad": 1}

_lib = None

_c_int32, _c_int64, _c_size, _c_float, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                               ctypes.c_float, ctypes.c_void_p)

SIGNATURES = {
    "sa_num_blocks": (_c_int32, [_c_int32]),
    "sa_num_sparse_blocks": (_c_int32, [_c_int32, _c_int32]),
    "sa_num_query_blocks": (_c_int32, [_c_int32, _c_int32, _c_int32]),
    "sa_topk_budget": (_c_int32, [_c_int32, _c_float]),
    "sa_max_selected": (_c_int32, [_c_int32, _c_int32, _c_int32, _c_float, _c_int32]),
    "sa_route_workspace_bytes": (_c_size, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32]),
    "sa_dense_workspace_bytes": (_c_size, [_c_int32, _c_int32, _c_int32, _c_int32]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_device_info": (ctypes.c_int, [_c_int32, _vp, _vp]),
    "sparse_attn_route": (ctypes.c_int, [
        _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
        _c_float, _c_int32, _vp, _c_int32, _vp, _vp, _vp, _c_size, _vp]),
    "sparse_attn_route_noalloc": (ctypes.c_int, [
        _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
        _c_float, _c_int32, _vp, _c_int32, _vp, _vp, _vp]),
    "sparse_attn_fwd": (ctypes.c_int, [
        _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
        _vp, _c_int64, _vp, _vp, _c_int32, _c_float, _vp, _vp, _vp]),
    "dense_sink_fwd": (ctypes.c_int, [
        _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
        _vp, _c_int64, _c_float, _vp, _vp, _vp, _c_size, _vp]),
    "sparse_attn_pool": (ctypes.c_int, [
        _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _vp, _c_size, _vp]),
    "sparse_attn_fwd_fused": (ctypes.c_int, [
        _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
        _c_float, _c_int32, _vp, _c_int64, _vp, _c_size, _c_float, _vp, _vp, _vp, _c_int32, _vp, _vp]),
    "sa_anchor_workspace_bytes": (_c_size, [_c_int32, _c_int32, _c_int32, _c_int32]),
    "spark_global_anchor": (ctypes.c_int, [
        _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _vp, _vp, _c_size, _vp]),
    "spark_reweight": (ctypes.c_int, [
        _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_float, _c_int32,
        _vp, _vp, _vp, _vp]),
    "sparse_attn_fwd_spark": (ctypes.c_int, [
        _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
        _vp, _c_int64, _vp, _vp, _c_int32, _vp, _vp, _vp, _c_float, _vp, _vp, _vp]),
}


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_attention_05_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != SA_OK:
        msg = lib().sa_last_error().decode(errors="replace")
        raise SparseAttnError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_qkv(*ts: torch.Tensor):
    ref = ts[0]
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k, v must be bfloat16")
        if not t.is_cuda:
            raise ValueError("q, k, v must be on a GPU device")
        if t.dim() != 4 or t.shape[-1] != HEAD_DIM:
            raise ValueError("q, k, v must be [B, T, H, 128]")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
        if t.shape != ref.shape or t.device != ref.device:
            raise ValueError("q, k, v must share shape and device")


def _mode(video_tail_mode) -> int:
    if video_tail_mode not in VIDEO_TAIL_MODES:
        raise ValueError(f"video_tail_mode must be one of {sorted(VIDEO_TAIL_MODES)}")
    return VIDEO_TAIL_MODES[video_tail_mode]


def check_key_bias(key_bias: torch.Tensor, B: int, T: int, sink_start: int) -> None:
    """Raise ValueError unless ``key_bias`` (B*T values, natural log, read as
    [B, T]) is zero on every key below 64 * (sink_start // 64), i.e. on every key
    of a routed (non-sink) block.  The pages require biased key blocks to be
    sink-routed (page "Add key bias to chunked Sol-Attn producers",
    Contract); the library itself reads the bias only on sink keys.  NaN
    counts as non-zero.  On a GPU tensor this waits for one small reduction
    (a device-to-host copy of one count)."""
    if key_bias.numel() != B * T:
        raise ValueError(f"key_bias must hold exactly B*T = {B * T} elements, got {key_bias.numel()}")
    kb = key_bias.reshape(B, T)
    routed = BLOCK * (int(sink_start) // BLOCK)
    if routed <= 0:
        return
    bad = int(torch.count_nonzero(kb[:, :routed]).item())
    if bad:
        raise ValueError(f"key_bias is non-zero on {bad} key(s) below 64*NVB = {routed}: biased keys "
                         "must lie in sink blocks (pass check_bias=False to have the library "
                         "ignore bias on routed keys instead)")


def _bias(key_bias: Optional[torch.Tensor], B: int, T: int, device, sink_start: int, check: bool):
    """Normalize the natural-log key bias to the float32 [B, T] contract;
    reject a wrong element count, and (``check``) a non-zero bias on a routed
    key, before anything runs."""
    if key_bias is None:
        return None, 0
    if key_bias.numel() != B * T:
        raise ValueError(f"key_bias must hold exactly B*T = {B * T} elements, got {key_bias.numel()}")
    if key_bias.device != device:
        raise ValueError("key_bias must be on the same device as q")
    kb = key_bias.reshape(B, T)
    if kb.dtype != torch.float32 or not kb.is_contiguous():
        kb = kb.to(torch.float32).contiguous()
    if check:
        check_key_bias(kb, B, T, sink_start)
    return kb, kb.numel()


# ---- shape helpers ---------------------------------------------------------

def sa_num_blocks(T: int) -> int:
    return lib().sa_num_blocks(T)


def sa_num_sparse_blocks(T: int, sink_start: int) -> int:
    return lib().sa_num_sparse_blocks(T, sink_start)


def sa_num_query_blocks(T: int, sink_start: int, video_tail_mode: str = "dense") -> int:
    return lib().sa_num_query_blocks(T, sink_start, _mode(video_tail_mode))


def sa_topk_budget(nvb: int, ratio: float) -> int:
    return lib().sa_topk_budget(nvb, ratio)


def sa_max_selected(T: int, sink_start: int, ratio: float, radius: int,
                    video_tail_mode: str = "dense") -> int:
    return lib().sa_max_selected(T, sink_start, _mode(video_tail_mode), ratio, radius)


def sa_route_workspace_bytes(B: int, T: int, H: int, sink_start: int,
                             video_tail_mode: str = "dense") -> int:
    return lib().sa_route_workspace_bytes(B, T, H, sink_start, _mode(video_tail_mode))


def sa_dense_workspace_bytes(B: int, T: int, H: int, sink_start: int) -> int:
    return lib().sa_dense_workspace_bytes(B, T, H, sink_start)


def sa_device_info(device: int = 0):
    """(compute units, peak shader clock in kHz) of a HIP device."""
    cu, clk = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().sa_device_info(int(device), ctypes.byref(cu), ctypes.byref(clk)))
    return cu.value, clk.value


# ---- entry points ----------------------------------------------------------

def sparse_attn_route(q: torch.Tensor, k: torch.Tensor, sink_start: int,
                      topk_ratio: float = 0.1, local_radius: int = 0, *,
                      video_tail_mode: str = "dense",
                      max_sel: Optional[int] = None, block_idx: Optional[torch.Tensor] = None,
                      block_cnt: Optional[torch.Tensor] = None,
                      route_scores: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact block lists of every routed query block.  Returns
    (block_idx int32 [B,H,NVQ,max_sel], block_cnt int32 [B,H,NVQ]);
    ``route_scores`` (fp32 [B,H,NVQ,NVB]) is filled when given.  NVQ is NVB,
    plus the block split by the video boundary in pad mode."""
    _check_qkv(q, k)
    B, T, H, D = q.shape
    L = lib()
    mode = _mode(video_tail_mode)
    nvb = L.sa_num_sparse_blocks(T, sink_start)
    if nvb < 0:
        raise ValueError("sink_start must lie in [0, T]")
    nvq = L.sa_num_query_blocks(T, sink_start, mode)
    if nvq < 0:
        raise ValueError("pad mode needs the context suffix to complete the split video block "
                         "(T >= 64*(NVB+1))")
    need = L.sa_max_selected(T, sink_start, mode, topk_ratio, local_radius)
    if max_sel is None:
        max_sel = max(need, 1)
    dev = q.device
    if block_idx is None:
        block_idx = torch.empty((B, H, nvq, max_sel), dtype=torch.int32, device=dev)
    if block_cnt is None:
        block_cnt = torch.empty((B, H, nvq), dtype=torch.int32, device=dev)
    ws_bytes = L.sa_route_workspace_bytes(B, T, H, sink_start, mode)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    for name, t, dt in (("block_idx", block_idx, torch.int32), ("block_cnt", block_cnt, torch.int32)):
        if t.dtype != dt or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 tensor on {dev}")
    if block_idx.numel() < B * H * nvq * max_sel or block_cnt.numel() < B * H * nvq:
        raise ValueError("block_idx / block_cnt too small")
    if route_scores is not None and (route_scores.dtype != torch.float32 or not route_scores.is_contiguous()
                                     or route_scores.numel() < B * H * nvq * nvb
                                     or route_scores.device != dev):
        raise ValueError("route_scores must be contiguous float32 [B,H,NVQ,NVB] on the device of q")
    _check(L.sparse_attn_route(
        _ptr(q), _ptr(k), B, T, H, D, sink_start, T - sink_start, mode, float(topk_ratio),
        int(local_radius), _ptr(block_idx), int(max_sel), _ptr(block_cnt), _ptr(route_scores),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return block_idx, block_cnt


def sparse_attn_route_noalloc(q: torch.Tensor, k: torch.Tensor, sink_start: int,
                              topk_ratio: float, local_radius: int, block_idx: torch.Tensor,
                              block_cnt: torch.Tensor, *, video_tail_mode: str = "dense",
                              route_scores: Optional[torch.Tensor] = None):
    """sparse_attn_route with the pooled means in the library's static device
    scratch: the caller supplies every output and nothing is allocated (at
    most SA_STATIC_SCRATCH_BYTES of means; calls overlapping on one GPU
    race)."""
    _check_qkv(q, k)
    B, T, H, D = q.shape
    dev = q.device
    for name, t in (("block_idx", block_idx), ("block_cnt", block_cnt)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 tensor on {dev}")
    if route_scores is not None and (route_scores.dtype != torch.float32 or not route_scores.is_contiguous()
                                     or route_scores.device != dev):
        raise ValueError("route_scores must be contiguous float32 on the device of q")
    mode = _mode(video_tail_mode)
    nvq = lib().sa_num_query_blocks(T, sink_start, mode)
    max_sel = block_idx.shape[-1] if block_idx.dim() == 4 else 0
    if nvq > 0 and (block_idx.dim() != 4 or tuple(block_idx.shape[:3]) != (B, H, nvq)
                    or block_cnt.numel() != B * H * nvq):
        raise ValueError("block_idx must be [B,H,NVQ,max_sel] and block_cnt [B,H,NVQ]")
    _check(lib().sparse_attn_route_noalloc(
        _ptr(q), _ptr(k), B, T, H, D, sink_start, T - sink_start, mode, float(topk_ratio),
        int(local_radius), _ptr(block_idx), int(max_sel), _ptr(block_cnt), _ptr(route_scores),
        _stream(dev)))
    return block_idx, block_cnt


def sparse_attn_fwd(q, k, v, sink_start: int, block_idx: torch.Tensor, block_cnt: torch.Tensor, *,
                    video_tail_mode: str = "dense",
                    key_bias: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    check_bias: bool = True):
    """Exact attention of the sparse rows ([0, 64*NVB), or [0, sink_start)
    in pad mode) over their block lists; writes those rows of ``out``
    (allocated if None) and returns it.  ``check_bias``: reject a key_bias
    that is non-zero on a routed key (see ``check_key_bias``; one host
    synchronisation); with False the library ignores such values."""
    _check_qkv(q, k, v)
    B, T, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    if block_idx.dtype != torch.int32 or block_cnt.dtype != torch.int32 or \
            not block_idx.is_contiguous() or not block_cnt.is_contiguous():
        raise ValueError("block_idx / block_cnt must be contiguous int32")
    mode = _mode(video_tail_mode)
    nvq = lib().sa_num_query_blocks(T, sink_start, mode)
    max_sel = block_idx.shape[-1] if block_idx.dim() == 4 else 0
    if nvq > 0 and (block_idx.dim() != 4 or tuple(block_idx.shape[:3]) != (B, H, nvq)
                    or block_cnt.numel() != B * H * nvq):
        raise ValueError("block_idx must be [B,H,NVQ,max_sel] and block_cnt [B,H,NVQ]")
    if block_idx.device != q.device or block_cnt.device != q.device:
        raise ValueError("block_idx / block_cnt must be on the device of q")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * T):
        raise ValueError("lse must be contiguous float32 [B,H,T]")
    kb, kb_n = _bias(key_bias, B, T, q.device, sink_start, check_bias)
    _check(lib().sparse_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), B, T, H, D, sink_start, T - sink_start, mode, _ptr(kb), kb_n,
        _ptr(block_idx), _ptr(block_cnt), int(max_sel), float(softmax_scale), _ptr(out), _ptr(lse),
        _stream(q.device)))
    return out


def dense_sink_fwd(q, k, v, sink_start: int, *, video_tail_mode: str = "dense",
                   key_bias: Optional[torch.Tensor] = None,
                   softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, workspace="auto", check_bias: bool = True):
    """Dense attention of the dense rows ([64*NVB, T), or [sink_start, T) in
    pad mode) over all keys; writes those rows of ``out`` (allocated if
    None) and returns it.  ``workspace``: a uint8 device tensor, None (no
    key split), or "auto" (allocate what the split needs).  ``check_bias``
    as for sparse_attn_fwd."""
    mode = _mode(video_tail_mode)
    _check_qkv(q, k, v)
    B, T, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * T):
        raise ValueError("lse must be contiguous float32 [B,H,T]")
    kb, kb_n = _bias(key_bias, B, T, q.device, sink_start, check_bias)
    if isinstance(workspace, str):
        n = lib().sa_dense_workspace_bytes(B, T, H, sink_start)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dense_sink_fwd(
        _ptr(q), _ptr(k), _ptr(v), B, T, H, D, sink_start, T - sink_start, mode, _ptr(kb), kb_n,
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(q.device)))
    return out


def routed_attention(q, k, v, sink_start: int, topk_ratio: float = 0.1, local_radius: int = 0, *,
                     video_tail_mode: str = "dense",
                     key_bias: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                     return_lse: bool = False, return_route: bool = False,
                     dense_stream: Optional[torch.cuda.Stream] = None, check_bias: bool = True):
    """One full call: sparse_attn_route + sparse_attn_fwd + dense_sink_fwd on
    the current stream.  With ``dense_stream`` (a stream of the same device)
    the dense rows, which need no routing, run there instead, forked from and
    joined back into the current stream; they write rows disjoint from the
    sparse rows', so the result is the same.  The key_bias precondition is
    checked once (``check_bias``)."""
    if key_bias is not None and check_bias:
        check_key_bias(key_bias, q.shape[0], q.shape[1], sink_start)
    cur = torch.cuda.current_stream(q.device)
    if dense_stream is not None:
        dense_stream.wait_stream(cur)
    block_idx, block_cnt = sparse_attn_route(q, k, sink_start, topk_ratio, local_radius,
                                             video_tail_mode=video_tail_mode)
    B, T, H, _ = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    if dense_stream is not None:
        # launched behind the routing kernels so those dispatch first
        with torch.cuda.stream(dense_stream):
            dense_sink_fwd(q, k, v, sink_start, video_tail_mode=video_tail_mode,
                           key_bias=key_bias, softmax_scale=softmax_scale, out=out, lse=lse,
                           check_bias=False)
    sparse_attn_fwd(q, k, v, sink_start, block_idx, block_cnt, video_tail_mode=video_tail_mode,
                    key_bias=key_bias, softmax_scale=softmax_scale, out=out, lse=lse, check_bias=False)
    if dense_stream is None:
        dense_sink_fwd(q, k, v, sink_start, video_tail_mode=video_tail_mode, key_bias=key_bias,
                       softmax_scale=softmax_scale, out=out, lse=lse, check_bias=False)
    else:
        cur.wait_stream(dense_stream)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_route:
        res.append((block_idx, block_cnt))
    return res[0] if len(res) == 1 else tuple(res)


# ---- Spark virtual summaries and the approximate branch --------------------

LOGMASS_KEYS = {"stored": 0, "pre_round": 1}


def sa_anchor_workspace_bytes(B: int, T: int, H: int, sink_start: int) -> int:
    return lib().sa_anchor_workspace_bytes(B, T, H, sink_start)


def spark_global_anchor(q: torch.Tensor, sink_start: int, *, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [B, 1, H, 128]: the mean of the video query rows [0, sink_start)
    of every (batch, head)."""
    _check_qkv(q)
    B, T, H, D = q.shape
    if out is None:
        out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or not out.is_contiguous() or out.numel() != B * H * D \
            or out.device != q.device:
        raise ValueError("out must be contiguous bfloat16 [B, 1, H, 128] on the device of q")
    n = lib().sa_anchor_workspace_bytes(B, T, H, sink_start)
    if workspace is None:
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    _check(lib().spark_global_anchor(
        _ptr(q), B, T, H, D, sink_start, T - sink_start, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out


def spark_reweight(a: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, softmax_scale: float = 0.0,
                   logmass_key: str = "stored", ak: Optional[torch.Tensor] = None,
                   av: Optional[torch.Tensor] = None, lm: Optional[torch.Tensor] = None):
    """Virtual summaries for anchors a [B, P, H, 128]: returns (ak, av bf16
    [B, P, H, NB, 128], lm fp32 [B, P, H, NB])."""
    _check_qkv(k, v)
    B, T, H, D = k.shape
    if a.dtype != torch.bfloat16 or a.dim() != 4 or a.shape[0] != B or a.shape[2] != H \
            or a.shape[3] != D or not a.is_contiguous() or a.device != k.device:
        raise ValueError("a must be contiguous bfloat16 [B, P, H, 128] on the device of k")
    if logmass_key not in LOGMASS_KEYS:
        raise ValueError(f"logmass_key must be one of {sorted(LOGMASS_KEYS)}")
    P = a.shape[1]
    nb = -(-T // BLOCK)
    dev = k.device
    if ak is None:
        ak = torch.empty((B, P, H, nb, D), dtype=torch.bfloat16, device=dev)
    if av is None:
        av = torch.empty((B, P, H, nb, D), dtype=torch.bfloat16, device=dev)
    if lm is None:
        lm = torch.empty((B, P, H, nb), dtype=torch.float32, device=dev)
    for name, t, dt, numel in (("ak", ak, torch.bfloat16, B * P * H * nb * D),
                               ("av", av, torch.bfloat16, B * P * H * nb * D),
                               ("lm", lm, torch.float32, B * P * H * nb)):
        if t.dtype != dt or not t.is_contiguous() or t.numel() != numel or t.device != dev:
            raise ValueError(f"{name} must be a contiguous {dt} tensor of {numel} elements on {dev}")
    _check(lib().spark_reweight(
        _ptr(a), _ptr(k), _ptr(v), B, P, T, H, D, float(softmax_scale), LOGMASS_KEYS[logmass_key],
        _ptr(ak), _ptr(av), _ptr(lm), _stream(dev)))
    return ak, av, lm


def sparse_attn_fwd_spark(q, k, v, sink_start: int, block_idx: torch.Tensor, block_cnt: torch.Tensor,
                          summaries, *, video_tail_mode: str = "dense",
                          key_bias: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          check_bias: bool = True):
    """sparse_attn_fwd plus one virtual key per skipped video block, from
    ``summaries`` = (ak, av, lm) of one anchor per (batch, head).
    ``check_bias`` as for sparse_attn_fwd."""
    _check_qkv(q, k, v)
    B, T, H, D = q.shape
    ak, av, lm = summaries
    nb = -(-T // BLOCK)
    for name, t, dt, numel in (("ak", ak, torch.bfloat16, B * H * nb * D),
                               ("av", av, torch.bfloat16, B * H * nb * D),
                               ("lm", lm, torch.float32, B * H * nb)):
        if t.dtype != dt or not t.is_contiguous() or t.numel() != numel or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous {dt} tensor of one anchor "
                             f"({numel} elements) on the device of q")
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    if block_idx.dtype != torch.int32 or block_cnt.dtype != torch.int32 or \
            not block_idx.is_contiguous() or not block_cnt.is_contiguous():
        raise ValueError("block_idx / block_cnt must be contiguous int32")
    mode = _mode(video_tail_mode)
    nvq = lib().sa_num_query_blocks(T, sink_start, mode)
    max_sel = block_idx.shape[-1] if block_idx.dim() == 4 else 0
    if nvq > 0 and (block_idx.dim() != 4 or tuple(block_idx.shape[:3]) != (B, H, nvq)
                    or block_cnt.numel() != B * H * nvq):
        raise ValueError("block_idx must be [B,H,NVQ,max_sel] and block_cnt [B,H,NVQ]")
    if block_idx.device != q.device or block_cnt.device != q.device:
        raise ValueError("block_idx / block_cnt must be on the device of q")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * T):
        raise ValueError("lse must be contiguous float32 [B,H,T]")
    kb, kb_n = _bias(key_bias, B, T, q.device, sink_start, check_bias)
    _check(lib().sparse_attn_fwd_spark(
        _ptr(q), _ptr(k), _ptr(v), B, T, H, D, sink_start, T - sink_start, mode, _ptr(kb), kb_n,
        _ptr(block_idx), _ptr(block_cnt), int(max_sel), _ptr(ak), _ptr(av), _ptr(lm),
        float(softmax_scale), _ptr(out), _ptr(lse), _stream(q.device)))
    return out


def routed_attention_spark(q, k, v, sink_start: int, topk_ratio: float = 0.1, local_radius: int = 0, *,
                           video_tail_mode: str = "dense", key_bias: Optional[torch.Tensor] = None,
                           softmax_scale: float = 0.0, return_lse: bool = False,
                           return_parts: bool = False, check_bias: bool = True):
    """One call of the Spark path: global anchor, virtual summaries, route,
    sparse rows with the approximate branch, dense rows, on the current
    stream.  The key_bias precondition is checked once (``check_bias``)."""
    if key_bias is not None and check_bias:
        check_key_bias(key_bias, q.shape[0], q.shape[1], sink_start)
    anchor = spark_global_anchor(q, sink_start)
    summaries = spark_reweight(anchor, k, v, softmax_scale=softmax_scale)
    block_idx, block_cnt = sparse_attn_route(q, k, sink_start, topk_ratio, local_radius,
                                             video_tail_mode=video_tail_mode)
    B, T, H, _ = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    sparse_attn_fwd_spark(q, k, v, sink_start, block_idx, block_cnt, summaries,
                          video_tail_mode=video_tail_mode, key_bias=key_bias,
                          softmax_scale=softmax_scale, out=out, lse=lse, check_bias=False)
    dense_sink_fwd(q, k, v, sink_start, video_tail_mode=video_tail_mode, key_bias=key_bias,
                   softmax_scale=softmax_scale, out=out, lse=lse, check_bias=False)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_parts:
        res.append(dict(anchor=anchor, summaries=summaries, block_idx=block_idx, block_cnt=block_cnt))
    return res[0] if len(res) == 1 else tuple(res)


# ---- fused route ------------------------------------------------------------

def sparse_attn_pool(q: torch.Tensor, k: torch.Tensor, sink_start: int, *,
                     video_tail_mode: str = "dense",
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pooled Q and K means into a route workspace (uint8 device tensor,
    allocated if None), which is returned."""
    _check_qkv(q, k)
    B, T, H, D = q.shape
    mode = _mode(video_tail_mode)
    n = lib().sa_route_workspace_bytes(B, T, H, sink_start, mode)
    if workspace is None:
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    _check(lib().sparse_attn_pool(_ptr(q), _ptr(k), B, T, H, D, sink_start, T - sink_start, mode,
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(q.device)))
    return workspace


def sparse_attn_fwd_fused(q, k, v, sink_start: int, topk_ratio: float, local_radius: int,
                          workspace: torch.Tensor, *, video_tail_mode: str = "dense",
                          key_bias: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_route: bool = False, check_bias: bool = True):
    """Sparse rows with the route inside the attention kernel, from the
    pooled means in ``workspace`` (see sparse_attn_pool).  With
    ``return_route`` the selected lists are returned too.  ``check_bias`` as
    for sparse_attn_fwd."""
    _check_qkv(q, k, v)
    B, T, H, D = q.shape
    mode = _mode(video_tail_mode)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * T):
        raise ValueError("lse must be contiguous float32 [B,H,T]")
    if workspace.device != q.device:
        raise ValueError("workspace must be on the device of q")
    kb, kb_n = _bias(key_bias, B, T, q.device, sink_start, check_bias)
    idx = cnt = None
    max_sel = 0
    if return_route:
        nvq = lib().sa_num_query_blocks(T, sink_start, mode)
        max_sel = max(1, lib().sa_max_selected(T, sink_start, mode, topk_ratio, local_radius))
        idx = torch.empty((B, H, max(nvq, 0), max_sel), dtype=torch.int32, device=q.device)
        cnt = torch.empty((B, H, max(nvq, 0)), dtype=torch.int32, device=q.device)
    _check(lib().sparse_attn_fwd_fused(
        _ptr(q), _ptr(k), _ptr(v), B, T, H, D, sink_start, T - sink_start, mode, float(topk_ratio),
        int(local_radius), _ptr(kb), kb_n, _ptr(workspace), workspace.numel() * workspace.element_size(),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(idx), int(max_sel), _ptr(cnt), _stream(q.device)))
    return (out, (idx, cnt)) if return_route else out


def routed_attention_fused(q, k, v, sink_start: int, topk_ratio: float = 0.1, local_radius: int = 0, *,
                           video_tail_mode: str = "dense", key_bias: Optional[torch.Tensor] = None,
                           softmax_scale: float = 0.0, return_lse: bool = False,
                           return_route: bool = False, check_bias: bool = True):
    """One call with the route fused into attention: pool, fused sparse rows,
    dense rows, on the current stream.  The key_bias precondition is checked
    once (``check_bias``)."""
    if key_bias is not None and check_bias:
        check_key_bias(key_bias, q.shape[0], q.shape[1], sink_start)
    ws = sparse_attn_pool(q, k, sink_start, video_tail_mode=video_tail_mode)
    B, T, H, _ = q.shape
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    out = torch.empty_like(q)
    r = sparse_attn_fwd_fused(q, k, v, sink_start, topk_ratio, local_radius, ws,
                              video_tail_mode=video_tail_mode, key_bias=key_bias,
                              softmax_scale=softmax_scale, out=out, lse=lse, return_route=return_route,
                              check_bias=False)
    dense_sink_fwd(q, k, v, sink_start, video_tail_mode=video_tail_mode, key_bias=key_bias,
                   softmax_scale=softmax_scale, out=out, lse=lse, check_bias=False)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_route:
        res.append(r[1])
    return res[0] if len(res) == 1 else tuple(res)
