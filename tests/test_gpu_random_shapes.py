"""Seeded random shapes through the whole call against the oracle (needs a
GPU): batch 1-2, 1-4 heads, 600-3100 tokens, a video boundary anywhere
(block-aligned or splitting a block, or no context at all), Top-K ratio
0.05-0.5, radius 0-2, with and without key_bias, both video tail modes.
Q and K at scale 0.5-2 (flat to peaked softmax), V at unit scale.  Every
list is checked (tie band), every element of out and LSE compared."""
import random

import pytest
import torch

import workloads
from gpu_helpers import full_parity, log

pytestmark = pytest.mark.gpu


def _case(seed):
    r = random.Random(seed)
    B = r.choice([1, 1, 2])
    H = r.randint(1, 4)
    T = r.randint(600, 3100)
    kind = r.choice(["aligned", "split", "split", "no_context"])
    if kind == "no_context":
        ss = T
    else:
        nvb = r.randint(1, T // 64 - 1)
        ss = 64 * nvb + (r.randint(1, 63) if kind == "split" else 0)
        ss = min(ss, T - 1)
    ratio = r.choice([0.05, 0.1, 0.2, 0.35, 0.5])
    radius = r.choice([0, 0, 1, 2])
    mode = r.choice(["dense", "pad"])
    # Q/K scale sets how peaked the softmax is; V stays N(0,1) so outputs keep
    # the unit scale the tolerance is stated for
    q, k, _ = workloads.random_qkv(B, T, H, seed=1000 + seed, scale=r.choice([0.5, 1.0, 2.0]))
    _, _, v = workloads.random_qkv(B, T, H, seed=3000 + seed)
    bias = workloads.sink_key_bias(B, T, ss, seed=2000 + seed) if (ss < T and r.random() < 0.5) else None
    wl = workloads.Workload(f"random_{seed}_B{B}_H{H}_T{T}_ss{ss}_{mode}", q, k, v, sink_start=ss,
                            topk_ratio=ratio, local_radius=radius, key_bias=bias, tail_mode=mode)
    return wl


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_against_oracle(seed):
    wl = _case(seed)
    log(f"[{wl.name}] ratio {wl.topk_ratio} radius {wl.local_radius} bias {wl.key_bias is not None}")
    full_parity(wl)
