"""Plant a plausible mistake in the oracle (on the CPU) and require that at
least one pin fails.  Shows that the pins would catch a dropped term, a wrong
sign, index or operand in each oracle function."""
import math

import numpy as np
import pytest

import oracle.sparse_attention as ra
import oracle.spark_summaries as sp
import oracle_checks as oc

_orig = {name: getattr(ra, name) for name in (
    "pool_means", "route_scores", "topk_budget", "select_row", "attend",
    "key_bias_vector", "sparse_block_output", "dense_rows_output", "forced_blocks",
    "route", "pad_query_block", "sparse_rows_end", "list_accepted")}


def pool_63(x, nvb, end=None):            # off-by-one block length
    out = _orig["pool_means"](x, nvb, end)
    x64 = np.asarray(x, np.float64)
    for i in range(nvb):
        out[:, :, i] = (x64[:, i * 64:i * 64 + 63].sum(1) / 64).astype(np.float32)
    return out


def pool_f32_sum(x, nvb, end=None):        # accumulates in fp32 in token order
    B, T, H, D = x.shape
    out = np.zeros((B, H, nvb, D), np.float32)
    for i in range(nvb):
        acc = np.zeros((B, H, D), np.float32)
        for t in range(i * 64, i * 64 + 64):
            acc = acc + np.asarray(x[:, t], np.float32)
        out[:, :, i] = acc / np.float32(64)
    return out


def scores_transposed(qbar, kbar):
    return np.swapaxes(_orig["route_scores"](qbar, kbar), -1, -2).copy()


def scores_bf16(qbar, kbar):
    import torch
    r = lambda a: torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    return _orig["route_scores"](r(qbar), r(kbar))


def budget_floor(nvb, ratio):
    if nvb <= 0:
        return 0
    return max(1, int(math.floor(float(np.float32(ratio)) * nvb)))


def select_ascending(scores_row, i, nvb, nb, budget, radius):
    return _orig["select_row"](-np.asarray(scores_row, np.float32), i, nvb, nb, budget, radius)


def select_tie_high_index(scores_row, i, nvb, nb, budget, radius):
    forced = ra.forced_blocks(i, nvb, radius)
    cand = np.array([j for j in range(nvb) if j not in forced], np.int64)
    k = min(budget, len(cand))
    s = np.asarray(scores_row, np.float32)[cand]
    order = np.lexsort((-cand, -s.astype(np.float64)))
    routed = sorted(int(j) for j in cand[order[:k]])
    sel = _orig["select_row"](scores_row, i, nvb, nb, budget, radius)
    sel.routed = routed
    sel.blocks = sorted(set(routed) | set(forced) | set(range(nvb, nb)))
    return sel


def select_forced_inside_budget(scores_row, i, nvb, nb, budget, radius):
    s = np.asarray(scores_row, np.float32)
    order = np.lexsort((np.arange(nvb), -s.astype(np.float64)))
    top = sorted(int(j) for j in order[:budget])
    forced = ra.forced_blocks(i, nvb, radius)
    sel = _orig["select_row"](scores_row, i, nvb, nb, budget, radius)
    sel.routed = [j for j in top if j not in forced]
    sel.blocks = sorted(set(top) | set(forced) | set(range(nvb, nb)))
    return sel


def attend_no_scale(qrows, keys, vals, bias, scale):
    return _orig["attend"](qrows, keys, vals, bias, 1.0)


def attend_bias_sign(qrows, keys, vals, bias, scale):
    return _orig["attend"](qrows, keys, vals, None if bias is None else -np.asarray(bias), scale)


def attend_bias_log2(qrows, keys, vals, bias, scale):     # log2 units fed to a natural exp
    return _orig["attend"](qrows, keys, vals, None if bias is None else np.asarray(bias) * math.log2(math.e), scale)


def attend_values_are_keys(qrows, keys, vals, bias, scale):
    return _orig["attend"](qrows, keys, keys, bias, scale)


def bias_on_all_keys(key_bias, b, T, nvb):
    if key_bias is None:
        return None
    return np.asarray(key_bias, np.float64).reshape(-1, T)[b].copy()


def gather_shifted(q, k, v, b, h, i, blocks, key_bias=None, nvb=None, scale=None, qrows=None):
    nb = -(-q.shape[1] // 64)
    return _orig["sparse_block_output"](q, k, v, b, h, i, [min(j + 1, nb - 1) for j in blocks],
                                        key_bias, nvb, scale, qrows)


def dense_without_sinks(q, k, v, b, h, rows, key_bias=None, nvb=0, scale=None):
    T = q.shape[1]
    keys = np.arange(0, max(64 * nvb, 1))
    kb = ra.key_bias_vector(key_bias, b, T, nvb)
    return ra.attend(q[b, rows, h], k[b, keys, h], v[b, keys, h],
                     None if kb is None else kb[keys], 1.0 / math.sqrt(128))


def forced_one_sided(i, nvb, radius):
    return [j for j in range(i, i + radius + 1) if 0 <= j < nvb]


def route_qk_swapped(q, k, sink_start, ratio, radius, tail_mode="dense"):
    return _orig["route"](k, q, sink_start, ratio, radius, tail_mode)


# A positive rescale of one centroid cannot change its row's selection, so
# only the pooling pin can see this one.
def pool_tail_by_64(x, nblocks, end=None):   # split block's sum divided by 64
    out = _orig["pool_means"](x, nblocks, end)
    if end is not None and end < 64 * nblocks:
        i = nblocks - 1
        s = np.asarray(x, np.float64)[:, 64 * i:end].sum(1)
        out[:, :, i] = (s / 64).astype(np.float32)
    return out


def pool_tail_physical(x, nblocks, end=None):  # pools the context rows too
    return _orig["pool_means"](x, nblocks)


def pad_zero_fill(q, b, h, i, sink_start):
    blk = _orig["pad_query_block"](q, b, h, i, sink_start)
    blk[sink_start - 64 * i:] = 0.0
    return blk


def route_without_tail(q, k, sink_start, ratio, radius, tail_mode="dense"):
    return _orig["route"](q, k, sink_start, ratio, radius)


def sparse_end_whole_block(T, sink_start, tail_mode="dense"):
    return -(-_orig["sparse_rows_end"](T, sink_start, tail_mode) // 64) * 64


_sp_orig = {name: getattr(sp, name) for name in (
    "virtual_summaries", "approx_block_output", "global_anchor", "log_mass")}


def log_mass_sign(a, keys, key_for_shift, scale):           # + instead of -
    z = _sp_orig["log_mass"](a, keys, key_for_shift, scale)
    return z + 2 * scale * float(np.dot(np.asarray(a, np.float64), np.asarray(key_for_shift, np.float64)))


def log_mass_unscaled_shift(a, keys, key_for_shift, scale):
    z = _sp_orig["log_mass"](a, keys, key_for_shift, scale)
    return z + (scale - 1.0) * float(np.dot(np.asarray(a, np.float64), np.asarray(key_for_shift, np.float64)))


def summaries_uniform(a, k, v, scale=None, logmass_key="stored", store="bf16"):
    """Plain block means with ln(n) mass: the summary without reweighting."""
    ak, av, lm = _sp_orig["virtual_summaries"](a, k, v, scale, logmass_key, store)
    T = k.shape[1]
    for j in range(ak.shape[3]):
        kk = np.asarray(k, np.float64)[:, 64 * j:min(T, 64 * j + 64)].mean(1)   # [B, H, D]
        vv = np.asarray(v, np.float64)[:, 64 * j:min(T, 64 * j + 64)].mean(1)
        ak[:, :, :, j] = kk[:, None]
        av[:, :, :, j] = vv[:, None]
        lm[:, :, :, j] = math.log(min(T, 64 * j + 64) - 64 * j)
    return ak, av, lm


def summaries_zero_padded(a, k, v, scale=None, logmass_key="stored", store="bf16"):
    """The partial final block padded with zero keys and values."""
    T = k.shape[1]
    pad = (-T) % 64
    z = np.zeros((k.shape[0], pad) + k.shape[2:], np.float32)
    return _sp_orig["virtual_summaries"](a, np.concatenate([k, z], 1), np.concatenate([v, z], 1),
                                         scale, logmass_key, store)


def approx_every_block_virtual(q, k, v, b, h, i, blocks, ak, av, lm, key_bias=None, nvb=0,
                               scale=None, qrows=None):
    """Exact blocks summarised too (their mass counted twice)."""
    T = q.shape[1]
    idx = np.concatenate([np.arange(j * 64, min(j * 64 + 64, T)) for j in blocks])
    kb = ra.key_bias_vector(key_bias, b, T, nvb)
    keys = np.concatenate([k[b, idx, h], ak[b, 0, h, :nvb]])
    vals = np.concatenate([v[b, idx, h], av[b, 0, h, :nvb]])
    bias = np.concatenate([np.zeros(len(idx)) if kb is None else kb[idx], lm[b, 0, h, :nvb]])
    if qrows is None:
        qrows = q[b, i * 64:min(i * 64 + 64, T), h]
    return ra.attend(qrows, keys, vals, bias, 1.0 / math.sqrt(128) if not scale else scale)


def approx_sinks_virtual(q, k, v, b, h, i, blocks, ak, av, lm, key_bias=None, nvb=0, scale=None,
                         qrows=None):
    """Sink blocks summarised instead of exact."""
    nb = -(-q.shape[1] // 64)
    kept = [j for j in blocks if j < nvb]
    return _sp_orig["approx_block_output"](q, k, v, b, h, i, kept, ak, av, lm, key_bias, nb, scale,
                                           qrows)


def approx_no_logmass(q, k, v, b, h, i, blocks, ak, av, lm, key_bias=None, nvb=0, scale=None,
                      qrows=None):
    return _sp_orig["approx_block_output"](q, k, v, b, h, i, blocks, ak, av, np.zeros_like(lm),
                                           key_bias, nvb, scale, qrows)


def approx_keys_as_values(q, k, v, b, h, i, blocks, ak, av, lm, key_bias=None, nvb=0, scale=None,
                          qrows=None):
    return _sp_orig["approx_block_output"](q, k, v, b, h, i, blocks, ak, ak, lm, key_bias, nvb,
                                           scale, qrows)


def anchor_all_rows(q, sink_start):                 # context query rows averaged in
    return _sp_orig["global_anchor"](q, q.shape[1])


def anchor_block_rows(q, sink_start):               # complete video blocks only
    return _sp_orig["global_anchor"](q, sink_start // 64 * 64)


# (oracle function, mutant, the pin expected to catch it)
def accept_any_in_tie_row(got, sel, scores_row, nvb):    # no band check at all
    return list(got) == sel.blocks or sel.near_tie


def accept_band_ignoring_forced(got, sel, scores_row, nvb):
    if list(got) == sel.blocks:
        return True
    lo, hi = sel.band
    return sel.near_tie and len(got) == len(sel.blocks) and list(got) == sorted(set(got)) and all(
        j >= nvb or lo <= float(scores_row[j]) <= hi for j in set(got) ^ set(sel.blocks))


MUTANTS = [
    ("pool_means", pool_63, oc.check_pool_exact),
    ("pool_means", pool_f32_sum, oc.check_pool_exact),
    ("route_scores", scores_transposed, oc.check_scores_exact),
    ("route_scores", scores_bf16, oc.check_scores_exact),
    ("topk_budget", budget_floor, oc.check_budget),
    ("select_row", select_ascending, oc.check_topk_bruteforce),
    ("select_row", select_tie_high_index, oc.check_topk_bruteforce),
    ("select_row", select_tie_high_index, oc.check_signed_zero_tie),
    ("select_row", select_forced_inside_budget, oc.check_topk_bruteforce),
    ("attend", attend_no_scale, oc.check_ratio_one_equals_sdpa),
    ("attend", attend_bias_sign, oc.check_bias_ln_m_duplicates_key),
    ("attend", attend_bias_log2, oc.check_bias_ln_m_duplicates_key),
    ("attend", attend_values_are_keys, oc.check_ratio_one_equals_sdpa),
    ("key_bias_vector", bias_on_all_keys, oc.check_bias_ignored_on_video_keys),
    ("sparse_block_output", gather_shifted, oc.check_token_mask_path),
    ("dense_rows_output", dense_without_sinks, oc.check_all_dense_when_no_video_block),
    ("dense_rows_output", dense_without_sinks, oc.check_ratio_one_equals_sdpa),
    ("forced_blocks", forced_one_sided, oc.check_topk_bruteforce),
    ("forced_blocks", forced_one_sided, oc.check_golden_pages_numbers),
    ("route", route_qk_swapped, oc.check_route_glue),
    ("pool_means", pool_tail_by_64, oc.check_pad_tail_means_exact),
    ("pool_means", pool_tail_physical, oc.check_pad_tail_means_exact),
    ("pad_query_block", pad_zero_fill, oc.check_pad_centroid_preserved),
    ("route", route_without_tail, oc.check_pad_route_and_mask),
    ("sparse_rows_end", sparse_end_whole_block, oc.check_pad_route_and_mask),
    ("sparse_rows_end", sparse_end_whole_block, oc.check_pad_modes_agree_where_they_must),
    ("forced_blocks", forced_one_sided, oc.check_pad_route_and_mask),
    ("list_accepted", accept_any_in_tie_row, oc.check_list_accepted),
    ("list_accepted", accept_band_ignoring_forced, oc.check_list_accepted),
]

SP_MUTANTS = [
    ("log_mass", log_mass_sign, oc.check_summaries_explicit_softmax),
    ("log_mass", log_mass_unscaled_shift, oc.check_summaries_explicit_softmax),
    ("log_mass", log_mass_unscaled_shift, oc.check_spark_anchor_rows_are_exact),
    ("virtual_summaries", summaries_uniform, oc.check_summaries_explicit_softmax),
    ("virtual_summaries", summaries_uniform, oc.check_spark_anchor_rows_are_exact),
    ("virtual_summaries", summaries_zero_padded, oc.check_log_mass_closed_forms),
    ("virtual_summaries", summaries_zero_padded, oc.check_summaries_explicit_softmax),
    ("approx_block_output", approx_every_block_virtual, oc.check_spark_anchor_rows_are_exact),
    ("approx_block_output", approx_every_block_virtual, oc.check_spark_ratio_one_is_exact),
    ("approx_block_output", approx_sinks_virtual, oc.check_spark_anchor_rows_are_exact),
    ("approx_block_output", approx_no_logmass, oc.check_spark_anchor_rows_are_exact),
    ("approx_block_output", approx_keys_as_values, oc.check_spark_anchor_rows_are_exact),
    ("global_anchor", anchor_all_rows, oc.check_anchor_exact),
    ("global_anchor", anchor_block_rows, oc.check_anchor_exact),
]


@pytest.mark.parametrize("name,mutant,check", MUTANTS,
                         ids=[f"{m.__name__}-{c.__name__}" for _, m, c in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, mutant, check):
    check()                                   # passes on the oracle as written
    monkeypatch.setattr(ra, name, mutant)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        check()


@pytest.mark.parametrize("name,mutant,check", SP_MUTANTS,
                         ids=[f"{m.__name__}-{c.__name__}" for _, m, c in SP_MUTANTS])
def test_summary_mutant_is_caught(monkeypatch, name, mutant, check):
    check()
    monkeypatch.setattr(sp, name, mutant)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        check()
