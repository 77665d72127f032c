"""Exact rational arithmetic used to pin the oracle's pooling and scores.

Independent of the oracle: block means and dot products are formed as exact
fractions and rounded once to fp32 (round to nearest, ties to even) by the
integer routine below.
"""
from fractions import Fraction

import numpy as np


def round_fraction_to_f32(x: Fraction) -> np.float32:
    """Correctly rounded fp32 value of an exact rational in the normal range."""
    if x == 0:
        return np.float32(0.0)
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if not (-126 <= e <= 127):
        raise ValueError("outside the fp32 normal range")
    scaled = a / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * m * 2.0 ** (e - 23))


def exact_block_means(x: np.ndarray, nvb: int, block: int = 64, end: int = None) -> np.ndarray:
    """x: [B, T, H, D] of bf16 values -> fp32 [B, H, NVB, D] exact means of
    rows [block*i, min(block*(i+1), end)) (end defaults to block*nvb)."""
    B, T, H, D = x.shape
    end = nvb * block if end is None else end
    out = np.zeros((B, H, nvb, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nvb):
                rows = range(i * block, min((i + 1) * block, end))
                for d in range(D):
                    s = sum(Fraction(float(x[b, t, h, d])) for t in rows)
                    out[b, h, i, d] = round_fraction_to_f32(s / len(rows))
    return out


def exact_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """fp32 [B, H, NQ, NK]: correctly rounded exact dot products."""
    B, H, NQ, D = qbar.shape
    NK = kbar.shape[2]
    out = np.zeros((B, H, NQ, NK), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            qf = [[Fraction(float(v)) for v in qbar[b, h, i]] for i in range(NQ)]
            kf = [[Fraction(float(v)) for v in kbar[b, h, j]] for j in range(NK)]
            for i in range(NQ):
                for j in range(NK):
                    out[b, h, i, j] = round_fraction_to_f32(sum(a * c for a, c in zip(qf[i], kf[j])))
    return out
