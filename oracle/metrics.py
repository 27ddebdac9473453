"""Comparison metrics.

Relative error of a tensor is max|x - ref| / max|ref| (an elementwise ratio
is unbounded near zero).  Greedy tokens are compared only where the
reference's top-2 logit gap exceeds the threshold (a scalar or one value per
row): below it, rounding in a lower precision may legitimately pick the
other token.
"""
import numpy as np


def relerr(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0:
        return float(num)
    return float(num / den)


def tokens_agree(tokens, ref_tokens, ref_gap, threshold=1e-2):
    """(all_equal_where_decided, number_compared)."""
    tokens = np.asarray(tokens)
    ref_tokens = np.asarray(ref_tokens)
    decided = np.asarray(ref_gap) > threshold
    ok = bool(np.all(tokens[decided] == ref_tokens[decided]))
    return ok, int(decided.sum())
