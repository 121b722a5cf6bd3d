"""Oracle part 4: base-2 log-sum-exp attention states and their merge.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

An attention state for one (query row, head) over a set of keys is the pair
(o, b): o is the softmax-weighted mean of the values over that key set and
b = log2(sum_j exp(s_j)) is the base-2 log of its total weight, with s_j the
already-scaled logits.  The empty key set is (zero vector, -inf).  Deep Dive -
FlashInfer, "Core mechanism: schedule work around state" and "A worked
split-KV example".
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def merge_state(o_a, b_a: float, o_b, b_b: float):
    """Merge two states over disjoint key sets (pure Python floats).

    Deep Dive - FlashInfer, "A worked split-KV example": take the larger
    statistic as the shift, form the base-2 weights 2^(b - shift),
    normalise them to scales before combining the vectors (so large values
    cannot overflow), and return shift + log2(sum of weights).  An empty state
    (-inf) passes the other state through unchanged; two empty states give an
    empty state.  Inputs are checked the way that section's reference checks
    them: equal positive dimension, finite vectors, statistics finite or -inf,
    and a zero vector wherever the statistic is -inf.
    """
    o_a = [float(x) for x in o_a]
    o_b = [float(x) for x in o_b]
    if not o_a or len(o_a) != len(o_b):
        raise ValueError("state vectors need one positive common dimension")
    if not all(math.isfinite(x) for x in o_a + o_b):
        raise ValueError("state vectors must be finite")
    for b in (b_a, b_b):
        if math.isnan(b) or b == math.inf:
            raise ValueError("a statistic is finite or -inf")
    for o, b in ((o_a, b_a), (o_b, b_b)):
        if b == NEG_INF and any(x != 0.0 for x in o):
            raise ValueError("an empty state carries the zero vector")
    if b_a == NEG_INF:
        return list(o_b), float(b_b)
    if b_b == NEG_INF:
        return list(o_a), float(b_a)
    shift = max(b_a, b_b)
    w_a = 2.0 ** (b_a - shift)
    w_b = 2.0 ** (b_b - shift)
    z = w_a + w_b
    sa, sb = w_a / z, w_b / z
    return [sa * x + sb * y for x, y in zip(o_a, o_b)], shift + math.log2(z)


def merge_state_arrays(v_a, s_a, v_b, s_b):
    """``merge_state`` applied independently to every (row, head) of arrays.

    v_* have shape [..., D] and s_* shape [...]; computed in float64.  Same
    recurrence as ``merge_state``: an -inf side passes the other through.
    """
    v_a = np.asarray(v_a, dtype=np.float64)
    v_b = np.asarray(v_b, dtype=np.float64)
    s_a = np.asarray(s_a, dtype=np.float64)
    s_b = np.asarray(s_b, dtype=np.float64)
    a_empty = np.isneginf(s_a)
    b_empty = np.isneginf(s_b)
    both = ~(a_empty | b_empty)
    shift = np.where(both, np.maximum(s_a, s_b), 0.0)
    w_a = np.where(both, np.exp2(np.where(both, s_a - shift, 0.0)), 0.0)
    w_b = np.where(both, np.exp2(np.where(both, s_b - shift, 0.0)), 0.0)
    z = np.where(both, w_a + w_b, 1.0)
    v = (w_a / z)[..., None] * v_a + (w_b / z)[..., None] * v_b
    s = np.where(both, shift + np.log2(z), 0.0)
    v = np.where(a_empty[..., None], v_b, np.where(b_empty[..., None], v_a, v))
    s = np.where(a_empty, s_b, np.where(b_empty, s_a, s))
    return v, s


def merge_states(v, s):
    """Merge K states per (row, head) by a left fold.

    v: [N, K, H, D], s: [N, K, H] -> ([N, H, D], [N, H]).  The merge is
    associative in exact arithmetic (Deep Dive - FlashInfer, "Core mechanism:
    schedule work around state"), so the fold order only changes rounding.
    With K == 0 the result is the empty state.
    """
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    n, k, h, d = v.shape
    acc_v = np.zeros((n, h, d))
    acc_s = np.full((n, h), NEG_INF)
    for i in range(k):
        acc_v, acc_s = merge_state_arrays(acc_v, acc_s, v[:, i], s[:, i])
    return acc_v, acc_s


def direct_state(scores, values, dim: int):
    """Unsplit state of one row: stable softmax over all keys, base-2 statistic.

    Deep Dive - FlashInfer, "A worked split-KV example" (the direct
    comparison): shift by the max score, exponentiate, normalise, and report
    (shift + ln(sum)) / ln 2.  No keys gives the empty state.
    """
    if not scores:
        return [0.0] * dim, NEG_INF
    shift = max(scores)
    w = [math.exp(x - shift) for x in scores]
    z = sum(w)
    out = [sum(wi * v[d] for wi, v in zip(w, values)) / z for d in range(dim)]
    return out, (shift + math.log(z)) / math.log(2.0)
