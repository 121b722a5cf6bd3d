"""Pins for oracle.merge against Deep Dive - FlashInfer, 'A worked split-KV example'."""

import math
import random

import numpy as np
import pytest

from oracle import merge as mg
from tests.conftest import load_golden


def test_worked_merge():
    w = load_golden("merge_example.json")["worked"]
    o, b = mg.merge_state(w["o_a"], w["b_a"], w["o_b"], w["b_b"])
    assert max(abs(x - y) for x, y in zip(o, w["o"])) < w["tol"]
    assert abs(b - (2.0 + math.log2(1.5))) < w["tol"]
    assert f"{[round(x, 4) for x in o]} {round(b, 4)}" == w["printed"]


def test_merge_identities():
    o, b = mg.merge_state([1.0, 0.0], 2.0, [0.0, 1.0], 1.0)
    assert mg.merge_state([0.0, 0.0], -math.inf, o, b) == (o, b)
    assert mg.merge_state(o, b, [0.0, 0.0], -math.inf) == (o, b)
    assert mg.merge_state([0.0, 0.0], -math.inf, [0.0, 0.0], -math.inf) == ([0.0, 0.0], -math.inf)
    assert mg.merge_state([1e308], 0.0, [1e308], 0.0)[0] == [1e308]


@pytest.mark.parametrize("bad", [
    dict(o_a=[], o_b=[]),
    dict(o_a=[1.0], o_b=[1.0, 2.0]),
    dict(o_a=[math.nan], o_b=[1.0]),
    dict(o_a=[1.0], o_b=[1.0], b_a=math.nan),
    dict(o_a=[1.0], o_b=[1.0], b_b=math.inf),
    dict(o_a=[1.0], o_b=[1.0], b_a=-math.inf),
])
def test_merge_rejects(bad):
    args = dict(o_a=[1.0], b_a=0.0, o_b=[1.0], b_b=0.0)
    args.update(bad)
    with pytest.raises(ValueError):
        mg.merge_state(args["o_a"], args["b_a"], args["o_b"], args["b_b"])


def test_split_sweep_168():
    """The split/direct sweep: every cut of every score list, merged, equals
    the direct state within 1e-10; the pages print 168 cases."""
    s = load_golden("merge_example.json")["split_sweep"]
    rng = random.Random(7)
    cases = 0
    for length in s["lengths"]:
        for offset in s["offsets"]:
            scores = [offset + rng.uniform(*s["score_range"]) for _ in range(length)]
            values = [[rng.uniform(*s["value_range"]), rng.uniform(*s["value_range"])] for _ in scores]
            want_o, want_b = mg.direct_state(scores, values, 2)
            for cut in range(length + 1):
                left = mg.direct_state(scores[:cut], values[:cut], 2)
                right = mg.direct_state(scores[cut:], values[cut:], 2)
                got_o, got_b = mg.merge_state(*left, *right)
                assert max(abs(a - b) for a, b in zip(got_o, want_o)) < s["tol"]
                assert abs(got_b - want_b) < s["tol"]
                cases += 1
    assert cases == s["cases"]


def test_overlap_and_wrong_base():
    g = load_golden("merge_example.json")
    scores, values = [0.0, 0.0], [[1.0, 0.0], [0.0, 1.0]]
    whole = mg.direct_state(scores, values, 2)
    dup = mg.merge_state(*whole, *mg.direct_state(scores[:1], values[:1], 2))
    assert abs(whole[0][0] - g["overlap"]["whole_first"]) < 1e-12
    assert f"{dup[0][0]:.4f}" == f"{g['overlap']['with_duplicate']:.4f}"
    correct = mg.merge_state([1.0, 0.0], 2.0, [0.0, 1.0], 1.0)
    wrong = mg.merge_state([1.0, 0.0], 2 * math.log(2), [0.0, 1.0], math.log(2))
    assert f"{correct[0][0]:.4f}" == f"{g['wrong_base']['correct_first']:.4f}"
    assert f"{wrong[0][0]:.4f}" == f"{g['wrong_base']['natural_log_first']:.4f}"
    assert abs(wrong[0][0] - correct[0][0]) > g["wrong_base"]["min_gap"]


def test_array_merge_matches_scalar_merge():
    rng = np.random.default_rng(3)
    n, h, d = 7, 3, 5
    va, vb = rng.standard_normal((n, h, d)), rng.standard_normal((n, h, d))
    sa, sb = rng.uniform(-50, 50, (n, h)), rng.uniform(-50, 50, (n, h))
    sa[0, 0] = -np.inf
    va[0, 0] = 0.0
    sb[1, 2] = -np.inf
    vb[1, 2] = 0.0
    sa[2, 1] = sb[2, 1] = -np.inf
    va[2, 1] = vb[2, 1] = 0.0
    v, s = mg.merge_state_arrays(va, sa, vb, sb)
    for i in range(n):
        for j in range(h):
            ro, rb = mg.merge_state(list(va[i, j]), float(sa[i, j]), list(vb[i, j]), float(sb[i, j]))
            assert np.allclose(v[i, j], ro, rtol=0, atol=1e-14)
            assert (s[i, j] == rb) or abs(s[i, j] - rb) < 1e-12


def test_multiway_merge_equals_direct_state():
    """A K-way fold of disjoint chunk states equals the direct state of the
    concatenated key set (the section's split invariance, K chunks at once),
    and does not depend on the order of the chunks beyond rounding."""
    rng = random.Random(11)
    for length in (1, 5, 40):
        scores = [rng.uniform(-30, 30) for _ in range(length)]
        values = [[rng.uniform(-1, 1) for _ in range(3)] for _ in scores]
        want_o, want_b = mg.direct_state(scores, values, 3)
        cuts = sorted(rng.sample(range(length + 1), min(4, length + 1)))
        bounds = [0] + cuts + [length]
        parts = [mg.direct_state(scores[a:b], values[a:b], 3) for a, b in zip(bounds, bounds[1:])]
        v = np.array([[[p[0]] for p in parts]])          # [1, K, 1, 3]
        s = np.array([[[p[1]] for p in parts]])          # [1, K, 1]
        for order in (list(range(len(parts))), list(reversed(range(len(parts))))):
            got_v, got_s = mg.merge_states(v[:, order], s[:, order])
            assert np.allclose(got_v[0, 0], want_o, atol=1e-12)
            assert abs(got_s[0, 0] - want_b) < 1e-10
    ev, es = mg.merge_states(np.zeros((2, 0, 1, 3)), np.zeros((2, 0, 1)))
    assert np.all(ev == 0) and np.all(np.isneginf(es))
