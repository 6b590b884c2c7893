"""Pins of the oracle's sigmoid-group routing ([Edge0] App. A "Sigmoid-group
(K, G of n groups, scale s)", §2 "MoE routing") against values worked by
hand, a brute force over subsets, special cases and invariants."""
import itertools
import math
import os

import numpy as np
import pytest

from oracle.reference import sigmoid_group_gaps, sigmoid_group_topk, softmax_topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sigmoid_group_hand.txt")


def _hand_cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        elif key == "p":
            cur["p"] = np.array([float(v) for v in rest])
        elif key == "bias":
            cur["bias"] = None if rest == ["-"] else np.array([float(v) for v in rest])
        elif key == "n":
            f = dict(zip(rest[1::2], rest[2::2]))
            cur["n"], cur["G"], cur["K"], cur["s"] = int(rest[0]), int(f["G"]), int(f["K"]), float(f["s"])
        elif key == "ids":
            cur["ids"] = [int(v) for v in rest]
        elif key == "w":
            cur["w"] = np.array([float(v) for v in rest])
    return cases


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_sigmoid_group_hand_cases(case):
    p = case["p"]
    logits = np.log(p / (1.0 - p))
    ids, w = sigmoid_group_topk(logits, case["K"], case["n"], case["G"], case["s"], case["bias"])
    assert list(ids) == case["ids"]
    np.testing.assert_allclose(w, case["w"], rtol=1e-12)


def _brute(logits, bias, K, n, G):
    """The surviving groups maximise the sum of group scores over all
    G-subsets of groups (a group's score maximised over its pairs); the ids
    maximise the sum of selection scores over all K-subsets of survivors.
    Returns the id set, or None when the optimum is not unique by 1e-6."""
    E = len(logits)
    gs = E // n
    sig32 = (1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))).astype(np.float32)
    c = (sig32 + (np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32))).astype(np.float32)
    gsc = [max(float(np.float32(c[a] + c[b])) for a, b in itertools.combinations(range(i * gs, (i + 1) * gs), 2))
           for i in range(n)]
    sets = sorted(((sum(gsc[i] for i in S), S) for S in itertools.combinations(range(n), G)), reverse=True)
    if len(sets) > 1 and sets[0][0] - sets[1][0] < 1e-6:
        return None
    alive = [e for i in sets[0][1] for e in range(i * gs, (i + 1) * gs)]
    picks = sorted(((sum(float(c[e]) for e in S), S) for S in itertools.combinations(alive, K)), reverse=True)
    if len(picks) > 1 and picks[0][0] - picks[1][0] < 1e-6:
        return None
    return set(picks[0][1]), c


@pytest.mark.parametrize("seed", range(40))
def test_sigmoid_group_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    E, n = [(8, 4), (8, 2), (12, 3), (12, 6), (16, 4), (16, 8)][seed % 6]
    gs = E // n
    G = int(rng.integers(1, n + 1))
    K = int(rng.integers(1, min(G * gs, 6) + 1))
    logits = rng.normal(0.0, 2.0, E)
    bias = None if seed % 3 == 0 else rng.normal(0.0, 0.3, E)
    s = float(rng.uniform(0.5, 3.0))
    got = _brute(logits, bias, K, n, G)
    if got is None:
        pytest.skip("optimum not unique at this seed")
    want, c = got
    ids, w = sigmoid_group_topk(logits, K, n, G, s, bias)
    assert set(ids.tolist()) == want and len(set(ids.tolist())) == K
    # listed in rank order of the selection score
    assert all(c[ids[i]] >= c[ids[i + 1]] for i in range(K - 1))
    # weights: proportional to the raw sigmoid, summing to the scale
    sig = 1.0 / (1.0 + np.exp(-logits[ids]))
    assert math.isclose(float(w.sum()), s, rel_tol=1e-12)
    np.testing.assert_allclose(w / w[0], sig / sig[0], rtol=1e-12)


def test_sigmoid_group_single_group_no_bias_is_plain_topk():
    # one group (n = G = 1), no bias: sigmoid is increasing, so the ids are the
    # plain top-K of the logits, the ids softmax-top-K picks
    rng = np.random.default_rng(7)
    for _ in range(20):
        logits = rng.normal(0.0, 1.0, 64)
        ids, _ = sigmoid_group_topk(logits, 8, 1, 1, 1.0)
        ref, _ = softmax_topk(logits, 8)
        assert list(ids) == list(ref)


def test_sigmoid_group_all_groups_survive():
    # G = n masks nothing: the same ids as one group
    rng = np.random.default_rng(8)
    for _ in range(20):
        logits = rng.normal(0.0, 1.0, 32)
        bias = rng.normal(0.0, 0.2, 32)
        a, wa = sigmoid_group_topk(logits, 6, 8, 8, 2.5, bias)
        b, wb = sigmoid_group_topk(logits, 6, 1, 1, 2.5, bias)
        assert list(a) == list(b)
        np.testing.assert_allclose(wa, wb, rtol=0)


def test_sigmoid_group_extremes():
    # saturated sigmoid: logits of -1000 give sigma = 0 (weights stay finite
    # through the 1e-20 guard), +1000 gives 1
    logits = np.array([-1000.0] * 8)
    ids, w = sigmoid_group_topk(logits, 2, 4, 2, 2.5)
    assert list(ids) == [0, 1] and np.all(w == 0.0)
    logits = np.array([1000.0, -1000.0] * 4)
    ids, w = sigmoid_group_topk(logits, 2, 4, 2, 2.5)
    assert list(ids) == [0, 2]
    np.testing.assert_allclose(w, [1.25, 1.25], rtol=1e-15)


def test_sigmoid_group_rejects_bad_configs():
    l = np.zeros(8)
    for args in [(2, 3, 1), (2, 4, 0), (2, 4, 5), (2, 8, 1), (5, 4, 2)]:
        with pytest.raises(ValueError):
            sigmoid_group_topk(l, args[0], args[1], args[2], 1.0)


def test_sigmoid_group_gaps():
    # case A of the hand fixture: groups 1.25 1.15 | 0.9 0.9 -> group margin
    # 0.25; survivors .9 .75 .5 | .25 -> expert margin at K=3 is 0.25
    p = np.array([0.5, 0.75, 0.25, 0.9, 0.1, 0.8, 0.2, 0.7])
    gg, eg = sigmoid_group_gaps(np.log(p / (1 - p)), 3, 4, 2)
    assert gg == pytest.approx(0.25, abs=1e-6) and eg == pytest.approx(0.25, abs=1e-6)
    gg, eg = sigmoid_group_gaps(np.log(p / (1 - p)), 4, 4, 4)
    assert gg == math.inf and eg == pytest.approx(0.2, abs=1e-6)  # .7 vs .5
