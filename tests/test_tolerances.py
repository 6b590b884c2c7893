"""CPU checks of the comparison rules the GPU parity tests use.

* The bf16-rounding rule for the RMSNorm output (tests/layer_setup.py):
  an fp32 evaluation in the kernels' summation order with the right eps
  passes on every vector, and the same evaluation with eps 1e-5 in place of
  1e-6 (a 4.5e-6 relative shift) is rejected.
* The near-tie gap (oracle topk_gap) that decides which routing ids are
  compared bit-exactly: pinned by hand cases."""
import numpy as np
import pytest

import oracle as O
from synth import gen as G
from tests.layer_setup import RMSNORM_REL, check_bf16_rounding


def _fp32_rmsnorm_bits(h_bits, eps, per_thread=8):
    """x = bf16(h * 1/sqrt(sum(h^2)/d + eps)) evaluated in fp32 the way the
    kernels order it: sequential sums of `per_thread` squares per thread,
    then a pairwise tree over the threads."""
    h = O.bf16_to_f64(h_bits).astype(np.float32)
    sq = (h * h).astype(np.float32)
    parts = sq.reshape(-1, per_thread)
    acc = np.zeros(parts.shape[0], np.float32)
    for j in range(per_thread):
        acc = (acc + parts[:, j]).astype(np.float32)
    while acc.shape[0] > 1:
        acc = (acc[0::2] + acc[1::2]).astype(np.float32)
    d = np.float32(h.shape[0])
    inv = np.float32(1.0) / np.sqrt(np.float32(acc[0] / d) + np.float32(eps))
    return G.to_bf16_bits((h * inv).astype(np.float32))


def _vectors(n, seed):
    """Hidden states of RMS near 1 (each times a random factor in [0.9, 1.1]:
    the stack's h drifts; a bf16 h of RMS exactly 1 normalises to next to
    itself, a bf16 number far from every rounding midpoint)."""
    S = G.QWEN3_MOE
    rng = np.random.default_rng(seed)
    for i in range(n):
        f = (G.hidden(S, seed, i).astype(np.uint32) << 16).view(np.float32)
        yield G.to_bf16_bits(f * np.float32(rng.uniform(0.9, 1.1)))


def test_rmsnorm_rule_accepts_fp32_evaluation():
    for h in _vectors(400, 11):
        got = _fp32_rmsnorm_bits(h, 1e-6)
        check_bf16_rounding(got, O.rmsnorm(O.bf16_to_f64(h), 1e-6))


def _rejected(rel):
    n = 0
    for h in _vectors(400, 12):
        got = _fp32_rmsnorm_bits(h, 1e-5)
        try:
            check_bf16_rounding(got, O.rmsnorm(O.bf16_to_f64(h), 1e-6), rel=rel)
        except AssertionError:
            n += 1
    return n


def test_rmsnorm_rule_rejects_wrong_eps():
    """eps 1e-5 instead of 1e-6 moves x by about 4.5e-6 relative at RMS 1: a
    vector is rejected when one of its elements lies between the bound and
    that shift from a rounding midpoint.  A bf16 h times one constant puts its
    elements at few distinct positions relative to the midpoints, so a single
    vector is caught only sometimes; over 400 vectors (as over the layers and
    steps of a stack test) the bound catches the wrong eps many times, where
    a bound of 1e-5 never does."""
    assert _rejected(RMSNORM_REL) >= 10
    assert _rejected(1e-5) == 0
    assert RMSNORM_REL < 4.5e-6


# ----------------------------------------------------------- topk_gap pins
def test_topk_gap_hand_cases():
    """The gap between the K-th and (K+1)-th largest logit, by hand."""
    l = np.array([0.5, 3.0, -1.0, 2.0, 2.75])
    assert O.topk_gap(l, 1) == pytest.approx(0.25)      # 3.0 vs 2.75
    assert O.topk_gap(l, 2) == pytest.approx(0.75)      # 2.75 vs 2.0
    assert O.topk_gap(l, 3) == pytest.approx(1.5)       # 2.0 vs 0.5
    assert O.topk_gap(l, 4) == pytest.approx(1.5)       # 0.5 vs -1.0
    assert O.topk_gap(l, 5) == float("inf")             # K = E: nothing is left out


def test_topk_gap_exact_tie_and_order_free():
    l = np.array([1.0, 4.0, 1.0, 4.0, 0.0])
    assert O.topk_gap(l, 1) == 0.0                      # tie for first place
    assert O.topk_gap(l, 2) == 3.0                      # the tied pair is in, 1.0 out
    assert O.topk_gap(l, 3) == 0.0                      # tie at the boundary
    perm = np.random.default_rng(0).permutation(l.shape[0])
    for k in range(1, 5):
        assert O.topk_gap(l[perm], k) == O.topk_gap(l, k)


def test_topk_gap_matches_brute_force():
    """Against the smallest selected minus the largest unselected logit over
    the brute-force top-K set, on random tiny inputs."""
    import itertools
    rng = np.random.default_rng(1)
    for _ in range(200):
        E = int(rng.integers(2, 8))
        k = int(rng.integers(1, E))
        l = np.round(rng.normal(size=E), 1)          # ties are common at one decimal
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(l[list(c)]))
        sel = l[list(best)]
        rest = np.delete(l, list(best))
        assert O.topk_gap(l, k) == pytest.approx(sel.min() - rest.max())
