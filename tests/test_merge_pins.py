"""Pins of the oracle's merge-and-requantise functions ([Edge0] §3.3 and
its footnote 2): a worked example, exact idempotence on representable
groups, special deltas with closed-form retention (0, 1), the nearest-level
property against a brute force over the 16 levels, and the output-level
retention's closed forms."""
import math

import numpy as np
import pytest

import oracle as O


def _bf16(v):
    return O.bf16_to_f64(O.f64_to_bf16_bits(np.asarray(v, dtype=np.float64)))


def _representable(rng, rows, groups, g):
    """dequant(q, s, b) with every group's codes spanning 0..15 (so its min
    and max are b and 15 s + b)."""
    q = rng.integers(0, 16, size=(rows, groups * g))
    q[:, ::g] = 0
    q[:, 1::g] = 15
    s_bits = O.f64_to_bf16_bits(rng.uniform(0.005, 0.02, size=(rows, groups)))
    b_bits = O.f64_to_bf16_bits(-8.0 * O.bf16_to_f64(s_bits))
    W = O.bf16_to_f64(s_bits).repeat(g, axis=1) * q + O.bf16_to_f64(b_bits).repeat(g, axis=1)
    return q, s_bits, b_bits, W


def test_worked_example():
    # [0, 0.1, 0.2, 1.5]: min 0, max 1.5, s = bf16(0.1) = 0.10009765625,
    # codes round(w / s) = 0, 1, 2, 15 (14.985 rounds up)
    q, s, b = O.requantize_affine(np.array([[0.0, 0.1, 0.2, 1.5]]), 4)
    assert q.tolist() == [[0, 1, 2, 15]]
    assert O.bf16_to_f64(s)[0, 0] == 0.10009765625 and O.bf16_to_f64(b)[0, 0] == 0.0


def test_idempotent_on_representable_groups():
    rng = np.random.default_rng(1)
    q, s, b, W = _representable(rng, 6, 4, 64)
    q2, s2, b2 = O.requantize_affine(W, 64)
    assert np.array_equal(q2, q) and np.array_equal(s2, s) and np.array_equal(b2, b)


def test_nearest_level_brute_force():
    rng = np.random.default_rng(2)
    W = rng.normal(0.0, 0.05, size=(8, 128))
    q, s, b = O.requantize_affine(W, 32)
    sv = O.bf16_to_f64(s).repeat(32, axis=1)
    bv = O.bf16_to_f64(b).repeat(32, axis=1)
    levels = bv[:, :, None] + sv[:, :, None] * np.arange(16)[None, None, :]
    d = np.abs(W[:, :, None] - levels)
    best = d.min(axis=2)
    got = np.abs(W - (bv + sv * q))
    assert np.all(got <= best + 1e-15)


def _factors(delta_row_fn, r, n_in, n_out):
    """bf16 A [r][in], B [out][r] whose product B A is given exactly."""
    A, B = delta_row_fn(r, n_in, n_out)
    return O.f64_to_bf16_bits(A), O.f64_to_bf16_bits(B)


def test_constant_shift_survives_whole():
    # delta = c on every element (A = ones, B = c / scale): each group's min
    # and max move by c, b + c is a bf16 number, so the codes stay and the
    # whole delta survives: retention 1
    rng = np.random.default_rng(3)
    g = 64
    q = rng.integers(0, 16, size=(4, 2 * g))
    q[:, ::g], q[:, 1::g] = 0, 15
    s_bits = O.f64_to_bf16_bits(np.full((4, 2), 2.0 ** -7))
    b_bits = O.f64_to_bf16_bits(np.full((4, 2), -8 * 2.0 ** -7))
    words = _pack(q)
    c, scale = 2.0 ** -9, 2.0
    A = O.f64_to_bf16_bits(np.ones((1, 2 * g)))
    B = O.f64_to_bf16_bits(np.full((4, 1), c / scale))
    (_, s2, b2), actual, ret = O.merge_requant(words, s_bits, b_bits, A, B, scale, g)
    assert np.array_equal(s2, s_bits) and np.allclose(actual, c, rtol=0, atol=0)
    assert ret == 1.0


def test_small_interior_delta_is_erased():
    # |delta| < s / 4 on elements whose codes are 1..14 only: min, max and
    # every code stay, nothing survives: retention 0
    g = 32
    q = np.tile(np.r_[0, 15, np.arange(1, 15), np.arange(1, 15), 7, 8], (2, 1))
    words = _pack(q)
    s_bits = O.f64_to_bf16_bits(np.full((2, 1), 2.0 ** -6))
    b_bits = O.f64_to_bf16_bits(np.full((2, 1), -8 * 2.0 ** -6))
    A = np.zeros((1, g))
    A[0, 2:] = 1.0
    A = O.f64_to_bf16_bits(A)
    B = O.f64_to_bf16_bits(np.full((2, 1), 2.0 ** -9))  # delta = 2^-9 = s / 8
    _, actual, ret = O.merge_requant(words, s_bits, b_bits, A, B, 1.0, g)
    assert np.all(actual == 0.0) and ret == 0.0


def test_one_step_delta_survives():
    # delta = +s on one interior element (code 5 -> 6): exactly that survives
    g = 32
    q = np.r_[0, 15, np.full(g - 2, 5)][None, :]
    words = _pack(q)
    s = 2.0 ** -6
    s_bits = O.f64_to_bf16_bits(np.full((1, 1), s))
    b_bits = O.f64_to_bf16_bits(np.full((1, 1), 0.0))
    A = np.zeros((1, g))
    A[0, 9] = 1.0
    _, actual, ret = O.merge_requant(words, s_bits, b_bits, O.f64_to_bf16_bits(A),
                                     O.f64_to_bf16_bits(np.full((1, 1), s)), 1.0, g)
    assert actual[0, 9] == s and np.count_nonzero(actual) == 1 and ret == 1.0


def test_retention_small_on_synthetic_weights():
    # the pages' regime: delta RMS ~1e-3 against group steps of 0.005-0.02:
    # most of the delta is erased (the pages report 2-34 %)
    rng = np.random.default_rng(4)
    q, s, b, _ = _representable(rng, 64, 4, 64)
    A = O.f64_to_bf16_bits(rng.normal(0, 0.02, size=(16, 256)))
    B = O.f64_to_bf16_bits(rng.normal(0, 0.01, size=(64, 16)))
    _, actual, ret = O.merge_requant(_pack(q), s, b, A, B, 2.0, 64)
    assert 0.0 < ret < 0.5, ret


def test_layer_retention_closed_forms():
    rng = np.random.default_rng(5)
    U, B = rng.normal(size=32), rng.normal(size=32)
    assert O.layer_retention(U, U, B) == 1.0
    assert O.layer_retention(U, B, B) == 0.0
    assert math.isclose(O.layer_retention(U, (U + B) / 2, B), 0.5, rel_tol=1e-12)


def _pack(q):
    """Codes [out][in] to the u32 nibble words of the format (input i at bits 4 (i % 8))."""
    q = np.asarray(q, dtype=np.uint32)
    out_dim, in_dim = q.shape
    w = q.reshape(out_dim, in_dim // 8, 8) << (4 * np.arange(8, dtype=np.uint32))
    return np.bitwise_or.reduce(w, axis=2).astype(np.uint32)
