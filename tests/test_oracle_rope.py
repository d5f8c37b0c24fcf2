"""Pins for the oracle's RoPE pieces (CPU only).

RoPE itself is not printed on the pages (they name it and the Qwen3 models that
use it); the textbook form with rotate-half pairing and theta_d = b^(-2d/D) is
used.  These tests check the implementation against a polar-coordinate closed
form and against the algebraic properties the correction rotation relies on
(ResearchPod transcript, cache exchange: rotating a vector cached at position p
by c(p) = a(p) - p must land it at the aliased position a(p)).
"""

import math

import numpy as np

import oracle


def test_frequencies_closed_form():
    th = oracle.rope_frequencies(8, 10000.0)
    assert th.shape == (4,)
    assert th[0] == 1.0
    for d in range(4):
        assert math.isclose(th[d], 10000.0 ** (-d / 4), rel_tol=1e-15)
    th = oracle.rope_frequencies(128, 1e6)
    assert math.isclose(th[-1], 1e6 ** (-126 / 128), rel_tol=1e-14)
    assert np.all(np.diff(th) < 0)


def test_two_dim_polar_closed_form():
    # D = 2: one pair; theta_0 = 1, so position P rotates the vector by P radians
    # counter-clockwise: (r cos a, r sin a) -> (r cos(a+P), r sin(a+P)).
    rng = np.random.default_rng(1)
    for _ in range(50):
        r, a, p = rng.uniform(0.1, 3), rng.uniform(-4, 4), rng.integers(-100000, 100000)
        x = np.array([r * math.cos(a), r * math.sin(a)])
        y = oracle.rotate_half_pairs(x, oracle.rope_frequencies(2, 1e4) * p)
        assert np.allclose(y, [r * math.cos(a + p), r * math.sin(a + p)], atol=1e-9)


def test_matrix_matches_rotation_and_pairing():
    rng = np.random.default_rng(2)
    d = 16
    th = oracle.rope_frequencies(d, 1e4)
    x = rng.standard_normal(d)
    for p in (0, 1, 7, 12345):
        r = oracle.rotation_matrix(p * th)
        assert np.allclose(r @ x, oracle.rotate_half_pairs(x, p * th), atol=1e-12)
        assert np.allclose(r.T @ r, np.eye(d), atol=1e-12)
        # pairing is (d, d + D/2): the matrix only mixes those coordinates
        for i in range(d):
            nz = set(np.nonzero(np.abs(r[i]) > 0)[0]) - {i}
            assert nz <= {(i + d // 2) % d}


def test_composition_reaches_aliased_position():
    rng = np.random.default_rng(3)
    d = 128
    th = oracle.rope_frequencies(d, 1e6)
    for g in (2, 3, 4):
        for p in (0, 1, 5, 4095, 98303, 131071):
            raw = rng.standard_normal(d)
            cached = oracle.rotate_half_pairs(raw, p * th)
            corrected = oracle.rotate_half_pairs(cached, oracle.correction_offset(p, g) * th)
            direct = oracle.rotate_half_pairs(raw, oracle.aliased_position(p, g) * th)
            assert np.allclose(corrected, direct, atol=1e-9)
            assert math.isclose(np.linalg.norm(corrected), np.linalg.norm(raw), rel_tol=1e-12)
            assert oracle.correction_offset(p, g) <= 0


def test_relative_position_property():
    # R(a theta)^T R(b theta) = R((b - a) theta): dot products depend on b - a only.
    rng = np.random.default_rng(4)
    d = 32
    th = oracle.rope_frequencies(d, 1e4)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for a, b, shift in [(3, 9, 100), (0, 0, 7), (1000, 10, 55555)]:
        s1 = oracle.rotate_half_pairs(q, a * th) @ oracle.rotate_half_pairs(k, b * th)
        s2 = oracle.rotate_half_pairs(q, (a + shift) * th) @ oracle.rotate_half_pairs(k, (b + shift) * th)
        assert math.isclose(s1, s2, rel_tol=1e-9, abs_tol=1e-9)
        ra, rb = oracle.rotation_matrix(a * th), oracle.rotation_matrix(b * th)
        assert np.allclose(ra.T @ rb, oracle.rotation_matrix((b - a) * th), atol=1e-9)
