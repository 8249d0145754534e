"""Pins of the oracle's 3D RoPE against facts fixed independently of it.

RoLA (arXiv 2609.06712v3) §3 "3D RoPE", eq. 1: the head is partitioned
across the temporal and spatial axes and orthogonal rotations make scores
depend on relative offsets only. Special cases reduce to the textbook 1D
rotary embedding (RoFormer): pair j of a d-wide head at position p is the
complex number x_{2j} + i x_{2j+1} multiplied by exp(i p base^(-2j/d)).
"""
import itertools

import numpy as np
import pytest

import oracle


def _complex_rope_1d(x, pos, base):
    """Textbook 1D rotary embedding via complex multiplication."""
    d = x.shape[1]
    z = x[:, 0::2] + 1j * x[:, 1::2]
    freq = base ** (-2.0 * np.arange(d // 2) / d)
    z = z * np.exp(1j * np.outer(pos, freq))
    y = np.empty_like(x)
    y[:, 0::2], y[:, 1::2] = z.real, z.imag
    return y


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_single_axis_grid_is_1d_rope_on_that_chunk(axis):
    rng = np.random.default_rng(11)
    pairs = (3, 2, 4)
    D = 2 * sum(pairs)
    grid = [1, 1, 1]
    grid[axis] = 7
    x = rng.standard_normal((7, D))
    y = oracle.rope3d(x, tuple(grid), 10000.0, pairs)
    lo = 2 * sum(pairs[:axis])
    hi = lo + 2 * pairs[axis]
    want = x.copy()
    want[:, lo:hi] = _complex_rope_1d(x[:, lo:hi], np.arange(7), 10000.0)
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-13)


def test_single_pair_is_complex_rotation_by_position():
    # one pair, base irrelevant (theta_0 = 1): rotation by exactly p radians
    x = np.array([[0.3, -1.2]] * 5)
    y = oracle.rope3d(x, (5, 1, 1), 10000.0, (1, 0, 0))
    z = (0.3 - 1.2j) * np.exp(1j * np.arange(5))
    np.testing.assert_allclose(y[:, 0], z.real, atol=1e-15)
    np.testing.assert_allclose(y[:, 1], z.imag, atol=1e-15)


def test_origin_token_is_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((24, 20))
    y = oracle.rope3d(x, (2, 3, 4), 500.0, (4, 3, 3))
    np.testing.assert_array_equal(y[0], x[0])


@pytest.mark.parametrize("grid,pairs", [((2, 3, 4), (4, 3, 3)), ((3, 4, 5), (12, 10, 10))])
def test_norm_preserved(grid, pairs):
    rng = np.random.default_rng(3)
    L, D = int(np.prod(grid)), 2 * sum(pairs)
    x = rng.standard_normal((L, D))
    y = oracle.rope3d(x, grid, 10000.0, pairs)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def _coords(grid):
    T, Hg, Wg = grid
    return np.array(list(itertools.product(range(T), range(Hg), range(Wg))))


@pytest.mark.parametrize("grid,pairs", [((2, 3, 4), (4, 3, 3)), ((3, 4, 5), (12, 10, 10))])
def test_scores_depend_only_on_per_axis_offset(grid, pairs):
    """<R_m x, R_n y> over every token pair of a tiny grid: pairs that share
    the offset vector n - m agree to 1e-12 (brute force), and different
    offsets do give different scores (the rotation is not trivial)."""
    rng = np.random.default_rng(4)
    L, D = int(np.prod(grid)), 2 * sum(pairs)
    x, y = rng.standard_normal(D), rng.standard_normal(D)
    rx = oracle.rope3d(np.tile(x, (L, 1)), grid, 10000.0, pairs)
    ry = oracle.rope3d(np.tile(y, (L, 1)), grid, 10000.0, pairs)
    c = _coords(grid)
    groups = {}
    for m in range(L):
        for n in range(L):
            groups.setdefault(tuple(c[n] - c[m]), []).append(rx[m] @ ry[n])
    spread = max(max(v) - min(v) for v in groups.values())
    assert spread < 1e-12
    reps = np.array([v[0] for v in groups.values()])
    assert len(np.unique(np.round(reps, 9))) > len(groups) // 2


def test_origin_shift_leaves_relative_scores_unchanged():
    rng = np.random.default_rng(5)
    grid, pairs = (3, 4, 5), (4, 3, 3)
    L, D = 60, 20
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    a = oracle.rope3d(q, grid, 10000.0, pairs) @ oracle.rope3d(k, grid, 10000.0, pairs).T
    b = oracle.rope3d(q, grid, 10000.0, pairs, origin=(5, -2, 9)) @ \
        oracle.rope3d(k, grid, 10000.0, pairs, origin=(5, -2, 9)).T
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_flatten_order_is_t_major():
    """Token l sits at (l // (Hg Wg), (l // Wg) % Hg, l % Wg): on a 2x3x4 grid
    token 13 = (1, 0, 1) rotates its t chunk by one step and its w chunk by
    one step, its h chunk not at all."""
    pairs = (1, 1, 1)
    x = np.tile(np.array([1.0, 0.0, 1.0, 0.0, 1.0, 0.0]), (24, 1))
    y = oracle.rope3d(x, (2, 3, 4), 10000.0, pairs)
    np.testing.assert_allclose(y[13], [np.cos(1), np.sin(1), 1, 0, np.cos(1), np.sin(1)], atol=1e-15)
