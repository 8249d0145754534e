"""Pins of the oracle's block pooling and top-k selection.

RoLA (arXiv 2609.06712v3) Fig. 2 and §4.1: the sparse branch keeps the
top-k key blocks per query block. The scoring rule (mean-pooled rotated q
against mean-pooled rotated k, over 1/sqrt(D)), the tie rule (lower block
index first) and the ascending storage order are readings; these tests pin
the oracle to their plain definitions computed another way.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("L,bs", [(96, 32), (100, 32), (70, 16), (5, 8)])
def test_pooled_score_is_mean_of_token_scores(L, bs):
    rng = np.random.default_rng(7)
    D = 16
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    s = oracle.block_scores(oracle.block_mean(q, bs), oracle.block_mean(k, bs))
    nb = -(-L // bs)
    assert s.shape == (nb, nb)
    for i in range(nb):
        qi = q[i * bs:min((i + 1) * bs, L)]
        for j in range(nb):
            kj = k[j * bs:min((j + 1) * bs, L)]
            brute = sum(qa @ kb for qa in qi for kb in kj) / (len(qi) * len(kj)) / np.sqrt(D)
            assert abs(s[i, j] - brute) < 1e-12


def test_topk_equals_stable_full_sort_with_ties():
    rng = np.random.default_rng(8)
    n = 40
    s = rng.integers(0, 6, size=(n, n)).astype(float)  # many exact ties
    for k in (1, 3, 7, 20, 39, 40):
        idx, thr, nxt = oracle.topk_blocks(s, k)
        for i in range(n):
            order = np.argsort(-s[i], kind="stable")   # ties keep lower index first
            assert list(idx[i]) == sorted(order[:k])
            assert thr[i] == s[i, order[k - 1]]
            assert nxt[i] == (s[i, order[k]] if k < n else -np.inf)


def test_topk_all_blocks_when_k_is_nblk():
    s = np.random.default_rng(9).standard_normal((13, 13))
    idx, _, _ = oracle.topk_blocks(s, 13)
    np.testing.assert_array_equal(idx, np.tile(np.arange(13), (13, 1)))


def test_block_scores_shift_invariant():
    """Offsetting every position by the same vector leaves every pooled
    score unchanged (rotations enter only through offsets)."""
    rng = np.random.default_rng(10)
    grid, pairs, bs = (3, 4, 6), (4, 2, 2), 8
    L, D = 72, 16
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))

    def scores(origin):
        qr = oracle.rope3d(q, grid, 10000.0, pairs, origin)
        kr = oracle.rope3d(k, grid, 10000.0, pairs, origin)
        return oracle.block_scores(oracle.block_mean(qr, bs), oracle.block_mean(kr, bs))

    np.testing.assert_allclose(scores((0, 0, 0)), scores((4, 7, -3)), atol=1e-12)


def test_single_token_blocks_reduce_to_token_scores():
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal((9, 8)), rng.standard_normal((9, 8))
    s = oracle.block_scores(oracle.block_mean(q, 1), oracle.block_mean(k, 1))
    np.testing.assert_allclose(s, q @ k.T / np.sqrt(8), atol=1e-13)
