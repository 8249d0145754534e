"""Pins of the oracle's block-sparse softmax attention.

RoLA (arXiv 2609.06712v3) §4.1: block-sparse softmax attention over the
kept blocks; §3 "Full attention" is the dense case. Keeping every block must
reproduce dense softmax attention, and any selection must equal dense
attention with the dropped keys masked to -inf. The reference routines here
are the textbook softmax(Q K^T / sqrt(D)) V written with numpy matrix
products, independent of the oracle's loops.
"""
import numpy as np
import pytest

import oracle


def _softmax_attention(q, k, v, mask=None):
    s = q @ k.T / np.sqrt(q.shape[1])
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ v


@pytest.mark.parametrize("L,bs", [(128, 32), (100, 32), (37, 8)])
def test_all_blocks_is_dense_attention(L, bs):
    rng = np.random.default_rng(20)
    D = 16
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    got = oracle.dense_attention(q, k, v, bs)
    np.testing.assert_allclose(got, _softmax_attention(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L,bs,k", [(128, 32, 2), (100, 32, 1), (75, 16, 3)])
def test_selection_is_masked_dense_attention(L, bs, k):
    rng = np.random.default_rng(21)
    D = 16
    q, kk, v = (rng.standard_normal((L, D)) for _ in range(3))
    nb = -(-L // bs)
    idx = np.sort(np.stack([rng.choice(nb, size=k, replace=False) for _ in range(nb)]), axis=1).astype(np.int32)
    got = oracle.block_sparse_attention(q, kk, v, bs, idx).reshape(-1, D)
    blk = np.arange(L) // bs
    for i in range(nb):
        rows = np.arange(i * bs, min((i + 1) * bs, L))
        mask = np.isin(blk, idx[i])[None, :].repeat(len(rows), 0)
        want = _softmax_attention(q[rows], kk, v, mask)
        np.testing.assert_allclose(got[i * bs:i * bs + len(rows)], want, rtol=1e-12, atol=1e-12)
    # rows past L are left at zero
    assert not got[L:].any()


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(22)
    L, D, bs = 96, 8, 32
    q, k = rng.standard_normal((L, D)) * 3, rng.standard_normal((L, D)) * 3
    v = np.full((L, D), 0.625)
    idx = np.array([[0, 2], [1, 2], [0, 1]], dtype=np.int32)
    got = oracle.block_sparse_attention(q, k, v, bs, idx).reshape(-1, D)
    np.testing.assert_allclose(got, 0.625, rtol=0, atol=1e-14)


def test_query_block_subset_matches_full_pass():
    rng = np.random.default_rng(23)
    L, D, bs = 160, 8, 32
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    idx = np.array([[0, 1], [1, 4], [2, 3], [0, 4], [3, 4]], dtype=np.int32)
    full = oracle.block_sparse_attention(q, k, v, bs, idx)
    part = oracle.block_sparse_attention(q, k, v, bs, idx, qblocks=np.array([1, 4], dtype=np.int32))
    np.testing.assert_array_equal(part, full[[1, 4]])
