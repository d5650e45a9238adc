"""Pins of the oracle's block scores (oracle/blockscore.py): the factorised
pooled form against the definition evaluated term by term, closed forms on
constant blocks, and the group mean over query heads."""
import numpy as np
import pytest

from oracle import blockscore as B
from oracle import masks as M


@pytest.mark.parametrize("Hq,Hkv,G", [(4, 2, 2), (4, 2, 4), (2, 2, 2), (6, 3, 3)])
def test_pooled_equals_literal(Hq, Hkv, G):
    rng = np.random.default_rng([Hq, Hkv, G])
    T, d = 23, 5
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    qe = [0, 4, 9, 17, 23]
    ke = [0, 7, 8, 15, 23]
    a = B.pooled_scores(q, k, qe, ke, G, 0.37)
    b = B.literal_scores(q, k, qe, ke, G, 0.37)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_constant_blocks_closed_form():
    """Blocks whose rows are all one vector score scale * u . w exactly."""
    d = 4
    u = np.array([[1.0, 2.0, 0.0, -1.0], [0.5, 0.5, 0.5, 0.5]])
    w = np.array([[3.0, 0.0, 1.0, 1.0], [-2.0, 1.0, 0.0, 4.0], [0.0, 0.0, 1.0, 0.0]])
    qe, ke = [0, 3, 8], [0, 2, 6, 7]
    q = np.zeros((8, 1, d))
    k = np.zeros((7, 1, d))
    for a in range(2):
        q[qe[a]:qe[a + 1], 0] = u[a]
    for b in range(3):
        k[ke[b]:ke[b + 1], 0] = w[b]
    s = B.pooled_scores(q, k, qe, ke, 1, 2.0)
    assert np.array_equal(s[0], 2.0 * u @ w.T)


def test_group_mean_over_heads():
    """A GQA group's score is the mean of its heads' scores (one group per KV head)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((10, 4, 3))
    k = rng.standard_normal((10, 2, 3))
    e = [0, 5, 10]
    per_head = B.pooled_scores(q, k, e, e, 4, 1.0)   # one group per query head
    grouped = B.pooled_scores(q, k, e, e, 2, 1.0)    # one group per KV head
    assert np.allclose(grouped[0], per_head[0:2].mean(axis=0))
    assert np.allclose(grouped[1], per_head[2:4].mean(axis=0))


def test_group_spanning_two_kv_heads_is_rejected():
    q = np.zeros((4, 4, 2))
    k = np.zeros((4, 2, 2))
    with pytest.raises(AssertionError):
        B.pooled_scores(q, k, [0, 4], [0, 4], 1, 1.0)


def test_topk_on_pooled_scores_prefers_aligned_blocks():
    """Key blocks whose mean points along the query block's mean are kept first."""
    d = 2
    q = np.zeros((4, 1, d)); q[:, 0] = [1.0, 0.0]
    k = np.zeros((8, 1, d))
    k[0:2, 0] = [1.0, 0.0]; k[2:4, 0] = [-1.0, 0.0]; k[4:6, 0] = [0.5, 0.0]; k[6:8, 0] = [0.0, 1.0]
    s = B.pooled_scores(q, k, [0, 4], [0, 2, 4, 6, 8], 1, 1.0)
    keep = M.topk_keep(s, 50)  # k = 2
    assert keep[0, 0].tolist() == [True, False, True, False]
