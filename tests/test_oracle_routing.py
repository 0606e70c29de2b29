"""Pins for ranking, gates and the pair permutation.

Ranking: logit descending, ties to the lower index (the tiny workload's rule),
checked against numpy's stable argsort.  Gates: softmax over all experts then
renormalised over the selected ones (architecture sheet: softmax gating,
selected weights renormalised), checked against scipy's softmax of the
selected logits -- the same quantity by a different route.  Permutation:
checked against numpy's stable sort of the flattened expert ids."""
import numpy as np
import pytest
from scipy.special import softmax


def _ties(rng, T, E, levels):
    return rng.integers(0, levels, (T, E)).astype(np.float32) * np.float32(0.25)


@pytest.mark.parametrize("E,n", [(16, 2), (16, 3), (512, 11), (256, 10), (5, 5)])
def test_rank_matches_stable_argsort(oracle, E, n):
    rng = np.random.default_rng(E * 31 + n)
    for l in (rng.standard_normal((40, E)).astype(np.float32), _ties(rng, 40, E, 4)):
        got = oracle.rank(l, n)
        ref = np.argsort(-l, axis=1, kind="stable")[:, :n]
        np.testing.assert_array_equal(got, ref)


def test_rank_equal_logits_take_lowest_indices(oracle):
    l = np.zeros((3, 16), np.float32)
    np.testing.assert_array_equal(oracle.rank(l, 4), np.tile(np.arange(4), (3, 1)))


def test_rank_signed_zeros_compare_equal(oracle):
    l = np.array([[-0.0, 0.0, -1.0, -0.0]], np.float32)
    np.testing.assert_array_equal(oracle.rank(l, 3), [[0, 1, 3]])


def test_rank_invariants(oracle):
    rng = np.random.default_rng(9)
    l = rng.standard_normal((64, 512)).astype(np.float32)
    idx = oracle.rank(l, 10)
    for t in range(64):
        assert len(set(idx[t].tolist())) == 10
        assert ((idx[t] >= 0) & (idx[t] < 512)).all()
        v = l[t, idx[t]]
        assert (np.diff(v) <= 0).all()
        assert v[-1] >= np.delete(l[t], idx[t]).max()


@pytest.mark.parametrize("E,k", [(16, 2), (512, 10), (7, 7)])
def test_gates_equal_softmax_of_selected(oracle, E, k):
    rng = np.random.default_rng(E + k)
    l = (rng.standard_normal((32, E)) * 3).astype(np.float32)
    idx = oracle.rank(l, k)
    g = oracle.gates(l, idx, k)
    ref = softmax(np.take_along_axis(l, idx, 1).astype(np.float64), axis=1)
    np.testing.assert_allclose(g, ref, rtol=1e-12, atol=0)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=1e-12)
    assert (g > 0).all()
    if k == E:  # every expert selected: the gates are the plain softmax
        full = softmax(l.astype(np.float64), axis=1)
        np.testing.assert_allclose(g, np.take_along_axis(full, idx, 1), rtol=1e-12)


def test_gates_with_wider_index_rows(oracle):
    """Refill rows carry k+1 indices; gates use only the first k."""
    rng = np.random.default_rng(1)
    l = rng.standard_normal((8, 32)).astype(np.float32)
    idx11 = oracle.rank(l, 11)
    g = oracle.gates(l, idx11, 10)
    np.testing.assert_allclose(g, oracle.gates(l, oracle.rank(l, 10), 10), rtol=0, atol=0)


@pytest.mark.parametrize("T,k,E", [(64, 2, 16), (16, 10, 512), (1000, 11, 512), (0, 10, 512),
                                   (3, 1, 1)])
def test_permute_matches_stable_sort(oracle, T, k, E):
    rng = np.random.default_rng(T + k + E)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    off, sp, p2r = oracle.permute(idx, E)
    flat = idx.ravel()
    np.testing.assert_array_equal(sp, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(p2r[sp], np.arange(T * k))
    for e in range(E):  # rows of expert e hold exactly its pairs, ascending
        grp = sp[off[e]:off[e + 1]]
        assert (flat[grp] == e).all() and (np.diff(grp) > 0).all()
