"""Pins for the Refill-RMS statistics and keep-set (RAZOR E256of512 card,
"Selection and calibration": drop a selected expert, promote the
highest-ranked unselected one, RMS of the output change conditional on the
tokens routed to each expert, additive statistics).

The oracle re-evaluates the whole layer output for every drop.  It is checked
against: closed forms (k = 1 gives o_r - o_j; identical experts give zero),
invariances (shared expert; a global scale of the down projections), the
algebraic shortcut computed from per-pair outputs, exact counts, additivity
over batches and numpy's stable sort for the keep-set."""
import numpy as np
import pytest

from tests.helpers import bf16_bits_to_f64, random_bf16

import oracle as O
from tests.test_oracle_layer import _bf16_bank


def _setup(seed, T=24, H=32, F=32, E=12, k=3, std=0.1):
    rng = np.random.default_rng(seed)
    x = random_bf16(rng, (T, H))
    wr = random_bf16(rng, (E, H), 0.3)
    bank = _bf16_bank(rng, E, H, F, std)
    shared = _bf16_bank(rng, 1, H, F, std)
    logits, _ = O.router_logits(x, wr)
    return rng, x, wr, bank, shared, logits


def _acc(x, logits, k, bank, shared, valid=None):
    E = logits.shape[1]
    s, c = np.zeros(E), np.zeros(E, np.int64)
    O.refill_accumulate(x, logits, k, bank, shared, s, c, valid)
    return s, c


def test_counts_are_bincount_of_selected():
    _, x, _, bank, shared, logits = _setup(1)
    k = 3
    s, c = _acc(x, logits, k, bank, shared)
    idx = O.rank(logits, k)
    np.testing.assert_array_equal(c, np.bincount(idx.ravel(), minlength=logits.shape[1]))


def test_k1_delta_is_difference_of_two_experts():
    _, x, _, bank, shared, logits = _setup(2, k=1)
    s, c = _acc(x, logits, 1, bank, shared)
    idx2 = O.rank(logits, 2)
    rows = O.pair_outputs(x, idx2, bank).reshape(x.shape[0], 2, -1)
    ref = np.zeros(logits.shape[1])
    for t in range(x.shape[0]):
        ref[idx2[t, 0]] += np.sum((rows[t, 1] - rows[t, 0]) ** 2)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-15)


def test_identical_experts_score_zero():
    rng, x, _, bank, shared, logits = _setup(3)
    for p in (bank.gate, bank.up, bank.down):
        p.w[:] = p.w[0:1]
    s, c = _acc(x, logits, 3, bank, shared)
    assert (c.sum() == 3 * x.shape[0])
    assert np.abs(s).max() < 1e-24


def test_invariant_to_shared_expert():
    _, x, _, bank, shared, logits = _setup(4)
    s1, c1 = _acc(x, logits, 3, bank, shared)
    s0, c0 = _acc(x, logits, 3, bank, None)
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_allclose(s1, s0, rtol=1e-9, atol=1e-20)


def test_scaling_down_projection_scales_scores():
    _, x, _, bank, shared, logits = _setup(5)
    s1, c1 = _acc(x, logits, 3, bank, shared)
    bank.down.w[:] = (bank.down.w.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1: x2 exactly
    s2, c2 = _acc(x, logits, 3, bank, shared)
    np.testing.assert_allclose(s2, 4.0 * s1, rtol=1e-12, atol=0)
    sc1, _, _ = O.refill_finalize(s1, c1, bank.hidden, 6)
    sc2, _, _ = O.refill_finalize(s2, c2, bank.hidden, 6)
    np.testing.assert_allclose(sc2, 2.0 * sc1, rtol=1e-12, atol=0)


def test_matches_algebraic_shortcut():
    """Delta_j = (A - p_j o_j + p_r o_r)/Z' - A/Z, A = sum_S p o, Z = sum_S p."""
    _, x, _, bank, shared, logits = _setup(6)
    k = 3
    s, c = _acc(x, logits, k, bank, shared)
    T, E = logits.shape
    idx = O.rank(logits, k + 1)
    rows = O.pair_outputs(x, idx, bank).reshape(T, k + 1, -1)
    l64 = logits.astype(np.float64)
    ref = np.zeros(E)
    for t in range(T):
        p = np.exp(l64[t, idx[t]] - l64[t].max())
        A = (p[:k, None] * rows[t, :k]).sum(0)
        Z = p[:k].sum()
        for j in range(k):
            Z2 = Z - p[j] + p[k]
            d = (A - p[j] * rows[t, j] + p[k] * rows[t, k]) / Z2 - A / Z
            ref[idx[t, j]] += np.dot(d, d)
    np.testing.assert_allclose(s, ref, rtol=1e-9, atol=1e-20)


def test_statistics_are_additive_and_respect_valid_mask():
    _, x, _, bank, shared, logits = _setup(7, T=20)
    s_all, c_all = _acc(x, logits, 3, bank, shared)
    s_a, c_a = _acc(x[:7], logits[:7], 3, bank, shared)
    s_b, c_b = _acc(x[7:], logits[7:], 3, bank, shared)
    np.testing.assert_array_equal(c_a + c_b, c_all)
    np.testing.assert_allclose(s_a + s_b, s_all, rtol=1e-12, atol=1e-20)
    valid = np.zeros(20, np.uint8)
    valid[:7] = 1
    s_v, c_v = _acc(x, logits, 3, bank, shared, valid)
    np.testing.assert_array_equal(c_v, c_a)
    np.testing.assert_allclose(s_v, s_a, rtol=1e-12, atol=1e-20)


def test_finalize_ranks_with_lowest_index_ties_and_zero_counts():
    s = np.array([4.0, 0.0, 4.0, 9.0, 1.0, 4.0])
    c = np.array([1, 0, 1, 1, 4, 1], np.int64)
    score, mask, keep = O.refill_finalize(s, c, 1, 4)
    np.testing.assert_allclose(score, [2.0, 0.0, 2.0, 3.0, 0.5, 2.0])
    np.testing.assert_array_equal(keep, [0, 2, 3, 5])
    np.testing.assert_array_equal(mask, [1, 0, 1, 1, 0, 1])


@pytest.mark.parametrize("E,keep", [(512, 256), (512, 384), (16, 8)])
def test_finalize_matches_lexsort(E, keep):
    rng = np.random.default_rng(E + keep)
    s = np.round(rng.random(E) * 8) / 4  # many ties
    c = rng.integers(0, 5, E).astype(np.int64)
    H = 2560
    score, mask, kidx = O.refill_finalize(s, c, H, keep)
    ref_score = np.where(c > 0, np.sqrt(s / np.maximum(c, 1) / H), 0.0)
    np.testing.assert_allclose(score, ref_score, rtol=1e-15)
    order = np.lexsort((np.arange(E), -score))
    np.testing.assert_array_equal(kidx, np.sort(order[:keep]))
    assert mask.sum() == keep and (mask[kidx] == 1).all()
