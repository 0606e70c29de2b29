"""Pins for the oracle's router logits: the correctly rounded fp32 value of the
exact dot product (a reading of the architecture sheet's softmax router over
fp32 logits).  Checked against exact rational arithmetic, not against itself."""
import numpy as np
import pytest

from tests.helpers import exact_dot, f32_to_bf16_bits, is_rne_f32, random_bf16


def _cases(rng):
    H = 96
    yield "gaussian", random_bf16(rng, H), random_bf16(rng, H, 0.02)
    # wide exponent spread: forces roundings in a double accumulator
    a = rng.standard_normal(H).astype(np.float32) * np.float32(2.0) ** rng.integers(-60, 60, H)
    b = rng.standard_normal(H).astype(np.float32) * np.float32(2.0) ** rng.integers(-60, 60, H)
    yield "spread", f32_to_bf16_bits(a), f32_to_bf16_bits(b)
    # heavy cancellation: pairs that cancel plus a tiny remainder
    v = rng.standard_normal(H // 2).astype(np.float32)
    a = np.concatenate([v, v, [np.float32(1e-30)]]).astype(np.float32)
    b = np.concatenate([np.ones(H // 2), -np.ones(H // 2), [np.float32(3.0)]]).astype(np.float32)
    yield "cancel", f32_to_bf16_bits(a), f32_to_bf16_bits(b)
    # subnormal bf16 operands and products
    a = np.array([1e-39, -2e-39, 3e-38, 1.0, 5e-40], np.float32)
    b = np.array([1e-38, 1.0, 1e-39, 1e-39, 2.0], np.float32)
    yield "subnormal", f32_to_bf16_bits(a), f32_to_bf16_bits(b)
    # a sum that lands exactly halfway between two binary32 values
    a = np.array([1.0, 2.0 ** -24], np.float32)
    b = np.array([1.0, 1.0], np.float32)
    yield "tie_even", f32_to_bf16_bits(a), f32_to_bf16_bits(b)
    a = np.array([1.0 + 2.0 ** -7, 2.0 ** -24, 2.0 ** -24], np.float32)
    yield "tie_odd", f32_to_bf16_bits(a[:2]), f32_to_bf16_bits(np.array([1.0, 1.0], np.float32))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_dot_is_rne_of_rational_sum(oracle, seed):
    rng = np.random.default_rng(seed)
    for name, a, b in _cases(rng):
        got = oracle.dot_exact_f32(a, b)
        assert is_rne_f32(exact_dot(a, b), got), name


def test_certified_path_agrees_with_fixed_point(oracle):
    rng = np.random.default_rng(7)
    n_cert = 0
    for _ in range(200):
        a, b = random_bf16(rng, 256), random_bf16(rng, 256, 0.02)
        ok, s = oracle.dot_certified(a, b)
        if ok:
            n_cert += 1
            assert np.float32(s) == oracle.dot_exact_f32(a, b)
    assert n_cert > 150


def test_router_logits_against_rationals_including_fallback(oracle):
    rng = np.random.default_rng(3)
    T, H, E = 6, 64, 5
    x = random_bf16(rng, (T, H))
    w = random_bf16(rng, (E, H), 0.02)
    # one token with a wide exponent spread so that the double path cannot certify
    spread = rng.standard_normal(H).astype(np.float32) * np.float32(2.0) ** rng.integers(-70, 70, H)
    x[0] = f32_to_bf16_bits(spread)
    logits, nfb = oracle.router_logits(x, w)
    assert nfb > 0
    for t in range(T):
        for e in range(E):
            assert is_rne_f32(exact_dot(x[t], w[e]), logits[t, e]), (t, e)


def test_one_hot_tokens_read_router_columns(oracle):
    rng = np.random.default_rng(4)
    H, E = 32, 7
    w = random_bf16(rng, (E, H), 0.02)
    x = f32_to_bf16_bits(np.eye(H, dtype=np.float32))
    logits, _ = oracle.router_logits(x, w)
    wv = (w.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(logits, wv.T)
