"""Pins for the oracle's expert FFN, combine and whole layer.

The main pin is brute force: evaluate EVERY expert on EVERY token densely with
numpy matmuls and mix the outputs with the routing mask and gates; the sparse
oracle must agree to fp64 round-off.  Special cases reduce to closed forms:
k = E is the dense softmax mixture; identical experts give o + s whatever the
routing; zero up-projections leave only the shared expert.  AWQ weights are
unpacked by an independent numpy reading of the layout (tests/awq_ref.py)."""
import numpy as np
import pytest
from scipy.special import softmax

from tests import awq_ref, fp8_ref
from tests.helpers import bf16_bits_to_f64, f32_to_bf16_bits, random_bf16

import oracle as O


def _bf16_bank(rng, E, H, F, std=0.05):
    g, u, d = random_bf16(rng, (E, F, H), std), random_bf16(rng, (E, F, H), std), random_bf16(rng, (E, H, F), std)
    return O.Bank(E, H, F, O.Proj(O.BF16, H, F, w=g), O.Proj(O.BF16, H, F, w=u),
                  O.Proj(O.BF16, F, H, w=d))


def _awq_proj(rng, E, i, o, pow2_scales=False):
    q = rng.integers(0, 16, (E, i, o))
    z = rng.integers(0, 16, (E, i // 32, o))
    if pow2_scales:
        s = (2.0 ** rng.integers(-12, -4, (E, i // 32, o))).astype(np.float16)
    else:
        s = (np.abs(rng.standard_normal((E, i // 32, o))) * 0.002 + 1e-4).astype(np.float16)
    return O.Proj(O.AWQ, i, o, qweight=awq_ref.pack_nibbles(q), qzeros=awq_ref.pack_nibbles(z),
                  scales=s.view(np.uint16))


def _awq_bank(rng, E, H, F, pow2_scales=False):
    return O.Bank(E, H, F, _awq_proj(rng, E, H, F, pow2_scales), _awq_proj(rng, E, H, F, pow2_scales),
                  _awq_proj(rng, E, F, H, pow2_scales))


def _dense(p: O.Proj) -> np.ndarray:
    if p.fmt == O.BF16:
        return bf16_bits_to_f64(p.w)
    if p.fmt == O.FP8:
        return fp8_ref.dequant_dense(p.codes, p.bscales)
    return awq_ref.dequant_dense(p.qweight, p.qzeros, p.scales)


def _silu(a):
    return a / (1.0 + np.exp(-a))


def _all_expert_outputs(xd, bank):
    """[E, T, H]: every expert on every token."""
    Wg, Wu, Wd = _dense(bank.gate), _dense(bank.up), _dense(bank.down)
    out = np.empty((bank.num_experts, xd.shape[0], bank.hidden))
    for e in range(bank.num_experts):
        out[e] = (_silu(xd @ Wg[e].T) * (xd @ Wu[e].T)) @ Wd[e].T
    return out


def _brute_force(x, wr, k, bank, shared):
    logits, _ = O.router_logits(x, wr)
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    g = softmax(np.take_along_axis(logits, idx, 1).astype(np.float64), axis=1)
    xd = bf16_bits_to_f64(x)
    allout = _all_expert_outputs(xd, bank)
    mask = np.zeros((x.shape[0], bank.num_experts))
    np.put_along_axis(mask, idx, g, axis=1)
    y = np.einsum("te,eth->th", mask, allout)
    if shared is not None:
        y = y + _all_expert_outputs(xd, shared)[0]
    return y, idx, g


@pytest.mark.parametrize("fmt", ["bf16", "awq"])
@pytest.mark.parametrize("E,k", [(8, 2), (6, 6), (16, 3)])
def test_layer_equals_dense_brute_force(fmt, E, k):
    rng = np.random.default_rng(E * 10 + k + (fmt == "awq"))
    T, H, F = 12, 64, 32
    x = random_bf16(rng, (T, H))
    wr = random_bf16(rng, (E, H), 0.2)
    bank = _bf16_bank(rng, E, H, F) if fmt == "bf16" else _awq_bank(rng, E, H, F)
    shared = _bf16_bank(rng, 1, H, F)
    y, idx, g = O.layer(x, wr, k, bank, shared)
    yb, idxb, gb = _brute_force(x, wr, k, bank, shared)
    np.testing.assert_array_equal(idx, idxb)
    np.testing.assert_allclose(g, gb, rtol=1e-12)
    np.testing.assert_allclose(y, yb, rtol=1e-10, atol=1e-12)


def test_full_width_geometry_brute_force():
    """H = 2560, F = 640 (the pages' geometry), 32 experts, T = 2, k = 10."""
    rng = np.random.default_rng(11)
    T, H, F, E, k = 2, 2560, 640, 32, 10
    x = random_bf16(rng, (T, H))
    wr = random_bf16(rng, (E, H), 0.02)
    bank = _bf16_bank(rng, E, H, F, 0.02)
    shared = _bf16_bank(rng, 1, H, F, 0.02)
    y, idx, g = O.layer(x, wr, k, bank, shared)
    yb, idxb, _ = _brute_force(x, wr, k, bank, shared)
    np.testing.assert_array_equal(idx, idxb)
    np.testing.assert_allclose(y, yb, rtol=1e-9, atol=1e-12)


def test_full_width_awq_brute_force():
    rng = np.random.default_rng(12)
    T, H, F, E, k = 2, 2560, 640, 12, 10
    x = random_bf16(rng, (T, H))
    wr = random_bf16(rng, (E, H), 0.02)
    bank = _awq_bank(rng, E, H, F)
    y, idx, g = O.layer(x, wr, k, bank, None)
    yb, idxb, _ = _brute_force(x, wr, k, bank, None)
    np.testing.assert_array_equal(idx, idxb)
    np.testing.assert_allclose(y, yb, rtol=1e-9, atol=1e-12)


def test_identical_experts_give_single_expert_output():
    rng = np.random.default_rng(5)
    T, H, F, E, k = 9, 64, 32, 8, 3
    one = _bf16_bank(rng, 1, H, F)
    rep = lambda a: np.repeat(a, E, axis=0)
    bank = O.Bank(E, H, F, O.Proj(O.BF16, H, F, w=rep(one.gate.w)), O.Proj(O.BF16, H, F, w=rep(one.up.w)),
                  O.Proj(O.BF16, F, H, w=rep(one.down.w)))
    shared = _bf16_bank(rng, 1, H, F)
    x = random_bf16(rng, (T, H))
    y, _, _ = O.layer(x, random_bf16(rng, (E, H)), k, bank, shared)
    xd = bf16_bits_to_f64(x)
    ref = _all_expert_outputs(xd, one)[0] + _all_expert_outputs(xd, shared)[0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-13)


def test_zero_up_projection_leaves_shared_expert_only():
    rng = np.random.default_rng(6)
    T, H, F, E, k = 5, 64, 32, 8, 2
    bank = _bf16_bank(rng, E, H, F)
    bank.up.w[:] = 0
    shared = _bf16_bank(rng, 1, H, F)
    x = random_bf16(rng, (T, H))
    y, _, _ = O.layer(x, random_bf16(rng, (E, H)), k, bank, shared)
    np.testing.assert_array_equal(y, O.shared_outputs(x, shared))


def test_shared_scale_multiplies_shared_expert():
    rng = np.random.default_rng(8)
    T, H, F, E, k = 4, 32, 32, 4, 2
    bank, shared = _bf16_bank(rng, E, H, F), _bf16_bank(rng, 1, H, F)
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H))
    sc = np.array([0.0, 1.0, 2.0, -0.5])
    y0, idx, g = O.layer(x, wr, k, bank, None)
    y1, _, _ = O.layer(x, wr, k, bank, shared, shared_scale=sc)
    s = O.shared_outputs(x, shared)
    np.testing.assert_allclose(y1, y0 + sc[:, None] * s, rtol=1e-12, atol=1e-14)


def test_awq_weight_decode_matches_independent_unpack():
    rng = np.random.default_rng(13)
    E, i, o = 3, 64, 48
    p = _awq_proj(rng, E, i, o)
    dense = awq_ref.dequant_dense(p.qweight, p.qzeros, p.scales)
    for _ in range(300):
        e, oo, ii = rng.integers(0, E), rng.integers(0, o), rng.integers(0, i)
        assert O.proj_weight(p, e, oo, ii) == dense[e, oo, ii]


def test_awq_unit_scale_zero_eight_gives_code_minus_eight():
    rng = np.random.default_rng(14)
    E, i, o = 2, 32, 16
    q = rng.integers(0, 16, (E, i, o))
    p = O.Proj(O.AWQ, i, o, qweight=awq_ref.pack_nibbles(q),
               qzeros=awq_ref.pack_nibbles(np.full((E, 1, o), 8)),
               scales=np.ones((E, 1, o), np.float16).view(np.uint16))
    for e in range(E):
        for oo in range(o):
            for ii in range(i):
                assert O.proj_weight(p, e, oo, ii) == q[e, ii, oo] - 8


def test_awq_pack_unpack_round_trip():
    rng = np.random.default_rng(15)
    v = rng.integers(0, 16, (3, 5, 64))
    np.testing.assert_array_equal(awq_ref.unpack_nibbles(awq_ref.pack_nibbles(v)), v)


def test_awq_with_exact_bf16_weights_equals_bf16_path():
    """Power-of-two scales make every (q - z) * s exactly representable in bf16:
    the W4 layer must then equal the bf16 layer on the dequantised weights, bit for bit."""
    rng = np.random.default_rng(16)
    T, H, F, E, k = 6, 64, 32, 6, 2
    bank = _awq_bank(rng, E, H, F, pow2_scales=True)
    as_bf16 = lambda p: f32_to_bf16_bits(_dense(p).astype(np.float32))
    for p in (bank.gate, bank.up, bank.down):
        assert (bf16_bits_to_f64(as_bf16(p)) == _dense(p)).all()
    bbank = O.Bank(E, H, F, O.Proj(O.BF16, H, F, w=as_bf16(bank.gate)), O.Proj(O.BF16, H, F, w=as_bf16(bank.up)),
                   O.Proj(O.BF16, F, H, w=as_bf16(bank.down)))
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H))
    np.testing.assert_array_equal(O.layer(x, wr, k, bank)[0], O.layer(x, wr, k, bbank)[0])
