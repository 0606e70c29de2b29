"""Pins for the oracle's grouped fp64 evaluation (oracle/grouped.py).

The grouped path restates the expert output and the Refill-RMS
re-evaluation (RAZOR E256of512 card, "Selection and calibration") with one
fp64 matrix product per expert.  It must agree with the per-pair C oracle,
whose own pins are brute-force dense evaluation and the Refill-RMS closed
forms, to fp64 rounding; its weight decode must equal the C oracle's
element by element."""
import numpy as np
import pytest

import oracle as O
from oracle import grouped as G
from tests.helpers import random_bf16
from tests.test_oracle_layer import _awq_bank, _bf16_bank


def _bank(fmt, rng, E, H, F):
    return _bf16_bank(rng, E, H, F, 0.05) if fmt == "bf16" else _awq_bank(rng, E, H, F)


@pytest.mark.parametrize("fmt", ["bf16", "awq"])
def test_weight_decode_equals_c_oracle(fmt):
    rng = np.random.default_rng(5)
    E, H, F = 3, 64, 64
    bank = _bank(fmt, rng, E, H, F)
    for p in (bank.gate, bank.up, bank.down):
        for e in range(E):
            m = G.proj_matrix(p, e)
            assert m.shape == (p.out_dim, p.in_dim)
            for o, i in zip(rng.integers(0, p.out_dim, 40), rng.integers(0, p.in_dim, 40)):
                assert m[o, i] == O.proj_weight(p, e, int(o), int(i))


@pytest.mark.parametrize("fmt", ["bf16", "awq"])
def test_expert_outputs_equal_pair_outputs(fmt):
    rng = np.random.default_rng(6)
    T, H, F, E, k = 20, 64, 64, 6, 3
    bank = _bank(fmt, rng, E, H, F)
    x = random_bf16(rng, (T, H))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ref = O.pair_outputs(x, idx, bank)
    got = G.expert_outputs(x, idx, bank)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max())
    # a subset of pairs, in any order
    pairs = np.array([[3, 2], [0, 0], [19, 1], [3, 0]])
    sub = G.expert_outputs(x, idx, bank, pairs=pairs)
    np.testing.assert_allclose(sub, ref[pairs[:, 0] * k + pairs[:, 1]], rtol=1e-12,
                               atol=1e-14 * np.abs(ref).max())


@pytest.mark.parametrize("fmt", ["bf16", "awq"])
def test_refill_equals_c_oracle(fmt):
    rng = np.random.default_rng(7)
    T, H, F, E, k = 40, 64, 64, 10, 3
    bank = _bank(fmt, rng, E, H, F)
    x = random_bf16(rng, (T, H))
    wr = random_bf16(rng, (E, H), 0.3)
    logits, _ = O.router_logits(x, wr)
    valid = (rng.random(T) < 0.8).astype(np.uint8)
    rs, rc = np.zeros(E), np.zeros(E, np.int64)
    O.refill_accumulate(x, logits, k, bank, None, rs, rc, valid)
    gs, gc = np.zeros(E), np.zeros(E, np.int64)
    G.refill_accumulate(x, logits, k, bank, gs, gc, valid=valid, chunk=7)
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_allclose(gs, rs, rtol=1e-10, atol=1e-14 * rs.max())
    # a token subset adds exactly the statistics of those tokens
    toks = np.array([1, 5, 6, 30])
    ss, sc = np.zeros(E), np.zeros(E, np.int64)
    G.refill_accumulate(x, logits, k, bank, ss, sc, tokens=toks)
    rs2, rc2 = np.zeros(E), np.zeros(E, np.int64)
    O.refill_accumulate(x[toks], logits[toks], k, bank, None, rs2, rc2)
    np.testing.assert_array_equal(sc, rc2)
    np.testing.assert_allclose(ss, rs2, rtol=1e-10, atol=1e-14 * max(rs2.max(), 1e-300))


def test_output_major_awq_decodes_like_awq():
    """The output-major code layout holds the same codes: every weight the
    oracle decodes from it equals the AWQ decode (itself pinned by the
    independent unpacker and dense brute force), and so do the grouped
    matrices."""
    from tests import awq_ref
    rng = np.random.default_rng(8)
    E, H, F = 2, 64, 96
    a = _awq_bank(rng, E, H, F)
    om = {}
    for n, p in (("gate", a.gate), ("up", a.up), ("down", a.down)):
        om[n] = O.Proj(O.AWQ_OM, p.in_dim, p.out_dim, qweight=awq_ref.to_output_major(p.qweight),
                       qzeros=p.qzeros, scales=p.scales)
    b = O.Bank(E, H, F, om["gate"], om["up"], om["down"])
    for pa, pb in ((a.gate, b.gate), (a.up, b.up), (a.down, b.down)):
        for e in range(E):
            for o in range(pa.out_dim):
                for i in range(0, pa.in_dim, 7):
                    assert O.proj_weight(pa, e, o, i) == O.proj_weight(pb, e, o, i)
            np.testing.assert_array_equal(G.proj_matrix(pa, e), G.proj_matrix(pb, e))
    x = random_bf16(rng, (5, H))
    idx = np.array([[0, 1]] * 5, np.int32)
    np.testing.assert_array_equal(O.pair_outputs(x, idx, a), O.pair_outputs(x, idx, b))
