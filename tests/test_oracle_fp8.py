"""Pins for the oracle's FP8 E4M3 block-scaled experts (AWQ-g32 card,
"Optional FP8 MTP": routed experts in FP8 E4M3 with explicit block scales;
128 x 128 blocks of fp32 scales are the reading taken).  The code decode is
checked against torch's float8_e4m3fn conversion on every code, the layer
against dense brute force, and the block indexing by zeroing one block."""
import numpy as np

import oracle as O
from tests import fp8_ref
from tests.helpers import bf16_bits_to_f64, f32_to_bf16_bits, random_bf16
from tests.test_oracle_layer import _bf16_bank, _brute_force


def _fp8_proj(rng, E, i, o, unit_scales=False):
    codes = fp8_ref.random_codes(rng, (E, o, i))
    if unit_scales:
        s = np.ones((E, o // 128, i // 128), np.float32)
    else:
        s = (np.abs(rng.standard_normal((E, o // 128, i // 128))) * 1e-3 + 1e-5).astype(np.float32)
    return O.Proj(O.FP8, i, o, codes=codes, bscales=s)


def _fp8_bank(rng, E, H, F, unit_scales=False):
    return O.Bank(E, H, F, _fp8_proj(rng, E, H, F, unit_scales), _fp8_proj(rng, E, H, F, unit_scales),
                  _fp8_proj(rng, E, F, H, unit_scales))


def test_e4m3_decode_matches_torch_on_every_code():
    ref = fp8_ref.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        v = O.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


def test_fp8_weight_decode_matches_dense_reading():
    rng = np.random.default_rng(21)
    p = _fp8_proj(rng, 2, 256, 384)
    dense = fp8_ref.dequant_dense(p.codes, p.bscales)
    for _ in range(400):
        e, o, i = rng.integers(0, 2), rng.integers(0, 384), rng.integers(0, 256)
        assert O.proj_weight(p, e, o, i) == dense[e, o, i]


def test_fp8_layer_equals_dense_brute_force():
    rng = np.random.default_rng(22)
    T, H, F, E, k = 10, 256, 128, 6, 2
    x = random_bf16(rng, (T, H))
    wr = random_bf16(rng, (E, H), 0.2)
    bank = _fp8_bank(rng, E, H, F)
    shared = _bf16_bank(rng, 1, H, F)
    y, idx, g = O.layer(x, wr, k, bank, shared)
    yb, idxb, _ = _brute_force(x, wr, k, bank, shared)
    np.testing.assert_array_equal(idx, idxb)
    np.testing.assert_allclose(y, yb, rtol=1e-10, atol=1e-12)


def test_fp8_unit_scales_equal_the_bf16_path():
    """Every finite E4M3 value is exactly a bf16 value: with unit scales the FP8
    layer equals the bf16 layer on the decoded weights, bit for bit."""
    rng = np.random.default_rng(23)
    T, H, F, E, k = 6, 128, 128, 4, 2
    bank = _fp8_bank(rng, E, H, F, unit_scales=True)
    as_bf16 = lambda p: f32_to_bf16_bits(fp8_ref.dequant_dense(p.codes, p.bscales).astype(np.float32))
    for p in (bank.gate, bank.up, bank.down):
        assert (bf16_bits_to_f64(as_bf16(p)) == fp8_ref.dequant_dense(p.codes, p.bscales)).all()
    bbank = O.Bank(E, H, F, O.Proj(O.BF16, H, F, w=as_bf16(bank.gate)), O.Proj(O.BF16, H, F, w=as_bf16(bank.up)),
                   O.Proj(O.BF16, F, H, w=as_bf16(bank.down)))
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H))
    np.testing.assert_array_equal(O.layer(x, wr, k, bank)[0], O.layer(x, wr, k, bbank)[0])


def test_fp8_zero_block_scale_equals_zero_codes_in_that_block():
    """A zero scale for block (out 128..255, in 0..127) of the gate projection
    must act exactly like zero codes there (a transposed block index would not)."""
    rng = np.random.default_rng(24)
    T, H, F, E, k = 5, 256, 384, 3, 2
    bank = _fp8_bank(rng, E, H, F)
    a = O.Bank(E, H, F, O.Proj(O.FP8, H, F, codes=bank.gate.codes, bscales=bank.gate.bscales.copy()),
               bank.up, bank.down)
    a.gate.bscales[:, 1, 0] = 0.0
    codes = bank.gate.codes.copy()
    codes[:, 128:256, 0:128] = 0
    b = O.Bank(E, H, F, O.Proj(O.FP8, H, F, codes=codes, bscales=bank.gate.bscales), bank.up, bank.down)
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H))
    ya, yb = O.layer(x, wr, k, a)[0], O.layer(x, wr, k, b)[0]
    np.testing.assert_array_equal(ya, yb)
    assert not np.array_equal(ya, O.layer(x, wr, k, bank)[0])
