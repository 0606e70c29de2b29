"""Pins for the oracle's NVFP4 W4A4 experts (NVFP4 release card, precision
table: routed experts NVFP4 W4A4, group 16, FP8 block scales, FP32 global
scales; layouts and the activation recipe are the reading taken).

E2M1 values are checked against torch's E4M3 decode of the equivalent codes,
E2M1 rounding against midpoint thresholds, E4M3 rounding against torch's
float8_e4m3fn conversion, the quantiser on values it must reproduce, and the
W4A4 layer against dense brute force built from those pinned pieces."""
import numpy as np
import pytest
import torch

import oracle as O
from tests import fp8_ref
from tests.helpers import bf16_bits_to_f64, random_bf16
from tests.test_oracle_layer import _bf16_bank



def _e2m1_as_e4m3(c):
    """The E4M3 code of the same value: exponent field + 6 (bias 7 vs 1),
    mantissa bit in the top mantissa position; 0.5 (subnormal) is 2^-1."""
    sign, ex, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    if ex == 0:
        code = 0 if m == 0 else (6 << 3)
    else:
        code = ((ex + 6) << 3) | (m << 2)
    return (sign << 7) | code


def test_e2m1_values_match_e4m3_decode():
    for c in range(16):
        ref = fp8_ref.e4m3_decode(np.array([_e2m1_as_e4m3(c)], np.uint8))[0]
        assert O.e2m1_value(c) == ref, c
    assert [O.e2m1_value(c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _e2m1_round_ref(v):
    """Midpoint thresholds of the E2M1 grid; an exact midpoint goes to the
    neighbour whose mantissa bit is 0."""
    a = abs(v)
    lo_code = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    code = 7
    below = [0, 1, 2, 3, 4, 5, 6]
    for (t, tie), c in zip(lo_code, below):
        if a < t:
            code = c
            break
        if a == t:
            code = tie
            break
    return code | 8 if (code and v < 0) else code


def test_e2m1_round_against_midpoint_thresholds():
    rng = np.random.default_rng(31)
    vals = np.concatenate([rng.uniform(-8, 8, 4000), rng.uniform(-1, 1, 2000),
                           np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 100.0]),
                           # saturation far beyond 6, where fp32 distances to the grid tie
                           np.array([2.0**22, 2.0**22 + 1, 7.4e7, 1e30, 3.4e38, np.inf])])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    for v in vals:
        assert O.e2m1_round(v) == _e2m1_round_ref(float(v)), v


def test_e4m3_round_matches_torch():
    rng = np.random.default_rng(32)
    f = np.concatenate([np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 6000)),
                        rng.uniform(0, 2.0 ** -6, 500)]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties to even)
    vals = fp8_ref.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    f = np.concatenate([f, mids])
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(f, ref):
        assert O.e4m3_round(x) == r, (x, O.e4m3_round(x), r)
    assert O.e4m3_round(1e6) == 0x7E and O.e4m3_round(0.0) == 0


def test_quantizer_reproduces_values_on_its_grid():
    rng = np.random.default_rng(33)
    ga = 2.0 ** -9
    for _ in range(50):
        s = O.e4m3_value(int(rng.integers(0x28, 0x70)))
        codes = rng.integers(0, 16, 16)
        codes[0] = 7  # the group's largest magnitude is 6 * s
        v = np.array([O.e2m1_value(c) * s * ga for c in codes], np.float32)
        q = O.nvfp4_quantize(v, ga)
        np.testing.assert_array_equal(q * ga, v.astype(np.float64))
    assert not np.any(O.nvfp4_quantize(np.zeros(32, np.float32), 0.01))


def test_quantizer_error_is_bounded_by_half_a_grid_step():
    rng = np.random.default_rng(34)
    ga = 0.002
    v = rng.standard_normal(16 * 64).astype(np.float32)
    q = O.nvfp4_quantize(v, ga) * ga
    for g in range(64):
        blk, qb = v[16 * g:16 * g + 16].astype(np.float64), q[16 * g:16 * g + 16]
        # half of the widest grid step (4 -> 6) in units of the block scale,
        # which is amax / 6 rounded to E4M3 (at most 1/16 above)
        assert np.all(np.abs(qb - blk) <= np.max(np.abs(blk)) / 6 * (1 + 1 / 16) + 1e-12)


def _nvfp4_proj(rng, E, i, o, ga):
    codes = rng.integers(0, 256, (E, o, i // 2)).astype(np.uint8)
    gs = rng.integers(0x30, 0x49, (E, o, i // 16)).astype(np.uint8)
    wg = (0.004 * (1 + 0.1 * rng.random(E))).astype(np.float32)
    return O.Proj(O.NVFP4, i, o, codes=codes, gscales=gs, wglobal=wg, aglobal=ga)


def _dense_nvfp4(p):
    """[E][out][in] from an independent reading: nibble (low = even input),
    E2M1 via its E4M3 twin decoded by torch, group scale by torch, times the global scale."""
    E, o, i2 = p.codes.shape
    nib = np.empty((E, o, i2 * 2), np.uint8)
    nib[..., 0::2] = p.codes & 15
    nib[..., 1::2] = p.codes >> 4
    twin = np.vectorize(_e2m1_as_e4m3)(nib).astype(np.uint8)
    vals = fp8_ref.e4m3_decode(twin)
    sc = np.repeat(fp8_ref.e4m3_decode(p.gscales), 16, axis=2)
    return vals * sc * p.wglobal.astype(np.float64)[:, None, None]


def test_nvfp4_layer_equals_dense_brute_force():
    rng = np.random.default_rng(35)
    T, H, F, E, k = 7, 128, 64, 5, 2
    ga_gu, ga_dn = float(np.float32(0.002)), float(np.float32(0.0015))  # the scales are fp32
    bank = O.Bank(E, H, F, _nvfp4_proj(rng, E, H, F, ga_gu), _nvfp4_proj(rng, E, H, F, ga_gu),
                  _nvfp4_proj(rng, E, F, H, ga_dn))
    shared = _bf16_bank(rng, 1, H, F)
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H), 0.2)
    y, idx, g = O.layer(x, wr, k, bank, shared)
    # brute force: every expert on every token, with the pinned quantiser
    Wg, Wu, Wd = _dense_nvfp4(bank.gate), _dense_nvfp4(bank.up), _dense_nvfp4(bank.down)
    xd = bf16_bits_to_f64(x)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, idx, g, axis=1)
    ref = O.shared_outputs(x, shared).copy()
    for t in range(T):
        xq = O.nvfp4_quantize(xd[t].astype(np.float32), ga_gu) * ga_gu
        for e in range(E):
            if mask[t, e] == 0:
                continue
            a, u = Wg[e] @ xq, Wu[e] @ xq
            h = a / (1 + np.exp(-a)) * u
            hq = O.nvfp4_quantize(h.astype(np.float32), ga_dn) * ga_dn
            ref[t] += mask[t, e] * (Wd[e] @ hq)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-12)
