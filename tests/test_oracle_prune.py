"""Pins for expert pruning and the layer geometry.

RAZOR cards (E256of512 / E384of512, property tables): pruning only slices
router rows and expert weights.  The parameter counts printed on the pages are
reproduced exactly by the workloads' geometry (hidden 2560, width 640, three
bias-free projections per expert, one router row per expert, no router bias),
which pins those constants.  Router-norm keep policy checked against numpy."""
import json
import os

import numpy as np

import oracle as O
import workloads
from tests.helpers import bf16_bits_to_f64, random_bf16
from tests.test_oracle_layer import _awq_bank, _bf16_bank

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "param_counts.json")))


def _per_expert_params(H, F):
    return 3 * H * F + H  # gate, up, down (no bias) + one router row


def test_parameter_counts_pin_geometry():
    w = workloads.get("decode_bf16")
    assert (w.H, w.F, w.E, w.k, w.Fs) == (GOLD["d_model"], GOLD["expert_width"], GOLD["experts"],
                                          GOLD["top_k"], GOLD["shared_width"])
    per = _per_expert_params(w.H, w.F)
    L = GOLD["layers"]
    assert GOLD["main_lm_base"] - GOLD["main_lm_e256"] == L * 256 * per
    assert GOLD["main_lm_base"] - GOLD["main_lm_e384"] == L * 128 * per
    assert GOLD["mtp_base"] - GOLD["mtp_e256"] == GOLD["mtp_moe_layers"] * 256 * per
    assert GOLD["mtp_base"] - GOLD["mtp_e384"] == GOLD["mtp_moe_layers"] * 128 * per
    assert GOLD["complete_base"] - GOLD["complete_e256"] == (L + 1) * 256 * per
    assert GOLD["complete_base"] - GOLD["complete_e384"] == (L + 1) * 128 * per


def test_active_parameter_convention():
    w = workloads.get("decode_bf16")
    routed = GOLD["layers"] * w.E * 3 * w.H * w.F
    non_expert = GOLD["main_lm_base"] - routed - GOLD["embedding_plus_head_b"] * 1e9
    active = non_expert + routed * w.k / w.E
    assert abs(active / 1e9 - GOLD["active_non_embedding_b"]) < 0.001


def test_pruned_logits_are_columns_of_base_logits():
    rng = np.random.default_rng(21)
    T, H, E = 40, 128, 32
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H), 0.02)
    keep = np.sort(rng.choice(E, 16, replace=False)).astype(np.int32)
    bank = _awq_bank(rng, E, H, 32)
    wr2, bank2 = O.prune_slice(wr, bank, keep)
    base, _ = O.router_logits(x, wr)
    pruned, _ = O.router_logits(x, wr2)
    np.testing.assert_array_equal(pruned, base[:, keep])
    for name in ("qweight", "qzeros", "scales"):
        np.testing.assert_array_equal(getattr(bank2.down, name), getattr(bank.down, name)[keep])


def test_pruned_layer_equals_base_layer_with_dropped_experts_masked():
    rng = np.random.default_rng(22)
    T, H, F, E, k = 10, 64, 32, 12, 3
    x, wr = random_bf16(rng, (T, H)), random_bf16(rng, (E, H), 0.2)
    keep = np.sort(rng.choice(E, 6, replace=False)).astype(np.int32)
    bank = _bf16_bank(rng, E, H, F)
    wr2, bank2 = O.prune_slice(wr, bank, keep)
    y2, idx2, g2 = O.layer(x, wr2, k, bank2)
    base, _ = O.router_logits(x, wr)
    masked = np.full_like(base, -np.inf)
    masked[:, keep] = base[:, keep]
    idx = O.rank(masked, k)
    np.testing.assert_array_equal(keep[idx2], idx)
    g = O.gates(masked, idx, k)
    np.testing.assert_allclose(g2, g, rtol=1e-14)
    rows = O.pair_outputs(x, idx, bank)
    np.testing.assert_allclose(y2, O.combine(rows, g), rtol=1e-12, atol=1e-15)


def test_router_norm_keep_matches_lexsort():
    rng = np.random.default_rng(23)
    E, H = 64, 256
    wr = random_bf16(rng, (E, H), 0.02)
    wr[5] = wr[9]  # a tie: the lower index must win
    norm, keep = O.router_norm_keep(wr, 20)
    ref = np.sqrt((bf16_bits_to_f64(wr) ** 2).sum(1))
    np.testing.assert_allclose(norm, ref, rtol=1e-14)
    order = np.lexsort((np.arange(E), -norm))
    np.testing.assert_array_equal(keep, np.sort(order[:20]))
