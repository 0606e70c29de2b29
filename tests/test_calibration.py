"""Refill-RMS calibration over a stream of packed rows and several layers,
with checkpoints of the additive statistics (RAZOR E256of512 card, "Selection
and calibration": packed rows of calibration text, valid tokens only,
statistics additive across rows, every layer ranked on its own)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from sparse_moe_expert_router_amd.calibration import RefillCalibration
from tests.gpu_helpers import bits, oracle_bank


def test_checkpoint_round_trip_is_exact(tmp_path):
    c = RefillCalibration(layers=3, experts=16, hidden=64, k=2, device="cpu")
    g = torch.Generator().manual_seed(0)
    c.stat_sum.copy_(torch.rand((3, 16), generator=g) * 1e3)
    c.stat_count.copy_(torch.randint(0, 2**31 - 1, (3, 16), generator=g, dtype=torch.int32))
    c.rows_done = 7
    path = str(tmp_path / "refill.npz")
    c.save(path)
    r = RefillCalibration.load(path, device="cpu")
    assert (r.layers, r.experts, r.hidden, r.k, r.rows_done) == (3, 16, 64, 2, 7)
    assert torch.equal(r.stat_sum, c.stat_sum) and torch.equal(r.stat_count, c.stat_count)
    # plain arrays only: loadable without unpickling
    with np.load(path, allow_pickle=False) as z:
        assert sorted(z.files) == ["geometry", "rows_done", "stat_count", "stat_sum"]


def test_rows_longer_than_a_packed_row_are_refused():
    c = RefillCalibration(layers=1, experts=16, hidden=64, k=2, device="cpu")
    with pytest.raises(ValueError):
        c.add(0, torch.zeros((32769, 64), dtype=torch.bfloat16), torch.zeros((16, 64)), {})


# ----------------------------------------------------------------------------- on the GPU

GEO = dict(H=256, F=128, Fs=128, E=64, k=8)
ROWS = [(300, 260), (512, 512), (200, 137)]  # (tokens in the row, valid tokens)
LAYERS = 3


def _row_inputs(w, r, T, device):
    return [workloads.activations(w, seed=1000 * r + l, device=device, T=T) for l in range(LAYERS)]


def _valid(T, n):
    v = np.zeros(T, np.uint8)
    v[:n] = 1
    return v


@pytest.mark.gpu
def test_stream_with_checkpoint_matches_uninterrupted_run_and_oracle(tmp_path):
    from tests.gpu_helpers import require_gpu
    require_gpu()
    w = workloads.scaled(workloads.get("refill_bf16"), T=512, keep=32, **GEO)
    layers = [(workloads.router(w, seed=50 + l, device="cuda"), workloads.expert_bank(w, seed=50 + l, device="cuda"))
              for l in range(LAYERS)]

    def run(calib, rows):
        for r in rows:
            T, n = ROWS[r]
            calib.add_row(_row_inputs(w, r, T, "cuda"), layers, torch.from_numpy(_valid(T, n)).cuda())

    full = RefillCalibration(LAYERS, w.E, w.H, w.k)
    run(full, [0, 1, 2])
    part = RefillCalibration(LAYERS, w.E, w.H, w.k)
    run(part, [0, 1])
    path = str(tmp_path / "refill.npz")
    part.save(path)
    resumed = RefillCalibration.load(path)
    assert resumed.rows_done == 2
    run(resumed, [2])
    torch.cuda.synchronize()
    # resuming from the checkpoint changes nothing, bit for bit
    assert torch.equal(resumed.stat_sum, full.stat_sum)
    assert torch.equal(resumed.stat_count, full.stat_count)
    ks_full, ks_res = full.keep_sets(w.keep), resumed.keep_sets(w.keep)
    for a, b in zip(ks_full, ks_res):
        for ta, tb in zip(a, b):
            assert torch.equal(ta, tb)

    # every layer against the oracle's full re-evaluation over the valid tokens of all rows
    g_sum, g_cnt = full.stat_sum.cpu().numpy(), full.stat_count.cpu().numpy()
    for l in range(LAYERS):
        s = np.zeros(w.E)
        c = np.zeros(w.E, np.int64)
        ob = oracle_bank(layers[l][1])
        for r, (T, n) in enumerate(ROWS):
            xb = bits(_row_inputs(w, r, T, "cuda")[l])
            lg, _ = O.router_logits(xb, bits(layers[l][0]))
            O.refill_accumulate(xb, lg, w.k, ob, None, s, c, valid=_valid(T, n))
        np.testing.assert_array_equal(g_cnt[l].astype(np.int64), c)
        assert c.sum() == w.k * sum(n for _, n in ROWS)
        ref_score = np.where(c > 0, np.sqrt(s / np.maximum(c, 1) / w.H), 0.0)
        got_score = ks_full[l][0].cpu().numpy()
        np.testing.assert_allclose(got_score, ref_score, rtol=1e-3, err_msg=f"layer {l}")
        np.testing.assert_allclose(g_sum[l], s, rtol=1e-3, err_msg=f"layer {l}")
