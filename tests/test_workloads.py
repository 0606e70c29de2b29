"""The seeded input generator: shapes, reproducibility and value recipe."""
import numpy as np
import torch

import workloads
from tests import awq_ref
from tests.helpers import bf16_bits_to_f64


def test_tiny_shapes_and_reproducibility():
    w = workloads.get("tiny_bf16")
    a = workloads.generate(w, seed=0)
    b = workloads.generate(w, seed=0)
    c = workloads.generate(w, seed=0, copy=1)
    assert a["x"].shape == (64, 256) and a["x"].dtype == torch.bfloat16
    assert a["router"].shape == (16, 256)
    assert a["experts"]["gate"].shape == (16, 128, 256)
    assert a["experts"]["down"].shape == (16, 256, 128)
    assert a["shared"]["gate"].shape == (1, 128, 256)
    for key in ("x", "router"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert torch.equal(a["experts"]["down"], b["experts"]["down"])


def test_value_recipe():
    w = workloads.scaled(workloads.get("decode_awq"), E=4, T=256)
    d = workloads.generate(w, seed=0)
    x = bf16_bits_to_f64(workloads.bits(d["x"]))
    assert abs(x.std() - 1.0) < 0.02 and abs(x.mean()) < 0.02
    r = bf16_bits_to_f64(workloads.bits(d["router"]))
    assert abs(r.std() - 0.02) < 0.001
    ex = workloads.bank_numpy(d["experts"])
    assert ex["gate_qweight"].shape == (4, 2560, 80)
    assert ex["gate_qzeros"].shape == (4, 80, 80)
    assert ex["gate_scales"].shape == (4, 80, 640)
    assert ex["down_qweight"].shape == (4, 640, 320)
    q = awq_ref.unpack_nibbles(ex["gate_qweight"])
    counts = np.bincount(q.ravel(), minlength=16) / q.size
    assert np.abs(counts - 1 / 16).max() < 0.002
    s = ex["down_scales"].view(np.float16).astype(np.float64)
    assert s.min() >= 9.9e-5 and abs(s.mean() - (0.002 * np.sqrt(2 / np.pi) + 1e-4)) < 1e-4


def test_keep_set_is_seeded_sorted_subset():
    w = workloads.get("pruned_awq")
    k1, k2 = workloads.keep_set(w, 0), workloads.keep_set(w, 0)
    assert torch.equal(k1, k2)
    k = k1.numpy()
    assert len(k) == 256 and len(set(k.tolist())) == 256
    assert (np.diff(k) > 0).all() and k.min() >= 0 and k.max() < 512
