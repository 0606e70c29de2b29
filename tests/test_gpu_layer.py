"""GPU parity of the whole layer and of Refill-RMS against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.gpu_helpers import bits, check_close, oracle_bank, require_gpu

pytestmark = pytest.mark.gpu


def oracle_layer_sparse(x, wr, k, bank, shared, tokens=None, shared_scale=None):
    """Oracle layer for the given tokens, decoding only the experts they route to."""
    xb = bits(x)
    if tokens is not None:
        xb = xb[np.asarray(tokens)]
    logits, _ = O.router_logits(xb, bits(wr))
    idx = O.rank(logits, k)
    g = O.gates(logits, idx, k)
    used = np.unique(idx)
    local = np.searchsorted(used, idx).astype(np.int32)
    rows = O.pair_outputs(xb, local, oracle_bank(bank, used))
    s = O.shared_outputs(xb, oracle_bank(shared)) if shared is not None else None
    return O.combine(rows, g, s, shared_scale), idx, g


@pytest.mark.parametrize("name", ["tiny_bf16", "decode_bf16", "decode_awq", "decode_fp8", "decode_nvfp4"])
def test_layer_matches_oracle(name):
    moe = require_gpu()
    w = workloads.get(name)
    d = workloads.generate(w, device="cuda")
    y, mid = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"], keep_intermediates=True)
    torch.cuda.synchronize()
    ref_y, ref_idx, ref_g = oracle_layer_sparse(d["x"], d["router"], w.k, d["experts"], d["shared"])
    np.testing.assert_array_equal(mid["idx"].cpu().numpy(), ref_idx)
    np.testing.assert_allclose(mid["gate"].cpu().numpy(), ref_g, rtol=1e-5, atol=1e-7)
    ro, rs, rp = O.permute(ref_idx, w.E)
    np.testing.assert_array_equal(mid["offsets"].cpu().numpy(), ro)
    np.testing.assert_array_equal(mid["sorted_pair"].cpu().numpy(), rs)
    check_close(y.float().cpu().numpy(), ref_y, name)


def test_layer_with_shared_scale():
    moe = require_gpu()
    w = workloads.get("tiny_bf16")
    d = workloads.generate(w, device="cuda")
    sc = torch.linspace(-1.0, 2.0, w.T, device="cuda")
    y = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"], shared_scale=sc)
    torch.cuda.synchronize()
    ref_y, _, _ = oracle_layer_sparse(d["x"], d["router"], w.k, d["experts"], d["shared"],
                                      shared_scale=sc.double().cpu().numpy())
    check_close(y.float().cpu().numpy(), ref_y, "shared scale")


def test_layer_is_deterministic():
    moe = require_gpu()
    w = workloads.get("decode_awq")
    d = workloads.generate(w, device="cuda")
    a = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"]).clone()
    b = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"])
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["decode_bf16", "tiny_bf16"])
def test_layer_with_shared_expert_on_a_second_stream(name):
    """The shared expert beside the routed path on its own stream gives the same bits."""
    moe = require_gpu()
    w = workloads.get(name)
    d = workloads.generate(w, device="cuda")
    ref = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"]).clone()
    side = torch.cuda.Stream()
    for _ in range(3):
        y = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"], shared_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


# ----------------------------------------------------------------------------- Refill-RMS

def _gpu_refill(moe, d, w, keep, batches=1):
    E = w.E
    stat_sum = torch.zeros(E, dtype=torch.float32, device="cuda")
    stat_count = torch.zeros(E, dtype=torch.int32, device="cuda")
    T = w.T
    bounds = np.linspace(0, T, batches + 1).astype(int)
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        x = d["x"][b0:b1]
        idx, tl, gate, _ = moe.route(x, d["router"], w.k, extra=1)
        off, sp, p2r = moe.permute(idx, E)
        rows = moe.grouped_ffn(x, w.k + 1, d["experts"], off, sp, out_dtype=moe.OUT_F32)
        moe.refill_score(rows, off, sp, p2r, tl, stat_sum, stat_count)
    score, mask, kidx = moe.refill_finalize(stat_sum, stat_count, w.H, keep)
    torch.cuda.synchronize()
    return (stat_sum.cpu().numpy(), stat_count.cpu().numpy(), score.cpu().numpy(),
            mask.cpu().numpy(), kidx.cpu().numpy())


def _oracle_refill(d, w, keep):
    logits, _ = O.router_logits(bits(d["x"]), bits(d["router"]))
    s = np.zeros(w.E)
    c = np.zeros(w.E, np.int64)
    O.refill_accumulate(bits(d["x"]), logits, w.k, oracle_bank(d["experts"]), oracle_bank(d["shared"]), s, c)
    score, mask, kidx = O.refill_finalize(s, c, w.H, keep)
    return s, c, score, mask, kidx


def check_refill(gpu, ref, keep):
    gs, gc, gscore, gmask, gk = gpu
    rs, rc, rscore, rmask, rk = ref
    np.testing.assert_array_equal(gc.astype(np.int64), rc)
    assert (gscore[rc == 0] == 0).all()
    np.testing.assert_allclose(gscore, rscore, rtol=1e-3, atol=0)
    # the GPU keep-set is the exact ranking of the GPU's own scores ...
    order = np.lexsort((np.arange(len(gscore)), -gscore.astype(np.float64)))
    np.testing.assert_array_equal(gk, np.sort(order[:keep]))
    np.testing.assert_array_equal(gmask, np.isin(np.arange(len(gscore)), gk).astype(np.uint8))
    # ... and differs from the oracle's only at near-ties of the boundary score
    diff = np.setxor1d(gk, rk)
    if diff.size:
        ro = np.sort(rscore)[::-1]
        boundary = 0.5 * (ro[keep - 1] + ro[keep])
        assert (np.abs(rscore[diff] - boundary) <= 1e-3 * boundary).all(), diff


@pytest.mark.parametrize("T,H,F,E,k,keep,batches", [(2048, 256, 128, 64, 10, 32, 1),   # MFMA rows
                                                    (300, 256, 128, 64, 4, 40, 3),     # additive batches
                                                    (96, 2560, 640, 512, 10, 256, 1),   # full geometry
                                                    (256, 256, 128, 512, 10, 384, 1)])  # keep 384 of 512
def test_refill_matches_oracle(T, H, F, E, k, keep, batches):
    moe = require_gpu()
    w = workloads.scaled(workloads.get("refill_bf16"), T=T, H=H, F=F, Fs=F, E=E, k=k, keep=keep)
    d = workloads.generate(w, seed=4, device="cuda")
    gpu = _gpu_refill(moe, d, w, keep, batches)
    ref = _oracle_refill(d, w, keep)
    check_refill(gpu, ref, keep)


# ----------------------------------------------------------------------------- E384of512 budget

def test_pruned_e384_layer_matches_oracle():
    """Keep 384 of 512 AWQ experts (the other released budget): slice, route over
    384 logits (6 per lane) and run the layer."""
    moe = require_gpu()
    w = workloads.scaled(workloads.get("pruned_awq"), T=64, E=384, E_base=512)
    d = workloads.generate(w, seed=3, device="cuda")
    keep = d["keep_idx"]
    assert keep.numel() == 384
    wr, bank = moe.prune_slice(keep.cuda(), d["router"], d["experts"])
    y, mid = moe.moe_layer(d["x"], wr, w.k, bank, d["shared"], keep_intermediates=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(wr), bits(d["router"])[keep.numpy()])
    ref_y, ref_idx, ref_g = oracle_layer_sparse(d["x"], wr, w.k, bank, d["shared"])
    np.testing.assert_array_equal(mid["idx"].cpu().numpy(), ref_idx)
    np.testing.assert_allclose(mid["gate"].cpu().numpy(), ref_g, rtol=1e-5, atol=1e-7)
    # the pruned layer is the base layer with the dropped experts masked out
    base_l, _ = O.router_logits(bits(d["x"]), bits(d["router"]))
    masked = np.full_like(base_l, -np.inf)
    masked[:, keep.numpy()] = base_l[:, keep.numpy()]
    np.testing.assert_array_equal(keep.numpy()[ref_idx], O.rank(masked, w.k))
    check_close(y.float().cpu().numpy(), ref_y, "E384 layer")
