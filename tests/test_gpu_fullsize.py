"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Routing indices and the permutation are checked whole (the oracle computes
every exact logit); layer outputs are checked on sampled tokens, Refill-RMS
scores on sampled experts (the oracle re-evaluates every token routed to the
expert), keep-sets and counts by properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.gpu_helpers import bits, check_close, oracle_bank, require_gpu
from tests.test_gpu_layer import oracle_layer_sparse

pytestmark = pytest.mark.gpu


def _sample(n, T, seed):
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), n - 2, replace=False)]))


@pytest.mark.parametrize("name", ["prefill_awq", "pruned_awq", "prefill_fp8", "prefill_nvfp4"])
def test_fullsize_layer(name):
    moe = require_gpu()
    w = workloads.get(name)
    d = workloads.generate(w, device="cuda")
    wr, bank = d["router"], d["experts"]
    if w.E_base:
        keep = d["keep_idx"]
        wr, bank = moe.prune_slice(keep.cuda(), wr, bank)
        torch.cuda.synchronize()
        # slicing is an exact gather of router rows and whole expert tensors
        ref_wr, ref_bank = O.prune_slice(bits(d["router"]), oracle_bank(d["experts"]), keep.numpy())
        np.testing.assert_array_equal(bits(wr), ref_wr)
        got = oracle_bank(bank)
        for p in ("gate", "up", "down"):
            for a in ("qweight", "qzeros", "scales"):
                np.testing.assert_array_equal(getattr(getattr(got, p), a), getattr(getattr(ref_bank, p), a))
        del got, ref_bank
    y, mid = moe.moe_layer(d["x"], wr, w.k, bank, d["shared"], keep_intermediates=True)
    torch.cuda.synchronize()
    # every routing decision and the whole permutation
    ref_l, _ = O.router_logits(bits(d["x"]), bits(wr))
    ref_idx = O.rank(ref_l, w.k)
    np.testing.assert_array_equal(mid["idx"].cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(mid["topk_logit"].cpu().numpy(), np.take_along_axis(ref_l, ref_idx, 1))
    ro, rs, rp = O.permute(ref_idx, w.E)
    np.testing.assert_array_equal(mid["offsets"].cpu().numpy(), ro)
    np.testing.assert_array_equal(mid["sorted_pair"].cpu().numpy(), rs)
    np.testing.assert_array_equal(mid["pair_to_row"].cpu().numpy(), rp)
    # outputs of sampled tokens (first, last and random)
    tok = _sample(16, w.T, 1)
    ref_y, _, _ = oracle_layer_sparse(d["x"], wr, w.k, bank, d["shared"], tokens=tok)
    check_close(y.float().cpu().numpy()[tok], ref_y, name)


def test_fullsize_refill():
    moe = require_gpu()
    w = workloads.get("refill_bf16")
    d = workloads.generate(w, device="cuda")
    E, k = w.E, w.k
    idx, tl, gate, _ = moe.route(d["x"], d["router"], k, extra=1)
    off, sp, p2r = moe.permute(idx, E)
    rows = moe.grouped_ffn(d["x"], k + 1, d["experts"], off, sp, out_dtype=moe.OUT_F32)
    stat_sum = torch.zeros(E, dtype=torch.float32, device="cuda")
    stat_count = torch.zeros(E, dtype=torch.int32, device="cuda")
    moe.refill_score(rows, off, sp, p2r, idx, tl, stat_sum, stat_count)
    score, mask, kidx = moe.refill_finalize(stat_sum, stat_count, w.H, w.keep)
    torch.cuda.synchronize()

    ref_l, _ = O.router_logits(bits(d["x"]), bits(d["router"]))
    ref_idx = O.rank(ref_l, k + 1)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    # counts: how often each expert is among a token's first k
    np.testing.assert_array_equal(stat_count.cpu().numpy(), np.bincount(ref_idx[:, :k].ravel(), minlength=E))
    # fp32 expert rows of sampled pairs
    rng = np.random.default_rng(2)
    pairs = rng.choice(w.T * (k + 1), 48, replace=False)
    toks, slots = pairs // (k + 1), pairs % (k + 1)
    used = np.unique(ref_idx[toks, slots])
    ob = oracle_bank(d["experts"], used)
    ref_rows = O.pair_outputs(bits(d["x"])[toks], np.searchsorted(used, ref_idx[toks, slots])[:, None].astype(np.int32), ob)
    got_rows = rows.cpu().numpy()[p2r.cpu().numpy()[pairs]]
    check_close(got_rows, ref_rows, "refill rows")
    # scores of sampled experts: the oracle re-evaluates every token routed to each
    g_score = score.cpu().numpy()
    full_bank = oracle_bank(d["experts"])
    xb = bits(d["x"])
    for e in rng.choice(E, 3, replace=False):
        toks_e = np.nonzero((ref_idx[:, :k] == e).any(1))[0]
        s = np.zeros(E)
        c = np.zeros(E, np.int64)
        O.refill_accumulate(xb[toks_e], ref_l[toks_e], k, full_bank, None, s, c)
        ref_score = np.sqrt(s[e] / (c[e] * w.H)) if c[e] else 0.0
        assert c[e] == len(toks_e)
        np.testing.assert_allclose(g_score[e], ref_score, rtol=1e-3, err_msg=f"expert {e}")
    # keep-set: the exact ranking of the GPU scores, as mask and ascending list
    order = np.lexsort((np.arange(E), -g_score.astype(np.float64)))
    np.testing.assert_array_equal(kidx.cpu().numpy(), np.sort(order[:w.keep]))
    assert mask.cpu().numpy().sum() == w.keep
    assert np.isfinite(g_score).all() and (g_score >= 0).all()
