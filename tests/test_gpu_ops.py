"""GPU parity of each C-ABI call against the oracle, on the same seeded inputs.

Routing indices, exact logits, the permutation, slices and keep-sets must match
bit for bit; gates within rtol 1e-5; expert outputs and layer outputs within
|d| <= 1e-2 + 2e-2 |ref| elementwise and 1e-2 normwise."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.gpu_helpers import bits, check_close, oracle_bank, require_gpu

pytestmark = pytest.mark.gpu


def _wl(T, H, E, F=128, fmt="bf16", Fs=None):
    return workloads.scaled(workloads.get("tiny_bf16"), T=T, H=H, E=E, F=F, Fs=Fs or F, fmt=fmt)


# ----------------------------------------------------------------------------- route

@pytest.mark.parametrize("T,H,E,k,extra", [(64, 256, 16, 2, 0), (16, 2560, 512, 10, 0),
                                           (16, 2560, 512, 10, 1), (300, 512, 100, 7, 1),
                                           (3, 64, 1, 1, 0), (70, 128, 1024, 10, 1),
                                           (33, 256, 65, 64, 0), (40, 2560, 384, 10, 1),
                                           (200, 512, 384, 10, 0)])
def test_route_matches_oracle(T, H, E, k, extra):
    moe = require_gpu()
    w = _wl(T, H, E)
    x = workloads.activations(w, seed=1, device="cuda")
    wr = workloads.router(w, seed=1, device="cuda")
    idx, tl, gate, logits = moe.route(x, wr, k, extra, want_logits=True)
    idx2, tl2, gate2, _ = moe.route(x, wr, k, extra)
    torch.cuda.synchronize()
    ref_l, _ = O.router_logits(bits(x), bits(wr))
    np.testing.assert_array_equal(logits.cpu().numpy(), ref_l)
    ref_idx = O.rank(ref_l, k + extra)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(idx2.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(tl2.cpu().numpy(), np.take_along_axis(ref_l, ref_idx, 1))
    g = O.gates(ref_l, ref_idx, k)
    np.testing.assert_allclose(gate2.cpu().numpy(), g, rtol=1e-5, atol=1e-7)
    np.testing.assert_array_equal(gate.cpu().numpy(), gate2.cpu().numpy())


@pytest.mark.parametrize("T,H,E,k,extra", [(4096, 2560, 512, 10, 0), (2000, 2560, 256, 10, 1),
                                           (300, 2560, 100, 7, 0),   # inputs in registers, 2 keys per lane
                                           (200, 512, 512, 10, 1),   # inputs in registers, one vector per lane
                                           (64, 256, 256, 8, 1), (517, 512, 1024, 20, 0)])
def test_route_screened_matches_oracle(T, H, E, k, extra):
    """Batches of >= 64 tokens with E % 256 == 0 take the screened path."""
    moe = require_gpu()
    w = _wl(T, H, E)
    x = workloads.activations(w, seed=5, device="cuda")
    wr = workloads.router(w, seed=5, device="cuda")
    idx, tl, gate, _ = moe.route(x, wr, k, extra)
    torch.cuda.synchronize()
    ref_l, _ = O.router_logits(bits(x), bits(wr))
    ref_idx = O.rank(ref_l, k + extra)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(tl.cpu().numpy(), np.take_along_axis(ref_l, ref_idx, 1))
    np.testing.assert_allclose(gate.cpu().numpy(), O.gates(ref_l, ref_idx, k), rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("H", [512, 2560])
def test_route_screened_ties_and_degenerate_tokens(H):
    """Exact ties between router rows, and tokens whose logits are all equal
    (every expert is a candidate: the per-token fallback)."""
    moe = require_gpu()
    w = _wl(256, H, 256)
    x = workloads.activations(w, seed=6, device="cuda")
    wr = workloads.router(w, seed=6, device="cuda")
    for dst, src in ((9, 4), (100, 4), (200, 17), (201, 17)):
        wr[dst] = wr[src]
    x[5] = 0          # all logits 0: top-k = lowest indices
    x[6] = x[7]
    idx, tl, gate, _ = moe.route(x, wr, 10, 1)
    torch.cuda.synchronize()
    ref_l, _ = O.router_logits(bits(x), bits(wr))
    ref_idx = O.rank(ref_l, 11)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(idx.cpu().numpy()[5], np.arange(11))
    np.testing.assert_allclose(gate.cpu().numpy()[5], 0.1, rtol=1e-6)


def test_route_ties_take_lowest_index():
    moe = require_gpu()
    w = _wl(40, 128, 32)
    x = workloads.activations(w, device="cuda")
    wr = workloads.router(w, device="cuda")
    wr[7] = wr[3]
    wr[20] = wr[3]
    wr[30] = 0
    wr[31] = 0
    idx, tl, gate, _ = moe.route(x, wr, 6, 1)
    ref_l, _ = O.router_logits(bits(x), bits(wr))
    np.testing.assert_array_equal(idx.cpu().numpy(), O.rank(ref_l, 7))
    z = torch.zeros_like(wr)
    idx0, _, g0, _ = moe.route(x, z, 4)
    np.testing.assert_array_equal(idx0.cpu().numpy(), np.tile(np.arange(4), (40, 1)))
    np.testing.assert_allclose(g0.cpu().numpy(), 0.25, rtol=1e-6)


@pytest.mark.parametrize("T,H,E,k", [(16, 2560, 512, 10), (1, 2560, 512, 10), (63, 512, 1024, 64),
                                     (40, 256, 65, 64), (5, 64, 1, 1), (300, 512, 100, 7),
                                     (70, 128, 1024, 10), (64, 256, 256, 8), (600, 512, 512, 10)])
def test_route_permute_matches_oracle(T, H, E, k):
    """One call for route + permute: the single-workgroup selection and
    permutation for small batches, the two separate paths otherwise.  The
    results equal the oracle's ranking and permutation bit for bit, and those
    of the two separate calls."""
    moe = require_gpu()
    w = _wl(T, H, E)
    x = workloads.activations(w, seed=11, device="cuda")
    wr = workloads.router(w, seed=11, device="cuda")
    if E > 20:
        wr[E - 1] = wr[3]  # a tie between experts 3 and E - 1
    idx, tl, gate, off, sp, p2r = moe.route_permute(x, wr, k)
    idx2, tl2, gate2, _ = moe.route(x, wr, k)
    off2, sp2, p2r2 = moe.permute(idx2, E)
    torch.cuda.synchronize()
    ref_l, _ = O.router_logits(bits(x), bits(wr))
    ref_idx = O.rank(ref_l, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(tl.cpu().numpy(), np.take_along_axis(ref_l, ref_idx, 1))
    np.testing.assert_allclose(gate.cpu().numpy(), O.gates(ref_l, ref_idx, k), rtol=1e-5, atol=1e-7)
    ro, rs, rp = O.permute(ref_idx.astype(np.int32), E)
    np.testing.assert_array_equal(off.cpu().numpy(), ro)
    np.testing.assert_array_equal(sp.cpu().numpy(), rs)
    np.testing.assert_array_equal(p2r.cpu().numpy(), rp)
    for a, b in ((idx, idx2), (tl, tl2), (gate, gate2), (off, off2), (sp, sp2), (p2r, p2r2)):
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E,skew", [(16, 10, 512, False), (64, 2, 16, False), (4096, 10, 512, False),
                                        (32768, 10, 256, False), (5000, 3, 1024, False),
                                        (100, 1, 1, False), (3000, 4, 64, True), (409, 10, 512, True)])
def test_permute_matches_oracle(T, k, E, skew):
    moe = require_gpu()
    g = torch.Generator(device="cpu").manual_seed(T * 7 + k)
    if skew:  # most pairs on a few experts
        idx = torch.where(torch.rand((T, k), generator=g) < 0.8,
                          torch.randint(0, 3, (T, k), generator=g), torch.randint(0, E, (T, k), generator=g))
    else:
        idx = torch.randint(0, E, (T, k), generator=g)
    idx = idx.to(torch.int32)
    off, sp, p2r = moe.permute(idx.cuda(), E)
    ro, rs, rp = O.permute(idx.numpy(), E)
    np.testing.assert_array_equal(off.cpu().numpy(), ro)
    np.testing.assert_array_equal(sp.cpu().numpy(), rs)
    np.testing.assert_array_equal(p2r.cpu().numpy(), rp)


def test_permute_is_deterministic():
    moe = require_gpu()
    idx = torch.randint(0, 256, (32768, 10), generator=torch.Generator().manual_seed(5)).int().cuda()
    a = moe.permute(idx, 256)
    b = moe.permute(idx, 256)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ----------------------------------------------------------------------------- grouped experts

def _random_routing(T, k, E, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)


@pytest.mark.parametrize("fmt", ["bf16", "awq", "fp8", "nvfp4"])
@pytest.mark.parametrize("T,E,k,H,F", [(32, 8, 2, 256, 128),      # few rows per expert: streaming
                                       (200, 8, 2, 256, 128),     # 50 rows: MFMA, 64-row tiles
                                       (300, 8, 2, 256, 128),     # 75 rows: 96-row tiles (uneven A chunks)
                                       (400, 8, 2, 256, 128),     # 100 rows: 128-row tiles
                                       (600, 8, 2, 256, 128),     # 150 rows: 192-row tiles
                                       (1100, 8, 2, 256, 128),    # 275 rows: 256-row tiles + tails
                                       (1700, 8, 2, 256, 128),    # 425 rows: tiles of 7 or 8 row blocks
                                       (8, 4, 2, 2560, 640),      # full width, streaming
                                       (16, 512, 10, 2560, 640),  # decode geometry, streaming
                                       (100, 4, 2, 2560, 640),    # full width, MFMA
                                       (400, 8, 2, 256, 96)])     # width the MFMA path does not take:
                                                                  # 100 rows per expert streamed
def test_grouped_ffn_matches_oracle(fmt, T, E, k, H, F):
    if fmt == "fp8" and (H % 128 or F % 128):
        pytest.skip("FP8 experts take multiples of the 128 x 128 scale block")
    moe = require_gpu()
    w = _wl(T, H, E, F=F, fmt=fmt)
    x = workloads.activations(w, seed=2, device="cuda")
    bank = workloads.expert_bank(w, seed=2, device="cuda")
    idx = _random_routing(T, k, E, seed=T)
    off, sp, p2r = moe.permute(idx.cuda(), E)
    for out_dtype in (moe.OUT_BF16, moe.OUT_F32):
        rows = moe.grouped_ffn(x, k, bank, off, sp, out_dtype=out_dtype)
        torch.cuda.synchronize()
        ref = O.pair_outputs(bits(x), idx.numpy(), oracle_bank(bank))
        got = rows.float().cpu().numpy()[p2r.cpu().numpy().astype(np.int64)]
        check_close(got, ref, f"{fmt} T={T} E={E} out={out_dtype}")


# ----------------------------------------------------------------------------- NVFP4 activations

def _nvfp4_cases():
    """bf16 rows exercising every branch of the NVFP4 quantiser: N(0,1) rows,
    an all-zero group, groups whose block scale saturates at 448 or is an E4M3
    subnormal, values exactly on E2M1 midpoints, and +-0."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn((37, 2560), generator=g)
    x[1, :16] = 0.0                                           # zero group: scale 0, codes 0
    x[2] *= 1e4                                               # amax / (6 ga) > 448: saturated scale
    x[3] *= 1e-4                                              # subnormal E4M3 scales
    x[4, :16] = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                              -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6.0])  # midpoints
    x[5, :16] = torch.tensor([-0.0] * 8 + [0.0] * 7 + [1.0])  # signed zeros
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("ga", [0.002, 1.0 / 6.0, 3.0e-7])
def test_nvfp4_quantize_is_bit_exact(ga):
    moe = require_gpu()
    x = _nvfp4_cases()
    got = moe.nvfp4_quantize(x.cuda(), ga)
    torch.cuda.synchronize()
    ref = O.nvfp4_quantize(x.float().numpy(), ga)
    g = got.float().cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(g, ref)
    # the signs of zeros are not part of the contract; the values are
    assert np.all(np.isfinite(g))


def test_nvfp4_quantize_ragged_rows_and_empty():
    moe = require_gpu()
    x = _nvfp4_cases()[:, :48].contiguous()  # 3 groups a row
    got = moe.nvfp4_quantize(x.cuda(), 0.01)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.float().cpu().numpy().astype(np.float64),
                                  O.nvfp4_quantize(x.float().numpy(), 0.01))
    empty = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert moe.nvfp4_quantize(empty, 0.01).shape == (0, 64)


# 700 and 600 tokens: 256-row gate/up and down tiles with a ragged last tile
@pytest.mark.parametrize("T,H,F", [(16, 2560, 640), (100, 2560, 640), (5, 256, 128), (700, 256, 128),
                                   (600, 2560, 640)])
def test_shared_expert_identity_mode(T, H, F):
    moe = require_gpu()
    w = _wl(T, H, 8, F=F)
    x = workloads.activations(w, seed=3, device="cuda")
    sh = workloads.shared_bank(w, seed=3, device="cuda")
    s = moe.grouped_ffn(x, 1, sh)
    torch.cuda.synchronize()
    ref = O.shared_outputs(bits(x), oracle_bank(sh))
    check_close(s.float().cpu().numpy(), ref, f"shared T={T}")


def test_grouped_ffn_is_deterministic():
    moe = require_gpu()
    w = _wl(1100, 256, 8, fmt="awq")
    x = workloads.activations(w, device="cuda")
    bank = workloads.expert_bank(w, device="cuda")
    idx = _random_routing(1100, 2, 8, seed=1)
    off, sp, p2r = moe.permute(idx.cuda(), 8)
    a = moe.grouped_ffn(x, 2, bank, off, sp).clone()
    b = moe.grouped_ffn(x, 2, bank, off, sp)
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------- combine

@pytest.mark.parametrize("rows_f32", [False, True])
@pytest.mark.parametrize("T,k,H,with_shared", [(50, 3, 256, True),      # one wave per 64 vectors
                                               (16, 10, 2560, True),    # decode shape: one batch of 10 (fp32: 8 + 2)
                                               (4200, 2, 256, True),    # one workgroup per token, 32 of 64 lanes
                                               (1000, 11, 2560, True),  # five waves per token, batch of 11 (8 + 2 + 1)
                                               (5000, 16, 512, False),  # one full batch of 16 (fp32: 8 + 8)
                                               (7, 70, 136, False),     # k > 64: slots in two chunks, 17 vectors
                                               (3, 13, 64, False),      # batch of 13 (fp32: 8 + 4 + 1)
                                               (3, 9, 64, False)])      # batch of 9 (fp32: 8 + 1)
def test_combine_matches_oracle(rows_f32, T, k, H, with_shared):
    moe = require_gpu()
    g = torch.Generator().manual_seed(9 + T + k)
    rows = torch.randn((T * k, H), generator=g).cuda()
    if not rows_f32:
        rows = rows.to(torch.bfloat16)
    perm = torch.randperm(T * k, generator=g).to(torch.int32).cuda()
    gate = torch.softmax(torch.randn((T, k), generator=g), 1).cuda()
    shared = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda() if with_shared else None
    scale = torch.randn(T, generator=g).cuda() if with_shared else None
    y = moe.combine(rows, perm, gate, shared, scale)
    torch.cuda.synchronize()
    r = rows.double().cpu().numpy()[perm.cpu().numpy().astype(np.int64)]
    sh = shared.double().cpu().numpy() if with_shared else None
    sc = scale.double().cpu().numpy() if with_shared else None
    ref = O.combine(r, gate.double().cpu().numpy(), sh, sc)
    check_close(y.float().cpu().numpy(), ref, f"combine T={T} k={k} H={H}")


# ----------------------------------------------------------------------------- pruning, keep policies

@pytest.mark.parametrize("fmt", ["bf16", "awq", "fp8", "nvfp4"])
def test_prune_slice_is_exact_gather(fmt):
    moe = require_gpu()
    w = _wl(8, 256, 32, fmt=fmt)
    wr = workloads.router(w, device="cuda")
    bank = workloads.expert_bank(w, device="cuda")
    keep = torch.tensor(sorted(torch.randperm(32, generator=torch.Generator().manual_seed(1))[:12].tolist()),
                        dtype=torch.int32)
    wr2, bank2 = moe.prune_slice(keep.cuda(), wr, bank)
    torch.cuda.synchronize()
    ref_wr, ref_bank = O.prune_slice(bits(wr), oracle_bank(bank), keep.numpy())
    np.testing.assert_array_equal(bits(wr2), ref_wr)
    got = oracle_bank(bank2)
    for p in ("gate", "up", "down"):
        for a in ("w", "qweight", "qzeros", "scales", "codes", "bscales", "gscales", "wglobal"):
            ra, ga = getattr(getattr(ref_bank, p), a), getattr(getattr(got, p), a)
            if ra is not None:
                np.testing.assert_array_equal(ga, ra)


@pytest.mark.parametrize("E,keep", [(512, 256), (512, 384), (16, 5), (1000, 1)])
def test_router_norm_keep_matches_oracle(E, keep):
    moe = require_gpu()
    w = _wl(1, 2560, E)
    wr = workloads.router(w, device="cuda")
    norm, kidx = moe.router_norm_keep(wr, keep)
    torch.cuda.synchronize()
    rn, rk = O.router_norm_keep(bits(wr), keep)
    np.testing.assert_allclose(norm.cpu().numpy(), rn, rtol=1e-6)
    np.testing.assert_array_equal(kidx.cpu().numpy(), rk)
