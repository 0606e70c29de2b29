"""AWQ W4A16 g32 experts with output-major codes (MOE_W_AWQ_G32_OM): the code
conversion against an independent numpy repacker, bit for bit, and the MFMA
grouped GEMM that reads the layout against the oracle on every row-tile size
(64, 96, 128, 192 and 256 rows), tiles of 192- and 256-row kernels that run
one or two row blocks short, ragged last tiles, decode batches and the full
layer width."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests import awq_ref
from tests.gpu_helpers import bits, check_close, oracle_bank, require_gpu

pytestmark = pytest.mark.gpu


def _wl(T, H, E, F, k=2):
    return workloads.scaled(workloads.get("prefill_awq"), T=T, H=H, E=E, F=F, Fs=F, k=k)


@pytest.mark.parametrize("E,H,F", [(3, 256, 128), (2, 2560, 640), (5, 512, 384)])
def test_awq_to_output_major_is_exact(E, H, F):
    moe = require_gpu()
    bank = workloads.expert_bank(_wl(8, H, E, F), seed=5, device="cuda")
    om = moe.awq_to_output_major(bank)
    torch.cuda.synchronize()
    for n in ("gate", "up", "down"):
        ref = awq_ref.to_output_major(bits(bank[n + "_qweight"]))
        np.testing.assert_array_equal(bits(om[n + "_qweight"]), ref)
        assert om[n + "_qzeros"].data_ptr() == bank[n + "_qzeros"].data_ptr()
        assert om[n + "_scales"].data_ptr() == bank[n + "_scales"].data_ptr()


def _routing(T, k, E, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)


@pytest.mark.parametrize("T,E,k,H,F", [(100, 8, 2, 256, 128),     # 25 rows per expert: 64-row tiles
                                       (280, 8, 2, 256, 128),     # 70 rows: 96-row tiles
                                       (400, 8, 2, 256, 128),     # 100 rows: 128-row tiles
                                       (560, 8, 2, 256, 128),     # 140 rows: 192-row tiles
                                       (1100, 8, 2, 256, 128),    # 275 rows: 256-row tiles + ragged tails
                                       (1700, 8, 2, 256, 128),    # 425 rows: tiles of 7 or 8 row blocks
                                       (220, 2, 2, 2560, 640),    # 220 rows, full width: one 7-block tile
                                       (100, 4, 2, 2560, 640),    # full width
                                       (16, 512, 10, 2560, 640),  # decode batch: 1-2 rows per expert
                                       (900, 3, 1, 512, 384)])    # one expert idle or nearly
def test_om_grouped_ffn_matches_oracle(T, E, k, H, F):
    moe = require_gpu()
    w = _wl(T, H, E, F, k)
    x = workloads.activations(w, seed=3, device="cuda")
    bank = moe.awq_to_output_major(workloads.expert_bank(w, seed=3, device="cuda"))
    idx = _routing(T, k, E, seed=T + E)
    if E == 3:
        idx[:] = torch.where(idx == 2, torch.zeros_like(idx), idx)   # expert 2 gets no rows
    off, sp, p2r = moe.permute(idx.cuda(), E)
    ref = O.pair_outputs(bits(x), idx.numpy(), oracle_bank(bank))
    for out_dtype in (moe.OUT_BF16, moe.OUT_F32):
        rows = moe.grouped_ffn(x, k, bank, off, sp, out_dtype=out_dtype)
        torch.cuda.synchronize()
        got = rows.float().cpu().numpy()[p2r.cpu().numpy().astype(np.int64)]
        check_close(got, ref, f"awq_om T={T} E={E} out={out_dtype}")


def test_om_run_twice_is_bit_identical():
    moe = require_gpu()
    w = _wl(1100, 256, 8, 128)
    x = workloads.activations(w, seed=4, device="cuda")
    bank = moe.awq_to_output_major(workloads.expert_bank(w, seed=4, device="cuda"))
    off, sp, _ = moe.permute(_routing(1100, 2, 8, 1).cuda(), 8)
    a = moe.grouped_ffn(x, 2, bank, off, sp)
    b = moe.grouped_ffn(x, 2, bank, off, sp)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
