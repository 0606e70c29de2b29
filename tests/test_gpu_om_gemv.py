"""The streaming GEMV on output-major AWQ codes (decode-sized calls: fewer than
32 rows per active expert) against the oracle: the full layer geometry, both
projection shapes the pass split takes (1 to 5 passes, 16, 8 and 4 blocks a
column), experts with more rows than one 4-row chunk (ragged chunks), a
hidden size whose LDS stage takes half the column sets a wave (hidden 3584:
the scales and zero words staged through registers, not by loads to LDS), the
one-expert identity call of a shared expert, a single token, and a shape the
GEMV does not take (hidden 8192, which falls back to the MFMA GEMM)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.gpu_helpers import bits, check_close, oracle_bank, require_gpu

pytestmark = pytest.mark.gpu


def _wl(T, H, E, F, k):
    return workloads.scaled(workloads.get("decode_awq"), T=T, H=H, E=E, F=F, Fs=F, k=k)


def _routing(T, k, E, seed, heavy=None):
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    if heavy is not None:  # expert 0 in the first `heavy` tokens' lists (first slot)
        for t in range(heavy):
            row = idx[t]
            if 0 not in row.tolist():
                row[0] = 0
    return idx


@pytest.mark.parametrize("T,E,k,H,F,heavy", [
    (16, 512, 10, 2560, 640, None),   # the decode layer: 1-2 rows per expert, 5 + 5 passes
    (40, 64, 2, 256, 128, 9),         # expert 0: 9 rows = chunks of 4, 4, 1
    (12, 16, 2, 512, 384, 7),         # 16 blocks x 1 pass; 4 blocks x 3 passes
    (6, 8, 3, 1024, 256, None),       # 16 blocks x 2 passes; 8 blocks x 1 pass
    (1, 32, 4, 2560, 640, None),      # one token
    (5, 8, 2, 3584, 256, None),       # 7 passes: half the sets a wave, scales staged through registers
    (4, 2, 1, 8192, 128, None),       # hidden beyond the GEMV's LDS stage: the MFMA GEMM
])
def test_om_gemv_matches_oracle(T, E, k, H, F, heavy):
    moe = require_gpu()
    w = _wl(T, H, E, F, k)
    print(f"om gemv T={T} E={E} k={k} H={H} F={F}", flush=True)
    x = workloads.activations(w, seed=5, device="cuda")
    awq = workloads.expert_bank(w, seed=5, device="cuda")
    bank = moe.awq_to_output_major(awq)
    idx = _routing(T, k, E, seed=T * 7 + E, heavy=heavy)
    off, sp, p2r = moe.permute(idx.cuda(), E)
    used = np.unique(idx.numpy())
    ref = O.pair_outputs(bits(x), np.searchsorted(used, idx.numpy()).astype(np.int32), oracle_bank(bank, used))
    p2r_h = p2r.cpu().numpy().astype(np.int64)
    for out_dtype in (moe.OUT_BF16, moe.OUT_F32):
        rows = moe.grouped_ffn(x, k, bank, off, sp, out_dtype=out_dtype)
        torch.cuda.synchronize()
        check_close(rows.float().cpu().numpy()[p2r_h], ref, f"om gemv T={T} E={E} out={out_dtype}")
    # the AWQ-layout streaming kernels compute the same function
    rows_awq = moe.grouped_ffn(x, k, awq, off, sp, out_dtype=moe.OUT_F32)
    torch.cuda.synchronize()
    check_close(rows_awq.cpu().numpy()[p2r_h], ref, "awq layout")


def test_om_gemv_identity_call():
    """A one-expert bank applied to every token (the shared-expert call): 16
    rows in four chunks."""
    moe = require_gpu()
    w = _wl(16, 2560, 1, 640, 1)
    x = workloads.activations(w, seed=6, device="cuda")
    bank = moe.awq_to_output_major(workloads.expert_bank(w, seed=6, device="cuda"))
    rows = moe.grouped_ffn(x, 1, bank)
    torch.cuda.synchronize()
    ref = O.pair_outputs(bits(x), np.zeros((16, 1), np.int32), oracle_bank(bank))
    check_close(rows.float().cpu().numpy(), ref, "identity")


def test_om_gemv_is_deterministic():
    moe = require_gpu()
    w = workloads.get("decode_awq")
    d = workloads.generate(w, seed=2, device="cuda")
    bank = moe.awq_to_output_major(d["experts"])
    a = moe.layer(d["x"], d["router"], w.k, bank, d["shared"]).clone()
    for _ in range(3):
        b = moe.layer(d["x"], d["router"], w.k, bank, d["shared"], side_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        assert torch.equal(a, b)
