"""The shared expert of a decode step (one bf16 expert applied to at most 16
tokens: the split-K 16x16x32 MFMA path) against the oracle, at the layer's
full geometry and a small one, for 1, 7 and 16 tokens and both output types;
17 tokens take the streaming kernels instead and must agree as well."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.gpu_helpers import bits, check_close, oracle_bank, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1, 7, 16, 17])
@pytest.mark.parametrize("H,F", [(2560, 640), (256, 128)])
def test_shared_expert_matches_oracle(T, H, F):
    moe = require_gpu()
    w = workloads.scaled(workloads.get("decode_bf16"), T=T, H=H, Fs=F, F=F, E=16)
    print(f"shared T={T} H={H} F={F}", flush=True)
    d = workloads.generate(w, seed=T, device="cuda")
    ref = O.shared_outputs(bits(d["x"]), oracle_bank(d["shared"]))
    for out_dtype in (moe.OUT_BF16, moe.OUT_F32):
        rows = moe.grouped_ffn(d["x"], 1, d["shared"], out_dtype=out_dtype)
        torch.cuda.synchronize()
        check_close(rows.float().cpu().numpy(), ref, f"shared T={T} out={out_dtype}")
    again = moe.grouped_ffn(d["x"], 1, d["shared"])
    torch.cuda.synchronize()
    assert torch.equal(again, moe.grouped_ffn(d["x"], 1, d["shared"]))
