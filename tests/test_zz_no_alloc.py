"""The allocation-free grouped-expert entry point (moe_grouped_ffn_noalloc)
against moe_grouped_ffn with a caller workspace: the same kernels run on the
library's per-GPU scratch array, so the rows must be identical bit for bit.
Two calls in a row, the second smaller, on the streaming (few rows per
expert, both AWQ code layouts), MFMA (many rows per expert, both GEMMs), NVFP4
and shared-expert paths; a call
whose scratch need exceeds the array is refused before anything runs."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def _routed(moe, w, d, T):
    x = d["x"][:T].contiguous()
    idx, _, _, off, sp, _ = moe.route_permute(x, d["router"], w.k)
    return x, off, sp


@pytest.mark.parametrize("name,T1,T2,changes,om", [
    ("decode_awq", 16, 5, {}, False),                                      # streaming kernels
    ("decode_awq", 16, 5, {}, True),                                       # MFMA streaming, output-major codes
    ("decode_nvfp4", 16, 3, {}, False),                                    # + quantised input in scratch
    ("tiny_bf16", 1024, 700, dict(T=1024, E=16, k=2), False),              # MFMA grouped GEMM
    ("prefill_awq", 256, 200, dict(T=256, E=8, k=2), False),               # AWQ GEMM, full width
    ("prefill_awq", 256, 200, dict(T=256, E=8, k=2), True),                # register-B GEMM, output-major
])
def test_noalloc_equals_workspace_call(name, T1, T2, changes, om):
    moe = require_gpu()
    w = workloads.scaled(workloads.get(name), **changes) if changes else workloads.get(name)
    d = workloads.generate(w, seed=7, device="cuda")
    if om:
        d["experts"] = moe.awq_to_output_major(d["experts"])
    for T in (T1, T2):
        x, off, sp = _routed(moe, w, d, T)
        need = moe.workspace_bytes(moe.OP_GROUPED_FFN_NVFP4 if w.fmt == "nvfp4" else moe.OP_GROUPED_FFN,
                                   T, w.k, w.E, w.H, w.F)
        assert 0 < need <= moe.noalloc_max_bytes()
        ref = moe.grouped_ffn(x, w.k, d["experts"], off, sp, ws=moe.Workspace("cuda"))
        got = moe.grouped_ffn_noalloc(x, w.k, d["experts"], off, sp)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name} T={T}"
        # the shared expert (identity mode) on the same scratch
        s_ref = moe.grouped_ffn(x, 1, d["shared"], ws=moe.Workspace("cuda"))
        s_got = moe.grouped_ffn_noalloc(x, 1, d["shared"])
        torch.cuda.synchronize()
        assert torch.equal(s_got.view(torch.int16), s_ref.view(torch.int16)), f"{name} shared T={T}"


def test_noalloc_refuses_calls_beyond_its_scratch():
    moe = require_gpu()
    w = workloads.scaled(workloads.get("decode_awq"), T=256)
    assert moe.workspace_bytes(moe.OP_GROUPED_FFN, 256, w.k, w.E, w.H, w.F) > moe.noalloc_max_bytes()
    d = workloads.generate(w, seed=1, device="cuda")
    x, off, sp = _routed(moe, w, d, 256)
    rows = torch.full((256 * w.k, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="workspace"):
        moe.grouped_ffn_noalloc(x, w.k, d["experts"], off, sp, rows=rows)
    torch.cuda.synchronize()
    assert bool((rows == 7.0).all())   # nothing was enqueued
