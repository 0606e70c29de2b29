"""moe_layer (the whole layer in one library call) against the four calls it
stands for, made one after the other: the same bits for every weight format,
every routing path (the single-workgroup selection that also builds the GEMV
slot table; the per-token selection whose (token, slot) pairs the streaming
kernels take directly, on output-major codes below 64 tokens, at 1 to 63
tokens and over 384 or 512 experts; the screened
router for larger batches), both grouped-expert families (streaming GEMV and
MFMA GEMM), with the shared expert on the same stream or on a side stream.  The four calls are themselves checked against
the oracle (test_gpu_layer.py, test_gpu_fullsize.py), and the layer call is
also checked against the oracle directly on two formats."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import check_close, require_gpu
from tests.test_gpu_layer import oracle_layer_sparse

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "gemm_bf16":        # 128 rows per expert: MFMA GEMM, screened router off (E % 256)
        return workloads.scaled(workloads.get("tiny_bf16"), T=1024)
    if name == "screened_awq":     # T >= 64, E = 512: screened router, streaming GEMV
        return workloads.scaled(workloads.get("decode_awq"), T=96)
    if name == "prefill_awq_om":   # output-major AWQ codes, MFMA GEMM, 40 rows per expert
        return workloads.scaled(workloads.get("prefill_awq"), T=2048)
    # output-major codes below 64 tokens: the streaming kernels take their
    # rows by (token, slot) pair, with no permutation
    if name in ("decode_awq_om", "same_tokens_om"):
        return workloads.get("decode_awq")
    if name == "decode_awq_om_t1":
        return workloads.scaled(workloads.get("decode_awq"), T=1)
    if name == "decode_awq_om_t40":   # 400 pairs: the pair scan over seven 64-pair chunks
        return workloads.scaled(workloads.get("decode_awq"), T=40)
    if name == "decode_awq_om_t63":   # 630 pairs: three batches of the pair scan, the largest fused batch
        return workloads.scaled(workloads.get("decode_awq"), T=63)
    if name == "decode_awq_om_e384":  # a 384-expert bank (E384of512 pruning) at decode
        return workloads.scaled(workloads.get("decode_awq"), E=384)
    return workloads.get(name)


CASES = ["tiny_bf16", "decode_bf16", "decode_awq", "decode_fp8", "decode_nvfp4", "gemm_bf16", "screened_awq",
         "prefill_awq_om", "decode_awq_om", "decode_awq_om_t1", "decode_awq_om_t40", "decode_awq_om_t63",
         "decode_awq_om_e384", "same_tokens_om"]


@pytest.mark.parametrize("name", CASES)
@pytest.mark.parametrize("side", [False, True])
def test_layer_call_equals_the_four_calls(name, side):
    moe = require_gpu()
    w = _case(name)
    print(f"case {name} side={side} T={w.T} E={w.E} fmt={w.fmt}", flush=True)
    d = workloads.generate(w, device="cuda")
    if name == "same_tokens_om":
        # every token routes to the same k experts: 16 rows each, in chunks of 4
        d["x"] = d["x"][:1].expand_as(d["x"]).contiguous()
    bank = moe.awq_to_output_major(d["experts"]) if "_om" in name else d["experts"]
    ref, mid = moe.moe_layer(d["x"], d["router"], w.k, bank, d["shared"], keep_intermediates=True)
    ref = ref.clone()
    idx = torch.full((w.T, w.k), -1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream() if side else None
    for _ in range(2):
        y = moe.layer(d["x"], d["router"], w.k, bank, d["shared"], topk_idx=idx, side_stream=s)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), name
        assert torch.equal(idx, mid["idx"])


@pytest.mark.parametrize("name", ["decode_awq", "decode_awq_om", "tiny_bf16"])
def test_layer_call_matches_oracle(name):
    """The layer call against the oracle directly; decode_awq_om runs the
    16-token W4A16 layer on output-major codes, as bench.py does."""
    moe = require_gpu()
    om = name.endswith("_om")
    w = workloads.get(name[:-3] if om else name)
    d = workloads.generate(w, seed=4, device="cuda")
    bank = moe.awq_to_output_major(d["experts"]) if om else d["experts"]
    sc = torch.linspace(-0.5, 1.5, w.T, device="cuda")
    y = moe.layer(d["x"], d["router"], w.k, bank, d["shared"], shared_scale=sc,
                  side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    ref_y, _, _ = oracle_layer_sparse(d["x"], d["router"], w.k, d["experts"], d["shared"],
                                      shared_scale=sc.double().cpu().numpy())
    check_close(y.float().cpu().numpy(), ref_y, name)


@pytest.mark.parametrize("om", [False, True])
def test_layer_call_without_shared_expert(om):
    moe = require_gpu()
    w = workloads.get("decode_awq")
    d = workloads.generate(w, device="cuda")
    bank = moe.awq_to_output_major(d["experts"]) if om else d["experts"]
    ref = moe.moe_layer(d["x"], d["router"], w.k, bank, None).clone()
    y = moe.layer(d["x"], d["router"], w.k, bank, None)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


@pytest.mark.parametrize("T", [1, 16, 63])
@pytest.mark.parametrize("side", [False, True])
def test_layer_call_pairs_with_shared_scale(T, side):
    """Rows by (token, slot) pair on output-major codes, with a per-token
    shared scale, the shared expert on the same stream or on a side stream:
    the same bits as the four calls, on three calls in a row with different
    tokens in between (nothing of one call's intermediates leaks into the
    next)."""
    moe = require_gpu()
    w = workloads.scaled(workloads.get("decode_awq"), T=T)
    print(f"case T={T} side={side}", flush=True)
    d = workloads.generate(w, seed=11, device="cuda")
    bank = moe.awq_to_output_major(d["experts"])
    sc = torch.linspace(-0.75, 1.25, w.T, device="cuda")
    x2 = workloads.generate(w, seed=12, device="cuda")["x"]
    s = torch.cuda.Stream() if side else None
    for x in (d["x"], x2, d["x"]):
        ref = moe.moe_layer(x, d["router"], w.k, bank, d["shared"], shared_scale=sc).clone()
        y = moe.layer(x, d["router"], w.k, bank, d["shared"], shared_scale=sc, side_stream=s)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


def test_prepared_layer_call_and_routed_events():
    """LayerCall repeats the same bits; the events bracket the routed call."""
    moe = require_gpu()
    w = workloads.get("decode_awq")
    d = workloads.generate(w, device="cuda")
    ref = moe.layer(d["x"], d["router"], w.k, d["experts"], d["shared"]).clone()
    call = moe.LayerCall(d["x"], d["router"], w.k, d["experts"], d["shared"], side_stream=torch.cuda.Stream())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
    for a, b in evs:  # torch creates the HIP events on first record
        a.record()
        b.record()
    for a, b in evs:
        y = call((a, b))
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    for a, b in evs:
        ms = a.elapsed_time(b)
        assert 0.0 < ms < 100.0, ms
    # a batch of different tokens through the same prepared call shape
    x2 = workloads.generate(w, seed=7, device="cuda")["x"]
    call.x.copy_(x2)
    y2 = call().clone()
    torch.cuda.synchronize()
    assert torch.equal(y2, moe.layer(x2, d["router"], w.k, d["experts"], d["shared"]))
    assert not torch.equal(y2, ref)


def test_layer_call_zero_tokens():
    moe = require_gpu()
    w = workloads.get("tiny_bf16")
    d = workloads.generate(w, device="cuda")
    y = moe.layer(d["x"][:0], d["router"], w.k, d["experts"], d["shared"])
    torch.cuda.synchronize()
    assert y.shape == (0, w.H)
