"""The layer replayed from a HIP graph: every replay, with eager work and
synchronisation between replays, gives the eager result bit for bit."""
import pytest
import torch

import workloads
from tests.gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,side_stream", [("tiny_bf16", False), ("decode_awq", True)])
def test_layer_graph_replays_match_eager(name, side_stream):
    moe = require_gpu()
    w = workloads.get(name)
    d = workloads.generate(w, device="cuda")
    other = workloads.generate(w, seed=7, device="cuda")
    ws, sws = moe.Workspace(), moe.Workspace()
    side = torch.cuda.Stream() if side_stream else None
    kw = dict(ws=ws, shared_stream=side, shared_ws=sws)
    ref = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"], **kw).clone()
    ref_other = moe.moe_layer(other["x"], other["router"], w.k, other["experts"], other["shared"],
                              **kw).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = moe.moe_layer(d["x"], d["router"], w.k, d["experts"], d["shared"], **kw)
    for _ in range(3):
        # eager work on the same workspaces between replays
        y2 = moe.moe_layer(other["x"], other["router"], w.k, other["experts"], other["shared"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(y2, ref_other)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


@pytest.mark.parametrize("name,side_stream,om", [("tiny_bf16", False, False), ("decode_awq", True, True),
                                                 ("decode_bf16", True, False)])
def test_layer_call_graph_replays_match_eager(name, side_stream, om):
    """moe_layer captured whole (its side-stream fork and join become graph
    edges): every replay equals the eager call, with eager calls of the same
    prepared call shape on other inputs in between."""
    moe = require_gpu()
    w = workloads.get(name)
    d = workloads.generate(w, device="cuda")
    other = workloads.generate(w, seed=7, device="cuda")
    bank = moe.awq_to_output_major(d["experts"]) if om else d["experts"]
    bank_o = moe.awq_to_output_major(other["experts"]) if om else other["experts"]
    side = torch.cuda.Stream() if side_stream else None
    call = moe.LayerCall(d["x"], d["router"], w.k, bank, d["shared"], side_stream=side)
    call_o = moe.LayerCall(other["x"], other["router"], w.k, bank_o, other["shared"], side_stream=side)
    ref = call().clone()
    ref_o = call_o().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = call()
    for _ in range(3):
        y2 = call_o()
        torch.cuda.synchronize()
        assert torch.equal(y2, ref_o)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
