"""Helpers for the GPU parity tests: device inputs from the seeded generator,
oracle banks built from the same bytes, and the tolerance checks."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.helpers import allclose_report

# Output tolerance for bf16 layer outputs: |gpu - ref| <= ATOL + RTOL * |ref|, ref = fp64 oracle.
ATOL, RTOL = 1e-2, 2e-2
# A normwise bound that systematic errors (a dropped term, a wrong scale) cannot
# hide under the elementwise allowance: ||gpu - ref|| <= NORM_RTOL * ||ref||.
# bf16 storage of h and of the outputs contributes ~2^-9 relative each.
NORM_RTOL = 1e-2


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_expert_router_amd as moe
    moe.lib()  # fails loudly when the library is missing
    return moe


def bits(t):
    return workloads.bits(t)


def oracle_bank(bank: dict, experts=None) -> O.Bank:
    """Oracle view of a device bank dict, optionally only the listed experts (host copies)."""
    sel = None if experts is None else torch.as_tensor(np.asarray(experts), dtype=torch.long)
    d = {}
    for name, t in bank.items():
        if name == "fmt" or isinstance(t, float):
            d[name] = t
        else:
            tt = t if sel is None else t.index_select(0, sel.to(t.device))
            d[name] = bits(tt)
    return O.bank_from_tensors(d)


def check_close(got, ref, what="", atol=ATOL, rtol=RTOL, norm_rtol=NORM_RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ok, excess, i = allclose_report(got, ref, atol, rtol)
    assert ok, f"{what}: elementwise tolerance exceeded by {excess:.3e} at flat index {i} " \
               f"(got {got.ravel()[i]:.6g}, ref {ref.ravel()[i]:.6g})"
    num = np.linalg.norm(got - ref)
    den = np.linalg.norm(ref)
    assert num <= norm_rtol * den + 1e-12, f"{what}: normwise error {num / max(den, 1e-30):.3e}"


def gpu_inputs(w, seed=0, device="cuda", copy=0):
    return workloads.generate(w, seed=seed, device=device, copy=copy)


def screen_margin(moe, x, wr, k, extra, ref_l):
    """Measured margin of the screened router's error bound.

    Runs moe_route without the logits output (the screened path for batches
    of at least 64 tokens and E a multiple of 256), reads the approximate MFMA
    logits la that the call leaves at the start of its workspace ([T][E]
    fp32), and compares them with the oracle's exact logits l over every
    (token, expert) pair.  Returns (max |la - l| / delta, max |la - l| /
    (2^-24 (S + 1) ||x|| ||w||)): the first must stay below 1 (delta =
    2^-17 (S + 2) ||x|| ||w|| + H 2^-100 is the bound the refine step uses,
    S = H / 32 MFMA K-steps); the second is the worst error in units of one
    fp32 rounding (relative 2^-24) per K-step."""
    T, H = x.shape
    E = wr.shape[0]
    ws = moe.Workspace(x.device)
    moe.route(x, wr, k, extra=extra, ws=ws)
    torch.cuda.synchronize()
    la = ws.buf[: T * E * 4].view(torch.float32).view(T, E).cpu().numpy().astype(np.float64)
    xf = O.bf16_bits_to_f64(bits(x))
    wf = O.bf16_bits_to_f64(bits(wr))
    xn = np.sqrt((xf * xf).sum(1))
    wn = np.sqrt((wf * wf).sum(1))
    S = (H + 31) // 32
    scale = np.outer(xn, wn)
    err = np.abs(la - np.asarray(ref_l, np.float64))
    delta = np.ldexp(S + 2.0, -17) * scale + H * np.ldexp(1.0, -100)
    units = np.ldexp(S + 1.0, -24) * scale
    return float((err / delta).max()), float((err / np.maximum(units, 1e-300)).max())
