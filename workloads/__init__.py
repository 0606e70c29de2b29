"""Seeded synthetic inputs for the MoE feed-forward layer workloads.

This module only draws random tensors with the shapes and value distributions
of the workloads; it holds none of the layer's arithmetic.  The oracle and the
HIP library both read the bytes it produces.

Value recipe (shared by every workload):
  * activations x: N(0, 1) drawn in fp32, rounded to bf16 (round to nearest even);
  * router rows and bf16 expert / shared-expert weights: N(0, 0.02) -> bf16;
  * AWQ W4A16 g32 experts: every 4-bit code and zero point uniform in 0..15
    (a uniformly random int32 word has 8 independent uniform nibbles), fp16
    scales |N(0, 0.002)| + 1e-4 drawn in fp32 then rounded to fp16;
  * FP8 block-scaled experts: N(0, 0.02) weights in fp32, per 128 x 128 block
    scale = largest |w| / 448, codes = w / scale rounded to E4M3;
  * NVFP4 experts: uniform E2M1 codes, E4M3 group scales with values in
    [0.5, 4], weight global scales 0.004 * (1 + U(0, 0.1)) per expert and
    activation global scales 0.002;
  * the pruned workload's keep-set: a seeded random choice of 256 of the 512
    base experts, listed in ascending index order.
Each tensor draws from its own torch.Generator, seeded from (seed, copy,
tensor id), so one tensor can be regenerated without the others and distinct
`copy` values give independent weight sets (used to defeat the on-chip cache
when timing).  Values depend on the device the generator runs on; both sides
of a comparison always read the same bytes.

The synthetic inputs stand in for the trained checkpoint and the calibration
corpora the pages describe, which are not available: a random N(0, 0.02)
router gives near-uniform routing, as a load-balanced router would.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden size
    E: int            # routed experts seen by the layer (after pruning)
    k: int            # experts per token
    F: int            # routed expert width
    Fs: int           # shared expert width
    fmt: str          # routed expert weight format: "bf16" or "awq"
    E_base: int = 0   # experts of the unpruned base (0: no pruning)
    refill: bool = False
    keep: int = 0     # Refill-RMS keep count

    @property
    def pairs(self) -> int:
        return self.T * (self.k + (1 if self.refill else 0))

    def as_dict(self):
        return asdict(self)


WORKLOADS = {
    # tiny layer: 64 tokens, hidden 256, 16 experts top-2, width 128, shared width 128, bf16
    "tiny_bf16": Workload("tiny_bf16", T=64, H=256, E=16, k=2, F=128, Fs=128, fmt="bf16"),
    # one decode step at full geometry, bf16 experts
    "decode_bf16": Workload("decode_bf16", T=16, H=2560, E=512, k=10, F=640, Fs=640, fmt="bf16"),
    # same geometry, AWQ W4A16 g32 routed experts, decode and prefill batches
    "decode_awq": Workload("decode_awq", T=16, H=2560, E=512, k=10, F=640, Fs=640, fmt="awq"),
    # same geometry, FP8 E4M3 routed experts with 128 x 128 block scales
    "decode_fp8": Workload("decode_fp8", T=16, H=2560, E=512, k=10, F=640, Fs=640, fmt="fp8"),
    "prefill_fp8": Workload("prefill_fp8", T=4096, H=2560, E=512, k=10, F=640, Fs=640, fmt="fp8"),
    # NVFP4 W4A4 routed experts (group 16, E4M3 group scales, fp32 global scales)
    "decode_nvfp4": Workload("decode_nvfp4", T=16, H=2560, E=512, k=10, F=640, Fs=640, fmt="nvfp4"),
    "prefill_nvfp4": Workload("prefill_nvfp4", T=4096, H=2560, E=512, k=10, F=640, Fs=640,
                              fmt="nvfp4"),
    "prefill_awq": Workload("prefill_awq", T=4096, H=2560, E=512, k=10, F=640, Fs=640, fmt="awq"),
    # 256 of 512 experts kept; one packed row of 32768 tokens
    "pruned_awq": Workload("pruned_awq", T=32768, H=2560, E=256, k=10, F=640, Fs=640, fmt="awq",
                           E_base=512),
    # Refill-RMS scoring: top-10 plus the 11th-ranked expert, keep 256 of 512
    "refill_bf16": Workload("refill_bf16", T=8192, H=2560, E=512, k=10, F=640, Fs=640,
                            fmt="bf16", refill=True, keep=256),
}


def get(name_or_workload) -> Workload:
    if isinstance(name_or_workload, Workload):
        return name_or_workload
    return WORKLOADS[name_or_workload]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some sizes changed (used for small parity cases)."""
    d = w.as_dict()
    d.update(changes)
    return Workload(**d)


# tensor ids for the per-tensor generator streams
_IDS = {"x": 1, "router": 2, "gate": 3, "up": 4, "down": 5, "shared_gate": 6, "shared_up": 7,
        "shared_down": 8, "keep": 11, "valid": 12}
_SUB = {"w": 0, "qweight": 1, "qzeros": 2, "scales": 3}


def _gen(device, seed: int, copy: int, tid: int, sub: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + copy * 10_007 + tid * 101 + sub) & 0x7FFF_FFFF_FFFF)
    return g


def _normal(shape, std, g, device, out_dtype, chunk_rows=16):
    """N(0, std) drawn in fp32 in chunks along dim 0, rounded once to out_dtype."""
    out = torch.empty(shape, dtype=out_dtype, device=device)
    for i in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - i)
        v = torch.randn((n,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        out[i:i + n] = (v * std).to(out_dtype)
    return out


def _words(shape, g, device, chunk_rows=16):
    """Uniformly random int32 words (8 independent uniform 4-bit fields each)."""
    out = torch.empty(shape, dtype=torch.int32, device=device)
    for i in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - i)
        out[i:i + n] = torch.randint(-2**31, 2**31, (n,) + tuple(shape[1:]), generator=g,
                                     device=device, dtype=torch.int64).to(torch.int32)
    return out


def _scales(shape, g, device, chunk_rows=16):
    out = torch.empty(shape, dtype=torch.float16, device=device)
    for i in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - i)
        v = torch.randn((n,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        out[i:i + n] = (v * 0.002).abs_().add_(1e-4).to(torch.float16)
    return out


def activations(w: Workload, seed: int = 0, device="cpu", copy: int = 0, T: int | None = None):
    T = w.T if T is None else T
    return _normal((T, w.H), 1.0, _gen(device, seed, copy, _IDS["x"]), device, torch.bfloat16,
                   chunk_rows=4096)


def router(w: Workload, seed: int = 0, device="cpu", copy: int = 0, E: int | None = None):
    E = (w.E_base or w.E) if E is None else E
    return _normal((E, w.H), 0.02, _gen(device, seed, copy, _IDS["router"]), device,
                   torch.bfloat16, chunk_rows=E)


def expert_bank(w: Workload, seed: int = 0, device="cpu", copy: int = 0, E: int | None = None,
                fmt: str | None = None) -> dict:
    """Routed experts of the (unpruned) base: E = E_base or E experts."""
    E = (w.E_base or w.E) if E is None else E
    fmt = w.fmt if fmt is None else fmt
    H, F = w.H, w.F
    out = {"fmt": fmt}
    dims = {"gate": (F, H), "up": (F, H), "down": (H, F)}  # (out, in)
    for name, (o, i) in dims.items():
        tid = _IDS[name]
        if fmt == "bf16":
            out[name] = _normal((E, o, i), 0.02, _gen(device, seed, copy, tid), device,
                                torch.bfloat16)
        elif fmt == "awq":
            assert o % 8 == 0 and i % 32 == 0
            out[name + "_qweight"] = _words((E, i, o // 8), _gen(device, seed, copy, tid, 1),
                                            device)
            out[name + "_qzeros"] = _words((E, i // 32, o // 8), _gen(device, seed, copy, tid, 2),
                                           device)
            out[name + "_scales"] = _scales((E, i // 32, o), _gen(device, seed, copy, tid, 3),
                                            device)
        elif fmt == "fp8":
            assert o % 128 == 0 and i % 128 == 0
            out[name + "_codes"], out[name + "_bscales"] = _fp8_blocks(
                (E, o, i), _gen(device, seed, copy, tid, 4), device)
        elif fmt == "nvfp4":
            assert i % 32 == 0
            g = _gen(device, seed, copy, tid, 5)
            # two uniform E2M1 codes per byte (all 16 codes, -0 included)
            out[name + "_fp4"] = torch.randint(0, 256, (E, o, i // 2), generator=g, device=device,
                                               dtype=torch.int64).to(torch.uint8)
            # E4M3 block scales with values in [0.5, 4] (codes 0x30..0x48)
            out[name + "_fp4scales"] = torch.randint(0x30, 0x49, (E, o, i // 16), generator=g,
                                                     device=device, dtype=torch.int64).to(torch.uint8)
            # weight global scale per expert: 0.004 * (1 + U(0, 0.1))
            out[name + "_wglobal"] = (0.004 * (1.0 + 0.1 * torch.rand(E, generator=g, device=device,
                                                                       dtype=torch.float32)))
        else:
            raise ValueError(fmt)
    if fmt == "nvfp4":
        # static activation global scales (the inputs' largest magnitudes are
        # about 6 * 448 * scale): one for the gate/up input, one for down's
        out["act_global_gu"] = 0.002
        out["act_global_down"] = 0.002
    return out


def _fp8_blocks(shape, g, device, chunk_rows=16):
    """FP8 E4M3 codes and 128 x 128 block scales of N(0, 0.02) weights: each
    block's scale is its largest |w| / 448 (the largest finite E4M3 value),
    the codes are w / scale rounded to E4M3 by torch's conversion."""
    E, O, I = shape
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scales = torch.empty((E, O // 128, I // 128), dtype=torch.float32, device=device)
    for e0 in range(0, E, chunk_rows):
        n = min(chunk_rows, E - e0)
        w = torch.randn((n, O, I), generator=g, device=device, dtype=torch.float32) * 0.02
        blk = w.view(n, O // 128, 128, I // 128, 128)
        amax = blk.abs().amax(dim=(2, 4))
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (blk / sc[:, :, None, :, None]).to(torch.float8_e4m3fn)
        codes[e0:e0 + n] = q.view(torch.uint8).view(n, O, I)
        scales[e0:e0 + n] = sc
    return codes, scales


def shared_bank(w: Workload, seed: int = 0, device="cpu", copy: int = 0) -> dict:
    H, F = w.H, w.Fs
    return {"fmt": "bf16",
            "gate": _normal((1, F, H), 0.02, _gen(device, seed, copy, _IDS["shared_gate"]),
                            device, torch.bfloat16),
            "up": _normal((1, F, H), 0.02, _gen(device, seed, copy, _IDS["shared_up"]),
                          device, torch.bfloat16),
            "down": _normal((1, H, F), 0.02, _gen(device, seed, copy, _IDS["shared_down"]),
                            device, torch.bfloat16)}


def keep_set(w: Workload, seed: int = 0) -> torch.Tensor:
    """Seeded keep-set for the pruned workload: w.E of w.E_base experts, ascending (CPU int32)."""
    assert w.E_base > w.E
    g = _gen("cpu", seed, 0, _IDS["keep"])
    perm = torch.randperm(w.E_base, generator=g)
    return torch.sort(perm[: w.E]).values.to(torch.int32)


def generate(w, seed: int = 0, device="cpu", copy: int = 0, with_shared: bool = True) -> dict:
    """Every input of one layer call of workload `w`.  For a pruned workload the
    expert bank and router are the unpruned base; `keep_idx` says what to keep."""
    w = get(w)
    d = {"workload": w, "x": activations(w, seed, device, copy), "router": router(w, seed, device, copy),
         "experts": expert_bank(w, seed, device, copy)}
    if with_shared:
        d["shared"] = shared_bank(w, seed, device, copy)
    if w.E_base:
        d["keep_idx"] = keep_set(w, seed)
    return d


def bits(t: torch.Tensor):
    """Raw bit pattern of a torch tensor as a numpy array (uint16 for 16-bit types)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def bank_numpy(bank: dict) -> dict:
    """Numpy bit patterns of an expert-bank dict (for the oracle)."""
    return {k: (v if isinstance(v, (str, float)) else bits(v)) for k, v in bank.items()}
