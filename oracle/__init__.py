"""CPU oracle of the routed mixture-of-experts feed-forward layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: it runs the
HIP library and fails loudly when that library is missing.

The arithmetic lives in ``moe_oracle.c`` (plain fp64 loops, one function per
step of the layer, each citing the page passage it follows).  This module only
builds that file with gcc and marshals numpy arrays to it.  Inputs are raw bit
patterns: bf16 and fp16 as ``uint16`` arrays, AWQ codes / zeros as ``int32``.

Pins (what the oracle is checked against, in ``tests/test_oracle_*.py``):
exact-rational dot products, numpy's stable argsort, scipy's softmax, numpy's
stable sort of the pair list, brute-force dense evaluation of every expert on
tiny inputs, an independent AWQ packer, algebraic identities of Refill-RMS and
the pages' parameter counts.  Absolute layer outputs at full geometry have no
printed value on the pages to compare with: beyond those pins they are parity
unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, AWQ, FP8, NVFP4, AWQ_OM = 0, 1, 2, 3, 4


def build(verbose: bool = False) -> str:
    """Compile moe_oracle.c into liboracle.so with gcc (IEEE double, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-std=c11", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Proj(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("in_dim", ctypes.c_int32), ("out_dim", ctypes.c_int32),
                ("w", ctypes.c_void_p), ("qweight", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("bscales", ctypes.c_void_p),
                ("gscales", ctypes.c_void_p), ("wglobal", ctypes.c_void_p), ("aglobal", ctypes.c_float)]


class _Bank(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("gate", _Proj), ("up", _Proj), ("down", _Proj)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.oracle_dot_exact_f32.restype = ctypes.c_float
    lib.oracle_dot_exact_f32.argtypes = [P, P, i64]
    lib.oracle_dot_certified.restype = ctypes.c_int
    lib.oracle_dot_certified.argtypes = [P, P, i64, P]
    lib.oracle_router_logits.restype = i64
    lib.oracle_router_logits.argtypes = [P, P, i64, i64, i64, P]
    lib.oracle_rank.restype = None
    lib.oracle_rank.argtypes = [P, i64, i64, i64, P]
    lib.oracle_gates.restype = None
    lib.oracle_gates.argtypes = [P, P, i64, i64, i64, i64, P]
    lib.oracle_permute.restype = None
    lib.oracle_permute.argtypes = [P, i64, i64, i64, P, P, P]
    lib.oracle_proj_weight.restype = ctypes.c_double
    lib.oracle_proj_weight.argtypes = [ctypes.POINTER(_Proj), i64, i64, i64]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_round.restype = ctypes.c_int
    lib.oracle_e2m1_round.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_round.restype = ctypes.c_int
    lib.oracle_e4m3_round.argtypes = [ctypes.c_float]
    lib.oracle_nvfp4_quantize.restype = None
    lib.oracle_nvfp4_quantize.argtypes = [P, i64, ctypes.c_float, P]
    lib.oracle_pair_outputs.restype = None
    lib.oracle_pair_outputs.argtypes = [P, i64, i64, P, ctypes.POINTER(_Bank), P]
    lib.oracle_shared_outputs.restype = None
    lib.oracle_shared_outputs.argtypes = [P, i64, ctypes.POINTER(_Bank), P]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [P, P, P, P, i64, i64, i64, P]
    lib.oracle_layer.restype = None
    lib.oracle_layer.argtypes = [P, P, i64, i64, i64, ctypes.POINTER(_Bank),
                                 ctypes.POINTER(_Bank), P, P, P, P]
    lib.oracle_refill_accumulate.restype = None
    lib.oracle_refill_accumulate.argtypes = [P, P, i64, i64, i64, ctypes.POINTER(_Bank),
                                             ctypes.POINTER(_Bank), P, P, P]
    lib.oracle_refill_finalize.restype = None
    lib.oracle_refill_finalize.argtypes = [P, P, i64, i64, i64, P, P, P]
    lib.oracle_router_norm_keep.restype = None
    lib.oracle_router_norm_keep.argtypes = [P, i64, i64, i64, P, P]
    del i32
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


# --------------------------------------------------------------------------- banks

class Proj:
    """One projection of a bank of experts, as raw arrays (see moe_oracle.c for layouts)."""

    def __init__(self, fmt, in_dim, out_dim, w=None, qweight=None, qzeros=None, scales=None,
                 codes=None, bscales=None, gscales=None, wglobal=None, aglobal=1.0):
        self.fmt, self.in_dim, self.out_dim = fmt, int(in_dim), int(out_dim)
        self.gscales = None if gscales is None else _c(gscales, np.uint8)
        self.wglobal = None if wglobal is None else _c(wglobal, np.float32)
        self.aglobal = float(np.float32(aglobal))
        self.w = None if w is None else _c(w, np.uint16)
        self.qweight = None if qweight is None else _c(qweight, np.int32)
        self.qzeros = None if qzeros is None else _c(qzeros, np.int32)
        self.scales = None if scales is None else _c(scales, np.uint16)
        self.codes = None if codes is None else _c(codes, np.uint8)
        self.bscales = None if bscales is None else _c(bscales, np.float32)

    def _struct(self):
        return _Proj(self.fmt, self.in_dim, self.out_dim, _ptr(self.w), _ptr(self.qweight),
                     _ptr(self.qzeros), _ptr(self.scales), _ptr(self.codes), _ptr(self.bscales),
                     _ptr(self.gscales), _ptr(self.wglobal), self.aglobal)

    def take(self, experts) -> "Proj":
        """Expert-granular slice (used by tests to pass only the experts they need)."""
        experts = np.asarray(experts, dtype=np.int64)
        pick = (lambda a: None if a is None else a[experts])
        return Proj(self.fmt, self.in_dim, self.out_dim, pick(self.w), pick(self.qweight),
                    pick(self.qzeros), pick(self.scales), pick(self.codes), pick(self.bscales),
                    pick(self.gscales), pick(self.wglobal), self.aglobal)


class Bank:
    """A bank of SwiGLU experts: gate/up map hidden->inter, down maps inter->hidden."""

    def __init__(self, num_experts, hidden, inter, gate: Proj, up: Proj, down: Proj):
        self.num_experts, self.hidden, self.inter = int(num_experts), int(hidden), int(inter)
        self.gate, self.up, self.down = gate, up, down

    def _struct(self):
        return _Bank(self.num_experts, self.hidden, self.inter, self.gate._struct(),
                     self.up._struct(), self.down._struct())

    def take(self, experts) -> "Bank":
        experts = np.asarray(experts)
        return Bank(len(experts), self.hidden, self.inter, self.gate.take(experts),
                    self.up.take(experts), self.down.take(experts))


def bank_from_tensors(d: dict, prefix: str = "") -> Bank:
    """Build a Bank from a dict of numpy arrays named like the workload generator's."""
    fmt = d[prefix + "fmt"]
    if fmt == "bf16":
        E, F, H = d[prefix + "gate"].shape
        return Bank(E, H, F,
                    Proj(BF16, H, F, w=d[prefix + "gate"]),
                    Proj(BF16, H, F, w=d[prefix + "up"]),
                    Proj(BF16, F, H, w=d[prefix + "down"]))
    if fmt == "nvfp4":
        E, F, H2 = d[prefix + "gate_fp4"].shape
        H = H2 * 2
        mk = lambda n, i, o, ga: Proj(NVFP4, i, o, codes=d[prefix + n + "_fp4"],
                                      gscales=d[prefix + n + "_fp4scales"],
                                      wglobal=d[prefix + n + "_wglobal"], aglobal=ga)
        ga_gu, ga_dn = float(d[prefix + "act_global_gu"]), float(d[prefix + "act_global_down"])
        return Bank(E, H, F, mk("gate", H, F, ga_gu), mk("up", H, F, ga_gu), mk("down", F, H, ga_dn))
    if fmt == "fp8":
        E, F, H = d[prefix + "gate_codes"].shape
        mk = lambda n, i, o: Proj(FP8, i, o, codes=d[prefix + n + "_codes"],
                                  bscales=d[prefix + n + "_bscales"])
        return Bank(E, H, F, mk("gate", H, F), mk("up", H, F), mk("down", F, H))
    if fmt == "awq_om":
        # AWQ codes stored output-major: qweight [E][out][in/8], nibble j of
        # word w = input 8w + j; zeros and scales as in the AWQ layout
        E, F, H8 = d[prefix + "gate_qweight"].shape
        H = H8 * 8
        fmt_id = AWQ_OM
    else:
        E, H, F8 = d[prefix + "gate_qweight"].shape
        F = F8 * 8
        fmt_id = AWQ
    mk = lambda n, i, o: Proj(fmt_id, i, o, qweight=d[prefix + n + "_qweight"],
                              qzeros=d[prefix + n + "_qzeros"], scales=d[prefix + n + "_scales"])
    return Bank(E, H, F, mk("gate", H, F), mk("up", H, F), mk("down", F, H))


# --------------------------------------------------------------------------- steps

def dot_exact_f32(a_bits: np.ndarray, b_bits: np.ndarray) -> np.float32:
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    return np.float32(_load().oracle_dot_exact_f32(_ptr(a), _ptr(b), a.size))


def dot_certified(a_bits, b_bits):
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    out = np.zeros(1, np.float64)
    ok = _load().oracle_dot_certified(_ptr(a), _ptr(b), a.size, _ptr(out))
    return bool(ok), float(out[0])


def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray):
    """Exact router logits [T, E] (fp32) and the number of fixed-point fallbacks."""
    x, w = _c(x_bits, np.uint16), _c(w_router_bits, np.uint16)
    T, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    out = np.empty((T, E), np.float32)
    nfb = _load().oracle_router_logits(_ptr(x), _ptr(w), T, H, E, _ptr(out))
    return out, int(nfb)


def rank(logits: np.ndarray, n: int) -> np.ndarray:
    l = _c(logits, np.float32)
    T, E = l.shape
    idx = np.empty((T, n), np.int32)
    _load().oracle_rank(_ptr(l), T, E, n, _ptr(idx))
    return idx


def gates(logits: np.ndarray, idx: np.ndarray, k: int) -> np.ndarray:
    l, ix = _c(logits, np.float32), _c(idx, np.int32)
    T, E = l.shape
    g = np.empty((T, k), np.float64)
    _load().oracle_gates(_ptr(l), _ptr(ix), T, E, k, ix.shape[1], _ptr(g))
    return g


def permute(idx: np.ndarray, E: int):
    ix = _c(idx, np.int32)
    T, k = ix.shape
    offsets = np.empty(E + 1, np.int32)
    sorted_pair = np.empty(T * k, np.int32)
    pair_to_row = np.empty(T * k, np.int32)
    _load().oracle_permute(_ptr(ix), T, k, E, _ptr(offsets), _ptr(sorted_pair), _ptr(pair_to_row))
    return offsets, sorted_pair, pair_to_row


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e2m1_round(v: float) -> int:
    return int(_load().oracle_e2m1_round(float(np.float32(v))))


def e4m3_round(f: float) -> int:
    return int(_load().oracle_e4m3_round(float(np.float32(f))))


def nvfp4_quantize(v, ga: float) -> np.ndarray:
    """NVFP4 quantisation of fp32 values in groups of 16 (see moe_oracle.c);
    returns e2m1(code) * block scale, without the global factor ga."""
    a = _c(v, np.float32)
    out = np.empty(a.shape, np.float64)
    _load().oracle_nvfp4_quantize(_ptr(a), a.size, float(np.float32(ga)), _ptr(out))
    return out


def e4m3_value(code: int) -> float:
    """Exact value of an OCP FP8 E4M3 code."""
    return float(_load().oracle_e4m3_value(int(code)))


def proj_weight(p: Proj, e: int, o: int, i: int) -> float:
    s = p._struct()
    return float(_load().oracle_proj_weight(ctypes.byref(s), e, o, i))


def pair_outputs(x_bits: np.ndarray, idx: np.ndarray, bank: Bank) -> np.ndarray:
    """Per-pair expert outputs [T*k, H] in pair order p = t*k + slot."""
    x, ix = _c(x_bits, np.uint16), _c(idx, np.int32)
    T, k = ix.shape
    assert x.shape == (T, bank.hidden)
    rows = np.empty((T * k, bank.hidden), np.float64)
    b = bank._struct()
    _load().oracle_pair_outputs(_ptr(x), T, k, _ptr(ix), ctypes.byref(b), _ptr(rows))
    return rows


def shared_outputs(x_bits: np.ndarray, shared: Bank) -> np.ndarray:
    x = _c(x_bits, np.uint16)
    T = x.shape[0]
    s = np.empty((T, shared.hidden), np.float64)
    b = shared._struct()
    _load().oracle_shared_outputs(_ptr(x), T, ctypes.byref(b), _ptr(s))
    return s


def combine(rows: np.ndarray, g: np.ndarray, s=None, shared_scale=None) -> np.ndarray:
    T, k = g.shape
    H = rows.shape[1]
    r, gg = _c(rows, np.float64), _c(g, np.float64)
    ss = None if s is None else _c(s, np.float64)
    sc = None if shared_scale is None else _c(shared_scale, np.float64)
    y = np.empty((T, H), np.float64)
    _load().oracle_combine(_ptr(r), _ptr(gg), _ptr(ss), _ptr(sc), T, k, H, _ptr(y))
    return y


def layer(x_bits, w_router_bits, k: int, bank: Bank, shared: Bank | None = None,
          shared_scale=None):
    """Whole layer: returns (y [T,H] fp64, idx [T,k] int32, gates [T,k] fp64)."""
    x, w = _c(x_bits, np.uint16), _c(w_router_bits, np.uint16)
    T = x.shape[0]
    E = w.shape[0]
    y = np.empty((T, bank.hidden), np.float64)
    idx = np.empty((T, k), np.int32)
    g = np.empty((T, k), np.float64)
    b = bank._struct()
    sb = shared._struct() if shared is not None else None
    sc = None if shared_scale is None else _c(shared_scale, np.float64)
    _load().oracle_layer(_ptr(x), _ptr(w), T, E, k, ctypes.byref(b),
                         ctypes.byref(sb) if sb is not None else None, _ptr(sc), _ptr(y),
                         _ptr(idx), _ptr(g))
    return y, idx, g


def refill_accumulate(x_bits, logits, k: int, bank: Bank, shared: Bank | None,
                      stat_sum: np.ndarray, stat_count: np.ndarray, valid=None):
    """Adds this batch's Refill-RMS statistics into stat_sum (fp64 [E]) / stat_count (int64 [E])."""
    x, l = _c(x_bits, np.uint16), _c(logits, np.float32)
    T, E = l.shape
    assert stat_sum.dtype == np.float64 and stat_count.dtype == np.int64
    assert stat_sum.flags.c_contiguous and stat_count.flags.c_contiguous
    v = None if valid is None else _c(valid, np.uint8)
    b = bank._struct()
    sb = shared._struct() if shared is not None else None
    _load().oracle_refill_accumulate(_ptr(x), _ptr(l), T, E, k, ctypes.byref(b),
                                     ctypes.byref(sb) if sb is not None else None, _ptr(v),
                                     _ptr(stat_sum), _ptr(stat_count))


def refill_finalize(stat_sum, stat_count, H: int, keep: int):
    s, c = _c(stat_sum, np.float64), _c(stat_count, np.int64)
    E = s.shape[0]
    score = np.empty(E, np.float64)
    mask = np.empty(E, np.uint8)
    keep_idx = np.empty(keep, np.int32)
    _load().oracle_refill_finalize(_ptr(s), _ptr(c), E, H, keep, _ptr(score), _ptr(mask),
                                   _ptr(keep_idx))
    return score, mask, keep_idx


def router_norm_keep(w_router_bits, keep: int):
    w = _c(w_router_bits, np.uint16)
    E, H = w.shape
    norm = np.empty(E, np.float64)
    keep_idx = np.empty(keep, np.int32)
    _load().oracle_router_norm_keep(_ptr(w), E, H, keep, _ptr(norm), _ptr(keep_idx))
    return norm, keep_idx


def prune_slice(w_router_bits, bank: Bank, keep_idx):
    """Pruning keeps router rows and expert tensors of the kept experts, in the
    keep-set's order ([RAZOR] card: surviving expert weights and router rows are
    slices of the base checkpoint, in matching order)."""
    keep_idx = np.asarray(keep_idx)
    return _c(w_router_bits, np.uint16)[keep_idx], bank.take(keep_idx)


# --------------------------------------------------------------------------- bits helpers

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round to nearest even, via fp32 (exact for values already fp32)."""
    f = np.asarray(v, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)
