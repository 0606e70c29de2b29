"""ctypes binding of libmoe.so: argument marshalling only.

Every step of the layer runs in the HIP library; this module allocates the
output tensors with torch (device memory is torch's), passes raw device
pointers and torch's current HIP stream, and turns status codes into
exceptions.  It fails loudly when libmoe.so has not been built.

Expert banks are dicts of device tensors:
  bf16: {"fmt": "bf16", "gate": [E,F,H], "up": [E,F,H], "down": [E,H,F]}  (torch.bfloat16)
  awq : {"fmt": "awq", "gate_qweight": [E,H,F/8] int32, "gate_qzeros": [E,H/32,F/8] int32,
         "gate_scales": [E,H/32,F] fp16, and the same for "up_*" and "down_*"
         (down: [E,F,H/8], [E,F/32,H/8], [E,F/32,H])}
  awq_om: as "awq" with output-major codes: "gate_qweight" [E,F,H/8], "down_qweight" [E,H,F/8]
         (word w of a column holds inputs 8w..8w+7, input 8w+j in nibble j)
  fp8 : {"fmt": "fp8", "gate_codes": [E,F,H] uint8 E4M3, "gate_bscales": [E,F/128,H/128] f32,
         and the same for "up_*" and "down_*" (down: [E,H,F], [E,H/128,F/128])}
  nvfp4: {"fmt": "nvfp4", "gate_fp4": [E,F,H/2] uint8 (two E2M1 codes, low nibble = even
         input), "gate_fp4scales": [E,F,H/16] uint8 E4M3, "gate_wglobal": [E] f32, the same
         for "up_*" and "down_*" (down: [E,H,F/2], [E,H,F/16], [E]), and the activation
         global scales "act_global_gu" (gate and up inputs) and "act_global_down" (floats)}
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

OP_ROUTE, OP_PERMUTE, OP_GROUPED_FFN, OP_REFILL_SCORE, OP_GROUPED_FFN_NVFP4, OP_ROUTE_PERMUTE = 0, 1, 2, 3, 4, 5
W_BF16, W_AWQ, W_FP8, W_NVFP4, W_AWQ_OM = 0, 1, 2, 3, 4
OUT_BF16, OUT_F32 = 0, 1

EXPORTS = ["moe_route", "moe_permute", "moe_route_permute", "moe_grouped_ffn", "moe_grouped_ffn_noalloc",
           "moe_grouped_ffn_noalloc_max_bytes", "moe_layer", "moe_layer_workspace_bytes", "moe_combine",
           "moe_refill_score",
           "moe_refill_finalize", "moe_prune_slice", "moe_router_norm_keep",
           "moe_nvfp4_quantize", "moe_awq_to_output_major", "moe_workspace_bytes", "moe_status_string",
           "moe_last_hip_error"]


class MoeError(RuntimeError):
    pass


class _Proj(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("in_dim", ctypes.c_int32), ("out_dim", ctypes.c_int32),
                ("w", ctypes.c_void_p), ("qweight", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("block_scales", ctypes.c_void_p),
                ("group_scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("act_scale", ctypes.c_float)]


class _Experts(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("gate", _Proj), ("up", _Proj), ("down", _Proj)]


_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                       "(python sparse_moe_expert_router_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_route": [P, P, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P],
        "moe_permute": [P, i32, i32, i32, P, P, P, P, sz, P],
        "moe_route_permute": [P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P],
        "moe_grouped_ffn": [P, i32, i32, ctypes.POINTER(_Experts), P, P, i32, P, P, sz, P],
        "moe_grouped_ffn_noalloc": [P, i32, i32, ctypes.POINTER(_Experts), P, P, i32, P, P],
        "moe_combine": [P, i32, P, P, i32, i32, i32, P, P, P, P],
        "moe_refill_score": [P, P, P, P, P, P, i32, i32, i32, i32, P, P, P, sz, P],
        "moe_refill_finalize": [P, P, i32, i32, i32, P, P, P, P],
        "moe_prune_slice": [P, i32, P, P, i32, ctypes.POINTER(_Experts), ctypes.POINTER(_Experts), P],
        "moe_router_norm_keep": [P, i32, i32, i32, P, P, P],
        "moe_nvfp4_quantize": [P, i32, i32, ctypes.c_float, P, P],
        "moe_awq_to_output_major": [ctypes.POINTER(_Experts), ctypes.POINTER(_Experts), P],
        "moe_layer": [P, i32, P, i32, ctypes.POINTER(_Experts), ctypes.POINTER(_Experts), P, P, P, P, sz, P,
                      P, ctypes.POINTER(P)],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.moe_grouped_ffn_noalloc_max_bytes.argtypes = []
    L.moe_grouped_ffn_noalloc_max_bytes.restype = ctypes.c_size_t
    L.moe_layer_workspace_bytes.argtypes = [i32, i32, ctypes.POINTER(_Experts), ctypes.POINTER(_Experts)]
    L.moe_layer_workspace_bytes.restype = ctypes.c_size_t
    L.moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.moe_workspace_bytes.restype = ctypes.c_size_t
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_hip_error.argtypes = []
    L.moe_last_hip_error.restype = ctypes.c_int32
    _lib = L
    return L


def _check(name, status):
    if status != 0:
        L = lib()
        msg = L.moe_status_string(status).decode()
        raise MoeError(f"{name}: {msg} (status {status}, hip error {L.moe_last_hip_error()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(op, T, k, E, H, F=0) -> int:
    return int(lib().moe_workspace_bytes(op, T, k, E, H, F))


class Workspace:
    """A grow-only device scratch buffer for the calls that need one."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device or "cuda")
        return self.buf, self.buf.numel()


_default_ws = {}


def _ws(ws, device):
    if ws is not None:
        return ws
    key = str(device)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def experts_struct(bank: dict):
    """ctypes struct of a bank dict (see module docstring); the dict keeps the memory alive."""
    fmt = bank["fmt"]
    if fmt == "bf16":
        E, F, H = bank["gate"].shape
        mk = lambda t, i, o: _Proj(W_BF16, i, o, t.data_ptr(), None, None, None, None, None)
        return _Experts(E, H, F, mk(bank["gate"], H, F), mk(bank["up"], H, F), mk(bank["down"], F, H))
    if fmt == "fp8":
        E, F, H = bank["gate_codes"].shape
        mk = lambda n, i, o: _Proj(W_FP8, i, o, None, None, None, None, bank[n + "_codes"].data_ptr(),
                                   bank[n + "_bscales"].data_ptr())
        return _Experts(E, H, F, mk("gate", H, F), mk("up", H, F), mk("down", F, H))
    if fmt == "nvfp4":
        E, F, H2 = bank["gate_fp4"].shape
        H = H2 * 2
        ga = {"gate": bank["act_global_gu"], "up": bank["act_global_gu"], "down": bank["act_global_down"]}
        mk = lambda n, i, o: _Proj(W_NVFP4, i, o, None, None, None, None, bank[n + "_fp4"].data_ptr(), None,
                                   bank[n + "_fp4scales"].data_ptr(), bank[n + "_wglobal"].data_ptr(),
                                   float(ga[n]))
        return _Experts(E, H, F, mk("gate", H, F), mk("up", H, F), mk("down", F, H))
    E, H, F = bank_dims(bank)
    fid = W_AWQ_OM if fmt == "awq_om" else W_AWQ
    mk = lambda n, i, o: _Proj(fid, i, o, None, bank[n + "_qweight"].data_ptr(),
                               bank[n + "_qzeros"].data_ptr(), bank[n + "_scales"].data_ptr())
    return _Experts(E, H, F, mk("gate", H, F), mk("up", H, F), mk("down", F, H))


def bank_dims(bank: dict):
    if bank["fmt"] == "bf16":
        E, F, H = bank["gate"].shape
    elif bank["fmt"] == "fp8":
        E, F, H = bank["gate_codes"].shape
    elif bank["fmt"] == "nvfp4":
        E, F, H2 = bank["gate_fp4"].shape
        H = H2 * 2
    elif bank["fmt"] == "awq_om":
        E, F, H8 = bank["gate_qweight"].shape
        H = H8 * 8
    else:
        E, H, F8 = bank["gate_qweight"].shape
        F = F8 * 8
    return int(E), int(H), int(F)


# ----------------------------------------------------------------------------- calls

def route(x, w_router, k: int, extra: int = 0, want_logits: bool = False, ws=None):
    """Returns (topk_idx [T,k+extra] int32, topk_logit [T,k+extra] f32, gate [T,k] f32, logits|None)."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    idx = torch.empty((T, k + extra), dtype=torch.int32, device=dev)
    tl = torch.empty((T, k + extra), dtype=torch.float32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    buf, n = _ws(ws, dev).get(0 if want_logits else workspace_bytes(OP_ROUTE, T, k, E, H))
    _check("moe_route", lib().moe_route(_ptr(x), _ptr(w_router), T, H, E, k, extra, _ptr(idx),
                                        _ptr(tl), _ptr(gate), _ptr(logits), _ptr(buf), n, _stream()))
    return idx, tl, gate, logits


def permute(topk_idx, E: int, ws=None):
    """Returns (expert_offsets [E+1], sorted_pair [T*k], pair_to_row [T*k]) int32."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2r = torch.empty(T * k, dtype=torch.int32, device=dev)
    buf, n = _ws(ws, dev).get(workspace_bytes(OP_PERMUTE, T, k, E, 0))
    _check("moe_permute", lib().moe_permute(_ptr(topk_idx), T, k, E, _ptr(off), _ptr(sp), _ptr(p2r),
                                            _ptr(buf), n, _stream()))
    return off, sp, p2r


def route_permute(x, w_router, k: int, ws=None):
    """route (extra = 0) then permute in one call.  Returns (topk_idx, topk_logit, gate,
    expert_offsets, sorted_pair, pair_to_row), as the two calls return them."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tl = torch.empty((T, k), dtype=torch.float32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2r = torch.empty(T * k, dtype=torch.int32, device=dev)
    buf, n = _ws(ws, dev).get(workspace_bytes(OP_ROUTE_PERMUTE, T, k, E, H))
    _check("moe_route_permute", lib().moe_route_permute(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(idx), _ptr(tl),
                                                        _ptr(gate), _ptr(off), _ptr(sp), _ptr(p2r), _ptr(buf),
                                                        n, _stream()))
    return idx, tl, gate, off, sp, p2r


def grouped_ffn(x, k: int, bank: dict, offsets=None, sorted_pair=None, out_dtype=OUT_BF16,
                ws=None, rows=None):
    """rows [T*k, H]: expert outputs in grouped order (identity order when offsets is None)."""
    T, H = x.shape
    E, Hb, F = bank_dims(bank)
    dev = x.device
    if rows is None:
        rows = torch.empty((T * k, H), dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                           device=dev)
    st = experts_struct(bank)
    op = OP_GROUPED_FFN_NVFP4 if bank["fmt"] == "nvfp4" else OP_GROUPED_FFN
    buf, n = _ws(ws, dev).get(workspace_bytes(op, T, k, E, H, F))
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(_ptr(x), T, k, ctypes.byref(st), _ptr(offsets),
                                                    _ptr(sorted_pair), out_dtype, _ptr(rows),
                                                    _ptr(buf), n, _stream()))
    return rows


def grouped_ffn_noalloc(x, k: int, bank: dict, offsets=None, sorted_pair=None, out_dtype=OUT_BF16,
                        rows=None):
    """grouped_ffn through the allocation-free entry point: the library's own
    per-GPU scratch array instead of a workspace (at most
    noalloc_max_bytes() of scratch; larger calls raise)."""
    T, H = x.shape
    dev = x.device
    if rows is None:
        rows = torch.empty((T * k, H), dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                           device=dev)
    st = experts_struct(bank)
    _check("moe_grouped_ffn_noalloc", lib().moe_grouped_ffn_noalloc(
        _ptr(x), T, k, ctypes.byref(st), _ptr(offsets), _ptr(sorted_pair), out_dtype, _ptr(rows), _stream()))
    return rows


def noalloc_max_bytes() -> int:
    return int(lib().moe_grouped_ffn_noalloc_max_bytes())


def combine(rows, pair_to_row, gate, shared=None, shared_scale=None, y=None):
    T, k = gate.shape
    H = rows.shape[1]
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=rows.device)
    rdt = OUT_F32 if rows.dtype == torch.float32 else OUT_BF16
    _check("moe_combine", lib().moe_combine(_ptr(rows), rdt, _ptr(pair_to_row), _ptr(gate), T, k, H,
                                            _ptr(shared), _ptr(shared_scale), _ptr(y), _stream()))
    return y


def refill_score(rows, offsets, sorted_pair, pair_to_row, topk_logit, stat_sum,
                 stat_count, token_valid=None, ws=None):
    """Adds Refill-RMS statistics of one batch into stat_sum (f32 [E]) and stat_count (int32 [E],
    read as uint32)."""
    T, K1 = topk_logit.shape
    k = K1 - 1
    H = rows.shape[1]
    E = stat_sum.shape[0]
    buf, n = _ws(ws, rows.device).get(workspace_bytes(OP_REFILL_SCORE, T, k, E, H))
    _check("moe_refill_score", lib().moe_refill_score(
        _ptr(rows), _ptr(offsets), _ptr(sorted_pair), _ptr(pair_to_row), _ptr(topk_logit), _ptr(token_valid), T, k, H, E, _ptr(stat_sum), _ptr(stat_count),
        _ptr(buf), n, _stream()))


def refill_finalize(stat_sum, stat_count, H: int, keep: int):
    E = stat_sum.shape[0]
    dev = stat_sum.device
    score = torch.empty(E, dtype=torch.float32, device=dev)
    mask = torch.empty(E, dtype=torch.uint8, device=dev)
    keep_idx = torch.empty(keep, dtype=torch.int32, device=dev)
    _check("moe_refill_finalize", lib().moe_refill_finalize(_ptr(stat_sum), _ptr(stat_count), E, H, keep,
                                                            _ptr(score), _ptr(mask), _ptr(keep_idx),
                                                            _stream()))
    return score, mask, keep_idx


def prune_slice(keep_idx, w_router, bank: dict):
    """Router rows and expert tensors of the kept experts, in keep-set order."""
    n = keep_idx.shape[0]
    H = w_router.shape[1] if w_router is not None else bank_dims(bank)[1]
    out = {"fmt": bank["fmt"]}
    for name, t in bank.items():
        if name == "fmt" or isinstance(t, float):
            out[name] = t
        else:
            out[name] = torch.empty((n,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    wr2 = None
    if w_router is not None:
        wr2 = torch.empty((n, H), dtype=w_router.dtype, device=w_router.device)
    src, dst = experts_struct(bank), experts_struct(out)
    _check("moe_prune_slice", lib().moe_prune_slice(_ptr(keep_idx), n, _ptr(w_router), _ptr(wr2), H,
                                                    ctypes.byref(src), ctypes.byref(dst), _stream()))
    return wr2, out


def nvfp4_quantize(x, act_scale: float, out=None):
    """NVFP4 activation quantisation of bf16 x [T, n] (n % 16 == 0) under the
    global scale act_scale: per 16 values the E4M3 block scale s and E2M1 codes,
    returned as bf16 e2m1 * s (exact), the form the NVFP4 experts consume."""
    T, n = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check("moe_nvfp4_quantize", lib().moe_nvfp4_quantize(_ptr(x), T, n, float(act_scale), _ptr(out),
                                                          _stream()))
    return out


def awq_to_output_major(bank: dict) -> dict:
    """The AWQ bank with its codes rearranged output-major (format "awq_om"); the
    zeros and scales tensors are shared with `bank`, not copied."""
    assert bank["fmt"] == "awq"
    E, H, F = bank_dims(bank)
    out = {"fmt": "awq_om"}
    for n, (i, o) in (("gate", (H, F)), ("up", (H, F)), ("down", (F, H))):
        q = bank[n + "_qweight"]
        out[n + "_qweight"] = torch.empty((E, o, i // 8), dtype=torch.int32, device=q.device)
        out[n + "_qzeros"] = bank[n + "_qzeros"]
        out[n + "_scales"] = bank[n + "_scales"]
    src, dst = experts_struct(bank), experts_struct(out)
    _check("moe_awq_to_output_major", lib().moe_awq_to_output_major(ctypes.byref(src), ctypes.byref(dst),
                                                                    _stream()))
    return out


def router_norm_keep(w_router, keep: int):
    E, H = w_router.shape
    norm = torch.empty(E, dtype=torch.float32, device=w_router.device)
    keep_idx = torch.empty(keep, dtype=torch.int32, device=w_router.device)
    _check("moe_router_norm_keep", lib().moe_router_norm_keep(_ptr(w_router), E, H, keep, _ptr(norm),
                                                              _ptr(keep_idx), _stream()))
    return norm, keep_idx


# ----------------------------------------------------------------------------- layer

def layer_workspace_bytes(T: int, k: int, bank: dict, shared: dict | None = None) -> int:
    st = experts_struct(bank)
    sh = experts_struct(shared) if shared is not None else None
    return int(lib().moe_layer_workspace_bytes(T, k, ctypes.byref(st), ctypes.byref(sh) if sh else None))


def _events_arg(events):
    if events is None:
        return None
    return (ctypes.c_void_p * 2)(*[ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events])


class LayerCall:
    """A prepared moe_layer call (the whole layer in one library call): the
    banks' structs, the workspace, y and every pointer are marshalled once, so
    that a call costs one ctypes call.  Calling it enqueues one layer step on
    torch's current stream and returns y (the same tensor every call).

    side_stream (a torch.cuda.Stream, default priority) runs the shared
    expert beside the routed path.  Timing events passed to __call__ must be
    torch.cuda.Event objects that have been recorded once (torch creates the
    underlying HIP event on first record)."""

    def __init__(self, x, w_router, k: int, bank: dict, shared: dict | None = None, shared_scale=None,
                 side_stream=None, ws=None, topk_idx=None):
        T, H = x.shape
        self.x, self.w_router, self.k = x, w_router, k
        self.bank, self.shared, self.shared_scale = bank, shared, shared_scale
        self.st = experts_struct(bank)
        self.sh = experts_struct(shared) if shared is not None else None
        need = int(lib().moe_layer_workspace_bytes(T, k, ctypes.byref(self.st),
                                                   ctypes.byref(self.sh) if self.sh else None))
        if T > 0 and need == 0:
            raise MoeError("moe_layer_workspace_bytes: invalid bank")
        self.ws_buf, self.ws_n = (ws or Workspace(x.device)).get(need)
        self.y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
        self.topk_idx = topk_idx
        self.side = side_stream
        self._args = (_ptr(x), T, _ptr(w_router), k, ctypes.byref(self.st),
                      ctypes.byref(self.sh) if self.sh else None, _ptr(shared_scale), _ptr(self.y),
                      _ptr(topk_idx), _ptr(self.ws_buf), self.ws_n)
        self._side = ctypes.c_void_p(side_stream.cuda_stream) if side_stream is not None else None

    def __call__(self, events=None):
        _check("moe_layer", lib().moe_layer(*self._args, _stream(), self._side, _events_arg(events)))
        return self.y


def layer(x, w_router, k: int, bank: dict, shared: dict | None = None, shared_scale=None, y=None,
          topk_idx=None, ws=None, side_stream=None, routed_events=None):
    """moe_layer: the whole layer in one library call; returns y [T, H] bf16."""
    T, H = x.shape
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    st = experts_struct(bank)
    sh = experts_struct(shared) if shared is not None else None
    shp = ctypes.byref(sh) if sh else None
    buf, n = _ws(ws, x.device).get(int(lib().moe_layer_workspace_bytes(T, k, ctypes.byref(st), shp)))
    side = ctypes.c_void_p(side_stream.cuda_stream) if side_stream is not None else None
    _check("moe_layer", lib().moe_layer(_ptr(x), T, _ptr(w_router), k, ctypes.byref(st), shp, _ptr(shared_scale),
                                        _ptr(y), _ptr(topk_idx), _ptr(buf), n, _stream(), side,
                                        _events_arg(routed_events)))
    return y


def moe_layer(x, w_router, k: int, bank: dict, shared: dict | None = None, shared_scale=None,
              ws=None, keep_intermediates: bool = False, shared_stream=None, shared_ws=None):
    """The MoE feed-forward layer: route -> permute -> routed experts -> shared expert -> combine.

    With `shared_stream` (a torch.cuda.Stream) the shared expert, which needs
    only x, runs on that stream beside routing and the routed experts, with its
    own workspace `shared_ws`; the combine waits for it."""
    main = torch.cuda.current_stream(x.device)
    s = None
    if shared is not None and shared_stream is not None:
        if shared_ws is None:  # calls on different streams need different workspaces
            key = (str(x.device), shared_stream.cuda_stream)
            shared_ws = _default_ws.setdefault(key, Workspace(x.device))
        shared_stream.wait_stream(main)
        with torch.cuda.stream(shared_stream):
            s = grouped_ffn(x, 1, shared, ws=shared_ws)
        x.record_stream(shared_stream)
    idx, tl, gate, off, sp, p2r = route_permute(x, w_router, k, ws=ws)
    rows = grouped_ffn(x, k, bank, off, sp, ws=ws)
    if shared is not None and shared_stream is None:
        s = grouped_ffn(x, 1, shared, ws=ws)
    elif s is not None:
        main.wait_stream(shared_stream)
        s.record_stream(main)
    y = combine(rows, p2r, gate, s, shared_scale)
    if keep_intermediates:
        return y, dict(idx=idx, topk_logit=tl, gate=gate, offsets=off, sorted_pair=sp,
                       pair_to_row=p2r, rows=rows, shared=s)
    return y
