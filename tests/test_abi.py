"""The C-ABI library loads, exports every entry point include/moe.h declares,
and rejects bad arguments on the host before touching the GPU (these calls
return before any HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import sparse_moe_expert_router_amd as moe
from sparse_moe_expert_router_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")
OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    L = moe.lib()
    for s in range(6):
        assert L.moe_status_string(s)
    assert L.moe_last_hip_error() == 0


def test_route_validation():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    args = lambda T, H, E, k, extra, x=fake: (x, fake, T, H, E, k, extra, fake, None, fake, None,
                                              fake, 1 << 30, None)
    assert L.moe_route(*args(4, 64, 8, 9, 0)) == SHAPE       # k > E
    assert L.moe_route(*args(4, 64, 8, 8, 1)) == SHAPE       # k + extra > E
    assert L.moe_route(*args(-1, 64, 8, 2, 0)) == SHAPE
    assert L.moe_route(*args(4, 64, 2048, 2, 0)) == UNSUP    # E > 1024
    assert L.moe_route(*args(4, 60, 8, 2, 0)) == UNSUP       # H % 8
    assert L.moe_route(*args(0, 64, 8, 2, 0)) == OK          # T = 0: no-op
    assert L.moe_route(*args(4, 64, 8, 2, 0, x=None)) == NULL
    assert L.moe_route(fake, fake, 4, 64, 8, 2, 0, fake, None, fake, None, fake, 16, None) == WS


def test_route_permute_validation():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    args = lambda T, H, E, k, x=fake, off=fake, ws=fake, n=1 << 30: (
        x, fake, T, H, E, k, fake, None, fake, off, fake, fake, ws, n, None)
    assert L.moe_route_permute(*args(4, 64, 8, 9)) == SHAPE        # k > E
    assert L.moe_route_permute(*args(-1, 64, 8, 2)) == SHAPE
    assert L.moe_route_permute(*args(4, 64, 2048, 2)) == UNSUP     # E > 1024
    assert L.moe_route_permute(*args(4, 60, 8, 2)) == UNSUP        # H % 8
    assert L.moe_route_permute(*args(4, 64, 128, 65)) == UNSUP     # k > 64
    assert L.moe_route_permute(*args(0, 64, 8, 2)) == OK           # T = 0: no-op
    assert L.moe_route_permute(*args(4, 64, 8, 2, x=None)) == NULL
    assert L.moe_route_permute(*args(4, 64, 8, 2, off=None)) == NULL
    need = L.moe_workspace_bytes(5, 4, 2, 8, 64, 0)
    assert need >= L.moe_workspace_bytes(0, 4, 2, 8, 64, 0)
    assert need >= L.moe_workspace_bytes(1, 4, 2, 8, 64, 0)
    assert L.moe_route_permute(*args(4, 64, 8, 2, n=need - 1)) == WS
    assert L.moe_route_permute(*args(4, 64, 8, 2, ws=None, n=need)) == NULL


def test_permute_and_combine_validation():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    assert L.moe_permute(fake, 4, 0, 8, fake, fake, fake, None, 0, None) == SHAPE
    assert L.moe_permute(fake, 4, 2, 4096, fake, fake, fake, None, 0, None) == UNSUP
    assert L.moe_permute(None, 4, 2, 8, fake, fake, fake, None, 0, None) == NULL
    assert L.moe_permute(fake, 100000, 10, 512, fake, fake, fake, None, 0, None) == WS
    assert L.moe_combine(fake, 0, fake, fake, 4, 2, 60, None, None, fake, None) == UNSUP
    assert L.moe_combine(fake, 7, fake, fake, 4, 2, 64, None, None, fake, None) == UNSUP
    assert L.moe_combine(None, 0, fake, fake, 4, 2, 64, None, None, fake, None) == NULL


def _bank(fmt=0, E=4, H=256, F=128, ptr=256):
    mk = lambda i, o: _lib._Proj(fmt, i, o, ptr, ptr, ptr, ptr)
    return _lib._Experts(E, H, F, mk(H, F), mk(H, F), mk(F, H))


def test_grouped_ffn_validation():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    b = _bank()
    call = lambda bank, T=8, k=2, off=fake, sp=fake, dt=0, ws=1 << 30: L.moe_grouped_ffn(
        fake, T, k, ctypes.byref(bank), off, sp, dt, fake, fake, ws, None)
    assert call(b, k=0) == SHAPE
    assert call(_bank(E=0)) == SHAPE
    assert call(_bank(H=200)) == UNSUP                     # hidden % 64
    assert call(_bank(fmt=1, F=48)) == UNSUP               # AWQ width % 32
    assert call(_bank(fmt=5)) == UNSUP
    assert call(b, off=None) == NULL                       # half of the permutation
    assert call(b, off=None, sp=None) == SHAPE             # identity needs one expert and k = 1
    assert call(_bank(E=1), k=1, off=None, sp=None, T=0) == OK
    assert call(b, dt=3) == UNSUP
    assert call(b, ws=0) == WS
    bad = _bank()
    bad.down.in_dim = 64                                   # inconsistent projection sizes
    assert call(bad) == SHAPE
    assert L.moe_grouped_ffn(fake, 8, 2, None, fake, fake, 0, fake, fake, 1 << 30, None) == NULL


def _nvfp4_bank(E=4, H=256, F=128, act=(0.01, 0.01, 0.01), gptr=256):
    mk = lambda i, o, a: _lib._Proj(3, i, o, None, None, None, None, 256, None, gptr, 256, a)
    return _lib._Experts(E, H, F, mk(H, F, act[0]), mk(H, F, act[1]), mk(F, H, act[2]))


def test_nvfp4_validation():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    call = lambda bank: L.moe_grouped_ffn(fake, 8, 2, ctypes.byref(bank), fake, fake, 0, fake, fake,
                                          1 << 30, None)
    assert call(_nvfp4_bank(F=48)) == UNSUP                     # inter % 32
    assert call(_nvfp4_bank(act=(0.0, 0.0, 0.01))) == SHAPE     # act_scale must be > 0
    assert call(_nvfp4_bank(act=(0.01, 0.01, float("nan")))) == SHAPE
    assert call(_nvfp4_bank(act=(0.01, 0.02, 0.01))) == SHAPE   # gate and up share their input
    assert call(_nvfp4_bank(gptr=257)) == UNSUP                 # group scales read two at a time
    assert call(_nvfp4_bank(gptr=0)) == NULL
    # the NVFP4 workspace covers the quantised input as well
    for T in (1, 16, 4096):
        assert L.moe_workspace_bytes(4, T, 10, 512, 2560, 640) >= \
            L.moe_workspace_bytes(2, T, 10, 512, 2560, 640) + T * 2560 * 2
    q = L.moe_nvfp4_quantize
    assert q(fake, 4, 24, ctypes.c_float(0.01), fake, None) == UNSUP   # n % 16
    assert q(fake, 4, 32, ctypes.c_float(-1.0), fake, None) == SHAPE
    assert q(fake, -1, 32, ctypes.c_float(0.01), fake, None) == SHAPE
    assert q(None, 0, 32, ctypes.c_float(0.01), None, None) == OK      # nothing to do
    assert q(None, 4, 32, ctypes.c_float(0.01), fake, None) == NULL
    assert q(ctypes.c_void_p(264), 4, 32, ctypes.c_float(0.01), fake, None) == UNSUP


def test_refill_and_keep_validation():
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    assert L.moe_refill_score(fake, fake, fake, fake, fake, None, 8, 10, 64, 10, fake, fake,
                              fake, 1 << 30, None) == SHAPE   # E < k + 1
    assert L.moe_refill_score(fake, fake, fake, fake, fake, None, 8, 40, 64, 512, fake, fake,
                              fake, 1 << 30, None) == UNSUP   # k + 1 > 32
    assert L.moe_refill_score(fake, fake, fake, fake, fake, None, 8, 10, 64, 512, fake, fake,
                              fake, 0, None) == WS
    assert L.moe_refill_score(fake, fake, fake, fake, fake, None, 8, 10, 64, 512, fake, fake,
                              ctypes.c_void_p(260), 1 << 30, None) == UNSUP   # misaligned workspace
    assert L.moe_refill_finalize(fake, fake, 16, 64, 17, fake, fake, fake, None) == SHAPE
    assert L.moe_refill_finalize(fake, fake, 2048, 64, 17, fake, fake, fake, None) == UNSUP
    assert L.moe_router_norm_keep(fake, 16, 64, -1, fake, fake, None) == SHAPE
    src, dst = _bank(E=8), _bank(E=3)
    assert L.moe_prune_slice(fake, 4, fake, fake, 256, ctypes.byref(src), ctypes.byref(dst), None) == SHAPE
    assert L.moe_prune_slice(fake, 3, fake, None, 256, ctypes.byref(src), ctypes.byref(dst), None) == NULL


def test_workspace_sizes_monotone_in_tokens():
    for op, k in ((moe.OP_ROUTE, 10), (moe.OP_PERMUTE, 10), (moe.OP_GROUPED_FFN, 10),
                  (moe.OP_REFILL_SCORE, 10)):
        sizes = [moe.workspace_bytes(op, T, k, 512, 2560, 640) for T in (16, 256, 4096, 32768)]
        assert sizes == sorted(sizes), (op, sizes)


def test_streaming_workspace_covers_every_row_when_the_gemm_cannot_run():
    # width 96 is not a multiple of the GEMM's 128-column tile, so every row of
    # every expert goes through the streaming kernels: the workspace keeps growing
    sizes = [moe.workspace_bytes(moe.OP_GROUPED_FFN, T, 2, 8, 256, 96) for T in (100, 1000, 10000)]
    assert sizes[0] < sizes[1] < sizes[2]
    assert sizes[2] >= 9 * sizes[1]


def test_grouped_ffn_noalloc_validation():
    L = moe.lib()
    assert L.moe_grouped_ffn_noalloc_max_bytes() == 16 << 20
    fake = ctypes.c_void_p(256)
    b = _bank(E=512, H=2560, F=640)
    # a decode batch far beyond the scratch array is refused before any HIP call
    assert L.moe_grouped_ffn_noalloc(fake, 4096, 10, ctypes.byref(b), fake, fake, 0, fake, None) == WS
    assert L.moe_grouped_ffn_noalloc(fake, -1, 10, ctypes.byref(b), fake, fake, 0, fake, None) == SHAPE
    assert L.moe_grouped_ffn_noalloc(fake, 16, 10, None, fake, fake, 0, fake, None) == NULL
    assert L.moe_grouped_ffn_noalloc(None, 0, 10, ctypes.byref(b), fake, fake, 0, None, None) == OK


def test_awq_to_output_major_validation():
    L = moe.lib()
    src, dst = _bank(fmt=1, E=4, H=256, F=128), _bank(fmt=4, E=4, H=256, F=128)
    assert L.moe_awq_to_output_major(None, ctypes.byref(dst), None) == NULL
    assert L.moe_awq_to_output_major(ctypes.byref(dst), ctypes.byref(dst), None) == SHAPE   # src not AWQ
    assert L.moe_awq_to_output_major(ctypes.byref(src), ctypes.byref(src), None) == SHAPE   # dst not AWQ_OM
    assert L.moe_awq_to_output_major(ctypes.byref(src), ctypes.byref(_bank(fmt=4, E=5)), None) == SHAPE
    # the output-major layout needs hidden % 256 and inter % 128
    assert L.moe_awq_to_output_major(ctypes.byref(_bank(fmt=1, H=192, F=128)),
                                     ctypes.byref(_bank(fmt=4, H=192, F=128)), None) == UNSUP
    # codes that overlap are refused (the fake banks point every tensor at one address)
    assert L.moe_awq_to_output_major(ctypes.byref(src), ctypes.byref(dst), None) == SHAPE


def test_layer_validation():
    """moe_layer checks everything the four calls it stands for check, before
    any HIP call (the fake pointers are never dereferenced)."""
    L = moe.lib()
    fake = ctypes.c_void_p(256)
    b, sh = _bank(E=16, H=256, F=128), _bank(E=1, H=256, F=256)
    need = L.moe_layer_workspace_bytes(8, 2, ctypes.byref(b), ctypes.byref(sh))
    assert need > 0
    assert L.moe_layer_workspace_bytes(16, 2, ctypes.byref(b), ctypes.byref(sh)) >= need
    assert L.moe_layer_workspace_bytes(8, 2, ctypes.byref(b), None) < need
    assert L.moe_layer_workspace_bytes(0, 2, ctypes.byref(b), None) == 0
    assert L.moe_layer_workspace_bytes(8, 2, ctypes.byref(_bank(fmt=5)), None) == 0

    def call(T=8, k=2, bank=b, shared=sh, scale=None, x=fake, y=fake, ws=fake, n=need, side=None):
        return L.moe_layer(x, T, fake, k, ctypes.byref(bank) if bank is not None else None,
                           ctypes.byref(shared) if shared is not None else None, scale, y, None, ws, n, None,
                           side, None)
    assert call(k=0) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(k=17) == SHAPE                              # k > E
    assert call(bank=None) == NULL
    assert call(bank=_bank(H=200)) == UNSUP
    assert call(shared=_bank(E=2, H=256)) == SHAPE          # the shared bank holds one expert
    assert call(shared=_bank(E=1, H=512, F=128)) == SHAPE   # of the same hidden size
    assert call(shared=None, scale=fake) == SHAPE           # a scale without a shared expert
    assert call(x=None) == NULL
    assert call(y=None) == NULL
    assert call(ws=None) == NULL
    assert call(n=need - 1) == WS
    assert call(x=ctypes.c_void_p(258)) == UNSUP            # misaligned
    assert call(T=0, x=None, y=None, ws=None, n=0) == OK
