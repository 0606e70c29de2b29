"""Refill-RMS calibration over a stream of packed rows and many layers.

RAZOR E256of512 card, "Selection and calibration": the saliency statistics
are gathered over packed rows of calibration text (at most 32768 tokens a
row, only valid tokens counted), are additive across rows, and the experts of
every layer are then ranked by their Refill-RMS score.  This module drives the
library calls over such a stream: per row and per layer it routes with the
highest-ranked unselected expert, permutes, evaluates the routed experts in
fp32 and adds the layer's statistics; the per-layer sums and counts can be
saved and restored between rows, so a long calibration can stop and resume
with the same result, bit for bit, as an uninterrupted run.

The statistics live on the device as fp32 sums and uint32 counts (int32
tensors read as uint32), one row of E per layer.  A checkpoint is a plain
.npz file (no pickled objects) with the sums, the counts, the number of rows
consumed and the geometry.
"""
from __future__ import annotations

import os

import numpy as np
import torch

from . import _lib

MAX_ROW_TOKENS = 32768


class RefillCalibration:
    """Additive Refill-RMS statistics of `layers` MoE layers with `experts`
    experts each, hidden size `hidden`, `k` experts per token."""

    def __init__(self, layers: int, experts: int, hidden: int, k: int, device="cuda"):
        self.layers, self.experts, self.hidden, self.k = int(layers), int(experts), int(hidden), int(k)
        self.device = torch.device(device)
        self.stat_sum = torch.zeros((self.layers, self.experts), dtype=torch.float32, device=self.device)
        self.stat_count = torch.zeros((self.layers, self.experts), dtype=torch.int32, device=self.device)
        self.rows_done = 0
        self.ws = _lib.Workspace(self.device)

    # ------------------------------------------------------------------ stream
    def add(self, layer: int, x, w_router, bank: dict, token_valid=None):
        """Add one packed row's statistics for one layer.  x: [T, H] bf16 layer
        input (T <= 32768); token_valid: [T] uint8 or None (all valid)."""
        T, H = x.shape
        if T > MAX_ROW_TOKENS:
            raise ValueError(f"a packed row holds at most {MAX_ROW_TOKENS} tokens, got {T}")
        if H != self.hidden or w_router.shape[0] != self.experts:
            raise ValueError("row geometry does not match the calibration")
        idx, tl, _, _ = _lib.route(x, w_router, self.k, extra=1, ws=self.ws)
        off, sp, p2r = _lib.permute(idx, self.experts, ws=self.ws)
        rows = _lib.grouped_ffn(x, self.k + 1, bank, off, sp, out_dtype=_lib.OUT_F32, ws=self.ws)
        _lib.refill_score(rows, off, sp, p2r, tl, self.stat_sum[layer], self.stat_count[layer],
                          token_valid=token_valid, ws=self.ws)

    def add_row(self, layer_inputs, layers, token_valid=None):
        """One packed row through every layer: layer_inputs[l] is layer l's input
        for this row, layers[l] = (w_router, bank)."""
        if len(layer_inputs) != self.layers or len(layers) != self.layers:
            raise ValueError("one input and one (router, bank) per layer")
        for l in range(self.layers):
            self.add(l, layer_inputs[l], layers[l][0], layers[l][1], token_valid)
        self.rows_done += 1

    # ---------------------------------------------------------------- results
    def keep_sets(self, keep: int):
        """Per layer: (score [E] f32, keep_mask [E] u8, keep_idx [keep] ascending)."""
        return [_lib.refill_finalize(self.stat_sum[l], self.stat_count[l], self.hidden, keep)
                for l in range(self.layers)]

    # ------------------------------------------------------------- checkpoint
    def state(self) -> dict:
        return {"stat_sum": self.stat_sum.cpu().numpy(), "stat_count": self.stat_count.cpu().numpy(),
                "rows_done": np.int64(self.rows_done),
                "geometry": np.array([self.layers, self.experts, self.hidden, self.k], np.int64)}

    def save(self, path: str):
        """Write the statistics to `path` (.npz); the file is replaced atomically."""
        tmp = path + ".tmp.npz"
        np.savez(tmp, **self.state())
        os.replace(tmp, path)

    @classmethod
    def load(cls, path: str, device="cuda") -> "RefillCalibration":
        with np.load(path, allow_pickle=False) as z:
            L, E, H, k = (int(v) for v in z["geometry"])
            c = cls(L, E, H, k, device)
            c.stat_sum.copy_(torch.from_numpy(z["stat_sum"]))
            c.stat_count.copy_(torch.from_numpy(z["stat_count"]))
            c.rows_done = int(z["rows_done"])
        return c
